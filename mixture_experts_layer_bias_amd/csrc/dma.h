// Direct global -> LDS loads (global_load_lds_dwordx4) and explicit waits, for gfx950.
//
// One instruction moves 16 bytes per lane: lane l's bytes land at the wave's LDS
// base + 16 l, so a wave writes 1 KB of LDS contiguously.  The loads count
// against vmcnt; the LDS writes are complete once vmcnt has dropped past them.
#pragma once

#include "common.h"

namespace moe {

typedef const void __attribute__((address_space(1)))* dma_gptr_t;
typedef void __attribute__((address_space(3)))* dma_lptr_t;

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((dma_gptr_t)src, (dma_lptr_t)lds_wave_base, 16, 0, 0);
}

// The same load at device scope (sc1): served from the device's coherence point rather than from
// lines this CU or this XCD's L2 may still hold, so it sees data that another XCD has written
// with device-scope stores.
__device__ __forceinline__ void dma16_device_scope(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((dma_gptr_t)src, (dma_lptr_t)lds_wave_base, 16, 0, 16);
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void dma_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 0xF) | ((N >> 4) << 14));
}

}  // namespace moe
