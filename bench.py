"""Benchmark of the MoE layer forward on one MI355X.

A step is one whole layer forward (router GEMM, scoring + top-K, sort by
expert, grouped gate/up + SwiGLU, grouped down, unpermute-reduce and blends)
over one batch of seeded synthetic tokens, with every input resident in HBM.
Prints one JSON line.  The default workload is the decode layer (4 tokens,
H 2048, 128 experts, top-8, I 768); --workload picks another.

The dominant kernel is timed with HIP events recorded on the stream the
library launches on, over the same kind of steps, and reported against the
binding roofline: for a decode batch with bf16 weights and no shared expert,
the one launch that runs the routed gate/up GEMM, the down GEMM and the
unpermute-reduce (through moe_experts_forward); otherwise the routed gate/up
grouped GEMM.  The oracle (float64 numpy on the
host cores) is timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 5000.0}  # dense MFMA peaks (mxfp4: e4m3 x e2m1 MFMA)

# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch averaged over the kernel's dispatches), each scaled by
# what the same counter reads for a plain 1 GiB device copy (FETCH_SIZE reads half the bytes moved:
# x2.0; WRITE_SIZE reads them all: x1.0).  An entry holds only while the kernel's sources hash to the
# value they had when the counters were taken; otherwise the traffic is reported as null.
MEASURED_TRAFFIC = {
    "decode_4tok_h2048_e128_top8_i768": {
        "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_decode.hip",
                    "mixture_experts_layer_bias_amd/csrc/dma.h",
                    "mixture_experts_layer_bias_amd/csrc/gemm_common.h",
                    "mixture_experts_layer_bias_amd/csrc/unpermute.h",
                    "mixture_experts_layer_bias_amd/csrc/common.h"],
        "sha256": "74c10d1180400613c8c488d4182eaa59096788872960652ab2e8dcf822e7b8af",
        "fetch_kib": 140121.41, "write_kib": 253.78, "fetch_scale": 2.0, "write_scale": 1.0,
    },
}


def measured_traffic(workload: str):
    """Bytes per launch of the dominant kernel from the stored counter readings, or None."""
    import hashlib

    rec = MEASURED_TRAFFIC.get(workload)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["sha256"]:
        return None
    return (rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "prefill_zipf", "fp8_sigmoid",
                                                              "zero_experts", "mxfp4_sigmoid"])
    ap.add_argument("--layers", type=int, default=0,
                    help="distinct weight copies cycled through (0: enough to exceed the 256 MB MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes --steps times (the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters), then exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every box here has a single MI355X "
              f"and the multi-GPU expert-parallel path is design only.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_layer_bias_amd as moe
    import moe_inputs as mi
    import moe_inputs.device as mid

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "steps": args.steps}))
        return
    wl = mi.WORKLOADS[args.workload]
    N, H, E, R, K, I, Is = (wl.num_tokens, wl.hidden, wl.num_experts, wl.router_width, wl.top_k, wl.inter,
                            wl.shared_inter)
    fp8 = wl.weight_dtype != "bf16"  # fp8 and mxfp4 experts take e4m3 activations
    abytes = 1 if fp8 else 2  # activation and h element bytes
    wbytes = {"bf16": 2, "fp8": 1, "mxfp4": 0.5 + 1 / 32}[wl.weight_dtype]  # mxfp4: codes + E8M0 per 32
    layer_bytes = 3 * E * I * H * wbytes
    # enough distinct weight copies that the touched experts of consecutive steps cannot be
    # served from the 256 MB Infinity Cache (at least ~8 GB of weights in rotation, at most 8 copies)
    n_layers = args.layers or max(2, min(8, int(np.ceil(8.0e9 / layer_bytes))))
    if layer_bytes * n_layers > 150e9:
        n_layers = max(1, int(150e9 // layer_bytes))

    cfg = moe.make_config(N, H, E, R, K, I, Is, wl.scoring, wl.renormalize, wl.routed_scale, wl.weight_dtype)
    layers = []
    for l in range(n_layers):
        dl = mid.device_layer(wl, layer=l, device="cuda:0")
        w = moe.weights_from_stacked(dl.router, dl.bias, dl.gate, dl.up, dl.down, dl.gate_s, dl.up_s, dl.down_s,
                                     dl.sh_gate, dl.sh_up, dl.sh_down, dl.sh_gate_s, dl.sh_up_s, dl.sh_down_s,
                                    sh_expert_gate=dl.sh_expert_gate)
        layers.append((dl, w))
    # zeroed once: the decode experts path keeps its counters in the workspace and leaves them zero
    ws = torch.zeros(moe.moe_workspace_size(cfg), dtype=torch.uint8, device=dev)
    out = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    L = moe.moe_workspace_layout(cfg)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(i):
        dl, w = layers[i % n_layers]
        moe.moe_forward(cfg, w, dl.x, out, ws, stream)

    # ---- whole-layer timing, eager launches
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_eager = (t1 - t0) * 1e3 / args.steps

    # ---- the same steps replayed from HIP graphs (one captured moe_forward per weight copy), the way a
    # serving loop runs a decode layer: the launches are the library's own, only host overhead goes away
    ms_graph = None
    if not args.no_graph:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for l in range(n_layers):
                gph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gph, stream=cap):
                    dl, w = layers[l]
                    moe.moe_forward(cfg, w, dl.x, out, ws)
                graphs.append(gph)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % n_layers].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % n_layers].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_graph = (t1 - t0) * 1e3 / args.steps
    # the faster of the two launch modes is reported (named in "timing"); both run the same kernels
    use_graph = ms_graph is not None and ms_graph < ms_eager
    ms = ms_graph if use_graph else ms_eager

    # ---- realised routing per layer (for the algorithmic bytes / flops)
    touched, rows_real = [], []
    for l in range(n_layers):
        step(l)
        torch.cuda.synchronize()
        counts = ws[L["counts"]:L["counts"] + 4 * R].view(torch.int32).cpu().numpy()
        touched.append(int((counts[:E] > 0).sum()))
        rows_real.append(int(counts[:E].sum()))
    e_t = float(np.mean(touched))
    p_r = float(np.mean(rows_real))

    # ---- dominant kernel, timed with events on the launch stream.  The calls below reuse
    # moe_forward's own routing and intermediates in the workspace (refreshed before every launch).
    # A decode batch (bf16 weights, a few rows per touched expert, no shared expert) runs its experts
    # as one launch: routed gate/up + SwiGLU, down and the unpermute-reduce.  Otherwise the routed
    # gate/up grouped GEMM dominates.
    P = N * K
    one_launch = not fp8 and Is == 0 and P <= min(8 * E, 512) and H % 128 == 0 and I % 64 == 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    a_off = L["xq"] if fp8 else None
    base = ws.data_ptr()
    for i in range(args.warmup + args.steps):
        dl, w = layers[i % n_layers]
        moe.moe_forward(cfg, w, dl.x, out, ws, stream)  # refreshes ids / offsets / quantised x for this batch
        if i >= args.warmup:
            ev[i - args.warmup][0].record(stream)
        if one_launch:
            moe.moe_experts_forward(cfg, w, dl.x, base + L["topk_ids"], base + L["topk_w"], base + L["offsets"],
                                    base + L["sorted_ids"], base + L["inv_perm"], out, ws, stream)
        else:
            a = dl.x if not fp8 else base + a_off
            a_sc = None if not fp8 else base + L["x_scales"]
            hs = None if not fp8 else base + L["h_scales"]
            moe.moe_grouped_gemm(cfg, moe.MOE_STAGE_GATE_UP, moe.MOE_GROUP_ROUTED, w, a, a_sc,
                                 base + L["sorted_ids"], base + L["offsets"], base + L["h"], hs, ws, stream)
        if i >= args.warmup:
            ev[i - args.warmup][1].record(stream)
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    if one_launch:
        # touched experts' gate, up and down weights, x read, out written (h and y are intermediates)
        k_bytes = e_t * 3 * I * H * wbytes + 2 * N * H * 2
        k_flops = 6.0 * p_r * H * I
        k_name = "routed gate/up + SwiGLU, down, unpermute-reduce (one launch)"
    else:
        # touched experts' gate and up weights (+ block scales), x read, h written
        k_bytes = (e_t * 2 * I * H * wbytes + (e_t * 2 * (I // 128) * (H // 128) * 4 if wl.weight_dtype == "fp8" else 0)
                   + N * H * abytes + p_r * I * abytes)
        k_flops = 4.0 * p_r * H * I
        k_name = "grouped gate/up + SwiGLU (routed)"
    # whole layer
    layer_flops = 2.0 * N * H * R + 6.0 * p_r * H * I + 6.0 * N * H * Is
    layer_bytes_alg = (e_t * 3 * I * H * wbytes + R * H * 2 + 2 * N * H * 2 + 3 * Is * H * wbytes)
    ai = k_flops / k_bytes
    ridge = MFMA_PEAK_TFLOPS[wl.weight_dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": k_bytes / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": k_flops / (k_ms * 1e-3) / 1e12,
                "peak": MFMA_PEAK_TFLOPS[wl.weight_dtype], "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl.name)  # bytes per launch (HBM, counters), or null
    roof["alg_bytes"] = k_bytes
    roof["kernel"] = k_name
    roof["kernel_us"] = k_ms * 1e3

    result = {
        "metric": "MoE-layer tokens/sec (prefill) + decode µs/layer; % of MFMA / HBM peak",
        "value": N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_layer": ms * 1e3,
        "timing": "hip_graph_replay" if use_graph else "eager",
        "ms_per_step_eager": ms_eager,
        "ms_per_step_graph": ms_graph,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.weight_dtype,
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": wl.name, "num_tokens": N, "hidden": H, "num_experts": E, "router_width": R,
                   "top_k": K, "inter": I, "shared_inter": Is, "scoring": wl.scoring,
                   "weight_copies_cycled": n_layers, "experts_touched": e_t, "routed_rows": p_r},
        "layer": {"flops": layer_flops, "alg_bytes": layer_bytes_alg,
                  "hbm_frac": layer_bytes_alg / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                  "mfma_frac": layer_flops / (ms * 1e-3) / (MFMA_PEAK_TFLOPS[wl.weight_dtype] * 1e12)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result))


def cpu_baseline(wl, seconds: float):
    """The oracle as it stands, timed on the host cores on a bounded sample:
    up to 64 tokens of the same layer shape, over 4 weight copies whose touched
    experts are generated (and cached) before the timed runs."""
    from threadpoolctl import threadpool_info

    import moe_inputs as mi
    from oracle import workloads as ow

    n = min(wl.num_tokens, 64)
    sw = wl.with_tokens(n)
    copies = []
    for l in range(4):
        inp, cache = mi.host_inputs(sw, layer=l), {}
        ow.run(sw, layer=l, inputs=inp, expert_cache=cache)  # untimed: fills the expert cache
        copies.append((l, inp, cache))
    done, t_used, runs = 0, 0.0, 0
    while t_used < seconds and runs < 10000:
        l, inp, cache = copies[runs % len(copies)]
        t0 = time.perf_counter()
        ow.run(sw, layer=l, inputs=inp, expert_cache=cache)
        t_used += time.perf_counter() - t0
        done += n
        runs += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": done / t_used, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} oracle runs over {n} tokens of the {wl.name} layer shape (4 weight copies, experts "
                      f"pre-generated), {t_used:.1f} s of host time"}


if __name__ == "__main__":
    main()
