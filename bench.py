"""Benchmark of the MoE layer forward on one MI355X, over the five workloads.

A step is one whole layer forward (router GEMM, scoring + top-K, sort by
expert, grouped gate/up + SwiGLU, grouped down, unpermute-reduce and blends)
over one batch of seeded synthetic tokens, with every input resident in HBM.
Every workload is timed in the same run:

  tiny          16 tokens, H 256, 8 experts, top-2, I 128, shared expert 256
  decode        4 tokens, H 2048, 128 experts, top-8, I 768
  prefill_zipf  4096 tokens of the decode layer, Zipf(1.1)-skewed expert loads
  fp8_sigmoid   2048 tokens, H 7168, 256 fp8 experts, top-8, I 2048, shared 2048,
                sigmoid + correction bias, weights x 2.5
  zero_experts  512 tokens, H 6144, 256 experts + 128 identity experts, top-12, I 2048

One JSON line is printed.  Its headline (`value`, `ms_per_step`, `config`,
`roofline`, `cpu_baseline`) is the prefill layer's tokens/s; `decode_us_per_layer`
names the decode layer's time; `workloads` holds every workload's entry (layer
time, tokens/s, the dominant kernels against their rooflines, the oracle beside
it).  The kernels are timed with HIP events recorded on the stream the library
launches on: for a decode-sized batch the expert half of the layer
(moe_experts_forward: one launch for the routed gate/up, down and reduce),
otherwise the routed gate/up and the routed down grouped GEMMs
(moe_grouped_gemm), each on the layer's own routing.  The oracle (float64 numpy
on the host cores) is timed on a bounded sample of each workload.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 5000.0}  # dense MFMA peaks (mxfp4: e4m3 x e2m1 MFMA)
ORDER = ["tiny", "decode", "prefill_zipf", "fp8_sigmoid", "zero_experts"]
HEADLINE = "prefill_zipf"
# tokens of the oracle's bounded sample per workload: its cost is dominated by the touched experts
CPU_SAMPLE_TOKENS = {"tiny": 16, "decode": 4, "prefill_zipf": 32, "fp8_sigmoid": 2, "zero_experts": 4,
                     "mxfp4_sigmoid": 2}

# HBM traffic of a kernel per launch, from two rocprofv3 --pmc runs of this script per workload
# (`--workload W --steps 5 --warmup 1 --no-cpu-baseline --no-graph` under FETCH_SIZE, then WRITE_SIZE;
# KiB per dispatch, averaged over the dispatches of the timed launch: the kernel's smallest grid, i.e.
# the routed-only launch where the layer's own launch also carries the shared expert), each scaled by
# what the same counter reads for a plain 1 GiB device copy (`--copy-bytes 1073741824 --steps 5`:
# FETCH_SIZE reads half the bytes moved, so x2.0; WRITE_SIZE reads them all, x1.0).  An entry holds only
# while its sources hash to the value they had when the counters were taken; otherwise the traffic is
# reported as null.  The summaries the entries come from are in profiles/.
MEASURED_TRAFFIC = {
    ('tiny', 'experts'): {"kernel": "k_decode_fused", "grid": 128, "dispatches": 26, "fetch_kib": 1107.8, "write_kib": 50.0, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_decode.hip", "mixture_experts_layer_bias_amd/csrc/dma.h", "mixture_experts_layer_bias_amd/csrc/unpermute.h", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "5f0969ff965ac1d5e8a40b7e637adeb726657facc25ead23b2c1b31fe4ee2ab3"},
    ('decode', 'experts'): {"kernel": "k_decode_fused", "grid": 1384, "dispatches": 25, "fetch_kib": 140213.6, "write_kib": 231.0, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_decode.hip", "mixture_experts_layer_bias_amd/csrc/dma.h", "mixture_experts_layer_bias_amd/csrc/unpermute.h", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "5f0969ff965ac1d5e8a40b7e637adeb726657facc25ead23b2c1b31fe4ee2ab3"},
    ('prefill_zipf', 'gate_up'): {"kernel": "k_grouped_gemm_bf16<0, unsigned int>", "grid": 2312, "dispatches": 31, "fetch_kib": 620077.2, "write_kib": 49152.1, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_bf16.hip", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "388072bc0bfe3cf4403ff1fda7838fcc6f7c1628489bfea3c1fdee3664b66d71"},
    ('prefill_zipf', 'down'): {"kernel": "k_grouped_gemm_bf16_persistent<2, unsigned int>", "grid": 512, "dispatches": 31, "fetch_kib": 282820.8, "write_kib": 131074.3, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_bf16.hip", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "388072bc0bfe3cf4403ff1fda7838fcc6f7c1628489bfea3c1fdee3664b66d71"},
    ('zero_experts', 'gate_up'): {"kernel": "k_grouped_gemm_bf16<0, unsigned int>", "grid": 5392, "dispatches": 26, "fetch_kib": 1775895.0, "write_kib": 47390.1, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_bf16.hip", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "388072bc0bfe3cf4403ff1fda7838fcc6f7c1628489bfea3c1fdee3664b66d71"},
    ('zero_experts', 'down'): {"kernel": "k_grouped_gemm_bf16<2, unsigned int>", "grid": 7320, "dispatches": 26, "fetch_kib": 784991.0, "write_kib": 57051.1, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_bf16.hip", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "388072bc0bfe3cf4403ff1fda7838fcc6f7c1628489bfea3c1fdee3664b66d71"},
    ('fp8_sigmoid', 'gate_up'): {"kernel": "k_grouped_gemm_fp8_stream<0>", "grid": 6160, "dispatches": 6, "fetch_kib": 2417893.0, "write_kib": 36083.3, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_fp8.hip", "mixture_experts_layer_bias_amd/csrc/dma.h", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "4880c928a54794c85dea8c89df521a19bc135cbc31f9d68406448607fcdce96e"},
    ('fp8_sigmoid', 'down'): {"kernel": "k_grouped_gemm_fp8_down_persistent", "grid": 256, "dispatches": 26, "fetch_kib": 1211944.4, "write_kib": 229376.0, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_fp8.hip", "mixture_experts_layer_bias_amd/csrc/dma.h", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "4880c928a54794c85dea8c89df521a19bc135cbc31f9d68406448607fcdce96e"},
    ('mxfp4_sigmoid', 'gate_up'): {"kernel": "k_grouped_gemm_mxfp4<0, true>", "grid": 6160, "dispatches": 6, "fetch_kib": 1518118.4, "write_kib": 35707.8, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_mxfp4.hip", "mixture_experts_layer_bias_amd/csrc/dma.h", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "bfd1716498a87e0240a1a00b11aef637c73295b0146ed0916e6684d324128c16"},
    ('mxfp4_sigmoid', 'down'): {"kernel": "k_grouped_gemm_mxfp4_down_persistent", "grid": 512, "dispatches": 26, "fetch_kib": 648870.7, "write_kib": 251756.3, "fetch_scale": 1.9999, "write_scale": 1.0, "sources": ["mixture_experts_layer_bias_amd/csrc/gemm_mxfp4.hip", "mixture_experts_layer_bias_amd/csrc/dma.h", "mixture_experts_layer_bias_amd/csrc/gemm_common.h", "mixture_experts_layer_bias_amd/csrc/common.h", "mixture_experts_layer_bias_amd/csrc/kernels.h"], "sha256": "bfd1716498a87e0240a1a00b11aef637c73295b0146ed0916e6684d324128c16"},
}


def measured_traffic(workload: str, kernel: str):
    """Bytes per launch of a kernel from the stored counter readings, or None."""
    import hashlib

    rec = MEASURED_TRAFFIC.get((workload, kernel))
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default=",".join(ORDER),
                    help="comma-separated workloads to time (tiny, decode, prefill_zipf, fp8_sigmoid, zero_experts, "
                         "mxfp4_sigmoid); the headline is the prefill layer when it is among them")
    ap.add_argument("--workload", default=None, help="time this one workload only (same as --workloads W)")
    ap.add_argument("--layers", type=int, default=0,
                    help="distinct weight copies cycled through (0: enough to exceed the 256 MB MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=4.0, help="target CPU time of each workload's oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes --steps times (the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters), then exit")
    return ap.parse_args()


def host_info() -> dict:
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"nproc": os.cpu_count(), "cpus_available": avail, "cpu_model": model}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every box here has a single MI355X "
              f"and the multi-GPU expert-parallel path is design only.", file=sys.stderr)
        sys.exit(2)
    import torch

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
    names = [args.workload] if args.workload else [w for w in args.workloads.split(",") if w]
    entries = {}
    for name in names:
        print(f"[bench] {name} ...", file=sys.stderr, flush=True)
        entries[name] = measure(name, args)
        torch.cuda.empty_cache()
        print(f"[bench] {name}: {entries[name]['us_per_layer']:.1f} us/layer", file=sys.stderr, flush=True)
    head = HEADLINE if HEADLINE in entries else names[0]
    h = entries[head]
    result = {
        "metric": "MoE-layer tokens/sec (prefill) + decode µs/layer; % of MFMA / HBM peak",
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["us_per_layer"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": h["config"],
        "headline": f"{head}: {h['tokens_per_s']:.4g} tokens/s ({h['us_per_layer']:.1f} us/layer)",
        "decode_us_per_layer": entries["decode"]["us_per_layer"] if "decode" in entries else None,
        "roofline": h["roofline"],
        "after_load": {"us_per_layer": h["us_per_layer_eager_after_load"],
                       "tokens_per_s": h["config"]["num_tokens"] / (h["us_per_layer_eager_after_load"] * 1e-6),
                       "note": "the same steps, eager, timed again after the kernel-timing legs (tens of ms of "
                               "load): outside the clock dip at the onset of sustained load; not the value"},
        "host": host_info(),
        "workloads": entries,
    }
    if "cpu_baseline" in h:
        result["cpu_baseline"] = h["cpu_baseline"]
    print(json.dumps(result))


def one_launch_experts(wl) -> bool:
    """Whether the workload is a decode-sized bf16 batch whose experts the library runs as one launch
    (the routed gate/up, down and the reduce), i.e. what moe_experts_forward times as one kernel."""
    P = wl.num_tokens * wl.top_k
    return (wl.weight_dtype == "bf16" and wl.num_tokens <= 64 and P <= 1024 and P <= min(8 * wl.num_experts, 512)
            and wl.hidden % 256 == 0 and wl.inter % 64 == 0)


def measure(name: str, args) -> dict:
    import numpy as np
    import torch

    import mixture_experts_layer_bias_amd as moe
    import moe_inputs as mi
    import moe_inputs.device as mid

    dev = torch.device("cuda:0")
    wl = mi.WORKLOADS[name]
    N, H, E, R, K, I, Is = (wl.num_tokens, wl.hidden, wl.num_experts, wl.router_width, wl.top_k, wl.inter,
                            wl.shared_inter)
    fp8 = wl.weight_dtype != "bf16"  # fp8 and mxfp4 experts take e4m3 activations
    abytes = 1 if fp8 else 2  # activation and h element bytes
    wbytes = {"bf16": 2, "fp8": 1, "mxfp4": 0.5 + 1 / 32}[wl.weight_dtype]  # mxfp4: codes + E8M0 per 32
    sbytes = (4.0 / (128 * 128)) if wl.weight_dtype == "fp8" else 0.0  # fp8 block scales per weight element
    layer_bytes = 3 * E * I * H * wbytes
    # enough distinct weight copies that the touched experts of consecutive steps cannot be served from
    # the 256 MB Infinity Cache (at least ~8 GB of weights in rotation, at most 8 copies; two copies of
    # the layers whose steps touch gigabytes each)
    n_layers = args.layers or max(2, min(8, int(np.ceil(8.0e9 / layer_bytes))))
    if layer_bytes * n_layers > 60e9:
        n_layers = max(1, int(60e9 // layer_bytes))

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

    # ---- whole-layer timing, eager launches, between a barrier-free pair of device synchronisations
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps

    # ---- the same steps replayed from HIP graphs (one captured moe_forward per weight copy), the way a
    # serving loop runs a decode layer: the launches are the library's own, only host overhead goes away
    ms_graph = None
    if not args.no_graph and N <= 64:
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
        ms_graph = (time.perf_counter() - t0) * 1e3 / args.steps
        del graphs
    # the faster of the two launch modes is reported (named in "timing"); both run the same kernels
    use_graph = ms_graph is not None and ms_graph < ms_eager
    ms = ms_graph if use_graph else ms_eager

    # ---- realised routing per weight copy (for the algorithmic bytes / flops)
    touched, rows_real = [], []
    for l in range(n_layers):
        step(l)
        torch.cuda.synchronize()
        counts = ws[L["counts"]:L["counts"] + 4 * R].view(torch.int32).cpu().numpy()
        touched.append(int((counts[:E] > 0).sum()))
        rows_real.append(int(counts[:E].sum()))
    e_t = float(np.mean(touched))
    p_r = float(np.mean(rows_real))

    # ---- the dominant kernels, timed with events on the launch stream over the same kind of steps.
    # The calls reuse moe_forward's own routing and intermediates in the workspace, refreshed by a
    # moe_forward (outside the events) before every timed launch.
    base = ws.data_ptr()
    one = one_launch_experts(wl)
    if one:
        kinds = ["experts"]
    else:
        kinds = ["gate_up", "down"]

    def launch(kind, w, dl):
        if kind == "experts":
            moe.moe_experts_forward(cfg, w, dl.x, base + L["topk_ids"], base + L["topk_w"], base + L["offsets"],
                                    base + L["sorted_ids"], base + L["inv_perm"], out, ws, stream)
        elif kind == "gate_up":
            a = dl.x if not fp8 else base + L["xq"]
            a_sc = None if not fp8 else base + L["x_scales"]
            hs = None if not fp8 else base + L["h_scales"]
            moe.moe_grouped_gemm(cfg, moe.MOE_STAGE_GATE_UP, moe.MOE_GROUP_ROUTED, w, a, a_sc,
                                 base + L["sorted_ids"], base + L["offsets"], base + L["h"], hs, ws, stream)
        else:
            hs = None if not fp8 else base + L["h_scales"]
            moe.moe_grouped_gemm(cfg, moe.MOE_STAGE_DOWN, moe.MOE_GROUP_ROUTED, w, base + L["h"], hs,
                                 base + L["sorted_ids"], base + L["offsets"], base + L["y"], None, ws, stream)

    k_us = {}
    for kind in kinds:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.warmup + args.steps):
            dl, w = layers[i % n_layers]
            moe.moe_forward(cfg, w, dl.x, out, ws, stream)  # refreshes ids / offsets / quantised x / h
            if i >= args.warmup:
                ev[i - args.warmup][0].record(stream)
            launch(kind, w, dl)
            if i >= args.warmup:
                ev[i - args.warmup][1].record(stream)
        torch.cuda.synchronize()
        k_us[kind] = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3

    # ---- the same eager steps timed once more, after the legs above have kept the GPU busy for tens of
    # milliseconds.  At the onset of sustained load the chip lowers its clocks for some 10-20 ms (every
    # kernel of the layer, the short latency-bound ones too, runs 10-30% longer), and the first window can
    # fall inside that dip.  Reported beside `us_per_layer`, never in its place.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_after = (time.perf_counter() - t0) * 1e3 / args.steps

    # ---- algorithmic bytes and flops (touched experts' weights counted once; h, y intermediates not
    # counted by the one-launch kernel, which never needs them in HBM)
    w_touched = e_t * I * H * (wbytes + sbytes)  # one of the three matrices, all touched experts
    sh_w = Is * H * (wbytes + sbytes)  # one shared matrix
    alg = {
        "experts": (3 * w_touched + 3 * sh_w + 2 * N * H * 2, 6.0 * p_r * H * I + 6.0 * N * H * Is,
                    "routed gate/up + SwiGLU, down, unpermute-reduce (one launch)"
                    + (", shared expert as one more group" if Is else "")),
        "gate_up": (2 * w_touched + N * H * abytes + p_r * I * abytes, 4.0 * p_r * H * I,
                    "routed grouped gate/up + SwiGLU"),
        "down": (w_touched + p_r * I * abytes + p_r * H * 2, 2.0 * p_r * H * I, "routed grouped down"),
    }
    ridge = MFMA_PEAK_TFLOPS[wl.weight_dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)

    def roof(kind):
        b, f, label = alg[kind]
        t = k_us[kind] * 1e-6
        hbm = b / t / 1e9
        mfma = f / t / 1e12
        if f / b < ridge:
            r = {"bound": "hbm", "achieved": hbm, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        else:
            r = {"bound": "mfma", "achieved": mfma, "peak": MFMA_PEAK_TFLOPS[wl.weight_dtype], "unit": "TFLOP/s"}
        r["frac"] = r["achieved"] / r["peak"]
        r["traffic"] = measured_traffic(name, kind)
        r.update({"kernel": label, "kernel_us": k_us[kind], "alg_bytes": b, "alg_flops": f,
                  "hbm_frac": hbm / HBM_PEAK_GBS, "mfma_frac": mfma / MFMA_PEAK_TFLOPS[wl.weight_dtype]})
        return r

    rooflines = {k: roof(k) for k in kinds}
    dominant = max(kinds, key=lambda k: k_us[k])
    layer_flops = 2.0 * N * H * R + 6.0 * p_r * H * I + 6.0 * N * H * Is
    layer_bytes_alg = 3 * w_touched + R * H * 2 + 2 * N * H * 2 + 3 * sh_w
    t_star = max(layer_flops / (MFMA_PEAK_TFLOPS[wl.weight_dtype] * 1e12), layer_bytes_alg / (HBM_PEAK_GBS * 1e9))
    entry = {
        "us_per_layer": ms * 1e3,
        "tokens_per_s": N / (ms * 1e-3),
        "timing": "hip_graph_replay" if use_graph else "eager",
        "us_per_layer_eager": ms_eager * 1e3,
        "us_per_layer_graph": None if ms_graph is None else ms_graph * 1e3,
        "us_per_layer_eager_after_load": ms_after * 1e3,
        "dtype": wl.weight_dtype,
        "config": {"workload": wl.name, "num_tokens": N, "hidden": H, "num_experts": E, "router_width": R,
                   "top_k": K, "inter": I, "shared_inter": Is, "scoring": wl.scoring,
                   "weight_copies_cycled": n_layers, "experts_touched": e_t, "routed_rows": p_r},
        "layer": {"flops": layer_flops, "alg_bytes": layer_bytes_alg, "t_star_us": t_star * 1e6,
                  "roofline_frac": t_star / (ms * 1e-3),
                  "hbm_frac": layer_bytes_alg / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                  "mfma_frac": layer_flops / (ms * 1e-3) / (MFMA_PEAK_TFLOPS[wl.weight_dtype] * 1e12)},
        "roofline": rooflines[dominant],
        "kernels": rooflines,
    }
    del layers, ws, out
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        entry["cpu_baseline"] = cpu_baseline(name, wl, args.cpu_seconds)
    return entry


def cpu_baseline(name: str, wl, seconds: float):
    """The oracle as it stands, timed on the host cores on a bounded sample: the first few tokens of
    the same layer shape (one weight copy), whose touched experts are generated (and cached) before
    the timed runs; runs repeat until about `seconds` of host time are spent."""
    from threadpoolctl import threadpool_info

    import moe_inputs as mi
    from oracle import workloads as ow

    n = min(wl.num_tokens, CPU_SAMPLE_TOKENS.get(name, 4))
    sw = wl.with_tokens(n)
    inp, cache = mi.host_inputs(sw), {}
    ow.run(sw, inputs=inp, expert_cache=cache)  # untimed: fills the expert cache
    done, t_used, runs = 0, 0.0, 0
    while (t_used < seconds or runs == 0) and runs < 10000:
        t0 = time.perf_counter()
        ow.run(sw, inputs=inp, expert_cache=cache)
        t_used += time.perf_counter() - t0
        done += n
        runs += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": done / t_used, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} oracle runs over the first {n} tokens of the {wl.name} layer (experts touched by "
                      f"them generated beforehand), {t_used:.1f} s of host time; the BLAS pool's threads are the "
                      f"cores counted"}


if __name__ == "__main__":
    main()
