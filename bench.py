#!/usr/bin/env python3
"""Benchmark of one MI355X's share of the FP8 routed-expert MoE layer.

A step is one pass of the whole hot path over one batch of routed rows:
count / prefix-sum / stable-rank / permute (moe_dispatch_layout), FP8 grouped
GEMM gate/up, SiLU-mul-requant, FP8 grouped GEMM down, weighted combine.
Default workload: the prefill share of an EP32 deployment at 4K context (9
local experts of a 288-expert pool, H=7168, I=2048, 65,536 source tokens,
top-8, 131,040 routed rows, contiguous layout).  Inputs are synthetic
(seeded), quantised on the device by the library's own quantiser and
resident in HBM before timing starts.

Prints one JSON line: MoE-layer FP8 TFLOP/s (value), token-rows/s, the
fraction of the FP8 MFMA peak, per-kernel times, the roofline of the dominant
kernel (GEMM1, events on the launch stream) and the CPU oracle timed on a
bounded sample of the same workload.

Other workloads (--config 1-5) are the decode shares; --graph replays the
step from one hipGraph (the decode mode), and --flush-mib writes a scratch
buffer between steps, outside the timed span, so that weights are streamed
from HBM rather than found in the memory-side cache.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE-layer FP8 TFLOP/s + % of MFMA peak; routed token-rows/s per GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm1_act_ep32_prefill_traffic.json")
GEMM_SRC = os.path.join(ROOT, "fp8_routed_expert_amd", "csrc", "gemm.hip")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def gemm_source_hash():
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]


def stored_traffic(launch_key):
    """HBM bytes per launch of the fused gate/up + activation kernel from the
    committed rocprofv3 --pmc summary, or None when that summary is absent or
    was taken on another kernel or workload."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha") != gemm_source_hash() or rec.get("launch") != launch_key:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, idx, w, n_tokens):
    """Time the CPU oracle (as it stands) on a seeded sample of source tokens.

    The sample's activations and all experts' weights are quantised by the
    oracle itself (untimed); the timed call is the oracle's layer: the layout
    over all tokens and the float stages for the sampled tokens' rows."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_info
    from oracle import moe
    from workloads import activations, weights, bf16_to_f32

    g = np.random.default_rng([0, cfg.cid, 99])
    toks = np.sort(g.choice(cfg.T, size=min(n_tokens, cfg.T), replace=False))
    xb = activations(cfg)
    x = np.zeros((cfg.T, cfg.H), np.uint8)
    xs = np.ones((cfg.T, cfg.H // 128), np.float32)
    x[toks], xs[toks] = moe.quantize_blocks(bf16_to_f32(xb[toks]), 1)
    E = cfg.E
    w13 = np.empty((E, 2 * cfg.I, cfg.H), np.uint8)
    s13 = np.empty((E, 2 * cfg.I // 128, cfg.H // 128), np.float32)
    w2 = np.empty((E, cfg.H, cfg.I), np.uint8)
    s2 = np.empty((E, cfg.H // 128, cfg.I // 128), np.float32)

    def qe(e):
        a, b = weights(cfg, experts=[e])
        w13[e], s13[e] = moe.quantize_blocks(bf16_to_f32(a[0]), 128)
        w2[e], s2[e] = moe.quantize_blocks(bf16_to_f32(b[0]), 128)
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(qe, range(E)))
    rows = int((idx >= 0).sum()) + E * (cfg.align_m - 1)
    kw = dict(capacity=cfg.capacity) if cfg.layout == moe.LAYOUT_MASKED else \
        dict(align_m=cfg.align_m, rows=rows)
    stages = {}
    t0 = time.perf_counter()
    res = moe.layer(x, xs, idx, w, w13, s13, w2, s2, cfg.layout, tokens=toks,
                    stage_seconds=stages, **kw)
    dt = time.perf_counter() - t0
    n_rows = len(res["slots"])
    flops = 2 * n_rows * (2 * cfg.I) * cfg.H + 2 * n_rows * cfg.H * cfg.I
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "kind": "oracle",
            "sample": f"{len(toks)} of {cfg.T} source tokens ({n_rows} routed rows), seeded; "
                      f"layout over all tokens; fp64 numpy, BLAS threads={threads}",
            "seconds": round(dt, 3), "rows_per_s": n_rows / dt,
            "stage_seconds": {k: round(v, 3) for k, v in stages.items()}}


def measure_ceilings(dev, reps=5):
    """What this GPU sustains, measured now with the library's helpers: a
    plain 1 GiB device copy (2 GiB of HBM traffic) and a register-only chain
    of the GEMMs' FP8 MFMA instruction.  Best of `reps` launches each."""
    import torch
    import fp8_routed_expert_amd as fre
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    sink = torch.zeros(2048, dtype=torch.float32, device=dev)

    def best(fn):
        fn()                                   # warm-up
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts), out
    t_copy, _ = best(lambda: fre.moe_ceiling_copy(src, dst))
    t_mfma, flops = best(lambda: fre.moe_ceiling_mfma_fp8(2048, 2000, sink))
    del src, dst
    return {"hbm_copy_gbs": round(2 * n / (t_copy * 1e-3) / 1e9, 1),
            "fp8_mfma_tflops": round(flops / (t_mfma * 1e-3) / 1e12, 1),
            "source": "measured in this run: moe_ceiling_copy (1 GiB device copy, read + "
                      "write counted) and moe_ceiling_mfma_fp8 (register-only E4M3 "
                      "16x16x128 MFMA chain), best of 5"}


def bench_dense(args, M, N, K):
    """Dense block-scaled FP8 GEMM: c[M, N] = A[M, K] W[N, K]^T with 1x128
    activation and 128x128 weight scales.  Operands are seeded N(0, 1) and
    N(0, 0.02) bf16 values quantised on the device."""
    import numpy as np
    import torch
    import fp8_routed_expert_amd as fre
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    xb = torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)
    wb = (torch.randn(N, K, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    a = torch.empty(M, K, dtype=torch.uint8, device=dev)
    sa_rows = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    w = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sw = torch.empty(N // 128, K // 128, dtype=torch.float32, device=dev)
    fre.moe_quantize_fp8(xb, 1, a, sa_rows)
    fre.moe_quantize_fp8(wb, 128, w, sw)
    sa = sa_rows.t().contiguous()           # K-block-major
    del xb, wb, sa_rows
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        fre.moe_gemm_fp8(a, sa, w, sw, c)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        fre.moe_gemm_fp8(a, sa, w, sw, c)
        e1.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kern_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    flops = 2.0 * M * N * K
    nbytes = M * K + M * (K // 128) * 4 + N * K + (N // 128) * (K // 128) * 4 + M * N * 2
    tf = flops / (kern_ms * 1e-3) / 1e12
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    mfma = flops / nbytes >= FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return {
        "metric": "dense block-scaled FP8 GEMM TFLOP/s", "value": round(tf, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": f"dense gemm M={M} N={N} K={K}, 1x128 / 128x128 scales",
                   "M": M, "N": N, "K": K},
        "roofline": ({"kernel": "grouped_gemm_fp8 (dense)", "bound": "mfma",
                      "achieved": round(tf, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(tf / FP8_PEAK_TFLOPS, 4), "traffic": None} if mfma else
                     {"kernel": "grouped_gemm_fp8 (dense)", "bound": "hbm",
                      "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="workload id (1-5)")
    ap.add_argument("--cpu-tokens", type=int, default=6144,
                    help="source tokens in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step's launches in one hipGraph and time replays")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="write a scratch buffer of this many MiB before every timed step "
                         "(outside the timed span) to evict the memory-side cache")
    ap.add_argument("--scales", choices=("fp32", "e8m0"), default="fp32",
                    help="block-scale format: fp32 (default) or packed power-of-two "
                         "exponents applied by the matrix cores")
    ap.add_argument("--dense", type=int, nargs=3, metavar=("M", "N", "K"), default=None,
                    help="time the dense FP8 GEMM (moe_gemm_fp8) at this shape instead "
                         "of the layer")
    ap.add_argument("--unfused", action="store_true",
                    help="run the gate/up GEMM and the activation as two calls "
                         "(default: the layer's choice)")
    ap.add_argument("--fused", action="store_true",
                    help="run the gate/up GEMM with the activation fused (one call)")
    ap.add_argument("--zipf", type=float, default=1.0,
                    help="Zipf exponent of the per-expert load (the EP48 decode share, "
                         "--config 3); 1.0 is the workload's, 0.613 gives hottest = 3x coldest")
    ap.add_argument("--no-gather", action="store_true",
                    help="copy the routed rows into the permuted buffer in the dispatch "
                         "(default: the gate/up GEMM gathers them from x in its tile loads)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip measuring the copy and MFMA ceilings")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first "
                         "(reference for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the expert-parallel layer and "
              "runs on a single GPU only (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import fp8_routed_expert_amd as fre
    from workloads import CONFIGS, routing, activations, weights

    dev = torch.device("cuda:0")
    if args.dense:
        print(json.dumps(bench_dense(args, *args.dense)), flush=True)
        return
    cfg = CONFIGS[args.config]
    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceil = None if args.no_ceilings else measure_ceilings(dev)
    if ceil:
        log(f"ceilings: copy {ceil['hbm_copy_gbs']} GB/s, FP8 MFMA {ceil['fp8_mfma_tflops']} TF/s")
    log(f"workload {cfg.name}: E={cfg.E} H={cfg.H} I={cfg.I} T={cfg.T} K={cfg.K}")
    if args.zipf != 1.0 and args.config != 3:
        raise SystemExit("--zipf applies to --config 3 only")
    idx, w = routing(cfg, zipf_s=args.zipf)
    R = int((idx >= 0).sum())
    xb = activations(cfg)
    w13b, w2b = weights(cfg)
    log(f"generated inputs ({R} routed rows)")

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    E, H, I, T, K = cfg.E, cfg.H, cfg.I, cfg.T, cfg.K
    x = torch.empty(T, H, dtype=torch.uint8, device=dev)
    w13 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device=dev)
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device=dev)
    if args.scales == "e8m0":
        hw, iw = (H // 128 + 3) // 4, (I // 128 + 3) // 4
        xs = torch.empty(T, hw, dtype=torch.int32, device=dev)
        s13 = torch.empty(E, 2 * I // 128, hw, dtype=torch.int32, device=dev)
        s2 = torch.empty(E, H // 128, iw, dtype=torch.int32, device=dev)
        quant = fre.moe_quantize_fp8_e8m0
    else:
        xs = torch.empty(T, H // 128, dtype=torch.float32, device=dev)
        s13 = torch.empty(E, 2 * I // 128, H // 128, dtype=torch.float32, device=dev)
        s2 = torch.empty(E, H // 128, I // 128, dtype=torch.float32, device=dev)
        quant = fre.moe_quantize_fp8
    quant(bf(xb), 1, x, xs)
    quant(bf(w13b), 128, w13, s13)
    quant(bf(w2b), 128, w2, s2)
    del xb, w13b, w2b
    idx_d = torch.from_numpy(idx).to(dev)
    w_d = torch.from_numpy(w).to(dev)
    rows = cfg.capacity if cfg.layout == fre.LAYOUT_MASKED else fre.contiguous_rows(R, E, cfg.align_m)
    layer = fre.MoELayer(E, H, I, T, K, cfg.layout, rows, align_m=cfg.align_m, device=dev,
                         scale_fmt=args.scales, fuse_act=False if args.unfused else (True if args.fused else "auto"),
                         gather=not args.no_gather)
    fused = layer.fuse_act
    torch.cuda.synchronize()

    if fused:
        names = ["dispatch_layout", "gemm1_gate_up_act", "gemm2_down", "combine"]
        stages = [lambda: layer.dispatch(idx_d, x, xs), lambda: layer.gemm1_act(w13, s13),
                  lambda: layer.gemm2(w2, s2), lambda: layer.combine(w_d)]
    else:
        names = ["dispatch_layout", "gemm1_gate_up", "act_requant", "gemm2_down", "combine"]
        stages = [lambda: layer.dispatch(idx_d, x, xs), lambda: layer.gemm1(w13, s13),
                  lambda: layer.act(), lambda: layer.gemm2(w2, s2), lambda: layer.combine(w_d)]
    n_ev = len(stages) + 1

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        for i, f in enumerate(stages):
            f()
            if evs is not None:
                evs[i + 1].record()

    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()                      # untimed launch on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    def run_step(evs=None):
        if graph is None:
            step(evs)
            return
        if evs is not None:
            evs[0].record()
        graph.replay()
        if evs is not None:
            evs[-1].record()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    st = int(layer.status.item())
    if st != 0:
        raise RuntimeError(f"device status word {st} after warm-up")

    warm_ms = None
    scratch = None
    if args.flush_mib:
        # the same steps without the flush first: the memory-side cache then
        # holds what the previous step left (reported next to the flushed run)
        wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in wev:
            e0.record()
            run_step()
            e1.record()
        torch.cuda.synchronize()
        warm_ms = [e0.elapsed_time(e1) for e0, e1 in wev]
        scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if scratch is not None:
            scratch.fill_(k & 0xff)     # outside the events of step k
        run_step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = [events[k][0].elapsed_time(events[k][n_ev - 1]) for k in range(args.steps)]
    # wall clock over exactly K steps, unless flushes sit between them: then
    # the sum of the steps' own event spans
    ms = (t1 - t0) * 1e3 / args.steps if scratch is None else float(np.mean(step_ms))
    per = None
    if graph is None:
        per = {n: float(np.mean([events[k][i].elapsed_time(events[k][i + 1])
                                 for k in range(args.steps)])) for i, n in enumerate(names)}

    flops1 = 2.0 * R * (2 * I) * H
    flops2 = 2.0 * R * H * I
    flops = flops1 + flops2
    hb, ib = H // 128, I // 128
    # dispatch: x read once and the routed rows written once (unless the
    # gate/up GEMM gathers them), scales the same way, routing read
    bytes_perm = (T + R) * 4 * hb + T * K * 4 + (0 if layer.gather else (T + R) * H)
    bytes_act = R * (4 * I + I + 4 * ib)
    bytes_comb = R * 2 * H + T * 2 * H + T * K * 8
    # GEMM bytes: weights (and scales) of experts with rows, A and its scales, C
    live = int(np.count_nonzero(np.bincount(idx[idx >= 0], minlength=E)))
    # gate/up: writes h (bf16), or with the activation fused q2 and its scales
    bytes_g1 = (live * (2 * I * H + (2 * I // 128) * hb * 4) + R * (H + 4 * hb) +
                (R * (I + 4 * ib) if fused else R * 2 * I * 2))
    bytes_g2 = live * (H * I + hb * ib * 4) + R * (I + 4 * ib) + R * H * 2
    tflops = flops / (ms * 1e-3) / 1e12
    launch_key = f"{cfg.name}:R={R}:rows={rows}" + (":gather" if layer.gather else "")
    traffic = stored_traffic(launch_key) if args.scales == "fp32" and fused else None
    kname = "gate/up GEMM + activation (fused)" if fused else "grouped_gemm_fp8 (gate/up)"
    pct = lambda q: round(float(np.percentile(step_ms, q)), 4)
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {E} local experts, H={H}, I={I}, "
                               f"{T} source tokens, top-{K}, {R} routed rows, "
                               f"{'masked' if cfg.layout else 'contiguous'} layout",
                   "experts": E, "hidden": H, "intermediate": I, "tokens": T,
                   "topk": K, "routed_rows": R, "buffer_rows": layer.rows_total,
                   **({"zipf_s": args.zipf} if args.config == 3 else {}),
                   "experts_with_rows": live, "block_scales": args.scales,
                   "gate_up_activation": "fused" if fused else "separate calls",
                   "row_permutation": ("gathered by the gate/up GEMM's tile loads (x[row_src])"
                                       if layer.gather else "copied by the dispatch")},
        "timing": {"mode": "hipgraph replay" if graph is not None else "eager launches",
                   "cache_flush_mib": args.flush_mib,
                   "step_ms_p10": pct(10), "step_ms_p50": pct(50), "step_ms_p90": pct(90),
                   **({"warm_step_ms_p10": round(float(np.percentile(warm_ms, 10)), 4),
                       "warm_step_ms_p50": round(float(np.percentile(warm_ms, 50)), 4),
                       "warm_step_ms_p90": round(float(np.percentile(warm_ms, 90)), 4)}
                      if warm_ms is not None else {})},
        "mfma_peak_frac": round(tflops / FP8_PEAK_TFLOPS, 4),
        "token_rows_per_s": round(R / (ms * 1e-3), 1),
    }
    # the step's roofline: each stage at the slower of its two bounds (its
    # flops at the FP8 MFMA peak, its algorithmic bytes at the HBM peak)
    work = {"dispatch_layout": (0.0, bytes_perm), names[1]: (flops1, bytes_g1),
            "gemm2_down": (flops2, bytes_g2), "combine": (0.0, bytes_comb)}
    if not fused:
        work["act_requant"] = (0.0, bytes_act)
    bound_ms = {n: 1e3 * max(f / (FP8_PEAK_TFLOPS * 1e12), b / (HBM_PEAK_GBS * 1e9))
                for n, (f, b) in work.items()}
    att = sum(bound_ms.values())
    result["attainable"] = {"step_ms": round(att, 4), "frac": round(att / ms, 4),
                            "per_kernel_ms": {n: round(bound_ms[n], 4) for n in names}}
    if per is not None:
        result["attainable"]["per_kernel_frac"] = {
            n: round(bound_ms[n] / per[n], 4) for n in names}
        t1 = per[names[1]]
        g1 = flops1 / (t1 * 1e-3) / 1e12
        g1_gbs = bytes_g1 / (t1 * 1e-3) / 1e9
        result["per_kernel_ms"] = {k: round(v, 4) for k, v in per.items()}
        result["per_kernel_rate"] = {
            "gemm1_tflops": round(g1, 1),
            "gemm1_gbs": round(g1_gbs, 1),
            "gemm2_tflops": round(flops2 / (per["gemm2_down"] * 1e-3) / 1e12, 1),
            "gemm2_gbs": round(bytes_g2 / (per["gemm2_down"] * 1e-3) / 1e9, 1),
            "dispatch_gbs": round(bytes_perm / (per["dispatch_layout"] * 1e-3) / 1e9, 1),
            "combine_gbs": round(bytes_comb / (per["combine"] * 1e-3) / 1e9, 1),
        }
        if not fused:
            result["per_kernel_rate"]["act_gbs"] = round(
                bytes_act / (per["act_requant"] * 1e-3) / 1e9, 1)
        # GEMM1 dominates every workload; below the ridge point (peak flop/s over
        # peak bytes/s) its bound is weight streaming from HBM
        ridge = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        tsrc = ("stored: rocprofv3 --pmc FETCH_SIZE + WRITE_SIZE of this kernel source and "
                "launch, scaled by a 1 GiB copy (" + os.path.relpath(TRAFFIC_FILE, ROOT) + ")"
                if traffic is not None else
                "none: no counter record for this kernel source and launch")
        if flops1 / bytes_g1 >= ridge:
            result["roofline"] = {"kernel": kname, "bound": "mfma",
                                  "achieved": round(g1, 2), "peak": FP8_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(g1 / FP8_PEAK_TFLOPS, 4),
                                  "traffic": traffic, "traffic_source": tsrc}
        else:
            result["roofline"] = {"kernel": kname, "bound": "hbm",
                                  "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(g1_gbs / HBM_PEAK_GBS, 4),
                                  "traffic": traffic, "traffic_source": tsrc}
        if ceil:
            r = result["per_kernel_rate"]
            fr = {"gemm1": round(r["gemm1_tflops"] / ceil["fp8_mfma_tflops"], 4)
                  if flops1 / bytes_g1 >= ridge else
                  round(r["gemm1_gbs"] / ceil["hbm_copy_gbs"], 4),
                  "gemm2": round(r["gemm2_tflops"] / ceil["fp8_mfma_tflops"], 4)
                  if flops2 / bytes_g2 >= ridge else
                  round(r["gemm2_gbs"] / ceil["hbm_copy_gbs"], 4),
                  "dispatch": round(r["dispatch_gbs"] / ceil["hbm_copy_gbs"], 4),
                  "combine": round(r["combine_gbs"] / ceil["hbm_copy_gbs"], 4)}
            if "act_gbs" in r:
                fr["act"] = round(r["act_gbs"] / ceil["hbm_copy_gbs"], 4)
            result["ceiling_frac"] = fr
    if ceil:
        result["ceilings"] = ceil
    if not args.no_cpu_baseline and args.scales == "fp32":
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(cfg, idx, w, args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
