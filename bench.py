"""Benchmark of the NVFP4 MoE expert-FFN layer on one MI355X.

One step = one full layer forward (quantize x, route, L1 grouped GEMM with the
SiLU*up epilogue, re-quantize h, L2 grouped GEMM, weighted scatter) over one
batch of synthetic input already resident in HBM.

Default workload: the prefill-shaped shard (8192 tokens, top-8 of 384 experts,
this GPU's 48 local experts 96..143, hidden 7168, intermediate 3072, uniform
router logits). The decode-shaped shard (64 tokens, same weights) is measured
alongside. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config prefill|decode|skewed]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + grouped-GEMM TFLOPS & HBM GB/s (% of roofline), 1 GPU"
PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense fp4 MFMA (not usable for block-16 E4M3 scales)
PEAK_HBM_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
COPY_CAL_BYTES = 1 << 30      # bytes read (and written) by the calibration copy


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of grouped_gemm.hip's code: // comments, trailing blanks and blank
    lines removed, so that a comment edit keeps the measured traffic valid."""
    p = os.path.join(ROOT, "nvfp4_quantized_moe_amd", "csrc", "grouped_gemm.hip")
    code = []
    for line in open(p, encoding="utf-8"):
        line = line.split("//", 1)[0].rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def read_traffic(workload: str):
    """Per-launch HBM bytes of the L1 GEMM from the committed counter summary,
    or None when absent or taken on a different kernel source."""
    p = os.path.join(PROFILE_DIR, f"l1_gemm_{workload}_traffic.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    return float(kv["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="prefill", choices=["prefill", "decode", "skewed", "quantize"],
                    help="headline workload (quantize: only with --summarize-trace of a --quantize-only run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed GPU time spent on the workload before the warmup steps, so that "
                         "the clocks leave their start-of-load transient (steady state is timed)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (elementwise negate) three times, "
                         "so that counter runs can scale FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the per-launch HBM traffic of the L1 GEMM from two rocprofv3 --pmc "
                         "csv runs (FETCH_SIZE, WRITE_SIZE) to profiles/ and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write the per-kernel table of a rocprofv3 --kernel-trace --stats csv run to "
                         "profiles/ and exit")
    ap.add_argument("--trace-all", action="store_true",
                    help="with --summarize-trace: the trace is of the whole default run (no --no-decode)")
    ap.add_argument("--quantize-only", action="store_true",
                    help="time only the activation quantizer on the 4096 x 7168 tensor and print its object "
                         "(for a kernel trace of the quantizer alone); not the benchmark line")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="write the MFMA counters of the L1 GEMM from a rocprofv3 --pmc csv run to "
                         "profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.config, *args.summarize_traffic)
        return
    if args.summarize_trace:
        summarize_trace(args.config, args.summarize_trace, args.trace_all)
        return
    if args.summarize_mfma:
        summarize_mfma(args.config, args.summarize_mfma)
        return
    if args.config == "quantize" and not args.quantize_only:
        raise SystemExit("bench.py: --config quantize only names the trace of a --quantize-only run")
    if args.gpus != 1:
        print(f"bench.py: the layer runs one rank's share of the experts on one GPU; --gpus {args.gpus} is not "
              f"supported (expert-parallel sharding across GPUs and its all-reduce are not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_quantized_moe_amd as nv
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.quantize_only:
        print(json.dumps({"quantize": quantize_c1(nv, W, dev, args.settle_ms)}), flush=True)
        return
    cfg = W.get_config(args.config)
    t0 = time.time()
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    log(f"generated {cfg.name} inputs in {time.time() - t0:.1f}s")

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    weights = nv.prepare_weights(bf16(wg), bf16(wu), bf16(wd))
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def run_layer(cfg_, ids_, w_, x_, steps, warmup):
        T, k = ids_.shape
        d_x, d_ids, d_w = bf16(x_), torch.from_numpy(ids_).to(dev), torch.from_numpy(w_).to(dev)
        out = torch.empty((T, cfg_.hidden), dtype=torch.bfloat16, device=dev)
        lay = nv.nvfp4_moe_ws_layout(T, k, cfg_.hidden, cfg_.inter, cfg_.num_local)
        ws = torch.empty(lay["end"], dtype=torch.uint8, device=dev)

        def step():
            nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, cfg_.expert_start, out=out, ws=ws)

        settle(step, args.settle_ms)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t) * 1e3 / steps
        # the dominant kernel, L1 grouped GEMM, timed alone on the stream it is launched on
        cap = T * k
        S = int(nv.ws_view(ws, lay, "offsets", torch.int32, (cfg_.num_local + 1,))[-1].item())
        counts = nv.ws_view(ws, lay, "counts", torch.int32, (cfg_.num_local,)).cpu().numpy()
        tile_m = nv.nvfp4_moe_tile_m(T, k, cfg_.num_local)
        gargs = (nv.ws_view(ws, lay, "x_q", torch.uint8, (T, cfg_.hidden // 2)),
                 nv.ws_view(ws, lay, "x_sf", torch.uint8, (T, cfg_.hidden // 16)),
                 nv.ws_view(ws, lay, "slot_token", torch.int32, (cap,)),
                 nv.ws_view(ws, lay, "scalars", torch.float32, (4,))[0:1],
                 weights.w1, weights.w1_gs,
                 nv.ws_view(ws, lay, "offsets", torch.int32, (cfg_.num_local + 1,)),
                 nv.ws_view(ws, lay, "tiles", torch.int32, (nv.nvfp4_tile_table_len(cap, cfg_.num_local, tile_m),)))
        h = torch.empty((cap, cfg_.inter), dtype=torch.bfloat16, device=dev)
        amax = torch.zeros(1, dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_l1 = max(steps, 5)
        settle(lambda: nv.nvfp4_grouped_gemm(*gargs, cap, tile_m, nv.EPI_SILU_MUL, d=h, amax_out=amax),
               args.settle_ms / 2)
        ev0.record(stream)
        for _ in range(n_l1):
            nv.nvfp4_grouped_gemm(*gargs, cap, tile_m, nv.EPI_SILU_MUL, d=h, amax_out=amax)
        ev1.record(stream)
        torch.cuda.synchronize()
        l1_ms = ev0.elapsed_time(ev1) / n_l1
        return dict(ms=ms, S=S, touched=int((counts > 0).sum()), l1_ms=l1_ms, tile_m=tile_m, out=out)

    log(f"timing {cfg.name}: {args.warmup} warmup + {args.steps} steps")
    r = run_layer(cfg, ids, w, x, args.steps, args.warmup)
    T, k, H, I = cfg.tokens, cfg.top_k, cfg.hidden, cfg.inter
    S = r["S"]
    tok_s = T / (r["ms"] * 1e-3)
    l1_flop = S * 2.0 * (2 * I) * H                       # per slot: 2 * 2I * H (88.08 MFLOP)
    layer_flop = S * 2.0 * (2 * I * H + H * I)            # per slot: 132.12 MFLOP
    l1_tflops = l1_flop / (r["l1_ms"] * 1e-3) / 1e12
    l1_w_bytes = r["touched"] * 2 * I * (H // 2 + H // 16)  # FP4 weights + scales of touched experts
    traffic = read_traffic(cfg.name)
    roofline = {
        "kernel": "grouped_gemm L1 (gate+up, SiLU*up epilogue)",
        "bound": "mfma", "achieved": round(l1_tflops, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(l1_tflops / PEAK_FP16_TFLOPS, 4), "traffic": traffic,
        "avg_launch_ms": round(r["l1_ms"], 4), "flop_per_launch": l1_flop,
        "frac_of_fp4_peak": round(l1_tflops / PEAK_FP4_TFLOPS, 4),
    }
    if cfg.name == "decode":
        gbs = l1_w_bytes / (r["l1_ms"] * 1e-3) / 1e9
        roofline.update(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(gbs / PEAK_HBM_GBS, 4), bytes_per_launch=l1_w_bytes)
    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic (seeded NumPy draws, random-init weights)",
        "config": {"workload": f"{cfg.name} shard: T={T}, top-{k} of {cfg.num_global} experts, local "
                               f"{cfg.expert_start}..{cfg.expert_start + cfg.num_local - 1}, H={H}, I={I}",
                   "tokens": T, "top_k": k, "local_experts": cfg.num_local, "hidden": H, "inter": I,
                   "slots": S, "touched_experts": r["touched"], "tile_m": r["tile_m"]},
        "layer_tflops": round(layer_flop / (r["ms"] * 1e-3) / 1e12, 2),
        "roofline": roofline,
    }
    if cfg.name == "prefill" and not args.no_decode:
        dcfg = W.get_config("decode")
        dids, dw = W.make_router(dcfg)
        dx = W.make_activations(dcfg)
        rd = run_layer(dcfg, dids, dw, dx, max(args.steps, 50), args.warmup)
        bytes_w = rd["touched"] * (2 * I * (H // 2 + H // 16) + H * (I // 2 + I // 16))
        gbs = bytes_w / (rd["ms"] * 1e-3) / 1e9
        l1b = rd["touched"] * 2 * I * (H // 2 + H // 16)
        l1g = l1b / (rd["l1_ms"] * 1e-3) / 1e9
        result["decode"] = {
            "workload": "decode shard: T=64, top-8 of 384, local 96..143, same weights",
            "tokens_per_s": round(dcfg.tokens / (rd["ms"] * 1e-3), 1), "ms_per_step": round(rd["ms"], 4),
            "touched_experts": rd["touched"], "slots": rd["S"],
            "layer_weight_GBs": round(gbs, 1), "layer_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "l1_gemm_ms": round(rd["l1_ms"], 4), "l1_gemm_GBs": round(l1g, 1),
            "l1_gemm_hbm_frac": round(l1g / PEAK_HBM_GBS, 4),
        }
    if cfg.name == "prefill" and not args.no_decode:
        result["decode"]["flushed"] = decode_flushed(nv, weights, W.get_config("decode"), dev)
        result["decode"]["graph"] = decode_graph(nv, weights, W.get_config("decode"), dev, max(args.steps, 50))
        result["quantize"] = quantize_c1(nv, W, dev, args.settle_ms)
        result["skewed"] = skewed_shard(nv, W, dev, args.settle_ms, max(args.steps, 10))
        result["static_scales"] = static_scales(nv, weights, W, dev, args.settle_ms)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, ids, w, x, wg, wu, wd, T)
    print(json.dumps(result), flush=True)


def decode_flushed(nv, weights, dcfg, dev, steps=30):
    """Decode shard with the last-level cache (256 MB) flushed before every step:
    each step timed alone with events, after a 512 MB read outside the events."""
    import torch
    import workloads as W
    ids, w = W.make_router(dcfg)
    x = W.make_activations(dcfg)
    T, k = ids.shape
    d_x = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    d_ids, d_w = torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    lay = nv.nvfp4_moe_ws_layout(T, k, dcfg.hidden, dcfg.inter, dcfg.num_local)
    ws = torch.empty(lay["end"], dtype=torch.uint8, device=dev)
    out = torch.empty((T, dcfg.hidden), dtype=torch.bfloat16, device=dev)
    scratch = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    # flush (a 512 MB read, which leaves no dirty lines to write back), then the
    # step between two events, all enqueued without host waits, so the host's
    # launch latency is not inside the events
    evs = []
    for i in range(steps + 3):
        torch.sum(scratch, dim=0, out=sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, dcfg.expert_start, out=out, ws=ws)
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs[3:]]
    counts = nv.ws_view(ws, lay, "counts", torch.int32, (dcfg.num_local,)).cpu().numpy()
    touched = int((counts > 0).sum())
    H, I = dcfg.hidden, dcfg.inter
    bytes_w = touched * (2 * I * (H // 2 + H // 16) + H * (I // 2 + I // 16))
    med = float(np.median(times))
    return {"ms_per_step_median": round(med, 4), "ms_p10": round(float(np.percentile(times, 10)), 4),
            "ms_p90": round(float(np.percentile(times, 90)), 4),
            "tokens_per_s": round(T / (med * 1e-3), 1),
            "layer_weight_GBs": round(bytes_w / (med * 1e-3) / 1e9, 1),
            "layer_hbm_frac": round(bytes_w / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def decode_graph(nv, weights, dcfg, dev, steps):
    """Decode shard with the whole layer captured once in a HIP graph (through
    torch.cuda.graph) and replayed back to back: the launch latency of the
    layer's small kernels is what this removes."""
    import torch
    import workloads as W
    ids, w = W.make_router(dcfg)
    x = W.make_activations(dcfg)
    T, k = ids.shape
    d_x = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    d_ids, d_w = torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    lay = nv.nvfp4_moe_ws_layout(T, k, dcfg.hidden, dcfg.inter, dcfg.num_local)
    ws = torch.empty(lay["end"], dtype=torch.uint8, device=dev)
    out = torch.empty((T, dcfg.hidden), dtype=torch.bfloat16, device=dev)
    fwd = lambda: nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, dcfg.expert_start, out=out, ws=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fwd()
    torch.cuda.current_stream().wait_stream(s)
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), eager.view(torch.int16)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    counts = nv.ws_view(ws, lay, "counts", torch.int32, (dcfg.num_local,)).cpu().numpy()
    touched = int((counts > 0).sum())
    H, I = dcfg.hidden, dcfg.inter
    bytes_w = touched * (2 * I * (H // 2 + H // 16) + H * (I // 2 + I // 16))
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "layer_weight_GBs": round(bytes_w / (ms * 1e-3) / 1e9, 1),
            "layer_hbm_frac": round(bytes_w / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "replay_equals_eager": same}


def skewed_shard(nv, W, dev, settle_ms, steps):
    """Skewed-load shard (16384 tokens, Zipf popularity with empty and hot
    local experts, W_up 30x): layer throughput and grouped-GEMM FLOP rate."""
    import torch
    cfg = W.get_config("skewed")
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    weights = nv.prepare_weights(bf(wg), bf(wu), bf(wd))
    del wg, wu, wd
    T, k = ids.shape
    d_x, d_ids, d_w = bf(x), torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    lay = nv.nvfp4_moe_ws_layout(T, k, cfg.hidden, cfg.inter, cfg.num_local)
    ws = torch.empty(lay["end"], dtype=torch.uint8, device=dev)
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=dev)
    step = lambda: nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, cfg.expert_start, out=out, ws=ws)
    settle(step, settle_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    counts = nv.ws_view(ws, lay, "counts", torch.int32, (cfg.num_local,)).cpu().numpy()
    S = int(counts.sum())
    H, I = cfg.hidden, cfg.inter
    return {"workload": f"skewed shard: T={T}, top-{k} of {cfg.num_global}, Zipf(1.2) popularity, local "
                        f"{cfg.expert_start}..{cfg.expert_start + cfg.num_local - 1}, H={H}, I={I}",
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4), "slots": S,
            "empty_experts": int((counts == 0).sum()), "max_expert_share": round(float(counts.max()) / S, 4),
            "layer_tflops": round(S * 2.0 * (2 * I * H + H * I) / (ms * 1e-3) / 1e12, 2)}


def static_scales(nv, weights, W, dev, settle_ms, rounds=5):
    """The layer with fixed global scales (calibrated on the same batch, so the
    output must equal the dynamic layer's) beside the dynamic layer, on the
    prefill and decode shards, timed in alternating blocks on one stream."""
    import torch
    res = {}
    for name, n in (("prefill", 10), ("decode", 50)):
        cfg = W.get_config(name)
        ids, w = W.make_router(cfg)
        x = W.make_activations(cfg)
        T, k = ids.shape
        d_x = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        d_ids, d_w = torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
        lay = nv.nvfp4_moe_ws_layout(T, k, cfg.hidden, cfg.inter, cfg.num_local)
        ws = torch.empty(lay["end"], dtype=torch.uint8, device=dev)
        o_dyn = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=dev)
        o_sta = torch.empty_like(o_dyn)
        gs = nv.calibrate_static_gs(weights, d_x, d_ids, d_w, cfg.expert_start)
        fns = {"dynamic": lambda: nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, cfg.expert_start, out=o_dyn, ws=ws),
               "static": lambda: nv.nvfp4_moe_forward_static(weights, d_x, d_ids, d_w, cfg.expert_start, gs,
                                                             out=o_sta, ws=ws)}
        settle(fns["dynamic"], settle_ms)
        times = {key: [] for key in fns}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(rounds):
            for key, fn in fns.items():
                e0.record()
                for _ in range(n):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                times[key].append(e0.elapsed_time(e1) / n)
        ms_s, ms_d = float(np.median(times["static"])), float(np.median(times["dynamic"]))
        res[name] = {"ms_per_step": round(ms_s, 4), "tokens_per_s": round(T / (ms_s * 1e-3), 1),
                     "dynamic_ms_per_step": round(ms_d, 4), "speedup_vs_dynamic": round(ms_d / ms_s, 4),
                     "equals_dynamic": bool(torch.equal(o_sta.view(torch.int16), o_dyn.view(torch.int16)))}
    res["note"] = ("fixed gs_x, gs_h measured once by a dynamic pass (calibrate_static_gs); no amax passes; "
                   "prefill: h written as NVFP4 by the L1 epilogue, decode: BF16 h + one fixed-scale quantize; "
                   "medians of alternating blocks")
    return res


def quantize_c1(nv, W, dev, settle_ms, reps=50):
    """Activation quantizer alone on the 4096 x 7168 Student-t(3) tensor with
    +-2000 outliers: HBM bytes of one ideal pass (read x once, write codes,
    scales and gs) over the measured time."""
    import torch
    qc = W.get_config("quant")
    xq = W.make_quant_input(qc)
    d = torch.from_numpy(xq.view(np.int16)).view(torch.bfloat16).to(dev)
    M, K = xq.shape
    q = torch.empty((1, M, K // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((1, M, K // 16), dtype=torch.uint8, device=dev)
    gs = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(max(nv.nvfp4_quantize_ws_bytes(1, M, K), 256), dtype=torch.uint8, device=dev)
    fn = lambda: nv.nvfp4_quantize(d, q=q, sf=sf, gs=gs, ws=ws)
    settle(fn, settle_ms / 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    ideal = M * K * 2 + M * K // 2 + M * K // 16 + 4
    return {"workload": f"activation quantizer alone, [{M}, {K}] Student-t(3) with 0.1% at +-2000",
            "us_per_call": round(us, 2), "ideal_bytes": ideal,
            "GBs": round(ideal / (us * 1e-6) / 1e9, 1), "hbm_frac": round(ideal / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "gs": float(gs.item())}


def settle(fn, ms):
    """Run fn back to back for about ms milliseconds of GPU time (untimed)."""
    import torch
    if ms <= 0:
        return
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    n = max(1, int(ms / max(e0.elapsed_time(e1), 1e-3)))
    for _ in range(min(n, 20000)):
        fn()
    torch.cuda.synchronize()


def _counter_rows(d, counter):
    """(kernel name, value) per dispatch from a rocprofv3 csv counter run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_traffic(workload, fetch_dir, write_dir):
    """Per-launch HBM bytes of the L1 GEMM (the grouped GEMM instance with the
    SiLU*up epilogue), each counter scaled by what it reads for the plain
    1 GiB copy of --copy-calibration."""
    out = {}
    for tag, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        cal = [v for n, v in rows if "neg" in n.lower()]
        l1 = [v for n, v in rows if "grouped_gemm_kernel" in n and n.replace(" ", "").split(">")[0].endswith(",1")]
        if not cal or not l1:
            raise SystemExit(f"{counter}: calibration dispatches {len(cal)}, L1 GEMM dispatches {len(l1)}")
        factor = COPY_CAL_BYTES / (float(np.median(cal)) * 1024.0)
        out[tag] = dict(kib=float(np.mean(l1)), factor=factor, n=len(l1),
                        bytes=float(np.mean(l1)) * 1024.0 * factor)
    path = os.path.join(PROFILE_DIR, f"l1_gemm_{workload}_traffic.txt")
    with open(path, "w") as f:
        f.write(f"# HBM traffic of the L1 grouped GEMM (gate+up, SiLU*up epilogue), {workload} shard\n")
        f.write("# counters from two rocprofv3 runs on the MI355X box, from the repository root:\n")
        for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            f.write(f"#   timeout -s KILL 180 rocprofv3 --pmc {c} -f csv -d {d} -o run -- python -u bench.py "
                    f"--config {workload} --steps 2 --warmup 1 --no-decode --no-cpu-baseline --settle-ms 0 "
                    f"--copy-calibration\n")
        f.write(f"# summarized with: python bench.py --config {workload} --summarize-traffic {fetch_dir} {write_dir}\n")
        f.write("# each counter (KiB per dispatch) is scaled by bytes / counter of a plain 1 GiB copy\n")
        f.write(f"kernel_source_sha = {kernel_source_sha()}\n")
        for tag in ("fetch", "write"):
            o = out[tag]
            f.write(f"{tag}_kib_per_launch = {o['kib']:.1f}\n{tag}_copy_factor = {o['factor']:.4f}\n"
                    f"{tag}_dispatches = {o['n']}\n{tag}_bytes_per_launch = {o['bytes']:.0f}\n")
        f.write(f"hbm_bytes_per_launch = {out['fetch']['bytes'] + out['write']['bytes']:.0f}\n")
    print(open(path).read())


def _short_kernel_name(n):
    n = n.split("(")[0].replace("void ", "").replace("nvfp4::", "")
    return n if len(n) < 90 else n[:87] + "..."


def summarize_trace(workload, d, all_workloads=False):
    """Per-kernel table (calls, total, average, min, max) of a rocprofv3
    --kernel-trace --stats csv run: of the headline workload alone
    (--no-decode), or with all_workloads of the whole default run (decode,
    skewed and static-scale objects too)."""
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(f[0])))
    if workload == "quantize":
        name = "quantize_activation_kernel_trace.md"
    else:
        name = "layer_all_workloads_kernel_trace.md" if all_workloads else f"layer_{workload}_kernel_trace.md"
    path = os.path.join(PROFILE_DIR, name)
    with open(path, "w") as o:
        if workload == "quantize":
            o.write("# Kernel trace of the activation quantizer alone (4096 x 7168 BF16, Student-t(3) with 0.1% "
                    "at +-2000): amax pass, then quantize\n\n")
            o.write("Command, from the repository root on the MI355X box:\n\n```\n")
            o.write(f"rocprofv3 --kernel-trace --stats -f csv -d {d} -o run -- python -u bench.py --quantize-only\n")
            o.write(f"python bench.py --config quantize --summarize-trace {d}\n```\n\n")
            o.write("The settle period (75 ms of back-to-back calls) and the 50 timed calls are all in the "
                    "trace.\n\n")
            o.write("| kernel | calls | total ms | avg us | min us | max us | share |\n|---|---|---|---|---|---|---|\n")
            for r in rows:
                o.write(f"| `{_short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                        f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                        f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |\n")
            print(open(path).read())
            return
        if all_workloads:
            o.write(f"# Kernel trace of the whole benchmark run ({workload} headline; decode, skewed and "
                    "static-scale objects beside it)\n\n")
        else:
            o.write(f"# Kernel trace of the benchmark, {workload} shard alone\n\n")
        o.write("Command, from the repository root on the MI355X box:\n\n```\n")
        o.write(f"rocprofv3 --kernel-trace --stats -f csv -d {d} -o run -- python -u bench.py --config {workload} "
                f"--steps 5 --warmup 1 --no-cpu-baseline --settle-ms 100{'' if all_workloads else ' --no-decode'}\n")
        o.write(f"python bench.py --config {workload} --summarize-trace {d}{' --trace-all' if all_workloads else ''}"
                "\n```\n\n")
        o.write("Grouped GEMM template arguments: <SUB_M, SUB_N, WAVES, stages in flight, epilogue> "
                "(epilogue 1 = L1 with SiLU*up, 0 = L2). The settle period, the warmup and the timed "
                "steps are all in the trace.\n\n")
        o.write("| kernel | calls | total ms | avg us | min us | max us | share |\n|---|---|---|---|---|---|---|\n")
        for r in rows:
            o.write(f"| `{_short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                    f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                    f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |\n")
        if not all_workloads:
            # the benchmark's last GPU work is the L1 GEMM timed alone with events (5 launches in the command
            # above): the same launches, read from the per-dispatch trace
            t = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
            if t:
                l1 = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                            for r in csv.DictReader(open(t[0]))
                            if "grouped_gemm_kernel<" in r["Kernel_Name"]
                            and _short_kernel_name(r["Kernel_Name"]).rstrip(">").endswith(", 1"))
                last = [(e - b) / 1e3 for b, e in l1[-5:]]
                if last:
                    o.write(f"\nL1 GEMM, the last {len(last)} dispatches (the launches the benchmark times with HIP "
                            f"events for `roofline.avg_launch_ms`): {np.mean(last):.1f} us on average "
                            f"(min {min(last):.1f}, max {max(last):.1f}).\n")
    print(open(path).read())


def summarize_mfma(workload, d):
    """MFMA work of the L1 GEMM from one rocprofv3 --pmc run: executed MFMA
    instructions (32x32x16 fp16: 32768 FLOP each) against the algorithmic
    FLOP, and the MFMA-busy share of the SIMD cycles."""
    ins = _counter_rows(d, "SQ_INSTS_MFMA")
    busy = _counter_rows(d, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _counter_rows(d, "GRBM_GUI_ACTIVE")
    sqb = _counter_rows(d, "SQ_BUSY_CYCLES")
    sel = lambda rows: [v for n, v in rows if "grouped_gemm_kernel" in n and
                        n.replace(" ", "").split(">")[0].endswith(",1")]
    i, b, g, q = (float(np.mean(sel(r))) for r in (ins, busy, gui, sqb))
    path = os.path.join(PROFILE_DIR, f"l1_gemm_{workload}_mfma.txt")
    with open(path, "w") as o:
        o.write(f"# MFMA counters of the L1 grouped GEMM (gate+up, SiLU*up epilogue), {workload} shard\n")
        o.write("# command, from the repository root on the MI355X box:\n")
        o.write(f"#   timeout -s KILL 180 rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
                f"SQ_WAVES GRBM_GUI_ACTIVE -f csv -d {d} -o run -- python -u bench.py --config {workload} "
                f"--steps 2 --warmup 1 --no-decode --no-cpu-baseline --settle-ms 0\n")
        o.write(f"# summarized with: python bench.py --config {workload} --summarize-mfma {d}\n")
        o.write(f"kernel_source_sha = {kernel_source_sha()}\n")
        o.write(f"dispatches = {len(sel(ins))}\n")
        o.write(f"mfma_instructions_per_launch = {i:.0f}\n")
        o.write(f"executed_mfma_flop_per_launch = {i * 32768:.0f}\n")
        o.write(f"mfma_busy_cycles_per_launch = {b:.0f}   # summed over SIMDs; 32 per 32x32x16 fp16 MFMA\n")
        o.write(f"grbm_gui_active_per_launch = {g:.0f}\n")
        o.write(f"sq_busy_cycles_per_launch = {q:.0f}\n")
    print(open(path).read())


def cpu_baseline(cfg, ids, w, x, wg, wu, wd, T):
    """The CPU oracle timed on the same workload: whole forward passes (steps
    a1..a8 over all T tokens) repeated until at least NVFP4_BENCH_ORACLE_SECONDS
    (default 10) have passed, experts spread over a pool of worker threads with
    one BLAS thread each, so the core count is the pool size. Weight
    preparation (offline) is not timed."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    budget = float(os.environ.get("NVFP4_BENCH_ORACLE_SECONDS", "10"))
    cores = len(os.sched_getaffinity(0))
    threads = min(16, cores)
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        P = O.prepare_weights(wg, wu, wd, map_fn=ex.map)
    log(f"oracle weight preparation (untimed) {time.time() - t0:.1f}s")
    reps = 0
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=threads) as ex:
        t = time.perf_counter()
        while True:
            O.moe_forward(x, ids, w, cfg.expert_start, P, map_fn=ex.map)
            reps += 1
            dt = time.perf_counter() - t
            log(f"oracle forward pass {reps} over {T} tokens: {dt:.1f}s total")
            if dt >= budget:
                break
    return {"value": round(reps * T / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} whole forward passes of the {cfg.name} shard ({T} tokens each, steps a1-a8) "
                      f"in {dt:.1f}s; experts on {threads} worker threads with one BLAS thread each; "
                      f"{cores} host cores visible"}


if __name__ == "__main__":
    main()
