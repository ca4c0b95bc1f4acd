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
N_XCD = 8                     # GRBM_GUI_ACTIVE counts the GPU-busy cycles of every XCD
TRACE_STEPS = 5               # --steps of the kernel-trace commands the trace summaries name


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="prefill", choices=["prefill", "decode", "skewed", "quantize", "peaks"],
                    help="headline workload (quantize, peaks: only with --summarize-trace of a --quantize-only or "
                         "--peaks run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed GPU time spent on the workload before the warmup steps, so that "
                         "the clocks leave their start-of-load transient (steady state is timed)")
    ap.add_argument("--no-decode", action="store_true",
                    help="time the headline workload only (no decode, tiny, quantizer, skewed, static-scale "
                         "and peak objects)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (elementwise negate) three times, "
                         "so that counter runs can scale FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the per-launch HBM traffic of the grouped GEMMs from two rocprofv3 --pmc "
                         "csv runs (FETCH_SIZE, WRITE_SIZE) to profiles/ and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write the per-kernel table of a rocprofv3 --kernel-trace --stats csv run to "
                         "profiles/ and exit")
    ap.add_argument("--trace-all", action="store_true",
                    help="with --summarize-trace: the trace is of the whole default run (no --no-decode)")
    ap.add_argument("--quantize-only", action="store_true",
                    help="time only the activation quantizer on the 4096 x 7168 tensor and print its object "
                         "(for a kernel trace of the quantizer alone); not the benchmark line")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the achievable HBM streaming-read rate and MFMA rate on this GPU and print "
                         "them; not the benchmark line")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="write the MFMA counters of the grouped GEMMs from a rocprofv3 --pmc csv run to "
                         "profiles/ and exit")
    ap.add_argument("--summarize-valu", metavar="PMC_DIR",
                    help="write the VALU/SALU/MFMA instruction counts of the grouped GEMMs from a rocprofv3 "
                         "--pmc csv run to profiles/ and exit")
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
    if args.summarize_valu:
        summarize_valu(args.config, args.summarize_valu)
        return
    if args.config in ("quantize", "peaks") and not (args.quantize_only or args.peaks):
        raise SystemExit(f"bench.py: --config {args.config} only names the trace of a --quantize-only or --peaks run")
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
    if args.peaks:
        print(json.dumps({"achievable_peaks": achievable_peaks(dev)}), flush=True)
        return
    cfg = W.get_config(args.config)
    t0 = time.time()
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    log(f"generated {cfg.name} inputs in {time.time() - t0:.1f}s")
    bf16_w = (_bf16(wg, dev), _bf16(wu, dev), _bf16(wd, dev))
    weights = nv.prepare_weights(*bf16_w)
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    log(f"timing {cfg.name}: {args.warmup} warmup + {args.steps} steps")
    r = measure_layer(nv, weights, cfg, ids, w, x, dev, args.steps, args.warmup, args.settle_ms,
                      flushed=cfg.name != "decode")
    T, k, H, I = cfg.tokens, cfg.top_k, cfg.hidden, cfg.inter
    S = r["S"]
    tok_s = T / (r["ms"] * 1e-3)
    layer_flop = S * 2.0 * (2 * I * H + H * I)            # per slot: 132.12 MFLOP
    roof_l1, roof_l2 = gemm_rooflines(cfg, r)
    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic (seeded NumPy draws, random-init weights)",
        "config": {"workload": f"{cfg.name} shard: T={T}, top-{k} of {cfg.num_global} experts, local "
                               f"{cfg.expert_start}..{cfg.expert_start + cfg.num_local - 1}, H={H}, I={I}",
                   "tokens": T, "top_k": k, "local_experts": cfg.num_local, "hidden": H, "inter": I,
                   "slots": S, "touched_experts": r["touched"], "tile_m": r["tile_m"]},
        "layer_tflops": round(layer_flop / (r["ms"] * 1e-3) / 1e12, 2),
        "roofline": roof_l1,
        "roofline_l2": roof_l2,
        "step_ms": r["step"],
        "stages_ms": r["stages"],
        "stage_bandwidth": stage_bandwidth(cfg, r),
        "ms_per_step_without_stage_events": round(r["plain_ms"], 4),
        "timing_note": ("value and ms_per_step: wall clock over the timed steps (synchronized on both sides), "
                        "each step with HIP events on the layer's stream around its L1 grouped GEMM; roofline: "
                        "algorithmic work over the mean L1 launch time from those events; step_ms, stages_ms "
                        "and roofline_l2: a second pass of as many steps with events between all stages "
                        "(median, p10, p90 per step; medians per stage; mean L2 launch); "
                        "ms_per_step_without_stage_events: a third pass without events"),
    }
    if "flushed" in r:
        result["step_ms_flushed"] = r["flushed"]
    if not args.no_decode:
        result["accuracy"] = {
            "cosine_vs_bf16_weights": layer_cosine_bf16(cfg, ids, w, x, bf16_w, r["out"], dev),
            "gate": 0.98,
            "note": "cosine of the layer output against the same layer with the original, unquantized BF16 weights "
                    "(float32 torch matmuls on the GPU, computed here): the gate read literally, not met on these "
                    "Gaussian weights (four NVFP4 roundings; the oracle lands at the same value). The parity tests "
                    "gate the cosine against the layer built from the dequantized NVFP4 weights (>= 0.98, met)"}
    if cfg.name == "prefill" and not args.no_decode:
        # the decode shard uses the same weights
        result["decode"] = decode_shard(nv, weights, W, dev, max(args.steps, 50), args.warmup, args.settle_ms,
                                        bf16_w=bf16_w)
        del bf16_w
        result["tiny"] = tiny_layer(nv, W, dev, args.settle_ms)
        result["quantize"] = quantize_c1(nv, W, dev, args.settle_ms)
        result["skewed"] = skewed_shard(nv, W, dev, args.settle_ms, max(args.steps, 10), args.warmup)
        result["static_scales"] = static_scales(nv, weights, W, dev, args.settle_ms)
        result["achievable_peaks"] = achievable_peaks(dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, ids, w, x, wg, wu, wd, T)
    print(json.dumps(result), flush=True)


def _bf16(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def stats(times_ms):
    a = np.asarray(times_ms, np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


class Flush:
    """Evicts the 256 MB last-level cache: a 512 MB read (no dirty lines left to
    write back during the step that follows)."""

    def __init__(self, dev):
        import torch
        self.buf = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def _events(n):
    """n timing events, each recorded once so that it exists (the library
    records them again on its stream)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    return evs


def per_call_times(fn, n, flush=None):
    """Times of n calls of fn, each between two events on the current stream;
    with flush, the cache is flushed before every call (outside the events).
    Everything is enqueued without host waits."""
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in pairs:
        if flush:
            flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def measure_layer(nv, weights, cfg, ids, w, x, dev, steps, warmup, settle_ms, flushed=False):
    """The timed region: `steps` layer steps back to back, each through
    nvfp4_moe_forward_stage_events with HIP events recorded on the layer's
    stream only just before and just after the L1 grouped GEMM (a timing
    event costs a few microseconds); wall clock around the region
    (synchronized on both sides) gives ms_per_step, the events the L1 launch
    times. Then a pass of the same number of steps with events between all
    stages (per-step and per-stage times; the L2 launch times), a pass
    without events, and optionally steps with the cache flushed before each."""
    import torch
    T, k = ids.shape
    d_x, d_ids, d_w = _bf16(x, dev), torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=dev)
    lay = nv.nvfp4_moe_ws_layout(T, k, cfg.hidden, cfg.inter, cfg.num_local)
    ws = torch.empty(lay["end"], dtype=torch.uint8, device=dev)
    plain = lambda: nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, cfg.expert_start, out=out, ws=ws)
    staged = lambda ev: nv.nvfp4_moe_forward_stage_events(weights, d_x, d_ids, d_w, cfg.expert_start, ev,
                                                          out=out, ws=ws)
    ns = len(nv.STAGES) + 1
    i_l1 = nv.STAGES.index("a4_a5_l1_gemm")
    l1_evs = [_events(2) for _ in range(steps)]
    l1_only = [[None] * ns for _ in range(steps)]
    for i in range(steps):
        l1_only[i][i_l1], l1_only[i][i_l1 + 1] = l1_evs[i]
    all_evs = [_events(ns) for _ in range(steps)]
    flush = Flush(dev) if flushed else None
    settle(plain, settle_ms)
    for _ in range(warmup):
        plain()
    torch.cuda.synchronize()
    # The passes follow one another with nothing but a synchronization
    # between them (the event times are read at the end): an idle gap of a
    # few tens of milliseconds lets the clocks drop, and the first steps
    # after it run up to 40% slower.
    t = time.perf_counter()
    for i in range(steps):
        staged(l1_only[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / steps
    for i in range(steps):
        staged(all_evs[i])
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        plain()
    torch.cuda.synchronize()
    plain_ms = (time.perf_counter() - t) * 1e3 / steps
    fl = per_call_times(plain, steps, flush) if flushed else None
    l1 = [a.elapsed_time(b) for a, b in l1_evs]
    step = [e[0].elapsed_time(e[-1]) for e in all_evs]
    stage = {name: [e[i].elapsed_time(e[i + 1]) for e in all_evs] for i, name in enumerate(nv.STAGES)}
    res = dict(ms=ms, step=stats(step),
               stages={n: round(float(np.median(v)), 4) for n, v in stage.items()},
               l1_ms=float(np.mean(l1)), l2_ms=float(np.mean(stage["a7_l2_gemm"])), plain_ms=plain_ms)
    if flushed:
        res["flushed"] = stats(fl)
        del flush
    counts = nv.ws_view(ws, lay, "counts", torch.int32, (cfg.num_local,)).cpu().numpy()
    res.update(S=int(counts.sum()), touched=int((counts > 0).sum()),
               tile_m=nv.nvfp4_moe_tile_m(T, k, cfg.num_local), out=out, d=(d_x, d_ids, d_w), ws=ws, lay=lay)
    return res


def stage_bandwidth(cfg, r):
    """The memory-bound stages against HBM peak: algorithmic bytes of each
    (read x for the amax; read x, write codes and scales for quantize x; the
    same for h's S valid rows; read the k local slots' rows of Y and write the
    output for the scatter) over the stage's median time from the
    stage-evented pass (which includes a few microseconds of event overhead)."""
    T, H, I, S = cfg.tokens, cfg.hidden, cfg.inter, r["S"]
    st = r["stages"]
    rows = {"a1_amax_route": T * H * 2,
            "a2_quantize_x": T * H * 2 + T * H // 2 + T * H // 16,
            "a6_quantize_h": S * I * 2 + S * I // 2 + S * I // 16,
            "a8_scatter": S * H * 2 + T * H * 2}
    out = {}
    for name, b in rows.items():
        ms = st[name]
        gbs = b / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        out[name] = {"bytes": b, "ms": ms, "GBs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def gemm_rooflines(cfg, r):
    """Roofline objects of the L1 and L2 grouped GEMMs from the mean launch
    times of the timed region: algorithmic FLOP (slots x 2 x N x K, padding
    rows not counted) against the dense fp16 MFMA peak; for decode-shaped
    batches, algorithmic weight bytes (FP4 values + E4M3 scales of the
    touched experts) against HBM. traffic: HBM bytes per launch from the
    committed counter summary of the current GEMM source, else null."""
    H, I, S, nt = cfg.hidden, cfg.inter, r["S"], r["touched"]
    out = []
    for gemm, name, ms, n, kk in (("l1", "L1 grouped GEMM (gate+up, SiLU*up epilogue)", r["l1_ms"], 2 * I, H),
                                  ("l2", "L2 grouped GEMM (down_proj)", r["l2_ms"], H, I)):
        flop = S * 2.0 * n * kk
        wbytes = nt * n * (kk // 2 + kk // 16)
        roof = {"kernel": name, "bound": "mfma", "achieved": round(flop / (ms * 1e-3) / 1e12, 2),
                "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s", "frac": round(flop / (ms * 1e-3) / 1e12 /
                                                                             PEAK_FP16_TFLOPS, 4),
                "traffic": read_traffic(cfg.name, gemm), "avg_launch_ms": round(ms, 4), "flop_per_launch": flop,
                "weight_bytes_per_launch": wbytes}
        if cfg.name == "decode":
            gbs = wbytes / (ms * 1e-3) / 1e9
            roof.update(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(gbs / PEAK_HBM_GBS, 4))
        out.append(roof)
    return out


def layer_cosine_bf16(cfg, ids, w, x, bf16_w, out, dev):
    """Cosine between the layer's output and the same layer with the original,
    unquantized BF16 weights (the accuracy gate's literal reference), here
    with plain float32 torch matmuls on the GPU: for each local expert, its
    tokens' rows of x times W_gate and W_up, silu(gate) * up, times W_down,
    weighted and summed per token. A reported figure, not a parity check."""
    import torch
    wg, wu, wd = bf16_w
    xf = _bf16(x, dev).float()
    ids_t = torch.from_numpy(ids).to(dev)
    w_t = torch.from_numpy(w).to(dev)
    ref = torch.zeros((ids.shape[0], cfg.hidden), dtype=torch.float32, device=dev)
    for e in range(cfg.num_local):
        rows, js = (ids_t == cfg.expert_start + e).nonzero(as_tuple=True)
        if rows.numel() == 0:
            continue
        xe = xf[rows]
        g = torch.matmul(xe, wg[e].float().t().contiguous())
        u = torch.matmul(xe, wu[e].float().t().contiguous())
        y = torch.matmul(torch.nn.functional.silu(g) * u, wd[e].float().t().contiguous())
        ref.index_add_(0, rows, y * w_t[rows, js][:, None])
    o = out.float()
    cos = float((o * ref).sum() / (o.norm() * ref.norm()))
    return round(cos, 5)


def decode_shard(nv, weights, W, dev, steps, warmup, settle_ms, bf16_w=None):
    """Decode shard (64 tokens, same weights): the evented timed steps, the L1
    and L2 rooflines against HBM, steps with a cold last-level cache, and the
    whole layer replayed from a HIP graph."""
    dcfg = W.get_config("decode")
    ids, w = W.make_router(dcfg)
    x = W.make_activations(dcfg)
    rd = measure_layer(nv, weights, dcfg, ids, w, x, dev, steps, warmup, settle_ms, flushed=True)
    H, I = dcfg.hidden, dcfg.inter
    bytes_w = rd["touched"] * (2 * I * (H // 2 + H // 16) + H * (I // 2 + I // 16))
    gbs = bytes_w / (rd["ms"] * 1e-3) / 1e9
    l1, l2 = gemm_rooflines(dcfg, rd)
    fl = rd["flushed"]["median"]
    res = {
        "workload": "decode shard: T=64, top-8 of 384, local 96..143, same weights",
        "tokens_per_s": round(dcfg.tokens / (rd["ms"] * 1e-3), 1), "ms_per_step": round(rd["ms"], 4),
        "ms_per_step_without_stage_events": round(rd["plain_ms"], 4),
        "touched_experts": rd["touched"], "slots": rd["S"], "weight_bytes_per_step": bytes_w,
        "layer_weight_GBs": round(gbs, 1), "layer_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "step_ms": rd["step"], "stages_ms": rd["stages"], "stage_bandwidth": stage_bandwidth(dcfg, rd),
        "roofline_l1": l1, "roofline_l2": l2,
        "flushed": dict(rd["flushed"], layer_hbm_frac=round(bytes_w / (fl * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)),
    }
    if bf16_w is not None:
        res["cosine_vs_bf16_weights"] = layer_cosine_bf16(dcfg, ids, w, x, bf16_w, rd["out"], dev)
    res["graph"] = layer_graph(nv, weights, dcfg, rd, dev, steps, bytes_w)
    res["graph_8_layers"] = layer_graph(nv, weights, dcfg, rd, dev, 8 * steps, bytes_w, layers=8)
    res["graph_note"] = ("graph: one layer call per graph; graph_8_layers: eight calls in one graph (a model's decode "
                         "graph holds all its MoE layers), times per call. Each replay starts about 8 us after the "
                         "previous one ends, whatever the graph holds.")
    return res


def layer_graph(nv, weights, cfg, r, dev, steps, bytes_w=None, layers=1):
    """The whole layer captured once in a HIP graph (torch.cuda.graph) and
    replayed: back-to-back replays (wall clock and per-replay events) and
    whether the replay equals the eager output bit for bit. With layers > 1
    the graph holds that many calls of the layer one after the other, as the
    graph of a model's decode step holds all of its MoE layers; times are then
    per layer call."""
    import torch
    d_x, d_ids, d_w = r["d"]
    out, ws = r["out"], r["ws"]
    fwd = lambda: nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, cfg.expert_start, out=out, ws=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fwd()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(layers):
            fwd()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), eager.view(torch.int16)))
    reps = max(steps // layers, 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * layers)
    per_replay = stats([t / layers for t in per_call_times(g.replay, reps)])
    res = {"ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.tokens / (ms * 1e-3), 1),
           "replay_ms": per_replay, "replay_equals_eager": same}
    if layers > 1:
        res["layers_per_graph"] = layers
    if bytes_w:
        res["layer_hbm_frac"] = round(bytes_w / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    return res


def tiny_layer(nv, W, dev, settle_ms, steps=100):
    """The tiny layer (32 tokens, 8 experts, H=256, I=128): latency of one
    eager step and of one graph replay."""
    cfg = W.get_config("tiny")
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    weights = nv.prepare_weights(_bf16(wg, dev), _bf16(wu, dev), _bf16(wd, dev))
    r = measure_layer(nv, weights, cfg, ids, w, x, dev, steps, 5, settle_ms / 10)
    g = layer_graph(nv, weights, cfg, r, dev, steps)
    return {"workload": "tiny layer: T=32, top-2 of 8 experts (all local), H=256, I=128",
            "step_latency_us": {k: (round(v * 1e3, 2) if k != "n" else v) for k, v in r["step"].items()},
            "graph_replay_latency_us": {k: (round(v * 1e3, 2) if k != "n" else v)
                                        for k, v in g["replay_ms"].items()},
            "stages_us": {k: round(v * 1e3, 2) for k, v in r["stages"].items()}}


def skewed_shard(nv, W, dev, settle_ms, steps, warmup):
    """Skewed-load shard (16384 tokens, Zipf popularity with empty and hot
    local experts, W_up 30x): throughput, per-step distribution (warm and
    flushed), per-stage times and the rooflines of both grouped GEMMs."""
    import torch
    cfg = W.get_config("skewed")
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    weights = nv.prepare_weights(_bf16(wg, dev), _bf16(wu, dev), _bf16(wd, dev))
    del wg, wu, wd
    r = measure_layer(nv, weights, cfg, ids, w, x, dev, steps, warmup, settle_ms, flushed=True)
    counts = nv.ws_view(r["ws"], r["lay"], "counts", torch.int32, (cfg.num_local,)).cpu().numpy()
    T, k, H, I, S = cfg.tokens, cfg.top_k, cfg.hidden, cfg.inter, r["S"]
    l1, l2 = gemm_rooflines(cfg, r)
    return {"workload": f"skewed shard: T={T}, top-{k} of {cfg.num_global}, Zipf(1.2) popularity, local "
                        f"{cfg.expert_start}..{cfg.expert_start + cfg.num_local - 1}, H={H}, I={I}",
            "tokens_per_s": round(T / (r["ms"] * 1e-3), 1), "ms_per_step": round(r["ms"], 4), "slots": S,
            "empty_experts": int((counts == 0).sum()), "max_expert_share": round(float(counts.max()) / S, 4),
            "layer_tflops": round(S * 2.0 * (2 * I * H + H * I) / (r["ms"] * 1e-3) / 1e12, 2),
            "step_ms": r["step"], "step_ms_flushed": r["flushed"], "stages_ms": r["stages"],
            "stage_bandwidth": stage_bandwidth(cfg, r), "roofline_l1": l1, "roofline_l2": l2}


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
        d_x = _bf16(x, dev)
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
    +-2000 outliers: bytes of one ideal pass (read x once, write codes, scales
    and gs) over the time of a call, each call timed with events after the
    last-level cache was flushed (the headline), and back to back."""
    import torch
    qc = W.get_config("quant")
    xq = W.make_quant_input(qc)
    d = _bf16(xq, dev)
    M, K = xq.shape
    q = torch.empty((1, M, K // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((1, M, K // 16), dtype=torch.uint8, device=dev)
    gs = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(max(nv.nvfp4_quantize_ws_bytes(1, M, K), 256), dtype=torch.uint8, device=dev)
    fn = lambda: nv.nvfp4_quantize(d, q=q, sf=sf, gs=gs, ws=ws)
    settle(fn, settle_ms / 4)
    flushed = stats(per_call_times(fn, reps, Flush(dev)))
    warm = stats(per_call_times(fn, reps))
    ideal = M * K * 2 + M * K // 2 + M * K // 16 + 4
    us = flushed["median"] * 1e3
    gbs = lambda ms: round(ideal / (ms * 1e-3) / 1e9, 1)
    return {"workload": f"activation quantizer alone, [{M}, {K}] Student-t(3) with 0.1% at +-2000",
            "us_per_call": round(us, 2), "ideal_bytes": ideal, "GBs": gbs(flushed["median"]),
            "hbm_frac": round(ideal / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "flushed_ms": flushed, "back_to_back_ms": warm, "back_to_back_GBs": gbs(warm["median"]),
            "note": "us_per_call, GBs, hbm_frac: median over calls each preceded by a 512 MB read that evicts "
                    "the last-level cache", "gs": float(gs.item())}


PEAK_READ_BYTES = 3 << 29                  # bytes the read probe streams
PEAK_MFMA_FLOP = 512 * 4.0 * 20000 * 4 * 32768   # FLOP of one MFMA probe launch on 256 CUs


def achievable_peaks(dev, read_bytes=PEAK_READ_BYTES, reps=10):
    """What this GPU sustains in practice: a streaming read of a 1.5 GiB
    buffer (well past the 256 MB last-level cache) and a loop of independent
    fp16 MFMAs without memory traffic, each timed with events (median of
    reps launches)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "nvfp4_quantized_moe_amd", "libnvfp4probe.so"))
    lib.nvfp4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.nvfp4probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.ones(read_bytes // 4, dtype=torch.float32, device=dev)
    rgrid = n_cu * 32
    rout = torch.empty(rgrid, dtype=torch.int32, device=dev)

    def read():
        if lib.nvfp4probe_read(ctypes.c_void_p(buf.data_ptr()), read_bytes, ctypes.c_void_p(rout.data_ptr()),
                               rgrid, stream):
            raise RuntimeError("nvfp4probe_read failed")
    read()
    rt = stats(per_call_times(read, reps))
    del buf
    iters, mgrid = 20000, n_cu * 2
    mout = torch.empty(mgrid * 4, dtype=torch.float32, device=dev)

    def mfma():
        if lib.nvfp4probe_mfma(iters, ctypes.c_void_p(mout.data_ptr()), mgrid, stream):
            raise RuntimeError("nvfp4probe_mfma failed")
    mfma()
    mt = stats(per_call_times(mfma, reps))
    flop = mgrid * 4.0 * iters * 4 * 32768
    gbs = read_bytes / (rt["median"] * 1e-3) / 1e9
    tfs = flop / (mt["median"] * 1e-3) / 1e12
    return {"hbm_read_GBs": round(gbs, 1), "hbm_read_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
            "hbm_read_bytes": read_bytes, "hbm_read_ms": rt,
            "mfma_fp16_TFLOPs": round(tfs, 1), "mfma_frac_of_peak": round(tfs / PEAK_FP16_TFLOPS, 4),
            "mfma_flop": flop, "mfma_ms": mt,
            "note": f"read: {rgrid} workgroups of 256 threads, eight 16-byte non-temporal loads in flight per thread; MFMA: "
                    f"{mgrid} workgroups of 4 waves (2 per SIMD), 4 independent v_mfma_f32_32x32x16_f16 chains "
                    f"per wave, no memory traffic in the loop"}


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


def _short_kernel_name(n):
    n = n.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("nvfp4::", "")
    return n if len(n) < 90 else n[:87] + "..."


def _gemm_epi(name):
    """Epilogue template argument of a grouped GEMM kernel name (1, 2: L1 with
    SiLU*up; 3: L1 writing NVFP4 h; 0: L2), else None."""
    if "grouped_gemm_kernel<" not in name:
        return None
    args = name.replace(" ", "").split("grouped_gemm_kernel<", 1)[1].split(">")[0].split(",")
    return int(args[-1]) if args and args[-1].isdigit() else None


def _kernel_label(name):
    epi = _gemm_epi(name)
    if epi is not None:
        return {0: "l2_gemm", 1: "l1_gemm", 2: "l1_gemm", 3: "l1_gemm_nvfp4"}.get(epi, "gemm")
    return _short_kernel_name(name)


def _per_kernel(rows):
    """Mean counter value per dispatch, by kernel label: {label: (mean, dispatches)}."""
    by = {}
    for n, v in rows:
        by.setdefault(_kernel_label(n), []).append(v)
    return {k: (float(np.mean(v)), len(v)) for k, v in by.items()}


def _profile_header(f, what, workload, cmds, summarize, title=None):
    f.write(f"# {what}, {title or workload + ' shard'}\n")
    f.write("# command(s), from the repository root on the MI355X box:\n")
    for c in cmds:
        f.write(f"#   {c}\n")
    f.write(f"# summarized with: python bench.py --config {workload} {summarize}\n")
    f.write(f"kernel_source_sha = {kernel_source_sha()}\n")


def _bench_cmd(workload, extra=""):
    return (f"python -u bench.py --config {workload} --steps 2 --warmup 1 --no-decode --no-cpu-baseline "
            f"--settle-ms 0{extra}")


def _kv(path):
    """key = value lines of a profile summary (comments skipped)."""
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.split("#")[0].strip()
    return kv


def read_traffic(workload: str, gemm: str = "l1"):
    """Per-launch HBM bytes of the L1 or L2 grouped GEMM from the committed
    counter summary, or None when absent or taken on a different kernel
    source."""
    p = os.path.join(PROFILE_DIR, f"gemm_{workload}_traffic.txt")
    if not os.path.exists(p):
        return None
    kv = _kv(p)
    if kv.get("kernel_source_sha") != kernel_source_sha() or f"{gemm}_hbm_bytes_per_launch" not in kv:
        return None
    return float(kv[f"{gemm}_hbm_bytes_per_launch"])


def summarize_traffic(workload, fetch_dir, write_dir):
    """Per-launch HBM bytes of every kernel of the run, each counter (KiB per
    dispatch) scaled by what it reads for the plain 1 GiB copy of
    --copy-calibration; the grouped GEMMs' figures also as key = value lines.
    workload quantize: the two runs are of --quantize-only, which has no
    calibration copy; the factors of the committed prefill summary (same
    counters, same GPU model) scale them."""
    per, fac = {}, {}
    quant = workload == "quantize"
    for tag, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        cal = [v for n, v in rows if "neg" in n.lower()]
        if cal:
            fac[tag] = COPY_CAL_BYTES / (float(np.median(cal)) * 1024.0)
        elif quant:
            fac[tag] = float(_kv(os.path.join(PROFILE_DIR, "gemm_prefill_traffic.txt"))[f"{tag}_copy_factor"])
        else:
            raise SystemExit(f"{counter}: no calibration copy dispatches (run with --copy-calibration)")
        per[tag] = _per_kernel([(n, v) for n, v in rows if "neg" not in n.lower()])
    name = "quantize_activation_traffic.txt" if quant else f"gemm_{workload}_traffic.txt"
    path = os.path.join(PROFILE_DIR, name)
    cmd = "python -u bench.py --quantize-only" if quant else _bench_cmd(workload, " --copy-calibration")
    with open(path, "w") as f:
        _profile_header(f, "HBM traffic per kernel launch (FETCH_SIZE, WRITE_SIZE, copy-calibrated)",
                        workload,
                        [f"timeout -s KILL 180 rocprofv3 --pmc {c} -f csv -d {d} -o run -- " + cmd
                         for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))],
                        f"--summarize-traffic {fetch_dir} {write_dir}",
                        title="activation quantizer alone (4096 x 7168 BF16, amax pass then quantize)" if quant
                        else None)
        src = "the factors of gemm_prefill_traffic.txt" if quant else "a plain 1 GiB copy"
        f.write(f"# each counter (KiB per dispatch) is scaled by bytes / counter of {src}: "
                f"fetch x{fac['fetch']:.4f}, write x{fac['write']:.4f}\n")
        f.write("# kernel | dispatches | fetch MB/launch | write MB/launch\n")
        for k in sorted(per["fetch"]):
            fm, n = per["fetch"][k]
            wm = per["write"].get(k, (0.0, 0))[0]
            f.write(f"#   {k} | {n} | {fm * 1024 * fac['fetch'] / 1e6:.2f} | {wm * 1024 * fac['write'] / 1e6:.2f}\n")
        f.write(f"fetch_copy_factor = {fac['fetch']:.4f}\nwrite_copy_factor = {fac['write']:.4f}\n")
        keys = ((("amax_kernel", "amax"), ("quantize_kernel<false>", "quantize")) if quant else
                (("l1_gemm", "l1"), ("l2_gemm", "l2")))
        for g, key in keys:
            if g in per["fetch"]:
                fb = per["fetch"][g][0] * 1024 * fac["fetch"]
                wb = per["write"].get(g, (0.0, 0))[0] * 1024 * fac["write"]
                f.write(f"{key}_fetch_bytes_per_launch = {fb:.0f}\n{key}_write_bytes_per_launch = {wb:.0f}\n"
                        f"{key}_hbm_bytes_per_launch = {fb + wb:.0f}\n")
        if quant:
            M, K = 4096, 7168
            f.write(f"# algorithmic: x read once {M * K * 2} B; codes {M * K // 2} B + scales {M * K // 16} B "
                    f"+ gs 4 B written\n")
    print(open(path).read())


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
    if workload == "peaks":
        path = os.path.join(PROFILE_DIR, "achievable_peaks_kernel_trace.md")
        with open(path, "w") as o:
            o.write("# Kernel trace of the achievable-peak probes (bench.py --peaks): a streaming read of a 1.5 GiB "
                    "buffer and a loop of independent fp16 MFMAs\n\n")
            o.write("Command, from the repository root on the MI355X box:\n\n```\n")
            o.write(f"rocprofv3 --kernel-trace --stats -f csv -d {d} -o run -- python -u bench.py --peaks\n")
            o.write(f"python bench.py --config peaks --summarize-trace {d}\n```\n\n")
            o.write("Each probe runs once untimed, then 10 times between events (the JSON medians).\n\n")
            o.write("| kernel | calls | avg us | min us | max us | rate at the minimum |\n|---|---|---|---|---|---|\n")
            for r in rows:
                n = _short_kernel_name(r["Name"])
                mn = float(r["MinNs"]) / 1e3
                rate = ""
                if "read" in n:
                    rate = f"{PEAK_READ_BYTES / (mn * 1e-6) / 1e12:.2f} TB/s"
                elif "mfma" in n:
                    rate = f"{PEAK_MFMA_FLOP / (mn * 1e-6) / 1e12:.0f} TFLOP/s"
                o.write(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {mn:.1f} | "
                        f"{float(r['MaxNs']) / 1e3:.1f} | {rate} |\n")
        print(open(path).read())
        return
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
                f"--steps {TRACE_STEPS} --warmup 1 --no-cpu-baseline --settle-ms 100{'' if all_workloads else ' --no-decode'}\n")
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
            # measure_layer runs its passes back to back after the settle period and the warmup: the L1
            # launches evented for roofline.avg_launch_ms, the all-stage pass, the plain pass and (not for
            # decode) the flushed pass, TRACE_STEPS steps each; they are the last L1 dispatches of the trace
            t = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
            if t:
                l1 = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                            for r in csv.DictReader(open(t[0]))
                            if _gemm_epi(r["Kernel_Name"]) in (1, 2))
                passes = ["evented L1 (roofline.avg_launch_ms)", "all stages evented", "no events",
                          "cache flushed before each step"][:3 if workload == "decode" else 4]
                n = TRACE_STEPS
                if len(l1) >= n * len(passes):
                    o.write("\nL1 GEMM launches of the timed passes, from the per-dispatch trace:\n\n"
                            "| pass | launches | avg us | min us | max us |\n|---|---|---|---|---|\n")
                    tail = l1[len(l1) - n * len(passes):]
                    for i, pname in enumerate(passes):
                        dur = [(e - b) / 1e3 for b, e in tail[i * n:(i + 1) * n]]
                        o.write(f"| {pname} | {len(dur)} | {np.mean(dur):.1f} | {min(dur):.1f} | "
                                f"{max(dur):.1f} |\n")
    print(open(path).read())


MFMA_COUNTERS = ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_BUSY_CYCLES",
                 "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAVES", "GRBM_GUI_ACTIVE"]
VALU_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM",
                 "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAVES"]
STALL_COUNTERS = ["SQ_WAIT_ANY", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_ANY",
                  "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_VMEM", "SQ_WAVE_CYCLES"]


def _counter_table(dirs, counters):
    """{kernel label: {counter: mean per dispatch, 'n': dispatches}} over one
    or more rocprofv3 csv runs (each counter from the runs that hold it)."""
    tab = {}
    for d in dirs:
        for c in counters:
            try:
                rows = _counter_rows(d, c)
            except SystemExit:
                continue
            for k, (m, n) in _per_kernel(rows).items():
                tab.setdefault(k, {"n": n})[c] = m
    return tab


def summarize_mfma(workload, d):
    """MFMA work of the grouped GEMMs from one rocprofv3 --pmc run: executed
    MFMA instructions (32x32x16 fp16: 32768 FLOP each) and the MFMA-busy
    cycles against the kernel's active cycles on all SIMDs."""
    tab = _counter_table([d], MFMA_COUNTERS)
    path = os.path.join(PROFILE_DIR, f"gemm_{workload}_mfma.txt")
    with open(path, "w") as o:
        _profile_header(o, "MFMA counters of the grouped GEMMs", workload,
                        [f"timeout -s KILL 180 rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} -f csv -d {d} -o run -- "
                         + _bench_cmd(workload)], f"--summarize-mfma {d}")
        o.write("# mfma_busy_share = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): the\n"
                "# share of the kernel's active cycles in which a SIMD's matrix core works (both counters per\n"
                "# launch, GRBM_GUI_ACTIVE summed over the 8 XCDs; a 32x32x16 fp16 MFMA keeps the matrix core\n"
                "# busy for 32 of these cycles: mfma_busy_cycles = 32 x mfma_instructions)\n")
        for g in ("l1_gemm", "l2_gemm", "l1_gemm_nvfp4"):
            if g not in tab:
                continue
            t = tab[g]
            key = g.replace("_gemm", "")
            o.write(f"{key}_dispatches = {t['n']}\n")
            o.write(f"{key}_mfma_instructions_per_launch = {t['SQ_INSTS_MFMA']:.0f}\n")
            o.write(f"{key}_executed_mfma_flop_per_launch = {t['SQ_INSTS_MFMA'] * 32768:.0f}\n")
            o.write(f"{key}_mfma_busy_cycles_per_launch = {t['SQ_VALU_MFMA_BUSY_CYCLES']:.0f}\n")
            o.write(f"{key}_grbm_gui_active_per_launch = {t['GRBM_GUI_ACTIVE']:.0f}\n")
            o.write(f"{key}_mfma_busy_share = "
                    f"{t['SQ_VALU_MFMA_BUSY_CYCLES'] / (t['GRBM_GUI_ACTIVE'] / N_XCD * 1024):.4f}\n")
            o.write(f"{key}_valu_mfma_coexec_cycles_per_launch = {t['SQ_VALU_MFMA_COEXEC_CYCLES']:.0f}\n")
            o.write(f"{key}_active_inst_valu_per_launch = {t['SQ_ACTIVE_INST_VALU']:.0f}\n")
            o.write(f"{key}_active_inst_lds_per_launch = {t['SQ_ACTIVE_INST_LDS']:.0f}\n")
    print(open(path).read())


def summarize_valu(workload, dirs):
    """Instruction mix and stalls of every kernel from two rocprofv3 --pmc runs
    (comma-separated directories: the VALU_COUNTERS run, then the
    STALL_COUNTERS run; per wave instruction counts summed over the launch):
    VALU (including MFMA), SALU, MFMA, LDS and vector-memory instructions, the
    share of wave cycles spent waiting for an instruction to be issued; for the
    grouped GEMMs also the non-MFMA VALU and the SALU instructions per MFMA,
    LDS bank conflicts and waits."""
    dl = dirs.split(",")
    tab = _counter_table(dl, VALU_COUNTERS + STALL_COUNTERS)
    path = os.path.join(PROFILE_DIR, f"gemm_{workload}_valu.txt")
    with open(path, "w") as o:
        _profile_header(o, "Instruction mix and stalls per kernel launch", workload,
                        [f"timeout -s KILL 180 rocprofv3 --pmc {' '.join(cs)} -f csv -d {d} -o run -- "
                         + _bench_cmd(workload) for cs, d in zip((VALU_COUNTERS, STALL_COUNTERS), dl)],
                        f"--summarize-valu {dirs}")
        o.write("# kernel | dispatches | VALU | SALU | MFMA | LDS | VMEM | wait-inst share of wave cycles\n")
        for k in sorted(tab):
            t = tab[k]
            wait = t.get("SQ_WAIT_INST_ANY", 0.0) / max(t.get("SQ_WAVE_CYCLES", 1.0), 1.0)
            o.write(f"#   {k} | {t['n']} | {t.get('SQ_INSTS_VALU', 0):.0f} | {t.get('SQ_INSTS_SALU', 0):.0f} | "
                    f"{t.get('SQ_INSTS_MFMA', 0):.0f} | {t.get('SQ_INSTS_LDS', 0):.0f} | "
                    f"{t.get('SQ_INSTS_VMEM', 0):.0f} | {wait:.3f}\n")
        for g in ("l1_gemm", "l2_gemm", "l1_gemm_nvfp4"):
            if g not in tab or not tab[g].get("SQ_INSTS_MFMA"):
                continue
            t = tab[g]
            m = t["SQ_INSTS_MFMA"]
            key = g.replace("_gemm", "")
            o.write(f"{key}_valu_non_mfma_per_mfma = {(t['SQ_INSTS_VALU'] - m) / m:.3f}\n")
            o.write(f"{key}_salu_per_mfma = {t['SQ_INSTS_SALU'] / m:.3f}\n")
            o.write(f"{key}_lds_per_mfma = {t['SQ_INSTS_LDS'] / m:.3f}\n")
            o.write(f"{key}_wait_inst_share = {t['SQ_WAIT_INST_ANY'] / t['SQ_WAVE_CYCLES']:.4f}\n")
            if "SQ_WAIT_ANY" in t:
                o.write(f"{key}_wait_any_share = {t['SQ_WAIT_ANY'] / t['SQ_WAVE_CYCLES']:.4f}\n")
                o.write(f"{key}_wait_inst_lds_share = {t['SQ_WAIT_INST_LDS'] / t['SQ_WAVE_CYCLES']:.4f}\n")
                o.write(f"{key}_lds_bank_conflict_per_launch = {t['SQ_LDS_BANK_CONFLICT']:.0f}\n")
                o.write(f"{key}_lds_idx_active_per_launch = {t['SQ_LDS_IDX_ACTIVE']:.0f}\n")
                o.write(f"{key}_active_inst_vmem_per_launch = {t['SQ_ACTIVE_INST_VMEM']:.0f}\n")
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
