"""Fixed (calibrated) global scales on the GPU, through the C ABI
(nvfp4_cutedsl.py history, page 2, static-scale commit: warmup measures gs
for the L1 input and the L1 output; inference quantizes with them and no max
reduction).

Bar: the fixed-scale quantizer is bit-exact against the oracle (saturating
and small-scale cases included); the L1 epilogue that writes h as NVFP4 is
bit-exact against the oracle's fixed-scale quantization of the BF16 h that
the plain SiLU*up epilogue computes on the same inputs; the layer with fixed
scales equals the calibration pass bit for bit, its h codes are the oracle's
quantization of the calibration pass's h, and its output is within 1e-2 x
max|oracle| of the oracle layer given the same scales.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _cases import near_midpoint_blocks, quant_case
from _layer_checks import check_static_h
from _parity_log import record

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


def log(msg):
    print(f"[gpu-static] {msg}", flush=True)


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_quantized_moe_amd as nv
    return nv


def to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rel_err(got, ref):
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / scale if scale > 0 else float(np.abs(got).max())


def _own_gs(xb):
    a = np.abs(O.bf16_to_f64(xb))
    return O.global_scale(a.max() if a.size else 0.0)


# ------------------------------------------------------------- quantizer

@pytest.mark.parametrize("case", ["tiny_x", "t3_outliers", "ties", "scale_ties", "subnormal", "zeros", "ragged_rows"])
@pytest.mark.parametrize("factor", [1 / 64.0, 1.0, 7.5])
def test_quantize_static_bit_exact(nv, case, factor):
    xb = quant_case(case)
    gs = np.float32(_own_gs(xb) * np.float32(factor))
    log(f"quantize_static {case} shape={xb.shape} factor={factor}")
    q, sf = nv.nvfp4_quantize_static(to_bf16(xb), to_dev(np.array([gs], np.float32)))
    torch.cuda.synchronize()
    oq, osf, _ = O.quantize(xb, gs=gs)
    assert np.array_equal(sf.cpu().numpy(), osf)
    assert np.array_equal(q.cpu().numpy(), oq)


@pytest.mark.parametrize("x_exp,gs", [
    (-57, 2.0 ** -60), (-57, float(np.nextafter(np.float32(2.0 ** -60), np.float32(0)))), (-57, 2.0 ** -61),
    (63, 2.0 ** 60), (63, float(np.nextafter(np.float32(2.0 ** 60), np.float32(np.inf)))), (63, 2.0 ** 61),
    (0, 1e-25), (0, 1e25), (-130, 2.0 ** -135)])
def test_quantize_static_extreme_scales(nv, x_exp, gs):
    # global scales at and past the ends of the range where the block scale
    # code comes from the float32 estimate (the others take the float64
    # quotient), on inputs scaled to give codes across the E4M3 range; also
    # every block saturated (1e-25), every block zero (1e25) and BF16
    # subnormal inputs with a float32 subnormal scale
    rng = np.random.default_rng(abs(x_exp) + 7)
    x = (rng.standard_normal((24, 256)) * np.exp2(np.float64(x_exp))).astype(np.float32)
    xb = W.bf16_bits(x)
    g = np.float32(gs)
    log(f"quantize_static extreme gs={float(g):.3e} x_exp={x_exp}")
    q, sf = nv.nvfp4_quantize_static(to_bf16(xb), to_dev(np.array([g], np.float32)))
    torch.cuda.synchronize()
    oq, osf, _ = O.quantize(xb, gs=g)
    assert np.array_equal(sf.cpu().numpy(), osf)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_quantize_static_batched_and_zero_scale(nv):
    rng = np.random.default_rng(15)
    x = (rng.standard_normal((3, 40, 256)) * np.array([1.0, 300.0, 1e-3])[:, None, None]).astype(np.float32)
    xb = W.bf16_bits(x)
    gs = np.array([_own_gs(xb[0]), _own_gs(xb[1]) * np.float32(0.25), 0.0], np.float32)
    log("quantize_static batched B=3 (own, saturating, zero)")
    q, sf = nv.nvfp4_quantize_static(to_bf16(xb), to_dev(gs))
    torch.cuda.synchronize()
    for b in range(3):
        oq, osf, _ = O.quantize(xb[b], gs=gs[b])
        assert np.array_equal(sf[b].cpu().numpy(), osf), b
        assert np.array_equal(q[b].cpu().numpy(), oq), b
    assert not sf[2].any().item() and not (q[2] & 0x77).any().item()


@pytest.mark.parametrize("seed", [3, 4])
def test_quantize_static_near_midpoints(nv, seed):
    # elements within a few float32 ulps of an E2M1 midpoint, where a rounding
    # decided from an inexact quotient would go the wrong way
    bits, gs = near_midpoint_blocks(seed)
    log(f"quantize_static near midpoints seed={seed} blocks={bits.shape[0]}")
    q, sf = nv.nvfp4_quantize_static(to_bf16(bits), to_dev(gs))
    torch.cuda.synchronize()
    q, sf = q.cpu().numpy(), sf.cpu().numpy()
    for b in range(bits.shape[0]):
        oq, osf, _ = O.quantize(bits[b], gs=gs[b])
        assert np.array_equal(sf[b], osf) and np.array_equal(q[b], oq), b


# ---------------------------------------------------- L1 with NVFP4 output

GEMM_CASES = {
    # name: (L, N = 2I, K, T, counts)
    "ragged": (5, 256, 512, 50, [3, 0, 70, 33, 1]),
    "decode_like": (8, 512, 1024, 24, [1, 2, 0, 0, 3, 1, 0, 1]),
    "prefill_like": (3, 768, 768, 400, [171, 129, 100]),
    "many_items": (4, 4096, 256, 600, [700, 500, 0, 800]),   # two or more items per workgroup
    "single_stage": (3, 256, 128, 40, [20, 0, 33]),           # K = 128: one stage per item
}


@pytest.mark.parametrize("case", list(GEMM_CASES))
@pytest.mark.parametrize("tile_m", [32, 64, 96, 128])
@pytest.mark.parametrize("dual", [0, 1])
def test_gemm_silu_nvfp4(nv, case, tile_m, dual):
    L, N, K, T, counts = GEMM_CASES[case]
    seed = len(case) + tile_m + dual
    a_q, a_sf = W.random_fp4_operands(seed, T, K)
    b_q, b_sf = W.random_fp4_operands(seed + 1, L * N, K)
    b_q, b_sf = b_q.reshape(L, N, K // 2), b_sf.reshape(L, N, K // 16)
    rng = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S = int(offsets[-1])
    ri = rng.integers(0, T, S).astype(np.int32)
    a_gs = np.array([0.37], np.float32)
    b_gs = rng.uniform(0.01, 2.0, (L, 2) if dual else L).astype(np.float32)
    cap = S + 5
    tiles = O.tile_schedule(np.diff(offsets), offsets, tile_m)
    tt = np.zeros(nv.nvfp4_tile_table_len(cap, L, tile_m), np.int32)
    tt[0] = len(tiles)
    tt[1:1 + 2 * len(tiles)] = tiles.reshape(-1)
    I = N // 2
    # gs of h: 0.7 x the one of the oracle's h, so that some blocks saturate
    h_ref = O.silu_mul(O.grouped_gemm(a_q, a_sf, ri, a_gs[0], b_q, b_sf, b_gs, offsets), I)
    gs_h = np.float32(_own_gs(h_ref) * np.float32(0.7))
    d_args = (to_dev(a_q), to_dev(a_sf), to_dev(ri), to_dev(a_gs))
    b_packed = nv.nvfp4_pack_weights(to_dev(b_q), to_dev(b_sf))
    rest = (b_packed, to_dev(b_gs), to_dev(offsets), to_dev(tt), cap, tile_m)
    log(f"gemm_silu_nvfp4 {case} tile_m={tile_m} dual={dual} S={S}")
    hq = torch.full((cap, I // 2), 0xAB, dtype=torch.uint8, device=DEV)
    hsf = torch.full((cap, I // 16), 0xCD, dtype=torch.uint8, device=DEV)
    nv.nvfp4_grouped_gemm_silu_nvfp4(*d_args, *rest, to_dev(np.array([gs_h], np.float32)), d_q=hq, d_sf=hsf)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    h = nv.nvfp4_grouped_gemm(*d_args, *rest, epilogue=2 if dual else 1, amax_out=amax)
    torch.cuda.synchronize()
    got_q, got_sf = hq.cpu().numpy(), hsf.cpu().numpy()
    assert np.all(got_q[S:] == 0xAB) and np.all(got_sf[S:] == 0xCD), "rows outside the tiles were written"
    # the epilogue's quantization is the oracle's fixed-scale quantization of the BF16 h
    # that the same GEMM computes (the GPU's h: float32 summation order is not the oracle's)
    h_bits = h[:S].view(torch.int16).cpu().numpy().view(np.uint16)
    oq, osf, _ = O.quantize(h_bits, gs=gs_h)
    assert np.array_equal(got_sf[:S], osf), "epilogue block scales differ from the oracle's"
    assert np.array_equal(got_q[:S], oq), "epilogue codes differ from the oracle's"
    # and close to the oracle's codes for the oracle's own h
    if S:
        oq2, osf2, _ = O.quantize(h_ref, gs=gs_h)
        same = float((got_sf[:S] == osf2).mean())
        cos = O.cosine(O.dequantize(got_q[:S], got_sf[:S], gs_h), O.dequantize(oq2, osf2, gs_h))
        log(f"  bit-exact on the GPU's h; vs the oracle's own h: scale codes equal {same:.4f}, cosine of "
            f"dequantized h {cos:.6f}, saturated blocks {(osf2 == 0x7E).sum()}")
        record(f"gemm_silu_nvfp4:{case}:tile{tile_m}:dual{dual}", codes_bit_exact=True,
               cosine_vs_oracle_h=cos)
        assert cos >= 0.995


# ------------------------------------------------------------------ layer

def _layer(name):
    cfg = W.get_config(name)
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    return cfg, ids, w, x, wg, wu, wd


@pytest.mark.parametrize("name,fold", [("tiny", True), ("mid", True), ("mid_skew", True), ("mid_skew", False),
                                       ("mid_route3", True), ("wide_route", True), ("long_k1", True)])
def test_layer_static(nv, name, fold):
    cfg, ids, w, x, wg, wu, wd = _layer(name)
    log(f"layer_static {name} fold={fold} T={cfg.tokens} k={cfg.top_k} L={cfg.num_local}")
    weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd), fold=fold)
    d_x, d_ids, d_w = to_bf16(x), to_dev(ids), to_dev(w)
    # 1. with the scales the dynamic pass measures, the static pass is that pass, and
    #    its h codes are the oracle's quantization (fixed gs_h) of the dynamic pass's h
    T, k = ids.shape
    cap = T * k
    lay = nv.nvfp4_moe_ws_layout(T, k, cfg.hidden, cfg.inter, cfg.num_local)
    ws_d = torch.empty(lay["end"], dtype=torch.uint8, device=DEV)
    ws_s = torch.empty(lay["end"], dtype=torch.uint8, device=DEV)
    dyn = nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, cfg.expert_start, ws=ws_d)
    gs_cal = nv.calibrate_static_gs(weights, d_x, d_ids, d_w, cfg.expert_start)
    st = nv.nvfp4_moe_forward_static(weights, d_x, d_ids, d_w, cfg.expert_start, gs_cal, ws=ws_s)
    torch.cuda.synchronize()
    assert torch.equal(st.view(torch.int16), dyn.view(torch.int16))
    S = int(nv.ws_view(ws_d, lay, "offsets", torch.int32, (cfg.num_local + 1,))[-1].item())
    h_bits = nv.ws_view(ws_d, lay, "h", torch.int16, (cap, cfg.inter))[:S].cpu().numpy().view(np.uint16)
    check_static_h(nv, ws_s, lay, cap, cfg.inter, S, h_bits, gs_cal[1].item())
    # 2. against the oracle, both given the oracle's calibrated scales
    P = O.prepare_weights(wg, wu, wd, fold=fold)
    tr = O.moe_forward(x, ids, w, cfg.expert_start, P)
    assert gs_cal[0].item() == tr.gs_x
    gs_o = np.array([tr.gs_x, tr.gs_h], np.float32)
    for scale in (1.0, 1.25):
        xs = W.bf16_bits(O.bf16_to_f32(x) * np.float32(scale))
        ws_buf = torch.full((lay["end"] + 4096,), 0xA5, dtype=torch.uint8, device=DEV)   # canary bytes past the end
        ws = ws_buf[:lay["end"]]
        out = nv.nvfp4_moe_forward_static(weights, to_bf16(xs), d_ids, d_w, cfg.expert_start, to_dev(gs_o), ws=ws)
        torch.cuda.synchronize()
        assert bool((ws_buf[lay["end"]:] == 0xA5).all()), "bytes past the workspace were written"
        ref = O.moe_forward(xs, ids, w, cfg.expert_start, P, static_gs=(gs_o[0], gs_o[1]))
        H = cfg.hidden
        assert np.array_equal(nv.ws_view(ws, lay, "x_q", torch.uint8, (T, H // 2)).cpu().numpy(), ref.x_q)
        assert np.array_equal(nv.ws_view(ws, lay, "x_sf", torch.uint8, (T, H // 16)).cpu().numpy(), ref.x_sf)
        err = rel_err(out.float().cpu().numpy(), O.bf16_to_f32(ref.out))
        log(f"  x{scale}: out rel err {err:.3e}")
        record(f"layer_static:{name}:fold{int(fold)}:x{scale}", rel_err=err, h_codes_bit_exact=True)
        assert err <= TOL


def test_layer_static_edge_cases(nv):
    cfg, ids, w, x, wg, wu, wd = _layer("tiny")
    weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd))
    gs = to_dev(np.array([0.01, 0.02], np.float32))
    log("layer_static: no local expert, T = 0, zero scales")
    out = nv.nvfp4_moe_forward_static(weights, to_bf16(x), to_dev(ids), to_dev(w), 100, gs)
    e = nv.nvfp4_moe_forward_static(weights, to_bf16(x[:0]), to_dev(ids[:0]), to_dev(w[:0]), 0, gs)
    z = nv.nvfp4_moe_forward_static(weights, to_bf16(x), to_dev(ids), to_dev(w), cfg.expert_start,
                                    to_dev(np.zeros(2, np.float32)))
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item() and e.shape == (0, cfg.hidden)
    assert not z.float().abs().sum().item()


@pytest.mark.parametrize("name", ["tiny", "mid_skew"])   # decode-shaped (BF16 h) and prefill-shaped (NVFP4 epilogue)
def test_layer_static_graph_replay(nv, name):
    cfg, ids, w, x, wg, wu, wd = _layer(name)
    weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd))
    T, k = ids.shape
    d_x, d_ids, d_w = to_bf16(x), to_dev(ids), to_dev(w)
    gs = nv.calibrate_static_gs(weights, d_x, d_ids, d_w, cfg.expert_start)
    lay = nv.nvfp4_moe_ws_layout(T, k, cfg.hidden, cfg.inter, cfg.num_local)
    ws = torch.empty(lay["end"], dtype=torch.uint8, device=DEV)
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=DEV)
    fwd = lambda: nv.nvfp4_moe_forward_static(weights, d_x, d_ids, d_w, cfg.expert_start, gs, out=out, ws=ws)
    log("layer_static graph: eager warm-up on a side stream")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fwd()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for r in range(3):
        out.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"layer_static graph: replay {r}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
    # the replayed output against the oracle layer given the same fixed scales
    gs_np = gs.cpu().numpy()
    ref = O.moe_forward(x, ids, w, cfg.expert_start, O.prepare_weights(wg, wu, wd), static_gs=(gs_np[0], gs_np[1]))
    err = rel_err(out.float().cpu().numpy(), O.bf16_to_f32(ref.out))
    log(f"layer_static graph: replay vs oracle rel err {err:.3e}")
    record(f"graph_static:{name}", rel_err=err, replays_equal_eager=3)
    assert err <= TOL
