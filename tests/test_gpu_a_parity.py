"""HIP path vs the CPU oracle, through the C ABI, at sizes the oracle finishes
in seconds (several tiles per dimension, ragged tails, empty experts).

Bar: bit-exact for quantized codes, scales, global scales, routing arrays,
the scale fold, the weighted scatter and the re-quantization of the layer's
own h; layer and GEMM outputs within 1e-2 x max|oracle| (float32
accumulation order differs), and BF16 GEMM outputs also within a few BF16
ulps element by element; cosine >= 0.98 against the BF16 layer built from
the dequantized NVFP4 weights.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _cases import pack_weights_np, quant_case
from _layer_checks import check_requant_h
from _parity_log import record, ulp_error

pytestmark = pytest.mark.gpu
TOL = 1e-2
ULP_TOL_BF16 = 2.0   # D = RN_bf16(alpha * sum), BF16 ulps (see test_grouped_gemm)
ULP_TOL_SILU = 4.0   # h = RN_bf16(silu(RN_bf16(g)) * RN_bf16(u)), BF16 ulps


def log(msg):
    print(f"[gpu-parity] {msg}", flush=True)


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_quantized_moe_amd as nv
    return nv


DEV = "cuda:0"


def to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bits_of(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rel_err(got, ref):
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / scale if scale > 0 else float(np.abs(got).max())


# ------------------------------------------------------------------- quantizer

@pytest.mark.parametrize("case", ["tiny_x", "mid_x", "t3_outliers", "ties", "scale_ties", "subnormal", "zeros",
                                  "wide", "ragged_rows", "quant_full", "large_outliers"])
def test_quantize_bit_exact(nv, case):
    xb = quant_case(case)
    log(f"quantize {case} shape={xb.shape}")
    q, sf, gs = nv.nvfp4_quantize(to_bf16(xb))
    torch.cuda.synchronize()
    oq, osf, ogs = O.quantize(xb)
    assert gs.cpu().numpy()[0] == ogs
    assert np.array_equal(sf.cpu().numpy(), osf)
    assert np.array_equal(q.cpu().numpy(), oq)
    record(f"quantize:{case}", bit_exact_arrays=3)


@pytest.mark.parametrize("x_exp", [-100, -52, -50, 70, -128])
def test_quantize_tiny_and_huge_tensors(nv, x_exp):
    # tensors whose own global scale amax/2688 lies outside [2^-60, 2^60] (the
    # block scale codes then come from the float64 quotient: 2^-100, 2^-52,
    # 2^70, and BF16 subnormals at 2^-128) or just inside it (2^-50)
    rng = np.random.default_rng(x_exp + 200)
    x = (rng.standard_normal((32, 512)) * np.exp2(np.float64(x_exp))).astype(np.float32)
    xb = W.bf16_bits(x)
    log(f"quantize scaled by 2^{x_exp}")
    q, sf, gs = nv.nvfp4_quantize(to_bf16(xb))
    torch.cuda.synchronize()
    oq, osf, ogs = O.quantize(xb)
    assert gs.cpu().numpy()[0] == ogs
    assert np.array_equal(sf.cpu().numpy(), osf)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_quantize_batched_and_amax_in(nv):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((3, 40, 256)) * np.array([1.0, 300.0, 1e-3])[:, None, None]).astype(np.float32)
    x[1, 0, 0] = 4000.0
    xb = W.bf16_bits(x)
    log("quantize batched B=3")
    q, sf, gs = nv.nvfp4_quantize(to_bf16(xb))
    oq, osf, ogs = O.quantize_batched(xb)
    assert np.array_equal(gs.cpu().numpy(), ogs)
    assert np.array_equal(sf.cpu().numpy(), osf) and np.array_equal(q.cpu().numpy(), oq)
    # external amax (the h path): 2688 forces gs = 1 and saturates the 4000 block
    amax = np.array([2.0, 2688.0, 5e-3], np.float32)
    log("quantize amax_in")
    q2, sf2, gs2 = nv.nvfp4_quantize(to_bf16(xb), amax_in=to_dev(amax))
    oq2, osf2, ogs2 = O.quantize_batched(xb, amax=amax)
    assert np.array_equal(gs2.cpu().numpy(), ogs2)
    assert np.array_equal(sf2.cpu().numpy(), osf2) and np.array_equal(q2.cpu().numpy(), oq2)


# --------------------------------------------------------------------- routing

def _router_case(name):
    if name in W.CONFIGS and isinstance(W.CONFIGS[name], W.LayerConfig):
        cfg = W.get_config(name)
        ids, w = W.make_router(cfg)
        return ids, w, cfg.expert_start, cfg.num_local
    rng = np.random.default_rng(7)
    if name == "random_out_of_range":
        ids = rng.integers(-5, 70, (77, 5)).astype(np.int32)
        return ids, rng.random((77, 5)).astype(np.float32), 10, 40
    if name == "empty":
        return np.zeros((0, 4), np.int32), np.zeros((0, 4), np.float32), 0, 8
    if name == "none_local":
        ids = rng.integers(0, 96, (50, 8)).astype(np.int32)
        return ids, rng.random((50, 8)).astype(np.float32), 96, 48
    if name in ("edge_1024", "edge_1025"):
        # flat sizes on both sides of the single-workgroup route path
        T, k = (128, 8) if name == "edge_1024" else (205, 5)
        ids = rng.integers(0, 64, (T, k)).astype(np.int32)
        return ids, rng.random((T, k)).astype(np.float32), 16, 32
    if name == "big_L":
        ids = rng.integers(0, 3000, (600, 6)).astype(np.int32)
        return ids, rng.random((600, 6)).astype(np.float32), 500, 2100
    if name == "many_counts":
        # 36 chunks x 2000 local experts = 72000 histogram entries: past the one-launch scan/scatter's
        # limit (65536), so the separate scan and scatter kernels run
        ids = rng.integers(0, 2400, (4500, 8)).astype(np.int32)
        return ids, rng.random((4500, 8)).astype(np.float32), 300, 2000
    raise KeyError(name)


@pytest.mark.parametrize("case", ["tiny", "mid", "mid_k1", "mid_skew", "decode", "prefill", "skewed",
                                  "random_out_of_range", "empty", "none_local", "big_L", "edge_1024",
                                  "edge_1025", "many_counts"])
@pytest.mark.parametrize("tile_m", [32, 96, 128])
def test_route_bit_exact(nv, case, tile_m):
    ids, w, start, L = _router_case(case)
    log(f"route {case} T={ids.shape[0]} k={ids.shape[1]} L={L} tile_m={tile_m}")
    r = nv.moe_route_slots(to_dev(ids), to_dev(w), start, L, tile_m)
    torch.cuda.synchronize()
    o = O.route(ids, w, start, L)
    for key in ("counts", "offsets", "slot_token", "slot_expert", "slot_weight", "token_slot"):
        assert np.array_equal(r[key].cpu().numpy(), o[key]), key
    tiles = O.tile_schedule(o["counts"], o["offsets"], tile_m)
    tt = r["tile_table"].cpu().numpy()
    assert tt[0] == len(tiles)
    assert np.array_equal(tt[1:1 + 2 * len(tiles)].reshape(-1, 2), tiles)


# ------------------------------------------------------------------------ fold

def test_fold_bit_exact(nv):
    rng = np.random.default_rng(11)
    L, I, K = 6, 96, 512
    sf = rng.integers(0, 0x7F, (L, 2 * I, K // 16)).astype(np.uint8)
    g = np.array([1.0, 0.5, 3e-4, 2.0, 0.0, 7.5e-6], np.float32)
    u = np.array([1.0, 0.7, 9e-3, 0.06, 1.0, 2.2e-4], np.float32)
    log("fold")
    d_sf = to_dev(sf)
    gs1 = nv.nvfp4_fold_scales(d_sf, to_dev(g), to_dev(u))
    osf, ogs1 = O.fold_gate_up(sf, g, u, I)
    assert np.array_equal(gs1.cpu().numpy(), ogs1)
    assert np.array_equal(d_sf.cpu().numpy(), osf)


# ------------------------------------------------------------------- scatter

@pytest.mark.parametrize("T,k,H", [(37, 3, 256), (5, 8, 7168), (64, 1, 64), (6, 64, 512), (33, 8, 8320),
                                   (2048, 8, 7168)])
def test_scatter_bit_exact(nv, T, k, H):
    rng = np.random.default_rng(T * 131 + k)
    S = int(T * k * 0.6)
    y = W.bf16_bits(rng.standard_normal((S, H)).astype(np.float32))
    ts = np.full(T * k, -1, np.int32)
    ts[rng.choice(T * k, S, replace=False)] = rng.permutation(S).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    log(f"scatter T={T} k={k} H={H}")
    out = nv.moe_weighted_scatter(to_bf16(y), to_dev(ts), to_dev(w))
    assert np.array_equal(bits_of(out), O.scatter(y, ts, w))


# ------------------------------------------------------------- weight packing

@pytest.mark.parametrize("shape", [(1, 32, 128), (3, 96, 384), (2, 6144 // 8, 7168 // 4)])
def test_pack_weights(nv, shape):
    B, N, K = shape
    rng = np.random.default_rng(N + K)
    q = rng.integers(0, 256, (B, N, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 256, (B, N, K // 16), dtype=np.uint8)
    log(f"pack B={B} N={N} K={K}")
    got = nv.nvfp4_pack_weights(to_dev(q), to_dev(sf))
    torch.cuda.synchronize()
    assert got.numel() == nv.nvfp4_packed_bytes(B, N, K)
    assert np.array_equal(got.cpu().numpy(), pack_weights_np(q, sf))


def test_pack_weights_rejects_bad_shapes(nv):
    q = torch.zeros((1, 48, 64), dtype=torch.uint8, device=DEV)
    sf = torch.zeros((1, 48, 8), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        nv.nvfp4_pack_weights(q, sf)
    assert nv.nvfp4_packed_bytes(1, 48, 128) == -1


# --------------------------------------------------------------- grouped GEMM

def _gemm_inputs(seed, L, N, K, T, counts, gather):
    a_q, a_sf = W.random_fp4_operands(seed, T, K)
    b_q, b_sf = W.random_fp4_operands(seed + 1, L * N, K)
    b_q, b_sf = b_q.reshape(L, N, K // 2), b_sf.reshape(L, N, K // 16)
    rng = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S = int(offsets[-1])
    row_index = rng.integers(0, T, S).astype(np.int32) if gather else None
    a_gs = np.array([0.37], np.float32)
    b_gs = rng.uniform(0.01, 2.0, L).astype(np.float32)
    return a_q, a_sf, row_index, a_gs, b_q, b_sf, b_gs, offsets


GEMM_CASES = {
    # name: (L, N, K, T, counts, gather)
    "ragged_gather": (5, 256, 512, 50, [3, 0, 70, 33, 1], True),
    "decode_like": (8, 512, 1024, 24, [1, 2, 0, 0, 3, 1, 0, 1], True),
    "prefill_like": (3, 384, 768, 400, [171, 129, 100], True),
    "no_gather_long_k": (2, 128, 2048, 90, [45, 45], False),
    "one_expert_empty": (4, 256, 256, 10, [0, 0, 0, 0], True),
    # more items than workgroups: every workgroup runs two or more items, so the
    # loads of one item's last stages run into the next item (3 loop stages per
    # item with 3 in flight: the LDS buffer parity flips from item to item)
    "many_items": (4, 8192, 256, 600, [700, 500, 0, 800], True),
    # one K stage: fewer stages than the ring runs ahead (the rest read zeros)
    "single_stage": (3, 256, 128, 40, [20, 0, 33], True),
}


@pytest.mark.parametrize("case", list(GEMM_CASES))
@pytest.mark.parametrize("tile_m", [32, 64, 96, 128])
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_grouped_gemm(nv, case, tile_m, epi):
    L, N, K, T, counts, gather = GEMM_CASES[case]
    a_q, a_sf, ri, a_gs, b_q, b_sf, b_gs, offsets = _gemm_inputs(len(case), L, N, K, T, counts, gather)
    if epi == 2:   # gate and up halves with their own global scales
        b_gs = np.stack([b_gs, np.random.default_rng(L + N).uniform(0.01, 2.0, L).astype(np.float32)], axis=1)
    S = int(offsets[-1])
    cap = max(S, 1) + 7
    if ri is None and a_q.shape[0] < cap:
        # without a row index slot s reads row s, so the A operand spans every slot of the capacity
        a_q = np.concatenate([a_q, np.zeros((cap - a_q.shape[0], a_q.shape[1]), np.uint8)])
        a_sf = np.concatenate([a_sf, np.zeros((cap - a_sf.shape[0], a_sf.shape[1]), np.uint8)])
    counts_np = np.diff(offsets)
    tiles = O.tile_schedule(counts_np, offsets, tile_m)
    tt = np.zeros(nv.nvfp4_tile_table_len(cap, L, tile_m), np.int32)
    tt[0] = len(tiles)
    tt[1:1 + 2 * len(tiles)] = tiles.reshape(-1)
    n_out = N // 2 if epi in (1, 2) else N
    canary = torch.full((cap, n_out), -7.0, dtype=torch.bfloat16, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    log(f"gemm {case} tile_m={tile_m} epi={epi} S={S}")
    b_packed = nv.nvfp4_pack_weights(to_dev(b_q), to_dev(b_sf))
    d = nv.nvfp4_grouped_gemm(to_dev(a_q), to_dev(a_sf), None if ri is None else to_dev(ri), to_dev(a_gs),
                              b_packed, to_dev(b_gs), to_dev(offsets), to_dev(tt), cap, tile_m,
                              epilogue=epi, d=canary, amax_out=amax if epi in (1, 2) else None)
    torch.cuda.synchronize()
    got = d.float().cpu().numpy()
    assert np.all(got[S:] == -7.0), "rows outside the tiles were written"
    g = O.grouped_gemm(a_q, a_sf, ri, a_gs[0], b_q, b_sf, b_gs, offsets)
    if epi in (1, 2):
        ref = O.bf16_to_f32(O.silu_mul(g, N // 2))
        h = got[:S]
        assert amax.item() == (float(np.abs(h).max()) if S else 0.0)
    else:
        ref = O.bf16_to_f32(O.f32_to_bf16(g))
    if S:
        err = rel_err(got[:S], ref)
        ulps = ulp_error(got[:S], ref)
        log(f"  rel err {err:.3e}  max {ulps:.2f} BF16 ulps")
        record(f"gemm:{case}:tile{tile_m}:epi{epi}", rel_err=err, ulp_err=ulps)
        assert err <= TOL
        # D = RN_bf16(alpha * sum): float32 sums in another order differ by far less than
        # a BF16 ulp of a typical element, so the two roundings differ by at most one ulp
        # (a second one only for elements near the floor of ulp_error, whose sums cancel);
        # the SiLU*up epilogue rounds g and u to BF16 first and uses its own exp, so h may
        # move by a few ulps
        assert ulps <= (ULP_TOL_BF16 if epi == 0 else ULP_TOL_SILU)


# --------------------------------------------------------------------- layer

def _layer_inputs(name):
    cfg = W.get_config(name)
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    return cfg, ids, w, x, wg, wu, wd


def _deq_ref(P, cfg, x, ids, w):
    L, I = cfg.num_local, cfg.inter
    f = lambda q, sf, gs: O.f32_to_bf16(O.dequantize(q, sf, gs, np.float32))
    g1 = np.asarray(P["w1_gs"])
    gs_g = g1[:, 0] if g1.ndim == 2 else g1
    gs_u = g1[:, 1] if g1.ndim == 2 else g1
    dg = np.stack([f(P["w1_q"][e, :I], P["w1_sf"][e, :I], gs_g[e]) for e in range(L)])
    du = np.stack([f(P["w1_q"][e, I:], P["w1_sf"][e, I:], gs_u[e]) for e in range(L)])
    dd = np.stack([f(P["w2_q"][e], P["w2_sf"][e], P["w2_gs"][e]) for e in range(L)])
    return O.bf16_reference_layer(x, ids, w, cfg.expert_start, dg, du, dd)


@pytest.mark.parametrize("name,fold", [("tiny", True), ("mid", True), ("mid_k1", True), ("mid_skew", True),
                                       ("mid_route3", True), ("tiny", False), ("mid_skew", False),
                                       ("wide_route", True), ("long_k1", True)])
def test_layer(nv, name, fold):
    cfg, ids, w, x, wg, wu, wd = _layer_inputs(name)
    log(f"layer {name} fold={fold} T={cfg.tokens} k={cfg.top_k} L={cfg.num_local} H={cfg.hidden} I={cfg.inter}")
    weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd), keep_unpacked=True, fold=fold)
    P = O.prepare_weights(wg, wu, wd, fold=fold)
    for key in ("w1_q", "w1_sf", "w1_gs", "w2_q", "w2_sf", "w2_gs"):
        assert np.array_equal(getattr(weights, key).cpu().numpy(), P[key]), key
    assert np.array_equal(weights.w1.cpu().numpy(), pack_weights_np(P["w1_q"], P["w1_sf"]))
    assert np.array_equal(weights.w2.cpu().numpy(), pack_weights_np(P["w2_q"], P["w2_sf"]))
    T, k = ids.shape
    H = cfg.hidden
    lay = nv.nvfp4_moe_ws_layout(T, k, H, cfg.inter, cfg.num_local)
    guard = 4096
    ws_buf = torch.full((lay["end"] + guard,), 0xA5, dtype=torch.uint8, device=DEV)   # canary bytes past the workspace
    ws = ws_buf[:lay["end"]]
    buf = torch.full((T + 2, H), -3.0, dtype=torch.bfloat16, device=DEV)   # canary rows around out
    out = nv.nvfp4_moe_forward(weights, to_bf16(x), to_dev(ids), to_dev(w), cfg.expert_start,
                               out=buf[1:T + 1], ws=ws)
    torch.cuda.synchronize()
    b = buf.float().cpu().numpy()
    assert np.all(b[0] == -3.0) and np.all(b[T + 1] == -3.0)
    assert bool((ws_buf[lay["end"]:] == 0xA5).all()), "bytes past the workspace were written"
    tr = O.moe_forward(x, ids, w, cfg.expert_start, P)
    # stage checks from the workspace: activation quantization and routing are exact
    assert np.array_equal(nv.ws_view(ws, lay, "x_q", torch.uint8, (T, H // 2)).cpu().numpy(), tr.x_q)
    assert np.array_equal(nv.ws_view(ws, lay, "x_sf", torch.uint8, (T, H // 16)).cpu().numpy(), tr.x_sf)
    scal = nv.ws_view(ws, lay, "scalars", torch.float32, (4,)).cpu().numpy()
    assert scal[0] == tr.gs_x
    cap = T * k
    for key in ("slot_token", "token_slot", "slot_expert"):
        assert np.array_equal(nv.ws_view(ws, lay, key, torch.int32, (cap,)).cpu().numpy(), tr.routing[key]), key
    S = tr.routing["S"]
    h_t = nv.ws_view(ws, lay, "h", torch.bfloat16, (cap, cfg.inter))[:S]
    h = h_t.float().cpu().numpy()
    assert scal[1] == np.abs(h).max()                      # amax of h, taken in the epilogue
    check_requant_h(nv, ws, lay, cap, cfg.inter, S, bits_of(h_t), scal)
    eh = rel_err(h, O.bf16_to_f32(tr.h))
    got = out.float().cpu().numpy()
    ref = O.bf16_to_f32(tr.out)
    err = rel_err(got, ref)
    cos = O.cosine(got, _deq_ref(P, cfg, x, ids, w))
    log(f"  h rel err {eh:.3e}  out rel err {err:.3e}  cosine {cos:.4f}  S={S}")
    record(f"layer:{name}:fold{int(fold)}", h_rel_err=eh, rel_err=err, cosine_deq=cos, h_requant_bit_exact=True)
    assert eh <= TOL and err <= TOL
    assert cos >= 0.98
    # run-to-run determinism
    out2 = nv.nvfp4_moe_forward(weights, to_bf16(x), to_dev(ids), to_dev(w), cfg.expert_start)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))


def test_layer_no_local_tokens_and_empty(nv):
    cfg, ids, w, x, wg, wu, wd = _layer_inputs("tiny")
    weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd))
    log("layer with no local expert")
    out = nv.nvfp4_moe_forward(weights, to_bf16(x), to_dev(ids), to_dev(w), 100)
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item()
    log("layer with T = 0")
    e = nv.nvfp4_moe_forward(weights, to_bf16(x[:0]), to_dev(ids[:0]), to_dev(w[:0]), 0)
    torch.cuda.synchronize()
    assert e.shape == (0, cfg.hidden)


# ------------------------------------------------------------ layer edge cases

def _edge_layer(nv, name, ids, w, x, cfg_name="mid"):
    cfg = W.get_config(cfg_name)
    wg, wu, wd = W.make_weights(cfg)
    weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd))
    P = O.prepare_weights(wg, wu, wd)
    log(f"layer edge case {name}: T={ids.shape[0]} k={ids.shape[1]}")
    out = nv.nvfp4_moe_forward(weights, to_bf16(x), to_dev(ids), to_dev(w), cfg.expert_start)
    torch.cuda.synchronize()
    tr = O.moe_forward(x, ids, w, cfg.expert_start, P)
    return out.float().cpu().numpy(), O.bf16_to_f32(tr.out), tr


def test_layer_zero_activations(nv):
    """x = 0: gs_x = 0, every scale and magnitude 0, h = 0, gs_h = 0, out = 0."""
    cfg = W.get_config("mid")
    ids, w = W.make_router(cfg)
    x = np.zeros((cfg.tokens, cfg.hidden), np.uint16)
    got, ref, tr = _edge_layer(nv, "zero x", ids, w, x)
    assert tr.gs_x == 0 and tr.gs_h == 0
    assert np.array_equal(got, ref) and not np.any(got)


def test_layer_single_token(nv):
    cfg = W.get_config("mid")
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    got, ref, _ = _edge_layer(nv, "one token", ids[:1], w[:1], x[:1])
    assert rel_err(got, ref) <= TOL


def test_layer_all_tokens_one_expert(nv):
    """Top-1 with every token on the same local expert: one group of T rows
    (several row tiles), every other expert empty."""
    cfg = W.get_config("mid")
    T = 300
    ids = np.full((T, 1), cfg.expert_start + 5, np.int32)
    w = np.ones((T, 1), np.float32)
    x = W.make_activations(cfg)
    x = np.concatenate([x, x])[:T]
    got, ref, tr = _edge_layer(nv, "one expert", ids, w, x)
    assert tr.routing["counts"][5] == T and tr.routing["S"] == T
    assert rel_err(got, ref) <= TOL


def test_layer_duplicate_ids_in_a_token(nv):
    """The same expert twice in one token's top-k: two slots, summed in j order."""
    cfg = W.get_config("mid")
    ids, w = W.make_router(cfg)
    ids = ids.copy()
    ids[:, 1] = ids[:, 0]
    x = W.make_activations(cfg)
    got, ref, tr = _edge_layer(nv, "duplicate ids", ids, w, x)
    assert rel_err(got, ref) <= TOL


def test_layers_on_two_streams(nv):
    """Two different layers (their own weights, inputs and workspaces) issued
    alternately on two streams with no synchronization between them: each
    call's output equals that layer's output computed alone, bit for bit (the
    library keeps no state between calls besides the caller's buffers)."""
    runs = []
    for name in ("mid", "mid_skew"):
        cfg, ids, w, x, wg, wu, wd = _layer_inputs(name)
        weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd))
        args = (weights, to_bf16(x), to_dev(ids), to_dev(w), cfg.expert_start)
        alone = nv.nvfp4_moe_forward(*args)
        torch.cuda.synchronize()
        runs.append((args, bits_of(alone)))
    log("layers mid and mid_skew on two streams, 4 calls each")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    torch.cuda.synchronize()
    for _ in range(4):
        for i, (args, _) in enumerate(runs):
            with torch.cuda.stream(streams[i]):
                outs[i].append(nv.nvfp4_moe_forward(*args))
    torch.cuda.synchronize()
    for i, (_, ref) in enumerate(runs):
        for o in outs[i]:
            assert np.array_equal(bits_of(o), ref), i


@pytest.mark.parametrize("name", ["tiny", "mid_route3", "long_k1"])
def test_layer_with_stage_events(nv, name):
    """nvfp4_moe_forward_stage_events (the layer with events between its
    launches, for timing) gives the plain call's output bit for bit; its events
    are recorded in stage order (every span >= 0), with some of them left out
    too."""
    cfg, ids, w, x, wg, wu, wd = _layer_inputs(name)
    weights = nv.prepare_weights(to_bf16(wg), to_bf16(wu), to_bf16(wd))
    args = (weights, to_bf16(x), to_dev(ids), to_dev(w), cfg.expert_start)
    ref = nv.nvfp4_moe_forward(*args)
    torch.cuda.synchronize()
    log(f"layer {name} with stage events")
    for skip in ((), (2, 5)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(nv.STAGES) + 1)]
        for e in ev:
            e.record()
        torch.cuda.synchronize()
        events = [None if i in skip else e for i, e in enumerate(ev)]
        out = nv.nvfp4_moe_forward_stage_events(*args, events)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), bits_of(ref))
        kept = [e for e in events if e is not None]
        for a, b in zip(kept, kept[1:]):
            assert a.elapsed_time(b) >= 0.0


# ------------------------------------------------------- binding validation

def test_binding_rejects_bad_buffers(nv):
    """The library sees only addresses, so the binding checks the shapes,
    dtypes and sizes of the tensors it passes; a bad one raises before any
    launch."""
    T, k, L, H, I = 6, 2, 2, 256, 128
    w = nv.prepare_weights(torch.zeros((L, I, H), dtype=torch.bfloat16, device=DEV),
                           torch.zeros((L, I, H), dtype=torch.bfloat16, device=DEV),
                           torch.zeros((L, H, I), dtype=torch.bfloat16, device=DEV))
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    tw = torch.ones((T, k), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="x"):
        nv.nvfp4_moe_forward(w, x[:, :128].contiguous(), ids, tw, 0)
    with pytest.raises(ValueError, match="topk_w"):
        nv.nvfp4_moe_forward(w, x, ids, tw[:, :1].contiguous(), 0)
    with pytest.raises(ValueError, match="out"):
        nv.nvfp4_moe_forward(w, x, ids, tw, 0, out=torch.empty((T - 1, H), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="out"):
        nv.nvfp4_moe_forward(w, x, ids, tw, 0, out=torch.empty((T, H), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="ws"):
        nv.nvfp4_moe_forward(w, x, ids, tw, 0, ws=torch.empty(1024, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError, match="topk_w"):
        nv.moe_route_slots(ids, tw[:-1].contiguous(), 0, L, 32)
    with pytest.raises(ValueError, match="q"):
        nv.nvfp4_quantize(x, q=torch.empty((T, H // 2 - 1), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError, match="gs"):
        nv.nvfp4_quantize_static(x.view(2, T // 2, H), torch.ones(1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="x"):
        nv.nvfp4_quantize(x.t())          # not contiguous
    r = nv.moe_route_slots(ids, tw, 0, L, 32)
    xq, xsf, gs = nv.nvfp4_quantize(x)
    cap = T * k
    with pytest.raises(ValueError, match="d"):
        nv.nvfp4_grouped_gemm(xq, xsf, r["slot_token"], gs, w.w1, w.w1_gs, r["offsets"], r["tile_table"], cap, 32,
                              epilogue=nv.EPI_SILU_MUL, d=torch.empty((cap - 1, I), dtype=torch.bfloat16, device=DEV),
                              amax_out=torch.zeros(1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="tile_table"):
        nv.nvfp4_grouped_gemm(xq, xsf, r["slot_token"], gs, w.w1, w.w1_gs, r["offsets"], r["tile_table"][:3].contiguous(),
                              cap, 32, epilogue=nv.EPI_SILU_MUL, amax_out=torch.zeros(1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="a_q"):
        nv.nvfp4_grouped_gemm(xq[:, :64].contiguous(), xsf, r["slot_token"], gs, w.w1, w.w1_gs, r["offsets"],
                              r["tile_table"], cap, 32, epilogue=nv.EPI_SILU_MUL,
                              amax_out=torch.zeros(1, dtype=torch.float32, device=DEV))
    # without a row index, slot s reads row s: T rows cannot serve rows_cap = T * k slots
    with pytest.raises(ValueError, match="a_q"):
        nv.nvfp4_grouped_gemm(xq, xsf, None, gs, w.w1, w.w1_gs, r["offsets"], r["tile_table"], cap, 32,
                              epilogue=nv.EPI_SILU_MUL, amax_out=torch.zeros(1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="b_packed"):
        nv.nvfp4_grouped_gemm(xq, xsf, r["slot_token"], gs, w.w1[..., :2048].contiguous(), w.w1_gs, r["offsets"],
                              r["tile_table"], cap, 32, epilogue=nv.EPI_SILU_MUL,
                              amax_out=torch.zeros(1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="w2_gs"):
        nv.MoEWeights(w.w1, w.w1_gs, w.w2, w.w2_gs.double())
    with pytest.raises(ValueError, match="w2_gs"):
        nv.MoEWeights(w.w1, w.w1_gs, w.w2, w.w2_gs[:1].contiguous())
    with pytest.raises(ValueError, match="w1_gs"):
        nv.MoEWeights(w.w1, torch.ones((L, 3), dtype=torch.float32, device=DEV), w.w2, w.w2_gs)
    torch.cuda.synchronize()
