"""Grouped GEMMs, SiLU*up, weighted scatter and the whole layer — oracle
(test infrastructure only).

The six steps follow the tests history, moe_pipeline commit: quantize the
BF16 activation to NVFP4; L1 GEMM (gate+up) NVFP4 x NVFP4 -> BF16; SiLU(gate)
* up in BF16; re-quantize to NVFP4; L2 GEMM (down_proj) NVFP4 x NVFP4 -> BF16;
scatter back with the routing weights -> BF16. Also:
  * nvfp4_mega_moe.py history, alpha commit: D = alpha * A @ B with alpha the
    product of the activation's and the weight's global scales; L1 takes the
    activation quantizer's gs, L2 the gs returned by re-quantizing h.
  * src history, gather commits: L1 gathers activation rows by slot_token,
    L2 reads its rows in slot order with no gather.
  * nvfp4_cutedsl.py history, intermediate-split commit: gate = L1 out[:, :I],
    up = L1 out[:, I:].
  * nvfp4_cutedsl.py history, GPU-native routing commit: the scatter adds
    each slot's row times its routing weight into its token's row.
  * nvfp4_mega_moe.py history, expert-parallel note: the layer writes a local
    partial output; the caller reduces across ranks.

Readings: dequantized operands are exact (an E2M1 value times an E4M3 scale
has at most 6 significant bits), products accumulate in float32 (np.matmul),
alpha = RN_f32(gs_a * gs_b) multiplies the float32 sum; BF16 roundings sit
where the pipeline names BF16 (L1 out, SiLU*up, L2 out, final output);
silu(g) = g / (1 + exp(-g)) in float32 on the BF16 gate, times the BF16 up,
rounded once; the scatter sums w * Y over j = 0..k-1 in float32 in increasing
j and rounds once; a token with no local expert gets zeros.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16
from .quantize import quantize, dequantize
from .route import route


def _deq32(q, sf):
    # exact: every dequantized element has at most 6 significant bits
    return dequantize(q, sf, 1.0, dtype=np.float32)


def grouped_gemm(a_q, a_sf, a_row_index, a_gs, b_q, b_sf, b_gs, offsets, map_fn=map) -> np.ndarray:
    """Per-expert NVFP4 GEMM in slot order.

    Row s in [offsets[e], offsets[e+1]) uses A row a_row_index[s] (or s when
    a_row_index is None) and expert e's weight b_q[e] [N, K/2] / b_sf[e] [N, K/16].
    Returns float32 [S, N] = RN_f32(alpha_e * (A_hat @ W_hat_e^T)) with
    alpha_e = RN_f32(a_gs * b_gs[e]). With b_gs of shape [L, 2] (gate and up
    global scales of an unfolded L1 weight), columns [0, N/2) take
    RN_f32(a_gs * b_gs[e, 0]) and columns [N/2, N) RN_f32(a_gs * b_gs[e, 1]).
    Experts are independent; map_fn lets a caller run them on several
    threads (same result).
    """
    offsets = np.asarray(offsets)
    L = len(offsets) - 1
    S = int(offsets[-1])
    N = b_q.shape[1]
    out = np.zeros((S, N), np.float32)

    def one(e):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            return
        rows = np.arange(r0, r1) if a_row_index is None else np.asarray(a_row_index[r0:r1])
        a_hat = _deq32(a_q[rows], a_sf[rows])
        w_hat = _deq32(b_q[e], b_sf[e])
        acc = np.matmul(a_hat, w_hat.T)
        gs_e = np.asarray(b_gs[e], np.float32)
        if gs_e.ndim == 0:
            out[r0:r1] = acc * np.float32(np.float32(a_gs) * gs_e)
        else:
            half = N // 2
            out[r0:r1, :half] = acc[:, :half] * np.float32(np.float32(a_gs) * gs_e[0])
            out[r0:r1, half:] = acc[:, half:] * np.float32(np.float32(a_gs) * gs_e[1])

    list(map_fn(one, range(L)))
    return out


def silu_mul(g_out: np.ndarray, inter: int) -> np.ndarray:
    """L1 out (float32 [S, 2I]) -> h BF16 bits [S, I]."""
    g = bf16_to_f32(f32_to_bf16(g_out[:, :inter]))
    u = bf16_to_f32(f32_to_bf16(g_out[:, inter:2 * inter]))
    with np.errstate(over="ignore"):
        silu = g / (np.float32(1.0) + np.exp(-g))
    return f32_to_bf16((silu * u).astype(np.float32))


def scatter(y_bits: np.ndarray, token_slot: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    """out[t] = BF16(sum_j w[t, j] * Y[token_slot[t*k + j]]) over local j; [T, H] bits."""
    T, k = topk_w.shape
    H = y_bits.shape[1]
    ts = np.asarray(token_slot).reshape(T, k)
    acc = np.zeros((T, H), np.float32)
    for j in range(k):
        sel = ts[:, j] >= 0
        if not np.any(sel):
            continue
        rows = bf16_to_f32(y_bits[ts[sel, j]])
        acc[sel] = acc[sel] + np.asarray(topk_w, np.float32)[sel, j][:, None] * rows
    return f32_to_bf16(acc)


@dataclasses.dataclass
class OracleTrace:
    x_q: np.ndarray
    x_sf: np.ndarray
    gs_x: np.float32
    routing: dict
    h: np.ndarray
    h_q: np.ndarray
    h_sf: np.ndarray
    gs_h: np.float32
    y: np.ndarray
    out: np.ndarray


def moe_forward(x_bits, topk_ids, topk_w, expert_start, w: dict, map_fn=map, static_gs=None) -> OracleTrace:
    """Whole layer on one rank's share; w as returned by prepare_weights.

    static_gs: optional (gs_x, gs_h), global scales measured once beforehand
    (nvfp4_cutedsl.py history, page 2, static-scale commit: warmup measures the
    L1 input's and the L1 output's gs; inference quantizes with them and no
    max reduction). By default each activation gets the gs of its own amax.
    """
    L, I = w["num_local"], w["inter"]
    gs_fix = (None, None) if static_gs is None else (np.float32(static_gs[0]), np.float32(static_gs[1]))
    x_q, x_sf, gs_x = quantize(x_bits, gs=gs_fix[0])
    r = route(topk_ids, topk_w, expert_start, L)
    S = r["S"]
    g_out = grouped_gemm(x_q, x_sf, r["slot_token"], gs_x, w["w1_q"], w["w1_sf"], w["w1_gs"],
                         r["offsets"], map_fn)
    h = silu_mul(g_out, I)
    h_q, h_sf, gs_h = quantize(h, gs=gs_fix[1])
    y = f32_to_bf16(grouped_gemm(h_q, h_sf, None, gs_h, w["w2_q"], w["w2_sf"], w["w2_gs"],
                                 r["offsets"], map_fn))
    out = scatter(y, r["token_slot"], np.asarray(topk_w, np.float32))
    assert y.shape[0] == S
    return OracleTrace(x_q, x_sf, gs_x, r, h, h_q, h_sf, gs_h, y, out)


def bf16_reference_layer(x_bits, topk_ids, topk_w, expert_start, w_gate, w_up, w_down):
    """Unquantized layer in float32 from the BF16 weights, same routing:
    out[t] = sum_j w_tj * W_down_e (silu(W_gate_e x_t) * (W_up_e x_t))."""
    L = w_gate.shape[0]
    x = bf16_to_f32(x_bits)
    T, k = np.asarray(topk_ids).shape
    r = route(topk_ids, topk_w, expert_start, L)
    out = np.zeros((T, x.shape[1]), np.float32)
    for e in range(L):
        r0, r1 = int(r["offsets"][e]), int(r["offsets"][e + 1])
        if r1 == r0:
            continue
        toks = r["slot_token"][r0:r1]
        xe = x[toks]
        gate = xe @ bf16_to_f32(w_gate[e]).T
        up = xe @ bf16_to_f32(w_up[e]).T
        with np.errstate(over="ignore"):
            act = gate / (np.float32(1.0) + np.exp(-gate)) * up
        y = act @ bf16_to_f32(w_down[e]).T
        np.add.at(out, toks, r["slot_weight"][r0:r1, None] * y)
    return out


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 or nb == 0:
        return 1.0 if na == nb else 0.0
    return float(a @ b / (na * nb))
