"""Offline weight preparation — oracle (test infrastructure only).

Follows:
  * nvfp4_cutedsl.py history (also repeated in the tests history), the
    finalize_weights commit: gate and up carry different global scales; both
    are normalized to max(gs_gate, gs_up) by folding the ratio into the block
    scales of the other half through float32 — one multiply, then a round
    trip to float8. Global scales stay float32 and are not folded further.
  * nvfp4_cutedsl.py history, intermediate-split commit: the L1 weight holds
    gate rows [0, I) and up rows [I, 2I); intermediate_size is the size of
    gate (or up) alone.
  * nvfp4_mega_moe.py history, alpha commit: global scales are applied as
    GEMM alpha, so each (expert, projection) is quantized with its own gs.

Reading: ratio = gs_p / gs1 rounded to float32; each scale of the smaller-gs
half becomes RNE_E4M3(RN_f32(dec(sf) * ratio)), saturating at 448. When the
two scales are equal nothing changes.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_decode, e4m3_encode
from .quantize import quantize


def fold_gate_up(w1_sf: np.ndarray, gs_gate: np.ndarray, gs_up: np.ndarray, inter: int):
    """w1_sf [L, 2I, K/16] (gate rows then up rows); returns (folded copy, gs1 [L])."""
    sf = np.array(w1_sf, dtype=np.uint8, copy=True)
    L = sf.shape[0]
    gs_gate = np.asarray(gs_gate, np.float32)
    gs_up = np.asarray(gs_up, np.float32)
    gs1 = np.maximum(gs_gate, gs_up).astype(np.float32)
    for e in range(L):
        for lo, hi, gs_p in ((0, inter, gs_gate[e]), (inter, 2 * inter, gs_up[e])):
            if gs_p < gs1[e]:
                ratio = np.float32(gs_p / gs1[e])
                prod = (e4m3_decode(sf[e, lo:hi]).astype(np.float32) * ratio).astype(np.float32)
                sf[e, lo:hi] = e4m3_encode(prod.astype(np.float64))
    return sf, gs1


def prepare_weights(w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, map_fn=map,
                    fold: bool = True) -> dict:
    """BF16 bits W_gate, W_up [L, I, H] and W_down [L, H, I] -> NVFP4 layer weights.

    Each (expert, projection) is quantized on its own (own gs); the gate/up
    ratio is then folded. map_fn lets a caller spread experts over threads.
    Returns w1_q [L, 2I, H/2], w1_sf [L, 2I, H/16], w1_gs [L] (= gs1),
    w2_q [L, H, I/2], w2_sf [L, H, I/16], w2_gs [L], plus gs_gate and gs_up.

    fold=False keeps both halves' block scales as quantized and returns
    w1_gs [L, 2] = (gs_gate, gs_up): the L1 GEMM then applies one alpha per
    half (the alpha commit's treatment of a global scale, applied to gate and
    up separately) instead of the finalize_weights fold.
    """
    L, I, H = w_gate.shape
    res = list(map_fn(lambda e: (quantize(w_gate[e]), quantize(w_up[e]), quantize(w_down[e])),
                      range(L)))
    w1_q = np.stack([np.concatenate([g[0], u[0]]) for g, u, _ in res])
    w1_sf = np.stack([np.concatenate([g[1], u[1]]) for g, u, _ in res])
    gs_gate = np.array([g[2] for g, _, _ in res], np.float32)
    gs_up = np.array([u[2] for _, u, _ in res], np.float32)
    if fold:
        w1_sf, gs1 = fold_gate_up(w1_sf, gs_gate, gs_up, I)
    else:
        gs1 = np.stack([gs_gate, gs_up], axis=1).astype(np.float32)
    w2_q = np.stack([d[0] for _, _, d in res])
    w2_sf = np.stack([d[1] for _, _, d in res])
    w2_gs = np.array([d[2] for _, _, d in res], np.float32)
    return dict(w1_q=w1_q, w1_sf=w1_sf, w1_gs=gs1, w2_q=w2_q, w2_sf=w2_sf, w2_gs=w2_gs,
                gs_gate=gs_gate, gs_up=gs_up, inter=I, hidden=H, num_local=L)
