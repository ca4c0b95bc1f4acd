"""Checks shared by the GPU layer tests (small and full size)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O


def check_requant_h(nv, ws, lay, cap, inter, S, h_bits, scal):
    """Step a6 bit for bit: the layer's h_q, h_sf and gs_h are the oracle's
    quantization of the GPU's own h (its S valid rows) with amax_h from the
    L1 epilogue (nvfp4_mega_moe.py history, alpha commit: L2 takes the global
    scale that quantizing h returns). scal: the workspace scalars
    (gs_x, amax_h, gs_h, -) as float32."""
    oq, osf, ogs = O.quantize(h_bits, amax=np.float32(scal[1]))
    assert scal[2] == ogs == O.global_scale(scal[1]), (scal[2], ogs)
    h_q = nv.ws_view(ws, lay, "h_q", torch.uint8, (cap, inter // 2))[:S].cpu().numpy()
    h_sf = nv.ws_view(ws, lay, "h_sf", torch.uint8, (cap, inter // 16))[:S].cpu().numpy()
    assert np.array_equal(h_sf, osf), "h block scales differ from the oracle's quantization of the GPU's h"
    assert np.array_equal(h_q, oq), "h codes differ from the oracle's quantization of the GPU's h"


def check_static_h(nv, ws, lay, cap, inter, S, h_bits, gs_h):
    """The static layer's h_q, h_sf (written by the L1 epilogue for
    prefill-shaped batches, by a fixed-scale quantization of BF16 h for
    decode-shaped ones) are the oracle's quantization with the fixed gs_h of
    the same h, which the dynamic layer on the same inputs wrote as BF16
    (nvfp4_cutedsl.py history, static-scale commit)."""
    oq, osf, _ = O.quantize(h_bits, gs=np.float32(gs_h))
    h_q = nv.ws_view(ws, lay, "h_q", torch.uint8, (cap, inter // 2))[:S].cpu().numpy()
    h_sf = nv.ws_view(ws, lay, "h_sf", torch.uint8, (cap, inter // 16))[:S].cpu().numpy()
    assert np.array_equal(h_sf, osf), "static h block scales differ from the oracle's"
    assert np.array_equal(h_q, oq), "static h codes differ from the oracle's"


def dequantized_weights(P, experts, map_fn=map):
    """BF16 bits of the dequantized NVFP4 weights of the given local experts:
    (gate [n, I, H], up [n, I, H], down [n, H, I]), each half of W1 with its
    own global scale when the scales are not folded (w1_gs [L, 2])."""
    I = P["inter"]
    g1 = np.asarray(P["w1_gs"])
    f = lambda q, sf, gs: O.f32_to_bf16(O.dequantize(q, sf, gs, np.float32))

    def one(e):
        gg, gu = (g1[e, 0], g1[e, 1]) if g1.ndim == 2 else (g1[e], g1[e])
        return (f(P["w1_q"][e, :I], P["w1_sf"][e, :I], gg), f(P["w1_q"][e, I:], P["w1_sf"][e, I:], gu),
                f(P["w2_q"][e], P["w2_sf"][e], P["w2_gs"][e]))

    parts = list(map_fn(one, list(experts)))
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))
