"""BF16 -> NVFP4 quantization — oracle (test infrastructure only).

Follows, in order:
  * nvfp4_mega_moe.py history, overflow-fix commit: a per-tensor global scale
    gs = amax / (6 * 448) normalizes the tensor so that every block scale is
    at most 448 (the UE4M3 maximum).
  * nvfp4_mega_moe.py history, alpha commit: gs is not folded into the block
    scales; it is returned next to (x_fp4, x_sf) and applied later as the
    GEMM's alpha.
  * nvfp4_mega_moe.py history, three-quantizer-bugs commit: the stored block
    scale is block_max / 6 (the dequantization factor, after normalization
    by gs); magnitudes snap to the nearest E2M1 value; the sign is kept in
    bit 3 of the nibble.
  * tests history, packing-along-K commit: two nibbles per byte along K.

Readings where the pages leave a step open (each listed in the design notes):
  * Rounding: the scale and the magnitude are each rounded once from the
    exact real quotient, to nearest with ties to even (E4M3 code / E2M1
    code), the scale saturating at 448.
  * Elements are divided by the scale actually stored, dec(sf) * gs.
  * A block whose scale rounds to 0 stores magnitude 0 everywhere.
  * The sign bit is the sign bit of the BF16 input (so -0.0 keeps it).
  * amax == 0 gives gs = 0, all scales 0 and all magnitudes 0.

Exactness: inputs are BF16 (8 significant bits), gs is float32 (24 bits), an
E4M3 scale has 4 significant bits and the E2M1 rounding midpoints
(0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) have at most 3, so every product
formed below (6*gs, dec(sf)*gs, c*dec(sf)*gs) is exact in float64 and the
comparisons decide exactly. The one division, bmax / (6 gs), is rounded to
float64 before the E4M3 rounding; an E4M3 value or midpoint has at most 5
significant bits, so a quotient of an 8-bit by a 27-bit number that is not
one of them lies at least 2^-32 (relative) away — far beyond float64's
rounding — and the E4M3 decision is unaffected.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3_decode, e4m3_encode, pack_nibbles, e2m1_decode, unpack_nibbles

# midpoints between consecutive E2M1 magnitudes and whether an exact tie
# rounds up (the upper neighbour has the even code)
_MIDPOINTS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
              (2.5, False), (3.5, True), (5.0, False))

GS_DIVISOR = np.float32(6.0 * 448.0)  # 2688


def global_scale(amax) -> np.float32:
    """gs = amax / 2688, one float32 rounding (IEEE division of two floats)."""
    return np.float32(np.float32(amax) / GS_DIVISOR)


def quantize(x_bits: np.ndarray, amax=None):
    """Quantize one BF16 tensor [M, K] (uint16 bits, K % 16 == 0).

    amax: optional externally supplied amax (the h path, whose amax comes from
    the L1 epilogue); by default max |x| over the whole tensor.
    Returns (q uint8 [M, K/2], sf uint8 [M, K/16], gs float32).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    x = bf16_to_f64(x_bits)
    a = np.abs(x)
    if amax is None:
        amax = a.max() if a.size else 0.0
    gs = global_scale(amax)
    blocks = a.reshape(M, K // 16, 16)
    bmax = blocks.max(axis=2) if a.size else np.zeros((M, K // 16))
    if gs == 0:
        sf = np.zeros((M, K // 16), np.uint8)
    else:
        sf = e4m3_encode(bmax / (6.0 * np.float64(gs)))
    step = e4m3_decode(sf) * np.float64(gs)          # dequant factor per block, exact
    mag = np.zeros((M, K // 16, 16), np.uint8)
    for c, tie_up in _MIDPOINTS:
        t = (c * step)[..., None]                     # exact
        mag += (blocks >= t) if tie_up else (blocks > t)
    mag[step == 0] = 0
    sign = ((x_bits >> 15) & 1).astype(np.uint8).reshape(M, K // 16, 16)
    nib = (sign << 3) | mag
    q = pack_nibbles(nib.reshape(M, K))
    return q, sf, gs


def quantize_batched(x_bits: np.ndarray, amax=None):
    """[B, M, K] -> independent quantization of each x[b] (own amax and gs)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    outs = [quantize(x_bits[b], None if amax is None else amax[b]) for b in range(x_bits.shape[0])]
    q = np.stack([o[0] for o in outs])
    sf = np.stack([o[1] for o in outs])
    gs = np.array([o[2] for o in outs], dtype=np.float32)
    return q, sf, gs


def dequantize(q: np.ndarray, sf: np.ndarray, gs=1.0, dtype=np.float64) -> np.ndarray:
    """x_hat = E2M1(nibble) * dec(sf) * gs; [R, K/2], [R, K/16] -> [R, K]."""
    q = np.asarray(q, dtype=np.uint8)
    R, Kh = q.shape
    K = Kh * 2
    vals = e2m1_decode(unpack_nibbles(q)).reshape(R, K // 16, 16)
    s = e4m3_decode(sf)[..., None]
    out = (vals * s).reshape(R, K)
    if gs != 1.0:
        out = out * np.float64(gs)
    return out.astype(dtype)
