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
  * nvfp4_cutedsl.py history (page 2), static-scale commit: a warmup pass
    measures gs for each activation once; afterwards the activation is
    quantized with that fixed gs and no max reduction. With a fixed gs the
    tensor may exceed 2688 * gs: block scales then saturate at 448 and
    magnitudes at 6 (the same saturating roundings as above).

Readings where the pages leave a step open (each listed in the design notes):
  * Rounding: the scale and the magnitude are each rounded once from the
    exact real quotient, to nearest with ties to even (E4M3 code / E2M1
    code), the scale saturating at 448.
  * Elements are divided by the scale actually stored, dec(sf) * gs.
  * A block whose scale rounds to 0 stores magnitude 0 everywhere.
  * The sign bit is the sign bit of the BF16 input (so -0.0 keeps it).
  * amax == 0 gives gs = 0, all scales 0 and all magnitudes 0.

Exactness: inputs are BF16 (8 significant bits), gs is float32 (24 bits) and
an E4M3 scale has 4, so 6*gs and dec(sf)*gs are exact in float64. The two
quotients, bmax / (6 gs) and |x| / (dec(sf) gs), are rounded to float64
before they are compared with grid midpoints. A midpoint has at most 5
significant bits (E4M3) or 3 (E2M1: 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), so
a quotient of an 8-bit number by a number of at most 28 bits that is not
exactly a midpoint lies at least 2^-37 (relative) away from it — far beyond
float64's rounding error of 2^-53 — and an exact tie stays exact. Every
decision is therefore the one the real quotient gives.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3_decode, e4m3_encode, pack_nibbles, e2m1_decode, unpack_nibbles

# midpoints between consecutive E2M1 magnitudes; an exact tie rounds up at
# 0.75, 1.75 and 3.5 (the upper neighbour has the even code) and down elsewhere
_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_TIE_UP = np.array([0.75, 1.75, 3.5])

GS_DIVISOR = np.float32(6.0 * 448.0)  # 2688

# values of the two elements held by each byte: (element 2j, element 2j+1)
_BYTE_PAIRS = e2m1_decode(unpack_nibbles(np.arange(256, dtype=np.uint8)[:, None])).astype(np.float32)


def global_scale(amax) -> np.float32:
    """gs = amax / 2688, one float32 rounding (IEEE division of two floats)."""
    return np.float32(np.float32(amax) / GS_DIVISOR)


def quantize(x_bits: np.ndarray, amax=None, gs=None):
    """Quantize one BF16 tensor [M, K] (uint16 bits, K % 16 == 0).

    amax: optional externally supplied amax (the h path, whose amax comes from
    the L1 epilogue); by default max |x| over the whole tensor.
    gs: optional fixed global scale (float32) measured beforehand; it replaces
    the one derived from amax.
    Returns (q uint8 [M, K/2], sf uint8 [M, K/16], gs float32).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    x = bf16_to_f64(x_bits)
    a = np.abs(x)
    if gs is not None:
        gs = np.float32(gs)
    else:
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
    with np.errstate(divide="ignore", invalid="ignore"):
        r = blocks / step[..., None]                  # |x| in units of the block's step
    # nearest E2M1 index = number of midpoints below r, plus one at a tie that rounds up
    mag = np.zeros(r.shape, np.uint8)
    for c in _MIDPOINTS:
        mag += r > c
    for c in _TIE_UP:
        mag += r == c
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
    vals = _BYTE_PAIRS[q].reshape(R, K // 16, 16)    # byte -> (low nibble, high nibble) values
    s = e4m3_decode(sf)[..., None]
    out = (vals * s).reshape(R, K)
    if gs != 1.0:
        out = out * np.float64(gs)
    return out.astype(dtype)
