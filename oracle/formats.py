"""Number formats of NVFP4 — oracle (test infrastructure only).

* BF16 values are carried as uint16 bit patterns; float32 -> BF16 rounds to
  nearest, ties to even.
* E4M3 (float8_e4m3fn): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no
  infinities; codes 0x7F/0xFF are NaN; the largest finite value 0x7E = 448.
  Block scales are non-negative ("UE4M3"). The src history (commit on scale
  dtypes) and the tests history (layer-test commit) name float8_e4m3fn as the
  block-scale type; the nvfp4_mega_moe.py history (overflow fix) gives 448 as
  the scale ceiling.
* E2M1 nibble: bit 3 is the sign, bits 2:0 index the magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} (nvfp4_mega_moe.py history, commit fixing the
  three quantizer bugs: sign-magnitude nibbles and the E2M1 value set).
* Two nibbles per byte along K (tests history, packing-along-K commit); the
  element with the even K index sits in the low nibble.
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E4M3_MAX_CODE = 0x7E  # 448.0


# ----------------------------------------------------------------------------- BF16

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact value of BF16 bit patterns as float32 (BF16 is the top half of float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to BF16, nearest with ties to even; returns uint16 bits.

    The float32 bit pattern is split at bit 16: the discarded low half is
    compared with the halfway point 0x8000; above it (or at it with an odd
    kept half) the kept half is incremented. NaN maps to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    hi = (u >> 16).astype(np.uint32)
    lo = u & np.uint32(0xFFFF)
    round_up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = (hi + round_up.astype(np.uint32)).astype(np.uint32)
    nan = np.isnan(x)
    out = np.where(nan, (hi | 0x40), out)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------- E4M3

def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)       # subnormal: m * 2^-9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = _e4m3_table()
# non-negative finite codes 0x00..0x7E are increasing in value
_E4M3_POS = _E4M3[: E4M3_MAX_CODE + 1].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact value of E4M3 codes (float64)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Non-negative reals (float64) -> nearest E4M3 code, ties to the even code,
    saturating at 448 (0x7E). Used for block scales, which are never negative."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode takes non-negative finite scales")
    hi = np.searchsorted(_E4M3_POS, v, side="left")      # first code with value >= v
    hi = np.minimum(hi, E4M3_MAX_CODE)
    lo = np.maximum(hi - 1, 0)
    d_lo = v - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - v
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(v >= _E4M3_POS[E4M3_MAX_CODE], E4M3_MAX_CODE, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------- E2M1

_E2M1 = np.array([s * m for s in (1.0, -1.0) for m in E2M1_MAGNITUDES], dtype=np.float64)


def e2m1_decode(nibbles: np.ndarray) -> np.ndarray:
    """Value of E2M1 nibbles (bit 3 sign, bits 2:0 magnitude index) as float64."""
    return _E2M1[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[..., K] nibbles -> [..., K/2] bytes; element 2j in the low nibble of byte j."""
    nib = np.asarray(nib, dtype=np.uint8)
    if nib.shape[-1] % 2:
        raise ValueError("K must be even")
    return (nib[..., 0::2] & 0xF) | ((nib[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] nibbles (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
