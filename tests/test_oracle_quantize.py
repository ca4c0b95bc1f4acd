"""Pins for the oracle's NVFP4 quantizer (CPU only).

Pinned by: a hand-derived worked example (golden), an exact brute force over
rationals (fractions.Fraction) that searches the nearest E4M3 scale and the
nearest E2M1 magnitude directly, and the invariants the pages fix: block
scales <= 448, stored scale = block_max / 6, signs kept, the global scale
preventing scale overflow.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W
from _cases import adversarial_rows, near_midpoint_blocks, quant_case

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E4M3_POS = [Fraction(float(v)) for v in O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))]
E2M1 = [Fraction(m).limit_denominator(4) for m in O.E2M1_MAGNITUDES]


def _bits(vals):
    return W.bf16_bits(np.asarray(vals, np.float32))


def _f32_nearest(fr: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even mantissa."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def _nearest_code(r: Fraction, grid):
    """Index of the nearest grid value; ties go to the even index; saturates."""
    if r >= grid[-1]:
        return len(grid) - 1
    best = None
    for i, g in enumerate(grid):
        key = (abs(g - r), i % 2)
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def brute_quantize(x_bits, gs=None):
    x_bits = np.asarray(x_bits, np.uint16)
    M, K = x_bits.shape
    xs = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(x_bits)]
    if gs is None:
        amax = max((abs(v) for row in xs for v in row), default=Fraction(0))
        gs = _f32_nearest(amax / 2688)
    gs = np.float32(gs)
    gsf = Fraction(float(gs))
    sf = np.zeros((M, K // 16), np.uint8)
    nib = np.zeros((M, K), np.uint8)
    for i in range(M):
        for b in range(K // 16):
            blk = xs[i][16 * b:16 * b + 16]
            bmax = max(abs(v) for v in blk)
            code = 0 if gsf == 0 else _nearest_code(bmax / (6 * gsf), E4M3_POS)
            sf[i, b] = code
            s = E4M3_POS[code] * gsf
            for j, v in enumerate(blk):
                m = 0 if s == 0 else _nearest_code(abs(v) / s, E2M1)
                sign = (int(x_bits[i, 16 * b + j]) >> 15) & 1
                nib[i, 16 * b + j] = (sign << 3) | m
    return O.pack_nibbles(nib), sf, gs


def _adversarial_rows(rng, n_rows=6):
    return adversarial_rows(rng, n_rows)


def test_worked_example_from_pages():
    g = json.load(open(os.path.join(GOLD, "quantize_worked_example.json")))
    x = _bits([g["row"]])
    q, sf, gs = O.quantize(x)
    assert gs == np.float32(g["gs"])
    assert [int(s) for s in sf[0]] == [int(s, 16) for s in g["scales"]]
    assert list(O.unpack_nibbles(q)[0]) == g["nibbles"]


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_random(seed):
    rng = np.random.default_rng(seed)
    M, K = 3, 64
    scale = float(np.exp2(rng.uniform(-30, 30)))
    x = rng.standard_t(3, (M, K)).astype(np.float32) * np.float32(scale)
    x[rng.random((M, K)) < 0.1] = 0
    xb = _bits(x)
    q, sf, gs = O.quantize(xb)
    bq, bsf, bgs = brute_quantize(xb)
    assert gs == bgs
    assert np.array_equal(sf, bsf)
    assert np.array_equal(q, bq)


def test_brute_force_exact_ties():
    rng = np.random.default_rng(7)
    xb = _adversarial_rows(rng)
    q, sf, gs = O.quantize(xb)
    bq, bsf, bgs = brute_quantize(xb)
    assert gs == 1.0 == bgs
    assert np.array_equal(sf, bsf)
    assert np.array_equal(q, bq)


def test_brute_force_tiny_magnitudes():
    # subnormal BF16 inputs and a float32-subnormal global scale
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 32)) * 2.0 ** -128).astype(np.float32)
    xb = _bits(x)
    q, sf, gs = O.quantize(xb)
    bq, bsf, bgs = brute_quantize(xb)
    assert gs == bgs and gs < np.finfo(np.float32).tiny
    assert np.array_equal(sf, bsf) and np.array_equal(q, bq)


def _check_invariants(xb, q, sf, gs):
    x = O.bf16_to_f64(xb)
    M, K = x.shape
    a = np.abs(x)
    amax = a.max()
    assert gs == O.global_scale(amax)
    # I1: scales are finite and never exceed 448
    assert sf.max() <= 0x7E
    bmax = a.reshape(M, K // 16, 16).max(axis=2)
    s = O.e4m3_decode(sf)
    if amax > 0:
        # I2: the block holding amax gets scale 448, and amax gets magnitude 6
        assert sf.max() == 0x7E
        i, j = np.unravel_index(np.argmax(a), a.shape)
        assert sf[i, j // 16] == 0x7E
        assert O.unpack_nibbles(q)[i, j] & 7 == 7
    # I3: stored scale = block_max / 6 in units of gs, within half an E4M3 step
    target = bmax / (6.0 * np.float64(gs))
    codes = sf.astype(int)
    up = O.e4m3_decode(np.minimum(codes + 1, 0x7E).astype(np.uint8))
    dn = O.e4m3_decode(np.maximum(codes - 1, 0).astype(np.uint8))
    half_step = np.maximum(up - s, s - dn) / 2
    assert np.all(np.abs(s - target) <= half_step + 0.0)
    # I4: unclipped elements are within half an E2M1 step of their value
    xh = O.dequantize(q, sf, gs)
    step = np.repeat(s * np.float64(gs), 16, axis=1)
    clipped = a > 6 * step
    err = np.abs(xh - x)
    assert np.all(err[~clipped] <= 1.0 * step[~clipped] + 0.0)
    # signs are kept (the clamp(0,15) bug zeroed negatives)
    neg = x < 0
    assert np.all(O.unpack_nibbles(q)[neg] & 8)
    assert np.all(xh[neg] <= 0)


@pytest.mark.parametrize("dist", ["normal", "t3", "outliers", "wide"])
def test_invariants(dist):
    rng = np.random.default_rng(11)
    shape = (64, 512)
    if dist == "normal":
        x = rng.standard_normal(shape)
    elif dist == "t3":
        x = rng.standard_t(3, shape)
    elif dist == "outliers":
        x = rng.standard_t(3, shape)
        x[rng.random(shape) < 0.001] = 2000.0
    else:
        x = rng.standard_normal(shape) * np.exp2(rng.uniform(-20, 20, shape))
    xb = _bits(x.astype(np.float32))
    _check_invariants(xb, *O.quantize(xb))


def test_idempotent_when_gs_is_one():
    # I5: amax = 2688 gives gs = 1; quantize(dequantize(quantize(x))) == quantize(x)
    # on every block whose scale is normal (>= 0x08)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 256)).astype(np.float32) * 300
    x[0, 0] = 2688.0
    xb = _bits(x)
    q, sf, gs = O.quantize(xb)
    assert gs == 1.0
    xh = O.dequantize(q, sf, gs).astype(np.float32)
    q2, sf2, gs2 = O.quantize(_bits(xh))
    assert gs2 == 1.0
    normal = sf >= 0x08
    assert np.array_equal(sf[normal], sf2[normal])
    n1 = O.unpack_nibbles(q).reshape(32, 16, 16)[normal]
    n2 = O.unpack_nibbles(q2).reshape(32, 16, 16)[normal]
    assert np.array_equal(n1, n2)


def test_global_scale_prevents_scale_overflow():
    # pages (overflow-fix commit): without a global scale, block_max/6 exceeds 448
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[:, 5] = 4000.0
    xb = _bits(x)
    q1, sf1, gs1 = O.quantize(xb, amax=2688.0)         # gs forced to 1: no normalisation
    assert gs1 == 1.0
    assert np.all(sf1[:, 0] == 0x7E)                   # 4000/6 = 667 saturates at 448
    err1 = np.abs(O.dequantize(q1, sf1, gs1)[:, 5] - 4000.0)
    assert np.all(err1 > 1000)                          # saturated: 6 * 448 = 2688
    q2, sf2, gs2 = O.quantize(xb)                       # true amax: every scale fits
    err2 = np.abs(O.dequantize(q2, sf2, gs2)[:, 5] - 4000.0)
    assert np.all(err2 <= 4000.0 * 2.0 ** -22)             # only gs's float32 rounding
    assert sf2.max() == 0x7E


def test_global_scale_is_nearest_float32():
    rng = np.random.default_rng(2)
    for a in np.concatenate([W.bf16_bits(rng.standard_normal(200).astype(np.float32) * 1e3),
                             np.array([0x0001, 0x7F7F, 0x3F80], np.uint16)]):
        amax = float(O.bf16_to_f64(np.uint16(a)))
        amax = abs(amax)
        assert O.global_scale(amax) == _f32_nearest(Fraction(amax) / 2688)


def test_zero_and_negative_zero():
    xb = _bits(np.zeros((2, 32), np.float32))
    xb[1, 3] = 0x8000  # -0.0
    q, sf, gs = O.quantize(xb)
    assert gs == 0 and not sf.any()
    nib = O.unpack_nibbles(q)
    assert nib[1, 3] == 0x8 and nib.sum() == 0x8


def test_batched_uses_own_scales():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 16, 64)).astype(np.float32) * np.array([1, 100, 0.01], np.float32)[:, None, None]
    xb = _bits(x)
    q, sf, gs = O.quantize_batched(xb)
    for b in range(3):
        qb, sfb, gsb = O.quantize(xb[b])
        assert gs[b] == gsb and np.array_equal(q[b], qb) and np.array_equal(sf[b], sfb)
    assert len(set(gs.tolist())) == 3


# ---- fixed (calibrated) global scale: nvfp4_cutedsl.py history, static-scale commit

@pytest.mark.parametrize("seed", range(3))
def test_static_gs_of_own_amax_equals_dynamic(seed):
    # the fixed-gs path with gs = RN(amax / 2688) is the dynamic quantizer
    rng = np.random.default_rng(100 + seed)
    x = (rng.standard_t(3, (16, 256)) * np.exp2(rng.uniform(-10, 10))).astype(np.float32)
    xb = _bits(x)
    q, sf, gs = O.quantize(xb)
    q2, sf2, gs2 = O.quantize(xb, gs=O.global_scale(np.abs(O.bf16_to_f64(xb)).max()))
    assert gs2 == gs and np.array_equal(sf2, sf) and np.array_equal(q2, q)


@pytest.mark.parametrize("factor", [1 / 64.0, 1 / 3.0, 1.0, 7.5, 2.0 ** 20])
def test_brute_force_static_gs(factor):
    # a fixed gs below amax / 2688 saturates scales at 448 and magnitudes at 6;
    # one above it leaves small (subnormal E4M3) scales
    rng = np.random.default_rng(21)
    x = rng.standard_t(3, (3, 64)).astype(np.float32)
    x[rng.random((3, 64)) < 0.1] = 0
    xb = _bits(x)
    gs = np.float32(O.global_scale(np.abs(O.bf16_to_f64(xb)).max()) * np.float32(factor))
    q, sf, gs_out = O.quantize(xb, gs=gs)
    bq, bsf, bgs = brute_quantize(xb, gs=gs)
    assert gs_out == bgs == gs
    assert np.array_equal(sf, bsf) and np.array_equal(q, bq)
    if factor < 1:
        assert (sf == 0x7E).any() and (O.unpack_nibbles(q) & 7 == 7).sum() > 1


def test_static_gs_zero_gives_zeros():
    xb = _bits(np.linspace(-3, 3, 64, dtype=np.float32).reshape(2, 32))
    q, sf, gs = O.quantize(xb, gs=0.0)
    assert gs == 0 and not sf.any() and not (O.unpack_nibbles(q) & 7).any()


def test_brute_force_near_midpoints():
    # elements a few float32 ulps from an E2M1 midpoint (not on it): the exact
    # rounding must go to the nearer neighbour on the correct side
    bits, gs = near_midpoint_blocks(3)
    for b in range(bits.shape[0]):
        q, sf, _ = O.quantize(bits[b], gs=gs[b])
        bq, bsf, _ = brute_quantize(bits[b], gs=gs[b])
        assert np.array_equal(sf, bsf) and np.array_equal(q, bq), b


def test_brute_force_scale_ties():
    # block maxima at 6 x an E4M3 midpoint (gs = 1) and at the BF16 values next
    # to it: the scale rounds to the even code on the tie, to the side elsewhere
    xb = quant_case("scale_ties")
    q, sf, gs = O.quantize(xb)
    bq, bsf, bgs = brute_quantize(xb)
    assert gs == 1.0 == bgs
    assert np.array_equal(sf, bsf) and np.array_equal(q, bq)
