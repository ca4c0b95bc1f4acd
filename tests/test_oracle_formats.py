"""Pins for the oracle's number formats (CPU only).

E2M1 values come from the pages (golden file); E4M3 and BF16 are pinned
against torch's own float8_e4m3fn / bfloat16 types, a library independent of
the oracle's table-driven code.
"""
import json
import os

import numpy as np
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e2m1_value_set_from_pages():
    g = _gold("e2m1_values.json")
    mags = g["magnitudes"]
    assert list(O.E2M1_MAGNITUDES) == mags
    nib = np.arange(16, dtype=np.uint8)
    vals = O.e2m1_decode(nib)
    for n in range(16):
        sign = -1.0 if (n >> g["sign_bit"]) & 1 else 1.0
        assert vals[n] == sign * mags[n & 7] or (mags[n & 7] == 0 and vals[n] == 0)
        assert np.signbit(vals[n]) == bool(n & 8)


def test_e4m3_decode_matches_torch_float8_bit_view():
    # pages (float8 bit-view commit): scale bytes are reinterpreted, not value-converted
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], ours[~nan])
    assert O.e4m3_decode(np.uint8(0x7E)) == 448.0


def test_e4m3_view_is_not_value_conversion():
    # the bug the pages describe: byte 0x3F turned into float8(63.0) instead of the
    # float8 whose bit pattern is 0x3F. Pack (view) and unpack must be inverses.
    v = O.e4m3_decode(np.uint8(0x3F))
    assert v == 1.875 and v != 63.0
    codes = np.arange(0, O.E4M3_MAX_CODE + 1, dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


def test_e4m3_encode_matches_torch_rounding():
    rng = np.random.default_rng(0)
    # float32 values across the whole non-negative finite range, incl. subnormals
    v = np.concatenate([
        rng.uniform(0, 448, 20000), rng.uniform(0, 2 ** -6, 20000),
        np.exp2(rng.uniform(-12, 8.8, 20000)),
    ]).astype(np.float32)
    v = v[v <= 448]
    # exact midpoints between consecutive codes (ties)
    pos = O.e4m3_decode(np.arange(0, O.E4M3_MAX_CODE + 1, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    v = np.concatenate([v, mids, pos.astype(np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = O.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(ref, ours)


def test_e4m3_encode_ties_to_even_and_saturation():
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39)
    assert O.e4m3_encode(np.array([1.0625]))[0] == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even)
    assert O.e4m3_encode(np.array([1.1875]))[0] == 0x3A
    # half the smallest subnormal (2^-10) rounds to 0 (even), just above rounds up
    assert O.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00
    assert O.e4m3_encode(np.array([2.0 ** -10 * 1.0001]))[0] == 0x01
    # beyond 448 saturates to 0x7E
    assert list(O.e4m3_encode(np.array([448.0, 460.0, 1e9]))) == [0x7E] * 3


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 1e3,
        np.exp2(rng.uniform(-140, 120, 50000)).astype(np.float32),
        # exact ties: low half == 0x8000 with odd and even kept halves
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), ref)
    back = O.bf16_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_pack_unpack_inverse_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(O.pack_nibbles(O.unpack_nibbles(b)), b)
    nib = O.unpack_nibbles(b)
    # element 2j in the low nibble, 2j+1 in the high nibble (packing along K)
    assert np.array_equal(nib[0, 0::2], np.arange(256) & 0xF)
    assert np.array_equal(nib[0, 1::2], np.arange(256) >> 4)
