"""Shared test inputs and helpers (no method arithmetic here)."""
import zlib

import numpy as np

import workloads as W

E4M3_SCALES_FOR_TIES = [0x01, 0x05, 0x07, 0x08, 0x30, 0x38, 0x3F, 0x52, 0x7E]
E4M3_VALUES = {  # exact values of the codes above (E4M3: bias 7, subnormal step 2^-9)
    0x01: 2.0 ** -9, 0x05: 5 * 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
    0x38: 1.0, 0x3F: 1.875, 0x52: 10.0, 0x7E: 448.0,
}


def adversarial_rows(rng, n_rows=6):
    """BF16 rows with gs = 1 (one element 2688) and blocks whose elements sit
    exactly on E2M1 rounding midpoints of their block scale."""
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    scales = [E4M3_VALUES[c] for c in E4M3_SCALES_FOR_TIES]
    for _ in range(n_rows):
        row = [2688.0] + [0.0] * 15
        for s in rng.choice(scales, 3):
            vals = [6.0 * s] + [float(c * s) * float(rng.choice([-1, 1])) for c in rng.choice(mids, 15)]
            rng.shuffle(vals)
            row += vals
        rows.append(row)
    return W.bf16_bits(np.asarray(rows, np.float32))


def near_midpoint_blocks(seed, n_blocks=96):
    """One row of two 16-element BF16 blocks per tensor, with a float32 global
    scale per tensor, such that elements divided by their block's step (E4M3 scale d
    times gs) land within a few float32 ulps of an E2M1 rounding midpoint m
    without being on it: gs = RN_f32(x / (d * m)) for a chosen element x, and
    the block maximum RN_bf16(6 * d * gs) gives the block scale d. Returns
    (bits uint16 [n_blocks, 1, 32], gs float32 [n_blocks])."""
    rng = np.random.default_rng(seed)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    scales = [E4M3_VALUES[c] for c in (0x30, 0x38, 0x3F, 0x52)] + [1.125, 1.625, 13.0, 0.8125]
    blocks, gss = [], []
    for _ in range(n_blocks):
        m = float(rng.choice(mids))
        d = float(rng.choice(scales))
        xb = W.bf16_bits(np.array([(1 + rng.integers(0, 128) / 128.0) * 2.0 ** int(rng.integers(-6, 6))], np.float32))
        x = float((xb.astype(np.uint32) << 16).view(np.float32)[0])
        gs = np.float32(x / (d * m))
        bmax = np.float32(6.0 * d * float(gs))
        vals = [bmax, x, -x, x] + [float(rng.uniform(-1, 1)) * float(bmax) for _ in range(12)]
        # a few more elements placed on other midpoints of the same step (rounded to BF16)
        for i in range(4, 8):
            vals[i] = float(rng.choice(mids)) * d * float(gs) * float(rng.choice([-1, 1]))
        rng.shuffle(vals)
        second = list(vals)
        rng.shuffle(second)
        blocks.append(vals + second)   # two blocks of the same values (same scale): K = 32
        gss.append(gs)
    bits = W.bf16_bits(np.asarray(blocks, np.float32)).reshape(n_blocks, 1, 32)
    return bits, np.asarray(gss, np.float32)


# midpoints between adjacent E4M3 values (codes c and c + 1): 0x01/0x02,
# 0x07/0x08 (subnormal/normal), 0x30/0x31, 0x38/0x39, 0x3F/0x40 (binade),
# 0x52/0x53, 0x7D/0x7E (top)
E4M3_MIDPOINTS = [1.5 * 2.0 ** -9, 7.5 * 2.0 ** -9, 0.53125, 1.0625, 1.9375, 10.5, 432.0]


def scale_tie_rows(rng, n_rows=4):
    """BF16 rows with gs = 1 (one element 2688) whose blocks have their maximum
    at 6 x an E4M3 midpoint (an exact tie of the block scale) or at the BF16
    value just above or below it."""
    rows = []
    for _ in range(n_rows):
        row = [2688.0] + [0.0] * 15
        for m in E4M3_MIDPOINTS:
            tie = W.bf16_bits(np.array([6.0 * m], np.float32))[0]       # exact in BF16
            for bits in (tie, tie + 1, tie - 1):                          # the tie and its BF16 neighbours
                b = float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])
                blk = [b] + list(rng.uniform(-1, 1, 15) * b)
                rng.shuffle(blk)
                row += blk
        rows.append(row)
    return W.bf16_bits(np.asarray(rows, np.float32))


def quant_case(name):
    """BF16 bit arrays for the quantizer parity cases."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name == "tiny_x":
        return W.make_activations(W.get_config("tiny"))
    if name == "mid_x":
        return W.make_activations(W.get_config("mid"))
    if name == "t3_outliers":
        x = rng.standard_t(3, (256, 1024)).astype(np.float32)
        x[rng.random(x.shape) < 0.001] = 2000.0
        return W.bf16_bits(x)
    if name == "ties":
        return adversarial_rows(rng, 8)
    if name == "scale_ties":
        return scale_tie_rows(rng)
    if name == "subnormal":
        return W.bf16_bits((rng.standard_normal((4, 256)) * 2.0 ** -128).astype(np.float32))
    if name == "zeros":
        x = np.zeros((3, 64), np.float32)
        b = W.bf16_bits(x)
        b[1, 5] = 0x8000
        return b
    if name == "wide":
        return W.bf16_bits((rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-20, 20, (64, 512))))
                           .astype(np.float32))
    if name == "ragged_rows":
        return W.bf16_bits(rng.standard_normal((333, 96)).astype(np.float32))
    if name == "quant_full":
        return W.make_quant_input(W.get_config("quant"))
    if name == "large_outliers":
        # a 73 MB tensor with sparse outliers past 2688 (block scales saturate unless gs is applied)
        x = rng.standard_t(3, (5120, 7168)).astype(np.float32)
        x[rng.integers(0, 5120, 64), rng.integers(0, 7168, 64)] = 3000.0
        return W.bf16_bits(x)
    raise KeyError(name)


def pack_weights_np(q, sf):
    """The packed weight order of nvfp4_pack_weights, written from its
    definition in include/nvfp4moe.h with array reshapes:
    q uint8 [B, N, K/2], sf uint8 [B, N, K/16] -> uint8 [B, N/32, K/128, 2304]."""
    B, N, Kh = q.shape
    nsub, nst = N // 32, (2 * Kh) // 128
    # row = 32*sub + r; FP4 byte 64c + 32g + 16h + i  ->  chunk byte h*1024 + 16*(32g + r) + i
    qr = q.reshape(B, nsub, 32, nst, 2, 2, 16)                      # B, sub, r, c, g, h, i
    part_q = qr.transpose(0, 1, 3, 5, 4, 2, 6).reshape(B, nsub, nst, 2048)
    # scale byte 8c + 4g + i  ->  chunk byte 2048 + 4*(32g + r) + i
    sr = sf.reshape(B, nsub, 32, nst, 2, 4)                         # B, sub, r, c, g, i
    part_s = sr.transpose(0, 1, 3, 4, 2, 5).reshape(B, nsub, nst, 256)
    return np.ascontiguousarray(np.concatenate([part_q, part_s], axis=-1))
