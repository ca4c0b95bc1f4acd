"""Seeded synthetic workloads for the NVFP4 MoE expert-FFN path.

This module is shared by the CPU oracle's tests, the HIP path's tests, the
benchmark and the smoke check. It holds no step of the method: it only draws
random inputs (router logits -> top-k ids and weights, BF16 activations and
BF16 weights) with fixed seeds. BF16 rounding of the draws is done by torch's
float32 -> bfloat16 conversion, so this module shares no arithmetic with the
oracle or with the kernels.

The pages measure on a real checkpoint layer inside a serving engine; neither
is available, so these inputs stand in for it with the pages' shapes (384
routed experts, 48 per rank, intermediate 3072) and hidden 7168.

Random streams (numpy PCG64 via SeedSequence([0, cfg, stream(, expert)])):
  0 router logits / Gumbel noise, 1 activations, 2 W_gate, 3 W_up, 4 W_down,
  5 outlier positions and signs, 6 Zipf ranks and cold/hot expert choice.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

__all__ = [
    "LayerConfig", "QuantConfig", "CONFIGS", "get_config", "bf16_bits",
    "make_router", "make_activations", "make_weights", "make_quant_input",
    "random_fp4_operands",
]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One MoE layer shard: this GPU owns experts [start, start + num_local)."""
    name: str
    cfg_id: int
    tokens: int
    top_k: int
    num_global: int
    num_local: int
    expert_start: int
    hidden: int
    inter: int
    logits: str = "normal"          # "normal" | "uniform" | "zipf"
    weight_cfg_id: int | None = None  # reuse another config's weight streams
    up_scale: float = 1.0            # W_up = up_scale * N(0, 0.02)
    weight_std: float = 0.02

    @property
    def weight_seed_id(self) -> int:
        return self.cfg_id if self.weight_cfg_id is None else self.weight_cfg_id


@dataclasses.dataclass(frozen=True)
class QuantConfig:
    """Activation quantizer alone on a [rows, cols] BF16 tensor."""
    name: str
    cfg_id: int
    rows: int
    cols: int
    outlier_frac: float
    outlier_value: float


CONFIGS = {
    # tiny layer: every expert local, oracle finishes in well under a second
    "tiny": LayerConfig("tiny", 0, tokens=32, top_k=2, num_global=8, num_local=8,
                        expert_start=0, hidden=256, inter=128),
    # activation quantizer only, Student-t(3) with 0.1% outliers at +-2000
    "quant": QuantConfig("quant", 1, rows=4096, cols=7168, outlier_frac=0.001,
                         outlier_value=2000.0),
    # decode-shaped shard: 64 tokens, top-8 of 384, local experts 96..143
    "decode": LayerConfig("decode", 2, tokens=64, top_k=8, num_global=384, num_local=48,
                          expert_start=96, hidden=7168, inter=3072),
    # prefill-shaped shard: same weights as the decode shard, uniform logits
    "prefill": LayerConfig("prefill", 3, tokens=8192, top_k=8, num_global=384, num_local=48,
                           expert_start=96, hidden=7168, inter=3072, logits="uniform",
                           weight_cfg_id=2),
    # skewed shard: Zipf(1.2) popularity, cold local experts, W_up 30x larger
    "skewed": LayerConfig("skewed", 4, tokens=16384, top_k=8, num_global=384, num_local=48,
                          expert_start=96, hidden=7168, inter=3072, logits="zipf",
                          up_scale=30.0),
    # mid-sized layers for GPU parity: several tiles per dimension and ragged tails
    "mid": LayerConfig("mid", 10, tokens=200, top_k=4, num_global=64, num_local=16,
                       expert_start=16, hidden=512, inter=384),
    "mid_k1": LayerConfig("mid_k1", 11, tokens=300, top_k=1, num_global=12, num_local=12,
                          expert_start=0, hidden=384, inter=256),
    "mid_skew": LayerConfig("mid_skew", 12, tokens=640, top_k=8, num_global=384, num_local=48,
                            expert_start=96, hidden=256, inter=128, logits="zipf",
                            up_scale=30.0),
    # more than 1024 slot entries (the chunked route) with decode-height (32-row) tiles
    "mid_route3": LayerConfig("mid_route3", 13, tokens=200, top_k=8, num_global=384, num_local=48,
                              expert_start=96, hidden=256, inter=128),
    # top-1 with more than 1024 slot entries: the chunked route inside the quantize launch and prefill-height
    # (96-row) GEMM tiles at a small size
    "long_k1": LayerConfig("long_k1", 15, tokens=3000, top_k=1, num_global=12, num_local=12,
                           expert_start=0, hidden=256, inter=128),
    # many local experts: 36 route chunks x 2048 experts = 73728 histogram entries, past the limit of the
    # route's scan/scatter inside the quantize launch (the layer then launches them separately)
    "wide_route": LayerConfig("wide_route", 14, tokens=4608, top_k=8, num_global=2560, num_local=2048,
                              expert_start=256, hidden=128, inter=128),
}


def get_config(name: str):
    return CONFIGS[name]


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, *key])))


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round float32 draws to BF16 with torch's conversion; return uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------- router

def _topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    # highest k scores per row; equal scores -> lower expert id first
    order = np.argsort(-scores, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def make_router(cfg: LayerConfig):
    """Return (topk_ids int32 [T, k] global ids, topk_w float32 [T, k]).

    The weights are a softmax over the k selected logits (the router is outside
    the expert-FFN path; this is only how the synthetic workload draws them).
    """
    rng = _rng(cfg.cfg_id, 0)
    T, E, k = cfg.tokens, cfg.num_global, cfg.top_k
    if cfg.logits == "normal":
        logits = rng.standard_normal((T, E), dtype=np.float32)
    elif cfg.logits == "uniform":
        logits = rng.random((T, E), dtype=np.float32)
    elif cfg.logits == "zipf":
        logits = _zipf_logits(cfg, rng)
    else:
        raise ValueError(cfg.logits)
    ids = _topk_desc(logits, k)
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    w = _softmax_rows(sel)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


def _zipf_logits(cfg: LayerConfig, rng: np.random.Generator) -> np.ndarray:
    """Zipf(1.2) popularity with one hot local expert and 6 cold local experts.

    p_e ~ rank_e^-1.2 over a seeded rank permutation; a seeded local expert is
    given rank 1; 6 other seeded local experts get p = 0. Top-k of
    log p + Gumbel noise samples k experts per token without replacement.
    """
    E, L, s = cfg.num_global, cfg.num_local, cfg.expert_start
    prng = _rng(cfg.cfg_id, 6)
    ranks = prng.permutation(E) + 1
    local = np.arange(s, s + L)
    pick = prng.choice(local, size=7, replace=False)
    hot, cold = int(pick[0]), pick[1:]
    r1 = int(np.nonzero(ranks == 1)[0][0])
    ranks[r1], ranks[hot] = ranks[hot], ranks[r1]
    logp = -1.2 * np.log(ranks.astype(np.float64))
    logp[cold] = -np.inf
    g = rng.gumbel(size=(cfg.tokens, E))
    return (logp[None, :] + g).astype(np.float64)


# ---------------------------------------------------------------------- activations

def make_activations(cfg: LayerConfig) -> np.ndarray:
    """BF16 bits [T, H], N(0, 1) draws."""
    rng = _rng(cfg.cfg_id, 1)
    return bf16_bits(rng.standard_normal((cfg.tokens, cfg.hidden), dtype=np.float32))


def make_quant_input(cfg: QuantConfig) -> np.ndarray:
    """BF16 bits [rows, cols]: Student-t(3) with outlier_frac entries at +-outlier_value."""
    rng = _rng(cfg.cfg_id, 1)
    n = cfg.rows * cfg.cols
    x = rng.standard_t(3, size=n).astype(np.float32)
    orng = _rng(cfg.cfg_id, 5)
    n_out = int(round(cfg.outlier_frac * n))
    pos = orng.choice(n, size=n_out, replace=False)
    sign = np.where(orng.random(n_out) < 0.5, -1.0, 1.0).astype(np.float32)
    x[pos] = sign * np.float32(cfg.outlier_value)
    return bf16_bits(x.reshape(cfg.rows, cfg.cols))


# -------------------------------------------------------------------------- weights

def _expert_weights(cfg: LayerConfig, e: int):
    sid = cfg.weight_seed_id
    H, I, std = cfg.hidden, cfg.inter, np.float32(cfg.weight_std)
    wg = _rng(sid, 2, e).standard_normal((I, H), dtype=np.float32) * std
    wu = _rng(sid, 3, e).standard_normal((I, H), dtype=np.float32) * (std * np.float32(cfg.up_scale))
    wd = _rng(sid, 4, e).standard_normal((H, I), dtype=np.float32) * std
    return bf16_bits(wg), bf16_bits(wu), bf16_bits(wd)


def make_weights(cfg: LayerConfig, experts=None, threads: int | None = None):
    """BF16 bits W_gate [L, I, H], W_up [L, I, H], W_down [L, H, I] for local experts.

    `experts` selects a subset of local expert indices (the arrays then have
    len(experts) rows along the first axis, in the given order).
    """
    experts = list(range(cfg.num_local)) if experts is None else list(experts)
    n = len(experts)
    H, I = cfg.hidden, cfg.inter
    wg = np.empty((n, I, H), np.uint16)
    wu = np.empty((n, I, H), np.uint16)
    wd = np.empty((n, H, I), np.uint16)

    def one(i):
        wg[i], wu[i], wd[i] = _expert_weights(cfg, experts[i])

    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(n)))
    return wg, wu, wd


# ----------------------------------------------------- raw operands for stage tests

def random_fp4_operands(seed: int, rows: int, cols: int, max_scale_code: int = 0x50):
    """Random packed E2M1 bytes [rows, cols/2] and E4M3 scale codes [rows, cols/16].

    Scale codes are drawn uniformly from [0, max_scale_code] (all finite,
    non-negative), so the operands exercise zero, subnormal and normal scales.
    """
    rng = _rng(1000 + seed, 7)
    q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    sf = rng.integers(0, max_scale_code + 1, size=(rows, cols // 16), dtype=np.uint8)
    return q, sf
