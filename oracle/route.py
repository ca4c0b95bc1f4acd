"""Slot routing — oracle (test infrastructure only).

Follows:
  * nvfp4_mega_moe.py history, local-expert-id commit: top-k ids are global
    (0..383); a rank owns experts [start, start + num_local) and indexes its
    weights with id - start.
  * src history, 1-D slot id commits: both GEMMs use one 1-D slot order
    (slot_expert_ids, slot_token), built once by the outer routing.
  * nvfp4_cutedsl.py history, GPU-native routing and int32-offset commits:
    per-expert counts (bincount), int32 offsets (cumsum), a sort of the
    (token, k) pairs by expert, rows laid out [expert0 | expert1 | ...].
  * tests history, NVFP4-native layer-test commit: each expert's tokens form
    one contiguous block.

Reading: the sort is stable in the flattened index t*k + j, so within an
expert the slots follow token order (and k order within a token). Ids outside
[start, start + num_local) are dropped (another rank owns them). Slot arrays
have capacity T*k; entries s >= S (the number of local pairs) hold -1 (ints)
and 0.0 (weights).
"""
from __future__ import annotations

import numpy as np


def route(topk_ids: np.ndarray, topk_w: np.ndarray, expert_start: int, num_local: int) -> dict:
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    n = T * k
    local = (ids - expert_start).reshape(n)
    valid = (local >= 0) & (local < num_local)
    key = np.where(valid, local, num_local)          # dropped pairs sort last
    order = np.argsort(key, kind="stable")           # stable: flat index breaks ties
    counts = np.bincount(local[valid], minlength=num_local).astype(np.int32)
    offsets = np.zeros(num_local + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    S = int(offsets[-1])
    slots = order[:S]
    slot_token = np.full(n, -1, np.int32)
    slot_expert = np.full(n, -1, np.int32)
    slot_weight = np.zeros(n, np.float32)
    token_slot = np.full(n, -1, np.int32)
    slot_token[:S] = slots // k
    slot_expert[:S] = local[slots]
    slot_weight[:S] = np.asarray(topk_w, np.float32).reshape(n)[slots]
    token_slot[slots] = np.arange(S, dtype=np.int32)
    return dict(counts=counts, offsets=offsets, S=S, slot_token=slot_token,
                slot_expert=slot_expert, slot_weight=slot_weight, token_slot=token_slot)


def tile_schedule(counts: np.ndarray, offsets: np.ndarray, tile_m: int) -> np.ndarray:
    """GEMM row tiles in expert order: [(expert, first_slot_row), ...] as int32 [n, 2].

    Expert e with c rows contributes ceil(c / tile_m) tiles starting at
    offsets[e], offsets[e] + tile_m, ...; empty experts contribute none.
    """
    tiles = []
    for e, c in enumerate(np.asarray(counts)):
        for m0 in range(0, int(c), tile_m):
            tiles.append((e, int(offsets[e]) + m0))
    return np.array(tiles, dtype=np.int32).reshape(-1, 2)
