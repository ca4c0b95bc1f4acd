"""Pins for the oracle's slot routing (CPU only).

Pinned by a pure-Python brute force of the definition (for each local expert
in order, its (t, j) pairs in flat order), the pages' expert-id rule
(golden), the identity slot mapping at top-k = 1, and invariants.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def brute_route(ids, w, start, L):
    T, k = ids.shape
    slots = []
    for e in range(L):
        for t in range(T):
            for j in range(k):
                if ids[t, j] - start == e:
                    slots.append((t, j, e))
    S = len(slots)
    n = T * k
    st = [-1] * n
    se = [-1] * n
    sw = [0.0] * n
    ts = [-1] * n
    for s, (t, j, e) in enumerate(slots):
        st[s], se[s], sw[s] = t, e, float(w[t, j])
        ts[t * k + j] = s
    counts = [sum(1 for *_, e in slots if e == x) for x in range(L)]
    return S, counts, st, se, sw, ts


@pytest.mark.parametrize("seed", range(6))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(0, 40))
    k = int(rng.integers(1, 6))
    E = int(rng.integers(4, 30))
    L = int(rng.integers(1, E + 1))
    start = int(rng.integers(0, E - L + 1))
    ids = rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)  # includes out-of-range ids
    w = rng.random((T, k)).astype(np.float32)
    r = O.route(ids, w, start, L)
    S, counts, st, se, sw, ts = brute_route(ids, w, start, L)
    assert r["S"] == S
    assert r["counts"].tolist() == counts
    assert r["offsets"].tolist() == [0] + np.cumsum(counts).tolist()
    assert r["slot_token"].tolist() == st
    assert r["slot_expert"].tolist() == se
    assert np.array_equal(r["slot_weight"], np.array(sw, np.float32))
    assert r["token_slot"].tolist() == ts


def test_invariants_on_skewed_workload():
    cfg = W.get_config("mid_skew")
    ids, w = W.make_router(cfg)
    r = O.route(ids, w, cfg.expert_start, cfg.num_local)
    T, k = ids.shape
    S = r["S"]
    local = ids.reshape(-1) - cfg.expert_start
    valid = (local >= 0) & (local < cfg.num_local)
    assert S == valid.sum() == r["counts"].sum()
    assert np.all(np.diff(r["offsets"]) >= 0)
    # bijection between local (t, j) pairs and slots, token_slot is its inverse
    ts = r["token_slot"]
    assert sorted(ts[valid].tolist()) == list(range(S))
    assert np.all(ts[~valid] == -1)
    flat = np.arange(T * k)
    assert np.array_equal(r["slot_token"][ts[valid]], flat[valid] // k)
    # within each expert segment, flat indices strictly increase (stable order)
    for e in range(cfg.num_local):
        seg = np.nonzero(ts >= 0)[0][np.argsort(ts[ts >= 0])][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(r["slot_expert"][r["offsets"][e]:r["offsets"][e + 1]] == e)
    # padding entries past S
    assert np.all(r["slot_token"][S:] == -1) and np.all(r["slot_weight"][S:] == 0)
    # the skewed workload has empty experts and one hot expert
    assert (r["counts"] == 0).sum() >= 2
    assert r["counts"].max() > 0.2 * S


def test_topk1_identity_mapping():
    # pages (src history, identity-gather commit): at top-k = 1 with tokens already
    # in expert order the slot mapping is the identity; otherwise it is not,
    # even though the number of slots equals the number of tokens.
    T, L = 50, 6
    ids = np.sort(np.random.default_rng(0).integers(0, L, T)).astype(np.int32)[:, None]
    w = np.ones((T, 1), np.float32)
    r = O.route(ids, w, 0, L)
    assert r["S"] == T
    assert np.array_equal(r["slot_token"], np.arange(T))
    ids2 = np.random.default_rng(1).permutation(ids[:, 0])[:, None].astype(np.int32)
    r2 = O.route(ids2, w, 0, L)
    assert r2["S"] == T
    assert not np.array_equal(r2["slot_token"], np.arange(T))
    # the gathered ids are in expert order
    assert np.all(np.diff(ids2[r2["slot_token"], 0]) >= 0)


def test_global_to_local_ids_from_pages():
    g = json.load(open(os.path.join(GOLD, "expert_ids.json")))
    per = g["per_rank"]
    ids = np.array(g["example_ids"], np.int32)[None, :]
    w = np.ones_like(ids, dtype=np.float32)
    for rank in range(g["num_global"] // per):
        r = O.route(ids, w, rank * per, per)
        got = {int(ids[0, j]): int(r["slot_expert"][r["token_slot"][j]])
               for j in range(ids.shape[1]) if r["token_slot"][j] >= 0}
        want = {int(i): v[1] for i, v in g["owner_rank_and_local_id"].items() if v[0] == rank}
        assert got == want
    # rank 0 sees none of them: the zero-output symptom when ids are not shifted
    assert O.route(ids, w, 0, per)["S"] == 0


def test_shifting_start_moves_exactly_the_expected_entries():
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 384, (100, 8)).astype(np.int32)
    w = rng.random((100, 8)).astype(np.float32)
    for start in (0, 96, 336):
        r = O.route(ids, w, start, 48)
        expect = ((ids >= start) & (ids < start + 48)).reshape(-1)
        assert np.array_equal(r["token_slot"] >= 0, expect)


def test_tile_schedule_brute_force():
    counts = np.array([0, 5, 16, 17, 0, 1], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t = O.tile_schedule(counts, offsets, 16)
    assert t.tolist() == [[1, 0], [2, 5], [3, 21], [3, 37], [5, 38]]
    assert O.tile_schedule(np.zeros(3, np.int32), np.zeros(4, np.int32), 8).shape == (0, 2)
