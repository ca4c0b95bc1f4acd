"""The whole layer captured in a HIP graph (through torch.cuda.graph) and
replayed: every replay, with eager work and synchronizations in between,
must equal the eager output bit for bit, and the replayed output must match
the oracle layer within 1e-2 x max|oracle|, also after a new input. The
layer makes no host synchronisation, allocates nothing, and clears its
scalars with a kernel (no memset node), so it can be captured
(nvfp4_cutedsl.py history, graph-compatibility commits)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _parity_log import record

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


def rel_err(got, ref):
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / scale if scale > 0 else float(np.abs(got).max())


def log(msg):
    print(f"[gpu-graph] {msg}", flush=True)


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_quantized_moe_amd as nv
    return nv


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("name", ["tiny", "mid_skew"])
def test_graph_replay_matches_eager(nv, name):
    cfg = W.get_config(name)
    ids, w = W.make_router(cfg)
    x = W.make_activations(cfg)
    wg, wu, wd = W.make_weights(cfg)
    weights = nv.prepare_weights(_bf16(wg), _bf16(wu), _bf16(wd))
    T, k = ids.shape
    d_x, d_ids, d_w = _bf16(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    lay = nv.nvfp4_moe_ws_layout(T, k, cfg.hidden, cfg.inter, cfg.num_local)
    ws = torch.empty(lay["end"], dtype=torch.uint8, device=DEV)
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=DEV)
    fwd = lambda: nv.nvfp4_moe_forward(weights, d_x, d_ids, d_w, cfg.expert_start, out=out, ws=ws)
    log(f"{name}: eager warm-up on a side stream")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fwd()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    log(f"{name}: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for r in range(4):
        out.fill_(-1.0)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"{name}: replay {r}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
    P = O.prepare_weights(wg, wu, wd)
    err0 = rel_err(out.float().cpu().numpy(), O.bf16_to_f32(O.moe_forward(x, ids, w, cfg.expert_start, P).out))
    # a new input through the same graph: the replay follows the data
    x2 = W.make_activations(cfg)[::-1].copy()
    d_x.copy_(_bf16(x2))
    g.replay()
    torch.cuda.synchronize()
    replayed = out.clone()
    fwd()
    torch.cuda.synchronize()
    assert torch.equal(replayed.view(torch.int16), out.view(torch.int16))
    err1 = rel_err(replayed.float().cpu().numpy(), O.bf16_to_f32(O.moe_forward(x2, ids, w, cfg.expert_start, P).out))
    log(f"{name}: replay vs oracle rel err {err0:.3e}, with a new input {err1:.3e}")
    record(f"graph:{name}", rel_err=max(err0, err1), replays_equal_eager=5)
    assert err0 <= TOL and err1 <= TOL
