"""nvfp4_quantize_noalloc through the C ABI: the quantizer without a
workspace (its amax partials in the library's own device array) gives the
same q, sf and gs as nvfp4_quantize with a workspace, bit for bit, on two
calls in a row (the second on a smaller input, after the first left its
partials in the array), and it rejects more tensors than the array holds;
captured in a HIP graph, every replay equals the eager call, also with
other no-alloc calls (which overwrite the array) between the replays.
Collected last so that a failure here hides no other test."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _cases import quant_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_quantized_moe_amd as nv
    return nv


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _outputs(B, M, K):
    return (torch.full((B, M, K // 2), 0x5A, dtype=torch.uint8, device=DEV),
            torch.full((B, M, K // 16), 0x5A, dtype=torch.uint8, device=DEV),
            torch.full((B,), -1.0, dtype=torch.float32, device=DEV))


def _with_ws(nv, x):
    q, sf, gs = nv.nvfp4_quantize(x if x.dim() == 3 else x[None])
    return q, sf, gs


def test_noalloc_matches_workspace_entry_point(nv):
    rng = np.random.default_rng(77)
    big = quant_case("t3_outliers")                                            # [256, 1024], outliers at 2000
    small = W.bf16_bits((rng.standard_normal((3, 40, 256)) * np.array([1.0, 300.0, 1e-3])[:, None, None])
                        .astype(np.float32))                                   # 3 tensors, own scales each
    for i, bits in enumerate((big[None], small)):
        B, M, K = bits.shape
        x = _bf16(bits)
        log(f"call {i}: B={B} M={M} K={K}")
        q, sf, gs = _outputs(B, M, K)
        nv.nvfp4_quantize_noalloc(x, q, sf, gs)
        rq, rsf, rgs = _with_ws(nv, x)
        torch.cuda.synchronize()
        assert torch.equal(gs, rgs), i
        assert torch.equal(sf, rsf) and torch.equal(q, rq), i
        # and the oracle, tensor by tensor
        for b in range(B):
            oq, osf, ogs = O.quantize(bits[b])
            assert gs[b].item() == ogs
            assert np.array_equal(sf[b].cpu().numpy(), osf) and np.array_equal(q[b].cpu().numpy(), oq)


def test_noalloc_amax_in_and_limits(nv):
    rng = np.random.default_rng(78)
    bits = W.bf16_bits(rng.standard_normal((2, 16, 128)).astype(np.float32))
    x = _bf16(bits)
    amax = torch.tensor([2688.0, 3.0], dtype=torch.float32, device=DEV)
    q, sf, gs = _outputs(2, 16, 128)
    nv.nvfp4_quantize_noalloc(x, q, sf, gs, amax_in=amax)
    rq, rsf, rgs = nv.nvfp4_quantize(x, amax_in=amax)
    torch.cuda.synchronize()
    assert torch.equal(gs, rgs) and torch.equal(sf, rsf) and torch.equal(q, rq)
    # 129 tensors exceed the library's array: rejected before any launch
    big = torch.zeros((129, 1, 32), dtype=torch.bfloat16, device=DEV)
    q, sf, gs = _outputs(129, 1, 32)
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_quantize_noalloc(big, q, sf, gs)
    assert e.value.status == 4
    # 128 tensors fit
    nv.nvfp4_quantize_noalloc(big[:128], q[:128], sf[:128], gs[:128])
    torch.cuda.synchronize()
    assert not gs[:128].any().item() and not sf[:128].any().item()


def test_noalloc_graph_replay(nv):
    rng = np.random.default_rng(79)
    bits = quant_case("t3_outliers")[None]                                      # [1, 256, 1024]
    other = W.bf16_bits(rng.standard_normal((2, 64, 512)).astype(np.float32) * 40.0)
    x, xo = _bf16(bits), _bf16(other)
    q, sf, gs = _outputs(*bits.shape)
    qo, sfo, gso = _outputs(*other.shape)
    nv.nvfp4_quantize_noalloc(x, q, sf, gs)                   # eager reference (and the device array's set-up)
    torch.cuda.synchronize()
    ref = (q.clone(), sf.clone(), gs.clone())
    log("capture nvfp4_quantize_noalloc in a graph")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            nv.nvfp4_quantize_noalloc(x, q, sf, gs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        q.fill_(0x5A)
        sf.fill_(0x5A)
        gs.fill_(-1.0)
        nv.nvfp4_quantize_noalloc(xo, qo, sfo, gso)            # another call: new partials in the array
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gs, ref[2]) and torch.equal(sf, ref[1]) and torch.equal(q, ref[0]), r
    oq, osf, ogs = O.quantize(bits[0])
    assert gs[0].item() == ogs and np.array_equal(q[0].cpu().numpy(), oq)
