"""Python binding of libnvfp4moe.so — NVFP4 MoE expert FFN on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels;
torch provides device memory and the current stream. The functions carry the
names of the C entry points declared in include/nvfp4moe.h.

Importing this module loads the built library and fails loudly when it is
missing; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib", "LIB_PATH", "NVFP4Error", "EPI_BF16", "EPI_SILU_MUL", "EPI_SILU_MUL_DUAL", "WS_REGIONS", "nvfp4_quantize",
    "nvfp4_quantize_ws_bytes", "nvfp4_quantize_noalloc", "moe_route_slots", "moe_route_ws_bytes", "nvfp4_tile_table_len",
    "nvfp4_grouped_gemm", "moe_weighted_scatter", "nvfp4_fold_scales", "nvfp4_packed_bytes",
    "nvfp4_pack_weights", "nvfp4_moe_forward", "nvfp4_quantize_static", "nvfp4_grouped_gemm_silu_nvfp4",
    "nvfp4_moe_forward_static", "calibrate_static_gs", "nvfp4_moe_forward_stage_events", "STAGES",
    "nvfp4_moe_ws_bytes", "nvfp4_moe_ws_layout", "nvfp4_moe_tile_m", "MoEWeights", "prepare_weights",
    "ws_view",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4moe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python __graft_entry__.py` (build()) first")
lib = ctypes.CDLL(LIB_PATH)

EPI_BF16, EPI_SILU_MUL, EPI_SILU_MUL_DUAL = 0, 1, 2
WS_REGIONS = ["x_q", "x_sf", "scalars", "counts", "offsets", "slot_token", "slot_expert", "slot_weight",
              "token_slot", "tiles", "route_scratch", "h", "h_q", "h_sf", "y", "quant_scratch", "end"]

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class _Weights(ctypes.Structure):
    _fields_ = [("num_local", _i32), ("hidden", _i32), ("inter", _i32),
                ("w1", _vp), ("w1_gs", _vp), ("w2", _vp), ("w2_gs", _vp), ("w1_dual_gs", _i32)]


def _sig(name, res, *args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_status_string = _sig("nvfp4_status_string", ctypes.c_char_p, ctypes.c_int)
_version = _sig("nvfp4moe_version", ctypes.c_int)
_quantize_ws = _sig("nvfp4_quantize_ws_bytes", _sz, _i64, _i64, _i64)
_quantize = _sig("nvfp4_quantize", ctypes.c_int, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_quantize_noalloc = _sig("nvfp4_quantize_noalloc", ctypes.c_int, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp)
_quantize_static = _sig("nvfp4_quantize_static", ctypes.c_int, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp)
_route_ws = _sig("moe_route_ws_bytes", _sz, _i32, _i32, _i32)
_tile_len = _sig("nvfp4_tile_table_len", _i64, _i64, _i32, _i32)
_route = _sig("moe_route_slots", ctypes.c_int, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_gemm = _sig("nvfp4_grouped_gemm", ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
             _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp)
_gemm_nvfp4 = _sig("nvfp4_grouped_gemm_silu_nvfp4", ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                   _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp)
_packed_bytes = _sig("nvfp4_packed_bytes", _i64, _i64, _i64, _i64)
_pack = _sig("nvfp4_pack_weights", ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _vp, _vp)
_scatter = _sig("moe_weighted_scatter", ctypes.c_int, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp)
_fold = _sig("nvfp4_fold_scales", ctypes.c_int, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp)
_moe_ws_layout = _sig("nvfp4_moe_ws_layout", _sz, _i32, _i32, _i32, _i32, _i32, _i32,
                      ctypes.POINTER(_sz))
_moe_ws = _sig("nvfp4_moe_ws_bytes", _sz, _i32, _i32, _i32, _i32, _i32)
_moe_tile_m = _sig("nvfp4_moe_tile_m", _i32, _i32, _i32, _i32)
_forward = _sig("nvfp4_moe_forward", ctypes.c_int, ctypes.POINTER(_Weights), _vp, _i32, _vp, _vp,
                _i32, _i32, _vp, _vp, _sz, _vp)
_forward_stages = _sig("nvfp4_moe_forward_stage_events", ctypes.c_int, ctypes.POINTER(_Weights), _vp, _i32, _vp,
                       _vp, _i32, _i32, _vp, _vp, _sz, ctypes.POINTER(_vp), _vp)
_forward_static = _sig("nvfp4_moe_forward_static", ctypes.c_int, ctypes.POINTER(_Weights), _vp, _i32, _vp, _vp,
                       _i32, _i32, _vp, _vp, _vp, _sz, _vp)


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: status {status} ({_status_string(status).decode()})")
        self.status = status


def _check(status: int, call: str):
    if status != 0:
        raise NVFP4Error(status, call)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    """t must be a contiguous tensor of dtype on the current device (the
    device whose current stream the call is issued on)."""
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name}: expected a contiguous CUDA {dtype} tensor, got {t.dtype} on {t.device}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return t


def _buf(t, dtype, numel, name):
    """A caller-provided buffer (or None): as _dev, holding at least numel
    elements, since the library sees only its address."""
    if t is None:
        return None
    _dev(t, dtype, name)
    if t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, got {t.numel()}")
    return t


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def version() -> int:
    return _version()


def _alloc_ws(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------- quantize

def nvfp4_quantize_ws_bytes(B, M, K) -> int:
    return int(_quantize_ws(B, M, K))


def nvfp4_quantize(x, amax_in=None, q=None, sf=None, gs=None, ws=None):
    """x: BF16 [M, K] or [B, M, K] -> (q uint8 [..., K/2], sf uint8 [..., K/16], gs float32 [B])."""
    _dev(x, torch.bfloat16, "x")
    if x.dim() not in (2, 3):
        raise ValueError(f"x: expected [M, K] or [B, M, K], got shape {tuple(x.shape)}")
    batched = x.dim() == 3
    B, M, K = (x.shape if batched else (1, *x.shape))
    dev = x.device
    q = torch.empty((B, M, K // 2), dtype=torch.uint8, device=dev) if q is None else _buf(q, torch.uint8, B * M * K // 2, "q")
    sf = (torch.empty((B, M, K // 16), dtype=torch.uint8, device=dev) if sf is None
          else _buf(sf, torch.uint8, B * M * K // 16, "sf"))
    gs = torch.empty((B,), dtype=torch.float32, device=dev) if gs is None else _buf(gs, torch.float32, B, "gs")
    ws = _alloc_ws(nvfp4_quantize_ws_bytes(B, M, K), dev) if ws is None else _buf(ws, torch.uint8, 0, "ws")
    _buf(amax_in, torch.float32, B, "amax_in")
    _check(_quantize(_ptr(x), B, M, K, _ptr(amax_in), _ptr(q), _ptr(sf), _ptr(gs), _ptr(ws),
                     ws.numel(), _stream()), "nvfp4_quantize")
    if not batched:
        return q[0], sf[0], gs
    return q, sf, gs


def nvfp4_quantize_noalloc(x, q, sf, gs, amax_in=None):
    """nvfp4_quantize into caller-provided q, sf, gs without a workspace: the
    library keeps the amax partials in its own device array (at most 128
    tensors; calls that overlap on one device race). Allocates nothing."""
    _dev(x, torch.bfloat16, "x")
    if x.dim() not in (2, 3):
        raise ValueError(f"x: expected [M, K] or [B, M, K], got shape {tuple(x.shape)}")
    B, M, K = (x.shape if x.dim() == 3 else (1, *x.shape))
    _buf(q, torch.uint8, B * M * K // 2, "q")
    _buf(sf, torch.uint8, B * M * K // 16, "sf")
    _buf(gs, torch.float32, B, "gs")
    _buf(amax_in, torch.float32, B, "amax_in")
    _check(_quantize_noalloc(_ptr(x), B, M, K, _ptr(amax_in), _ptr(q), _ptr(sf), _ptr(gs), _stream()),
           "nvfp4_quantize_noalloc")


def nvfp4_quantize_static(x, gs, q=None, sf=None):
    """x: BF16 [M, K] or [B, M, K] quantized with the fixed global scales gs
    (float32 [B], device) -> (q uint8 [..., K/2], sf uint8 [..., K/16])."""
    _dev(x, torch.bfloat16, "x")
    if x.dim() not in (2, 3):
        raise ValueError(f"x: expected [M, K] or [B, M, K], got shape {tuple(x.shape)}")
    batched = x.dim() == 3
    B, M, K = (x.shape if batched else (1, *x.shape))
    _buf(gs, torch.float32, B, "gs")
    dev = x.device
    q = torch.empty((B, M, K // 2), dtype=torch.uint8, device=dev) if q is None else _buf(q, torch.uint8, B * M * K // 2, "q")
    sf = (torch.empty((B, M, K // 16), dtype=torch.uint8, device=dev) if sf is None
          else _buf(sf, torch.uint8, B * M * K // 16, "sf"))
    _check(_quantize_static(_ptr(x), B, M, K, _ptr(gs), _ptr(q), _ptr(sf), _stream()), "nvfp4_quantize_static")
    if not batched:
        return q[0], sf[0]
    return q, sf


# ------------------------------------------------------------------------- route

def moe_route_ws_bytes(T, k, num_local) -> int:
    return int(_route_ws(T, k, num_local))


def nvfp4_tile_table_len(cap, num_local, tile_m) -> int:
    return int(_tile_len(cap, num_local, tile_m))


def moe_route_slots(topk_ids, topk_w, expert_start, num_local, tile_m):
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_w, torch.float32, "topk_w")
    T, k = topk_ids.shape
    _shape(topk_w, (T, k), "topk_w")
    dev = topk_ids.device
    cap = T * k
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(
        counts=torch.empty(num_local, **i32), offsets=torch.empty(num_local + 1, **i32),
        slot_token=torch.empty(cap, **i32), slot_expert=torch.empty(cap, **i32),
        slot_weight=torch.empty(cap, dtype=torch.float32, device=dev), token_slot=torch.empty(cap, **i32),
        tile_table=torch.empty(nvfp4_tile_table_len(cap, num_local, tile_m), **i32),
    )
    ws = _alloc_ws(moe_route_ws_bytes(T, k, num_local), dev)
    _check(_route(_ptr(topk_ids), _ptr(topk_w), T, k, expert_start, num_local, tile_m,
                  _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["slot_token"]), _ptr(out["slot_expert"]),
                  _ptr(out["slot_weight"]), _ptr(out["token_slot"]), _ptr(out["tile_table"]),
                  _ptr(ws), ws.numel(), _stream()), "moe_route_slots")
    return out


# ------------------------------------------------------------------ grouped GEMM

def nvfp4_packed_bytes(B, N, K) -> int:
    return int(_packed_bytes(B, N, K))


def nvfp4_pack_weights(q, sf, out=None):
    """Row-major NVFP4 matrices q uint8 [B, N, K/2], sf uint8 [B, N, K/16] ->
    packed uint8 [B, N/32, K/128, 2304] in the grouped GEMM's operand order."""
    _dev(q, torch.uint8, "q")
    _dev(sf, torch.uint8, "sf")
    B, N, Kh = q.shape
    K = Kh * 2
    if tuple(sf.shape) != (B, N, K // 16):
        raise ValueError(f"sf shape {tuple(sf.shape)} does not match q {tuple(q.shape)}")
    if N % 32 or K % 128:
        raise ValueError(f"packing needs N % 32 == 0 and K % 128 == 0, got N={N}, K={K}")
    out = (torch.empty((B, N // 32, K // 128, 2304), dtype=torch.uint8, device=q.device) if out is None
           else _buf(out, torch.uint8, B * N * K // 32 * 18, "out"))
    _check(_pack(_ptr(q), _ptr(sf), B, N, K, _ptr(out), _stream()), "nvfp4_pack_weights")
    return out


def _check_gemm_operands(a_q, a_sf, a_row_index, a_gs, b_gs, offsets, tile_table, rows_cap, tile_m, L, K, n_b_gs):
    _dev(a_q, torch.uint8, "a_q")
    _dev(a_sf, torch.uint8, "a_sf")
    if a_q.dim() != 2 or a_q.shape[1] != K // 2 or tuple(a_sf.shape) != (a_q.shape[0], K // 16):
        raise ValueError(f"a_q {tuple(a_q.shape)} / a_sf {tuple(a_sf.shape)}: expected [rows, {K // 2}] / "
                         f"[rows, {K // 16}]")
    # rows read: slot s, or a_row_index[s], for the slots below offsets[L] (device data, at most rows_cap); with
    # a row index the indices' range is the caller's contract, without one every slot row must exist
    if a_row_index is None and a_q.shape[0] < rows_cap:
        raise ValueError(f"a_q: {a_q.shape[0]} rows, but slots up to rows_cap = {rows_cap} read their own row")
    _buf(a_row_index, torch.int32, 0, "a_row_index")
    _buf(a_gs, torch.float32, 1, "a_gs")
    _buf(b_gs, torch.float32, n_b_gs, "b_gs")
    _buf(offsets, torch.int32, L + 1, "offsets")
    _buf(tile_table, torch.int32, nvfp4_tile_table_len(rows_cap, L, tile_m), "tile_table")


def _packed_dims(b_packed, name="b_packed"):
    """(L, N, K) of packed weights uint8 [L, N/32, K/128, 2304]."""
    _dev(b_packed, torch.uint8, name)
    if b_packed.dim() != 4 or b_packed.shape[3] != 2304:
        raise ValueError(f"{name}: expected packed weights [L, N/32, K/128, 2304], got {tuple(b_packed.shape)}")
    L, n32, k128, _ = b_packed.shape
    return L, n32 * 32, k128 * 128


def nvfp4_grouped_gemm(a_q, a_sf, a_row_index, a_gs, b_packed, b_gs, offsets, tile_table, rows_cap,
                       tile_m, epilogue=EPI_BF16, d=None, amax_out=None):
    """b_packed: uint8 [L, N/32, K/128, 2304] from nvfp4_pack_weights. A rows:
    a_row_index[s] for slot s when given (device indices < a_q's row count,
    the caller's contract), else s (a_q then needs rows_cap rows)."""
    L, N, K = _packed_dims(b_packed)
    dev = b_packed.device
    n_out = N // 2 if epilogue in (EPI_SILU_MUL, EPI_SILU_MUL_DUAL) else N
    _check_gemm_operands(a_q, a_sf, a_row_index, a_gs, b_gs, offsets, tile_table, rows_cap, tile_m, L, K,
                         2 * L if epilogue == EPI_SILU_MUL_DUAL else L)
    d = (torch.empty((rows_cap, n_out), dtype=torch.bfloat16, device=dev) if d is None
         else _buf(d, torch.bfloat16, rows_cap * n_out, "d"))
    _buf(amax_out, torch.float32, 1, "amax_out")
    _check(_gemm(_ptr(a_q), _ptr(a_sf), _ptr(a_row_index), _ptr(a_gs), _ptr(b_packed), _ptr(b_gs),
                 _ptr(offsets), _ptr(tile_table), L, rows_cap, N, K, tile_m, epilogue, _ptr(d), _ptr(amax_out),
                 _stream()), "nvfp4_grouped_gemm")
    return d


def nvfp4_grouped_gemm_silu_nvfp4(a_q, a_sf, a_row_index, a_gs, b_packed, b_gs, offsets, tile_table, rows_cap,
                                  tile_m, out_gs, d_q=None, d_sf=None):
    """L1 with the SiLU*up epilogue writing h as NVFP4 with the fixed global
    scale out_gs [1]: returns (h_q uint8 [rows_cap, N/4], h_sf uint8 [rows_cap, N/32]).
    b_gs [L] (folded W1) or [L, 2] (gate and up global scales)."""
    L, N, K = _packed_dims(b_packed)
    dev = b_packed.device
    dual = 1 if b_gs.dim() == 2 else 0
    _check_gemm_operands(a_q, a_sf, a_row_index, a_gs, b_gs, offsets, tile_table, rows_cap, tile_m, L, K,
                         2 * L if dual else L)
    _buf(out_gs, torch.float32, 1, "out_gs")
    d_q = (torch.empty((rows_cap, N // 4), dtype=torch.uint8, device=dev) if d_q is None
           else _buf(d_q, torch.uint8, rows_cap * (N // 4), "d_q"))
    d_sf = (torch.empty((rows_cap, N // 32), dtype=torch.uint8, device=dev) if d_sf is None
            else _buf(d_sf, torch.uint8, rows_cap * (N // 32), "d_sf"))
    _check(_gemm_nvfp4(_ptr(a_q), _ptr(a_sf), _ptr(a_row_index), _ptr(a_gs), _ptr(b_packed), _ptr(b_gs), dual,
                       _ptr(offsets), _ptr(tile_table), L, rows_cap, N, K, tile_m, _ptr(out_gs), _ptr(d_q),
                       _ptr(d_sf), _stream()), "nvfp4_grouped_gemm_silu_nvfp4")
    return d_q, d_sf


def moe_weighted_scatter(y, token_slot, topk_w, out=None):
    """out[t] = sum over j of topk_w[t, j] * y[token_slot[t*k + j]] (slots >= 0),
    y BF16 [rows, H] with every slot index < rows (the caller's contract)."""
    _dev(y, torch.bfloat16, "y")
    _dev(topk_w, torch.float32, "topk_w")
    T, k = topk_w.shape
    H = y.shape[1]
    _buf(token_slot, torch.int32, T * k, "token_slot")
    out = (torch.empty((T, H), dtype=torch.bfloat16, device=y.device) if out is None
           else _buf(out, torch.bfloat16, T * H, "out"))
    _check(_scatter(_ptr(y), _ptr(token_slot), _ptr(topk_w), T, k, H, _ptr(out), _stream()),
           "moe_weighted_scatter")
    return out


def nvfp4_fold_scales(w1_sf, gs_gate, gs_up, gs1=None):
    """In place on w1_sf [L, 2I, K/16]; returns gs1 [L]."""
    _dev(w1_sf, torch.uint8, "w1_sf")
    L, two_i, k16 = w1_sf.shape
    _buf(gs_gate, torch.float32, L, "gs_gate")
    _buf(gs_up, torch.float32, L, "gs_up")
    gs1 = torch.empty(L, dtype=torch.float32, device=w1_sf.device) if gs1 is None else _buf(gs1, torch.float32, L, "gs1")
    _check(_fold(_ptr(w1_sf), _ptr(gs_gate), _ptr(gs_up), _ptr(gs1), L, two_i // 2, k16 * 16, _stream()),
           "nvfp4_fold_scales")
    return gs1


# --------------------------------------------------------------------- the layer

def nvfp4_moe_ws_layout(T, k, hidden, inter, num_local) -> dict:
    offs = (_sz * len(WS_REGIONS))()
    tile_m = nvfp4_moe_tile_m(T, k, num_local)
    _moe_ws_layout(T, k, hidden, inter, num_local, tile_m, offs)
    return {name: int(offs[i]) for i, name in enumerate(WS_REGIONS)}


def nvfp4_moe_ws_bytes(T, k, hidden, inter, num_local) -> int:
    return int(_moe_ws(T, k, hidden, inter, num_local))


def nvfp4_moe_tile_m(T, k, num_local) -> int:
    return int(_moe_tile_m(T, k, num_local))


def ws_view(ws, layout, region, dtype, shape):
    """A typed view of one workspace region (for reading intermediates)."""
    off = layout[region]
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).view(*shape)


class MoEWeights:
    """Device NVFP4 layer weights for one rank (L local experts): packed W1
    (gate rows then up rows) and packed W2. W1's gate/up scales are either
    folded to one global scale per expert (w1_gs [L]) or kept per half
    (w1_gs [L, 2] = gs_gate, gs_up). With keep_unpacked, prepare_weights also
    keeps the row-major forms (w1_q, w1_sf, w2_q, w2_sf) for inspection."""

    def __init__(self, w1, w1_gs, w2, w2_gs):
        self.w1, self.w1_gs, self.w2, self.w2_gs = w1, w1_gs, w2, w2_gs
        self.dual_gs = w1_gs.dim() == 2
        self.num_local, two_i, self.hidden = _packed_dims(w1, "w1")
        self.inter = two_i // 2
        if _packed_dims(w2, "w2") != (self.num_local, self.hidden, self.inter):
            raise ValueError(f"packed W2 shape {tuple(w2.shape)} does not match W1 {tuple(w1.shape)}")
        _dev(w1_gs, torch.float32, "w1_gs")
        _dev(w2_gs, torch.float32, "w2_gs")
        if tuple(w1_gs.shape) not in ((self.num_local,), (self.num_local, 2)):
            raise ValueError(f"w1_gs shape {tuple(w1_gs.shape)}: expected [L] or [L, 2]")
        if tuple(w2_gs.shape) != (self.num_local,):
            raise ValueError(f"w2_gs shape {tuple(w2_gs.shape)}: expected [L] = [{self.num_local}]")
        self._c = _Weights(self.num_local, self.hidden, self.inter, w1.data_ptr(), w1_gs.data_ptr(),
                           w2.data_ptr(), w2_gs.data_ptr(), 1 if self.dual_gs else 0)


def prepare_weights(w_gate, w_up, w_down, keep_unpacked=False, fold=True) -> MoEWeights:
    """Offline weight preparation on the GPU: quantize each (expert, projection)
    with its own global scale, fold the gate/up scale ratio (or, with
    fold=False, keep both halves' scales and global scales), and pack both
    matrices for the grouped GEMM.

    w_gate, w_up: BF16 [L, I, H]; w_down: BF16 [L, H, I].
    """
    L, I, H = w_gate.shape
    gate_up = torch.cat([w_gate, w_up], dim=1).contiguous()          # [L, 2I, H]: tensor b = 2e + p
    q1, sf1, gs_pair = nvfp4_quantize(gate_up.view(2 * L, I, H))
    del gate_up
    w1_q = q1.view(L, 2 * I, H // 2)
    w1_sf = sf1.view(L, 2 * I, H // 16)
    gs_pair = gs_pair.view(L, 2)
    gs_gate, gs_up = gs_pair[:, 0].contiguous(), gs_pair[:, 1].contiguous()
    w1_gs = nvfp4_fold_scales(w1_sf, gs_gate, gs_up) if fold else gs_pair.contiguous()
    w2_q, w2_sf, w2_gs = nvfp4_quantize(w_down.contiguous())
    w = MoEWeights(nvfp4_pack_weights(w1_q, w1_sf), w1_gs, nvfp4_pack_weights(w2_q, w2_sf), w2_gs)
    w.gs_gate, w.gs_up = gs_gate, gs_up
    if keep_unpacked:
        w.w1_q, w.w1_sf, w.w2_q, w.w2_sf = w1_q, w1_sf, w2_q, w2_sf
    return w


def _check_layer_inputs(weights, x, topk_w, T, k):
    _shape(x, (T, weights.hidden), "x")
    _shape(topk_w, (T, k), "topk_w")
    for name in ("w1", "w1_gs", "w2", "w2_gs"):
        _dev(getattr(weights, name), getattr(weights, name).dtype, f"weights.{name}")


def _layer_buffers(weights, x, topk_ids, topk_w, out, ws):
    _dev(x, torch.bfloat16, "x")
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_w, torch.float32, "topk_w")
    T, k = topk_ids.shape
    H = weights.hidden
    _check_layer_inputs(weights, x, topk_w, T, k)
    dev = x.device
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else _buf(out, torch.bfloat16, T * H, "out")
    need = nvfp4_moe_ws_bytes(T, k, H, weights.inter, weights.num_local)
    ws = _alloc_ws(need, dev) if ws is None else _buf(ws, torch.uint8, 0, "ws")
    return T, k, out, ws


def nvfp4_moe_forward(weights: MoEWeights, x, topk_ids, topk_w, expert_start, out=None, ws=None):
    """One rank's partial output BF16 [T, H] of the expert FFN."""
    T, k, out, ws = _layer_buffers(weights, x, topk_ids, topk_w, out, ws)
    _check(_forward(ctypes.byref(weights._c), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w), k, expert_start,
                    _ptr(out), _ptr(ws), ws.numel(), _stream()), "nvfp4_moe_forward")
    return out


# stages between the events of nvfp4_moe_forward_stage_events (NVFP4_STAGE_* order)
STAGES = ["a1_amax_route", "a2_quantize_x", "a3_route", "a4_a5_l1_gemm", "a6_quantize_h", "a7_l2_gemm",
          "a8_scatter"]


def nvfp4_moe_forward_stage_events(weights: MoEWeights, x, topk_ids, topk_w, expert_start, events, out=None,
                                   ws=None):
    """nvfp4_moe_forward with events recorded between its launches: events is
    a list of len(STAGES) + 1 torch.cuda.Event (timing enabled, each recorded
    once beforehand so that it exists) or None (no record there); events[i]
    to events[i + 1] spans stage STAGES[i] of this call."""
    if len(events) != len(STAGES) + 1:
        raise ValueError(f"events: expected {len(STAGES) + 1} entries, got {len(events)}")
    handles = (_vp * len(events))()
    for i, e in enumerate(events):
        if e is not None:
            if not e.cuda_event:
                raise ValueError(f"events[{i}]: not created yet (record it once first)")
            handles[i] = e.cuda_event
    T, k, out, ws = _layer_buffers(weights, x, topk_ids, topk_w, out, ws)
    _check(_forward_stages(ctypes.byref(weights._c), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w), k, expert_start,
                           _ptr(out), _ptr(ws), ws.numel(), handles, _stream()), "nvfp4_moe_forward_stage_events")
    return out


def nvfp4_moe_forward_static(weights: MoEWeights, x, topk_ids, topk_w, expert_start, gs, out=None, ws=None):
    """The layer with fixed global scales gs = float32 [2] (gs_x, gs_h) on the
    device, e.g. from calibrate_static_gs; no amax passes, h quantized in L1."""
    _dev(gs, torch.float32, "gs")
    if gs.numel() != 2:
        raise ValueError(f"gs: expected 2 values (gs_x, gs_h), got {gs.numel()}")
    T, k, out, ws = _layer_buffers(weights, x, topk_ids, topk_w, out, ws)
    _check(_forward_static(ctypes.byref(weights._c), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w), k, expert_start,
                           _ptr(gs), _ptr(out), _ptr(ws), ws.numel(), _stream()), "nvfp4_moe_forward_static")
    return out


def calibrate_static_gs(weights: MoEWeights, x, topk_ids, topk_w, expert_start):
    """Global scales (gs_x, gs_h) that nvfp4_moe_forward measures on a
    calibration batch, as a device float32 [2] for nvfp4_moe_forward_static."""
    T, k = topk_ids.shape
    ws = _alloc_ws(nvfp4_moe_ws_bytes(T, k, weights.hidden, weights.inter, weights.num_local), x.device)
    nvfp4_moe_forward(weights, x, topk_ids, topk_w, expert_start, ws=ws)
    lay = nvfp4_moe_ws_layout(T, k, weights.hidden, weights.inter, weights.num_local)
    sc = ws_view(ws, lay, "scalars", torch.float32, (4,))
    return torch.stack([sc[0], sc[2]]).contiguous()
