"""Thin Python binding of libmoe.so (the HIP library), same names as the C ABI.

Only argument marshalling lives here: torch tensors are checked for dtype,
device and contiguity, output tensors are allocated with torch (device memory
is torch's job), and the raw pointers plus the current HIP stream are passed
to the C entry points.  Every step of the layer runs in the library's HIP
kernels; there is no fallback path.  Importing this module raises if the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m fine_grained_moe_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

_i32, _i64, _sz, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/moe.h
_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_align": (_i32, []),
    "moe_capacity_rows": (_i64, [_i32, _i32, _i32]),
    "moe_route_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_permute_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_permute_check": (_i32, [_p]),
    "moe_permute_noalloc_max_tokens": (_i32, []),
    "moe_permute_noalloc": (_i32, [_i32, _i32, _i32, _i32, _i32, _p, _p, _i64, _p, _p, _p, _p, _p,
                                   _p, _p, _p]),
    "moe_route_bwd_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_seq_balance_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_route_bwd_dense_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_route": (_i32, [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_permute": (_i32, [_i32, _i32, _i32, _i32, _i32, _p, _p, _i64, _p, _p, _p, _p, _p, _p,
                           _p, _sz, _p]),
    "moe_grouped_swiglu_fwd": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p,
                                      _p, _p]),
    "moe_grouped_gate_up_fwd": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_down_fwd": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "moe_dense_fwd_split_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_dense_gate_up_fwd_split": (_i32, [_i64, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_dense_down_fwd_split": (_i32, [_i64, _i32, _i32, _p, _p, _p, _p, _sz, _p]),
    "moe_combine": (_i32, [_i32, _i32, _i32, _p, _p, _p, _p, _p, _p]),
    "moe_combine_bwd": (_i32, [_i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_swiglu_bwd": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p,
                                      _p, _p, _p, _p, _p, _p]),
    "moe_grouped_down_dgrad": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_down_wgrad": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_gate_up_dgrad": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_gate_up_wgrad": (_i32, [_i32, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "moe_route_bwd": (_i32, [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                             _p, _sz, _p]),
    "moe_permute_bwd": (_i32, [_i32, _i32, _i32, _p, _p, _p, _p, _p, _p]),
    "moe_route_permute_bwd": (_i32, [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                     _p, _p, _p, _p, _p, _sz, _p]),
    "moe_bias_update": (_i32, [_i32, _p, _p, ctypes.c_float, _p]),
    "moe_seq_balance_fwd": (_i32, [_i32, _i32, _i32, _i32, _p, _p, ctypes.c_float, _p, _p, _p, _sz,
                                   _p]),
    "moe_seq_balance_bwd": (_i32, [_i32, _i32, _i32, _i32, _p, _p, ctypes.c_float, _p, _p, _p]),
    "moe_route_dlogit": (_i32, [_i32, _i32, _i32, _p, _p, _p, _p, _p]),
    "moe_route_bwd_dense": (_i32, [_i32, _i32, _i32, _p, _p, _p, _p, _p, _i32, _p, _sz, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args

EXPORTED = tuple(_SIGS)


class MoEError(RuntimeError):
    pass


def _check(status: int):
    if status != 0:
        msg = _lib.moe_last_error().decode()
        raise MoEError(f"{_lib.moe_status_string(status).decode()} ({status}): {msg}")


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _expect(**items):
    """name=(tensor, shape): every given tensor must have exactly that shape.
    The library sees raw pointers only, so a buffer of the wrong size would be
    read or written out of bounds; the binding refuses it instead."""
    for name, (t, shape) in items.items():
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _seg_shapes(G, M, offsets, counts, tile_expert):
    """Segment tables of a grouped call (all None for a dense call)."""
    A = int(_lib.moe_align())
    _expect(offsets=(offsets, (G + 1,)), counts=(counts, (G,)), tile_expert=(tile_expert, (M // A,)))


def _stream():
    return torch.cuda.current_stream().cuda_stream


BF16, F32, I32 = torch.bfloat16, torch.float32, torch.int32


# ---------------------------------------------------------------------------
# host queries
# ---------------------------------------------------------------------------
def moe_align() -> int:
    return int(_lib.moe_align())


def moe_capacity_rows(T: int, E: int, K: int) -> int:
    return int(_lib.moe_capacity_rows(T, E, K))


def moe_route_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(_lib.moe_route_workspace_bytes(T, H, E))


def moe_permute_workspace_bytes(T: int, E: int, K: int) -> int:
    return int(_lib.moe_permute_workspace_bytes(T, E, K))


def moe_route_bwd_workspace_bytes(T: int, H: int, E: int, K: int) -> int:
    return int(_lib.moe_route_bwd_workspace_bytes(T, H, E, K))


# ---------------------------------------------------------------------------
# entry points (outputs allocated when not given)
# ---------------------------------------------------------------------------
def moe_seq_balance_workspace_bytes(T: int, E: int, seq_len: int) -> int:
    return int(_lib.moe_seq_balance_workspace_bytes(T, E, seq_len))


def moe_route_bwd_dense_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(_lib.moe_route_bwd_dense_workspace_bytes(T, H, E))


def moe_route(x, w_router, bias, K, topk_idx=None, topk_w=None, topk_s=None, ws=None,
              scores=None):
    """Returns (topk_idx, topk_w, topk_s); pass a [T,E] fp32 `scores` tensor to
    also receive every expert's score."""
    T, H = x.shape
    E = w_router.shape[1]
    dev = x.device
    topk_idx = torch.empty((T, K), dtype=I32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, K), dtype=F32, device=dev) if topk_w is None else topk_w
    topk_s = torch.empty((T, K), dtype=F32, device=dev) if topk_s is None else topk_s
    if ws is None:
        ws = torch.empty(max(moe_route_workspace_bytes(T, H, E), 1), dtype=torch.uint8, device=dev)
    _expect(w_router=(w_router, (H, E)), bias=(bias, (E,)), topk_idx=(topk_idx, (T, K)),
            topk_w=(topk_w, (T, K)), topk_s=(topk_s, (T, K)), scores=(scores, (T, E)))
    _check(_lib.moe_route(T, H, E, K, _ptr(x, BF16, "x"), _ptr(w_router, F32, "w_router"),
                          _ptr(bias, F32, "bias"), _ptr(topk_idx, I32, "topk_idx"),
                          _ptr(topk_w, F32, "topk_w"), _ptr(topk_s, F32, "topk_s"),
                          _ptr(scores, F32, "scores"), _ptr(ws), ws.numel(), _stream()))
    return topk_idx, topk_w, topk_s


def moe_permute(topk_idx, x, E, m_cap=None, out=None, ws=None):
    """Returns dict(counts, offsets, row_of, src_token, tile_expert, x_rows,
    status).  status is the call's data-check block (int32 [4], a view of the
    workspace's first 16 bytes, overwritten by the next call on the same
    workspace); moe_permute_check(status) decodes it."""
    T, K = topk_idx.shape
    H = x.shape[1]
    A = moe_align()
    m_cap = moe_capacity_rows(T, E, K) if m_cap is None else m_cap
    dev = x.device
    if out is None:
        out = dict(counts=torch.empty(E, dtype=I32, device=dev),
                   offsets=torch.empty(E + 1, dtype=I32, device=dev),
                   row_of=torch.empty((T, K), dtype=I32, device=dev),
                   src_token=torch.empty(m_cap, dtype=I32, device=dev),
                   tile_expert=torch.empty(m_cap // A, dtype=I32, device=dev),
                   x_rows=torch.empty((m_cap, H), dtype=BF16, device=dev))
    _expect(x=(x, (T, H)), counts=(out["counts"], (E,)), offsets=(out["offsets"], (E + 1,)),
            row_of=(out["row_of"], (T, K)), src_token=(out["src_token"], (m_cap,)),
            tile_expert=(out["tile_expert"], (m_cap // A,)), x_rows=(out["x_rows"], (m_cap, H)))
    nbytes = moe_permute_workspace_bytes(T, E, K)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(_lib.moe_permute(T, H, E, K, A, _ptr(topk_idx, I32, "topk_idx"), _ptr(x, BF16, "x"),
                            m_cap, _ptr(out["counts"], I32), _ptr(out["offsets"], I32),
                            _ptr(out["row_of"], I32), _ptr(out["src_token"], I32),
                            _ptr(out["tile_expert"], I32), _ptr(out["x_rows"], BF16),
                            _ptr(ws), ws.numel(), _stream()))
    out["status"] = ws[:16].view(I32)
    return out


def moe_permute_noalloc_max_tokens() -> int:
    return int(_lib.moe_permute_noalloc_max_tokens())


def moe_permute_noalloc(topk_idx, x, E, out, status=None):
    """moe_permute without a workspace (the library's static device array):
    every output buffer comes from the caller in `out` (the dict moe_permute
    returns, x_rows included), so the call allocates nothing.  status: int32
    [4] device tensor receiving the data-check block, or None.  Returns out."""
    T, K = topk_idx.shape
    H = x.shape[1]
    A = moe_align()
    m_cap = out["src_token"].shape[0]
    _expect(x=(x, (T, H)), counts=(out["counts"], (E,)), offsets=(out["offsets"], (E + 1,)),
            row_of=(out["row_of"], (T, K)), src_token=(out["src_token"], (m_cap,)),
            tile_expert=(out["tile_expert"], (m_cap // A,)), x_rows=(out["x_rows"], (m_cap, H)),
            status=(status, (4,)))
    _check(_lib.moe_permute_noalloc(T, H, E, K, A, _ptr(topk_idx, I32, "topk_idx"),
                                    _ptr(x, BF16, "x"), m_cap, _ptr(out["counts"], I32),
                                    _ptr(out["offsets"], I32), _ptr(out["row_of"], I32),
                                    _ptr(out["src_token"], I32), _ptr(out["tile_expert"], I32),
                                    _ptr(out["x_rows"], BF16), _ptr(status, I32, "status"),
                                    _stream()))
    return out


def moe_permute_check(status):
    """Decodes a moe_permute data-check block (int32 [4], on any device; this
    copies it to the host, so it waits for the call that wrote it).  Raises
    MoEError naming the rejected tokens, returns None when there are none."""
    words = status.detach().to("cpu", torch.int32).contiguous()
    _expect(status=(words, (4,)))
    _check(_lib.moe_permute_check(words.data_ptr()))


def moe_grouped_swiglu_fwd(x_rows, w1, w2, offsets=None, counts=None, tile_expert=None,
                           act=True, h=None, y_rows=None):
    """Grouped SwiGLU FFN.  act=True allocates the saved pre-activations,
    act=None skips them (inference), or pass a tensor.  Returns (act, h, y_rows)."""
    M, H = x_rows.shape
    G, twoF, H1 = w1.shape
    F = twoF // 2
    dev = x_rows.device
    if act is True:
        act = torch.empty((M, 2 * F), dtype=BF16, device=dev)
    elif act is False:
        act = None
    h = torch.empty((M, F), dtype=BF16, device=dev) if h is None else h
    y_rows = torch.empty((M, H), dtype=BF16, device=dev) if y_rows is None else y_rows
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(w1=(w1, (G, 2 * F, H)), w2=(w2, (G, H, F)), act=(act, (M, 2 * F)), h=(h, (M, F)),
            y_rows=(y_rows, (M, H)))
    _check(_lib.moe_grouped_swiglu_fwd(G, M, H, F, _ptr(offsets, I32), _ptr(counts, I32),
                                       _ptr(tile_expert, I32), _ptr(x_rows, BF16, "x_rows"),
                                       _ptr(w1, BF16, "w1"), _ptr(w2, BF16, "w2"),
                                       _ptr(act, BF16, "act"), _ptr(h, BF16, "h"),
                                       _ptr(y_rows, BF16, "y_rows"), _stream()))
    return act, h, y_rows


def moe_grouped_gate_up_fwd(x_rows, w1, offsets=None, counts=None, tile_expert=None, act=True,
                            h=None):
    """First half of moe_grouped_swiglu_fwd.  Returns (act, h)."""
    M, H = x_rows.shape
    G, twoF, _ = w1.shape
    F = twoF // 2
    dev = x_rows.device
    if act is True:
        act = torch.empty((M, 2 * F), dtype=BF16, device=dev)
    elif act is False:
        act = None
    h = torch.empty((M, F), dtype=BF16, device=dev) if h is None else h
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(w1=(w1, (G, 2 * F, H)), act=(act, (M, 2 * F)), h=(h, (M, F)))
    _check(_lib.moe_grouped_gate_up_fwd(G, M, H, F, _ptr(offsets, I32), _ptr(counts, I32),
                                        _ptr(tile_expert, I32), _ptr(x_rows, BF16, "x_rows"),
                                        _ptr(w1, BF16, "w1"), _ptr(act, BF16, "act"),
                                        _ptr(h, BF16, "h"), _stream()))
    return act, h


def moe_grouped_down_fwd(h, w2, offsets=None, counts=None, tile_expert=None, y_rows=None):
    """Second half of moe_grouped_swiglu_fwd.  Returns y_rows."""
    M, F = h.shape
    G, H, _ = w2.shape
    y_rows = torch.empty((M, H), dtype=BF16, device=h.device) if y_rows is None else y_rows
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(w2=(w2, (G, H, F)), y_rows=(y_rows, (M, H)))
    _check(_lib.moe_grouped_down_fwd(G, M, H, F, _ptr(offsets, I32), _ptr(counts, I32),
                                     _ptr(tile_expert, I32), _ptr(h, BF16, "h"),
                                     _ptr(w2, BF16, "w2"), _ptr(y_rows, BF16, "y_rows"),
                                     _stream()))
    return y_rows


def moe_dense_fwd_split_workspace_bytes(m_rows: int, H: int, F: int) -> int:
    return int(_lib.moe_dense_fwd_split_workspace_bytes(m_rows, H, F))


def _split_ws(ws, M, H, F, dev):
    if ws is None:
        ws = torch.empty(max(moe_dense_fwd_split_workspace_bytes(M, H, F), 1), dtype=torch.uint8,
                         device=dev)
    return ws


def moe_dense_gate_up_fwd_split(x, w1, act=True, h=None, ws=None):
    """Dense gate/up half (one group: the fused shared experts, w1 [1,2F,H])
    over all rows of x, the contraction split over workgroups when the batch
    is too small to fill the GPU.  Returns (act, h)."""
    M, H = x.shape
    twoF = w1.shape[1]
    F = twoF // 2
    dev = x.device
    if act is True:
        act = torch.empty((M, 2 * F), dtype=BF16, device=dev)
    elif act is False:
        act = None
    h = torch.empty((M, F), dtype=BF16, device=dev) if h is None else h
    ws = _split_ws(ws, M, H, F, dev)
    _expect(w1=(w1, (1, 2 * F, H)), act=(act, (M, 2 * F)), h=(h, (M, F)))
    _check(_lib.moe_dense_gate_up_fwd_split(M, H, F, _ptr(x, BF16, "x"), _ptr(w1, BF16, "w1"),
                                            _ptr(act, BF16, "act"), _ptr(h, BF16, "h"), _ptr(ws),
                                            ws.numel(), _stream()))
    return act, h


def moe_dense_down_fwd_split(h, w2, y=None, ws=None):
    """Dense down half (w2 [1,H,F]) with the same split.  Returns y."""
    M, F = h.shape
    H = w2.shape[1]
    y = torch.empty((M, H), dtype=BF16, device=h.device) if y is None else y
    ws = _split_ws(ws, M, H, F, h.device)
    _expect(w2=(w2, (1, H, F)), y=(y, (M, H)))
    _check(_lib.moe_dense_down_fwd_split(M, H, F, _ptr(h, BF16, "h"), _ptr(w2, BF16, "w2"),
                                         _ptr(y, BF16, "y"), _ptr(ws), ws.numel(), _stream()))
    return y


def moe_combine(y_rows, row_of, topk_w, y_shared=None, y=None):
    T, K = row_of.shape
    H = y_rows.shape[1]
    y = torch.empty((T, H), dtype=BF16, device=y_rows.device) if y is None else y
    _expect(topk_w=(topk_w, (T, K)), y_shared=(y_shared, (T, H)), y=(y, (T, H)))
    _check(_lib.moe_combine(T, H, K, _ptr(y_rows, BF16, "y_rows"), _ptr(row_of, I32, "row_of"),
                            _ptr(topk_w, F32, "topk_w"), _ptr(y_shared, BF16, "y_shared"),
                            _ptr(y, BF16, "y"), _stream()))
    return y


def moe_combine_bwd(dy, y_rows, row_of, topk_w, dy_rows=None, dg=None):
    T, K = row_of.shape
    H = dy.shape[1]
    dev = dy.device
    if dy_rows is None:
        dy_rows = torch.empty(y_rows.shape, dtype=BF16, device=dev)
    dg = torch.empty((T, K), dtype=F32, device=dev) if dg is None else dg
    _expect(dy=(dy, (T, H)), y_rows=(y_rows, (y_rows.shape[0], H)), topk_w=(topk_w, (T, K)),
            dy_rows=(dy_rows, tuple(y_rows.shape)), dg=(dg, (T, K)))
    _check(_lib.moe_combine_bwd(T, H, K, _ptr(dy, BF16, "dy"), _ptr(y_rows, BF16, "y_rows"),
                                _ptr(row_of, I32, "row_of"), _ptr(topk_w, F32, "topk_w"),
                                _ptr(dy_rows, BF16, "dy_rows"), _ptr(dg, F32, "dg"), _stream()))
    return dy_rows, dg


def moe_grouped_swiglu_bwd(x_rows, w1, w2, act, h, dy_rows, offsets=None, counts=None,
                           tile_expert=None, dact=None, dx_rows=None, dw1=None, dw2=None):
    """Returns (dact, dx_rows, dw1, dw2)."""
    M, H = x_rows.shape
    G, twoF, _ = w1.shape
    F = twoF // 2
    dev = x_rows.device
    dact = torch.empty((M, 2 * F), dtype=BF16, device=dev) if dact is None else dact
    dx_rows = torch.empty((M, H), dtype=BF16, device=dev) if dx_rows is None else dx_rows
    dw1 = torch.empty(w1.shape, dtype=BF16, device=dev) if dw1 is None else dw1
    dw2 = torch.empty(w2.shape, dtype=BF16, device=dev) if dw2 is None else dw2
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(w1=(w1, (G, 2 * F, H)), w2=(w2, (G, H, F)), act=(act, (M, 2 * F)), h=(h, (M, F)),
            dy_rows=(dy_rows, (M, H)), dact=(dact, (M, 2 * F)), dx_rows=(dx_rows, (M, H)),
            dw1=(dw1, (G, 2 * F, H)), dw2=(dw2, (G, H, F)))
    _check(_lib.moe_grouped_swiglu_bwd(G, M, H, F, _ptr(offsets, I32), _ptr(counts, I32),
                                       _ptr(tile_expert, I32), _ptr(x_rows, BF16, "x_rows"),
                                       _ptr(w1, BF16, "w1"), _ptr(w2, BF16, "w2"),
                                       _ptr(act, BF16, "act"), _ptr(h, BF16, "h"),
                                       _ptr(dy_rows, BF16, "dy_rows"), _ptr(dact, BF16, "dact"),
                                       _ptr(dx_rows, BF16, "dx_rows"), _ptr(dw1, BF16, "dw1"),
                                       _ptr(dw2, BF16, "dw2"), _stream()))
    return dact, dx_rows, dw1, dw2


def _seg(offsets, counts, tile_expert):
    return _ptr(offsets, I32), _ptr(counts, I32), _ptr(tile_expert, I32)


def moe_grouped_down_dgrad(w2, act, dy_rows, offsets=None, counts=None, tile_expert=None,
                           dact=None):
    """dact = SwiGLU-backward(dy_rows . w2[g], act).  Returns dact."""
    M, H = dy_rows.shape
    G, _, F = w2.shape
    dact = torch.empty((M, 2 * F), dtype=BF16, device=dy_rows.device) if dact is None else dact
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(w2=(w2, (G, H, F)), act=(act, (M, 2 * F)), dact=(dact, (M, 2 * F)))
    _check(_lib.moe_grouped_down_dgrad(G, M, H, F, *_seg(offsets, counts, tile_expert),
                                       _ptr(w2, BF16, "w2"), _ptr(act, BF16, "act"),
                                       _ptr(dy_rows, BF16, "dy_rows"), _ptr(dact, BF16, "dact"),
                                       _stream()))
    return dact


def moe_grouped_down_wgrad(dy_rows, h, G, offsets=None, counts=None, tile_expert=None, dw2=None):
    """dw2[g] = dy_rows_g^T . h_g.  Returns dw2 [G,H,F]."""
    M, H = dy_rows.shape
    F = h.shape[1]
    dw2 = torch.empty((G, H, F), dtype=BF16, device=h.device) if dw2 is None else dw2
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(h=(h, (M, F)), dw2=(dw2, (G, H, F)))
    _check(_lib.moe_grouped_down_wgrad(G, M, H, F, *_seg(offsets, counts, tile_expert),
                                       _ptr(dy_rows, BF16, "dy_rows"), _ptr(h, BF16, "h"),
                                       _ptr(dw2, BF16, "dw2"), _stream()))
    return dw2


def moe_grouped_gate_up_dgrad(w1, dact, offsets=None, counts=None, tile_expert=None, dx_rows=None):
    """dx_rows = dact . w1[g].  Returns dx_rows."""
    M, twoF = dact.shape
    G, _, H = w1.shape
    dx_rows = torch.empty((M, H), dtype=BF16, device=dact.device) if dx_rows is None else dx_rows
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(w1=(w1, (G, twoF, H)), dx_rows=(dx_rows, (M, H)))
    _check(_lib.moe_grouped_gate_up_dgrad(G, M, H, twoF // 2, *_seg(offsets, counts, tile_expert),
                                          _ptr(w1, BF16, "w1"), _ptr(dact, BF16, "dact"),
                                          _ptr(dx_rows, BF16, "dx_rows"), _stream()))
    return dx_rows


def moe_grouped_gate_up_wgrad(dact, x_rows, G, offsets=None, counts=None, tile_expert=None,
                              dw1=None):
    """dw1[g] = dact_g^T . x_rows_g.  Returns dw1 [G,2F,H]."""
    M, twoF = dact.shape
    H = x_rows.shape[1]
    dw1 = torch.empty((G, twoF, H), dtype=BF16, device=dact.device) if dw1 is None else dw1
    _seg_shapes(G, M, offsets, counts, tile_expert)
    _expect(x_rows=(x_rows, (M, H)), dw1=(dw1, (G, twoF, H)))
    _check(_lib.moe_grouped_gate_up_wgrad(G, M, H, twoF // 2, *_seg(offsets, counts, tile_expert),
                                          _ptr(dact, BF16, "dact"), _ptr(x_rows, BF16, "x_rows"),
                                          _ptr(dw1, BF16, "dw1"), _stream()))
    return dw1


def moe_route_bwd(x, w_router, topk_idx, topk_s, dg, row_of, offsets, counts, src_token,
                  dw_router=None, dx_router=None, ws=None):
    """Router gradients of the combine path (x [T,H] bf16 and moe_permute's
    row_of, offsets, counts and src_token).  Returns (dw_router [H,E] fp32,
    dx_router [T,H] fp32)."""
    T, K = topk_idx.shape
    H, E = w_router.shape
    dev = w_router.device
    dw_router = torch.empty((H, E), dtype=F32, device=dev) if dw_router is None else dw_router
    dx_router = torch.empty((T, H), dtype=F32, device=dev) if dx_router is None else dx_router
    nbytes = moe_route_bwd_workspace_bytes(T, H, E, K)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if ws is None else ws
    _expect(x=(x, (T, H)), topk_s=(topk_s, (T, K)), dg=(dg, (T, K)), row_of=(row_of, (T, K)),
            offsets=(offsets, (E + 1,)), counts=(counts, (E,)),
            src_token=(src_token, (src_token.shape[0],) if src_token is not None else ()),
            dw_router=(dw_router, (H, E)), dx_router=(dx_router, (T, H)))
    if src_token is not None and src_token.shape[0] < moe_capacity_rows(T, E, K):
        raise ValueError("src_token must hold at least moe_capacity_rows(T, E, K) entries")
    _check(_lib.moe_route_bwd(T, H, E, K, _ptr(x, BF16, "x"),
                              _ptr(w_router, F32, "w_router"), _ptr(topk_idx, I32, "topk_idx"),
                              _ptr(topk_s, F32, "topk_s"), _ptr(dg, F32, "dg"),
                              _ptr(row_of, I32, "row_of"), _ptr(offsets, I32, "offsets"),
                              _ptr(counts, I32, "counts"), _ptr(src_token, I32, "src_token"),
                              _ptr(dw_router, F32, "dw_router"), _ptr(dx_router, F32, "dx_router"),
                              _ptr(ws), ws.numel(), _stream()))
    return dw_router, dx_router


def moe_permute_bwd(dx_rows, row_of, dx_shared=None, dx_router=None, dx=None):
    T, K = row_of.shape
    H = dx_rows.shape[1]
    dx = torch.empty((T, H), dtype=BF16, device=dx_rows.device) if dx is None else dx
    _expect(dx_shared=(dx_shared, (T, H)), dx_router=(dx_router, (T, H)), dx=(dx, (T, H)))
    _check(_lib.moe_permute_bwd(T, H, K, _ptr(dx_rows, BF16, "dx_rows"), _ptr(row_of, I32, "row_of"),
                                _ptr(dx_shared, BF16, "dx_shared"), _ptr(dx_router, F32, "dx_router"),
                                _ptr(dx, BF16, "dx"), _stream()))
    return dx


def moe_route_permute_bwd(x, w_router, topk_idx, topk_s, dg, row_of, offsets, counts, src_token,
                          dx_rows, dx_shared=None, dw_router=None, dx=None, ws=None):
    """moe_route_bwd then moe_permute_bwd in one call, the router's input
    gradient added where dx is summed.  Returns (dw_router [H,E] fp32,
    dx [T,H] bf16), bit-identical to the two calls."""
    T, K = topk_idx.shape
    H, E = w_router.shape
    dev = w_router.device
    dw_router = torch.empty((H, E), dtype=F32, device=dev) if dw_router is None else dw_router
    dx = torch.empty((T, H), dtype=BF16, device=dev) if dx is None else dx
    nbytes = moe_route_bwd_workspace_bytes(T, H, E, K)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if ws is None else ws
    _expect(x=(x, (T, H)), topk_s=(topk_s, (T, K)), dg=(dg, (T, K)), row_of=(row_of, (T, K)),
            offsets=(offsets, (E + 1,)), counts=(counts, (E,)),
            src_token=(src_token, (src_token.shape[0],) if src_token is not None else ()),
            dx_rows=(dx_rows, (dx_rows.shape[0], H) if dx_rows is not None else ()),
            dx_shared=(dx_shared, (T, H)), dw_router=(dw_router, (H, E)), dx=(dx, (T, H)))
    if src_token is not None and src_token.shape[0] < moe_capacity_rows(T, E, K):
        raise ValueError("src_token must hold at least moe_capacity_rows(T, E, K) entries")
    if dx_rows is not None and dx_rows.shape[0] < moe_capacity_rows(T, E, K):
        raise ValueError("dx_rows must hold at least moe_capacity_rows(T, E, K) rows")
    _check(_lib.moe_route_permute_bwd(T, H, E, K, _ptr(x, BF16, "x"),
                                      _ptr(w_router, F32, "w_router"), _ptr(topk_idx, I32, "topk_idx"),
                                      _ptr(topk_s, F32, "topk_s"), _ptr(dg, F32, "dg"),
                                      _ptr(row_of, I32, "row_of"), _ptr(offsets, I32, "offsets"),
                                      _ptr(counts, I32, "counts"), _ptr(src_token, I32, "src_token"),
                                      _ptr(dx_rows, BF16, "dx_rows"),
                                      _ptr(dx_shared, BF16, "dx_shared"),
                                      _ptr(dw_router, F32, "dw_router"), _ptr(dx, BF16, "dx"),
                                      _ptr(ws), ws.numel(), _stream()))
    return dw_router, dx


def moe_bias_update(counts, bias, gamma):
    """Updates bias (fp32 [E], in place) from the per-expert counts; returns bias."""
    E = bias.shape[0]
    _expect(counts=(counts, (E,)), bias=(bias, (E,)))
    _check(_lib.moe_bias_update(E, _ptr(counts, I32, "counts"), _ptr(bias, F32, "bias"),
                                float(gamma), _stream()))
    return bias


def moe_seq_balance_fwd(scores, topk_idx, seq_len, alpha, loss=None, seq_f=None, ws=None):
    """Returns (loss [1] fp32, seq_f [T/seq_len, E] fp32)."""
    T, E = scores.shape
    K = topk_idx.shape[1]
    dev = scores.device
    loss = torch.empty(1, dtype=F32, device=dev) if loss is None else loss
    B = T // seq_len if seq_len > 0 else 0
    seq_f = torch.empty((max(B, 1), E), dtype=F32, device=dev) if seq_f is None else seq_f
    if ws is None:
        ws = torch.empty(max(moe_seq_balance_workspace_bytes(T, E, seq_len), 1), dtype=torch.uint8,
                         device=dev)
    _expect(topk_idx=(topk_idx, (T, K)), loss=(loss, (1,)), seq_f=(seq_f, (max(B, 1), E)))
    _check(_lib.moe_seq_balance_fwd(T, E, K, seq_len, _ptr(scores, F32, "scores"),
                                    _ptr(topk_idx, I32, "topk_idx"), float(alpha),
                                    _ptr(loss, F32, "loss"), _ptr(seq_f, F32, "seq_f"), _ptr(ws),
                                    ws.numel(), _stream()))
    return loss, seq_f


def moe_seq_balance_bwd(scores, seq_f, K, seq_len, alpha, dloss=None, dlogit=None):
    """Returns dlogit [T,E] fp32 (dloss: fp32 [1] device tensor or None for 1)."""
    T, E = scores.shape
    dlogit = torch.empty((T, E), dtype=F32, device=scores.device) if dlogit is None else dlogit
    B = T // seq_len if seq_len > 0 else 0
    _expect(seq_f=(seq_f, (max(B, 1), E)), dloss=(dloss, (1,)), dlogit=(dlogit, (T, E)))
    _check(_lib.moe_seq_balance_bwd(T, E, K, seq_len, _ptr(scores, F32, "scores"),
                                    _ptr(seq_f, F32, "seq_f"), float(alpha),
                                    _ptr(dloss, F32, "dloss"), _ptr(dlogit, F32, "dlogit"),
                                    _stream()))
    return dlogit


def moe_route_dlogit(topk_idx, topk_s, dg, dlogit):
    """Adds the combine path's logit gradient (K entries per token) into the
    dense fp32 dlogit [T,E], in place; returns dlogit."""
    T, K = topk_idx.shape
    E = dlogit.shape[1]
    _expect(topk_s=(topk_s, (T, K)), dg=(dg, (T, K)), dlogit=(dlogit, (T, E)))
    _check(_lib.moe_route_dlogit(T, E, K, _ptr(topk_idx, I32, "topk_idx"),
                                 _ptr(topk_s, F32, "topk_s"), _ptr(dg, F32, "dg"),
                                 _ptr(dlogit, F32, "dlogit"), _stream()))
    return dlogit


def moe_route_bwd_dense(x, w_router, dlogit, dw_router=None, dx_router=None, ws=None,
                        accumulate=True):
    """Router gradients of a dense dlogit [T,E]: added into dw_router [H,E] and
    dx_router [T,H] (fp32, in place) when accumulate, else written (then they
    may be None and are allocated)."""
    T, H = x.shape
    E = w_router.shape[1]
    if dw_router is None or dx_router is None:
        if accumulate:
            raise ValueError("accumulating needs dw_router and dx_router")
        dw_router = torch.empty((H, E), dtype=F32, device=x.device) if dw_router is None else dw_router
        dx_router = torch.empty((T, H), dtype=F32, device=x.device) if dx_router is None else dx_router
    if ws is None:
        ws = torch.empty(max(moe_route_bwd_dense_workspace_bytes(T, H, E), 1), dtype=torch.uint8,
                         device=x.device)
    _expect(w_router=(w_router, (H, E)), dlogit=(dlogit, (T, E)), dw_router=(dw_router, (H, E)),
            dx_router=(dx_router, (T, H)))
    _check(_lib.moe_route_bwd_dense(T, H, E, _ptr(x, BF16, "x"), _ptr(w_router, F32, "w_router"),
                                    _ptr(dlogit, F32, "dlogit"), _ptr(dw_router, F32, "dw_router"),
                                    _ptr(dx_router, F32, "dx_router"), 1 if accumulate else 0,
                                    _ptr(ws), ws.numel(), _stream()))
    return dw_router, dx_router


# ---------------------------------------------------------------------------
# the whole layer, composed from the entry points above
# ---------------------------------------------------------------------------
def fuse_shared(w1_sh, w2_sh):
    """[S,2F,H] / [S,H,F] shared experts -> one expert of width S*F:
    w1 = the S gate blocks, then the S up blocks ([1,2SF,H]); w2 = the S down
    matrices side by side ([1,H,SF])."""
    S, twoF, H = w1_sh.shape
    F = twoF // 2
    w1f = torch.cat([w1_sh[:, :F].reshape(S * F, H), w1_sh[:, F:].reshape(S * F, H)], 0)
    w2f = torch.cat([w2_sh[s] for s in range(S)], 1)
    return w1f.unsqueeze(0).contiguous(), w2f.unsqueeze(0).contiguous()


def layer_forward(x, w_router, bias, w1, w2, w1_shf, w2_shf, K, save_for_backward=True,
                  balance=None):
    """Forward of the MoE layer.  w1_shf / w2_shf are the fused shared weights
    (fuse_shared), or None for no shared experts.  balance = (alpha, seq_len)
    adds the sequence-wise balance loss (ctx["balance_loss"]).  Returns (y, ctx)."""
    E = w1.shape[0]
    T = x.shape[0]
    scores = None if balance is None else torch.empty((T, E), dtype=F32, device=x.device)
    topk_idx, topk_w, topk_s = moe_route(x, w_router, bias, K, scores=scores)
    p = moe_permute(topk_idx, x, E)
    act, h, y_rows = moe_grouped_swiglu_fwd(p["x_rows"], w1, w2, p["offsets"], p["counts"],
                                            p["tile_expert"], act=save_for_backward)
    y_sh = act_sh = h_sh = None
    if w1_shf is not None:
        # the dense product over all tokens: split over k at small batches
        act_sh, h_sh = moe_dense_gate_up_fwd_split(x, w1_shf, act=save_for_backward)
        y_sh = moe_dense_down_fwd_split(h_sh, w2_shf)
    y = moe_combine(y_rows, p["row_of"], topk_w, y_sh)
    ctx = dict(x=x, w_router=w_router, w1=w1, w2=w2, w1_shf=w1_shf, w2_shf=w2_shf,
               topk_idx=topk_idx, topk_w=topk_w, topk_s=topk_s, perm=p, act=act, h=h,
               y_rows=y_rows, y_sh=y_sh, act_sh=act_sh, h_sh=h_sh, balance=balance)
    if balance is not None:
        alpha, seq_len = balance
        ctx["scores"] = scores
        ctx["balance_loss"], ctx["seq_f"] = moe_seq_balance_fwd(scores, topk_idx, seq_len, alpha)
    return y, ctx


def layer_backward(dy, ctx, dloss=None, router_input_grad=False):
    """Backward of the MoE layer (dloss: upstream gradient of the balance
    loss, fp32 [1] device tensor, None = 1).  Returns dict(dx, dw1, dw2,
    dw1_sh, dw2_sh, dw_router) plus the intermediates.  Without the balance
    loss the router's input gradient is added inside the un-permute
    (moe_route_permute_bwd) and the intermediate dx_router is None, unless
    router_input_grad asks for it (moe_route_bwd, then moe_permute_bwd; the
    same dx and dw_router bit for bit)."""
    p = ctx["perm"]
    dy_rows, dg = moe_combine_bwd(dy, ctx["y_rows"], p["row_of"], ctx["topk_w"])
    dact, dx_rows, dw1, dw2 = moe_grouped_swiglu_bwd(p["x_rows"], ctx["w1"], ctx["w2"], ctx["act"],
                                                     ctx["h"], dy_rows, p["offsets"], p["counts"],
                                                     p["tile_expert"])
    dx_sh = dw1_sh = dw2_sh = None
    if ctx["w1_shf"] is not None:
        _, dx_sh, dw1_sh, dw2_sh = moe_grouped_swiglu_bwd(ctx["x"], ctx["w1_shf"], ctx["w2_shf"],
                                                          ctx["act_sh"], ctx["h_sh"], dy)
    dlogit_bal = dlogit = None
    if ctx.get("balance") is None and not router_input_grad:
        dw_router, dx = moe_route_permute_bwd(ctx["x"], ctx["w_router"], ctx["topk_idx"],
                                              ctx["topk_s"], dg, p["row_of"], p["offsets"],
                                              p["counts"], p["src_token"], dx_rows, dx_sh)
        return dict(dx=dx, dw1=dw1, dw2=dw2, dw1_sh=dw1_sh, dw2_sh=dw2_sh, dw_router=dw_router,
                    dg=dg, dy_rows=dy_rows, dact=dact, dx_rows=dx_rows, dx_shared=dx_sh,
                    dx_router=None, dlogit_balance=None, dlogit=None)
    if ctx.get("balance") is None:
        dw_router, dx_router = moe_route_bwd(ctx["x"], ctx["w_router"], ctx["topk_idx"],
                                             ctx["topk_s"], dg, p["row_of"], p["offsets"],
                                             p["counts"], p["src_token"])
    else:
        # the balance loss's logit gradient is dense; the combine path's is
        # added into (a copy of) it, and one dense router backward gives the
        # router gradients of both
        alpha, seq_len = ctx["balance"]
        dlogit_bal = moe_seq_balance_bwd(ctx["scores"], ctx["seq_f"], ctx["topk_idx"].shape[1],
                                         seq_len, alpha, dloss)
        dlogit = moe_route_dlogit(ctx["topk_idx"], ctx["topk_s"], dg, dlogit_bal.clone())
        dw_router, dx_router = moe_route_bwd_dense(ctx["x"], ctx["w_router"], dlogit,
                                                   accumulate=False)
    dx = moe_permute_bwd(dx_rows, p["row_of"], dx_sh, dx_router)
    return dict(dx=dx, dw1=dw1, dw2=dw2, dw1_sh=dw1_sh, dw2_sh=dw2_sh, dw_router=dw_router,
                dg=dg, dy_rows=dy_rows, dact=dact, dx_rows=dx_rows, dx_shared=dx_sh,
                dx_router=dx_router, dlogit_balance=dlogit_bal, dlogit=dlogit)
