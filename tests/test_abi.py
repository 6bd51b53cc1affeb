"""The C-ABI library without a GPU: it loads, exports every declared symbol,
answers the host queries, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fine_grained_moe_amd", "libmoe.so")
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return ctypes.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"


def test_binding_covers_every_symbol():
    import importlib.util
    spec = importlib.util.spec_from_file_location("moe_binding", os.path.join(ROOT, "fine_grained_moe_amd", "moe.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert sorted(mod.EXPORTED) == declared_functions()
    for n in declared_functions():
        if n not in ("moe_status_string", "moe_last_error"):
            assert callable(getattr(mod, n)), n


def test_host_queries(lib):
    lib.moe_capacity_rows.restype = ctypes.c_int64
    lib.moe_permute_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_route_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_route_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_status_string.restype = ctypes.c_char_p
    assert lib.moe_align() == 128
    # ceil((T*K + E*127)/128)*128
    assert lib.moe_capacity_rows(8192, 128, 6) == 65408
    assert lib.moe_capacity_rows(256, 128, 6) == 17792
    assert lib.moe_capacity_rows(0, 8, 2) == 1024
    assert lib.moe_capacity_rows(-1, 8, 2) == -1
    # weight parts (3 x 32*ceil(E/32) x H bf16) + S slices x T x 128 fp32 logits,
    # S doubled while the grid of ceil(T/128) x S workgroups stays below 256 and
    # H splits into whole 32-deep stages
    parts = 3 * 128 * 5120 * 2
    assert lib.moe_route_workspace_bytes(8192, 5120, 128) == parts + 4 * 8192 * 128 * 4
    assert lib.moe_route_workspace_bytes(16384, 5120, 128) == parts + 2 * 16384 * 128 * 4
    assert lib.moe_route_workspace_bytes(256, 5120, 128) == parts + 32 * 256 * 128 * 4
    assert lib.moe_route_workspace_bytes(0, 5120, 128) == parts
    assert lib.moe_route_workspace_bytes(128, 64, 8) == 3 * 32 * 64 * 2 + 2 * 128 * 128 * 4
    assert lib.moe_route_workspace_bytes(128, 64, 0) == 0
    assert lib.moe_route_workspace_bytes(128, 96, 8) == 0
    assert lib.moe_route_workspace_bytes(-1, 64, 8) == 0
    # 256-byte data-check block, per-chunk status (3 int32 per 256-token
    # chunk, rounded up to 256 bytes), per-chunk histograms and bases
    assert lib.moe_permute_workspace_bytes(8192, 128, 6) == 256 + 512 + 2 * 32 * 128 * 4
    assert lib.moe_permute_workspace_bytes(0, 128, 6) == 256
    assert lib.moe_route_bwd_workspace_bytes(8192, 5120, 128, 6) == 128 * 5120 * 4 + 65408 * 4
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(3) == b"workspace too small"


def _p(v):
    return ctypes.c_void_p(v)


FAKE = 0x1000  # never dereferenced: every call below is rejected on the host


def test_route_rejects(lib):
    f = lib.moe_route
    # x, w_router, bias, topk_idx, topk_w, topk_s, scores, ws
    f.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p]
    big = 1 << 30
    ok = [_p(FAKE)] * 7 + [_p(FAKE)]
    assert f(8, 64, 8, 9, *ok, big, _p(None)) == 1          # K > E
    assert f(8, 64, 8, 0, *ok, big, _p(None)) == 1          # K = 0
    assert f(-1, 64, 8, 2, *ok, big, _p(None)) == 1         # T < 0
    assert f(8, 96, 8, 2, *ok, big, _p(None)) == 2          # H % 64
    assert f(8, 64, 200, 2, *ok, big, _p(None)) == 2        # E > 128
    assert f(8, 64, 32, 17, *ok, big, _p(None)) == 2        # K > 16
    assert f(8, 64, 8, 2, _p(None), *[_p(FAKE)] * 7, big, _p(None)) == 1  # null x
    assert f(8, 64, 8, 2, *ok, 16, _p(None)) == 3           # workspace too small
    assert f(8, 64, 8, 2, *[_p(FAKE)] * 7, _p(None), big, _p(None)) == 3  # no workspace
    assert f(0, 64, 8, 2, *[_p(None)] * 8, 0, _p(None)) == 0   # T = 0 no-op
    lib.moe_last_error.restype = ctypes.c_char_p
    f(8, 64, 8, 9, *ok, big, _p(None))
    assert b"K > E" in lib.moe_last_error()


def test_permute_rejects(lib):
    f = lib.moe_permute
    f.argtypes = ([ctypes.c_int32] * 5 + [ctypes.c_void_p] * 2 + [ctypes.c_int64] +
                  [ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p])
    T, H, E, K = 100, 64, 8, 2
    cap = 100 * 2 + 8 * 127
    cap = (cap + 127) // 128 * 128
    ptrs = [_p(FAKE)] * 2
    outs = [_p(FAKE)] * 6
    assert f(T, H, E, K, 64, *ptrs, cap, *outs, _p(FAKE), 1 << 20, _p(None)) == 2    # align
    assert f(T, H, E, K, 128, *ptrs, cap - 128, *outs, _p(FAKE), 1 << 20, _p(None)) == 1  # m_cap
    assert f(T, H, E, K, 128, *ptrs, cap + 1, *outs, _p(FAKE), 1 << 20, _p(None)) == 1   # not multiple
    assert f(T, H, E, K, 128, *ptrs, cap, *outs, _p(FAKE), 4, _p(None)) == 3          # workspace
    assert f(T, H, E, K, 128, _p(None), _p(FAKE), cap, *outs, _p(FAKE), 1 << 20, _p(None)) == 1


def test_grouped_rejects(lib):
    f = lib.moe_grouped_swiglu_fwd
    f.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 10
    w = [_p(FAKE)] * 7
    assert f(4, 256, 64, 48, _p(FAKE), _p(FAKE), _p(FAKE), *w) == 2     # F % 32
    assert f(4, 256, 100, 32, _p(FAKE), _p(FAKE), _p(FAKE), *w) == 2    # H % 64
    assert f(4, 200, 64, 32, _p(FAKE), _p(FAKE), _p(FAKE), *w) == 1     # grouped rows % 128
    assert f(2, 200, 64, 32, _p(None), _p(None), _p(None), *w) == 1     # dense with G != 1
    assert f(1, 200, 64, 32, _p(FAKE), _p(None), _p(None), *w) == 1     # partial segment args
    assert f(1, 0, 64, 32, _p(None), _p(None), _p(None), *w) == 0       # empty
    g = lib.moe_grouped_swiglu_bwd
    g.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 14
    assert g(1, 128, 64, 32, _p(None), _p(None), _p(None), *[_p(FAKE)] * 9, _p(None), _p(None)) == 1


def test_row_kernels_reject(lib):
    for name, nptr in (("moe_combine", 6), ("moe_combine_bwd", 7), ("moe_permute_bwd", 6)):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * nptr
        assert f(4, 64, 0, *[_p(FAKE)] * nptr) == 1
        assert f(4, 60, 2, *[_p(FAKE)] * nptr) == 2
        assert f(0, 64, 2, *[_p(None)] * nptr) == 0
        assert f(4, 64, 2, *[_p(None)] * nptr) == 1


def test_route_bwd_rejects(lib):
    f = lib.moe_route_bwd
    # x, w_router, topk_idx, topk_s, dg, row_of, offsets, counts, src_token, dw_router, dx_router, ws
    f.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 12 + [ctypes.c_size_t, ctypes.c_void_p]
    assert f(16, 64, 8, 2, *[_p(FAKE)] * 12, 16, _p(None)) == 3
    assert f(16, 64, 8, 2, _p(None), *[_p(FAKE)] * 11, 1 << 30, _p(None)) == 1
    assert f(16, 64, 8, 2, *[_p(FAKE)] * 8, _p(None), *[_p(FAKE)] * 3, 1 << 30, _p(None)) == 1  # src_token


def test_route_permute_bwd_rejects(lib):
    f = lib.moe_route_permute_bwd
    # x, w_router, topk_idx, topk_s, dg, row_of, offsets, counts, src_token, dx_rows,
    # dx_shared, dw_router, dx, ws, ws_bytes, stream
    f.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 14 + [ctypes.c_size_t, ctypes.c_void_p]
    big = 1 << 30
    assert f(16, 64, 8, 2, *[_p(FAKE)] * 14, 16, _p(None)) == 3                  # workspace
    assert f(16, 64, 8, 2, _p(None), *[_p(FAKE)] * 13, big, _p(None)) == 1        # null x
    assert f(16, 64, 8, 2, *[_p(FAKE)] * 9, _p(None), *[_p(FAKE)] * 4, big, _p(None)) == 1  # dx_rows
    assert f(16, 64, 8, 2, *[_p(FAKE)] * 12, _p(None), _p(FAKE), big, _p(None)) == 1  # null dx
    assert f(16, 60, 8, 2, *[_p(FAKE)] * 14, big, _p(None)) == 2                  # H % 64
    assert f(16, 64, 8, 9, *[_p(FAKE)] * 14, big, _p(None)) != 0                  # K > E
    assert f(16, 64, 8, 2, *[_p(FAKE + 2)] * 14, big, _p(None)) == 1              # misaligned


def test_backward_steps_reject(lib):
    # (name, number of operand pointers after the three segment pointers)
    for name, nptr in (("moe_grouped_down_dgrad", 4), ("moe_grouped_down_wgrad", 3),
                       ("moe_grouped_gate_up_dgrad", 3), ("moe_grouped_gate_up_wgrad", 3)):
        f = getattr(lib, name)
        f.argtypes = ([ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] +
                      [ctypes.c_void_p] * (3 + nptr + 1))
        seg = [_p(FAKE)] * 3
        ops = [_p(FAKE)] * nptr
        assert f(4, 256, 64, 48, *seg, *ops, _p(None)) == 2, name            # F % 32
        assert f(4, 200, 64, 32, *seg, *ops, _p(None)) == 1, name            # rows % 128
        assert f(2, 256, 64, 32, _p(None), _p(None), _p(None), *ops, _p(None)) == 1, name
        assert f(4, 256, 64, 32, *seg, _p(None), *ops[1:], _p(None)) == 1, name  # null operand


def test_balance_rejects(lib):
    f = lib.moe_bias_update
    f.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
    assert f(0, _p(FAKE), _p(FAKE), 0.1, _p(None)) == 1      # E = 0
    assert f(129, _p(FAKE), _p(FAKE), 0.1, _p(None)) == 2    # E > 128
    assert f(8, _p(None), _p(FAKE), 0.1, _p(None)) == 1      # null counts

    f = lib.moe_seq_balance_fwd
    f.argtypes = ([ctypes.c_int32] * 4 + [ctypes.c_void_p] * 2 + [ctypes.c_float] +
                  [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p])
    big = 1 << 30
    ok = [_p(FAKE)] * 2
    assert f(8, 8, 2, 3, *ok, 0.1, *[_p(FAKE)] * 3, big, _p(None)) == 1   # T % seq_len
    assert f(8, 8, 9, 4, *ok, 0.1, *[_p(FAKE)] * 3, big, _p(None)) == 1   # K > E
    assert f(8, 200, 2, 4, *ok, 0.1, *[_p(FAKE)] * 3, big, _p(None)) == 2  # E > 128
    assert f(8, 8, 2, 0, *ok, 0.1, *[_p(FAKE)] * 3, big, _p(None)) == 1   # seq_len = 0
    assert f(8, 8, 2, 4, *ok, 0.1, _p(None), _p(FAKE), _p(FAKE), big, _p(None)) == 1  # null loss
    assert f(8, 8, 2, 4, *ok, 0.1, *[_p(FAKE)] * 3, 4, _p(None)) == 3     # workspace too small

    f = lib.moe_seq_balance_bwd
    f.argtypes = ([ctypes.c_int32] * 4 + [ctypes.c_void_p] * 2 + [ctypes.c_float] +
                  [ctypes.c_void_p] * 3)
    assert f(8, 8, 2, 3, _p(FAKE), _p(FAKE), 0.1, _p(None), _p(FAKE), _p(None)) == 1  # T % seq_len
    assert f(8, 8, 2, 4, _p(FAKE), _p(FAKE), 0.1, _p(None), _p(None), _p(None)) == 1  # null dlogit

    f = lib.moe_route_bwd_dense
    # x, w_router, dlogit, dw_router, dx_router, accumulate, ws, ws_bytes, stream
    f.argtypes = ([ctypes.c_int32] * 3 + [ctypes.c_void_p] * 5 + [ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p])
    ok5 = [_p(FAKE)] * 5
    assert f(8, 96, 8, *ok5, 1, _p(FAKE), big, _p(None)) == 2      # H % 64
    assert f(8, 64, 200, *ok5, 1, _p(FAKE), big, _p(None)) == 2    # E > 128
    assert f(8, 64, 8, *ok5, 1, _p(None), big, _p(None)) == 3      # no workspace
    assert f(8, 64, 8, *ok5, 1, _p(FAKE), 4, _p(None)) == 3        # workspace too small
    assert f(0, 64, 8, *[_p(None)] * 5, 1, _p(None), 0, _p(None)) == 0   # T = 0, adding: no-op
    assert f(0, 64, 8, *[_p(None)] * 5, 0, _p(None), 0, _p(None)) == 1   # T = 0, writing: dw_router

    f = lib.moe_route_dlogit
    f.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 5
    assert f(8, 8, 9, *[_p(FAKE)] * 4, _p(None)) == 1                # K > E
    assert f(8, 200, 2, *[_p(FAKE)] * 4, _p(None)) == 2              # E > 128
    assert f(8, 8, 2, _p(FAKE), _p(FAKE), _p(FAKE), _p(None), _p(None)) == 1   # null dlogit
    assert f(8, 8, 2, _p(FAKE), _p(FAKE + 4), _p(FAKE), _p(FAKE), _p(None)) == 1  # misaligned
    assert f(0, 8, 2, *[_p(None)] * 4, _p(None)) == 0                # T = 0 no-op

    lib.moe_seq_balance_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_route_bwd_dense_workspace_bytes.restype = ctypes.c_size_t
    assert lib.moe_seq_balance_workspace_bytes(8192, 128, 4096) > 0
    assert lib.moe_seq_balance_workspace_bytes(8192, 128, 3000) == 0
    assert lib.moe_route_bwd_dense_workspace_bytes(8192, 5120, 128) > 0


def test_misaligned_pointers_rejected(lib):
    """Every device pointer must be 16-byte aligned and every workspace
    256-byte aligned; the host check rejects the call before any launch."""
    big = 1 << 30
    f = lib.moe_route
    f.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p]
    ok = [_p(FAKE)] * 7
    assert f(8, 64, 8, 2, _p(FAKE + 8), *ok[1:], _p(FAKE), big, _p(None)) == 1   # x
    assert f(8, 64, 8, 2, *ok[:6], _p(FAKE + 4), _p(FAKE), big, _p(None)) == 1   # scores
    assert f(8, 64, 8, 2, *ok, _p(FAKE + 16), big, _p(None)) == 1                # workspace
    lib.moe_last_error.restype = ctypes.c_char_p
    assert b"256-byte" in lib.moe_last_error()
    g = lib.moe_grouped_gate_up_fwd
    g.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 8
    assert g(1, 128, 64, 32, _p(None), _p(None), _p(None), _p(FAKE), _p(FAKE + 2), _p(FAKE),
             _p(FAKE), _p(None)) == 1                                              # w1
    assert b"16-byte" in lib.moe_last_error()
    c = lib.moe_combine
    c.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 6
    assert c(4, 64, 2, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE + 8), _p(FAKE), _p(None)) == 1  # y_shared
    pb = lib.moe_permute_bwd
    pb.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 6
    assert pb(4, 64, 2, _p(FAKE), _p(FAKE), _p(None), _p(FAKE + 4), _p(FAKE), _p(None)) == 1  # dx_router


def test_segments_beyond_32_bit_offsets_rejected(lib):
    """Weight gradients address a whole segment with 32-bit byte offsets: m_rows
    rows of max(H, 2F) bf16 values must stay below 4 GiB (419,430 rows at
    H = 5120); the dense router gradient bounds its token slices the same way."""
    for name in ("moe_grouped_down_wgrad", "moe_grouped_gate_up_wgrad"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 7
        seg = [_p(FAKE)] * 3
        assert f(128, 419456, 5120, 1408, *seg, _p(None), _p(None), _p(None), _p(None)) == 2
        assert f(128, 419328, 5120, 1408, *seg, _p(None), _p(None), _p(None), _p(None)) == 1  # null
    g = lib.moe_grouped_swiglu_bwd
    g.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 14
    assert g(128, 419456, 5120, 1408, *[_p(FAKE)] * 3, *[_p(None)] * 11) == 2
    d = lib.moe_route_bwd_dense
    d.argtypes = ([ctypes.c_int32] * 3 + [ctypes.c_void_p] * 5 + [ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p])
    assert d(6_000_000, 5120, 128, *[_p(None)] * 5, 1, _p(None), 0, _p(None)) == 2
    assert d(5_000_000, 5120, 128, *[_p(None)] * 5, 1, _p(None), 0, _p(None)) == 1   # null pointers


def test_binding_rejects_wrong_shapes():
    """The library sees raw pointers only; the binding refuses a buffer whose
    shape differs from what the call reads or writes (checked before any
    device pointer is taken, so this runs on the CPU)."""
    import pytest
    torch = pytest.importorskip("torch")
    from fine_grained_moe_amd import moe as M
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    T, H, K, E = 4, 64, 2, 8
    y_rows = torch.empty((1024, H), dtype=bf)
    row_of = torch.empty((T, K), dtype=i32)
    with pytest.raises(ValueError, match="topk_w"):
        M.moe_combine(y_rows, row_of, torch.empty((T, K + 1), dtype=f32))
    with pytest.raises(ValueError, match="y must have shape"):
        M.moe_combine(y_rows, row_of, torch.empty((T, K), dtype=f32), y=torch.empty((T - 1, H), dtype=bf))
    with pytest.raises(ValueError, match="dw1"):
        M.moe_grouped_gate_up_wgrad(torch.empty((256, 64), dtype=bf), torch.empty((256, H), dtype=bf), 2,
                                    dw1=torch.empty((1, 64, H), dtype=bf))
    with pytest.raises(ValueError, match="tile_expert"):
        M.moe_grouped_down_fwd(torch.empty((256, 32), dtype=bf), torch.empty((2, H, 32), dtype=bf),
                               torch.empty(3, dtype=i32), torch.empty(2, dtype=i32),
                               torch.empty(3, dtype=i32))
    with pytest.raises(ValueError, match="dlogit"):
        M.moe_route_dlogit(row_of, torch.empty((T, K), dtype=f32), torch.empty((T, K), dtype=f32),
                           torch.empty((T - 1, E), dtype=f32))


def test_dense_split_workspace_and_rejects(lib):
    """The k-split dense forward halves: a workspace only when the product's
    128 x 256 tiles fill less than half of the 256 CUs (then 256 // tiles
    slices, at most 8, at least 4 64-deep k-stages each, fp32 partial products
    of the larger half); the checks run before any launch."""
    q = lib.moe_dense_fwd_split_workspace_bytes
    q.restype = ctypes.c_size_t
    q.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]

    def rule(M, H, F):
        def ks(N, K):
            tiles = -(-M // 128) * -(-N // 256)
            if M <= 0 or tiles >= 128:
                return 1
            k = min(256 // tiles, 8, -(-K // 64) // 4)
            return k if k >= 2 else 1
        k1, k2 = ks(2 * F, H), ks(H, F)
        return max(k1 * M * 2 * F * 4 if k1 > 1 else 0, k2 * M * H * 4 if k2 > 1 else 0)

    for M, H, F in ((256, 5120, 2816), (8192, 5120, 2816), (200, 1344, 800), (1, 64, 32),
                    (128, 512, 352), (1024, 5120, 2816), (2048, 5120, 2816), (0, 5120, 2816)):
        assert q(M, H, F) == rule(M, H, F), (M, H, F)
    # gate/up: 44 tiles -> 5 slices of [256, 5632]; down: 40 tiles -> 6 slices of [256, 5120]
    assert q(256, 5120, 2816) == max(5 * 256 * 5632 * 4, 6 * 256 * 5120 * 4)
    assert q(8192, 5120, 2816) == 0                      # 704 tiles: no split
    g = lib.moe_dense_gate_up_fwd_split
    g.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 5 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    need = q(256, 5120, 2816)
    assert g(256, 5120, 2816, _p(FAKE), _p(FAKE), _p(None), _p(FAKE), _p(FAKE), need - 1, _p(None)) == 3
    assert g(256, 5120, 2816, _p(FAKE), _p(FAKE), _p(None), _p(FAKE), _p(None), need, _p(None)) == 3
    assert g(256, 5120, 2816, _p(FAKE), _p(FAKE), _p(None), _p(FAKE), _p(FAKE + 16), need, _p(None)) == 1
    assert g(256, 5120, 2816, _p(None), _p(FAKE), _p(None), _p(FAKE), _p(FAKE), need, _p(None)) == 1
    assert g(256, 5100, 2816, _p(FAKE), _p(FAKE), _p(None), _p(FAKE), _p(FAKE), need, _p(None)) == 2
    assert g(0, 5120, 2816, _p(None), _p(None), _p(None), _p(None), _p(None), 0, _p(None)) == 0
    d = lib.moe_dense_down_fwd_split
    d.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 4 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    assert d(256, 5120, 2816, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), need - 1, _p(None)) == 3
    assert d(256, 5120, 2816, _p(FAKE), _p(FAKE), _p(None), _p(FAKE), need, _p(None)) == 1
    assert d(-1, 5120, 2816, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), need, _p(None)) == 1


def test_permute_check_decoder(lib):
    """moe_permute's data-check block, decoded on the host: flags (bit 0 an id
    outside [0,E), bit 1 an id repeated within a token), rejected tokens,
    first rejected token, marker."""
    f = lib.moe_permute_check
    f.argtypes = [ctypes.c_void_p]
    lib.moe_last_error.restype = ctypes.c_char_p
    MAGIC = 0x4D4F4550

    def call(words):
        arr = (ctypes.c_int32 * 4)(*words)
        return f(ctypes.cast(arr, ctypes.c_void_p)), lib.moe_last_error().decode()

    assert call([0, 0, -1, MAGIC])[0] == 0
    st, msg = call([1, 3, 17, MAGIC])
    assert st == 1 and "3 token(s)" in msg and "token 17" in msg and "outside [0,E)" in msg
    assert "repeated" not in msg
    st, msg = call([2, 1, 0, MAGIC])
    assert st == 1 and "repeated within a token" in msg and "outside" not in msg
    st, msg = call([3, 2, 5, MAGIC])
    assert st == 1 and "outside [0,E) and an expert id repeated" in msg
    # not a block moe_permute wrote, or an inconsistent one
    assert call([0, 0, -1, 0])[0] == 1 and "not a status block" in lib.moe_last_error().decode()
    for words in ([4, 1, 0, MAGIC], [1, 0, -1, MAGIC], [0, 2, 3, MAGIC], [1, 1, -1, MAGIC]):
        st, msg = call(words)
        assert st == 1 and "corrupt" in msg, words
    assert f(None) == 1


def _oob_sentinel():
    src = open(os.path.join(ROOT, "fine_grained_moe_amd", "csrc", "lds_dma.h")).read()
    return int(re.search(r"constexpr uint32_t kOOB = (0x[0-9A-Fa-f]+)u;", src).group(1), 16)


def _largest_admitted(call, lo, hi):
    """Largest n in [lo, hi) that `call(n)` admits (returns 1: the shape
    passed and the null pointers were refused) when every larger one is
    refused as an unsupported shape (2)."""
    assert call(lo) == 1 and call(hi) == 2
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if call(mid) == 1:
            lo = mid
        else:
            hi = mid
    return lo


def test_out_of_range_offset_above_every_buffer(lib):
    """The grouped GEMMs send masked rows, columns and k past a buffer to the
    offset kOOB, which must read as zeros: it must lie at or above the byte
    size (num_records) of every buffer resource the kernels build, at the
    largest shapes the host checks admit, and a 16-byte load there must not
    wrap in 32 bits.  The model below lists each resource's byte size."""
    kOOB = _oob_sentinel()
    assert kOOB + 12 < 1 << 32
    sizes = {}
    # K-grouped weight gradients: one resource per operand over a whole
    # segment of rows (dense call: m_rows rows), rows of H or 2F bf16 values
    for name in ("moe_grouped_down_wgrad", "moe_grouped_gate_up_wgrad"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 7
        for H, F in ((5120, 1408), (64, 32), (65536, 32), (128, 65536), (8192, 65536 // 64 * 32)):
            n = _largest_admitted(lambda m: f(1, m, H, F, *[_p(None)] * 7), 1, 1 << 31)
            sizes[f"{name} segment, H={H} F={F}"] = n * max(H, 2 * F) * 2
    # row-grouped products: a row tile (up to 256 rows) of the row operand, one
    # expert's weight matrix, the act tile of the SwiGLU-backward epilogue
    g = lib.moe_grouped_gate_up_fwd
    g.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 8
    Hmax = _largest_admitted(lambda h: g(1, 1, h * 64, 32, *[_p(None)] * 8), 1, 1 << 20) * 64
    Fmax = _largest_admitted(lambda fq: g(1, 1, 64, fq * 32, *[_p(None)] * 8), 1, 1 << 20) * 32
    assert Hmax == 65536 and Fmax == 65536
    FH = _largest_admitted(lambda fq: g(1, 1, 65536, fq * 32, *[_p(None)] * 8), 1, 2048) * 32 * 65536
    sizes["row tile"] = 256 * max(Hmax, 2 * Fmax) * 2
    sizes["expert weights"] = 2 * FH * 2
    sizes["act tile"] = 128 * 2 * Fmax * 2
    # router: a 128-token tile of x, the three bf16 parts of the weight
    r = lib.moe_route
    r.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p]
    Hr = _largest_admitted(lambda h: r(1, h * 64, 8, 2, *[_p(None)] * 8, 0, _p(None)), 1, 1 << 20) * 64
    sizes["router x tile"] = 128 * Hr * 2
    sizes["router weight parts"] = 3 * 128 * Hr * 2
    for k, v in sizes.items():
        assert 0 < v <= (1 << 32) - 128 <= kOOB, (k, v)
    # the dots.llm1 limit: 419,430 rows of 10 KB are admitted, one more is not
    assert sizes["moe_grouped_gate_up_wgrad segment, H=5120 F=1408"] == 419430 * 10240
