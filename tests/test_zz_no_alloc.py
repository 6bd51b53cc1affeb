"""moe_permute_noalloc (the permutation for callers that cannot allocate: its
workspace is the library's static device array) against moe_permute, through
the C ABI: two calls in a row on the same GPU, the second with fewer tokens,
each bit-identical to moe_permute on the same inputs, with valid routing and
with rejected tokens (data-check block written to the caller's status)."""
import numpy as np
import pytest

import parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fine_grained_moe_amd import moe
    return moe


def _outputs(M, T, E, K, H):
    m_cap = M.moe_capacity_rows(T, E, K)
    A = M.moe_align()
    i32 = torch.int32
    return dict(counts=torch.full((E,), -7, dtype=i32, device=DEV),
                offsets=torch.full((E + 1,), -7, dtype=i32, device=DEV),
                row_of=torch.full((T, K), -7, dtype=i32, device=DEV),
                src_token=torch.full((m_cap,), -7, dtype=i32, device=DEV),
                tile_expert=torch.full((m_cap // A,), -7, dtype=i32, device=DEV),
                x_rows=torch.zeros((m_cap, H), dtype=torch.bfloat16, device=DEV))


def _case(M, T, E, K, H, seed, bad=()):
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    for t in bad:
        idx[t, 0] = E            # an id outside [0,E): the token is rejected
    idx_g = torch.from_numpy(idx).to(DEV)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    print(f"case: T {T} E {E} K {K} H {H} rejected {len(bad)}", flush=True)
    ref = M.moe_permute(idx_g, x, E)
    ref_status = ref["status"].clone()
    got = M.moe_permute_noalloc(idx_g, x, E, _outputs(M, T, E, K, H),
                                status=torch.full((4,), -9, dtype=torch.int32, device=DEV))
    status = torch.full((4,), -9, dtype=torch.int32, device=DEV)
    got = M.moe_permute_noalloc(idx_g, x, E, _outputs(M, T, E, K, H), status=status)
    torch.cuda.synchronize()
    for k in ("counts", "offsets", "row_of", "src_token", "tile_expert"):
        assert torch.equal(got[k], ref[k]), k
    rows = ref["src_token"] >= 0
    assert torch.equal(got["x_rows"][rows], ref["x_rows"][rows])
    assert torch.equal(status, ref_status)
    assert P.to_np(status)[1] == len(bad)
    if bad:
        with pytest.raises(M.MoEError, match="outside"):
            M.moe_permute_check(status)
    else:
        M.moe_permute_check(status)


def test_noalloc_permute_matches_workspace_permute(M):
    """Dots shapes at 8192 tokens, then a smaller ragged batch on the same
    static array (its earlier contents must not leak into the result), then
    rejected tokens, then one token."""
    assert M.moe_permute_noalloc_max_tokens() == 131072
    _case(M, 8192, 128, 6, 5120, seed=1)
    _case(M, 777, 48, 3, 192, seed=2)
    _case(M, 1000, 16, 4, 256, seed=3, bad=(3, 998))
    _case(M, 1, 8, 2, 64, seed=4)


def test_noalloc_permute_rejects_beyond_its_scratch(M):
    T, E, K, H = M.moe_permute_noalloc_max_tokens() + 1, 8, 2, 64
    idx = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoEError, match="static scratch"):
        M.moe_permute_noalloc(idx, x, E, _outputs(M, T, E, K, H))
