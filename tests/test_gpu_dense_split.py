"""The dense forward halves with the contraction split over workgroups (the
fused shared experts at small batches) against the oracle and against the
unsplit dense call (needs an MI355X)."""
import pytest

from fine_grained_moe_amd.synthetic import generate_shard_torch
from oracle import moe_oracle as O
import parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fine_grained_moe_amd import moe
    return moe


# rows, H, fused width F, seed
CASES = {
    # a decode-sized batch at the fused shared width (2 x 1408): both halves split
    "decode": (256, 5120, 2816, 41),
    # ragged rows, slices of unequal length, a half-filled last k-stage (F = 800)
    "ragged": (200, 1344, 800, 42),
    # enough tiles to fill the GPU: no split, the dense call itself
    "nosplit": (2048, 5120, 2816, 43),
}


@pytest.fixture(autouse=True)
def _report():
    P.REPORT.clear()
    yield
    P.print_report()


@pytest.mark.parametrize("name", sorted(CASES))
def test_dense_split_forward(M, name):
    m, H, F, seed = CASES[name]
    print(f"case {name}: rows {m}, H {H}, F {F}", flush=True)
    g = generate_shard_torch("cuda", 1, m, H, F, seed)
    x, w1, w2 = g["x_rows"], g["w1"], g["w2"]
    nbytes = M.moe_dense_fwd_split_workspace_bytes(m, H, F)
    assert (nbytes > 0) == (name != "nosplit")
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    act, h = M.moe_dense_gate_up_fwd_split(x, w1, ws=ws)
    y = M.moe_dense_down_fwd_split(h, w2, ws=ws)
    # again on the same workspace, and without act (inference): the same bits
    act2, h2 = M.moe_dense_gate_up_fwd_split(x, w1, ws=ws)
    y2 = M.moe_dense_down_fwd_split(h2, w2, ws=ws)
    none, h3 = M.moe_dense_gate_up_fwd_split(x, w1, act=False, ws=ws)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(act, act2) and torch.equal(h, h2) and torch.equal(y, y2)
    assert torch.equal(h, h3)

    a_ref, h_ref, y_ref = O.expert_ffn(P.to_np(x), P.to_np(w1[0]), P.to_np(w2[0]))
    P.assert_close(f"{name} act", P.to_np(act), a_ref)
    P.assert_close(f"{name} h", P.to_np(h), h_ref)
    P.assert_close(f"{name} y", P.to_np(y), y_ref)

    # the unsplit dense call: the same up to the order of the fp32 sums (at
    # most one bf16 rounding step apart); bit-identical when nothing is split
    act_d, h_d = M.moe_grouped_gate_up_fwd(x, w1)
    y_d = M.moe_grouped_down_fwd(h, w2)
    torch.cuda.synchronize()
    if name == "nosplit":
        assert torch.equal(act, act_d) and torch.equal(h, h_d) and torch.equal(y, y_d)
    else:
        for n, a, b in (("act", act, act_d), ("h", h, h_d), ("y", y, y_d)):
            P.assert_close(f"{name} {n} vs unsplit", P.to_np(a), P.to_np(b), tol=8e-3, norm_tol=1e-3)
