"""Load-balancing entry points (bias step, sequence-wise balance loss and its
router gradients) against the CPU oracle, through the C ABI (needs an MI355X).

Downstream stages take the GPU's own routing (scores and picks) as their
input, as in the layer tests, so a near-tie flip cannot leak into them.
"""
import numpy as np
import pytest

from fine_grained_moe_amd.synthetic import WORKLOADS, Workload, generate_numpy, generate_torch
from oracle import moe_oracle as O
import bf16_pipeline as B
import parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda"
ALIGN = 128


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fine_grained_moe_amd import moe
    return moe


@pytest.fixture(autouse=True)
def _report():
    P.REPORT.clear()
    yield
    P.print_report()


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.int32)


# ---------------------------------------------------------------------------
# bias step: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("E", [1, 8, 48, 128])
def test_bias_update_bit_exact(M, E):
    rng = np.random.default_rng(100 + E)
    for trial, gamma in enumerate((1e-3, 0.0625, 3.3e-4)):
        counts = rng.integers(0, 200, E).astype(np.int32)
        if E > 2:
            # a third of the experts exactly at the mean load of 100
            counts[: E // 3] = 100
            counts[-1] = 100 * E - counts[:-1].sum()
            if counts[-1] < 0:
                counts[-1] = 0
        if trial == 2:
            counts[:] = 7  # all at the mean: nothing moves
        bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
        ref = O.bias_update(bias, counts, gamma)
        c_g = torch.from_numpy(counts).to(DEV)
        b_g = torch.from_numpy(bias.copy()).to(DEV)
        M.moe_bias_update(c_g, b_g, gamma)
        got = P.to_np(b_g)
        assert np.array_equal(_bits(got), _bits(ref)), (E, gamma, got, ref)


def test_bias_update_from_permute_counts(M):
    """The step on the counts moe_permute produced for a dots-shaped batch."""
    w = Workload("bal", T=8192, H=64, E=128, K=6, S=0, F=32, seed=31, router_std=0.3,
                 bias_std=0.05)
    inp = generate_numpy(w)
    x = torch.from_numpy(inp["x"]).to(DEV).to(torch.bfloat16)
    wr = torch.from_numpy(inp["w_router"]).to(DEV)
    b = torch.from_numpy(inp["bias"]).to(DEV)
    idx, _, _ = M.moe_route(x, wr, b, w.K)
    perm = M.moe_permute(idx, x, w.E)
    counts = P.to_np(perm["counts"])
    assert counts.sum() == w.T * w.K
    ref = O.bias_update(inp["bias"], counts, 1e-3)
    M.moe_bias_update(perm["counts"], b, 1e-3)
    assert np.array_equal(_bits(P.to_np(b)), _bits(ref))


# ---------------------------------------------------------------------------
# all-expert scores from the router
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,E,K", [(128, 64, 8, 2), (700, 192, 48, 3), (2048, 5120, 128, 6)])
def test_route_scores(M, T, H, E, K):
    w = Workload("scores", T=T, H=H, E=E, K=K, S=0, F=32, seed=40 + E, router_std=0.02)
    inp = generate_numpy(w)
    x = torch.from_numpy(inp["x"]).to(DEV).to(torch.bfloat16)
    scores = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx, _, ts = M.moe_route(x, torch.from_numpy(inp["w_router"]).to(DEV),
                             torch.from_numpy(inp["bias"]).to(DEV), K, scores=scores)
    s = P.to_np(scores)
    # the selected scores are the same fp32 values the router reports
    sel = np.take_along_axis(s, P.to_np(idx).astype(np.int64), axis=1)
    assert np.array_equal(_bits(sel), _bits(P.to_np(ts)))
    ref = O.router_scores(O.router_logits(inp["x"], inp["w_router"]))
    assert np.abs(s.astype(np.float64) - ref).max() < 2e-6


# ---------------------------------------------------------------------------
# sequence-wise balance loss
# ---------------------------------------------------------------------------
SEQ_CASES = {
    "T128_E8_K2_L32": (128, 8, 2, 32),
    "T300_E48_K3_L100": (300, 48, 3, 100),   # chunks ragged inside a sequence
    "T1000_E16_K4_L1000": (1000, 16, 4, 1000),  # one sequence
    "T512_E128_K6_L1": (512, 128, 6, 1),     # every token its own sequence
    "T8192_E128_K6_L4096": (8192, 128, 6, 4096),
    "T8192_E128_K6_L8192_skew": (8192, 128, 6, 8192),
}


def _routed(M, T, E, K, seed, skew=False):
    w = Workload("seq", T=T, H=64, E=E, K=K, S=0, F=32, seed=seed, router_std=0.3,
                 bias_kind="zipf" if skew else "normal", bias_std=0.05)
    inp = generate_numpy(w)
    x = torch.from_numpy(inp["x"]).to(DEV).to(torch.bfloat16)
    scores = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx, _, _ = M.moe_route(x, torch.from_numpy(inp["w_router"]).to(DEV),
                            torch.from_numpy(inp["bias"]).to(DEV), K, scores=scores)
    return scores, idx


@pytest.mark.parametrize("name", sorted(SEQ_CASES))
def test_seq_balance(M, name):
    T, E, K, L = SEQ_CASES[name]
    alpha = 0.01
    scores, idx = _routed(M, T, E, K, seed=50 + T % 97, skew=name.endswith("skew"))
    loss, seq_f = M.moe_seq_balance_fwd(scores, idx, L, alpha)
    s, ix = P.to_np(scores), P.to_np(idx)
    ref_loss = O.seq_balance_loss(s, ix, L, alpha)
    got_loss = float(P.to_np(loss)[0])
    assert abs(got_loss - ref_loss) <= 2e-5 * abs(ref_loss), (got_loss, ref_loss)
    ref_f, _ = O.seq_balance_stats(s, ix, L)
    assert np.allclose(P.to_np(seq_f), ref_f, rtol=1e-6, atol=0), "f"
    # backward with an upstream gradient that is not one
    dloss = torch.tensor([0.7], dtype=torch.float32, device=DEV)
    dlogit = M.moe_seq_balance_bwd(scores, seq_f, K, L, alpha, dloss)
    ref = O.seq_balance_bwd(s, ix, L, alpha, 0.7)
    P.assert_close(f"{name} dlogit", P.to_np(dlogit), ref, tol=1e-4, norm_tol=1e-5)
    # deterministic
    loss2, _ = M.moe_seq_balance_fwd(scores, idx, L, alpha)
    assert float(P.to_np(loss2)[0]) == got_loss


# ---------------------------------------------------------------------------
# router gradients of a dense logit gradient (accumulated into the outputs)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,E", [(128, 64, 8), (200, 128, 13), (300, 192, 48),
                                   (1000, 512, 128), (8192, 5120, 128)])
def test_route_bwd_dense(M, T, H, E):
    rng = np.random.default_rng(T + H + E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x_g = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    x = P.to_np(x_g)  # the bf16 values both sides use
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    dl = (rng.standard_normal((T, E)) * 1e-3).astype(np.float32)
    # starting values of the size of the increments
    dw0 = (rng.standard_normal((H, E)) * 1e-2).astype(np.float32)
    dx0 = (rng.standard_normal((T, H)) * 1e-4).astype(np.float32)
    dw_g = torch.from_numpy(dw0).to(DEV)
    dx_g = torch.from_numpy(dx0).to(DEV)
    M.moe_route_bwd_dense(x_g, torch.from_numpy(w).to(DEV), torch.from_numpy(dl).to(DEV),
                          dw_g, dx_g)
    ref_dw, ref_dx = O.router_bwd_dense(x, w, dl)
    # the added part, recovered in fp64 (the subtraction is exact to fp32 rounding of the sum)
    P.assert_close(f"T{T} dW_r increment", P.to_np(dw_g).astype(np.float64) - dw0, ref_dw,
                   tol=1e-4, norm_tol=1e-5)
    P.assert_close(f"T{T} dx_r increment", P.to_np(dx_g).astype(np.float64) - dx0, ref_dx,
                   tol=1e-4, norm_tol=1e-5)
    # from zero: the plain products
    dw_z = torch.zeros((H, E), dtype=torch.float32, device=DEV)
    dx_z = torch.zeros((T, H), dtype=torch.float32, device=DEV)
    M.moe_route_bwd_dense(x_g, torch.from_numpy(w).to(DEV), torch.from_numpy(dl).to(DEV),
                          dw_z, dx_z)
    P.assert_close(f"T{T} dW_r", P.to_np(dw_z), ref_dw, tol=1e-5, norm_tol=1e-6)
    P.assert_close(f"T{T} dx_r", P.to_np(dx_z), ref_dx, tol=1e-5, norm_tol=1e-6)
    # written over whatever the outputs held (NaN here), not added
    dw_n = torch.full((H, E), float("nan"), dtype=torch.float32, device=DEV)
    dx_n = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    M.moe_route_bwd_dense(x_g, torch.from_numpy(w).to(DEV), torch.from_numpy(dl).to(DEV),
                          dw_n, dx_n, accumulate=False)
    assert torch.equal(dw_n, dw_z) and torch.equal(dx_n, dx_z), "written != added to zero"


def test_route_bwd_dense_no_tokens(M):
    """T = 0: adding leaves the outputs alone, writing gives a zero dW_r."""
    H, E = 192, 48
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    w = torch.randn((H, E), device=DEV) * 0.02
    dl = torch.empty((0, E), dtype=torch.float32, device=DEV)
    dw = torch.full((H, E), 5.0, device=DEV)
    dx = torch.empty((0, H), dtype=torch.float32, device=DEV)
    M.moe_route_bwd_dense(x, w, dl, dw, dx)
    torch.cuda.synchronize()
    assert bool((dw == 5.0).all())
    M.moe_route_bwd_dense(x, w, dl, dw, dx, accumulate=False)
    torch.cuda.synchronize()
    assert bool((dw == 0.0).all())


# ---------------------------------------------------------------------------
# the combine path's logit gradient added into a dense one, and the single
# dense router backward that then replaces moe_route_bwd + moe_route_bwd_dense
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (50, 13, 3), (300, 48, 3), (1000, 128, 6), (8192, 128, 6)])
def test_route_dlogit(M, T, E, K):
    rng = np.random.default_rng(7 * T + E + K)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)   # K distinct experts
    ts = rng.uniform(0.05, 0.95, (T, K)).astype(np.float32)
    dg = rng.standard_normal((T, K)).astype(np.float32)
    base = (rng.standard_normal((T, E)) * 1e-3).astype(np.float32)
    dl = torch.from_numpy(base).to(DEV)
    M.moe_route_dlogit(torch.from_numpy(idx).to(DEV), torch.from_numpy(ts).to(DEV),
                       torch.from_numpy(dg).to(DEV), dl)
    H = 64
    _, _, sparse = O.router_bwd(np.zeros((T, H), np.float32), np.zeros((H, E), np.float32), idx,
                                ts, dg)
    P.assert_close(f"T{T} dlogit (dense + routed)", P.to_np(dl), base + sparse, tol=1e-5,
                   norm_tol=1e-6)
    # entries no token selected are untouched
    hit = np.zeros((T, E), bool)
    np.put_along_axis(hit, idx.astype(np.int64), True, axis=1)
    assert np.array_equal(P.to_np(dl)[~hit], base[~hit])


def test_one_dense_router_backward_equals_sparse_plus_dense(M):
    """At dots shapes on the GPU's own routing: moe_route_dlogit + one
    moe_route_bwd_dense (written) gives the router gradients that moe_route_bwd
    + moe_route_bwd_dense (added) give, to fp32 accuracy."""
    w = WORKLOADS["fwdbwd"]
    g = generate_torch(w, DEV)
    idx, _, ts = M.moe_route(g["x"], g["w_router"], g["bias"], w.K)
    p = M.moe_permute(idx, g["x"], w.E)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(71)
    dg = torch.randn((w.T, w.K), generator=gen, device=DEV)
    dl_bal = torch.randn((w.T, w.E), generator=gen, device=DEV) * 1e-4
    dw_a, dx_a = M.moe_route_bwd(g["x"], g["w_router"], idx, ts, dg, p["row_of"],
                                 p["offsets"], p["counts"], p["src_token"])
    M.moe_route_bwd_dense(g["x"], g["w_router"], dl_bal, dw_a, dx_a)
    dl = M.moe_route_dlogit(idx, ts, dg, dl_bal.clone())
    dw_b, dx_b = M.moe_route_bwd_dense(g["x"], g["w_router"], dl, accumulate=False)
    torch.cuda.synchronize()
    for name, a, b in (("dW_r", dw_a, dw_b), ("dx_router", dx_a, dx_b)):
        a, b = P.to_np(a).astype(np.float64), P.to_np(b).astype(np.float64)
        err = np.abs(a - b).max() / np.abs(a).max()
        print(f"{name}: max |fused - separate| / max = {err:.2e}", flush=True)
        assert err <= 1e-5, name


# ---------------------------------------------------------------------------
# the layer with the balance loss: router and input gradients end to end
# ---------------------------------------------------------------------------
def test_layer_with_balance_loss(M):
    w = Workload("mid-bal", T=1024, H=256, E=16, K=4, S=1, F=64, seed=61, router_std=0.08,
                 bias_std=0.05)
    inp = generate_numpy(w, with_dy=True)
    # a large coefficient, so that the balance terms are a visible part of the
    # router and input gradients (a missing term then fails the checks)
    alpha, L = 100.0, 256
    g = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV)
        g[k] = t if k in ("w_router", "bias") else t.to(torch.bfloat16)
    w1f, w2f = M.fuse_shared(g["w1_sh"], g["w2_sh"])
    y, ctx = M.layer_forward(g["x"], g["w_router"], g["bias"], g["w1"], g["w2"], w1f, w2f, w.K,
                             balance=(alpha, L))
    dloss = torch.tensor([3.0], dtype=torch.float32, device=DEV)
    grads = M.layer_backward(g["dy"], ctx, dloss)
    torch.cuda.synchronize()

    ref_fwd = O.forward(inp, w.K, ALIGN)
    idx = P.to_np(ctx["topk_idx"])
    assert np.array_equal(idx, ref_fwd["route"]["topk_idx"]), "routing differs (near-tie?)"
    s_ref = ref_fwd["route"]["scores"]
    ref_loss = O.seq_balance_loss(s_ref, idx, L, alpha)
    assert abs(float(P.to_np(ctx["balance_loss"])[0]) - ref_loss) <= 1e-4 * ref_loss

    ref_bwd = O.backward(inp, ref_fwd, inp["dy"])
    dl_bal = O.seq_balance_bwd(s_ref, idx, L, alpha, 3.0)
    dW_bal, dx_bal = O.router_bwd_dense(inp["x"], inp["w_router"], dl_bal)
    # the balance terms must matter at this alpha, or the check below sees nothing
    assert np.linalg.norm(dW_bal) > 0.5 * np.linalg.norm(ref_bwd["dW_r"])
    assert np.abs(dx_bal).max() > 0.04 * np.abs(ref_bwd["dx"]).max()
    P.assert_close("dlogit balance", P.to_np(grads["dlogit_balance"]), dl_bal, tol=1e-3,
                   norm_tol=1e-4)
    # the combine path's part comes through dg, a product with the stored
    # (bf16) expert rows: bounded against the bf16-storage pipeline
    emu = B.layer(inp, w.K, ALIGN, dy=inp["dy"], router_extra=(dW_bal, dx_bal))
    P.assert_close("dW_r with balance", P.to_np(grads["dw_router"]), ref_bwd["dW_r"] + dW_bal,
                   emu["dW_r"])
    P.assert_close("dx_router with balance", P.to_np(grads["dx_router"]),
                   ref_bwd["dx_router"] + dx_bal, emu["dx_router"])
    P.assert_close("dx with balance", P.to_np(grads["dx"]), ref_bwd["dx"] + dx_bal)
