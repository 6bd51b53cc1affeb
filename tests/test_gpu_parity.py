"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Small layers are compared element by element at every stage and end to end.
The full dots.llm1-shaped workloads run in the launch configuration the
benchmark times; there the oracle checks the complete routing and segment
layout, whole expert segments of sampled experts, sampled tokens end to end,
sampled hidden units of the shared experts, and the full router gradient.
"""
import os

import numpy as np
import pytest

from fine_grained_moe_amd.synthetic import (EP_SHARD, WORKLOADS, Workload, generate_numpy,
                                            generate_shard_torch, generate_torch)
from oracle import moe_oracle as O
import bf16_pipeline as B
import parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fine_grained_moe_amd import moe
    return moe


DEV = "cuda"
ALIGN = 128


@pytest.fixture(autouse=True)
def _report():
    """Print every comparison's errors: element-wise against the oracle,
    2-norm, and (where the bf16-storage pipeline is compared) that pipeline's
    own element-wise error and the kernels' error against it."""
    P.REPORT.clear()
    yield
    P.print_report()


class LazyExperts:
    """Per-expert fp32 view of a host bf16 tensor [E, R, C] (oracle input)."""

    def __init__(self, t):
        self.t = t.detach().to("cpu")
        self.shape = tuple(self.t.shape)

    def __getitem__(self, e):
        return self.t[e].float().numpy()


def unfuse_shared(dw1f, dw2f, S):
    """Fused [2SF,H] / [H,SF] shared gradients -> per expert [S,2F,H] / [S,H,F]."""
    twoSF, H = dw1f.shape
    F = twoSF // (2 * S)
    dw1 = np.stack([np.concatenate([dw1f[s * F:(s + 1) * F], dw1f[S * F + s * F:S * F + (s + 1) * F]])
                    for s in range(S)])
    dw2 = np.stack([dw2f[:, s * F:(s + 1) * F] for s in range(S)])
    return dw1, dw2


def to_gpu(inp):
    t = {}
    for k, v in inp.items():
        if k in ("w_router", "bias"):
            t[k] = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV)
        else:
            t[k] = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV).to(torch.bfloat16)
    return t


def run_layer(M, g, K, backward):
    """The layer forward and backward; the backward keeps the router's input
    gradient as an intermediate, so that it can be compared with the oracle."""
    w1f, w2f = M.fuse_shared(g["w1_sh"], g["w2_sh"]) if g["w1_sh"].shape[0] > 0 else (None, None)
    y, ctx = M.layer_forward(g["x"], g["w_router"], g["bias"], g["w1"], g["w2"], w1f, w2f, K)
    grads = M.layer_backward(g["dy"], ctx, router_input_grad=True) if backward else None
    torch.cuda.synchronize()
    return y, ctx, grads


def full_layer_checks(M, inp, K, backward=True, label=""):
    """Every stage and the whole layer against the full oracle (small layers).

    Stage checks feed the oracle the GPU's own inputs of that stage (its
    routing, rows, upstream gradient rows), so that each kernel is checked
    alone; the bf16-storage pipeline (exact arithmetic, bf16 stores) runs on
    the GPU's routing and gives the widened bound where bf16 storage alone
    exceeds the tolerance (see tests/parity.py)."""
    E = inp["w1"].shape[0]
    S = inp["w1_sh"].shape[0]
    g = to_gpu(inp)
    y, ctx, grads = run_layer(M, g, K, backward)
    p = {k: P.to_np(v) for k, v in ctx["perm"].items()}
    idx = P.to_np(ctx["topk_idx"])
    m_cap = p["x_rows"].shape[0]

    # routing
    ref_route = O.route(inp["x"], inp["w_router"], inp["bias"], K)
    n_diff, n_tie = P.check_route(idx, P.to_np(ctx["topk_w"]), P.to_np(ctx["topk_s"]), ref_route, label)
    # segments, on the GPU's own routing (bit-exact)
    ref_perm = O.permute(idx, E, ALIGN)
    P.check_permute(p, ref_perm, E, ALIGN, m_cap)
    valid = p["src_token"] >= 0
    nv = int(p["offsets"][E])
    assert np.array_equal(p["x_rows"][valid], inp["x"][p["src_token"][valid]]), "x_rows"
    # the bf16-storage pipeline on the GPU's routing
    gpu_route = dict(topk_idx=idx, topk_w=P.to_np(ctx["topk_w"]), topk_s=P.to_np(ctx["topk_s"]))
    emu = B.layer(inp, K, ALIGN, dy=inp["dy"] if backward else None, route=gpu_route)
    ev = emu["perm"]["src_token"] >= 0   # the same rows as `valid`, cut at offsets[E]
    # experts, on the GPU's own rows
    x_rows = p["x_rows"]
    act, hid, y_rows = O.experts_forward(x_rows, inp["w1"], inp["w2"], p["offsets"], p["counts"])
    P.assert_close(f"{label} act", P.to_np(ctx["act"])[valid], act[valid])
    P.assert_close(f"{label} h", P.to_np(ctx["h"])[valid], hid[valid])
    P.assert_close(f"{label} y_rows", P.to_np(ctx["y_rows"])[valid], y_rows[valid])
    y_sh = None
    if S > 0:
        y_sh_ref, _ = O.shared_forward(inp["x"], inp["w1_sh"], inp["w2_sh"])
        y_sh = P.to_np(ctx["y_sh"])
        P.assert_close(f"{label} y_shared", y_sh, y_sh_ref)
    # combine, on the GPU's own rows and weights
    y_comb = O.combine(P.to_np(ctx["y_rows"]), p["row_of"], P.to_np(ctx["topk_w"]), y_sh)
    P.assert_close(f"{label} combine", P.to_np(y), y_comb)
    # whole forward, on tokens whose routing agrees
    ref_fwd = O.forward(inp, K, ALIGN)
    same = np.all(idx == ref_fwd["route"]["topk_idx"], axis=1)
    P.assert_close(f"{label} y", P.to_np(y)[same], ref_fwd["y"][same])
    if not backward:
        return dict(n_diff=n_diff, n_tie=n_tie)

    dy = inp["dy"]
    # combine backward, on the GPU's own rows
    dy_rows_ref, dg_ref = O.combine_bwd(dy, P.to_np(ctx["y_rows"]), p["row_of"], P.to_np(ctx["topk_w"]), m_cap)
    P.assert_close(f"{label} dy_rows", P.to_np(grads["dy_rows"])[valid], dy_rows_ref[valid])
    P.assert_close(f"{label} dg", P.to_np(grads["dg"]), dg_ref)
    # expert backward, on the GPU's own rows and upstream rows
    dx_rows_ref, dW1_ref, dW2_ref, dact_ref = O.experts_backward(
        x_rows, inp["w1"], inp["w2"], act, P.to_np(grads["dy_rows"]), p["offsets"], p["counts"])
    P.assert_close(f"{label} dact", P.to_np(grads["dact"])[valid], dact_ref[valid],
                   emu["dact"][:nv][ev])
    P.assert_close(f"{label} dx_rows", P.to_np(grads["dx_rows"])[valid], dx_rows_ref[valid],
                   emu["dx_rows"][:nv][ev])
    # sums of absolute products of each expert's stored factors (the scale of
    # the componentwise gate), from the pipeline's stores on the same rows
    eo, ec = emu["perm"]["offsets"], emu["perm"]["counts"]

    def abs_prod(a, b):
        return lambda e: np.abs(a[eo[e]:eo[e] + ec[e]]).T @ np.abs(b[eo[e]:eo[e] + ec[e]])
    sc_dw1 = abs_prod(emu["dact"], emu["x_rows"])
    sc_dw2 = abs_prod(emu["dy_rows"], emu["h"])
    P.per_slice_close(f"{label} dW1", P.to_np(grads["dw1"]), dW1_ref, emu["dW1"], sc_dw1)
    P.per_slice_close(f"{label} dW2", P.to_np(grads["dw2"]), dW2_ref, emu["dW2"], sc_dw2)
    if S > 0:
        dW1s, dW2s = unfuse_shared(P.to_np(grads["dw1_sh"])[0], P.to_np(grads["dw2_sh"])[0], S)
        x64 = np.asarray(inp["x"], np.float64)
        s1, s2 = unfuse_shared(np.abs(emu["dact_sh"]).T @ np.abs(x64),
                               np.abs(np.asarray(dy, np.float64)).T @ np.abs(emu["h_sh"]), S)
        for s in range(S):
            a, _, _ = O.expert_ffn(inp["x"], inp["w1_sh"][s], inp["w2_sh"][s])
            _, dw1r, dw2r, _ = O.expert_ffn_bwd(inp["x"], inp["w1_sh"][s], inp["w2_sh"][s], a, dy)
            P.assert_close(f"{label} dW1_sh[{s}]", dW1s[s], dw1r, emu["dW1_sh"][s], s1[s])
            P.assert_close(f"{label} dW2_sh[{s}]", dW2s[s], dw2r, emu["dW2_sh"][s], s2[s])
    # router backward, on the GPU's own routing and dg (fp32 sums of fp32 inputs)
    dWr_ref, dxr_ref, _ = O.router_bwd(inp["x"], inp["w_router"], idx, P.to_np(ctx["topk_s"]),
                                        P.to_np(grads["dg"]))
    P.assert_close(f"{label} dW_r", P.to_np(grads["dw_router"]), dWr_ref)
    P.assert_close(f"{label} dx_router", P.to_np(grads["dx_router"]), dxr_ref)
    # un-permute-add, on the GPU's own terms
    extra = [P.to_np(grads["dx_router"])]
    if S > 0:
        extra.append(P.to_np(grads["dx_shared"]))
    dx_un = O.unpermute_add(P.to_np(grads["dx_rows"]), p["row_of"], extra)
    P.assert_close(f"{label} dx (un-permute)", P.to_np(grads["dx"]), dx_un)
    # whole backward against the oracle's own forward and backward
    ref_bwd = O.backward(inp, ref_fwd, dy)
    P.assert_close(f"{label} dx", P.to_np(grads["dx"])[same], ref_bwd["dx"][same])
    if same.all():
        P.per_slice_close(f"{label} dW1 (e2e)", P.to_np(grads["dw1"]), ref_bwd["dW1"], emu["dW1"],
                          sc_dw1)
        P.per_slice_close(f"{label} dW2 (e2e)", P.to_np(grads["dw2"]), ref_bwd["dW2"], emu["dW2"],
                          sc_dw2)
        P.assert_close(f"{label} dW_r (e2e)", P.to_np(grads["dw_router"]), ref_bwd["dW_r"],
                       emu["dW_r"])
    return dict(n_diff=n_diff, n_tie=n_tie)


# ---------------------------------------------------------------------------
# small layers: every stage, element by element
# ---------------------------------------------------------------------------
def test_tiny_workload(M):
    w = WORKLOADS["tiny"]
    inp = generate_numpy(w.with_(all_fp32=False), with_dy=True)  # GPU takes bf16 x / W1 / W2
    full_layer_checks(M, inp, w.K, label="tiny")


MID = {
    # several row tiles per expert, ragged tails, ragged N tiles (F=352), E=16
    "T1000_H512_E16_K4_F352": Workload("mid", T=1000, H=512, E=16, K=4, S=2, F=352, seed=21,
                                       router_std=0.08, bias_std=0.05),
    # dots-like expert count with small hidden size
    "T777_H256_E128_K6_F96": Workload("mid2", T=777, H=256, E=128, K=6, S=2, F=96, seed=22,
                                      router_std=0.1),
    # skewed: a Zipf bias concentrates tokens on few experts, most experts empty
    "T1500_H256_E64_K6_F64_skew": Workload("skew-small", T=1500, H=256, E=64, K=6, S=1, F=64,
                                           seed=23, bias_kind="zipf", router_std=0.02),
    # K = 1, no shared expert
    "T300_H128_E8_K1_S0": Workload("k1", T=300, H=128, E=8, K=1, S=0, F=64, seed=24,
                                   router_std=0.1),
    # K = E: every expert selected by every token
    "T200_H128_E4_K4": Workload("keqe", T=200, H=128, E=4, K=4, S=1, F=128, seed=25,
                                router_std=0.1),
    # a single token
    "T1_H256_E32_K6": Workload("t1", T=1, H=256, E=32, K=6, S=2, F=64, seed=26, router_std=0.1),
    # E not a multiple of 32 (a partial expert block in the router), H not a
    # multiple of 128, F not a multiple of 64
    "T700_H192_E48_K3_F160": Workload("odd", T=700, H=192, E=48, K=3, S=1, F=160, seed=27,
                                      router_std=0.1),
    # a single routed expert: every token's only choice, combine weight 1, and
    # the router gradient through the normalised weights vanishes exactly
    "T333_H128_E1_K1": Workload("e1", T=333, H=128, E=1, K=1, S=1, F=96, seed=28,
                                router_std=0.1),
    # more than eight selected experts (the combine kernels' second
    # instantiation), K not a power of two
    "T300_H192_E40_K10": Workload("k10", T=300, H=192, E=40, K=10, S=1, F=96, seed=29,
                                  router_std=0.1),
    # the largest K the library takes, every expert selected by every token
    "T260_H128_E16_K16": Workload("k16", T=260, H=128, E=16, K=16, S=2, F=64, seed=30,
                                  router_std=0.1),
    # a decode-like batch: at most 8 rows in any expert's 128-row tile
    "T40_H256_E64_K6_F160": Workload("few-rows", T=40, H=256, E=64, K=6, S=2, F=160, seed=33,
                                     router_std=0.1),
    # Zipf-skewed at a small batch: four experts hold all 150 tokens (two row
    # tiles each, the second ragged), the other 60 none
    "T150_H192_E64_K4_F96_skew": Workload("skew-k4", T=150, H=192, E=64, K=4, S=1, F=96,
                                          seed=34, bias_kind="zipf", router_std=0.02),
}


@pytest.mark.parametrize("name", sorted(MID))
def test_small_layers(M, name):
    w = MID[name]
    inp = generate_numpy(w, with_dy=True)
    full_layer_checks(M, inp, w.K, label=name)


def test_skew_has_empty_experts_with_zero_grad(M):
    w = MID["T1500_H256_E64_K6_F64_skew"]
    inp = generate_numpy(w, with_dy=True)
    g = to_gpu(inp)
    y, ctx, grads = run_layer(M, g, w.K, True)
    counts = P.to_np(ctx["perm"]["counts"])
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) > 10
    dw1 = P.to_np(grads["dw1"])
    dw2 = P.to_np(grads["dw2"])
    assert (dw1[empty] == 0).all() and (dw2[empty] == 0).all()
    assert (P.to_np(grads["dw_router"])[:, empty] == 0).all()


def test_deterministic(M):
    w = MID["T1000_H512_E16_K4_F352"]
    inp = generate_numpy(w, with_dy=True)
    g = to_gpu(inp)
    outs = []
    for _ in range(2):
        y, ctx, grads = run_layer(M, g, w.K, True)
        outs.append([y.clone(), grads["dx"].clone(), grads["dw1"].clone(), grads["dw2"].clone(),
                     grads["dw_router"].clone(), ctx["topk_idx"].clone(), ctx["perm"]["row_of"].clone()])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_backward_steps_match_composite(M):
    """The four backward step entry points, called one by one (weight
    gradients on a second stream), reproduce moe_grouped_swiglu_bwd bit for bit,
    routed (grouped) and shared (dense)."""
    w = MID["T1000_H512_E16_K4_F352"]
    inp = generate_numpy(w, with_dy=True)
    g = to_gpu(inp)
    y, ctx, grads = run_layer(M, g, w.K, True)
    p = ctx["perm"]
    E = g["w1"].shape[0]
    seg = (p["offsets"], p["counts"], p["tile_expert"])
    side = torch.cuda.Stream()
    dact = M.moe_grouped_down_dgrad(g["w2"], ctx["act"], grads["dy_rows"], *seg)
    side.wait_stream(torch.cuda.current_stream())
    dx_rows = M.moe_grouped_gate_up_dgrad(g["w1"], dact, *seg)
    with torch.cuda.stream(side):
        dw2 = M.moe_grouped_down_wgrad(grads["dy_rows"], ctx["h"], E, *seg)
        dw1 = M.moe_grouped_gate_up_wgrad(dact, p["x_rows"], E, *seg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    valid = p["src_token"] >= 0
    assert torch.equal(dact[valid], grads["dact"][valid])
    assert torch.equal(dx_rows[valid], grads["dx_rows"][valid])
    assert torch.equal(dw1, grads["dw1"]) and torch.equal(dw2, grads["dw2"])
    # shared experts: one dense group
    dact_sh = M.moe_grouped_down_dgrad(ctx["w2_shf"], ctx["act_sh"], g["dy"])
    dx_sh = M.moe_grouped_gate_up_dgrad(ctx["w1_shf"], dact_sh)
    dw2_sh = M.moe_grouped_down_wgrad(g["dy"], ctx["h_sh"], 1)
    dw1_sh = M.moe_grouped_gate_up_wgrad(dact_sh, g["x"], 1)
    torch.cuda.synchronize()
    assert torch.equal(dx_sh, grads["dx_shared"])
    assert torch.equal(dw1_sh, grads["dw1_sh"]) and torch.equal(dw2_sh, grads["dw2_sh"])


def _fused_route_permute(M, ctx, grads):
    p = ctx["perm"]
    return M.moe_route_permute_bwd(ctx["x"], ctx["w_router"], ctx["topk_idx"], ctx["topk_s"],
                                   grads["dg"], p["row_of"], p["offsets"], p["counts"],
                                   p["src_token"], grads["dx_rows"], grads["dx_shared"])


@pytest.mark.parametrize("name", ["T1000_H512_E16_K4_F352", "T300_H128_E8_K1_S0", "T1_H256_E32_K6",
                                  "T300_H192_E40_K10", "T260_H128_E16_K16", "fwdbwd"])
def test_route_permute_bwd_matches_two_calls(M, name):
    """moe_route_permute_bwd (the router's input gradient formed inside the
    un-permute) gives dW_r and dx bit for bit equal to moe_route_bwd followed
    by moe_permute_bwd, with and without shared experts, K up to 16, and at
    dots.llm1 shapes (T = 8192)."""
    if name == "fwdbwd":
        w = WORKLOADS["fwdbwd"]
        g = generate_torch(w, torch.device(DEV), with_dy=True)
    else:
        w = MID[name]
        g = to_gpu(generate_numpy(w, with_dy=True))
    print(f"route_permute_bwd {name}: T={w.T} H={w.H} E={w.E} K={w.K} S={w.S}", flush=True)
    y, ctx, grads = run_layer(M, g, w.K, True)
    dwr, dx = _fused_route_permute(M, ctx, grads)
    # the layer's default backward takes the fused call
    fused = M.layer_backward(g["dy"], ctx)
    torch.cuda.synchronize()
    assert torch.equal(dwr, grads["dw_router"])
    assert torch.equal(dx, grads["dx"])
    assert fused["dx_router"] is None
    for n in ("dx", "dw_router", "dw1", "dw2"):
        assert torch.equal(fused[n], grads[n]), n


def test_empty_batch(M):
    E, K, H, F = 8, 2, 64, 32
    x = torch.zeros((0, H), dtype=torch.bfloat16, device=DEV)
    wr = torch.randn((H, E), device=DEV)
    b = torch.zeros(E, device=DEV)
    w1 = torch.randn((E, 2 * F, H), device=DEV).to(torch.bfloat16)
    w2 = torch.randn((E, H, F), device=DEV).to(torch.bfloat16)
    idx, tw, ts = M.moe_route(x, wr, b, K)
    p = M.moe_permute(idx, x, E)
    torch.cuda.synchronize()
    assert (p["counts"] == 0).all() and (p["offsets"] == 0).all()
    assert (p["tile_expert"] == -1).all() and (p["src_token"] == -1).all()
    act, h, yr = M.moe_grouped_swiglu_fwd(p["x_rows"], w1, w2, p["offsets"], p["counts"], p["tile_expert"])
    dy_rows = torch.zeros_like(yr)
    _, _, dw1, dw2 = M.moe_grouped_swiglu_bwd(p["x_rows"], w1, w2, act, h, dy_rows, p["offsets"],
                                              p["counts"], p["tile_expert"])
    dg = torch.zeros((0, K), device=DEV)
    dwr, dxr = M.moe_route_bwd(x, wr, idx, ts, dg, p["row_of"], p["offsets"], p["counts"],
                               p["src_token"])
    dx_rows = torch.zeros((p["x_rows"].shape[0], H), dtype=torch.bfloat16, device=DEV)
    dwr2, dx2 = M.moe_route_permute_bwd(x, wr, idx, ts, dg, p["row_of"], p["offsets"],
                                        p["counts"], p["src_token"], dx_rows)
    torch.cuda.synchronize()
    assert (dw1 == 0).all() and (dw2 == 0).all() and (dwr == 0).all()
    assert (dwr2 == 0).all() and dx2.shape == (0, H)


@pytest.mark.parametrize("T,kind", [(1, "uniform"), (255, "uniform"), (256, "uniform"),
                                    (257, "uniform"), (512, "uniform"), (256, "skewed"),
                                    (257, "skewed")])
def test_permute_chunk_boundary(M, T, kind):
    """Batches on both sides of one 256-token chunk (the single-workgroup
    layout below it, the multi-chunk kernels above) at E = 128, K = 6, every
    output buffer pre-filled with a sentinel so that an unwritten entry shows:
    the layout bit for bit against the oracle's, every x row copied.  skewed:
    every token picks from the same eight experts, so segments run to T rows."""
    H, E, K = 256, 128, 6
    rng = np.random.default_rng(1000 + T)
    pool = E if kind == "uniform" else 8
    idx = np.stack([rng.permutation(pool)[:K] for _ in range(T)]).astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    m_cap = M.moe_capacity_rows(T, E, K)
    fill = lambda n, dt: torch.full(n, 0x3ead, dtype=dt, device=DEV)
    out = dict(counts=fill((E,), torch.int32), offsets=fill((E + 1,), torch.int32),
               row_of=fill((T, K), torch.int32), src_token=fill((m_cap,), torch.int32),
               tile_expert=fill((m_cap // ALIGN,), torch.int32),
               x_rows=torch.full((m_cap, H), 7.0, dtype=torch.bfloat16, device=DEV))
    print(f"case: permute chunk boundary T {T} {kind}", flush=True)
    p = M.moe_permute(torch.from_numpy(idx).to(DEV), x, E, out=out)
    torch.cuda.synchronize()
    M.moe_permute_check(p["status"])
    ref = O.permute(idx, E, ALIGN)
    g = {k: P.to_np(v) for k, v in p.items() if k not in ("x_rows", "status")}
    P.check_permute(g, ref, E, ALIGN, m_cap)
    rows = torch.from_numpy(ref["row_of"].reshape(-1)).to(DEV).long()
    toks = torch.from_numpy(np.repeat(np.arange(T), K)).to(DEV).long()
    assert torch.equal(p["x_rows"][rows], x[toks])


@pytest.mark.parametrize("T", [700, 200])
def test_permute_rejects_bad_ids(M, T):
    """The permutation's data check: tokens with an expert id outside [0,E)
    (too large, negative) or repeated within the token are rejected before
    any id indexes memory (no rows, row_of -1, x row not copied) and reported
    in the status block; every other token is permuted exactly as the oracle
    permutes the valid tokens alone.  A second call with valid ids on the same
    workspace reports nothing.  T = 200 is one chunk (the single-workgroup
    path), T = 700 three."""
    H, E, K = 128, 16, 4
    rng = np.random.default_rng(91)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    mid = T // 2
    bad = {5: (2, E), 6: (0, -1), mid: (1, 1 << 30), mid + 1: (3, None), T - 1: (0, None)}
    for t, (k, v) in bad.items():
        idx[t, k] = idx[t, (k + 1) % K] if v is None else v   # None: repeat another id
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    ws = torch.empty(M.moe_permute_workspace_bytes(T, E, K), dtype=torch.uint8, device=DEV)
    print(f"case: permute with {len(bad)} bad tokens, T {T} E {E} K {K}", flush=True)
    p = M.moe_permute(torch.from_numpy(idx).to(DEV), x, E, ws=ws)
    torch.cuda.synchronize()
    st = P.to_np(p["status"])
    assert st[0] == 3 and st[1] == len(bad) and st[2] == 5, st
    with pytest.raises(M.MoEError, match="rejected 5 token"):
        M.moe_permute_check(p["status"])
    good = np.array([t for t in range(T) if t not in bad])
    ref = O.permute(idx[good], E, ALIGN)
    g = {k: P.to_np(v) for k, v in p.items() if k not in ("x_rows", "status")}
    assert np.array_equal(g["counts"], ref["counts"]) and np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["row_of"][good], ref["row_of"])
    assert (g["row_of"][sorted(bad)] == -1).all()
    total = int(ref["offsets"][E])
    want_src = np.where(ref["src_token"] >= 0, good[np.maximum(ref["src_token"], 0)], -1)
    assert np.array_equal(g["src_token"][:total], want_src) and (g["src_token"][total:] == -1).all()
    rows = torch.from_numpy(ref["row_of"].reshape(-1)).to(DEV).long()
    toks = torch.from_numpy(np.repeat(good, K)).to(DEV).long()
    assert torch.equal(p["x_rows"][rows], x[toks])
    # valid ids on the same workspace: the block is rewritten, nothing rejected
    ok = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    p2 = M.moe_permute(torch.from_numpy(ok).to(DEV), x, E, ws=ws)
    M.moe_permute_check(p2["status"])
    assert P.to_np(p2["status"]).tolist()[:3] == [0, 0, -1]


def test_route_special_values(M):
    """Tokens with a NaN input (every logit NaN, ranked lowest: experts 0..K-1
    in index order, NaN weights), all-zero tokens (every score exactly 1/2, so
    the bias alone decides), and with a zero bias too exact key ties (lower
    index first)."""
    T, H, E, K = 64, 128, 16, 4
    rng = np.random.default_rng(77)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0:4, 5] = np.nan
    x[4:8] = 0.0
    xg = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    x = P.to_np(xg)
    wr = (rng.standard_normal((H, E)) * 0.1).astype(np.float32)
    for b in ((rng.standard_normal(E) * 0.05).astype(np.float32), np.zeros(E, np.float32)):
        idx, tw, ts = M.moe_route(xg, torch.from_numpy(wr).to(DEV), torch.from_numpy(b).to(DEV), K)
        idx, tw, ts = P.to_np(idx), P.to_np(tw), P.to_np(ts)
        ref = O.route(x, wr, b, K)
        assert (idx[0:4] == np.arange(K)).all() and (ref["topk_idx"][0:4] == np.arange(K)).all()
        assert np.isnan(tw[0:4]).all() and np.isnan(ref["topk_w"][0:4]).all()
        assert np.array_equal(idx[4:8], ref["topk_idx"][4:8])
        assert (ts[4:8] == 0.5).all() and np.array_equal(tw[4:8], ref["topk_w"][4:8])
        if not b.any():
            assert (idx[4:8] == np.arange(K)).all()
        sub = {k: (v[8:] if isinstance(v, np.ndarray) and v.shape[:1] == (T,) else v)
               for k, v in ref.items()}
        P.check_route(idx[8:], tw[8:], ts[8:], sub, "special")


# ---------------------------------------------------------------------------
# full dots.llm1-shaped workloads (the benchmark's launch configuration)
# ---------------------------------------------------------------------------
def pick_experts(counts, n, rng):
    """The smallest and the largest non-empty expert, the median one by
    count, then random non-empty experts up to n (sorted, distinct)."""
    nonempty = np.nonzero(counts)[0]
    by_count = nonempty[np.argsort(counts[nonempty], kind="stable")]
    pick = {int(by_count[0]), int(by_count[-1]), int(by_count[len(by_count) // 2])}
    rest = [int(e) for e in rng.permutation(nonempty) if int(e) not in pick]
    return sorted(pick | set(rest[:max(0, n - len(pick))]))


def unit_wgrad_checks(name, x_all, dy_all, w1e, w2e, dw1, dw2, units):
    """Weight gradients of single hidden units over all of an expert's rows:
    gate row f and up row F+f of dW1 and column f of dW2 depend on unit f
    alone (its two W1 rows and its W2 column).  x_all, dy_all: the expert's
    rows (fp32 arrays); dw1 [2F,H], dw2 [H,F]: the GPU's gradients (torch)."""
    F = w1e.shape[0] // 2
    for f in units:
        w1u = w1e[[f, F + f]]
        w2u = w2e[:, [f]]
        au, _, _ = O.expert_ffn(x_all, w1u, w2u)
        _, dw1u, dw2u, _ = O.expert_ffn_bwd(x_all, w1u, w2u, au, dy_all)
        ae, he, _ = B.expert_forward(x_all, w1u, w2u)
        _, dw1e, dw2e, dae = B.expert_backward(x_all, w1u, w2u, ae, he, dy_all)
        s1 = np.abs(dae).T @ np.abs(np.asarray(x_all, np.float64))   # [2, H]
        s2 = np.abs(np.asarray(dy_all, np.float64)).T @ np.abs(he)   # [H, 1]
        P.assert_close(f"{name} dW1[{f}] gate", P.to_np(dw1[f]), dw1u[0], dw1e[0], s1[0])
        P.assert_close(f"{name} dW1[{F + f}] up", P.to_np(dw1[F + f]), dw1u[1], dw1e[1], s1[1])
        P.assert_close(f"{name} dW2[:,{f}]", P.to_np(dw2[:, f]), dw2u[:, 0], dw2e[:, 0], s2[:, 0])


def sampled_checks(M, w, backward, n_tokens=12, n_experts=4, n_units=3, seed=0):
    g = generate_torch(w, DEV, with_dy=backward)
    K, E, S = w.K, w.E, w.S
    y, ctx, grads = run_layer(M, g, K, backward)
    x = P.to_np(g["x"])
    wr = P.to_np(g["w_router"])
    bias = P.to_np(g["bias"])
    W1, W2 = LazyExperts(g["w1"]), LazyExperts(g["w2"])
    W1s, W2s = P.to_np(g["w1_sh"]), P.to_np(g["w2_sh"])

    # full routing and segments
    idx = P.to_np(ctx["topk_idx"])
    ref_route = O.route(x, wr, bias, K)
    P.check_route(idx, P.to_np(ctx["topk_w"]), P.to_np(ctx["topk_s"]), ref_route, w.name)
    p = {k: P.to_np(v) for k, v in ctx["perm"].items() if k != "x_rows"}
    ref_perm = O.permute(idx, E, ALIGN)
    P.check_permute(p, ref_perm, E, ALIGN, p["src_token"].shape[0])
    src = torch.from_numpy(p["src_token"]).to(DEV).long()
    vmask = src >= 0
    assert torch.equal(ctx["perm"]["x_rows"][vmask], g["x"][src[vmask]]), "x_rows"

    # rows of sampled experts, stage by stage on the GPU's own rows (a random
    # subset of 2048 rows of a longer segment: each row's result depends on
    # that row alone)
    counts = p["counts"]
    rng = np.random.default_rng(seed)
    pick = pick_experts(counts, n_experts, rng)
    print(f"  {w.name}: sampled experts {pick} with {[int(counts[e]) for e in pick]} rows", flush=True)
    row_sets = {}
    for e in pick:
        r0, n = int(p["offsets"][e]), int(counts[e])
        rows = np.sort(rng.choice(n, 2048, replace=False)) + r0 if n > 2048 else np.arange(r0, r0 + n)
        row_sets[e] = rows
        sel = torch.from_numpy(rows).to(DEV)
        xr = P.to_np(ctx["perm"]["x_rows"][sel])
        a, hid, ye = O.expert_ffn(xr, W1[e], W2[e])
        P.assert_close(f"{w.name} act[e={e}]", P.to_np(ctx["act"][sel]), a)
        P.assert_close(f"{w.name} h[e={e}]", P.to_np(ctx["h"][sel]), hid)
        _, _, y_e = B.expert_forward(xr, W1[e], W2[e])
        P.assert_close(f"{w.name} y_rows[e={e}]", P.to_np(ctx["y_rows"][sel]), ye, y_e)

    # sampled tokens end to end (routing agreeing)
    toks = np.sort(rng.choice(w.T, n_tokens, replace=False))
    sub = dict(x=x[toks], w_router=wr, bias=bias, w1=W1, w2=W2, w1_sh=W1s, w2_sh=W2s)
    ref = O.forward(sub, K, ALIGN)
    same = np.all(idx[toks] == ref["route"]["topk_idx"], axis=1)
    P.assert_close(f"{w.name} y[sampled]", P.to_np(y)[toks][same], ref["y"][same])
    if not backward:
        return
    dy = P.to_np(g["dy"])
    sub["dy"] = dy[toks]
    ref_b = O.backward(sub, ref, sub["dy"])
    P.assert_close(f"{w.name} dx[sampled]", P.to_np(grads["dx"])[toks][same], ref_b["dx"][same])
    P.assert_close(f"{w.name} dg[sampled]", P.to_np(grads["dg"])[toks][same], ref_b["dg"][same])

    # backward of the sampled experts on the GPU's own upstream rows: dact and
    # dx_rows on the sampled rows, the weight gradients of sampled hidden
    # units over every row of the expert (however long the segment)
    F = w.F
    for e in pick:
        rows = row_sets[e]
        sel = torch.from_numpy(rows).to(DEV)
        xr = P.to_np(ctx["perm"]["x_rows"][sel])
        dyr = P.to_np(grads["dy_rows"][sel])
        a, _, _ = O.expert_ffn(xr, W1[e], W2[e])
        dxr, _, _, dar = O.expert_ffn_bwd(xr, W1[e], W2[e], a, dyr)
        ae, he, _ = B.expert_forward(xr, W1[e], W2[e])
        dx_e, _, _, dact_e = B.expert_backward(xr, W1[e], W2[e], ae, he, dyr)
        P.assert_close(f"{w.name} dact[e={e}]", P.to_np(grads["dact"][sel]), dar, dact_e)
        P.assert_close(f"{w.name} dx_rows[e={e}]", P.to_np(grads["dx_rows"][sel]), dxr, dx_e)
        r0, n = int(p["offsets"][e]), int(counts[e])
        all_rows = torch.arange(r0, r0 + n, device=DEV)
        unit_wgrad_checks(f"{w.name} e={e} ({n} rows)", P.to_np(ctx["perm"]["x_rows"][all_rows]),
                          P.to_np(grads["dy_rows"][all_rows]), W1[e], W2[e], grads["dw1"][e],
                          grads["dw2"][e], rng.choice(F, n_units, replace=False))
    empty = np.nonzero(counts == 0)[0]
    if len(empty):
        assert not grads["dw1"][torch.from_numpy(empty).to(DEV)].any()
        assert not grads["dw2"][torch.from_numpy(empty).to(DEV)].any()

    # shared experts: sampled hidden units (each unit's gradient depends on it alone)
    dw1f = grads["dw1_sh"][0]
    dw2f = grads["dw2_sh"][0]
    for s in range(S):
        for f in rng.choice(F, 3, replace=False):
            w1u = W1s[s][[f, F + f]]
            w2u = W2s[s][:, [f]]
            au, _, _ = O.expert_ffn(x, w1u, w2u)
            _, dw1u, dw2u, _ = O.expert_ffn_bwd(x, w1u, w2u, au, dy)
            ae, he, _ = B.expert_forward(x, w1u, w2u)
            _, dw1e, dw2e, dae = B.expert_backward(x, w1u, w2u, ae, he, dy)
            s1 = np.abs(dae).T @ np.abs(np.asarray(x, np.float64))
            s2 = np.abs(np.asarray(dy, np.float64)).T @ np.abs(he)
            gate_row, up_row = s * F + f, S * F + s * F + f
            P.assert_close(f"{w.name} dW1_sh[{s},{f}] gate", P.to_np(dw1f[gate_row]), dw1u[0],
                           dw1e[0], s1[0])
            P.assert_close(f"{w.name} dW1_sh[{s},{f}] up", P.to_np(dw1f[up_row]), dw1u[1], dw1e[1],
                           s1[1])
            P.assert_close(f"{w.name} dW2_sh[{s},{f}]", P.to_np(dw2f[:, s * F + f]), dw2u[:, 0],
                           dw2e[:, 0], s2[:, 0])

    # router gradient, full, on the GPU's own routing and dg
    dWr_ref, _, _ = O.router_bwd(x, wr, idx, P.to_np(ctx["topk_s"]), P.to_np(grads["dg"]))
    P.assert_close(f"{w.name} dW_r", P.to_np(grads["dw_router"]), dWr_ref)


@pytest.mark.timeout(600)
def test_decode_full_oracle(M):
    """T=256 at dots shapes: small enough for the whole oracle."""
    w = WORKLOADS["decode"]
    g = generate_torch(w, DEV, with_dy=True)
    inp = {k: P.to_np(v) for k, v in g.items()}
    full_layer_checks(M, inp, w.K, backward=True, label="decode")


@pytest.mark.timeout(600)
def test_prefill_sampled(M):
    sampled_checks(M, WORKLOADS["prefill"], backward=False)


@pytest.mark.timeout(600)
def test_skew_sampled(M):
    """The skewed batch: its largest segments hold thousands of rows (512
    k-stages per weight-gradient tile), compared over all of their rows."""
    sampled_checks(M, WORKLOADS["skew"], backward=True, n_experts=5)


@pytest.mark.timeout(600)
def test_fwdbwd_sampled(M):
    sampled_checks(M, WORKLOADS["fwdbwd"], backward=True, n_experts=8, n_units=2)


# The largest token count a training step accepts at dots shapes: the weight
# gradients address a segment of rows through 32-bit byte offsets, so the
# permuted capacity times a 10 KB row (H = 5120 bf16) must stay below 4 GiB.
# T is not a multiple of 32 either, so the last row tiles are ragged.
MAX_T = 67178


@pytest.mark.timeout(900)
def test_max_tokens_sampled(M):
    """Forward and backward at the largest accepted T: byte offsets of the
    permuted rows run past 2 GiB and up to 4 GiB, which every row kernel and
    GEMM tile must address in 64 bits or as unsigned 32-bit buffer offsets."""
    row_bytes = 2 * 5120
    m_cap = M.moe_capacity_rows(MAX_T, 128, 6)
    assert m_cap * row_bytes < 1 << 32 <= M.moe_capacity_rows(MAX_T + 1, 128, 6) * row_bytes
    assert m_cap * row_bytes > 1 << 31
    w = Workload("max_tokens", T=MAX_T, H=5120, E=128, K=6, S=2, F=1408, seed=6, backward=True)
    sampled_checks(M, w, backward=True, n_tokens=16)


@pytest.mark.timeout(600)
def test_ep_shard_sampled(M):
    """The six routed grouped products at one GPU's share of an 8-way
    expert-parallel layer (16 experts x 3072 rows, the benchmark's ep_shard
    configuration): sampled rows of sampled experts stage by stage, and the
    weight gradients of sampled hidden units over all of the expert's rows."""
    E, R, H, F = EP_SHARD["E"], EP_SHARD["rows"], EP_SHARD["H"], EP_SHARD["F"]
    g = generate_shard_torch(DEV, E, R, H, F, EP_SHARD["seed"])
    i32 = torch.int32
    offsets = torch.arange(E + 1, dtype=i32, device=DEV) * R
    counts = torch.full((E,), R, dtype=i32, device=DEV)
    tile_expert = (torch.arange(E * R // ALIGN, dtype=i32, device=DEV) // (R // ALIGN)).to(i32)
    seg = (offsets, counts, tile_expert)
    act, h = M.moe_grouped_gate_up_fwd(g["x_rows"], g["w1"], *seg)
    y_rows = M.moe_grouped_down_fwd(h, g["w2"], *seg)
    dact = M.moe_grouped_down_dgrad(g["w2"], act, g["dy_rows"], *seg)
    dx_rows = M.moe_grouped_gate_up_dgrad(g["w1"], dact, *seg)
    dw2 = M.moe_grouped_down_wgrad(g["dy_rows"], h, E, *seg)
    dw1 = M.moe_grouped_gate_up_wgrad(dact, g["x_rows"], E, *seg)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    W1, W2 = LazyExperts(g["w1"]), LazyExperts(g["w2"])
    for e in (0, 9, E - 1):
        rows = np.sort(rng.choice(R, 256, replace=False)) + e * R
        sel = torch.from_numpy(rows).to(DEV)
        xr = P.to_np(g["x_rows"][sel])
        dyr = P.to_np(g["dy_rows"][sel])
        a, hid, ye = O.expert_ffn(xr, W1[e], W2[e])
        ae, he, y_e = B.expert_forward(xr, W1[e], W2[e])
        P.assert_close(f"shard act[e={e}]", P.to_np(act[sel]), a)
        P.assert_close(f"shard h[e={e}]", P.to_np(h[sel]), hid)
        P.assert_close(f"shard y_rows[e={e}]", P.to_np(y_rows[sel]), ye, y_e)
        dxr, _, _, dar = O.expert_ffn_bwd(xr, W1[e], W2[e], a, dyr)
        dx_e, _, _, dact_e = B.expert_backward(xr, W1[e], W2[e], ae, he, dyr)
        P.assert_close(f"shard dact[e={e}]", P.to_np(dact[sel]), dar, dact_e)
        P.assert_close(f"shard dx_rows[e={e}]", P.to_np(dx_rows[sel]), dxr, dx_e)
        # weight gradients of sampled hidden units over all of the expert's rows
        all_rows = torch.arange(e * R, (e + 1) * R, device=DEV)
        unit_wgrad_checks(f"shard e={e}", P.to_np(g["x_rows"][all_rows]),
                          P.to_np(g["dy_rows"][all_rows]), W1[e], W2[e], dw1[e], dw2[e],
                          rng.choice(F, 2, replace=False))


@pytest.mark.timeout(600)
def test_wgrad_segment_past_2gib(M):
    """A dense gate/up weight gradient over one segment of 400,001 rows at
    H = 5120, F = 1408: both operands exceed 2 GiB (dact 2.25 GB, x rows
    4.1 GB; below the 4 GiB the ABI admits), and 400,001 is not a multiple of
    the 32-row k-stage, so the last stage holds 31 rows past the segment's
    end.  Those rows must read as zeros: their buffer offset lies past every
    admissible segment size.  Checked on sampled hidden units over all rows."""
    n, H, F = 400_001, 5120, 1408
    print(f"case: dense gate/up wgrad, {n} rows, H {H}, F {F}", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(404)
    x_rows = torch.randn((n, H), generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    dact = torch.empty((n, 2 * F), dtype=torch.bfloat16, device=DEV)
    for i in range(0, n, 65536):   # bounded fp32 staging
        m = min(65536, n - i)
        dact[i:i + m] = torch.randn((m, 2 * F), generator=gen, device=DEV).to(torch.bfloat16)
    assert n * 2 * F * 2 > 1 << 31 and n * H * 2 > 1 << 31 and n * H * 2 < 1 << 32
    dw1 = M.moe_grouped_gate_up_wgrad(dact, x_rows, 1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(404)
    for f in sorted(rng.choice(2 * F, 4, replace=False)):
        col = dact[:, f].float()
        ref = np.zeros(H, np.float64)
        for i in range(0, n, 65536):   # fp64 sum over all rows, in row blocks
            m = min(65536, n - i)
            ref += P.to_np(col[i:i + m]).astype(np.float64) @ P.to_np(x_rows[i:i + m]).astype(np.float64)
        got = P.to_np(dw1[0, f])
        P.assert_close(f"dW1[{f}] over {n} rows", got, ref)


def test_inference_forward_without_saved_activations(M):
    """save_for_backward=False skips the gate/up activations (the epilogue
    writes h only); h, the expert rows and y are bit-identical to the training
    forward, routed and shared."""
    w = MID["T1000_H512_E16_K4_F352"]
    inp = generate_numpy(w, with_dy=False)
    g = {k: torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV) for k, v in inp.items()}
    for k in ("x", "w1", "w2", "w1_sh", "w2_sh"):
        g[k] = g[k].to(torch.bfloat16)
    w1f, w2f = M.fuse_shared(g["w1_sh"], g["w2_sh"])
    args = (g["x"], g["w_router"], g["bias"], g["w1"], g["w2"], w1f, w2f, w.K)
    y_t, ctx_t = M.layer_forward(*args, save_for_backward=True)
    y_i, ctx_i = M.layer_forward(*args, save_for_backward=False)
    torch.cuda.synchronize()
    assert ctx_i["act"] is None and ctx_i["act_sh"] is None
    assert torch.equal(y_i, y_t)
    valid = ctx_t["perm"]["src_token"] >= 0
    assert torch.equal(ctx_i["h"][valid], ctx_t["h"][valid])
    assert torch.equal(ctx_i["y_rows"][valid], ctx_t["y_rows"][valid])
    assert torch.equal(ctx_i["h_sh"], ctx_t["h_sh"])
