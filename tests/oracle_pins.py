"""Checks that pin the CPU oracle to things other than itself.

Each check_* function raises AssertionError on failure.  The oracle's own
tests call them on the real oracle; the mutation tests call them on copies of
the oracle with a planted mistake and require at least one to fire.

Pins used:
  * exact sums (math.fsum of exact fp64 products) for the router logits;
  * hand-worked golden fixtures (tests/golden/*.json) for routing and segments;
  * brute force in plain Python (sorted tuples for top-K, per-token dense
    expert evaluation with math.exp, loop re-derivation of segments);
  * library special cases: torch fp64 nn.functional for a one-expert layer,
    torch fp64 autograd for the backward on a dense re-expression;
  * closed forms and invariants: sigmoid values, sum of combine weights,
    routing independence when all experts are identical, central finite
    differences of the forward.
  * load balancing: hand-worked bias steps and balance losses, the loss's
    closed forms (uniform scores or balanced picks give alpha, collapsed
    routing gives alpha E / K), the bias rule driving a skewed router towards
    balance, and central finite differences of the loss in the logits.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def small_inputs(T=24, H=16, E=6, K=2, S=1, F=8, seed=11, w_std=0.3):
    """Small random fp32 layer with O(1) logits so routing is not trivial."""
    rng = np.random.default_rng(seed)
    f = np.float32
    return dict(
        x=rng.standard_normal((T, H)).astype(f),
        w_router=(rng.standard_normal((H, E)) * 0.5).astype(f),
        bias=(rng.standard_normal(E) * 0.1).astype(f),
        w1=(rng.standard_normal((E, 2 * F, H)) * w_std).astype(f),
        w2=(rng.standard_normal((E, H, F)) * w_std).astype(f),
        w1_sh=(rng.standard_normal((S, 2 * F, H)) * w_std).astype(f),
        w2_sh=(rng.standard_normal((S, H, F)) * w_std).astype(f),
        dy=rng.standard_normal((T, H)).astype(f),
    ), K


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------
def check_logits_exact_sum(O, x, w):
    """Oracle logits equal the exact sum (fsum of exact fp64 products) rounded
    to fp32, up to one fp32 ulp (double rounding)."""
    got = O.router_logits(x, w)
    T, H = x.shape
    E = w.shape[1]
    exact = np.empty((T, E), np.float32)
    for t in range(T):
        for e in range(E):
            exact[t, e] = np.float32(math.fsum(float(x[t, h]) * float(w[h, e]) for h in range(H)))
    ulp = np.abs(got.view(np.int32).astype(np.int64) - exact.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, f"logits off by {ulp.max()} ulp"
    assert (ulp == 0).mean() > 0.99


def check_sigmoid_closed_form(O):
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0, 2.5, -7.25], np.float32)
    s = O.router_scores(z[None, :])[0].astype(np.float64)
    zf = z.astype(np.float64)
    expect = np.array([0.5, 0.75, 0.25, 1.0, math.exp(-40.0), 0, 0])
    assert s[0] == 0.5
    assert abs(s[1] - 1.0 / (1.0 + 1.0 / (math.exp(float(zf[1]))))) < 1e-7
    assert abs(s[1] - 0.75) < 1e-7 and abs(s[2] - 0.25) < 1e-7
    assert s[3] == 1.0 and abs(s[4] - expect[4]) < 1e-20
    # symmetry sigma(-z) = 1 - sigma(z) and the derivative identity via a
    # difference quotient: sigma'(z) = sigma(z)(1 - sigma(z))
    for zz in (0.3, 1.7, -2.2):
        a = float(O.router_scores(np.array([[zz]], np.float32))[0, 0])
        b = float(O.router_scores(np.array([[-zz]], np.float32))[0, 0])
        assert abs(a + b - 1.0) < 2e-7
        lo = O.sigmoid64(np.array(zz - 1e-6))
        hi = O.sigmoid64(np.array(zz + 1e-6))
        assert abs((hi - lo) / 2e-6 - a * (1 - a)) < 1e-6


def topk_bruteforce(keys, K):
    out = []
    for row in keys:
        items = sorted(((-(float(v) if not math.isnan(v) else -math.inf), e) for e, v in enumerate(row)))
        out.append([e for _, e in items[:K]])
    return np.array(out, np.int32)


def check_topk_bruteforce(O, keys, K):
    got = O.top_k(keys, K)
    exp = topk_bruteforce(keys, K)
    assert np.array_equal(got, exp), "top-K differs from brute force"
    for row in got:
        assert len(set(row.tolist())) == K


def check_route_golden(O):
    g = load_golden("route_small.json")
    ln3 = math.log(3.0)
    val = {"0": 0.0, "ln3": ln3, "-ln3": -ln3}
    w = np.array([[val[c] for c in row] for row in g["w_router"]], np.float32)
    r = O.route(np.array(g["x"], np.float32), w, np.array(g["bias"], np.float32), g["K"])
    assert np.array_equal(r["topk_idx"], np.array(g["topk_idx"])), r["topk_idx"]
    assert np.allclose(r["topk_w"], np.array(g["topk_w"]), atol=1e-6), r["topk_w"]
    assert np.allclose(r["scores"], np.array(g["scores"]), atol=1e-6)


def check_combine_weight_invariants(O, x, w, b, K):
    r = O.route(x, w, b, K)
    g = r["topk_w"].astype(np.float64)
    assert (g > 0).all()
    assert np.abs(g.sum(1) - 1.0).max() <= 1e-6
    # K = 1: weight exactly one; K = E: g = s / sum(s) over all experts
    r1 = O.route(x, w, b, 1)
    assert (r1["topk_w"] == 1.0).all()
    E = w.shape[1]
    rE = O.route(x, w, b, E)
    s = r["scores"].astype(np.float64)
    full = np.take_along_axis(s / s.sum(1, keepdims=True), rE["topk_idx"].astype(np.int64), 1)
    assert np.abs(rE["topk_w"] - full).max() < 1e-7
    # the weights follow the raw scores: s_k / s_j == g_k / g_j
    ratio_s = r["topk_s"][:, 0].astype(np.float64) / r["topk_s"][:, -1]
    ratio_g = g[:, 0] / g[:, -1]
    assert np.allclose(ratio_s, ratio_g, rtol=1e-6)


# ---------------------------------------------------------------------------
# Segments
# ---------------------------------------------------------------------------
def check_permute_golden(O):
    for c in load_golden("permute_small.json")["cases"]:
        p = O.permute(np.array(c["topk_idx"], np.int32), c["E"], c["align"])
        for key in ("counts", "offsets", "row_of", "src_token"):
            assert np.array_equal(p[key], np.array(c[key])), (c["name"], key, p[key])


def permute_bruteforce(topk_idx, E, align):
    T, K = topk_idx.shape
    counts = [0] * E
    for t in range(T):
        for k in range(K):
            counts[int(topk_idx[t, k])] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + -(-counts[e] // align) * align)
    nxt = offsets[:-1].copy()
    row_of = [[0] * K for _ in range(T)]
    for t in range(T):                      # ascending token order
        for e in range(E):                  # experts visited in index order
            for k in range(K):
                if int(topk_idx[t, k]) == e:
                    row_of[t][k] = nxt[e]
                    nxt[e] += 1
    src = [-1] * offsets[-1]
    for t in range(T):
        for k in range(K):
            src[row_of[t][k]] = t
    return counts, offsets, row_of, src


def check_permute_bruteforce(O, topk_idx, E, align):
    p = O.permute(topk_idx, E, align)
    counts, offsets, row_of, src = permute_bruteforce(topk_idx, E, align)
    assert p["counts"].tolist() == counts
    assert p["offsets"].tolist() == offsets
    assert p["row_of"].tolist() == row_of
    assert p["src_token"].tolist() == src


def check_permute_invariants(p, topk_idx, E, align):
    T, K = topk_idx.shape
    counts, offsets, row_of, src = p["counts"], p["offsets"], p["row_of"], p["src_token"]
    assert counts.sum() == T * K
    assert (offsets % align == 0).all() and offsets[0] == 0
    seg = np.diff(offsets)
    assert (seg >= counts).all() and (seg - counts < align).all()
    assert ((counts == 0) == (seg == 0)).all()
    flat = row_of.reshape(-1)
    assert len(np.unique(flat)) == T * K           # injective
    e_of = topk_idx.reshape(-1)
    assert (flat >= offsets[e_of]).all() and (flat < offsets[e_of] + counts[e_of]).all()
    assert (src[flat] == np.repeat(np.arange(T), K)).all()
    assert (src >= 0).sum() == T * K
    for e in range(E):                             # ascending tokens inside a segment
        tok = src[offsets[e]:offsets[e] + counts[e]]
        assert (np.diff(tok) > 0).all()
        assert (src[offsets[e] + counts[e]:offsets[e + 1]] == -1).all()


# ---------------------------------------------------------------------------
# Experts and whole forward
# ---------------------------------------------------------------------------
def dense_forward_bruteforce(inp, K):
    """Per-token dense evaluation in plain Python floats: every expert on every
    token, then keep the K selected ones with their weights.  No permutation.
    The routing decision (top-K of s + b, ties to the lower index) and the
    weights s_k / sum s are taken from their definitions with math.exp."""
    x, wr, b = inp["x"], inp["w_router"], inp["bias"]
    w1, w2, w1s, w2s = inp["w1"], inp["w2"], inp["w1_sh"], inp["w2_sh"]
    T, H = x.shape
    E = wr.shape[1]
    F = w1.shape[1] // 2

    def sig(z):
        return 1.0 / (1.0 + math.exp(-z)) if z > -700 else 0.0

    def ffn(xt, W1, W2):
        h = []
        for f in range(F):
            g = math.fsum(float(W1[f, i]) * xt[i] for i in range(H))
            u = math.fsum(float(W1[F + f, i]) * xt[i] for i in range(H))
            h.append(g * sig(g) * u)
        return [math.fsum(float(W2[o, f]) * h[f] for f in range(F)) for o in range(H)]

    y = np.zeros((T, H))
    sel_all = []
    for t in range(T):
        xt = [float(v) for v in x[t]]
        s = [float(np.float32(sig(float(np.float32(
            math.fsum(xt[i] * float(wr[i, e]) for i in range(H))))))) for e in range(E)]
        keys = [float(np.float32(np.float32(s[e]) + np.float32(b[e]))) for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-keys[e], e))[:K]
        sel_all.append(sel)
        tot = sum(s[e] for e in sel)
        out = [0.0] * H
        for e in range(E):                     # dense: every expert evaluated
            ye = ffn(xt, w1[e], w2[e])
            wgt = s[e] / tot if e in sel else 0.0
            out = [o + wgt * v for o, v in zip(out, ye)]
        for sidx in range(w1s.shape[0]):
            ys = ffn(xt, w1s[sidx], w2s[sidx])
            out = [o + v for o, v in zip(out, ys)]
        y[t] = out
    return y, np.array(sel_all)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


def check_forward_bruteforce(O, inp, K, align):
    out = O.forward(inp, K, align)
    y_ref, sel = dense_forward_bruteforce(inp, K)
    assert np.array_equal(out["route"]["topk_idx"], sel)
    e = rel_err(out["y"], y_ref)
    assert e < 1e-6, f"forward vs dense brute force: {e}"


def check_one_expert_is_dense_swiglu(O, seed=3):
    """E=1, K=1, S=0: the layer is a dense SwiGLU FFN (torch fp64 nn.functional)."""
    import torch
    import torch.nn.functional as Fn
    rng = np.random.default_rng(seed)
    T, H, F = 10, 12, 7
    inp = dict(x=rng.standard_normal((T, H)).astype(np.float32),
               w_router=rng.standard_normal((H, 1)).astype(np.float32),
               bias=np.zeros(1, np.float32),
               w1=(rng.standard_normal((1, 2 * F, H)) * 0.4).astype(np.float32),
               w2=(rng.standard_normal((1, H, F)) * 0.4).astype(np.float32),
               w1_sh=np.zeros((0, 2 * F, H), np.float32),
               w2_sh=np.zeros((0, H, F), np.float32))
    y = O.forward(inp, 1, 4)["y"]
    xt = torch.from_numpy(inp["x"]).double()
    wg = torch.from_numpy(inp["w1"][0, :F]).double()
    wu = torch.from_numpy(inp["w1"][0, F:]).double()
    wd = torch.from_numpy(inp["w2"][0]).double()
    ref = Fn.linear(Fn.silu(Fn.linear(xt, wg)) * Fn.linear(xt, wu), wd).numpy()
    assert rel_err(y, ref) < 1e-12, rel_err(y, ref)


def check_identical_experts_independent_of_routing(O, inp, K, align):
    """All routed experts equal => y = shared(x) + expert(x), whatever the bias
    selects, because the combine weights sum to one."""
    inp = dict(inp)
    E = inp["w1"].shape[0]
    inp["w1"] = np.repeat(inp["w1"][:1], E, axis=0)
    inp["w2"] = np.repeat(inp["w2"][:1], E, axis=0)
    _, _, ye = O.expert_ffn(inp["x"], inp["w1"][0], inp["w2"][0])
    ys = sum(O.expert_ffn(inp["x"], inp["w1_sh"][s], inp["w2_sh"][s])[2]
             for s in range(inp["w1_sh"].shape[0]))
    for bias in (inp["bias"], -inp["bias"] * 7.0):
        inp["bias"] = bias.astype(np.float32)
        y = O.forward(inp, K, align)["y"]
        assert rel_err(y, ys + ye) < 1e-6, rel_err(y, ys + ye)


def check_shared_fusion(O, inp):
    """Fused shared weights [2SF,H] / [H,SF] equal the per-expert sum."""
    w1s, w2s = inp["w1_sh"], inp["w2_sh"]
    S, twoF, H = w1s.shape
    F = twoF // 2
    w1f = np.concatenate([w1s[:, :F].reshape(S * F, H), w1s[:, F:].reshape(S * F, H)])
    w2f = np.concatenate([w2s[s] for s in range(S)], axis=1)
    _, _, yf = O.expert_ffn(inp["x"], w1f, w2f)
    y, _ = O.shared_forward(inp["x"], w1s, w2s)
    assert rel_err(yf, y) < 1e-12


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
def torch_dense_layer(inp, sel):
    """fp64 torch re-expression of the layer with the selection `sel` frozen:
    dense over experts with a 0/1 mask, so no permutation machinery."""
    import torch
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True)
         for k, v in inp.items() if k != "bias" and k != "dy"}
    x, wr, w1, w2 = t["x"], t["w_router"], t["w1"], t["w2"]
    T, H = x.shape
    E = wr.shape[1]
    F = w1.shape[1] // 2
    s = torch.sigmoid(x @ wr)
    mask = torch.zeros(T, E, dtype=torch.float64)
    mask[torch.arange(T)[:, None], torch.from_numpy(np.asarray(sel, np.int64))] = 1.0
    sm = s * mask
    g = sm / sm.sum(1, keepdim=True)
    y = torch.zeros(T, H, dtype=torch.float64)
    for e in range(E):
        a = x @ w1[e].T
        ye = (torch.nn.functional.silu(a[:, :F]) * a[:, F:]) @ w2[e].T
        y = y + g[:, e:e + 1] * ye
    for si in range(t["w1_sh"].shape[0]):
        a = x @ t["w1_sh"][si].T
        y = y + (torch.nn.functional.silu(a[:, :F]) * a[:, F:]) @ t["w2_sh"][si].T
    return t, y


def check_backward_autograd(O, inp, K, align):
    import torch
    fwd = O.forward(inp, K, align)
    bwd = O.backward(inp, fwd, inp["dy"])
    t, y = torch_dense_layer(inp, fwd["route"]["topk_idx"])
    (y * torch.from_numpy(inp["dy"].astype(np.float64))).sum().backward()
    pairs = [("dx", "x"), ("dW1", "w1"), ("dW2", "w2"), ("dW_r", "w_router"),
             ("dW1_sh", "w1_sh"), ("dW2_sh", "w2_sh")]
    assert rel_err(fwd["y"], y.detach().numpy()) < 1e-6
    for mine, theirs in pairs:
        ref = t[theirs].grad.numpy()
        e = rel_err(bwd[mine], ref)
        tol = 1e-6  # dW are stored as fp32
        assert e < tol, f"{mine}: {e}"


def frozen_loss(O, inp, sel, dy):
    """L = <dy, y> with the routing decision held fixed (fp64)."""
    # logits in fp64 without the fp32 rounding, so the finite difference sees
    # a smooth function
    logits = np.asarray(inp["x"], np.float64) @ np.asarray(inp["w_router"], np.float64)
    s = O.sigmoid64(logits)
    ssel = np.take_along_axis(s, sel.astype(np.int64), 1)
    g = ssel / ssel.sum(1, keepdims=True)
    y = np.zeros(inp["x"].shape, np.float64)
    for k in range(sel.shape[1]):
        for t in range(sel.shape[0]):
            e = int(sel[t, k])
            _, _, ye = O.expert_ffn(inp["x"][t:t + 1].astype(np.float64), inp["w1"][e], inp["w2"][e])
            y[t] += g[t, k] * ye[0]
    ys, _ = O.shared_forward(np.asarray(inp["x"], np.float64), inp["w1_sh"], inp["w2_sh"])
    return float(np.sum((y + ys) * dy))


def check_backward_finite_differences(O, inp, K, align, n_coords=12, seed=5):
    fwd = O.forward(inp, K, align)
    bwd = O.backward(inp, fwd, inp["dy"])
    sel = fwd["route"]["topk_idx"]
    dy = np.asarray(inp["dy"], np.float64)
    rng = np.random.default_rng(seed)
    base = {k: np.asarray(v, np.float64) for k, v in inp.items()}
    for name, gname in (("x", "dx"), ("w1", "dW1"), ("w2", "dW2"), ("w_router", "dW_r"),
                        ("w1_sh", "dW1_sh"), ("w2_sh", "dW2_sh")):
        arr = base[name]
        grad = np.asarray(bwd[gname], np.float64)
        for _ in range(n_coords):
            idx = tuple(int(rng.integers(0, d)) for d in arr.shape)
            h = 1e-5
            p = dict(base)
            p[name] = arr.copy()
            p[name][idx] += h
            lp = frozen_loss(O, p, sel, dy)
            p[name][idx] -= 2 * h
            lm = frozen_loss(O, p, sel, dy)
            fd = (lp - lm) / (2 * h)
            scale = max(1.0, float(np.abs(grad).max()))
            assert abs(fd - grad[idx]) <= 1e-5 * scale, (name, idx, fd, grad[idx])


# ---------------------------------------------------------------------------
# Load balancing
# ---------------------------------------------------------------------------
def check_bias_update_golden(O):
    for c in load_golden("balance_small.json")["bias_update"]:
        got = O.bias_update(np.array(c["bias"], np.float32), np.array(c["counts"], np.int32),
                            c["gamma"])
        assert got.dtype == np.float32
        assert np.array_equal(got, np.array(c["new_bias"], np.float32)), (c["name"], got)


def check_bias_update_invariants(O, seed=7):
    """Each bias moves by exactly +-gamma (to fp32 rounding) or not at all,
    against the sign of its load's excess over the mean (computed in fp64)."""
    rng = np.random.default_rng(seed)
    for E in (1, 2, 8, 128):
        counts = rng.integers(0, 50, E)
        if E > 2:
            counts[0] = counts[1:].sum() // (E - 1)  # some experts near the mean
        bias = rng.standard_normal(E).astype(np.float32)
        gamma = np.float32(1e-3)
        new = O.bias_update(bias, counts, gamma)
        step = new.astype(np.float64) - bias.astype(np.float64)
        excess = counts - counts.sum() / E
        for e in range(E):
            if excess[e] == 0:
                assert step[e] == 0.0
            else:
                assert -np.sign(excess[e]) * step[e] > 0.5 * gamma
                assert abs(abs(step[e]) - gamma) <= 1e-6 * max(1.0, abs(bias[e]))


def check_bias_update_balances_router(O, steps=60):
    """The rule's purpose: on a router whose bias strongly favours a few
    experts, repeated (route, count, update) steps spread the load."""
    rng = np.random.default_rng(21)
    T, H, E, K = 256, 16, 8, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((H, E)) * 0.1).astype(np.float32)
    bias = np.linspace(0.4, -0.4, E).astype(np.float32)

    def imbalance(b):
        idx = O.route(x, w, b, K)["topk_idx"]
        counts = np.bincount(idx.ravel(), minlength=E)
        return counts, counts.max() / (T * K / E)

    counts, start = imbalance(bias)
    for _ in range(steps):
        bias = O.bias_update(bias, counts, 0.02)
        counts, now = imbalance(bias)
    assert start > 3.0 and now < 1.5, (start, now)


def seq_loss_bruteforce(scores, topk_idx, seq_len, alpha):
    """Plain loops: per sequence and expert, the fraction of picks scaled by
    E/K, times the mean normalised score; averaged over sequences."""
    T, E = len(scores), len(scores[0])
    K = len(topk_idx[0])
    per_seq = []
    for b in range(T // seq_len):
        toks = range(b * seq_len, (b + 1) * seq_len)
        total = []
        for i in range(E):
            picks = sum(1 for t in toks if i in list(topk_idx[t]))
            f = E * picks / (K * seq_len)
            P = math.fsum(scores[t][i] / math.fsum(scores[t]) for t in toks) / seq_len
            total.append(f * P)
        per_seq.append(alpha * math.fsum(total))
    return math.fsum(per_seq) / len(per_seq)


def check_seq_loss_golden(O):
    for c in load_golden("balance_small.json")["seq_loss"]:
        got = O.seq_balance_loss(np.array(c["scores"], np.float32),
                                 np.array(c["topk_idx"], np.int32), c["seq_len"], c["alpha"])
        assert abs(got - c["loss"]) <= 1e-6 * abs(c["loss"]), (c["name"], got)


def check_seq_loss_closed_forms(O, seed=9):
    rng = np.random.default_rng(seed)
    T, E, K, L, alpha = 24, 8, 2, 6, 0.3
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    s = rng.uniform(0.05, 0.95, (T, E)).astype(np.float32)
    # every expert scored alike: P_i = 1/E, sum_i f_i = E, loss = alpha
    flat = np.full((T, E), 0.37, np.float32)
    assert abs(O.seq_balance_loss(flat, idx, L, alpha) - alpha) < 1e-9
    # every sequence picks each expert equally often: f_i = 1, loss = alpha
    bal = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], np.int32)
    assert abs(O.seq_balance_loss(s, bal, 4, alpha) - alpha) < 1e-9
    # collapsed: all tokens pick experts 0..K-1 and score only them
    col = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    sc = np.zeros((T, E), np.float32)
    sc[:, :K] = 0.6
    assert abs(O.seq_balance_loss(sc, col, L, alpha) - alpha * E / K) < 1e-9
    # plain-loop evaluation on random scores and picks
    ref = seq_loss_bruteforce(s.astype(np.float64).tolist(), idx.tolist(), L, alpha)
    assert abs(O.seq_balance_loss(s, idx, L, alpha) - ref) <= 1e-12 * abs(ref)


def check_seq_loss_finite_differences(O, seed=13, n_coords=24):
    """dlogit from seq_balance_bwd against central differences of the loss,
    with the selection held fixed, on the fp64 scores of perturbed logits."""
    rng = np.random.default_rng(seed)
    T, E, K, L, alpha, dloss = 12, 6, 2, 4, 0.7, 1.3
    logits = rng.standard_normal((T, E))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)

    def loss(lg):
        return dloss * O.seq_balance_loss(1.0 / (1.0 + np.exp(-lg)), idx, L, alpha)

    got = O.seq_balance_bwd(1.0 / (1.0 + np.exp(-logits)), idx, L, alpha, dloss)
    h = 1e-6
    for _ in range(n_coords):
        t, e = rng.integers(T), rng.integers(E)
        p, m = logits.copy(), logits.copy()
        p[t, e] += h
        m[t, e] -= h
        fd = (loss(p) - loss(m)) / (2 * h)
        assert abs(got[t, e] - fd) <= 1e-6 * max(1e-3, abs(fd)), (t, e, got[t, e], fd)


def check_router_bwd_dense(O, seed=17):
    """The dense router backward reproduces the sparse one on its own
    (sparse) logit gradient, and is the gradient of sum((x W) * dlogit)."""
    inp, K = small_inputs(seed=seed)
    x, w = inp["x"], inp["w_router"]
    r = O.route(x, w, inp["bias"], K)
    dg = np.random.default_rng(seed).standard_normal(r["topk_idx"].shape)
    dW, dx, dl = O.router_bwd(x, w, r["topk_idx"], r["topk_s"], dg)
    dW2, dx2 = O.router_bwd_dense(x, w, dl)
    assert np.allclose(dW, dW2, rtol=1e-12, atol=1e-12)
    assert np.allclose(dx, dx2, rtol=1e-12, atol=1e-12)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    for (h_, e_) in ((0, 0), (3, 5), (15, 2)):
        d = np.zeros_like(w64)
        d[h_, e_] = 1e-3
        fd = (np.sum((x64 @ (w64 + d)) * dl) - np.sum((x64 @ (w64 - d)) * dl)) / 2e-3
        assert abs(dW2[h_, e_] - fd) <= 1e-9 * max(1.0, abs(fd))
    for (t_, h_) in ((0, 0), (7, 9)):
        d = np.zeros_like(x64)
        d[t_, h_] = 1e-3
        fd = (np.sum(((x64 + d) @ w64) * dl) - np.sum(((x64 - d) @ w64) * dl)) / 2e-3
        assert abs(dx2[t_, h_] - fd) <= 1e-9 * max(1.0, abs(fd))
