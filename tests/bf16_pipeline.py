"""Exact arithmetic with bf16 stores: what storing the layer's intermediates in
bf16 costs, independent of any kernel (test infrastructure).

The HIP path keeps fp32 accumulators and rounds to bf16 (round to nearest
even) wherever it stores a tensor: act, h, y_rows, the shared outputs, y,
dy_rows, dact, dx_rows, the shared input gradient, dx and the expert weight
gradients.  This module evaluates the same layer with every product and sum
exact (fp64) and only those stores rounded, first to fp32 (the accumulator)
and then to bf16.  Its distance from the fp64 oracle is the error that
bf16 storage alone causes; a kernel's own error is its distance from this
pipeline.

The rounding function is a parameter: with `rnd=identity` the pipeline is the
oracle's arithmetic (tests/test_bf16_storage_bound.py checks that), so the
only thing this module adds is where the rounding happens.

Stores follow the layer's data flow (which values feed which product):
  forward   a = x W1^T;  act = r(a);  h = r(silu(a_gate) a_up)   (from the
            unrounded a: the epilogue holds the fp32 accumulators);
            y_rows = r(h W2^T);  shared experts fused, same stores;
            y = r(y_sh + sum_k g_k y_rows[row_of[t,k]])
  backward  dy_rows = r(g dy);  dg = <dy, y_rows>;
            dh = dy_rows W2;  dact = r(SwiGLU-backward(dh, act))  (act as
            stored);  dx_rows = r(dact W1);  dW2 = r(dy_rows^T h);
            dW1 = r(dact^T x_rows);  shared: the same with dy for dy_rows;
            router gradients fp32 from dg;  dx = r(sum of every dx path)
"""
from __future__ import annotations

import numpy as np

from fine_grained_moe_amd.synthetic import bf16_round
from oracle import moe_oracle as O

F64 = np.float64


def bf16_store(a):
    """fp64 value -> fp32 accumulator -> bf16 store (RNE), returned in fp64."""
    return bf16_round(np.asarray(a, np.float32)).astype(F64)


def no_store(a):
    return np.asarray(a, F64)


def _sig(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def expert_forward(x_rows, w1e, w2e, rnd=bf16_store):
    """(act, h, y) of one SwiGLU expert on a block of rows, as stored."""
    x = np.asarray(x_rows, F64)
    w1 = np.asarray(w1e, F64)
    w2 = np.asarray(w2e, F64)
    F = w1.shape[0] // 2
    a = x @ w1.T
    g, u = a[:, :F], a[:, F:]
    h = rnd(g * _sig(g) * u)
    return rnd(a), h, rnd(h @ w2.T)


def expert_backward(x_rows, w1e, w2e, act, h, dy_rows, rnd=bf16_store):
    """(dx_rows, dW1, dW2, dact) of one expert from its stored act/h and the
    stored upstream rows."""
    x = np.asarray(x_rows, F64)
    w1 = np.asarray(w1e, F64)
    w2 = np.asarray(w2e, F64)
    dy = np.asarray(dy_rows, F64)
    F = w1.shape[0] // 2
    gate, up = act[:, :F], act[:, F:]
    sg = _sig(gate)
    dh = dy @ w2
    dact = rnd(np.concatenate([dh * up * (sg * (1.0 + gate * (1.0 - sg))), dh * gate * sg], 1))
    return rnd(dact @ w1), rnd(dact.T @ x), rnd(dy.T @ h), dact


def fuse_shared(w1_sh, w2_sh):
    """The S shared experts as one expert of width S*F (gate blocks, then up
    blocks; down matrices side by side): the layout the HIP path computes the
    shared experts in, which fixes what one stored act/h row holds."""
    S, twoF, H = w1_sh.shape
    F = twoF // 2
    w1 = np.concatenate([w1_sh[:, :F].reshape(S * F, H), w1_sh[:, F:].reshape(S * F, H)], 0)
    w2 = np.concatenate([w2_sh[s] for s in range(S)], 1)
    return w1, w2


def layer(inp, K, align, dy=None, rnd=bf16_store, route=None, router_extra=None):
    """Forward (and backward when dy is given) of the layer with bf16 stores.

    Routing is the oracle's fp32 routing unless `route` (a dict with
    topk_idx, topk_w, topk_s, as the oracle's route returns) is given: the
    HIP path's own routing, so that a near-tie token does not move segments.
    router_extra = (dW_r, dx_r): router gradients of another loss (the
    sequence-wise balance loss), added to the combine path's in fp32 before
    dx is summed and stored.  Returns a dict of the stored tensors (fp64
    arrays holding bf16 or fp32 values)."""
    x = np.asarray(inp["x"], F64)
    T, H = x.shape
    E = inp["w1"].shape[0]
    S = inp["w1_sh"].shape[0]
    r = O.route(inp["x"], inp["w_router"], inp["bias"], K) if route is None else route
    idx = np.asarray(r["topk_idx"])
    g = np.asarray(r["topk_w"], F64)
    p = O.permute(idx, E, align)
    n_rows = int(p["offsets"][E])
    x_rows = np.zeros((n_rows, H), F64)
    valid = p["src_token"] >= 0
    x_rows[valid] = x[p["src_token"][valid]]
    twoF = inp["w1"].shape[1]
    act = np.zeros((n_rows, twoF), F64)
    hid = np.zeros((n_rows, twoF // 2), F64)
    y_rows = np.zeros((n_rows, H), F64)
    for e in range(E):
        r0, n = int(p["offsets"][e]), int(p["counts"][e])
        if n:
            sl = slice(r0, r0 + n)
            act[sl], hid[sl], y_rows[sl] = expert_forward(x_rows[sl], inp["w1"][e], inp["w2"][e], rnd)
    out = dict(route=r, perm=p, x_rows=x_rows, act=act, h=hid, y_rows=y_rows)
    y = np.zeros((T, H), F64)
    if S:
        w1f, w2f = fuse_shared(np.asarray(inp["w1_sh"]), np.asarray(inp["w2_sh"]))
        act_sh, h_sh, y_sh = expert_forward(x, w1f, w2f, rnd)
        out.update(act_sh=act_sh, h_sh=h_sh, y_shared=y_sh, w1f=w1f, w2f=w2f)
        y = y + y_sh
    for k in range(K):
        y = y + g[:, k:k + 1] * y_rows[p["row_of"][:, k]]
    out["y"] = rnd(y)
    if dy is None:
        return out

    dy = np.asarray(dy, F64)
    dy_rows = np.zeros((n_rows, H), F64)
    dg = np.zeros((T, K), F64)
    for k in range(K):
        rows = p["row_of"][:, k]
        dy_rows[rows] = rnd(g[:, k:k + 1] * dy)
        dg[:, k] = np.einsum("th,th->t", dy, y_rows[rows])
    dg = dg.astype(np.float32).astype(F64)
    dx_rows = np.zeros((n_rows, H), F64)
    dact = np.zeros((n_rows, twoF), F64)
    dW1 = np.zeros(inp["w1"].shape, np.float32)
    dW2 = np.zeros(inp["w2"].shape, np.float32)
    for e in range(E):
        r0, n = int(p["offsets"][e]), int(p["counts"][e])
        if n:
            sl = slice(r0, r0 + n)
            dx_rows[sl], dW1[e], dW2[e], dact[sl] = expert_backward(
                x_rows[sl], inp["w1"][e], inp["w2"][e], act[sl], hid[sl], dy_rows[sl], rnd)
    dx = np.zeros((T, H), F64)
    for k in range(K):
        dx = dx + dx_rows[p["row_of"][:, k]]
    out.update(dy_rows=dy_rows, dg=dg, dx_rows=dx_rows, dact=dact, dW1=dW1, dW2=dW2)
    if S:
        dx_sh, dW1f, dW2f, dact_sh = expert_backward(x, out["w1f"], out["w2f"], out["act_sh"],
                                                     out["h_sh"], dy, rnd)
        F = twoF // 2
        out.update(dx_shared=dx_sh, dact_sh=dact_sh,
                   dW1_sh=np.stack([np.concatenate([dW1f[s * F:(s + 1) * F],
                                                    dW1f[S * F + s * F:S * F + (s + 1) * F]])
                                    for s in range(S)]),
                   dW2_sh=np.stack([dW2f[:, s * F:(s + 1) * F] for s in range(S)]))
        dx = dx + dx_sh
    dW_r, dx_r, _ = O.router_bwd(inp["x"], inp["w_router"], idx, r["topk_s"], dg)
    if router_extra is not None:
        dW_r = dW_r + router_extra[0]
        dx_r = dx_r + router_extra[1]
    dW_r = dW_r.astype(np.float32).astype(F64)
    dx_r = dx_r.astype(np.float32).astype(F64)
    out.update(dW_r=dW_r, dx_router=dx_r, dx=rnd(dx + dx_r))
    return out
