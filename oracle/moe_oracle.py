"""CPU oracle for the dots.llm1 fine-grained MoE FFN layer (forward and backward).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The HIP library never calls
it, and it shares no code with the HIP library: the two meet only in the
seeded input arrays the generator module draws.

It is the plain, slow definition of what the layer computes, step by step, in
fp64 arithmetic on fp32 (or bf16-exact) inputs, one library matmul per
product.  Sources for each step are the dots.llm1 pages:

  [TR]    "dots.llm1 Technical Report" summary page, sections "Key claims" and
          "Method": 128 routed experts, top-6 plus 2 always-on shared experts,
          SwiGLU experts, FP32 gating, DeepSeek-style auxiliary-loss-free
          balancing by a bias, no token dropping, expert token segments padded
          to GEMM tile multiples.
  [CARD]  "dots.llm1: the first MoE large language model open-sourced by Little
          Red Book", section "Model Architecture Features": 6 routed + 2 shared
          experts per token, SwiGLU, load balancing through dynamic bias terms.
  [NEWS]  aibase news item on dots.llm1, architecture paragraph: each expert is
          a two-layer feed-forward network with SwiGLU.
  [SPEC]  "How dots.llm1's 14B MoE Architecture Matches 72B LLM Performance",
          section "MoE Architecture Specifications": 128 / 6 / 2 / hidden 5120.

Readings taken where the pages leave a step open (each is stated again on the
function that takes it):

  R1  score function: sigmoid of the fp32 logit (the DeepSeek aux-loss-free
      formulation the pages name); the bias enters the selection key only.
  R2  combine weights: the K selected scores normalised to sum to one; no
      extra scale; the bias is not part of the weight.
  R3  shared experts are added with weight 1.
  R4  top-K ties go to the lower expert index; NaN keys rank below everything.
  R5  within a token, the K experts are listed by key descending, then index.
  R6  rows of one expert segment are its tokens in ascending token order.
  R7  the backward is the true gradient with the routing decision held fixed;
      the selection bias receives no gradient; dx includes the router path.
  R8  an expert with no tokens owns no rows (not a padding tile); the segment
      of expert e starts at the sum of its predecessors' counts, each rounded
      up to the alignment.
  R9  no capacity limit: every token keeps all K of its experts.
  R10 experts have no linear biases; gate is the first F rows of W1, and the
      hidden activation is silu(gate) * up.
  R11 bias update (the auxiliary-loss-free balancing step; the pages name
      DeepSeek's bias-update trick but give neither rule nor rate): DeepSeek's
      published sign rule, bias[e] += gamma * sign(mean load - load[e]) over
      the per-expert token counts of a batch; an expert exactly at the mean
      keeps its bias.
  R12 sequence-wise balance loss (named on the pages as the complement of the
      bias update, not defined there): DeepSeek-V3's complementary
      sequence-wise auxiliary loss.  For a sequence of L tokens,
      s'[t,i] = s[t,i] / sum_j s[t,j] over all E experts, P_i = mean_t s'[t,i],
      f_i = E / (K L) * #{t : i selected by t}, loss = alpha * sum_i f_i P_i.
      A batch of T = B L tokens holds B consecutive sequences; its loss is the
      mean over them.  The selection is held fixed in the gradient (R7), so
      the loss reaches the logits through all E scores of each token.

Precision: products and sums in fp64; values that the method defines as fp32
(logit, score, key, combine weight) are rounded to fp32 where they are
defined, so that the fp32 routing decision is taken on fp32 keys on both sides.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
F32 = np.float32

# relative gap on the fp32 selection key between the K-th and (K+1)-th expert
# below which a token's routing is counted as a near-tie
NEAR_TIE_REL = 1e-6


# ---------------------------------------------------------------------------
# Routing ([TR] "Method": FP32 gating, aux-loss-free bias, top-6 of 128)
# ---------------------------------------------------------------------------
def router_logits(x, w_router):
    """logit[t,e] = sum_h x[t,h] * W_r[h,e]; fp64 sum, rounded once to fp32.

    [TR] "Method": the gating projection is computed in FP32.  W_r is [H, E].
    """
    return (np.asarray(x, F64) @ np.asarray(w_router, F64)).astype(F32)


def sigmoid64(z):
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def router_scores(logits):
    """s = sigmoid(logit), evaluated in fp64 on the fp32 logit, rounded to fp32 (R1)."""
    return sigmoid64(logits).astype(F32)


def selection_keys(scores, bias):
    """v[t,e] = s[t,e] + b[e], one fp32 addition ([CARD] dynamic bias terms; R1)."""
    return (np.asarray(scores, F32) + np.asarray(bias, F32)[None, :]).astype(F32)


def top_k(keys, K):
    """Indices of the K largest keys of each token, ordered key-descending then
    index-ascending (R4, R5).  NaN keys rank as -inf."""
    v = np.asarray(keys, F64)
    v = np.where(np.isnan(v), -np.inf, v)
    order = np.argsort(-v, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def combine_weights(scores, topk_idx):
    """g[t,k] = s[t,sel_k] / sum_j s[t,sel_j]; fp64 sum, rounded to fp32 (R2)."""
    sel = np.take_along_axis(np.asarray(scores, F64), topk_idx.astype(np.int64), axis=1)
    return (sel / sel.sum(axis=1, keepdims=True)).astype(F32)


def near_tie_mask(keys, K):
    """Tokens whose K-th and (K+1)-th largest fp32 keys differ by less than
    NEAR_TIE_REL relative to the K-th: their selection may legitimately differ
    between two correct fp32 evaluations of the logits."""
    v = np.asarray(keys, F64)
    E = v.shape[1]
    if K >= E:
        return np.zeros(v.shape[0], bool)
    v = np.where(np.isnan(v), -np.inf, v)
    srt = -np.sort(-v, axis=1)
    vk, vk1 = srt[:, K - 1], srt[:, K]
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = (vk - vk1) / np.abs(vk)
    return rel < NEAR_TIE_REL


def order_tie_mask(keys, K):
    """Tokens with two adjacent ranks among their K selected keys closer than
    NEAR_TIE_REL relative: the order of those two experts in the token's list
    may legitimately differ between two correct fp32 evaluations."""
    v = np.asarray(keys, F64)
    v = np.where(np.isnan(v), -np.inf, v)
    srt = -np.sort(-v, axis=1)[:, :K]
    if K < 2:
        return np.zeros(v.shape[0], bool)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = (srt[:, :-1] - srt[:, 1:]) / np.abs(srt[:, :-1])
    return np.any(rel < NEAR_TIE_REL, axis=1)


def route(x, w_router, bias, K):
    """Whole routing step: logits, scores, keys, top-K, combine weights."""
    logits = router_logits(x, w_router)
    s = router_scores(logits)
    v = selection_keys(s, bias)
    idx = top_k(v, K)
    return dict(logits=logits, scores=s, keys=v, topk_idx=idx,
                topk_w=combine_weights(s, idx),
                topk_s=np.take_along_axis(s, idx.astype(np.int64), axis=1),
                near_tie=near_tie_mask(v, K), order_tie=order_tie_mask(v, K))


# ---------------------------------------------------------------------------
# Permutation into padded expert segments ([TR] "Key claims" / "Method":
# expert token segments padded to the GEMM tile multiple; no token dropped)
# ---------------------------------------------------------------------------
def permute(topk_idx, E, align):
    """Expert segments, padded to `align` rows (R6, R8, R9).

    counts[e]     number of tokens that selected e
    offsets[e]    first row of e's segment; offsets[e+1]-offsets[e] is counts[e]
                  rounded up to a multiple of align; offsets[E] is the total
    row_of[t,k]   row that holds token t's copy for its k-th expert
    src_token[r]  token whose copy sits in row r, -1 for a padding row
    """
    T, K = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    padded = (counts + align - 1) // align * align
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(padded)
    # slots are numbered t*K+k; a stable sort by expert keeps ascending t
    # inside each expert because a token selects an expert at most once
    order = np.argsort(flat, kind="stable")
    starts = np.zeros(E + 1, np.int64)
    starts[1:] = np.cumsum(counts)
    rank = np.empty(T * K, np.int64)
    rank[order] = np.arange(T * K) - starts[flat[order]]
    row_of = (offsets[flat] + rank).reshape(T, K)
    src_token = np.full(int(offsets[E]), -1, np.int64)
    src_token[row_of.reshape(-1)] = np.repeat(np.arange(T), K)
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                row_of=row_of.astype(np.int32), src_token=src_token.astype(np.int32))


# ---------------------------------------------------------------------------
# Experts ([NEWS]: two feed-forward layers with SwiGLU; R10)
# ---------------------------------------------------------------------------
def silu64(z):
    return z * sigmoid64(z)


def expert_ffn(x_rows, w1e, w2e):
    """One SwiGLU expert on a block of rows, fp64.

    a = x W1^T  ([rows, 2F]; gate = a[:, :F], up = a[:, F:])
    h = silu(gate) * up
    y = h W2^T  ([rows, H])
    Returns (a, h, y) in fp64.
    """
    x = np.asarray(x_rows, F64)
    w1 = np.asarray(w1e, F64)
    w2 = np.asarray(w2e, F64)
    F = w1.shape[0] // 2
    a = x @ w1.T
    h = silu64(a[:, :F]) * a[:, F:]
    y = h @ w2.T
    return a, h, y


def expert_ffn_bwd(x_rows, w1e, w2e, a, dy_rows):
    """Backward of expert_ffn (R7), fp64.  `a` is the forward's [gate|up].

    dh    = dy W2
    dW2   = dy^T h
    dgate = dh * up * silu'(gate),  silu'(z) = sig(z) * (1 + z * (1 - sig(z)))
    dup   = dh * silu(gate)
    dW1   = [dgate|dup]^T x
    dx    = [dgate|dup] W1
    Returns (dx, dW1, dW2, da) in fp64.
    """
    x = np.asarray(x_rows, F64)
    w1 = np.asarray(w1e, F64)
    w2 = np.asarray(w2e, F64)
    dy = np.asarray(dy_rows, F64)
    F = w1.shape[0] // 2
    gate, up = a[:, :F], a[:, F:]
    sg = sigmoid64(gate)
    h = gate * sg * up
    dh = dy @ w2
    dW2 = dy.T @ h
    dgate = dh * up * (sg * (1.0 + gate * (1.0 - sg)))
    dup = dh * (gate * sg)
    da = np.concatenate([dgate, dup], axis=1)
    return da @ w1, da.T @ x, dW2, da


def experts_forward(x_rows, w1, w2, offsets, counts):
    """Run every routed expert on the valid rows of its segment.

    x_rows is [M, H] (M >= offsets[E]); rows of e are offsets[e] ..
    offsets[e]+counts[e]-1.  Padding rows of the outputs are zero.
    Returns (act [M,2F], h [M,F], y [M,H]) in fp64.
    """
    M = x_rows.shape[0]
    E, twoF, H = w1.shape
    act = np.zeros((M, twoF), F64)
    hid = np.zeros((M, twoF // 2), F64)
    y = np.zeros((M, H), F64)
    for e in range(E):
        r0, n = int(offsets[e]), int(counts[e])
        if n == 0:
            continue
        a, h, ye = expert_ffn(x_rows[r0:r0 + n], w1[e], w2[e])
        act[r0:r0 + n], hid[r0:r0 + n], y[r0:r0 + n] = a, h, ye
    return act, hid, y


def shared_forward(x, w1_sh, w2_sh):
    """Sum of the always-on shared experts, each with weight 1 (R3).  fp64."""
    y = np.zeros((x.shape[0], w2_sh.shape[1]), F64)
    acts = []
    for s in range(w1_sh.shape[0]):
        a, _, ys = expert_ffn(x, w1_sh[s], w2_sh[s])
        acts.append(a)
        y += ys
    return y, acts


# ---------------------------------------------------------------------------
# Combine ([CARD]: 6 routed + 2 shared experts active per token)
# ---------------------------------------------------------------------------
def combine(y_rows, row_of, topk_w, y_shared=None):
    """y[t] = y_shared[t] + sum_k g[t,k] * y_rows[row_of[t,k]]  (fp64)."""
    T, K = row_of.shape
    y = np.zeros((T, y_rows.shape[1]), F64) if y_shared is None else np.array(y_shared, F64)
    g = np.asarray(topk_w, F64)
    for k in range(K):
        y += g[:, k:k + 1] * np.asarray(y_rows[row_of[:, k]], F64)
    return y


# ---------------------------------------------------------------------------
# Backward stages (R7)
# ---------------------------------------------------------------------------
def combine_bwd(dy, y_rows, row_of, topk_w, n_rows):
    """dy_rows[row_of[t,k]] = g[t,k] * dy[t];  dg[t,k] = <dy[t], y_rows[row_of[t,k]]>.

    Padding rows of dy_rows are zero.  Returns (dy_rows fp64 [n_rows,H], dg fp64 [T,K]).
    """
    T, K = row_of.shape
    dy64 = np.asarray(dy, F64)
    g = np.asarray(topk_w, F64)
    dy_rows = np.zeros((n_rows, dy64.shape[1]), F64)
    dg = np.zeros((T, K), F64)
    for k in range(K):
        r = row_of[:, k]
        dy_rows[r] = g[:, k:k + 1] * dy64
        dg[:, k] = np.einsum("th,th->t", dy64, np.asarray(y_rows[r], F64))
    return dy_rows, dg


def router_bwd(x, w_router, topk_idx, topk_s, dg):
    """Gradient through g = s_sel / sum(s_sel) and s = sigmoid(logit).

    ds_k     = (dg_k - sum_j g_j dg_j) / sum_j s_j
    dlogit_k = ds_k * s_k * (1 - s_k)   on the K selected experts, 0 elsewhere
    dW_r     = x^T dlogit   ([H, E]),   dx_r = dlogit W_r^T   ([T, H])
    Returns (dW_r, dx_r, dlogit) in fp64.
    """
    s = np.asarray(topk_s, F64)
    dg = np.asarray(dg, F64)
    tot = s.sum(axis=1, keepdims=True)
    g = s / tot
    ds = (dg - (g * dg).sum(axis=1, keepdims=True)) / tot
    dl_sel = ds * s * (1.0 - s)
    T, K = topk_idx.shape
    E = w_router.shape[1]
    dlogit = np.zeros((T, E), F64)
    np.put_along_axis(dlogit, topk_idx.astype(np.int64), dl_sel, axis=1)
    x64 = np.asarray(x, F64)
    return x64.T @ dlogit, dlogit @ np.asarray(w_router, F64).T, dlogit


def experts_backward(x_rows, w1, w2, act, dy_rows, offsets, counts):
    """Per-expert backward over the valid rows of each segment.

    Returns (dx_rows [M,H], dW1 [E,2F,H], dW2 [E,H,F], dact [M,2F]); experts with
    no rows get exactly-zero weight gradients.  dW are fp32 (rounded once from
    the fp64 sums) to bound memory at full size; dx_rows and dact are fp64.
    """
    M = x_rows.shape[0]
    E, twoF, H = w1.shape
    dx_rows = np.zeros((M, H), F64)
    dact = np.zeros((M, twoF), F64)
    dW1 = np.zeros((E, twoF, H), F32)
    dW2 = np.zeros((E, H, twoF // 2), F32)
    for e in range(E):
        r0, n = int(offsets[e]), int(counts[e])
        if n == 0:
            continue
        sl = slice(r0, r0 + n)
        dxe, dw1e, dw2e, dae = expert_ffn_bwd(x_rows[sl], w1[e], w2[e], act[sl], dy_rows[sl])
        dx_rows[sl], dact[sl] = dxe, dae
        dW1[e], dW2[e] = dw1e, dw2e
    return dx_rows, dW1, dW2, dact


def unpermute_add(dx_rows, row_of, extra=()):
    """dx[t] = sum_k dx_rows[row_of[t,k]] + sum of the extra [T,H] terms (fp64)."""
    T, K = row_of.shape
    dx = np.zeros((T, dx_rows.shape[1]), F64)
    for k in range(K):
        dx += np.asarray(dx_rows[row_of[:, k]], F64)
    for e in extra:
        dx += np.asarray(e, F64)
    return dx


def router_bwd_dense(x, w_router, dlogit):
    """Router gradients of a dense logit gradient dlogit [T, E] (fp64):
    dW_r = x^T dlogit ([H, E]) and dx_r = dlogit W_r^T ([T, H])."""
    dl = np.asarray(dlogit, F64)
    return np.asarray(x, F64).T @ dl, dl @ np.asarray(w_router, F64).T


# ---------------------------------------------------------------------------
# Load balancing ([TR] "Method": DeepSeek's auxiliary-loss-free bias update,
# complemented by a sequence-wise balance loss; [CARD] "Model Architecture
# Features": load balancing through dynamic bias terms)
# ---------------------------------------------------------------------------
def bias_update(bias, counts, gamma):
    """One bias step from a batch's per-expert token counts (R11).

    An expert's load is compared with the mean load sum(counts)/E exactly, in
    integers (E * count against the total); the bias moves by gamma towards
    balance in one fp32 addition.  Returns the new fp32 bias.
    """
    c = np.asarray(counts, np.int64)
    E = c.shape[0]
    direction = np.sign(c.sum() - E * c).astype(F32)  # +1 below the mean, -1 above
    return (np.asarray(bias, F32) + direction * F32(gamma)).astype(F32)


def seq_balance_stats(scores, topk_idx, seq_len):
    """Per-sequence f [B, E] and P [B, E] of the sequence-wise balance loss (R12)."""
    s = np.asarray(scores, F64)
    T, E = s.shape
    K = topk_idx.shape[1]
    B = T // seq_len
    s_norm = s / s.sum(axis=1, keepdims=True)
    P = s_norm.reshape(B, seq_len, E).mean(axis=1)
    picked = np.zeros((T, E), F64)
    np.put_along_axis(picked, topk_idx.astype(np.int64), 1.0, axis=1)
    f = picked.reshape(B, seq_len, E).sum(axis=1) * (E / (K * seq_len))
    return f, P


def seq_balance_loss(scores, topk_idx, seq_len, alpha):
    """loss = mean over the B sequences of alpha * sum_i f_i P_i (R12); fp64."""
    f, P = seq_balance_stats(scores, topk_idx, seq_len)
    return float(alpha * (f * P).sum(axis=1).mean())


def seq_balance_bwd(scores, topk_idx, seq_len, alpha, dloss=1.0):
    """Gradient of dloss * loss with respect to the logits, dense [T, E] (fp64).

    With c_i = dloss * alpha * f_i / (B L) for the token's sequence,
    dL/ds'[t,i] = c_i; through s' = s / sum(s):
      ds[t,j]     = (c_j - sum_i c_i s'[t,i]) / sum_i s[t,i]
    and through s = sigmoid(logit): dlogit = ds * s * (1 - s).
    """
    s = np.asarray(scores, F64)
    T, E = s.shape
    B = T // seq_len
    f, _ = seq_balance_stats(scores, topk_idx, seq_len)
    c = np.repeat(f * (dloss * alpha / (B * seq_len)), seq_len, axis=0)
    tot = s.sum(axis=1, keepdims=True)
    ds = (c - (c * (s / tot)).sum(axis=1, keepdims=True)) / tot
    return ds * s * (1.0 - s)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def forward(inp, K, align):
    """Forward of the layer on the generator's input dict.

    Returns every stage: routing, segments, x_rows, act/h/y_rows, shared
    output and y (fp64 unless noted by the stage).
    """
    x = inp["x"]
    E = inp["w1"].shape[0]
    r = route(x, inp["w_router"], inp["bias"], K)
    p = permute(r["topk_idx"], E, align)
    n_rows = int(p["offsets"][E])
    x_rows = np.zeros((n_rows, x.shape[1]), F32)
    valid = p["src_token"] >= 0
    x_rows[valid] = x[p["src_token"][valid]]
    act, hid, y_rows = experts_forward(x_rows, inp["w1"], inp["w2"], p["offsets"], p["counts"])
    y_sh, act_sh = shared_forward(x, inp["w1_sh"], inp["w2_sh"])
    y = combine(y_rows, p["row_of"], r["topk_w"], y_sh)
    return dict(route=r, perm=p, x_rows=x_rows, act=act, h=hid, y_rows=y_rows,
                y_shared=y_sh, act_shared=act_sh, y=y)


def backward(inp, fwd, dy):
    """Backward of the layer (R7) given the forward's stages and dY [T,H].

    Returns dx [T,H], dW1, dW2, dW1_sh, dW2_sh, dW_r [H,E], and the
    intermediates dg, dy_rows, dact, dx_rows, dx_shared, dx_router.
    """
    x = inp["x"]
    r, p = fwd["route"], fwd["perm"]
    n_rows = fwd["x_rows"].shape[0]
    dy_rows, dg = combine_bwd(dy, fwd["y_rows"], p["row_of"], r["topk_w"], n_rows)
    dx_rows, dW1, dW2, dact = experts_backward(fwd["x_rows"], inp["w1"], inp["w2"], fwd["act"],
                                               dy_rows, p["offsets"], p["counts"])
    S = inp["w1_sh"].shape[0]
    dx_sh = np.zeros(x.shape, F64)
    dW1_sh = np.zeros(inp["w1_sh"].shape, F32)
    dW2_sh = np.zeros(inp["w2_sh"].shape, F32)
    for s in range(S):
        dxs, dw1s, dw2s, _ = expert_ffn_bwd(x, inp["w1_sh"][s], inp["w2_sh"][s],
                                            fwd["act_shared"][s], dy)
        dx_sh += dxs
        dW1_sh[s], dW2_sh[s] = dw1s, dw2s
    dW_r, dx_r, dlogit = router_bwd(x, inp["w_router"], r["topk_idx"], r["topk_s"], dg)
    dx = unpermute_add(dx_rows, p["row_of"], (dx_sh, dx_r))
    return dict(dx=dx, dW1=dW1, dW2=dW2, dW1_sh=dW1_sh, dW2_sh=dW2_sh, dW_r=dW_r,
                dg=dg, dy_rows=dy_rows, dact=dact, dx_rows=dx_rows,
                dx_shared=dx_sh, dx_router=dx_r, dlogit=dlogit)
