"""Plant plausible mistakes in the CPU oracle and require a pin to catch each.

The mistakes are planted in the oracle (on the CPU), never in GPU code.  Each
mutation replaces one oracle function for the duration of a test; the pins
(tests/oracle_pins.py) then run against the mutated oracle and at least one of
them must raise AssertionError.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
import oracle_pins as P

F64 = np.float64
_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _all_pins():
    inp, K = P.small_inputs()
    return [
        lambda: P.check_logits_exact_sum(O, inp["x"], inp["w_router"]),
        lambda: P.check_sigmoid_closed_form(O),
        lambda: P.check_route_golden(O),
        lambda: P.check_topk_bruteforce(O, O.route(inp["x"], inp["w_router"], inp["bias"], K)["keys"], K),
        lambda: P.check_combine_weight_invariants(O, inp["x"], inp["w_router"], inp["bias"], K),
        lambda: P.check_permute_golden(O),
        lambda: P.check_forward_bruteforce(O, inp, K, 4),
        lambda: P.check_one_expert_is_dense_swiglu(O),
        lambda: P.check_identical_experts_independent_of_routing(O, inp, K, 4),
        lambda: P.check_backward_autograd(O, inp, K, 4),
        lambda: P.check_bias_update_golden(O),
        lambda: P.check_bias_update_balances_router(O),
        lambda: P.check_seq_loss_golden(O),
        lambda: P.check_seq_loss_closed_forms(O),
        lambda: P.check_seq_loss_finite_differences(O),
        lambda: P.check_router_bwd_dense(O),
    ]


def _caught():
    fired = []
    for i, pin in enumerate(_all_pins()):
        try:
            pin()
        except AssertionError:
            fired.append(i)
    return fired


# --- mutations -------------------------------------------------------------
def m_logits_drop_last_term(x, w):
    return (np.asarray(x, F64)[:, :-1] @ np.asarray(w, F64)[:-1]).astype(np.float32)


def m_sigmoid_wrong_sign(z):
    return 1.0 / (1.0 + np.exp(np.asarray(z, F64)))


def m_keys_without_bias(s, b):
    return np.asarray(s, np.float32)


def m_topk_ties_to_higher_index(keys, K):
    v = np.asarray(keys, F64)[:, ::-1]
    order = np.argsort(-v, axis=1, kind="stable")
    return (v.shape[1] - 1 - order[:, :K]).astype(np.int32)


def m_weights_unnormalised(s, idx):
    return np.take_along_axis(np.asarray(s, np.float32), idx.astype(np.int64), axis=1)


def m_weights_from_keys(s, idx):
    # uses s + 0.3 as if the bias were in the weight
    sel = np.take_along_axis(np.asarray(s, F64) + 0.3, idx.astype(np.int64), axis=1)
    return (sel / sel.sum(1, keepdims=True)).astype(np.float32)


def m_permute_no_padding(topk_idx, E, align):
    return _orig["permute"](topk_idx, E, 1)


def m_permute_descending_tokens(topk_idx, E, align):
    p = _orig["permute"](topk_idx, E, align)
    row_of, src = p["row_of"].copy(), p["src_token"].copy()
    off, cnt = p["offsets"], p["counts"]
    for e in range(E):
        a, n = int(off[e]), int(cnt[e])
        src[a:a + n] = src[a:a + n][::-1].copy()
    T, K = row_of.shape
    for r in range(len(src)):
        t = src[r]
        if t >= 0:
            k = int(np.nonzero(topk_idx[t] == np.searchsorted(off, r, side="right") - 1)[0][0])
            row_of[t, k] = r
    return dict(p, row_of=row_of, src_token=src)


def m_swiglu_gate_up_swapped(x_rows, w1e, w2e):
    x = np.asarray(x_rows, F64)
    F = w1e.shape[0] // 2
    a = x @ np.asarray(w1e, F64).T
    h = O.silu64(a[:, F:]) * a[:, :F]
    return a, h, h @ np.asarray(w2e, F64).T


def m_swiglu_no_sigmoid(x_rows, w1e, w2e):
    x = np.asarray(x_rows, F64)
    F = w1e.shape[0] // 2
    a = x @ np.asarray(w1e, F64).T
    h = a[:, :F] * a[:, F:]
    return a, h, h @ np.asarray(w2e, F64).T


def m_combine_drops_shared(y_rows, row_of, topk_w, y_shared=None):
    return _orig["combine"](y_rows, row_of, topk_w, None)


def m_silu_grad_missing_term(x_rows, w1e, w2e, a, dy_rows):
    x, w1, w2, dy = (np.asarray(v, F64) for v in (x_rows, w1e, w2e, dy_rows))
    F = w1.shape[0] // 2
    gate, up = a[:, :F], a[:, F:]
    sg = O.sigmoid64(gate)
    h = gate * sg * up
    dh = dy @ w2
    da = np.concatenate([dh * up * sg, dh * gate * sg], axis=1)
    return da @ w1, da.T @ x, dy.T @ h, da


def m_router_bwd_sign(x, w_router, topk_idx, topk_s, dg):
    return _orig["router_bwd"](x, w_router, topk_idx, topk_s, -np.asarray(dg))


def m_router_bwd_no_dx(x, w_router, topk_idx, topk_s, dg):
    dW, dx, dl = _orig["router_bwd"](x, w_router, topk_idx, topk_s, dg)
    return dW, np.zeros_like(dx), dl


def m_dW2_transposed_rows(x_rows, w1e, w2e, a, dy_rows):
    dx, dW1, dW2, da = _orig["expert_ffn_bwd"](x_rows, w1e, w2e, a, dy_rows)
    return dx, dW1, dW2[::-1].copy(), da


def m_bias_update_sign_flipped(bias, counts, gamma):
    return _orig["bias_update"](bias, counts, -gamma)


def m_bias_update_moves_at_mean(bias, counts, gamma):
    c = np.asarray(counts, np.int64)
    d = np.where(c * len(c) >= c.sum(), -1.0, 1.0).astype(np.float32)
    return (np.asarray(bias, np.float32) + d * np.float32(gamma)).astype(np.float32)


def m_seq_loss_sum_over_sequences(scores, topk_idx, seq_len, alpha):
    B = len(scores) // seq_len
    return B * _orig["seq_balance_loss"](scores, topk_idx, seq_len, alpha)


def m_seq_stats_without_e_over_k(scores, topk_idx, seq_len):
    f, P = _orig["seq_balance_stats"](scores, topk_idx, seq_len)
    E, K = np.asarray(scores).shape[1], topk_idx.shape[1]
    return f * K / E, P


def m_seq_bwd_no_normalisation_term(scores, topk_idx, seq_len, alpha, dloss=1.0):
    s = np.asarray(scores, F64)
    B = s.shape[0] // seq_len
    f, _ = O.seq_balance_stats(scores, topk_idx, seq_len)
    c = np.repeat(f * (dloss * alpha / (B * seq_len)), seq_len, axis=0)
    return c / s.sum(axis=1, keepdims=True) * s * (1.0 - s)


def m_seq_bwd_no_sigmoid_grad(scores, topk_idx, seq_len, alpha, dloss=1.0):
    s = np.asarray(scores, F64)
    return _orig["seq_balance_bwd"](scores, topk_idx, seq_len, alpha, dloss) / (s * (1.0 - s))


def m_router_bwd_dense_drops_dx(x, w_router, dlogit):
    dW, dx = _orig["router_bwd_dense"](x, w_router, dlogit)
    return dW, 0.5 * dx


MUTATIONS = {
    "logits_drop_last_term": ("router_logits", m_logits_drop_last_term),
    "sigmoid_wrong_sign": ("sigmoid64", m_sigmoid_wrong_sign),
    "keys_without_bias": ("selection_keys", m_keys_without_bias),
    "topk_ties_to_higher_index": ("top_k", m_topk_ties_to_higher_index),
    "weights_unnormalised": ("combine_weights", m_weights_unnormalised),
    "weights_from_keys": ("combine_weights", m_weights_from_keys),
    "permute_no_padding": ("permute", m_permute_no_padding),
    "permute_descending_tokens": ("permute", m_permute_descending_tokens),
    "swiglu_gate_up_swapped": ("expert_ffn", m_swiglu_gate_up_swapped),
    "swiglu_no_sigmoid": ("expert_ffn", m_swiglu_no_sigmoid),
    "combine_drops_shared": ("combine", m_combine_drops_shared),
    "silu_grad_missing_term": ("expert_ffn_bwd", m_silu_grad_missing_term),
    "router_bwd_sign": ("router_bwd", m_router_bwd_sign),
    "router_bwd_no_dx": ("router_bwd", m_router_bwd_no_dx),
    "dW2_rows_reversed": ("expert_ffn_bwd", m_dW2_transposed_rows),
    "bias_update_sign_flipped": ("bias_update", m_bias_update_sign_flipped),
    "bias_update_moves_at_mean": ("bias_update", m_bias_update_moves_at_mean),
    "seq_loss_sum_over_sequences": ("seq_balance_loss", m_seq_loss_sum_over_sequences),
    "seq_stats_without_e_over_k": ("seq_balance_stats", m_seq_stats_without_e_over_k),
    "seq_bwd_no_normalisation_term": ("seq_balance_bwd", m_seq_bwd_no_normalisation_term),
    "seq_bwd_no_sigmoid_grad": ("seq_balance_bwd", m_seq_bwd_no_sigmoid_grad),
    "router_bwd_dense_scaled_dx": ("router_bwd_dense", m_router_bwd_dense_drops_dx),
}


def test_unmutated_oracle_passes_every_pin():
    assert _caught() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    assert _caught(), f"no pin caught mutation {name}"
