"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from fine_grained_moe_amd.synthetic import WORKLOADS, generate_numpy
import oracle_pins as P


@pytest.fixture(scope="module")
def small():
    return P.small_inputs()


@pytest.fixture(scope="module")
def tiny():
    w = WORKLOADS["tiny"]
    return generate_numpy(w, with_dy=True), w


def test_logits_exact_sum(small):
    inp, _ = small
    P.check_logits_exact_sum(O, inp["x"], inp["w_router"])


def test_logits_exact_sum_tiny(tiny):
    inp, _ = tiny
    P.check_logits_exact_sum(O, inp["x"][:16], inp["w_router"])


def test_sigmoid_closed_form():
    P.check_sigmoid_closed_form(O)


def test_topk_bruteforce(small, tiny):
    inp, K = small
    r = O.route(inp["x"], inp["w_router"], inp["bias"], K)
    P.check_topk_bruteforce(O, r["keys"], K)
    inp, w = tiny
    r = O.route(inp["x"], inp["w_router"], inp["bias"], w.K)
    P.check_topk_bruteforce(O, r["keys"], w.K)


def test_topk_ties_and_nan():
    keys = np.array([[0.5, 0.7, 0.7, 0.1, 0.7],
                     [np.nan, 0.2, np.nan, 0.2, -1.0],
                     [-np.inf, -np.inf, -np.inf, -np.inf, -np.inf]], np.float32)
    assert O.top_k(keys, 3).tolist() == [[1, 2, 4], [1, 3, 4], [0, 1, 2]]
    P.check_topk_bruteforce(O, keys, 3)


def test_route_golden():
    P.check_route_golden(O)


def test_combine_weight_invariants(small, tiny):
    inp, K = small
    P.check_combine_weight_invariants(O, inp["x"], inp["w_router"], inp["bias"], K)
    inp, w = tiny
    P.check_combine_weight_invariants(O, inp["x"], inp["w_router"], inp["bias"], w.K)


def test_near_tie_mask():
    keys = np.array([[0.9, 0.5, 0.5 * (1 - 2e-7), 0.1],
                     [0.9, 0.5, 0.49, 0.1]], np.float32)
    assert O.near_tie_mask(keys, 2).tolist() == [True, False]
    assert not O.near_tie_mask(keys, 4).any()


def test_order_tie_mask():
    keys = np.array([[0.9, 0.9 * (1 - 3e-7), 0.5, 0.1],     # ranks 1 and 2 nearly equal
                     [0.9, 0.8, 0.5, 0.5 * (1 - 3e-7)],     # tie only past rank K=3
                     [0.9, 0.8, 0.5, 0.1]], np.float32)
    assert O.order_tie_mask(keys, 3).tolist() == [True, False, False]
    assert O.near_tie_mask(keys, 3).tolist() == [False, True, False]
    assert not O.order_tie_mask(keys, 1).any()


def test_permute_golden():
    P.check_permute_golden(O)


@pytest.mark.parametrize("align", [1, 4, 32, 128])
def test_permute_bruteforce_and_invariants(small, tiny, align):
    for inp, K in (small, (tiny[0], tiny[1].K)):
        E = inp["w_router"].shape[1]
        idx = O.route(inp["x"], inp["w_router"], inp["bias"], K)["topk_idx"]
        P.check_permute_bruteforce(O, idx, E, align)
        P.check_permute_invariants(O.permute(idx, E, align), idx, E, align)


def test_permute_skewed_with_empty_experts():
    rng = np.random.default_rng(7)
    T, E, K = 300, 16, 3
    idx = np.stack([rng.choice(5, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    p = O.permute(idx, E, 8)
    assert (p["counts"][5:] == 0).all()
    assert (np.diff(p["offsets"])[5:] == 0).all()
    P.check_permute_invariants(p, idx, E, 8)
    P.check_permute_bruteforce(O, idx, E, 8)


def test_forward_dense_bruteforce(small):
    inp, K = small
    P.check_forward_bruteforce(O, inp, K, align=4)


def test_forward_dense_bruteforce_tiny(tiny):
    inp, w = tiny
    sub = dict(inp)
    sub["x"] = inp["x"][:12]
    P.check_forward_bruteforce(O, sub, w.K, align=32)


def test_one_expert_is_dense_swiglu():
    P.check_one_expert_is_dense_swiglu(O)


def test_identical_experts(small, tiny):
    inp, K = small
    P.check_identical_experts_independent_of_routing(O, inp, K, 4)
    inp, w = tiny
    P.check_identical_experts_independent_of_routing(O, inp, w.K, 32)


def test_shared_fusion(small, tiny):
    P.check_shared_fusion(O, small[0])
    P.check_shared_fusion(O, tiny[0])


def test_backward_autograd(small, tiny):
    inp, K = small
    P.check_backward_autograd(O, inp, K, 4)
    inp, w = tiny
    P.check_backward_autograd(O, inp, w.K, 32)


def test_backward_finite_differences(small):
    inp, K = small
    P.check_backward_finite_differences(O, inp, K, 4)


def test_empty_expert_weight_gradient_is_zero(small):
    inp, K = small
    inp = dict(inp)
    inp["bias"] = inp["bias"].copy()
    inp["bias"][0] = -100.0          # expert 0 is never selected
    fwd = O.forward(inp, K, 4)
    assert fwd["perm"]["counts"][0] == 0
    bwd = O.backward(inp, fwd, inp["dy"])
    assert (bwd["dW1"][0] == 0).all() and (bwd["dW2"][0] == 0).all()
    assert (bwd["dW_r"][:, 0] == 0).all()


def test_bias_update_golden():
    P.check_bias_update_golden(O)


def test_bias_update_invariants():
    P.check_bias_update_invariants(O)


def test_bias_update_balances_router():
    P.check_bias_update_balances_router(O)


def test_seq_loss_golden():
    P.check_seq_loss_golden(O)


def test_seq_loss_closed_forms():
    P.check_seq_loss_closed_forms(O)


def test_seq_loss_finite_differences():
    P.check_seq_loss_finite_differences(O)


def test_router_bwd_dense():
    P.check_router_bwd_dense(O)
