"""Comparison helpers shared by the GPU parity tests (test-side only).

Outputs must match the oracle within a max relative error of 2e-2 (bf16
operands, fp32 accumulation).  "Max relative error" is read element-wise:

    err(g, r) = max_i |g_i - r_i| / max(|r_i|, rms(r))

(rms over the whole tensor, or over one expert's slice for the expert weight
gradients; the rms floor keeps entries near zero from dividing by ~0).  An
all-zero reference slice must be exactly zero.

Every comparison gates err(g, r) <= 2e-2 against the fp64 oracle r, except
where storing the intermediates in bf16 alone costs more than that: the
SwiGLU-backward output dact (rounded act in, rounded dact out) and what is
summed from it or from the rounded h and dy rows (dx_rows, dW1, dW2, the
router gradient through dg).  tests/bf16_pipeline.py evaluates the layer with
exact arithmetic and only those bf16 stores; call its value e.  For such
tensors the gates are
    err(g, e) <= 2e-2      (the kernels' own error, denominators from r), and
    err(g, r) <= 2e-2 + err(e, r)
(the second follows from the first by the triangle inequality; it is checked
and reported as the distance from the oracle).  tests/test_bf16_storage_bound.py
records err(e, r) on the CPU: at the dots widths with 12 rows per expert it is
2.7e-2 on dact, 2.5e-2 on dx_rows and 4.5e-2 to 5.6e-2 on the expert weight
gradients.

A second gate bounds the 2-norm relative error ||g - r||_2 / ||r||_2 by
NORM_TOL on every comparison.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 2e-2
NORM_TOL = 1e-2


def elementwise_err(got, ref, base=None) -> float:
    """max_i |g_i - r_i| / max(|b_i|, rms(b)), b = base (default ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    b = ref if base is None else np.asarray(base, np.float64)
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(b * b)))
    if rms == 0.0:
        return float(np.max(np.abs(got - ref)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(b), rms)))


def norm_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = float(np.linalg.norm(ref))
    d = float(np.linalg.norm(got - ref))
    return d if n == 0.0 else d / n


REPORT = []


def assert_close(name, got, ref, emu=None, norm_tol=NORM_TOL, tol=TOL):
    """Element-wise gate of `got` against the oracle `ref`.  With `emu` (the
    bf16-storage pipeline's value of the same tensor) the bound against the
    oracle widens by that pipeline's own error, and the kernels' error
    err(got, emu) is gated at `tol` instead."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = elementwise_err(got, ref)
    n = norm_err(got, ref)
    bound = tol
    e_emu = e_kern = None
    if emu is not None:
        e_emu = elementwise_err(emu, ref)
        e_kern = elementwise_err(got, emu, base=ref)
        bound = tol + e_emu
    REPORT.append((name, e, n, e_emu, e_kern))
    if e_kern is not None:
        assert e_kern <= tol, f"{name}: error against the bf16-storage pipeline {e_kern:.3e} > {tol}"
    assert e <= bound, f"{name}: element-wise relative error {e:.3e} > {bound:.3e}"
    assert n <= norm_tol, f"{name}: 2-norm relative error {n:.3e} > {norm_tol}"
    return e


def per_slice_close(name, got, ref, emu=None):
    """Per leading-index slice (one expert's weight gradient; rms per slice);
    an all-zero reference slice must be exactly zero."""
    worst = 0.0
    for i in range(ref.shape[0]):
        r = np.asarray(ref[i], np.float64)
        g = np.asarray(got[i], np.float64)
        if not np.any(r):
            assert not np.any(g), f"{name}[{i}]: expected exact zeros"
            continue
        worst = max(worst, assert_close(f"{name}[{i}]", g, r,
                                        None if emu is None else np.asarray(emu[i], np.float64)))
    return worst


def to_np(t):
    """torch tensor (any device, bf16/fp32/int) -> numpy (bf16 -> fp32)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def check_route(gpu_idx, gpu_w, gpu_s, ref, label=""):
    """Routing against the oracle.

    The selected set must match exactly except on tokens whose K-th and
    (K+1)-th oracle keys are a near-tie; the order inside the set must match
    except where two adjacent selected keys are a near-tie.  Weights and scores
    are compared on the tokens whose list agrees.  Returns (differing tokens,
    oracle near-ties)."""
    idx_ref = ref["topk_idx"]
    set_same = np.all(np.sort(gpu_idx, 1) == np.sort(idx_ref, 1), axis=1)
    same = np.all(gpu_idx == idx_ref, axis=1)
    set_bad = ~set_same & ~ref["near_tie"]
    order_bad = set_same & ~same & ~ref["order_tie"]
    for t in np.nonzero(set_bad | order_bad)[0][:5]:
        keys = ref["keys"][t]
        print(f"  {label} token {t}: gpu {gpu_idx[t].tolist()} oracle {idx_ref[t].tolist()} "
              f"oracle keys of gpu choice {keys[gpu_idx[t]].tolist()} "
              f"of oracle choice {keys[idx_ref[t]].tolist()}", flush=True)
    assert not set_bad.any(), f"{label} selected set differs on {int(set_bad.sum())} non-tie tokens"
    assert not order_bad.any(), f"{label} selection order differs on {int(order_bad.sum())} non-tie tokens"
    if same.any():
        assert_close(f"{label} topk_w", gpu_w[same], ref["topk_w"][same])
        assert_close(f"{label} topk_s", gpu_s[same], ref["topk_s"][same], tol=1e-5, norm_tol=1e-5)
    print(f"  {label} routing: {int((~set_same).sum())} tokens select another set (all near-ties: "
          f"{int(ref['near_tie'].sum())} in the batch), {int((set_same & ~same).sum())} list the same "
          f"set in another order (all within order-tie keys: {int(ref['order_tie'].sum())} in the "
          f"batch)", flush=True)
    return int((~same).sum()), int(ref["near_tie"].sum())


def check_permute(gpu, ref, E, align, m_cap):
    """Bit-exact segment layout given the same topk_idx."""
    assert np.array_equal(gpu["counts"], ref["counts"]), "counts"
    assert np.array_equal(gpu["offsets"], ref["offsets"]), "offsets"
    assert np.array_equal(gpu["row_of"], ref["row_of"]), "row_of"
    total = int(ref["offsets"][E])
    assert np.array_equal(gpu["src_token"][:total], ref["src_token"]), "src_token"
    assert (gpu["src_token"][total:] == -1).all(), "src_token tail"
    te = np.full(m_cap // align, -1, np.int64)
    for e in range(E):
        a, b = int(ref["offsets"][e]) // align, int(ref["offsets"][e + 1]) // align
        te[a:b] = e
    assert np.array_equal(gpu["tile_expert"], te), "tile_expert"
