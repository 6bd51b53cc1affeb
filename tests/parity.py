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
summed from it or from the rounded h, y and dy rows (dx_rows, dW1, dW2, the
router gradients through dg).  tests/bf16_pipeline.py evaluates the layer
with exact arithmetic and only those bf16 stores; call its value e.  For such
tensors the gates are
    err(g, r) <= 2e-2 + err(e, r)      (2e-2 beyond what bf16 storage costs)
    err(g, e) <= max(2e-2, err(e, r))  (denominators from r)
The second bounds the kernels' own deviation from the exact bf16-storage
pipeline: its fp32 sums differ from exact ones in the last bits, which moves
some bf16 roundings of the intermediates by one unit, a second draw of the
same storage error.  For the expert weight gradients, sums over an expert's
rows (a dozen at decode), one such unit in one row is amplified by the rms
normalisation beyond either bound, so there the kernels' deviation is gated
componentwise instead, by the classical bound for a sum of products whose
stored factors may each differ by one bf16 unit (2^-7 of their value):
    |g - e| <= 2^-6 (|A|^T |B|) + 2^-7 |e|      (every element)
with |A|^T |B| the sum of the absolute products (dact^T x rows for dW1,
dy rows^T h for dW2), which no row count inflates.  The same amplification
makes the pipeline's own error on such a slice one realisation of the storage
error among many (which roundings a summation order moves differs between two
correct bf16 implementations), so the bound against the oracle for the expert
weight gradients allows two such draws: err(g, r) <= 2e-2 + 2 err(e, r).
tests/test_bf16_storage_bound.py records err(e, r) on the CPU: at the dots
widths with 12 rows per expert it is 2.7e-2 on dact, 2.5e-2 on dx_rows and
4.5e-2 to 5.6e-2 on the expert weight gradients.

A second gate bounds the 2-norm relative error ||g - r||_2 / ||r||_2 by
NORM_TOL (plus the bf16-storage pipeline's own 2-norm error, where it is
compared).
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


def componentwise_ratio(got, emu, scale) -> float:
    """max_i |g_i - e_i| / (2^-6 scale_i + 2^-7 |e_i|) (module doc); <= 1 passes."""
    got = np.asarray(got, np.float64)
    emu = np.asarray(emu, np.float64)
    bound = 2.0 ** -6 * np.asarray(scale, np.float64) + 2.0 ** -7 * np.abs(emu)
    d = np.abs(got - emu)
    if np.any((bound == 0) & (d > 0)):
        return float("inf")
    with np.errstate(invalid="ignore", divide="ignore"):
        return float(np.max(np.where(bound > 0, d / bound, 0.0)))


def assert_close(name, got, ref, emu=None, scale=None, norm_tol=NORM_TOL, tol=TOL):
    """Element-wise gate of `got` against the oracle `ref` (module doc).  With
    `emu`, the bf16-storage pipeline's value of the same tensor, the bounds
    widen by that pipeline's own error and the kernels' deviation from it is
    gated too: componentwise against `scale` (the sum of absolute products)
    when given, else element-wise."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = elementwise_err(got, ref)
    n = norm_err(got, ref)
    bound, nbound = tol, norm_tol
    e_emu = e_kern = None
    if emu is not None:
        e_emu = elementwise_err(emu, ref)
        # an expert weight gradient (scale given) takes two storage draws
        draws = 1 if scale is None else 2
        bound = tol + draws * e_emu
        nbound = norm_tol + draws * norm_err(emu, ref)
        if scale is not None:
            e_kern = componentwise_ratio(got, emu, scale)
            assert e_kern <= 1.0, (f"{name}: deviation from the bf16-storage pipeline beyond "
                                   f"the one-unit componentwise bound (ratio {e_kern:.3f})")
        else:
            e_kern = elementwise_err(got, emu, base=ref)
            assert e_kern <= max(tol, e_emu), (f"{name}: error against the bf16-storage pipeline "
                                               f"{e_kern:.3e} > {max(tol, e_emu):.3e}")
    REPORT.append((name, e, n, e_emu, e_kern))
    assert e <= bound, f"{name}: element-wise relative error {e:.3e} > {bound:.3e}"
    assert n <= nbound, f"{name}: 2-norm relative error {n:.3e} > {nbound:.3e}"
    return e


def print_report():
    """One line per comparison: element-wise and 2-norm error against the
    oracle and, where compared, the bf16-storage pipeline's own element-wise
    error and the kernels' error against that pipeline."""
    for name, e, n, e_emu, e_kern in REPORT:
        extra = "" if e_emu is None else f"  storage {e_emu:.2e}  kernel {e_kern:.2e}"
        # (kernel: element-wise error against the pipeline, or for the expert
        # weight gradients the componentwise ratio, at most 1)
        print(f"  {name:40s} elementwise {e:.2e}  norm {n:.2e}{extra}", flush=True)


def per_slice_close(name, got, ref, emu=None, scale=None):
    """Per leading-index slice (one expert's weight gradient; rms per slice);
    an all-zero reference slice must be exactly zero.  scale(i): the slice's
    sum of absolute products (a callable, computed per slice)."""
    worst = 0.0
    for i in range(ref.shape[0]):
        r = np.asarray(ref[i], np.float64)
        g = np.asarray(got[i], np.float64)
        if not np.any(r):
            assert not np.any(g), f"{name}[{i}]: expected exact zeros"
            continue
        worst = max(worst, assert_close(f"{name}[{i}]", g, r,
                                        None if emu is None else np.asarray(emu[i], np.float64),
                                        None if scale is None else scale(i)))
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
