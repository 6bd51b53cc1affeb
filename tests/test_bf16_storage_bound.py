"""What storing the layer's intermediates in bf16 costs, measured on the CPU.

tests/bf16_pipeline.py evaluates the layer with exact arithmetic and bf16
stores at the places the HIP path stores bf16.  Its element-wise distance from
the fp64 oracle (the C15 error, max |e - r| / max(|r|, rms r)) is the part of
a bf16 implementation's error that no kernel can remove; the GPU parity tests
bound the kernels' own error against this pipeline (tests/parity.py).  Here
the pipeline is first pinned to the oracle (without rounding it is the
oracle's arithmetic), then its error is recorded at a mid-size layer and at
the dots.llm1 widths with 12 rows per expert (the decode batch's rows per
expert), which is where the weight gradients sum the fewest rows.
"""
import math

import numpy as np
import pytest

from fine_grained_moe_amd.synthetic import Workload, generate_numpy
from oracle import moe_oracle as O
import bf16_pipeline as B

ALIGN = 128


def el(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms)))


def per_slice(got, ref):
    return max(el(got[i], ref[i]) for i in range(ref.shape[0]) if np.any(ref[i]))


def errors(w):
    inp = generate_numpy(w, with_dy=True)
    fwd = O.forward(inp, w.K, ALIGN)
    bwd = O.backward(inp, fwd, inp["dy"])
    emu = B.layer(inp, w.K, ALIGN, dy=inp["dy"])
    v = fwd["perm"]["src_token"] >= 0
    out = {n: el(emu[n][v], fwd[n][v]) for n in ("act", "h", "y_rows")}
    out.update({n: el(emu[n][v], bwd[n][v]) for n in ("dy_rows", "dact", "dx_rows")})
    out.update(y=el(emu["y"], fwd["y"]), y_shared=el(emu["y_shared"], fwd["y_shared"]),
               dg=el(emu["dg"], bwd["dg"]), dx=el(emu["dx"], bwd["dx"]),
               dW_r=el(emu["dW_r"], bwd["dW_r"]), dW1=per_slice(emu["dW1"], bwd["dW1"]),
               dW2=per_slice(emu["dW2"], bwd["dW2"]),
               dW1_sh=per_slice(emu["dW1_sh"], bwd["dW1_sh"]),
               dW2_sh=per_slice(emu["dW2_sh"], bwd["dW2_sh"]))
    print(f"{w.name}: " + ", ".join(f"{k} {v:.2e}" for k, v in out.items()), flush=True)
    return out


def test_pipeline_without_rounding_is_the_oracle():
    """With the stores left exact, the pipeline computes the oracle's values:
    the module adds nothing but where the rounding happens."""
    w = Workload("pin", T=300, H=128, E=8, K=3, S=2, F=64, seed=41, router_std=0.1, bias_std=0.05)
    inp = generate_numpy(w, with_dy=True)
    fwd = O.forward(inp, w.K, ALIGN)
    bwd = O.backward(inp, fwd, inp["dy"])
    ex = B.layer(inp, w.K, ALIGN, dy=inp["dy"], rnd=B.no_store)
    v = fwd["perm"]["src_token"] >= 0
    for n in ("act", "h", "y_rows"):
        assert np.allclose(ex[n][v], fwd[n][v], rtol=1e-12, atol=1e-12), n
    for n in ("dy_rows", "dact", "dx_rows"):
        assert np.allclose(ex[n][v], bwd[n][v], rtol=1e-12, atol=1e-12), n
    assert np.allclose(ex["y"], fwd["y"], rtol=1e-12, atol=1e-12)
    assert np.allclose(ex["y_shared"], fwd["y_shared"], rtol=1e-12, atol=1e-12)
    # quantities the layer defines in fp32 (dg, router gradients, dW) carry one fp32 rounding
    for n in ("dg", "dW_r", "dx", "dW1", "dW2", "dW1_sh", "dW2_sh"):
        ref = bwd[n]
        tol = 2e-7 * np.abs(ref).max() + 1e-30
        assert np.abs(np.asarray(ex[n], np.float64) - ref).max() <= tol, n
    # and with the stores rounded it differs from the oracle
    em = B.layer(inp, w.K, ALIGN, dy=inp["dy"])
    assert not np.allclose(em["act"][v], fwd["act"][v], rtol=1e-6, atol=0)


def test_storage_error_mid_layer():
    e = errors(Workload("mid", T=1000, H=512, E=16, K=4, S=2, F=352, seed=21, router_std=0.08,
                        bias_std=0.05))
    # a single rounding of a value: at most half a bf16 unit in the last place,
    # 2^-8 of the value (8 significant bits)
    for n in ("act", "h", "dy_rows"):
        assert e[n] <= 2.0 ** -8, n
    # forward outputs and input gradient stay within the 2e-2 bound on storage alone
    for n in ("y_rows", "y", "y_shared", "dx", "dg", "dW_r"):
        assert e[n] < 2e-2, n
    # the SwiGLU backward of a rounded act exceeds it
    assert e["dact"] > 2e-2


@pytest.mark.timeout(300)
def test_storage_error_dots_widths_12_rows_per_expert():
    """H = 5120, F = 1408 (the dots.llm1 shapes), 8 experts and 16 tokens with
    K = 6: 12 rows per expert on average, as in the T = 256 decode batch.
    The expert weight gradients, sums over so few rows of rounded dact, h and
    dy rows, carry several times the 2e-2 bound from storage alone, which is
    why the parity tests bound them against this pipeline."""
    e = errors(Workload("dots-12rows", T=16, H=5120, E=8, K=6, S=2, F=1408, seed=31))
    for n in ("act", "h", "dy_rows"):
        assert e[n] <= 2.0 ** -8, n
    for n in ("y", "y_shared", "dx"):
        assert e[n] < 2e-2, n
    assert e["dW1"] > 2e-2 and e["dW2"] > 2e-2
    assert max(e.values()) < 0.2
