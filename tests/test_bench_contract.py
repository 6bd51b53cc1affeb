"""The benchmark's command-line contract that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_gemm_flop_and_byte_accounting():
    """Useful flops of the twelve GEMM launches add up to the layer's GEMM
    flops (3 * (K+S) * 6HF per token); algorithmic bytes count each operand once."""
    sys.path.insert(0, ROOT)
    import bench
    from fine_grained_moe_amd.synthetic import WORKLOADS, gemm_useful_flops
    w = WORKLOADS["fwdbwd"]
    total = sum(bench.gemm_launch_flops(w, n) for n in bench.Layer.GEMMS)
    assert abs(total - gemm_useful_flops(w, True)) <= 1e-9 * total
    assert abs(total - 3 * (w.K + w.S) * 6 * w.H * w.F * w.T) <= 1e-9 * total
    # gate/up forward: x rows in, W1 once, act (2F) and h (F) out, bf16
    rows = w.T * w.K
    exp = 2 * (rows * w.H + w.E * 2 * w.F * w.H + rows * 3 * w.F)
    assert bench.gemm_launch_bytes(w, "gate_up_fwd") == exp
    # experts without rows: their weights are not read, but their (zero)
    # weight gradients are still written
    wt1 = 2 * 2 * w.F * w.H
    assert bench.gemm_launch_bytes(w, "gate_up_fwd", live=20) == exp - (w.E - 20) * wt1
    assert bench.gemm_launch_bytes(w, "gate_up_wgrad", live=20) == bench.gemm_launch_bytes(w, "gate_up_wgrad")
    assert bench.gemm_launch_bytes(w, "shared_gate_up_fwd", live=20) == bench.gemm_launch_bytes(w, "shared_gate_up_fwd")


def test_roofline_bound_follows_arithmetic_intensity():
    """A launch below the ridge (2516.6 TFLOP/s / 8 TB/s = 315 flop/B) is
    reported against HBM in GB/s, one above it against the bf16 MFMA peak."""
    sys.path.insert(0, ROOT)
    import bench
    from fine_grained_moe_amd.synthetic import WORKLOADS
    dec = bench.roofline_of("gate_up_fwd", WORKLOADS["decode"], 0.65)
    assert dec["bound"] == "hbm" and dec["unit"] == "GB/s" and dec["flop_per_byte"] < 315
    nbytes = bench.gemm_launch_bytes(WORKLOADS["decode"], "gate_up_fwd")
    assert abs(dec["achieved"] - nbytes / 0.65e-3 / 1e9) <= 0.1
    assert abs(dec["frac"] - dec["achieved"] / 8000.0) <= 1e-4
    big = bench.roofline_of("gate_up_wgrad", WORKLOADS["fwdbwd"], 2.0)
    assert big["bound"] == "mfma" and big["unit"] == "TFLOP/s" and big["flop_per_byte"] >= 315
    flops = bench.gemm_launch_flops(WORKLOADS["fwdbwd"], "gate_up_wgrad")
    assert abs(big["achieved"] - flops / 2.0e-3 / 1e12) <= 0.01
    # HBM bytes from the counters are reported only for the source they were taken on
    assert (big["traffic"] is None) == (bench.traffic_of("gate_up_wgrad", WORKLOADS["fwdbwd"])["traffic"] is None)


def test_row_op_bytes():
    """Routing, permutation and combine are priced at their inputs read once and
    outputs written once: at T = 8192 dots shapes the row copies dominate —
    permute 2H(1+K)T, combine 2H(K+2)T, combine backward 2H(2K+1)T,
    un-permute 2H(K+2)T + 4HT, router backward 2HT + 4HT (x gathered, dx_router
    written), the two fused 2HT + 2H(K+2)T (dx_router never stored) — plus their
    index and weight arrays."""
    sys.path.insert(0, ROOT)
    import bench
    from fine_grained_moe_amd.synthetic import WORKLOADS
    w = WORKLOADS["fwdbwd"]
    T, H, K = w.T, w.H, w.K
    rows = {"permute": 2 * H * (1 + K) * T, "combine": 2 * H * (K + 2) * T,
            "combine_bwd": 2 * H * (2 * K + 1) * T, "permute_bwd": 2 * H * (K + 2) * T + 4 * H * T,
            "route": 2 * H * T, "route_bwd": 2 * H * T + 4 * H * T,
            "route_permute_bwd": 2 * H * T + 2 * H * (K + 2) * T}
    for n, b in rows.items():
        got = bench.row_op_bytes(w, n)
        assert b <= got <= b * 1.01 + 8e6, (n, got, b)
