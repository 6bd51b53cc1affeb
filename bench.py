"""Benchmark of the MoE FFN layer hot path on one MI355X.

One step = one forward + backward pass of the whole layer (routing, permute,
grouped SwiGLU GEMMs, combine, and their backward) over T=8192 tokens at
dots.llm1 shapes (H=5120, 128 routed experts of width 1408, top-6, 2 shared
experts), synthetic seeded inputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload fwdbwd|prefill|decode|skew|ep_shard]
                    [--no-cpu-baseline] [--cpu-seconds S] [--no-configs] [--no-balance]
                    [--no-graph] [--copy-calibration]

The default fwd+bwd run also times the forward of the decode (T=256), prefill
(T=8192) and skewed (T=16384) configurations ("configs" in the JSON line).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0

# load balancing: sequences of 8192 tokens (the pre-training context length),
# balance-loss coefficient and bias step (values of the DeepSeek recipe's order)
SEQ_LEN, ALPHA, GAMMA = 8192, 1e-4, 1e-3
BALANCE_OPS = ("seq_loss_fwd", "seq_loss_bwd", "route_dlogit", "route_bwd_dense", "bias_update")


# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch) on this workload, scaled by the counters' reading for a plain 1 GiB
# device copy (FETCH_SIZE reads half the bytes a copy moves: factor 2.0;
# WRITE_SIZE reads them exactly: factor 1.0).  Valid only for the grouped-GEMM
# source they were taken on, identified by its SHA-256; otherwise reported null.
# HBM read rate of a plain streaming-read kernel on the MI355X (16-byte
# non-temporal loads over 4 GiB, 1k-16k workgroups: 7.0-7.1 TB/s); reported
# beside HBM-bound launches for context
STREAM_READ_GBS = 7050.0
COUNTER_FACTORS = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
TRAFFIC_SOURCE_SHA256 = "7341e5ef1c3bf94b9fc07a151537583e70a8a6e4109d133897c7c703e29e1c04"
TRAFFIC_KIB = {    # launch name -> (FETCH_SIZE KiB, WRITE_SIZE KiB), workload fwdbwd
    "gate_up_fwd": (3075470.4, 405504.1), "down_fwd": (1103172.3, 491545.1),
    "shared_gate_up_fwd": (348244.2, 135202.5), "shared_down_fwd": (180295.2, 81933.9),
    "down_dgrad": (1895078.9, 270336.1), "gate_up_dgrad": (2605795.1, 491629.5),
    "down_wgrad": (322732.3, 1802281.8), "gate_up_wgrad": (847809.1, 3605112.6),
    "shared_down_dgrad": (352385.2, 90118.5), "shared_gate_up_dgrad": (360515.4, 81921.8),
    "shared_down_wgrad": (217164.8, 28160.4), "shared_gate_up_wgrad": (434253.8, 56320.4),
}


def traffic_of(name, w):
    import hashlib
    src = os.path.join(ROOT, "fine_grained_moe_amd", "csrc", "grouped_gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if w.name != "fwdbwd" or sha != TRAFFIC_SOURCE_SHA256 or name not in TRAFFIC_KIB:
        return {"traffic": None}
    fk, wk = TRAFFIC_KIB[name]
    gb = (fk * COUNTER_FACTORS["FETCH_SIZE"] + wk * COUNTER_FACTORS["WRITE_SIZE"]) * 1024 / 1e9
    return {"traffic": round(gb, 3), "traffic_unit": "GB per launch",
            "traffic_read_gb": round(fk * COUNTER_FACTORS["FETCH_SIZE"] * 1024 / 1e9, 3),
            "traffic_write_gb": round(wk * COUNTER_FACTORS["WRITE_SIZE"] * 1024 / 1e9, 3)}


def roofline_of(name, w, launch_ms, traffic=True, live=None):
    """Roofline entry of one grouped-GEMM launch: MFMA-bound (useful TFLOP/s
    against the bf16 peak) when its arithmetic intensity (useful flops per
    algorithmic byte) is at or above the ridge, else HBM-bound (algorithmic
    GB/s against 8 TB/s).  `live`: routed experts that own rows."""
    flops, nbytes = gemm_launch_flops(w, name), gemm_launch_bytes(w, name, live)
    sec = launch_ms * 1e-3
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    tf, gbs = flops / sec / 1e12, nbytes / sec / 1e9
    if flops / nbytes >= ridge:
        r = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    else:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4), "achieved_tflops": round(tf, 2),
             # context, not the peak: what plain streaming reads reach on this card
             "reference_read_gbs": STREAM_READ_GBS,
             "frac_of_reference_read": round(gbs / STREAM_READ_GBS, 4)}
    r.update({"kernel": f"grouped GEMM {name}", "launch_ms": round(launch_ms, 4),
              "flop_per_byte": round(flops / nbytes, 1), "algorithmic_gb": round(nbytes / 1e9, 3)})
    r.update(traffic_of(name, w) if traffic else {"traffic": None})
    return r


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fwdbwd",
                    choices=["fwdbwd", "prefill", "skew", "decode", "ep_shard"],
                    help="ep_shard: the grouped expert products alone (fwd+bwd) at one GPU's "
                         "share of an 8-way expert-parallel layer, 16 experts x 3072 rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="about how long the timed CPU oracle run takes (its token count is "
                         "sized to this)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the forward timings of the decode, prefill and skewed configurations")
    ap.add_argument("--no-balance", action="store_true",
                    help="skip the timing of the step with load balancing")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the timing of the step captured as one HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device to device (known HBM bytes, for scaling "
                         "hardware byte counters)")
    return ap.parse_args()


class Layer:
    """All buffers of one fwd+bwd step, allocated once; step() only launches."""

    def __init__(self, M, g, K):
        import torch
        self.M, self.g, self.K = M, g, K
        x = g["x"]
        T, H = x.shape
        E, twoF, _ = g["w1"].shape
        F = twoF // 2
        dev = x.device
        bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
        self.T, self.H, self.E, self.F = T, H, E, F
        self.w1f, self.w2f = M.fuse_shared(g["w1_sh"], g["w2_sh"])
        SF = self.w2f.shape[2]
        m_cap = M.moe_capacity_rows(T, E, K)
        A = M.moe_align()
        e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device=dev)
        self.b = dict(
            topk_idx=e(T, K, dt=i32), topk_w=e(T, K, dt=f32), topk_s=e(T, K, dt=f32),
            perm=dict(counts=e(E, dt=i32), offsets=e(E + 1, dt=i32), row_of=e(T, K, dt=i32),
                      src_token=e(m_cap, dt=i32), tile_expert=e(m_cap // A, dt=i32),
                      x_rows=e(m_cap, H)),
            route_ws=e(M.moe_route_workspace_bytes(T, H, E), dt=torch.uint8),
            perm_ws=e(max(M.moe_permute_workspace_bytes(T, E, K), 1), dt=torch.uint8),
            act=e(m_cap, 2 * F), h=e(m_cap, F), y_rows=e(m_cap, H),
            act_sh=e(T, 2 * SF), h_sh=e(T, SF), y_sh=e(T, H), y=e(T, H),
            dy_rows=e(m_cap, H), dg=e(T, K, dt=f32), dact=e(m_cap, 2 * F), dx_rows=e(m_cap, H),
            dw1=e(E, 2 * F, H), dw2=e(E, H, F),
            dact_sh=e(T, 2 * SF), dx_sh=e(T, H), dw1_sh=e(1, 2 * SF, H), dw2_sh=e(1, H, SF),
            dw_router=e(H, E, dt=f32), dx_router=e(T, H, dt=f32),
            rb_ws=e(M.moe_route_bwd_workspace_bytes(T, H, E, K), dt=torch.uint8),
            dx=e(T, H),
            # load balancing (sequence-wise loss over sequences of SEQ_LEN tokens, bias step)
            scores=e(T, E, dt=f32), seq_f=e(max(T // SEQ_LEN, 1), E, dt=f32), loss=e(1, dt=f32),
            seq_ws=e(max(M.moe_seq_balance_workspace_bytes(T, E, SEQ_LEN), 1), dt=torch.uint8),
            dloss=torch.ones(1, dtype=f32, device=dev), dlogit_bal=e(T, E, dt=f32),
            dense_ws=e(max(M.moe_route_bwd_dense_workspace_bytes(T, H, E), 1), dt=torch.uint8),
            # the shared experts' forward at small T splits its contraction
            # over workgroups into fp32 partial products
            split_ws=e(max(M.moe_dense_fwd_split_workspace_bytes(T, H, SF), 1), dt=torch.uint8),
            bias_train=g["bias"].clone())
        self.ev = None

    # the twelve grouped-GEMM launches of one step, in launch order
    GEMMS = ("gate_up_fwd", "down_fwd", "shared_gate_up_fwd", "shared_down_fwd",
             "down_dgrad", "gate_up_dgrad", "down_wgrad", "gate_up_wgrad",
             "shared_down_dgrad", "shared_gate_up_dgrad", "shared_down_wgrad",
             "shared_gate_up_wgrad")

    def _gemm(self, name, ev, fn):
        """Launch one grouped GEMM, bracketed by events when ev is a dict."""
        if ev is not None and name in ev:
            ev[name][0].record()
        fn()
        if ev is not None and name in ev:
            ev[name][1].record()

    def forward(self, ev=None, balance=False):
        M, g, b, K = self.M, self.g, self.b, self.K
        p = b["perm"]
        seg = (p["offsets"], p["counts"], p["tile_expert"])
        self._gemm("route", ev, lambda: M.moe_route(
            g["x"], g["w_router"], g["bias"], K, b["topk_idx"], b["topk_w"], b["topk_s"],
            ws=b["route_ws"], scores=b["scores"] if balance else None))
        if balance:
            self._gemm("seq_loss_fwd", ev, lambda: M.moe_seq_balance_fwd(
                b["scores"], b["topk_idx"], SEQ_LEN, ALPHA, loss=b["loss"], seq_f=b["seq_f"],
                ws=b["seq_ws"]))
        self._gemm("permute", ev, lambda: M.moe_permute(
            b["topk_idx"], g["x"], self.E, out=p, ws=b["perm_ws"]))
        self._gemm("gate_up_fwd", ev, lambda: M.moe_grouped_gate_up_fwd(
            p["x_rows"], g["w1"], *seg, act=b["act"], h=b["h"]))
        self._gemm("down_fwd", ev, lambda: M.moe_grouped_down_fwd(
            b["h"], g["w2"], *seg, y_rows=b["y_rows"]))
        self._gemm("shared_gate_up_fwd", ev, lambda: M.moe_dense_gate_up_fwd_split(
            g["x"], self.w1f, act=b["act_sh"], h=b["h_sh"], ws=b["split_ws"]))
        self._gemm("shared_down_fwd", ev, lambda: M.moe_dense_down_fwd_split(
            b["h_sh"], self.w2f, y=b["y_sh"], ws=b["split_ws"]))
        self._gemm("combine", ev, lambda: M.moe_combine(
            b["y_rows"], p["row_of"], b["topk_w"], b["y_sh"], y=b["y"]))

    def backward(self, ev=None, balance=False):
        M, g, b = self.M, self.g, self.b
        p = b["perm"]
        seg = (p["offsets"], p["counts"], p["tile_expert"])
        E = self.E
        self._gemm("combine_bwd", ev, lambda: M.moe_combine_bwd(
            g["dy"], b["y_rows"], p["row_of"], b["topk_w"], dy_rows=b["dy_rows"], dg=b["dg"]))
        # routed experts: the four steps of moe_grouped_swiglu_bwd, one launch each
        self._gemm("down_dgrad", ev, lambda: M.moe_grouped_down_dgrad(
            g["w2"], b["act"], b["dy_rows"], *seg, dact=b["dact"]))
        self._gemm("gate_up_dgrad", ev, lambda: M.moe_grouped_gate_up_dgrad(
            g["w1"], b["dact"], *seg, dx_rows=b["dx_rows"]))
        self._gemm("down_wgrad", ev, lambda: M.moe_grouped_down_wgrad(
            b["dy_rows"], b["h"], E, *seg, dw2=b["dw2"]))
        self._gemm("gate_up_wgrad", ev, lambda: M.moe_grouped_gate_up_wgrad(
            b["dact"], p["x_rows"], E, *seg, dw1=b["dw1"]))
        # shared experts: one dense group of width S*F
        self._gemm("shared_down_dgrad", ev, lambda: M.moe_grouped_down_dgrad(
            self.w2f, b["act_sh"], g["dy"], dact=b["dact_sh"]))
        self._gemm("shared_gate_up_dgrad", ev, lambda: M.moe_grouped_gate_up_dgrad(
            self.w1f, b["dact_sh"], dx_rows=b["dx_sh"]))
        self._gemm("shared_down_wgrad", ev, lambda: M.moe_grouped_down_wgrad(
            g["dy"], b["h_sh"], 1, dw2=b["dw2_sh"]))
        self._gemm("shared_gate_up_wgrad", ev, lambda: M.moe_grouped_gate_up_wgrad(
            b["dact_sh"], g["x"], 1, dw1=b["dw1_sh"]))
        if not balance:
            # router gradients and the un-permute in one call: the router's
            # input gradient is added where dx is summed
            self._gemm("route_permute_bwd", ev, lambda: M.moe_route_permute_bwd(
                g["x"], g["w_router"], b["topk_idx"], b["topk_s"], b["dg"], p["row_of"],
                p["offsets"], p["counts"], p["src_token"], b["dx_rows"], b["dx_sh"],
                dw_router=b["dw_router"], dx=b["dx"], ws=b["rb_ws"]))
        else:
            # the balance loss's dense logit gradient, the combine path's added
            # into it, and one dense router backward for both
            self._gemm("seq_loss_bwd", ev, lambda: M.moe_seq_balance_bwd(
                b["scores"], b["seq_f"], self.K, SEQ_LEN, ALPHA, b["dloss"], dlogit=b["dlogit_bal"]))
            self._gemm("route_dlogit", ev, lambda: M.moe_route_dlogit(
                b["topk_idx"], b["topk_s"], b["dg"], b["dlogit_bal"]))
            self._gemm("route_bwd_dense", ev, lambda: M.moe_route_bwd_dense(
                g["x"], g["w_router"], b["dlogit_bal"], b["dw_router"], b["dx_router"],
                ws=b["dense_ws"], accumulate=False))
            self._gemm("permute_bwd", ev, lambda: M.moe_permute_bwd(
                b["dx_rows"], p["row_of"], b["dx_sh"], b["dx_router"], dx=b["dx"]))
        if balance:
            # the bias step on this batch's loads (a copy of the bias, so that
            # every timed step routes the same way)
            self._gemm("bias_update", ev, lambda: M.moe_bias_update(
                p["counts"], b["bias_train"], GAMMA))


    def step_two_streams(self, side, backward=True):
        """The same step (no load balancing) with the independent launches on a
        second stream, joined back through events: the shared experts' whole
        forward and backward (they need only x and dy) beside the router,
        permute and routed forward, and the routed weight gradients beside the
        routed data gradients (each as soon as its inputs exist).  Results are bit-identical to
        forward() + backward(); the launches share the card, so none of them
        can be timed alone here."""
        import torch
        M, g, b, K, E = self.M, self.g, self.b, self.K, self.E
        p = b["perm"]
        seg = (p["offsets"], p["counts"], p["tile_expert"])
        main = torch.cuda.current_stream()

        def mark(s):
            e = torch.cuda.Event()
            e.record(s)
            return e

        side.wait_event(mark(main))
        with torch.cuda.stream(side):
            M.moe_dense_gate_up_fwd_split(g["x"], self.w1f, act=b["act_sh"], h=b["h_sh"],
                                          ws=b["split_ws"])
            M.moe_dense_down_fwd_split(b["h_sh"], self.w2f, y=b["y_sh"], ws=b["split_ws"])
            shared_fwd = mark(side)
            if backward:
                M.moe_grouped_down_dgrad(self.w2f, b["act_sh"], g["dy"], dact=b["dact_sh"])
                M.moe_grouped_gate_up_dgrad(self.w1f, b["dact_sh"], dx_rows=b["dx_sh"])
                shared_dx = mark(side)
                M.moe_grouped_down_wgrad(g["dy"], b["h_sh"], 1, dw2=b["dw2_sh"])
                M.moe_grouped_gate_up_wgrad(b["dact_sh"], g["x"], 1, dw1=b["dw1_sh"])
        M.moe_route(g["x"], g["w_router"], g["bias"], K, b["topk_idx"], b["topk_w"], b["topk_s"],
                    ws=b["route_ws"])
        M.moe_permute(b["topk_idx"], g["x"], E, out=p, ws=b["perm_ws"])
        M.moe_grouped_gate_up_fwd(p["x_rows"], g["w1"], *seg, act=b["act"], h=b["h"])
        M.moe_grouped_down_fwd(b["h"], g["w2"], *seg, y_rows=b["y_rows"])
        main.wait_event(shared_fwd)
        M.moe_combine(b["y_rows"], p["row_of"], b["topk_w"], b["y_sh"], y=b["y"])
        if not backward:
            main.wait_stream(side)
            return
        M.moe_combine_bwd(g["dy"], b["y_rows"], p["row_of"], b["topk_w"], dy_rows=b["dy_rows"],
                          dg=b["dg"])
        side.wait_event(mark(main))
        with torch.cuda.stream(side):
            M.moe_grouped_down_wgrad(b["dy_rows"], b["h"], E, *seg, dw2=b["dw2"])
        M.moe_grouped_down_dgrad(g["w2"], b["act"], b["dy_rows"], *seg, dact=b["dact"])
        side.wait_event(mark(main))
        with torch.cuda.stream(side):
            M.moe_grouped_gate_up_wgrad(b["dact"], p["x_rows"], E, *seg, dw1=b["dw1"])
        M.moe_grouped_gate_up_dgrad(g["w1"], b["dact"], *seg, dx_rows=b["dx_rows"])
        # dx needs the shared experts' input gradient, not the weight gradients
        main.wait_event(shared_dx)
        M.moe_route_permute_bwd(g["x"], g["w_router"], b["topk_idx"], b["topk_s"], b["dg"],
                                p["row_of"], p["offsets"], p["counts"], p["src_token"],
                                b["dx_rows"], b["dx_sh"], dw_router=b["dw_router"], dx=b["dx"],
                                ws=b["rb_ws"])
        main.wait_stream(side)

# the entry points around the grouped GEMMs, timed like them in the main loop
ROW_OPS_FWD = ("route", "permute", "combine")
ROW_OPS_BWD = ("combine_bwd", "route_permute_bwd")


def row_op_bytes(w, name):
    """Algorithmic HBM bytes of one call of a routing / permutation / combine
    entry point: each of its inputs read once and each output written once,
    as the entry point takes and returns them (bf16 rows 2H bytes, fp32 rows
    4H; index and weight arrays of T*K entries)."""
    T, H, E, K = w.T, w.H, w.E, w.K
    row, tk = 2 * H, T * K
    if name == "route":        # x, W_r in; topk_idx / topk_w / topk_s out
        return T * row + 4 * H * E + 12 * tk
    if name == "permute":      # topk_idx, x in; x_rows (valid rows), row_of, src_token out
        m_cap = ((tk + E * 127 + 127) // 128) * 128
        return 4 * tk + T * row + tk * row + 4 * tk + 4 * m_cap
    if name == "combine":      # y_rows, y_shared, row_of, topk_w in; y out
        return tk * row + (T * row if w.S else 0) + 8 * tk + T * row
    if name == "combine_bwd":  # dy, y_rows, row_of, topk_w in; dy_rows, dg out
        return T * row + tk * row + 8 * tk + tk * row + 4 * tk
    if name == "route_bwd":    # x, W_r, topk_idx/s, dg, row_of, src_token in; dW_r, dx_router out
        m_cap = ((tk + E * 127 + 127) // 128) * 128
        return T * row + 4 * H * E + 16 * tk + 4 * m_cap + 4 * H * E + 4 * T * H
    if name == "permute_bwd":  # dx_rows, dx_shared, dx_router, row_of in; dx out
        return tk * row + (T * row if w.S else 0) + 4 * T * H + 4 * tk + T * row
    if name == "route_permute_bwd":  # both, without dx_router's write and read (and row_of once)
        return row_op_bytes(w, "route_bwd") + row_op_bytes(w, "permute_bwd") - 8 * T * H - 4 * tk
    raise KeyError(name)


def gemm_launch_flops(w, name):
    """Useful (padding-free) flops of one grouped-GEMM launch: 2*rows*N*K with
    rows = T*K routed rows, or T for the shared experts (one group of width S*F)."""
    shared = name.startswith("shared_")
    rows = w.T if shared else w.T * w.K
    F = w.S * w.F if shared else w.F
    mult = 2 if "gate_up" in name else 1      # gate/up GEMMs have 2F columns (or K = 2F)
    return 2.0 * rows * w.H * F * mult


def gemm_launch_bytes(w, name, live=None):
    """Algorithmic HBM bytes of one launch: every operand read once and every
    result written once, bf16, padding rows excluded.  `live` is the number of
    routed experts that own rows (default all E): the forward and data-gradient
    products read only their weights, while the weight gradients write all E
    (zeros for an expert without rows)."""
    shared = name.startswith("shared_")
    rows = w.T if shared else w.T * w.K
    G = 1 if shared else w.E
    if not shared and live is not None and not name.endswith("wgrad"):
        G = live
    F = w.S * w.F if shared else w.F
    H = w.H
    wt = 2 * G * 2 * F * H if "gate_up" in name else 2 * G * H * F      # one weight tensor
    if name.endswith("gate_up_fwd"):
        return rows * H * 2 + wt + rows * 3 * F * 2          # x rows; act (2F) + h (F)
    if name.endswith("down_fwd"):
        return rows * F * 2 + wt + rows * H * 2              # h; y rows
    if name.endswith("down_dgrad"):
        return rows * H * 2 + wt + rows * 2 * F * 2 * 2      # dy rows; act in, dact out
    if name.endswith("gate_up_dgrad"):
        return rows * 2 * F * 2 + wt + rows * H * 2          # dact; dx rows
    if name.endswith("down_wgrad"):
        return rows * H * 2 + rows * F * 2 + wt              # dy rows, h; dW2
    return rows * 2 * F * 2 + rows * H * 2 + wt              # dact, x rows; dW1


def _elementwise_err(a, r):
    """max_i |a_i - r_i| / max(|r_i|, rms(r)): the parity tests' element-wise
    relative error."""
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(a - r) / np.maximum(np.abs(r), rms)))


def cpu_baseline(w, g, gpu=None, budget_s=20.0, first_tokens=512):
    """The CPU oracle, untouched, on the first n tokens of the batch (forward,
    plus backward for the fwd+bwd workload), in the same unit (useful
    TFLOP/s).  The inputs are handed over as fp32 arrays, converted before the
    clock starts.  A first run on `first_tokens` tokens measures the host; n
    is then chosen so that the reported run takes about `budget_s` seconds (at
    most the whole batch).  With `gpu` (the GPU step's y, dx and topk_idx of
    every token) it also reports their agreement on the timed tokens: routing
    (near-ties counted apart) and the element-wise relative error of y and dx
    on the tokens whose routing agrees."""
    import torch
    from oracle import moe_oracle as O
    from fine_grained_moe_amd.synthetic import useful_flops
    tn = lambda t: t.detach().float().cpu().numpy()
    E = g["w1"].shape[0]
    W1 = np.empty(tuple(g["w1"].shape), np.float32)
    W2 = np.empty(tuple(g["w2"].shape), np.float32)
    for e in range(E):
        W1[e] = tn(g["w1"][e])
        W2[e] = tn(g["w2"][e])
    x_all, dy_all = tn(g["x"]), (tn(g["dy"]) if "dy" in g else None)
    backward = bool(w.backward) and dy_all is not None   # the workload's own direction

    def run(n):
        sub = dict(x=x_all[:n], w_router=tn(g["w_router"]), bias=tn(g["bias"]), w1=W1, w2=W2,
                   w1_sh=tn(g["w1_sh"]), w2_sh=tn(g["w2_sh"]))
        t0 = time.perf_counter()
        fwd = O.forward(sub, w.K, 128)
        bwd = O.backward(sub, fwd, dy_all[:n]) if backward else None
        return time.perf_counter() - t0, fwd, bwd

    # two sizing runs: the oracle's time is a fixed part (it converts every
    # expert's weights to fp64 once per pass) plus a part per token
    n0 = min(first_tokens, w.T)
    t0, fwd, bwd = run(n0)
    n, dt, first = n0, t0, [(n0, t0)]
    if w.T > n0:
        del fwd, bwd
        n1 = min(w.T, 2 * n0)
        t1, fwd, bwd = run(n1)
        first.append((n1, t1))
        per_token = max((t1 - t0) / (n1 - n0), 1e-9)
        fixed = max(t0 - n0 * per_token, 0.0)
        n, dt = n1, t1
        target = min(w.T, max(n1, int((budget_s - fixed) / per_token) // 64 * 64))
        if target > n1:
            del fwd, bwd
            n = target
            dt, fwd, bwd = run(n)
    flops = useful_flops(w.with_(T=n), backward)
    cores = len(os.sched_getaffinity(0))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    res = dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cores, cpu_model=cpu_model,
               kind="oracle",
               sample=(f"fp64 NumPy oracle, {'forward+backward' if backward else 'forward'} of the "
                       f"first {n} of the {w.T} tokens at the same shapes (all {E} experts' "
                       f"weights), one run, {dt:.1f} s, sized by runs of "
                       + ", ".join(f"{a} tokens ({b:.1f} s)" for a, b in first if a != n)
                       + f"; inputs converted to fp32 beforehand; "
                       f"BLAS threads {torch.get_num_threads()}"),
               seconds=dt, tokens=n)
    if gpu is not None:
        tie = np.asarray(fwd["route"]["near_tie"], bool)
        same = np.all(gpu["topk_idx"][:n] == fwd["route"]["topk_idx"], axis=1)
        par = {"tokens": int(n), "near_ties": int(tie.sum()),
               "routing_differs_outside_near_ties": int((~same & ~tie).sum()),
               "y_elementwise_rel_err": _elementwise_err(gpu["y"][:n][same], fwd["y"][same])}
        if backward:
            par["dx_elementwise_rel_err"] = _elementwise_err(gpu["dx"][:n][same], bwd["dx"][same])
        res["parity"] = par
    return res


SHARD_GEMMS = ("gate_up_fwd", "down_fwd", "down_dgrad", "gate_up_dgrad", "down_wgrad",
               "gate_up_wgrad")


def shard_main(args):
    """The six routed grouped-GEMM launches of one fwd+bwd step at the
    expert-parallel shard shape (rows already grouped by expert, as the
    dispatch exchange delivers them)."""
    import torch
    from fine_grained_moe_amd import moe as M
    from fine_grained_moe_amd.synthetic import EP_SHARD, Workload, generate_shard_torch
    E, R, H, F = EP_SHARD["E"], EP_SHARD["rows"], EP_SHARD["H"], EP_SHARD["F"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = generate_shard_torch(dev, E, R, H, F, EP_SHARD["seed"])
    A = M.moe_align()
    i32 = torch.int32
    offsets = torch.arange(E + 1, dtype=i32, device=dev) * R
    counts = torch.full((E,), R, dtype=i32, device=dev)
    tile_expert = (torch.arange(E * R // A, dtype=i32, device=dev) // (R // A)).to(i32)
    seg = (offsets, counts, tile_expert)
    bf = torch.bfloat16
    act = torch.empty((E * R, 2 * F), dtype=bf, device=dev)
    h = torch.empty((E * R, F), dtype=bf, device=dev)
    y_rows = torch.empty((E * R, H), dtype=bf, device=dev)
    dact = torch.empty_like(act)
    dx_rows = torch.empty_like(g["x_rows"])
    dw1 = torch.empty_like(g["w1"])
    dw2 = torch.empty_like(g["w2"])
    fns = {
        "gate_up_fwd": lambda: M.moe_grouped_gate_up_fwd(g["x_rows"], g["w1"], *seg, act=act, h=h),
        "down_fwd": lambda: M.moe_grouped_down_fwd(h, g["w2"], *seg, y_rows=y_rows),
        "down_dgrad": lambda: M.moe_grouped_down_dgrad(g["w2"], act, g["dy_rows"], *seg, dact=dact),
        "gate_up_dgrad": lambda: M.moe_grouped_gate_up_dgrad(g["w1"], dact, *seg, dx_rows=dx_rows),
        "down_wgrad": lambda: M.moe_grouped_down_wgrad(g["dy_rows"], h, E, *seg, dw2=dw2),
        "gate_up_wgrad": lambda: M.moe_grouped_gate_up_wgrad(dact, g["x_rows"], E, *seg, dw1=dw1),
    }
    for _ in range(args.warmup):
        for n in SHARD_GEMMS:
            fns[n]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for n in SHARD_GEMMS} for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        for n in SHARD_GEMMS:
            evs[i][n][0].record()
            fns[n]()
            evs[i][n][1].record()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    launch_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in SHARD_GEMMS}
    # the shard's rows stand for T*K routed rows of the layer: T = E*R/K with K = 6
    w = Workload("ep_shard", T=E * R // 6, H=H, E=E, K=6, S=0, F=F, seed=EP_SHARD["seed"])
    fl = {n: gemm_launch_flops(w, n) for n in SHARD_GEMMS}
    flops = sum(fl.values())
    tflops = flops / (ms * 1e-3) / 1e12
    dom = max(SHARD_GEMMS, key=lambda n: launch_ms[n])
    out = {
        "metric": "grouped expert GEMMs, useful TFLOP/s at the expert-parallel shard (fwd+bwd)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"grouped SwiGLU expert GEMMs fwd+bwd at one GPU's share of an "
                                f"8-way expert-parallel dots.llm1 layer: {E} experts x {R} rows, "
                                f"H={H}, F={F}"), "E": E, "rows_per_expert": R, "H": H, "F": F},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline_of(dom, w, launch_ms[dom], traffic=False),
        "gemm_launches": {n: {"ms": round(launch_ms[n], 4),
                              "tflops": round(fl[n] / (launch_ms[n] * 1e-3) / 1e12, 1)}
                          for n in SHARD_GEMMS},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = shard_cpu_baseline(g, R, F, w, n_experts=8)
    print(json.dumps(out), flush=True)


def shard_cpu_baseline(g, R, F, w, n_experts):
    """The oracle's expert forward and backward on all rows of the first
    n_experts experts of the shard (same unit: useful TFLOP/s)."""
    import torch
    from oracle import moe_oracle as O
    dt = 0.0
    for e in range(n_experts):
        x = g["x_rows"][e * R:(e + 1) * R].float().cpu().numpy()
        w1 = g["w1"][e].float().cpu().numpy()
        w2 = g["w2"][e].float().cpu().numpy()
        dy = g["dy_rows"][e * R:(e + 1) * R].float().cpu().numpy()
        t0 = time.perf_counter()
        a, _, _ = O.expert_ffn(x, w1, w2)
        O.expert_ffn_bwd(x, w1, w2, a, dy)
        dt += time.perf_counter() - t0
    flops = 18.0 * n_experts * R * w.H * F
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=len(os.sched_getaffinity(0)),
                kind="oracle", seconds=dt,
                sample=(f"fp64 NumPy oracle, forward+backward of {n_experts} of the {w.E} experts "
                        f"(all {R} rows each), {dt:.1f} s; BLAS threads {torch.get_num_threads()}"))


FORWARD_CONFIGS = ("decode", "prefill", "skew")


def forward_config(M, name, steps, warmup):
    """One forward configuration (its own seeded inputs): the whole forward
    timed over `steps` steps (eager, and captured as one graph), every
    grouped-GEMM launch and routing/permutation/combine call by its own
    events, the dominant launch against its roofline."""
    import torch
    from fine_grained_moe_amd.synthetic import WORKLOADS, generate_torch, useful_flops
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    g = generate_torch(w, dev, with_dy=False)
    layer = Layer(M, g, w.K)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.forward()
    torch.cuda.synchronize()
    names = Layer.GEMMS[:4]
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for n in names + ROW_OPS_FWD} for _ in range(steps)]
    for i in range(steps):
        layer.forward(evs[i])
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record(stream)
    for _ in range(steps):
        layer.forward()
    f1.record(stream)
    torch.cuda.synchronize()
    ms = f0.elapsed_time(f1) / steps
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        layer.forward()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward()
    graph.replay()
    torch.cuda.synchronize()
    f0.record(stream)
    for _ in range(steps):
        graph.replay()
    f1.record(stream)
    torch.cuda.synchronize()
    graph_ms = f0.elapsed_time(f1) / steps
    del graph
    # the forward as the layer runs it: one graph, the shared experts'
    # products on a second stream beside the routing and routed products
    side2 = torch.cuda.Stream()
    layer.step_two_streams(side2, backward=False)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step_two_streams(side2, backward=False)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    f0.record(stream)
    for _ in range(steps):
        graph.replay()
    f1.record(stream)
    torch.cuda.synchronize()
    ms2 = f0.elapsed_time(f1) / steps
    del graph
    launch_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in names}
    row_us = {n: 1e3 * float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs]))
              for n in ROW_OPS_FWD}
    live = int((layer.b["perm"]["counts"] > 0).sum().item())
    dom = max(names, key=lambda n: launch_ms[n])
    tf = useful_flops(w, False) / (ms2 * 1e-3) / 1e12
    res = {"workload": (f"dots.llm1 MoE FFN layer forward, T={w.T}, H={w.H}, {w.E} routed experts "
                        f"of width {w.F}, top-{w.K}, {w.S} shared experts"
                        + (", Zipf(1.2) selection bias" if w.bias_kind == "zipf" else "")),
           "T": w.T, "seed": w.seed, "ms": round(ms2, 4), "tflops": round(tf, 2),
           "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
           "schedule": "HIP graph, two streams", "eager_ms": round(ms, 4),
           "graph_one_stream_ms": round(graph_ms, 4), "routed_nonempty_experts": live,
           "roofline": roofline_of(dom, w, launch_ms[dom], traffic=False, live=live),
           "gemm_launches": {n: {"ms": round(launch_ms[n], 4),
                                 "tflops": round(gemm_launch_flops(w, n) / (launch_ms[n] * 1e-3) / 1e12, 1),
                                 "algorithmic_gb": round(gemm_launch_bytes(w, n, live) / 1e9, 3)}
                             for n in names},
           "row_ops_us": {n: round(row_us[n], 2) for n in ROW_OPS_FWD}}
    del layer, g
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the layer's multi-GPU "
              "sharding (expert parallel all-to-all) is not built", file=sys.stderr)
        sys.exit(2)
    if args.workload == "ep_shard":
        return shard_main(args)
    import torch
    from fine_grained_moe_amd import moe as M
    from fine_grained_moe_amd.synthetic import WORKLOADS, generate_torch, useful_flops, gemm_useful_flops

    w = WORKLOADS[args.workload]
    backward = args.workload == "fwdbwd"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = generate_torch(w, dev, with_dy=True)
    layer = Layer(M, g, w.K)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        # one plain copy kernel reading and writing exactly 2^30 bytes each
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        layer.forward(ev)
        if backward:
            layer.backward(ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # eager steps with an event pair around every grouped-GEMM launch and
    # every routing / permutation / combine call: each launch has the card to
    # itself, so these time each kernel alone (the roofline entry's source)
    names = Layer.GEMMS if backward else Layer.GEMMS[:4]
    row_names = ROW_OPS_FWD + (ROW_OPS_BWD if backward else ())
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for n in names + row_names} for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms = t_start.elapsed_time(t_end) / args.steps
    launch_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in names}
    gemm_ms = sum(launch_ms.values())
    row_us = {n: 1e3 * float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs]))
              for n in row_names}

    # forward alone, eager, timed the same way
    torch.cuda.synchronize()
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        layer.forward()
    f1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / args.steps

    def timed_replays(graph):
        """W untimed replays, then exactly K timed ones between two events,
        synchronised on both sides, with an event at every step boundary."""
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        marks[0].record(stream)
        for i in range(args.steps):
            graph.replay()
            marks[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
        return marks[0].elapsed_time(marks[-1]) / args.steps, per

    # the step as the layer runs it: captured once as a HIP graph with the
    # independent launches on a second stream (the shared experts' forward
    # and backward beside the router, permute and routed forward; the routed
    # weight gradients beside the routed data gradients), results
    # bit-identical to the eager step.  Its replays are the timed
    # region of the metric; the one-stream graph is timed beside it.
    graph_ms = None
    ms, step_ms, schedule = eager_ms, None, "eager, one stream"
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph_ms, _ = timed_replays(graph)
        del graph
        side2 = torch.cuda.Stream()
        layer.step_two_streams(side2, backward)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer.step_two_streams(side2, backward)
        ms, step_ms = timed_replays(graph)
        schedule = "HIP graph, two streams"
        del graph
    else:
        step_ms = [ms] * args.steps

    # the step with load balancing (balance loss forward/backward, its dense
    # router gradients, the bias step), and each of those launches
    bal = None
    if backward and not args.no_balance:
        def bal_step(ev=None):
            layer.forward(ev, balance=True)
            layer.backward(ev, balance=True)
        for _ in range(2):
            bal_step()
        bevs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for n in BALANCE_OPS} for _ in range(args.steps)]
        torch.cuda.synchronize()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for i in range(args.steps):
            bal_step(bevs[i])
        b1.record(stream)
        torch.cuda.synchronize()
        bal_ms = b0.elapsed_time(b1) / args.steps
        op_us = {n: 1e3 * float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in bevs]))
                 for n in BALANCE_OPS}
        # the two fp32 products (useful flops) run as 6 + 3 bf16 part products
        dense_flops = 2 * 2.0 * w.T * w.H * w.E
        dense_tf = dense_flops / (op_us["route_bwd_dense"] * 1e-6) / 1e12
        part_tf = dense_flops / 2 * (6 + 3) / (op_us["route_bwd_dense"] * 1e-6) / 1e12
        bal = {"seq_len": SEQ_LEN, "alpha": ALPHA, "gamma": GAMMA,
               "ms_per_step": round(bal_ms, 4),
               "extra_ms": round(bal_ms - eager_ms, 4),   # both eager
               **{f"{n}_us": round(op_us[n], 2) for n in BALANCE_OPS},
               "route_bwd_dense_roofline": {"bound": "mfma", "achieved": round(part_tf, 2),
                                            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                            "frac": round(part_tf / PEAK_BF16_TFLOPS, 4),
                                            "fp32_equivalent_tflops": round(dense_tf, 2)}}

    flops = useful_flops(w, backward)
    tflops = flops / (ms * 1e-3) / 1e12
    fwd_tflops = useful_flops(w, False) / (fwd_ms * 1e-3) / 1e12
    gemm_flops = gemm_useful_flops(w, backward)
    # the dominant kernel: the grouped-GEMM launch with the longest average time
    dom = max(names, key=lambda n: launch_ms[n])
    counts = layer.b["perm"]["counts"].cpu().numpy()
    live = int((counts > 0).sum())
    launches = {n: {"ms": round(launch_ms[n], 4),
                    "tflops": round(gemm_launch_flops(w, n) / (launch_ms[n] * 1e-3) / 1e12, 1),
                    "algorithmic_gb": round(gemm_launch_bytes(w, n, live) / 1e9, 3)} for n in names}

    out = {
        "metric": "MoE layer useful TFLOP/s at T=8192 (fwd, fwd+bwd); % of bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(np.min(step_ms)), 4),
        "schedule": schedule,
        "eager_ms_per_step": round(eager_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"dots.llm1 MoE FFN layer {'forward+backward' if backward else 'forward'}"
                                f", T={w.T}, H={w.H}, {w.E} routed experts of width {w.F}, top-{w.K}"
                                f", {w.S} shared experts"),
                   "T": w.T, "H": w.H, "E": w.E, "F": w.F, "K": w.K, "S": w.S, "seed": w.seed},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_ms": round(fwd_ms, 4),
        "fwd_pct_of_bf16_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "gemm_pct_of_bf16_peak": round(100 * gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "gemm_ms": round(gemm_ms, 4),
        "graph_one_stream_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "routed_nonempty_experts": live,
        "roofline": roofline_of(dom, w, launch_ms[dom], live=live),
        "gemm_launches": launches,
        # routing, permutation and combine: algorithmic bytes (every input read
        # once, every output written once) over the call's time, against 8 TB/s
        "row_ops": {n: {"us": round(row_us[n], 2),
                        "algorithmic_gb": round(row_op_bytes(w, n) / 1e9, 4),
                        "gbs": round(row_op_bytes(w, n) / (row_us[n] * 1e-6) / 1e9, 1),
                        "frac_of_hbm_peak": round(row_op_bytes(w, n) / (row_us[n] * 1e-6) / 1e9
                                                  / PEAK_HBM_GBS, 4)}
                    for n in row_names},
    }
    if bal is not None:
        out["load_balancing"] = bal
    gpu_out = None
    if not args.no_cpu_baseline:
        # the plain step once more, so that y and dx hold its outputs (the
        # balance loop changed dx); a token's y and dx depend on that token
        # only, so the oracle's run on the first tokens checks them
        step()
        torch.cuda.synchronize()
        gpu_out = {"y": layer.b["y"].float().cpu().numpy(),
                   "topk_idx": layer.b["topk_idx"].cpu().numpy()}
        if backward:
            gpu_out["dx"] = layer.b["dx"].float().cpu().numpy()
    if backward and not args.no_configs:
        # the other configurations of the layer, forward only, each on its own
        # seeded inputs (the step's buffers freed first)
        del layer
        torch.cuda.empty_cache()
        out["configs"] = {n: forward_config(M, n, max(args.steps // 2, 5), 3)
                          for n in FORWARD_CONFIGS}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, g, gpu_out, budget_s=args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
