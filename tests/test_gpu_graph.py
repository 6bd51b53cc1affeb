"""The whole layer step captured as one HIP graph (needs an MI355X).

Every entry point only launches kernels on the caller's stream (no device
allocation, memset, copy or synchronisation inside the library), so a
forward + backward step over preallocated buffers can be captured once and
replayed.  Each replay must reproduce the eager step bit for bit: before every
replay the outputs and intermediates are overwritten eagerly with NaN, so a
buffer the graph failed to rewrite shows up, and the eager work and
synchronisation between replays exercise the graph against other work on the
card.
"""
import pytest

from fine_grained_moe_amd.synthetic import WORKLOADS, Workload, generate_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# buffers the step writes in full (the router's [T,H] input gradient only
# with load balancing: without it that gradient is added inside the un-permute)
OUTPUTS = ("y", "dx", "dw1", "dw2", "dw1_sh", "dw2_sh", "dw_router", "dg",
           "act_sh", "dact_sh", "topk_idx", "topk_w", "topk_s")
# row buffers of the routed path: pad rows are never written, only valid rows compare
ROWS = ("act", "h", "y_rows", "dy_rows", "dact", "dx_rows")
BALANCE_OUTPUTS = ("loss", "seq_f", "dlogit_bal", "scores", "bias_train", "dx_router")


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fine_grained_moe_amd import moe
    return moe


def _scribble(b, names):
    for n in names:
        t = b[n]
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _step(layer, balance):
    layer.forward(balance=balance)
    layer.backward(balance=balance)


@pytest.mark.parametrize("case", ["mid", "dots_balance"])
def test_step_graph_replays_match_eager(M, case):
    import bench

    if case == "mid":
        w = Workload("graph-mid", T=1000, H=512, E=16, K=4, S=2, F=352, seed=31,
                     router_std=0.08, bias_std=0.05)
        balance = False
    else:
        w = WORKLOADS["fwdbwd"]           # T = 8192, one sequence of 8192 tokens
        balance = True
        assert w.T % bench.SEQ_LEN == 0
    dev = torch.device("cuda:0")
    g = generate_torch(w, dev, with_dy=True)
    layer = bench.Layer(M, g, w.K)
    names = OUTPUTS + (BALANCE_OUTPUTS if balance else ())
    bias0 = g["bias"].clone()

    # eager reference (twice: the second run is the one kept); the bias step
    # updates bias_train in place, so it is reset before every step
    for _ in range(2):
        layer.b["bias_train"].copy_(bias0)
        _step(layer, balance)
    torch.cuda.synchronize()
    ref = {n: layer.b[n].clone() for n in names}
    valid = layer.b["perm"]["src_token"] >= 0
    ref_rows = {n: layer.b[n][valid].clone() for n in ROWS}

    # capture on a side stream, as torch requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.b["bias_train"].copy_(bias0)
        _step(layer, balance)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(layer, balance)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: overwrite everything the step writes
        _scribble(layer.b, names + ROWS)
        layer.b["bias_train"].copy_(bias0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(layer.b[n], ref[n]), f"{case}: replay {rep}: {n} differs from eager"
        for n in ROWS:
            assert torch.equal(layer.b[n][valid], ref_rows[n]), f"{case}: replay {rep}: {n} rows differ"
    del graph


def test_two_stream_step_matches_eager(M):
    """The step with its independent launches on a second stream, eager and
    captured as one graph (the streams become parallel branches), equals the
    one-stream step bit for bit."""
    import bench

    w = Workload("graph-2s", T=1000, H=512, E=16, K=4, S=2, F=352, seed=32,
                 router_std=0.08, bias_std=0.05)
    dev = torch.device("cuda:0")
    g = generate_torch(w, dev, with_dy=True)
    layer = bench.Layer(M, g, w.K)
    names = OUTPUTS
    _step(layer, False)
    torch.cuda.synchronize()
    ref = {n: layer.b[n].clone() for n in names}
    valid = layer.b["perm"]["src_token"] >= 0
    ref_rows = {n: layer.b[n][valid].clone() for n in ROWS}

    side = torch.cuda.Stream()
    _scribble(layer.b, names + ROWS)
    layer.step_two_streams(side)
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(layer.b[n], ref[n]), f"two streams, eager: {n} differs"
    for n in ROWS:
        assert torch.equal(layer.b[n][valid], ref_rows[n]), f"two streams, eager: {n} rows differ"

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step_two_streams(side)
    torch.cuda.synchronize()
    for rep in range(3):
        _scribble(layer.b, names + ROWS)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(layer.b[n], ref[n]), f"two streams, replay {rep}: {n} differs"
        for n in ROWS:
            assert torch.equal(layer.b[n][valid], ref_rows[n]), f"two streams, replay {rep}: {n} rows"
    del graph
