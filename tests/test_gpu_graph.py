"""The entry points enqueue plain kernel launches on the caller's stream and
allocate nothing, so a captured HIP graph replays them.  Each replay here
starts from the same pool and buffers (restored outside the graph), runs
between eager work and synchronisations, and must reproduce the eager
result byte for byte."""
import pytest
import torch

from speculative_decode_amd import ops, workloads

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.load_library()
    return torch.device("cuda:0")


def _graph_matches_eager(dev, run, state, out):
    """run() updates `state` in place and writes `out`; both compared."""
    state0 = state.clone()
    out0 = out.clone()
    run()                                            # eager reference
    torch.cuda.synchronize()
    want_state, want_out = state.clone(), out.clone()

    s = torch.cuda.Stream()                          # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm-up on the capture stream
        state.copy_(state0)
        out.copy_(out0)
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(REPLAYS):
        state.copy_(state0)
        out.copy_(out0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, want_state), f"replay {i}: pool differs"
        assert torch.equal(out, want_out), f"replay {i}: out differs"
        _ = (state0.float().sum() + 1.0).item()      # eager work between replays


@pytest.mark.parametrize("name", ["mtp_b32", "mixed_b128", "mtp_b128_f8"])
def test_decode_update_in_graph(dev, name):
    b = workloads.make(name)
    kw = ops.batch_args(b, dev)
    kw["out"] = torch.zeros((b.n_tok, b.HV, b.V), dtype=b.out_dtype, device=dev)
    _graph_matches_eager(dev, lambda: ops.forward_core(**kw), kw["state"], kw["out"])


def test_conv_update_in_graph(dev):
    b = workloads.make_conv("conv_mtp_b128")
    kw = ops.conv_batch_args(b, dev)
    kw["out"] = torch.zeros(b.x.shape, dtype=b.out_dtype, device=dev)
    _graph_matches_eager(dev, lambda: ops.conv_spec_update(**kw), kw["cache"], kw["out"])


def test_prefill_update_in_graph(dev):
    b = workloads.make_prefill("prefill_small")
    kw = ops.prefill_batch_args(b, dev)
    kw["out"] = torch.zeros((b.n_tok, b.HV, b.V), dtype=b.out_dtype, device=dev)
    _graph_matches_eager(dev, lambda: ops.prefill_update(**kw), kw["state"], kw["out"])
