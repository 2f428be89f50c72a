"""The layer's forward and backward captured in a HIP graph (through
torch.cuda.CUDAGraph on a stream of their own) and replayed: every replay
must reproduce the eager result bit for bit (both paths are deterministic).
Eager work runs between the replays, which are checked one by one. The
backward's side stream (router and down-projection weight gradients) is
forked and joined inside the graph by the events of the call."""
import numpy as np
import pytest

from sparse_mixture_experts_20_amd import workloads as W
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_mod():
    if not G.have_gpu():
        pytest.skip("no HIP device")
    import torch
    from sparse_mixture_experts_20_amd import binding as B
    B.lib()
    return torch


@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_graph_replays_match_eager(torch_mod, act):
    torch = torch_mod
    from sparse_mixture_experts_20_amd import binding as B
    from sparse_mixture_experts_20_amd import device as D
    wl = W.custom(f"graph_{act}", N=1024, d=256, E=8, k=2, d_ff=512, dtype="bf16", cf=1.0,
                  sigma=0.5, seed=501, w_std=0.05, act=act,
                  bias_std=0.05 if act == "gelu" else 0.0)
    G.say(f"[graph] {wl.cfg.name}: N={wl.N} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff}")
    dev = D.upload(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dout = torch.from_numpy(wl.dout().view(np.int16)).view(torch.bfloat16).to("cuda")
        fwd = B.Forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                        wl.cfg.cf, stream=s, act=act, b_up=dev["b_up"], b_down=dev["b_down"])
        bwd = B.Backward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                         wl.cfg.cf, dout, stream=s, act=act, b_up=dev["b_up"],
                         b_down=dev["b_down"])

        def step():
            out = fwd()
            grads = bwd()
            return out, grads

        # eager reference (this also creates the library's side stream)
        out, grads = step()
        outs = [out] + list(grads)
        names = ["out", "dx", "dW_g", "dW_up", "dW_down"]
        if act == "gelu":
            outs += [bwd.db_up, bwd.db_down]
            names += ["db_up", "db_down"]
        ref = [t.clone() for t in outs]
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between the replays: scribble over the results
        with torch.cuda.stream(s):
            for t in outs:
                t.fill_(float("nan") if t.dtype == torch.float32 else 7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, outs, ref):
            assert torch.equal(got, want), (rep, name)
        G.say(f"[graph] replay {rep}: out and every gradient bit-identical to eager")
    del graph, fwd, bwd, dev
    torch.cuda.synchronize()
