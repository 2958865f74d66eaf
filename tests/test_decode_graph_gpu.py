"""Decode steps captured in a HIP graph: every replay, with eager work and synchronisation
between replays, must equal the same steps launched one by one, bit for bit."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_gla_amd as m
    m.lib()
    return m


def test_graph_replays_equal_eager(gla):
    import torch
    w = W.WORKLOADS["decode"]
    T = 8
    dd = W.decode_inputs(w, T=T, B=8)
    dt = torch.bfloat16
    qs, ks, vs, gs = (torch.from_numpy(dd[n]).to("cuda", dt) for n in ("q", "k", "v", "g"))
    state0 = torch.from_numpy(dd["state"]).cuda()
    state = state0.clone()
    o = torch.empty(8, w.H, w.Dv, device="cuda", dtype=dt)

    def run_all():
        for t in range(T):
            gla.gla_decode_step(qs[t], ks[t], vs[t], gs[t], state, out=o)

    run_all()
    torch.cuda.synchronize()
    ref_state, ref_o = state.clone(), o.clone()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            run_all()
    torch.cuda.current_stream().wait_stream(cap)
    for replay in range(3):
        state.copy_(state0)
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), f"replay {replay}: state"
        assert torch.equal(o, ref_o), f"replay {replay}: output"
        run_all()                                     # eager work between replays
        torch.cuda.synchronize()
