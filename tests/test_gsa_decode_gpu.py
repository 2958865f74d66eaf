"""GPU parity of the GSA decode step (gsa_decode_step, through the C ABI) against the fp64
oracle: outputs and both in-place slot memories, step after step; continuation of a gsa_fwd
prefill; extreme gates; the full decode batch."""
import numpy as np
import pytest

import workloads as W
from oracle import gsa_decode_step as ref_step
from oracle import gsa_recurrent_fwd
from tests.helpers import assert_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_gla_amd as m
    m.lib()
    return m


def run_chain(gla, d, dt, T, act="softmax"):
    """T steps on the GPU and in the oracle; returns both sides' outputs and final memories."""
    import torch
    hk, hv = dev(d["hk"]), dev(d["hv"])
    rk, rv = d["hk"], d["hv"]
    outs, routs = [], []
    for t in range(T):
        o = gla.gsa_decode_step(dev(d["q"][t], dt), dev(d["k"][t], dt), dev(d["v"][t], dt), dev(d["g"][t], dt),
                                hk, hv, act=act)
        outs.append(o)
        ro, rk, rv = ref_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], rk, rv, act=act)
        routs.append(ro)
    torch.cuda.synchronize()
    return np.stack([host(o) for o in outs]), np.stack(routs), host(hk), rk, host(hv), rv


SHAPES = [
    # (B, H, Dk, Dv, m, dtype)
    (2, 3, 128, 128, 64, "bf16"),
    (1, 2, 16, 16, 16, "bf16"),
    (3, 1, 48, 80, 48, "bf16"),
    (1, 2, 256, 512, 64, "bf16"),
    (2, 2, 64, 96, 128, "bf16"),
    (1, 1, 32, 48, 256, "bf16"),
    (1, 1, 256, 16, 256, "bf16"),
    (2, 2, 128, 128, 64, "f32"),
    (1, 3, 48, 112, 32, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_steps_match_oracle(gla, shape):
    B, H, Dk, Dv, m, dt = shape
    w = W.GsaDecodeWorkload("gsa-dec", 4, B, H, Dk, Dv, m, dt, 600 + Dk + Dv + m)
    d = W.gsa_decode_inputs(w)
    print(f"[gsa decode] B={B} H={H} Dk={Dk} Dv={Dv} m={m} {dt}", flush=True)
    o, ro, hk, rk, hv, rv = run_chain(gla, d, dt, w.T)
    assert_close("o", o, ro, dt)
    # the memories are float32 whatever the token dtype: hold them to the fp32 bound
    assert_close("hk", hk, rk, "f32")
    assert_close("hv", hv, rv, "f32")


@pytest.mark.parametrize("act", ["swish", "relu", "relu2", "none"])
@pytest.mark.parametrize("shape", [(2, 3, 128, 128, 64, "bf16"), (1, 2, 48, 80, 48, "f32"),
                                   (1, 1, 32, 48, 256, "bf16")], ids=lambda s: "x".join(map(str, s)))
def test_read_outs(gla, shape, act):
    """The element-wise read-outs in place of the softmax (o is continuous in z for all)."""
    B, H, Dk, Dv, m, dt = shape
    w = W.GsaDecodeWorkload("gsa-dec-act", 4, B, H, Dk, Dv, m, dt, 620 + Dk + m)
    d = W.gsa_decode_inputs(w)
    print(f"[gsa decode] B={B} H={H} Dk={Dk} Dv={Dv} m={m} {dt} act={act}", flush=True)
    o, ro, hk, rk, hv, rv = run_chain(gla, d, dt, w.T, act)
    assert_close("o", o, ro, dt)
    assert_close("hk", hk, rk, "f32")
    assert_close("hv", hv, rv, "f32")


def test_extreme_gates(gla):
    """g = 0 freezes the memories (bit for bit) and g = -30 overwrites every slot."""
    import torch
    w = W.GsaDecodeWorkload("gsa-dec-gates", 1, 2, 2, 64, 64, 32, "bf16", 611)
    d = W.gsa_decode_inputs(w)
    for gval in (0.0, -30.0):
        g = np.full_like(d["g"][0], gval)
        hk, hv = dev(d["hk"]), dev(d["hv"])
        o = gla.gsa_decode_step(dev(d["q"][0], "bf16"), dev(d["k"][0], "bf16"), dev(d["v"][0], "bf16"),
                                dev(g, "bf16"), hk, hv)
        torch.cuda.synchronize()
        ro, rk, rv = ref_step(d["q"][0], d["k"][0], d["v"][0], g, d["hk"], d["hv"])
        print(f"[gsa decode] g = {gval}", flush=True)
        assert_close("o", host(o), ro, "bf16")
        assert_close("hk", host(hk), rk, "f32")
        assert_close("hv", host(hv), rv, "f32")
        if gval == 0.0:
            assert np.array_equal(host(hk), d["hk"]) and np.array_equal(host(hv), d["hv"])


def test_continues_forward_prefill(gla):
    """gsa_fwd over a prefix, then decode steps from its final memories, equals the oracle's
    recurrence over the whole sequence."""
    import torch
    gw = W.GsaWorkload("gsa-prefill", 1, 2, 100, 64, 64, 32, 64, "bf16", 612)
    y = W.gsa_inputs(gw, with_grad=False)
    P, T = 90, 10
    _, hkt, hvt = gla.gsa_fwd(*(dev(y[n][:, :, :P], "bf16") for n in ("q", "k", "v", "g")), C=64)
    outs = []
    for t in range(P, P + T):
        outs.append(gla.gsa_decode_step(*(dev(y[n][:, :, t], "bf16") for n in ("q", "k", "v", "g")), hkt, hvt))
    torch.cuda.synchronize()
    ro, rhk, rhv = gsa_recurrent_fwd(y["q"], y["k"], y["v"], y["g"])
    print("[gsa decode] prefill 90 + 10 steps", flush=True)
    assert_close("o", np.stack([host(o) for o in outs], axis=2), ro[:, :, P:], "bf16")
    assert_close("hk", host(hkt), rhk, "bf16")
    assert_close("hv", host(hvt), rhv, "bf16")


def test_full_size_batch(gla):
    """The GSA decode workload's whole batch (64 x 4 heads, Dk = Dv = 128, m = 64), in the
    launch configuration the benchmark times, a few steps, every unit."""
    w = W.WORKLOADS["gsa_decode"]
    d = W.gsa_decode_inputs(w, T=3)
    print(f"[gsa decode] full batch B={w.B} H={w.H}", flush=True)
    o, ro, hk, rk, hv, rv = run_chain(gla, d, w.dtype, 3)
    assert_close("o", o, ro, w.dtype)
    assert_close("hk", hk, rk, "f32")
    assert_close("hv", hv, rv, "f32")


def test_deterministic(gla):
    import torch
    w = W.GsaDecodeWorkload("gsa-dec-det", 1, 8, 4, 128, 128, 64, "bf16", 613)
    d = W.gsa_decode_inputs(w)
    res = []
    for _ in range(2):
        hk, hv = dev(d["hk"]), dev(d["hv"])
        o = gla.gsa_decode_step(*(dev(d[n][0], "bf16") for n in ("q", "k", "v", "g")), hk, hv)
        torch.cuda.synchronize()
        res.append((host(o), host(hk), host(hv)))
    for a, b in zip(*res):
        assert np.array_equal(a, b)
