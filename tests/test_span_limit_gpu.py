"""GPU parity of the factorised intra-chunk path near its limit.

A chunk takes the factorised form (decayed queries times inversely decayed keys on the matrix
cores) when every |b| in it, the chunk-local prefix sum of the gates in log2 units, is at most
32; the inversely decayed keys then reach 2^32 and the products lean on the hi/lo operand
splits.  The gates below put each chunk's span just under that bound for every chunk size
(C |g| log2(e) between 31.3 and 31.95 after bf16 rounding): uniform over all key channels, and
mixed with ordinary channels.  Forward, backward, the saved-activation path and GSA are
compared with the fp64 oracle at the usual bound.
"""
import numpy as np
import pytest

import workloads as W
from oracle import gla_recurrent_bwd, gla_recurrent_fwd, gsa_recurrent_bwd, gsa_recurrent_fwd
from tests.helpers import assert_close, dev, host

pytestmark = pytest.mark.gpu

# gate value per chunk size: C * |g| * log2(e) just under 32
G_LIMIT = {16: -1.38, 32: -0.69, 64: -0.34, 128: -0.17}
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def gla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_gla_amd as m
    m.lib()
    return m


def limit_gates(x, C, dtype, mix, spread=0.0):
    """Gates at the span limit on every key channel (mix=False) or on every other one, the rest
    keeping the workload's own law (mix=True).  spread > 0 scales channel j's limit gate by
    1 - spread * j / width, so that no two channels share a gate (GSA's slots, below)."""
    g = x["g"].copy()
    width = g.shape[-1]
    gl = np.float32(G_LIMIT[C]) * (1.0 - spread * np.arange(width, dtype=np.float32) / width)
    if mix:
        g[..., ::2] = gl[::2]
    else:
        g[:] = gl
    g = W.round_bf16(g) if dtype == "bf16" else g
    assert 31.0 < max_span(g, C) <= 31.98      # the fast path, within a unit of its bound
    return g


def max_span(g, C):
    """Largest |b| over all chunks: b is each chunk's inclusive prefix sum of g, in log2 units."""
    L = g.shape[2]
    pad = (-L) % C
    gp = np.pad(g.astype(np.float64), [(0, 0), (0, 0), (0, pad), (0, 0)])
    gp = gp.reshape(g.shape[0], g.shape[1], -1, C, g.shape[3])
    return float(np.max(np.abs(np.cumsum(gp, axis=3)))) * LOG2E


CASES = [
    # (B, H, L, Dk, Dv, C, dtype, mix)
    (1, 2, 200, 64, 64, 64, "bf16", False),
    (1, 2, 200, 64, 64, 64, "bf16", True),
    (2, 2, 150, 128, 256, 64, "bf16", True),
    (1, 2, 300, 128, 128, 128, "bf16", False),
    (1, 2, 300, 64, 96, 128, "bf16", True),
    (1, 2, 130, 64, 64, 32, "bf16", False),
    (2, 1, 140, 128, 64, 32, "bf16", True),
    (1, 2, 90, 64, 48, 16, "bf16", False),
    (1, 2, 90, 32, 64, 16, "bf16", True),
    (1, 2, 150, 64, 64, 64, "f32", False),
    (1, 2, 150, 48, 32, 32, "f32", True),
    (1, 1, 100, 32, 32, 16, "f32", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda s: "x".join(map(str, s)))
def test_gla_at_span_limit(gla, case):
    import torch
    B, H, L, Dk, Dv, C, dt, mix = case
    w = W.GlaWorkload("span", B, H, L, Dk, Dv, C, dt, 500 + L + Dk + C, h0=True, gate_law="iid")
    x = W.gla_inputs(w)
    x["g"] = limit_gates(x, C, dt, mix)
    q, k, v, g, do = (dev(x[n], dt) for n in ("q", "k", "v", "g", "do"))
    h0, dht = dev(x["h0"]), dev(x["dht"])
    print(f"[span] B={B} H={H} L={L} Dk={Dk} Dv={Dv} C={C} {dt} mix={mix} g={G_LIMIT[C]}", flush=True)
    ro, rht = gla_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["h0"])
    o, ht = gla.gla_fwd(q, k, v, g, C=C, h0=h0)
    assert_close("o", host(o), ro, dt)
    assert_close("ht", host(ht), rht, dt)
    if dt == "f32" and C == 128:
        return                                  # fp32 has no C = 128 backward
    ref = gla_recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["do"], x["h0"], x["dht"])
    grads = gla.gla_bwd(q, k, v, g, do, C=C, h0=h0, dht=dht, want_dh0=True)
    for name, got in zip(("dq", "dk", "dv", "dg", "dh0"), grads):
        assert_close(name, host(got), ref[name], dt)
    # the saved-activation path (the training step's form)
    so, sht, saved = gla.gla_fwd_save(q, k, v, g, C=C, h0=h0)
    sgrads = gla.gla_bwd_saved(q, k, v, g, do, saved, C=C, h0=h0, dht=dht, want_dh0=True)
    torch.cuda.synchronize()
    assert_close("saved o", host(so), ro, dt)
    for name, got in zip(("dq", "dk", "dv", "dg", "dh0"), sgrads):
        assert_close("saved " + name, host(got), ref[name], dt)


GSA_CASES = [
    # (B, H, L, Dk, Dv, m, C, dtype, mix)
    (1, 2, 200, 64, 64, 32, 64, "bf16", False),
    (1, 2, 200, 64, 64, 64, 64, "bf16", True),
    (1, 2, 130, 64, 96, 32, 32, "bf16", False),
    (2, 1, 90, 32, 32, 16, 16, "bf16", True),
    (1, 2, 100, 64, 64, 32, 32, "f32", True),
]


@pytest.mark.parametrize("case", GSA_CASES, ids=lambda s: "x".join(map(str, s)))
def test_gsa_at_span_limit(gla, case):
    """GSA's slot gates drive both passes' chunk spans to the limit: slot j's gate is the limit
    gate times 1 - 0.9 j / m, so the first slot's span sits just under the bound and the others
    spread down to a tenth of it.  Slots whose gates (nearly) coincide keep (nearly) the same
    memory; the softmax's gradient dZ = P (dP - <dP, P>) then cancels, and what is left of it
    carries the rounding of the bf16 chunk-start states at a large relative size.  One gate
    shared by every slot makes that cancellation total, a degenerate input for any chunk form
    that keeps its states in bf16 (dq off by 1.4e-2 of its largest value at g = -0.05, far from
    the span limit)."""
    B, H, L, Dk, Dv, m, C, dt, mix = case
    w = W.GsaWorkload("span", B, H, L, Dk, Dv, m, C, dt, 600 + L + m + C, h0=True)
    x = W.gsa_inputs(w)
    x["g"] = limit_gates(x, C, dt, mix, spread=0.9)
    args = [dev(x[n], dt) for n in ("q", "k", "v", "g")]
    hk0, hv0 = dev(x["hk0"]), dev(x["hv0"])
    print(f"[gsa span] B={B} H={H} L={L} Dk={Dk} Dv={Dv} m={m} C={C} {dt} mix={mix}", flush=True)
    o, hkt, hvt = gla.gsa_fwd(*args, C=C, hk0=hk0, hv0=hv0)
    ro, rhk, rhv = gsa_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["hk0"], x["hv0"])
    assert_close("o", host(o), ro, dt)
    assert_close("hkt", host(hkt), rhk, dt)
    assert_close("hvt", host(hvt), rhv, dt)
    grads = gla.gsa_bwd(*args, dev(x["do"], dt), C=C, hk0=hk0, hv0=hv0, dhkt=dev(x["dhkt"]),
                        dhvt=dev(x["dhvt"]), want_dh0=True)
    rb = gsa_recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["do"], x["hk0"], x["hv0"], x["dhkt"], x["dhvt"])
    for name, got in zip(("dq", "dk", "dv", "dg", "dhk0", "dhv0"), grads):
        assert_close(name, host(got), rb[name], dt)
