"""GPU parity of the saved-activation path (gla_fwd_save then gla_bwd_saved, through the C
ABI): the forward outputs equal gla_fwd's bit for bit, and the gradients match the fp64
oracle's reverse sweep to the same bound as gla_bwd."""
import numpy as np
import pytest

import workloads as W
from oracle import gla_recurrent_bwd, gla_recurrent_fwd
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


def check_saved(gla, w, x, units=None, with_dht=True):
    import torch
    dt = w.dtype
    q, k, v, g, do = (dev(x[n], dt) for n in ("q", "k", "v", "g", "do"))
    h0 = dev(x["h0"])
    dht = dev(x["dht"]) if with_dht else None
    o, ht, saved = gla.gla_fwd_save(q, k, v, g, C=w.C, h0=h0)
    o_ref, ht_ref = gla.gla_fwd(q, k, v, g, C=w.C, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref), "gla_fwd_save differs from gla_fwd"
    dq, dk, dv, dg, dh0 = (host(t) for t in gla.gla_bwd_saved(q, k, v, g, do, saved, C=w.C, h0=h0, dht=dht,
                                                             want_dh0=True))
    sel = (slice(None), slice(None)) if units is None else units
    rh0 = None if x["h0"] is None else x["h0"][sel]
    rdht = x["dht"][sel] if with_dht else None
    ref = gla_recurrent_bwd(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], x["do"][sel], rh0, rdht)
    print(f"[{w.name}] B={w.B} H={w.H} L={x['q'].shape[2]} Dk={w.Dk} Dv={w.Dv} C={w.C} {dt} "
          f"h0={x['h0'] is not None} dht={with_dht}", flush=True)
    ro, rht = gla_recurrent_fwd(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], rh0)
    assert_close("o", host(o)[sel], ro, dt)
    assert_close("ht", host(ht)[sel], rht, dt)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg), ("dh0", dh0)):
        assert_close(name, got[sel], ref[name], dt)


SHAPES = [
    # (B, H, L, Dk, Dv, C, dtype, h0, dht)
    (2, 2, 150, 64, 64, 64, "bf16", True, True),
    (1, 3, 200, 128, 256, 64, "bf16", False, False),
    (2, 1, 77, 16, 48, 16, "bf16", True, True),
    (1, 2, 300, 128, 128, 128, "bf16", True, True),
    (1, 1, 129, 256, 512, 64, "bf16", True, True),
    (2, 4, 130, 256, 512, 64, "bf16", True, True),   # 64-row walk tiles
    (4, 4, 150, 128, 256, 64, "bf16", True, True),   # 32-row walk tiles
    (1, 2, 1, 128, 64, 64, "bf16", True, True),
    (2, 2, 90, 48, 32, 16, "f32", True, True),
    (1, 2, 70, 128, 96, 64, "f32", True, True),
    # the walk and the outputs as one kernel (32-column tiles filling a 256-CU device), which
    # keeps the states for the backward; with 32 value columns (states padded to 64) the plain
    # walk keeps them instead
    (32, 4, 100, 128, 64, 64, "bf16", True, True),
    (64, 4, 100, 128, 32, 64, "bf16", True, True),
    (16, 4, 129, 128, 128, 64, "bf16", True, False),
    (32, 4, 1, 128, 64, 64, "bf16", True, True),     # one token
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(gla, shape):
    B, H, L, Dk, Dv, C, dt, h0, dht = shape
    w = W.GlaWorkload("saved", B, H, L, Dk, Dv, C, dt, 411 + L + Dk, h0=h0, gate_law="iid")
    check_saved(gla, w, W.gla_inputs(w), with_dht=dht)


def test_extreme_gates(gla):
    """Every chunk takes the exact intra-chunk path."""
    w = W.GlaWorkload("saved-gates", 1, 2, 150, 64, 64, 64, "bf16", 419, h0=True, gate_law="iid")
    x = W.gla_inputs(w)
    x["g"] = np.full_like(x["g"], -30.0)
    check_saved(gla, w, x)


def test_full_size_config_sampled(gla):
    """The 340M-layer workload, in the launch configuration the benchmark times."""
    w = W.WORKLOADS["gla_340m"]
    x = W.gla_inputs(w)
    units = (np.array([0, 7])[:, None], np.array([0, 3])[None, :])
    check_saved(gla, w, x, units=units, with_dht=False)


@pytest.mark.parametrize("B,H", [(2, 2), (16, 4)], ids=["walk", "fused-walk-output"])
def test_matches_recomputing_backward(gla, B, H):
    """gla_bwd_saved and gla_bwd agree to within rounding (they differ only in how the
    chunk-start states were accumulated: at B=16, H=4 the saving forward runs the walk and the
    outputs as one kernel, the recomputing backward the plain walk)."""
    import torch
    w = W.GlaWorkload("saved-vs-bwd", B, H, 257, 128, 128, 64, "bf16", 423, h0=True, gate_law="iid")
    x = W.gla_inputs(w)
    q, k, v, g, do = (dev(x[n], "bf16") for n in ("q", "k", "v", "g", "do"))
    h0, dht = dev(x["h0"]), dev(x["dht"])
    _, _, saved = gla.gla_fwd_save(q, k, v, g, C=64, h0=h0)
    a = gla.gla_bwd_saved(q, k, v, g, do, saved, C=64, h0=h0, dht=dht, want_dh0=True)
    b = gla.gla_bwd(q, k, v, g, do, C=64, h0=h0, dht=dht, want_dh0=True)
    torch.cuda.synchronize()
    for name, s, t in zip(("dq", "dk", "dv", "dg", "dh0"), a, b):
        s, t = host(s), host(t)
        e = np.max(np.abs(s - t)) / max(np.max(np.abs(t)), 1e-30)
        print(f"  {name}: max|saved - recomputed| / max|recomputed| = {e:.2e}", flush=True)
        assert e <= 1e-2, name
