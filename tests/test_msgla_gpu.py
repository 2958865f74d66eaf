"""GPU parity of the MS-GLA front end (msgla_fwd, through the C ABI) against the fp64 oracle:
pooling per head group, GLA on the pooled sequences, causal hold and fusion weights."""
import numpy as np
import pytest

import workloads as W
from oracle import msgla_fwd as ref_msgla
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


def fusion_weights(seed, B, L, n):
    """Per-token weights over the groups, positive and summing to 1 (as a softmax router's)."""
    x = np.random.default_rng(seed).standard_normal((B, L, n)).astype(np.float32)
    e = np.exp(x - x.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def check(gla, w, x, scales, heads, wts, units=None):
    dt = w.dtype
    q, k, v, g = (dev(x[n], dt) for n in ("q", "k", "v", "g"))
    h0 = dev(x["h0"]) if x["h0"] is not None else None
    o, ht = gla.msgla_fwd(q, k, v, g, scales, heads, None if wts is None else dev(wts), C=w.C, h0=h0)
    bsel = slice(None) if units is None else units
    wref = np.ones((x["q"].shape[0], x["q"].shape[2], len(scales))) if wts is None else wts
    ro, rht = ref_msgla(x["q"][bsel], x["k"][bsel], x["v"][bsel], x["g"][bsel], scales, heads, wref[bsel],
                        None if x["h0"] is None else x["h0"][bsel])
    print(f"[msgla] B={w.B} H={w.H} L={x['q'].shape[2]} Dk={w.Dk} Dv={w.Dv} C={w.C} {dt} scales={scales} "
          f"heads={heads} h0={x['h0'] is not None} w={'given' if wts is not None else 'none'}", flush=True)
    assert_close("o", host(o)[bsel], ro, dt)
    assert_close("ht", host(ht)[bsel], rht, dt)


SHAPES = [
    # (B, H, L, Dk, Dv, C, dtype, scales, heads, h0, weights)
    (2, 4, 300, 64, 64, 64, "bf16", (1, 2, 4), (2, 1, 1), True, True),
    (1, 3, 77, 32, 48, 16, "bf16", (1, 3, 5), (1, 1, 1), False, True),
    (1, 2, 130, 128, 256, 64, "bf16", (2,), (2,), True, False),
    (1, 4, 200, 64, 64, 32, "f32", (1, 2, 4, 8), (1, 1, 1, 1), True, True),
    (1, 2, 10, 64, 64, 16, "bf16", (1, 16), (1, 1), True, True),        # a scale longer than L
    (2, 5, 257, 128, 128, 64, "bf16", (4, 1), (3, 2), False, True),      # coarse group first
    (2, 5, 190, 64, 128, 64, "bf16", (2, 1, 4), (1, 3, 1), True, True),  # in-place group in the middle
    (1, 2, 1100, 64, 64, 64, "bf16", (1, 8), (1, 1), True, True),        # 512 held tokens per chunk
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:7])) + "-" + "_".join(map(str, s[7])))
def test_small_shapes(gla, shape):
    B, H, L, Dk, Dv, C, dt, scales, heads, h0, wts = shape
    w = W.GlaWorkload("msgla", B, H, L, Dk, Dv, C, dt, 700 + L + H, h0=h0, gate_law="iid")
    x = W.gla_inputs(w, with_grad=False)
    check(gla, w, x, list(scales), list(heads), fusion_weights(701 + L, B, L, len(scales)) if wts else None)


def test_single_group_at_scale_one_is_gla_fwd(gla):
    """One group at scale 1 with no weights is gla_fwd itself, bit for bit: the group reads the
    inputs in place and the hold multiplies by 1."""
    import torch
    w = W.GlaWorkload("msgla-id", 2, 3, 200, 64, 128, 64, "bf16", 711, h0=True, gate_law="iid")
    x = W.gla_inputs(w, with_grad=False)
    q, k, v, g = (dev(x[n], "bf16") for n in ("q", "k", "v", "g"))
    h0 = dev(x["h0"])
    o, ht = gla.msgla_fwd(q, k, v, g, [1], [3], None, C=64, h0=h0)
    ro, rht = gla.gla_fwd(q, k, v, g, C=64, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(o, ro) and torch.equal(ht, rht)


def test_full_size_340m_three_scales_sampled(gla):
    """MS-GLA {1, 2, 4} on the 340M-layer shape (B=8, H=4, L=2048, Dk=128, Dv=256, C=64) with the
    head budget split 2/1/1, in the launch configuration the benchmark times; two batch rows
    against the oracle."""
    w = W.WORKLOADS["gla_340m"]
    x = W.gla_inputs(w, with_grad=False)
    check(gla, w, x, [1, 2, 4], [2, 1, 1], fusion_weights(712, w.B, w.L, 3), units=np.array([0, 5]))


def test_deterministic(gla):
    import torch
    w = W.GlaWorkload("msgla-det", 2, 4, 300, 64, 64, 64, "bf16", 713, gate_law="iid")
    x = W.gla_inputs(w, with_grad=False)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "g")]
    wt = dev(fusion_weights(714, 2, 300, 3))
    a = gla.msgla_fwd(*args, [1, 2, 4], [2, 1, 1], wt)
    b = gla.msgla_fwd(*args, [1, 2, 4], [2, 1, 1], wt)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
