"""GPU parity of gated slot attention (two passes on the GPU) against the fp64 oracle, which
evaluates the slot memories directly, token by token."""
import numpy as np
import pytest

import workloads as W
from oracle import gsa_recurrent_bwd, gsa_recurrent_fwd
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


def check_gsa(gla, w, x, units=None, with_state=True, with_dstate=True, act="softmax", backward=True,
              saved=False):
    """saved: run gsa_fwd_save and gsa_bwd_saved instead of gsa_fwd and gsa_bwd."""
    dt = w.dtype
    args = [dev(x[n], dt) for n in ("q", "k", "v", "g")]
    hk0 = dev(x["hk0"]) if with_state else None
    hv0 = dev(x["hv0"]) if with_state else None
    if saved:
        o, hkt, hvt, sv = gla.gsa_fwd_save(*args, C=w.C, hk0=hk0, hv0=hv0, act=act)
    else:
        o, hkt, hvt = gla.gsa_fwd(*args, C=w.C, hk0=hk0, hv0=hv0, act=act)
    sel = (slice(None), slice(None)) if units is None else units
    s0 = (lambda a: None if (a is None or not with_state) else a[sel])
    ro, rhk, rhv = gsa_recurrent_fwd(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], s0(x["hk0"]), s0(x["hv0"]),
                                     act=act)
    print(f"[{w.name}] B={w.B} H={w.H} L={x['q'].shape[2]} Dk={w.Dk} Dv={w.Dv} m={w.m} C={w.C} {dt} "
          f"h0={with_state} dht={with_dstate} act={act} saved={saved}", flush=True)
    assert_close("o", host(o)[sel], ro, dt)
    assert_close("hkt", host(hkt)[sel], rhk, dt)
    assert_close("hvt", host(hvt)[sel], rhv, dt)
    if not backward:
        return
    kw = dict(C=w.C, hk0=hk0, hv0=hv0, dhkt=dev(x["dhkt"]) if with_dstate else None,
              dhvt=dev(x["dhvt"]) if with_dstate else None, want_dh0=True, act=act)
    if saved:
        dq, dk, dv, dg, dhk0, dhv0 = gla.gsa_bwd_saved(*args, dev(x["do"], dt), sv, **kw)
    else:
        dq, dk, dv, dg, dhk0, dhv0 = gla.gsa_bwd(*args, dev(x["do"], dt), **kw)
    rb = gsa_recurrent_bwd(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], x["do"][sel], s0(x["hk0"]),
                           s0(x["hv0"]), x["dhkt"][sel] if with_dstate else None,
                           x["dhvt"][sel] if with_dstate else None, act=act)
    assert_close("dq", host(dq)[sel], rb["dq"], dt)
    assert_close("dk", host(dk)[sel], rb["dk"], dt)
    assert_close("dv", host(dv)[sel], rb["dv"], dt)
    assert_close("dg", host(dg)[sel], rb["dg"], dt)
    assert_close("dhk0", host(dhk0)[sel], rb["dhk0"], dt)
    assert_close("dhv0", host(dhv0)[sel], rb["dhv0"], dt)


SHAPES = [
    # (B, H, L, Dk, Dv, m, C, dtype, h0, dht)
    (1, 2, 150, 64, 64, 32, 64, "bf16", True, True),
    (2, 1, 77, 32, 48, 16, 16, "bf16", True, True),
    (1, 2, 130, 128, 128, 64, 32, "bf16", False, False),
    (1, 1, 200, 96, 160, 48, 64, "bf16", True, True),
    (1, 2, 1, 64, 64, 64, 64, "bf16", True, True),
    (1, 2, 64, 128, 128, 64, 64, "bf16", True, False),
    (1, 1, 90, 256, 64, 32, 32, "bf16", True, True),
    (2, 1, 70, 32, 32, 32, 16, "f32", True, True),
    (1, 2, 100, 64, 96, 64, 32, "f32", True, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(gla, shape):
    B, H, L, Dk, Dv, m, C, dt, h0, dht = shape
    w = W.GsaWorkload("sweep", B, H, L, Dk, Dv, m, C, dt, 300 + L + m, h0=True)
    check_gsa(gla, w, W.gsa_inputs(w), with_state=h0, with_dstate=dht)


WIDE_SHAPES = [
    # (B, H, L, Dk, Dv, m, C, dtype, h0, dht): more than 64 slots
    (1, 2, 150, 64, 64, 128, 32, "bf16", True, True),
    (2, 1, 77, 32, 48, 96, 16, "bf16", True, True),
    (1, 1, 130, 128, 128, 80, 32, "bf16", False, True),
    (1, 2, 200, 64, 96, 112, 32, "bf16", True, False),
]


@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_wide_slot_counts(gla, shape):
    """Slot counts up to 128 (the GSA summary's ablation doubles m from 64 to 128), forward and
    backward at the chunk sizes whose kernels hold them."""
    B, H, L, Dk, Dv, m, C, dt, h0, dht = shape
    w = W.GsaWorkload("wide", B, H, L, Dk, Dv, m, C, dt, 700 + L + m, h0=True)
    check_gsa(gla, w, W.gsa_inputs(w), with_state=h0, with_dstate=dht)


@pytest.mark.parametrize("shape", [
    # (B, H, L, Dk, Dv, m, C, dtype, h0, dht)
    (1, 2, 150, 64, 64, 128, 64, "bf16", True, True),   # backward at C = 32
    (1, 1, 90, 48, 64, 64, 64, "f32", True, True),      # fp32 backward at C = 32
    (1, 2, 150, 64, 64, 64, 128, "bf16", True, True),   # C = 128: forward and backward at 64
    (1, 2, 130, 64, 96, 128, 128, "bf16", False, True),  # C = 128 with 128 slots: 64, and 32 backward
], ids=lambda s: "x".join(map(str, s)))
def test_chunk_sizes_beyond_the_tiles(gla, shape):
    """A chunk size whose GSA tiles exceed a CU's LDS runs at the largest smaller one whose
    tiles fit (the result does not depend on the chunk size): forward and backward, through
    both entry-point pairs, match the oracle."""
    B, H, L, Dk, Dv, m, C, dt, h0, dht = shape
    w = W.GsaWorkload("tile-c", B, H, L, Dk, Dv, m, C, dt, 740 + L + m, h0=True)
    x = W.gsa_inputs(w)
    check_gsa(gla, w, x, with_state=h0, with_dstate=dht)
    check_gsa(gla, w, x, with_state=h0, with_dstate=dht, saved=True)


@pytest.mark.parametrize("shape", [(1, 2, 100, 64, 96, 128, 64, "f32"), (1, 2, 100, 64, 96, 128, 128, "f32")],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward_only_shapes(gla, shape):
    """fp32 with more than 64 slots: no chunk size holds the pass-1 backward's tiles.  The
    forward matches the oracle, and the backward and the saving forward are refused before
    anything runs."""
    import torch
    B, H, L, Dk, Dv, m, C, dt = shape
    w = W.GsaWorkload("fwd-only", B, H, L, Dk, Dv, m, C, dt, 720 + L + m, h0=True)
    x = W.gsa_inputs(w)
    check_gsa(gla, w, x, backward=False)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    assert gla.gsa_bwd_workspace_bytes(B, H, L, Dk, Dv, m, C, tdt) == 0
    assert gla.gsa_saved_bytes(B, H, L, Dk, Dv, m, C, tdt) == 0
    args = [dev(x[n], dt) for n in ("q", "k", "v", "g")]
    with pytest.raises(gla.GlaError):
        gla.gsa_bwd(*args, dev(x["do"], dt), C=C)


def test_full_size_m128_sampled(gla):
    """The GSA layer with 128 slots (B=8, H=4, L=2048, Dk=Dv=128, C=32) through the saved path,
    as the benchmark runs it, sampled units; and its forward at C = 64."""
    w = W.WORKLOADS["gsa_340m_m128"]
    x = W.gsa_inputs(w)
    units = (np.array([1, 6])[:, None], np.array([2])[None, :])
    check_gsa(gla, w, x, units=units, with_state=False, with_dstate=False, saved=True)
    w64 = W.GsaWorkload("gsa_340m_m128_c64", 8, 4, 2048, 128, 128, 128, 64, "bf16", 1007)
    check_gsa(gla, w64, x, units=(np.array([3])[:, None], np.array([0, 3])[None, :]), with_state=False,
              backward=False)


@pytest.mark.parametrize("gval", [-3.0, -30.0])
def test_extreme_gates(gla, gval):
    """Strong forgetting on every other slot (normal gates on the rest): every chunk fails the
    span check and takes the exact intra-chunk path, while the slots still differ."""
    w = W.GsaWorkload("gates", 1, 2, 150, 64, 64, 32, 64, "bf16", 31, h0=True)
    x = W.gsa_inputs(w)
    x["g"][..., ::2] = gval
    check_gsa(gla, w, x)


def test_identical_slots_degenerate(gla):
    """The same gate g = -30 on every slot makes all slots identical: z is uniform, the
    softmax gradient vanishes, and dq, dk, dg are analytically ~1e-13 of the gradient scale.
    Check the outputs that stay O(1) to the bound and the vanishing ones against the scale."""
    w = W.GsaWorkload("degenerate", 1, 2, 150, 64, 64, 32, 64, "bf16", 35, h0=True)
    x = W.gsa_inputs(w)
    x["g"] = np.full_like(x["g"], -30.0)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "g")]
    hk0, hv0 = dev(x["hk0"]), dev(x["hv0"])
    o, hkt, hvt = gla.gsa_fwd(*args, C=64, hk0=hk0, hv0=hv0)
    dq, dk, dv, dg, _, dhv0 = gla.gsa_bwd(*args, dev(x["do"], "bf16"), C=64, hk0=hk0, hv0=hv0,
                                          dhkt=dev(x["dhkt"]), dhvt=dev(x["dhvt"]), want_dh0=True)
    ro, rhk, rhv = gsa_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["hk0"], x["hv0"])
    rb = gsa_recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["do"], x["hk0"], x["hv0"], x["dhkt"], x["dhvt"])
    assert_close("o", host(o), ro, "bf16")
    assert_close("hvt", host(hvt), rhv, "bf16")
    assert_close("dv", host(dv), rb["dv"], "bf16")
    assert_close("dhv0", host(dhv0), rb["dhv0"], "bf16")
    scale = np.max(np.abs(rb["dv"]))
    for name, t in (("dq", dq), ("dk", dk), ("dg", dg)):
        e = np.max(np.abs(host(t) - rb[name])) / scale
        print(f"  {name}: max|d| / max|dv_ref| = {e:.3e}", flush=True)
        assert e <= 1e-2, name


def test_open_gates_zero_state_gives_zero(gla):
    """g = 0 means w = 0: with zero initial memories nothing is ever written, so o = 0."""
    import torch
    w = W.GsaWorkload("open", 1, 2, 100, 64, 64, 32, 64, "bf16", 32)
    x = W.gsa_inputs(w, with_grad=False)
    o, hkt, hvt = gla.gsa_fwd(dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"),
                              dev(np.zeros_like(x["g"]), "bf16"), C=64)
    torch.cuda.synchronize()
    assert float(o.abs().max()) == 0.0 and float(hkt.abs().max()) == 0.0 and float(hvt.abs().max()) == 0.0


def test_mixed_chunks(gla):
    w = W.GsaWorkload("mixed", 1, 2, 256, 64, 64, 64, 64, "bf16", 33, h0=True)
    x = W.gsa_inputs(w)
    x["g"][:, :, 64:128] = -2.0
    x["g"][:, 1, 200:210, :5] = -40.0
    check_gsa(gla, w, x)


def test_full_size_config_sampled(gla):
    """The GSA workload (B=8, H=4, L=2048, Dk=Dv=128, m=64, C=64), sampled units."""
    w = W.WORKLOADS["gsa_340m"]
    x = W.gsa_inputs(w)
    units = (np.array([0, 5])[:, None], np.array([1, 3])[None, :])
    check_gsa(gla, w, x, units=units, with_state=False, with_dstate=False)


def test_full_size_config_sampled_saved_path(gla):
    """The GSA workload through gsa_fwd_save / gsa_bwd_saved, as the benchmark runs it."""
    w = W.WORKLOADS["gsa_340m"]
    x = W.gsa_inputs(w)
    units = (np.array([2, 7])[:, None], np.array([0, 2])[None, :])
    check_gsa(gla, w, x, units=units, with_state=False, with_dstate=False, saved=True)


@pytest.mark.parametrize("act", ["softmax", "swish", "relu2"])
def test_saved_path_matches_recomputing_backward(gla, act):
    """gsa_fwd_save and gsa_bwd_saved give gsa_fwd's outputs and gsa_bwd's gradients bit for
    bit: what the saved backward reads is what the recomputing one rebuilds with the same
    kernels from the same inputs."""
    import torch
    w = W.GsaWorkload("gsa-saved", 2, 2, 257, 64, 96, 48, 64, "bf16", 431, h0=True)
    x = W.gsa_inputs(w)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "g")]
    st = dict(C=64, hk0=dev(x["hk0"]), hv0=dev(x["hv0"]), act=act)
    o, hkt, hvt, saved = gla.gsa_fwd_save(*args, **st)
    ref = gla.gsa_fwd(*args, **st)
    do, dhkt, dhvt = dev(x["do"], "bf16"), dev(x["dhkt"]), dev(x["dhvt"])
    a = gla.gsa_bwd_saved(*args, do, saved, dhkt=dhkt, dhvt=dhvt, want_dh0=True, **st)
    b = gla.gsa_bwd(*args, do, dhkt=dhkt, dhvt=dhvt, want_dh0=True, **st)
    torch.cuda.synchronize()
    for name, s_, t in zip(("o", "hkt", "hvt"), (o, hkt, hvt), ref):
        assert torch.equal(s_, t), name
    for name, s_, t in zip(("dq", "dk", "dv", "dg", "dhk0", "dhv0"), a, b):
        assert torch.equal(s_, t), name


def test_deterministic(gla):
    import torch
    w = W.GsaWorkload("det", 2, 2, 300, 64, 64, 64, 64, "bf16", 34)
    x = W.gsa_inputs(w)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "g", "do")]
    a = gla.gsa_bwd(*args, C=64)
    b = gla.gsa_bwd(*args, C=64)
    fa = gla.gsa_fwd(*args[:4], C=64)
    fb = gla.gsa_fwd(*args[:4], C=64)
    torch.cuda.synchronize()
    assert all(torch.equal(s, t) for s, t in zip(a[:4], b[:4]))
    assert all(torch.equal(s, t) for s, t in zip(fa, fb))


# ---------------------------------------------------------------- read-outs other than softmax
def slot_scores(q, k, g, hk0):
    """z_t[s] = <Kmem_t[s], q_t> with the slot keys written token by token (test-side helper,
    used only to check that every score is well away from ReLU's kink)."""
    B, H, L, Dk = q.shape
    m = g.shape[-1]
    K = np.zeros((B, H, Dk, m)) if hk0 is None else hk0.astype(np.float64).copy()
    z = np.empty((B, H, L, m))
    for t in range(L):
        a = np.exp(g[:, :, t].astype(np.float64))
        K = K * a[:, :, None, :] + k[:, :, t, :, None] * (1.0 - a)[:, :, None, :]
        z[:, :, t] = np.einsum("bhi,bhis->bhs", q[:, :, t], K)
    return z


READ_OUT_SHAPES = [
    # (B, H, L, Dk, Dv, m, C, dtype)
    (1, 2, 150, 64, 64, 32, 64, "bf16"),
    (2, 1, 77, 32, 48, 16, 16, "bf16"),
    (1, 1, 130, 128, 128, 64, 32, "bf16"),
    (1, 2, 100, 64, 96, 64, 32, "f32"),
]


@pytest.mark.parametrize("act", ["swish", "relu2", "none"])
@pytest.mark.parametrize("shape", READ_OUT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_read_outs(gla, shape, act):
    """Swish, ReLU^2 and no read-out, forward and backward (their derivatives are continuous)."""
    B, H, L, Dk, Dv, m, C, dt = shape
    w = W.GsaWorkload("read-out", B, H, L, Dk, Dv, m, C, dt, 500 + L + m, h0=True)
    check_gsa(gla, w, W.gsa_inputs(w), act=act)


@pytest.mark.parametrize("shape", READ_OUT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_relu_forward(gla, shape):
    """ReLU read-out, forward on the general inputs (the output is continuous in z)."""
    B, H, L, Dk, Dv, m, C, dt = shape
    w = W.GsaWorkload("relu", B, H, L, Dk, Dv, m, C, dt, 520 + L + m, h0=True)
    check_gsa(gla, w, W.gsa_inputs(w), act="relu", backward=False)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_relu_backward_clear_margin(gla, dt):
    """ReLU's derivative jumps at z = 0, and the two sides compute z in different precision, so
    the backward is compared where every score is decided: initial slot keys carry a strong
    signed component along key channel 0 that q_t reads with weight 1, gates are close to 0
    (the keys persist) and every |z| is asserted to stay above 0.5, far beyond either side's
    rounding of z."""
    w = W.GsaWorkload("relu-margin", 1, 2, 150, 64, 64, 32, 64, dt, 541, h0=True)
    x = W.gsa_inputs(w)
    rng = np.random.default_rng(542)
    sign = np.where(rng.random(w.m) < 0.5, -1.0, 1.0).astype(np.float32)
    x["hk0"][:, :, 0, :] = 3.0 * sign
    x["q"][:, :, :, 0] = 1.0
    x["g"] = (x["g"] / 400.0).astype(np.float32)
    if dt == "bf16":
        x["g"] = W.round_bf16(x["g"])
    z = slot_scores(x["q"], x["k"], x["g"], x["hk0"])
    print(f"  min |z| = {np.min(np.abs(z)):.3f}", flush=True)
    assert np.min(np.abs(z)) > 0.5
    check_gsa(gla, w, x, act="relu")
