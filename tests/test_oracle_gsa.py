"""Pins of the fp64 GSA oracle (CPU only).

The GSA oracle runs the slot memories directly.  These tests tie it to (a) the two-pass form
the GSA summaries describe (GLA into m slots, softmax over slots, GLA readout), built here from
the separately pinned GLA oracle, (b) closed forms for one slot and for frozen memories,
(c) central finite differences, and (d) the chain rule taken through the two GLA passes.
"""
import numpy as np
import pytest

from oracle import (GSA_ACTS, gla_recurrent_bwd, gla_recurrent_fwd, gsa_decode_step, gsa_recurrent_bwd,
                    gsa_recurrent_fwd)


def rand_gsa(seed, B=1, H=2, L=19, Dk=4, Dv=3, m=5, h0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, Dk))
    k = rng.standard_normal((B, H, L, Dk))
    v = rng.standard_normal((B, H, L, Dv))
    g = -np.log1p(np.exp(-rng.standard_normal((B, H, L, m)) * 2.0))
    hk0 = rng.standard_normal((B, H, Dk, m)) if h0 else None
    hv0 = rng.standard_normal((B, H, m, Dv)) if h0 else None
    return q, k, v, g, hk0, hv0


def softmax(z):
    z = z - z.max(-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(-1, keepdims=True)


# Read-outs between the passes and their derivatives, written here from their textbook
# definitions (independently of the oracle's own).
def read_out(z, act):
    return {"softmax": lambda: softmax(z),
            "swish": lambda: z / (1.0 + np.exp(-z)),
            "relu": lambda: np.where(z > 0, z, 0.0),
            "relu2": lambda: np.where(z > 0, z * z, 0.0),
            "none": lambda: z}[act]()


def read_out_bwd(z, p, dp, act):
    if act == "softmax":
        return p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    sig = 1.0 / (1.0 + np.exp(-z))
    d = {"swish": sig + z * sig * (1.0 - sig), "relu": np.where(z > 0, 1.0, 0.0),
         "relu2": np.where(z > 0, 2.0 * z, 0.0), "none": np.ones_like(z)}[act]
    return d * dp


def two_pass_forward(q, k, v, g, hk0, hv0, act="softmax"):
    """Pass 1 per slot s is a GLA with scalar gate g[..., s] on every key channel, keys k and a
    single value column w[..., s]; its output is z[..., s].  Pass 2 is a GLA with queries p,
    keys w, values v and the slot gates."""
    B, H, L, Dk = q.shape
    m = g.shape[-1]
    w = -np.expm1(g)
    z = np.empty((B, H, L, m))
    hkt = np.empty((B, H, Dk, m))
    for s in range(m):
        gs = np.repeat(g[..., s:s + 1], Dk, axis=-1)
        h0s = None if hk0 is None else hk0[..., :, s:s + 1]
        zs, hs = gla_recurrent_fwd(q, k, w[..., s:s + 1], gs, h0s)
        z[..., s] = zs[..., 0]
        hkt[..., :, s] = hs[..., 0]
    p = read_out(z, act)
    o, hvt = gla_recurrent_fwd(p, w, v, g, hv0)
    return o, hkt, hvt, z, p, w


@pytest.mark.parametrize("act", GSA_ACTS)
@pytest.mark.parametrize("h0", [False, True])
def test_two_pass_equals_slot_memory(h0, act):
    """P12: the two-pass GLA form reproduces the direct slot-memory recurrence, for every
    read-out between the passes."""
    q, k, v, g, hk0, hv0 = rand_gsa(1, h0=h0)
    o, hkt, hvt = gsa_recurrent_fwd(q, k, v, g, hk0, hv0, act=act)
    o2, hkt2, hvt2, *_ = two_pass_forward(q, k, v, g, hk0, hv0, act)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hkt, hkt2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hvt, hvt2, rtol=1e-12, atol=1e-12)


def test_single_slot_is_moving_average():
    """P13: with m = 1 the softmax is 1, so o_t = alpha_t o_{t-1} + (1 - alpha_t) v_t, an
    exponential moving average of v that ignores q and k."""
    q, k, v, g, hk0, hv0 = rand_gsa(2, m=1)
    o, _, hvt = gsa_recurrent_fwd(q, k, v, g, hk0, hv0)
    prev = hv0[:, :, 0, :]
    for t in range(q.shape[2]):
        a = np.exp(g[:, :, t, 0])[..., None]
        prev = a * prev + (1 - a) * v[:, :, t]
        np.testing.assert_allclose(o[:, :, t], prev, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hvt[:, :, 0], prev, rtol=1e-12, atol=1e-12)


def test_open_gates_freeze_memory():
    """P14: g = 0 means alpha = 1, w = 0: memories never change, so o_t is softmax attention
    of q_t over the m fixed initial slots, and zero memories give o = 0."""
    q, k, v, g, hk0, hv0 = rand_gsa(3)
    g = np.zeros_like(g)
    o, hkt, hvt = gsa_recurrent_fwd(q, k, v, g, hk0, hv0)
    z = q @ hk0                                   # [B,H,L,m]
    np.testing.assert_allclose(o, softmax(z) @ hv0, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(hkt, hk0)
    np.testing.assert_array_equal(hvt, hv0)
    o0, _, _ = gsa_recurrent_fwd(q, k, v, g)
    np.testing.assert_array_equal(o0, np.zeros_like(o0))


def _loss(a, do, dhkt, dhvt, act="softmax"):
    o, hkt, hvt = gsa_recurrent_fwd(a["q"], a["k"], a["v"], a["g"], a["hk0"], a["hv0"], act=act)
    return float(np.sum(o * do) + np.sum(hkt * dhkt) + np.sum(hvt * dhvt))


@pytest.mark.parametrize("act", GSA_ACTS)
def test_backward_finite_differences(act):
    """P15: every GSA gradient matches central differences (final-state gradients non-zero),
    for every read-out.  ReLU's derivative jumps at z = 0, so the inputs keep every slot score
    well away from 0 (asserted), where central differences are exact to rounding."""
    q, k, v, g, hk0, hv0 = rand_gsa(4, B=1, H=1, L=7, Dk=3, Dv=2, m=3)
    z = two_pass_forward(q, k, v, g, hk0, hv0)[3]
    assert np.min(np.abs(z)) > 1e-3
    rng = np.random.default_rng(5)
    do = rng.standard_normal(v.shape)
    dhkt = rng.standard_normal(hk0.shape)
    dhvt = rng.standard_normal(hv0.shape)
    grads = gsa_recurrent_bwd(q, k, v, g, do, hk0, hv0, dhkt, dhvt, checkpoint=3, act=act)
    args = dict(q=q, k=k, v=v, g=g, hk0=hk0, hv0=hv0)
    eps = 1e-6
    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd[idx] = (_loss(dict(args, **{name: xp}), do, dhkt, dhvt, act)
                       - _loss(dict(args, **{name: xm}), do, dhkt, dhvt, act)) / (2 * eps)
        np.testing.assert_allclose(grads["d" + name], fd, rtol=1e-6, atol=1e-7,
                                   err_msg="d" + name)


@pytest.mark.parametrize("act", GSA_ACTS)
def test_backward_chain_rule_through_gla_passes(act):
    """P16: chaining the (separately pinned) GLA oracle's backward through pass 2, the read-out
    and pass 1 gives the GSA gradients; the gate gradient is
    dg = (gate-gradient of pass 1) + (gate-gradient of pass 2) - alpha * (dw1 + dw2)."""
    q, k, v, g, hk0, hv0 = rand_gsa(6, L=23)
    rng = np.random.default_rng(7)
    do = rng.standard_normal(v.shape)
    dhkt = rng.standard_normal(hk0.shape)
    dhvt = rng.standard_normal(hv0.shape)
    ref = gsa_recurrent_bwd(q, k, v, g, do, hk0, hv0, dhkt, dhvt, checkpoint=6, act=act)
    _, _, _, z, p, w = two_pass_forward(q, k, v, g, hk0, hv0, act)
    g2 = gla_recurrent_bwd(p, w, v, g, do, hv0, dhvt)
    dp, dw2 = g2["dq"], g2["dk"]
    dz = read_out_bwd(z, p, dp, act)
    Dk, m = q.shape[-1], g.shape[-1]
    dq = np.zeros_like(q); dk = np.zeros_like(k)
    dw1 = np.zeros_like(g); dg1 = np.zeros_like(g); dhk0 = np.zeros_like(hk0)
    for s in range(m):
        gs = np.repeat(g[..., s:s + 1], Dk, axis=-1)
        r = gla_recurrent_bwd(q, k, w[..., s:s + 1], gs, dz[..., s:s + 1],
                              hk0[..., :, s:s + 1], dhkt[..., :, s:s + 1])
        dq += r["dq"]; dk += r["dk"]
        dw1[..., s] = r["dv"][..., 0]
        dg1[..., s] = r["dg"].sum(-1)
        dhk0[..., :, s] = r["dh0"][..., 0]
    dg = dg1 + g2["dg"] - np.exp(g) * (dw1 + dw2)
    for name, val in [("dq", dq), ("dk", dk), ("dv", g2["dv"]), ("dg", dg),
                      ("dhk0", dhk0), ("dhv0", g2["dh0"])]:
        np.testing.assert_allclose(ref[name], val, rtol=1e-10, atol=1e-10, err_msg=name)


@pytest.mark.parametrize("act", GSA_ACTS)
def test_gate_gradient_identity(act):
    """dg = revcumsum(dB1 + dB2) - alpha*(dw1 + dw2) + final-state terms, where
    dB1 = z*dz - w*dw1 and dB2 = p*dp - w*dw2: the reverse-prefix-sum form of the gate
    gradient (decay factors enter only through exp of prefix sums of g)."""
    q, k, v, g, hk0, hv0 = rand_gsa(8, L=21)
    rng = np.random.default_rng(9)
    do = rng.standard_normal(v.shape)
    dhkt = rng.standard_normal(hk0.shape)
    dhvt = rng.standard_normal(hv0.shape)
    ref = gsa_recurrent_bwd(q, k, v, g, do, hk0, hv0, dhkt, dhvt, act=act)
    o, hkt, hvt, z, p, w = two_pass_forward(q, k, v, g, hk0, hv0, act)
    g2 = gla_recurrent_bwd(p, w, v, g, do, hv0, dhvt)
    dp, dw2 = g2["dq"], g2["dk"]
    dz = read_out_bwd(z, p, dp, act)
    dw1 = np.zeros_like(g)
    Dk, m = q.shape[-1], g.shape[-1]
    for s in range(m):
        gs = np.repeat(g[..., s:s + 1], Dk, axis=-1)
        r = gla_recurrent_bwd(q, k, w[..., s:s + 1], gs, dz[..., s:s + 1],
                              hk0[..., :, s:s + 1], dhkt[..., :, s:s + 1])
        dw1[..., s] = r["dv"][..., 0]
    dB = z * dz - w * dw1 + p * dp - w * dw2
    rc = np.flip(np.cumsum(np.flip(dB, axis=2), axis=2), axis=2)
    final = np.sum(dhkt * hkt, axis=-2) + np.sum(dhvt * hvt, axis=-1)      # [B,H,m]
    dg = rc + final[:, :, None, :] - np.exp(g) * (dw1 + dw2)
    np.testing.assert_allclose(ref["dg"], dg, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("act", GSA_ACTS)
@pytest.mark.parametrize("h0", [False, True])
def test_decode_steps_equal_two_pass_forward(h0, act):
    """P17: T single-token GSA decode steps reproduce the two-pass form (built from the
    separately pinned GLA oracle): every output and both final memories, for every read-out."""
    q, k, v, g, hk0, hv0 = rand_gsa(11, B=2, H=2, L=9, Dk=5, Dv=4, m=3, h0=h0)
    o2, hkt2, hvt2, *_ = two_pass_forward(q, k, v, g, hk0, hv0, act)
    B, H, L, Dk = q.shape
    hk = np.zeros((B, H, Dk, 3)) if hk0 is None else hk0
    hv = np.zeros((B, H, 3, 4)) if hv0 is None else hv0
    for t in range(L):
        ot, hk, hv = gsa_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], hk, hv, act=act)
        np.testing.assert_allclose(ot, o2[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hk, hkt2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hv, hvt2, rtol=1e-12, atol=1e-12)


def test_decode_step_closed_forms():
    """P18: closed forms of one decode step.
    (a) g = 0: alpha = 1, w = 0, the memories are unchanged and o = softmax(q hk) hv;
    (b) g -> -inf: alpha = 0, w = 1, every slot is overwritten with the token, the slots are
        equal, the softmax is uniform and o = v;
    (c) m = 1: o = alpha hv + (1 - alpha) v whatever q and k are."""
    q, k, v, g, hk0, hv0 = rand_gsa(12, L=1, Dk=6, Dv=5, m=4)
    q, k, v, g = q[:, :, 0], k[:, :, 0], v[:, :, 0], g[:, :, 0]
    o, hk, hv = gsa_decode_step(q, k, v, np.zeros_like(g), hk0, hv0)
    np.testing.assert_array_equal(hk, hk0)
    np.testing.assert_array_equal(hv, hv0)
    z = (q[..., None, :] @ hk0)[..., 0, :]
    np.testing.assert_allclose(o, (softmax(z)[..., None, :] @ hv0)[..., 0, :], rtol=1e-12, atol=1e-12)
    o, hk, hv = gsa_decode_step(q, k, v, np.full_like(g, -800.0), hk0, hv0)
    np.testing.assert_array_equal(hk, np.repeat(k[..., :, None], 4, axis=-1))
    np.testing.assert_array_equal(hv, np.repeat(v[..., None, :], 4, axis=-2))
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)
    q1, k1, v1, g1, hk1, hv1 = rand_gsa(13, L=1, Dk=6, Dv=5, m=1)
    o, _, hv = gsa_decode_step(q1[:, :, 0], k1[:, :, 0], v1[:, :, 0], g1[:, :, 0], hk1, hv1)
    a = np.exp(g1[:, :, 0])
    np.testing.assert_allclose(o, a * hv1[:, :, 0] + (1 - a) * v1[:, :, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hv[:, :, 0], o, rtol=1e-12, atol=1e-12)


def test_plain_read_out_with_frozen_memory_is_bilinear():
    """P19: with no read-out nonlinearity and open gates (g = 0), the memories never change and
    o_t = (q_t hk0) hv0, a bilinear function of q_t; ReLU keeps only the positive scores."""
    q, k, v, g, hk0, hv0 = rand_gsa(14)
    g = np.zeros_like(g)
    o, _, _ = gsa_recurrent_fwd(q, k, v, g, hk0, hv0, act="none")
    np.testing.assert_allclose(o, (q @ hk0) @ hv0, rtol=1e-12, atol=1e-12)
    o, _, _ = gsa_recurrent_fwd(q, k, v, g, hk0, hv0, act="relu")
    np.testing.assert_allclose(o, np.clip(q @ hk0, 0, None) @ hv0, rtol=1e-12, atol=1e-12)
