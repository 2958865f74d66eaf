"""Pins of the fp64 GLA oracle against things other than itself (CPU only).

Each test ties the oracle to a closed form, a textbook special case, an invariant of the
method, brute force on tiny inputs, finite differences or an independent autograd engine, so
that a dropped term, a wrong sign or index, or a transposed operand in the oracle fails one
of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import gla_chunkwise_fwd, gla_decode_step, gla_recurrent_bwd, gla_recurrent_fwd

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(seed, B=2, H=2, L=23, Dk=5, Dv=4, h0=True, gate_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, Dk))
    k = rng.standard_normal((B, H, L, Dk))
    v = rng.standard_normal((B, H, L, Dv))
    # log-sigmoid gates, some channels near alpha = 1, some strongly forgetting
    g = -np.log1p(np.exp(-rng.standard_normal((B, H, L, Dk)) * 2.0)) * gate_scale
    S0 = rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, S0


def test_hand_worked_example():
    """Exact rational example worked by hand from the recurrence (tests/golden)."""
    with open(os.path.join(HERE, "golden", "gla_hand_worked.json")) as f:
        fx = json.load(f)
    q = np.array(fx["q"], float)[None, None]
    k = np.array(fx["k"], float)[None, None]
    v = np.array(fx["v"], float)[None, None]
    g = np.log(np.array(fx["alpha"], float))[None, None]
    for case in fx["cases"]:
        h0 = None if case["h0"] is None else np.array(case["h0"], float)[None, None]
        o, ht = gla_recurrent_fwd(q, k, v, g, h0)
        np.testing.assert_allclose(o[0, 0], np.array(case["o"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(ht[0, 0], np.array(case["ht"]), rtol=0, atol=1e-13)


def _brute_force_exact(q, k, v, alpha, h0):
    """O(L^2) closed form in exact rationals: o_t = sum_{j<=t} sum_i q_t[i] k_j[i]
    (prod_{j<s<=t} alpha_s[i]) v_j + sum_i q_t[i] (prod_{s<=t} alpha_s[i]) h0[i, :]."""
    L, Dk = len(q), len(q[0])
    Dv = len(v[0])
    o = []
    for t in range(L):
        row = [Fraction(0)] * Dv
        for i in range(Dk):
            for j in range(t + 1):
                decay = Fraction(1)
                for s in range(j + 1, t + 1):
                    decay *= alpha[s][i]
                for c in range(Dv):
                    row[c] += q[t][i] * k[j][i] * decay * v[j][c]
            decay0 = Fraction(1)
            for s in range(0, t + 1):
                decay0 *= alpha[s][i]
            for c in range(Dv):
                row[c] += q[t][i] * decay0 * h0[i][c]
        o.append(row)
    return o


def test_brute_force_rational():
    """P1: the oracle equals the gated O(L^2) double sum evaluated in exact rationals."""
    rng = np.random.default_rng(7)
    L, Dk, Dv = 9, 3, 2
    ints = lambda *s: rng.integers(-4, 5, size=s)
    q, k, v, h0 = ints(L, Dk), ints(L, Dk), ints(L, Dv), ints(Dk, Dv)
    expo = rng.integers(0, 4, size=(L, Dk))              # alpha = 2^-e, e in {0..3}
    alpha = [[Fraction(1, 2 ** int(e)) for e in row] for row in expo]
    ref = _brute_force_exact(q.tolist(), k.tolist(), v.tolist(), alpha, h0.tolist())
    g = -expo * np.log(2.0)
    o, _ = gla_recurrent_fwd(q[None, None], k[None, None], v[None, None], g[None, None],
                             h0[None, None].astype(float))
    np.testing.assert_allclose(o[0, 0], np.array(ref, dtype=float), rtol=1e-13, atol=1e-12)


def test_ungated_is_causal_linear_attention():
    """P2: g = 0 gives causal linear attention o = tril(Q K^T) V + Q h0 (Katharopoulos et al.,
    listed by the GLA visual companion as the ungated ancestor)."""
    q, k, v, _, S0 = rand_inputs(1)
    g = np.zeros_like(q)
    o, ht = gla_recurrent_fwd(q, k, v, g, S0)
    L = q.shape[2]
    mask = np.tril(np.ones((L, L)))
    ref = (q @ np.swapaxes(k, -1, -2) * mask) @ v + q @ S0
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht, np.swapaxes(k, -1, -2) @ v + S0, rtol=1e-12, atol=1e-12)


def test_full_forgetting_is_memoryless():
    """P3: g = -30 (alpha ~ 1e-13) makes the memory forget everything but the last token:
    o_t = (q_t . k_t) v_t and ht = k_L^T v_L."""
    q, k, v, _, S0 = rand_inputs(2)
    g = np.full_like(q, -30.0)
    o, ht = gla_recurrent_fwd(q, k, v, g, S0)
    ref = np.sum(q * k, axis=-1, keepdims=True) * v
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(ht, k[:, :, -1, :, None] * v[:, :, -1, None, :], atol=1e-10)


def test_final_state_closed_form():
    """P4: ht = sum_t Diag(prod_{s>t} alpha_s) k_t^T v_t + Diag(prod_s alpha_s) h0."""
    q, k, v, g, S0 = rand_inputs(3)
    _, ht = gla_recurrent_fwd(q, k, v, g, S0)
    L = q.shape[2]
    alpha = np.exp(g)
    ref = np.prod(alpha, axis=2)[..., None] * S0
    for t in range(L):
        later = np.prod(alpha[:, :, t + 1:, :], axis=2)      # empty product = 1 at t = L-1
        ref = ref + later[..., None] * (k[:, :, t, :, None] * v[:, :, t, None, :])
    np.testing.assert_allclose(ht, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C", [1, 2, 3, 4, 8, 16, 32, 64])
def test_chunk_size_independence(C):
    """P5: the chunkwise form equals the recurrence for every chunk size (incl. ragged tails)."""
    q, k, v, g, S0 = rand_inputs(4, L=37)
    o_r, ht_r = gla_recurrent_fwd(q, k, v, g, S0)
    o_c, ht_c = gla_chunkwise_fwd(q, k, v, g, S0, C=C)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(ht_c, ht_r, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("L1", [1, 7, 16, 22])
def test_state_chaining(L1):
    """P6: running [0, L) equals running [0, L1) then [L1, L) from the carried state."""
    q, k, v, g, S0 = rand_inputs(5)
    o, ht = gla_recurrent_fwd(q, k, v, g, S0)
    o1, h1 = gla_recurrent_fwd(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], g[:, :, :L1], S0)
    o2, h2 = gla_recurrent_fwd(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], g[:, :, L1:], h1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h2, ht, rtol=1e-12, atol=1e-12)


def test_decode_steps_equal_forward():
    """P7: T single-token decode steps reproduce the forward outputs and final state."""
    q, k, v, g, S0 = rand_inputs(6)
    o, ht = gla_recurrent_fwd(q, k, v, g, S0)
    S = S0
    for t in range(q.shape[2]):
        ot, S = gla_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], S)
        np.testing.assert_allclose(ot, o[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, ht, rtol=1e-12, atol=1e-12)


def test_linearity_and_independence():
    """P8: outputs are linear in (v, h0) jointly; value columns and (b, h) units independent."""
    q, k, v, g, S0 = rand_inputs(8)
    _, _, v2, _, S2 = rand_inputs(9)
    a, b = 0.7, -1.3
    o1, h1 = gla_recurrent_fwd(q, k, v, g, S0)
    o2, h2 = gla_recurrent_fwd(q, k, v2, g, S2)
    o3, h3 = gla_recurrent_fwd(q, k, a * v + b * v2, g, a * S0 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h3, a * h1 + b * h2, rtol=1e-12, atol=1e-12)
    oc, hc = gla_recurrent_fwd(q, k, v[..., 1:3], g, S0[..., 1:3])
    np.testing.assert_allclose(oc, o1[..., 1:3], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hc, h1[..., 1:3], rtol=1e-12, atol=1e-12)
    ou, hu = gla_recurrent_fwd(q[1:, 1:], k[1:, 1:], v[1:, 1:], g[1:, 1:], S0[1:, 1:])
    np.testing.assert_allclose(ou, o1[1:, 1:], rtol=1e-12, atol=1e-12)


def _loss(q, k, v, g, S0, do, dht):
    o, ht = gla_recurrent_fwd(q, k, v, g, S0)
    return float(np.sum(o * do) + np.sum(ht * dht))


def test_backward_finite_differences():
    """P9: every gradient (dq, dk, dv, dg, dh0, with dht != 0) matches central differences."""
    q, k, v, g, S0 = rand_inputs(10, B=1, H=1, L=11, Dk=3, Dv=2)
    rng = np.random.default_rng(11)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(S0.shape)
    grads = gla_recurrent_bwd(q, k, v, g, do, S0, dht, checkpoint=4)
    args = {"q": q, "k": k, "v": v, "g": g, "h0": S0}
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "h0": "dh0"}
    eps = 1e-6
    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a_p = dict(args, **{name: xp})
            a_m = dict(args, **{name: xm})
            fd[idx] = (_loss(a_p["q"], a_p["k"], a_p["v"], a_p["g"], a_p["h0"], do, dht)
                       - _loss(a_m["q"], a_m["k"], a_m["v"], a_m["g"], a_m["h0"], do, dht)) / (2 * eps)
        np.testing.assert_allclose(grads[names[name]], fd, rtol=1e-6, atol=1e-7,
                                   err_msg=f"d{name}")


def test_dg_identity():
    """P10: dg_t = sum_{s>=t} (q_s*dq_s - k_s*dk_s) + [t = L-1..] rowsum(dht*ht) for every t.

    q_t[i] only enters as q_t[i] e^{G_t[i]} and k_j[i] only as k_j[i] e^{-G_j[i]} (G the
    prefix sum of g), plus e^{G_L} in ht, so the gate gradient is a reverse prefix sum."""
    q, k, v, g, S0 = rand_inputs(12, L=29)
    rng = np.random.default_rng(13)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(S0.shape)
    grads = gla_recurrent_bwd(q, k, v, g, do, S0, dht, checkpoint=8)
    _, ht = gla_recurrent_fwd(q, k, v, g, S0)
    dG = q * grads["dq"] - k * grads["dk"]
    ref = np.flip(np.cumsum(np.flip(dG, axis=2), axis=2), axis=2)
    ref = ref + np.sum(dht * ht, axis=-1)[:, :, None, :]
    np.testing.assert_allclose(grads["dg"], ref, rtol=1e-10, atol=1e-10)


def test_backward_matches_torch_autograd():
    """P11: a third witness, torch float64 autograd through a plain loop of the recurrence."""
    torch = pytest.importorskip("torch")
    q, k, v, g, S0 = rand_inputs(14, L=17)
    rng = np.random.default_rng(15)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(S0.shape)
    T = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for n, x in dict(q=q, k=k, v=v, g=g, h0=S0).items()}
    S = T["h0"]
    outs = []
    for t in range(q.shape[2]):
        S = torch.exp(T["g"][:, :, t]).unsqueeze(-1) * S + \
            T["k"][:, :, t].unsqueeze(-1) * T["v"][:, :, t].unsqueeze(-2)
        outs.append((T["q"][:, :, t].unsqueeze(-2) @ S).squeeze(-2))
    o = torch.stack(outs, dim=2)
    loss = (o * torch.tensor(do)).sum() + (S * torch.tensor(dht)).sum()
    loss.backward()
    grads = gla_recurrent_bwd(q, k, v, g, do, S0, dht, checkpoint=5)
    for n, gn in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("h0", "dh0")]:
        np.testing.assert_allclose(grads[gn], T[n].grad.numpy(), rtol=1e-11, atol=1e-11,
                                   err_msg=gn)


def test_backward_without_optional_states():
    """dh0 and dht default to zero state / zero gradient: compare with explicit zeros."""
    q, k, v, g, _ = rand_inputs(16, L=13)
    do = np.random.default_rng(17).standard_normal(v.shape)
    a = gla_recurrent_bwd(q, k, v, g, do)
    z = np.zeros(q.shape[:2] + (q.shape[-1], v.shape[-1]))
    b = gla_recurrent_bwd(q, k, v, g, do, z, z)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])


def test_large_negative_gate_is_finite():
    """Reading: g is any real; alpha -> 0 must give finite results (no NaN from e^{-big})."""
    q, k, v, g, S0 = rand_inputs(18)
    g = g * 0 - 1e4
    o, ht = gla_recurrent_fwd(q, k, v, g, S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    oc, hc = gla_chunkwise_fwd(q, k, v, g, S0, C=8)
    np.testing.assert_allclose(oc, o, atol=1e-12)
