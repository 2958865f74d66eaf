"""Pins of the fp64 MS-GLA front-end oracle (CPU only).

They tie it to (a) the separately pinned GLA oracle (one group at scale 1 with unit weights is
plain GLA), (b) a brute force written from the definitions in a different form (explicit block
sums, the closed-form GLA double sum, and the hold as "the latest block whose last token has
been seen"), in exact rationals where the gates allow, (c) causality, and (d) pooling and
fusion identities."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gla_recurrent_fwd
from oracle.msgla_oracle import msgla_fwd, msgla_hold, msgla_pool


def rand_in(seed, B=1, H=3, L=11, Dk=3, Dv=2, G=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, Dk))
    k = rng.standard_normal((B, H, L, Dk))
    v = rng.standard_normal((B, H, L, Dv))
    g = -np.log1p(np.exp(-rng.standard_normal((B, H, L, Dk))))
    w = rng.random((B, L, G))
    return q, k, v, g, w


def test_scale_one_is_gla():
    """One group at scale 1 with unit weights is the GLA recurrence itself."""
    q, k, v, g, _ = rand_in(1)
    h0 = np.random.default_rng(2).standard_normal((1, 3, 3, 2))
    o, ht = msgla_fwd(q, k, v, g, [1], [3], np.ones((1, 11, 1)), h0)
    ro, rht = gla_recurrent_fwd(q, k, v, g, h0)
    np.testing.assert_allclose(o, ro, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ht, rht, rtol=1e-13, atol=1e-13)


def brute_force(q, k, v, g, scales, heads, w, exp=np.exp):
    """Per (b, h, t), from the definitions: block averages by explicit sums, GLA as the
    closed-form double sum o_j = sum_{i<=j} sum_c q_j[c] k_i[c] prod_{u=i+1..j} alpha_u[c] v_i,
    and the hold as the largest block j whose last token j*s + s - 1 is <= t.  Also the final
    state S[c][d] = sum_i prod_{u=i+1..n-1} alpha_u[c] k_i[c] v_i[d] over all n pooled tokens
    (the only place the trailing partial block shows)."""
    B, H, L, Dk = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Dv = len(v[0][0][0])
    out = [[[[0] * Dv for _ in range(L)] for _ in range(H)] for _ in range(B)]
    fin = [[[[0] * Dv for _ in range(Dk)] for _ in range(H)] for _ in range(B)]
    grp = [i for i, n in enumerate(heads) for _ in range(n)]
    for b in range(B):
        for h in range(H):
            s = scales[grp[h]]
            n = (L + s - 1) // s

            def pool(x):
                res = []
                for j in range(n):
                    rows = [x[b][h][t] for t in range(j * s, min(j * s + s, L))]
                    res.append([sum(r[c] for r in rows) / len(rows) for c in range(len(rows[0]))])
                return res
            qp, kp, vp, gp = pool(q), pool(k), pool(v), pool(g)
            op = []
            for j in range(n):
                acc = [0] * Dv
                for i in range(j + 1):
                    for c in range(Dk):
                        decay = 1
                        for u in range(i + 1, j + 1):
                            decay = decay * exp(gp[u][c])
                        coef = qp[j][c] * kp[i][c] * decay
                        for d in range(Dv):
                            acc[d] = acc[d] + coef * vp[i][d]
                op.append(acc)
            for t in range(L):
                done = [j for j in range(n) if j * s + s - 1 <= t]
                if done:
                    wt = w[b][t][grp[h]]
                    out[b][h][t] = [wt * x for x in op[max(done)]]
            for c in range(Dk):
                for d in range(Dv):
                    for i in range(n):
                        decay = 1
                        for u in range(i + 1, n):
                            decay = decay * exp(gp[u][c])
                        fin[b][h][c][d] = fin[b][h][c][d] + decay * kp[i][c] * vp[i][d]
    return out, fin


def test_brute_force_exact_rationals():
    """Open gates (alpha = 1, exact) and small rationals: the oracle equals the brute force in
    exact arithmetic, for scales 1, 2 and 3 with a ragged tail (L = 7)."""
    rng = np.random.default_rng(3)
    B, H, L, Dk, Dv = 1, 3, 7, 2, 2
    qi = rng.integers(-3, 4, (B, H, L, Dk))
    ki = rng.integers(-3, 4, (B, H, L, Dk))
    vi = rng.integers(-3, 4, (B, H, L, Dv))
    wi = rng.integers(0, 5, (B, L, 3))
    F = lambda a, d: [[[[Fraction(int(x), d) for x in r] for r in hh] for hh in bb] for bb in a]
    q, k, v = F(qi, 2), F(ki, 3), F(vi, 1)
    g = [[[[Fraction(0)] * Dk for _ in range(L)] for _ in range(H)] for _ in range(B)]
    w = [[[Fraction(int(x), 4) for x in r] for r in bb] for bb in wi]
    ref, fin = brute_force(q, k, v, g, [1, 2, 3], [1, 1, 1], w, exp=lambda x: Fraction(1))
    o, ht = msgla_fwd(qi / 2, ki / 3, vi.astype(float), np.zeros((B, H, L, Dk)), [1, 2, 3], [1, 1, 1], wi / 4)
    np.testing.assert_allclose(o, np.array(ref, dtype=float), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(ht, np.array(fin, dtype=float), rtol=1e-14, atol=1e-14)


def test_brute_force_general_gates():
    """Data-dependent gates, two heads per group at scales 4 and 2 (L = 11: ragged tails)."""
    q, k, v, g, w = rand_in(4, B=2, H=4, L=11, G=2)
    ref, fin = brute_force(q.tolist(), k.tolist(), v.tolist(), g.tolist(), [4, 2], [2, 2], w.tolist(), exp=np.exp)
    o, ht = msgla_fwd(q, k, v, g, [4, 2], [2, 2], w)
    np.testing.assert_allclose(o, np.array(ref), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht, np.array(fin), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s", [1, 2, 4])
def test_causal(s):
    """Changing token t' changes no output at t < t', and does change the outputs from the end
    of t''s block on."""
    q, k, v, g, w = rand_in(5, H=2, L=13, G=1)
    o, _ = msgla_fwd(q, k, v, g, [s], [2], w)
    for tp in (0, 5, 9):
        q2 = q.copy()
        q2[:, :, tp] += 1.0
        o2, _ = msgla_fwd(q2, k, v, g, [s], [2], w)
        np.testing.assert_array_equal(o2[:, :, :tp], o[:, :, :tp])
        end = (tp // s) * s + s - 1
        if end < 13:
            assert np.all(np.abs(o2[:, :, end] - o[:, :, end]) > 0)


def test_pool_of_block_constant_inputs_and_hold_alignment():
    """Inputs constant on each block of s tokens pool to the block values (the trailing
    partial block included), and the hold repeats block j on tokens (j+1)s - 1 ... (j+2)s - 2."""
    s, L = 3, 10
    rng = np.random.default_rng(6)
    blocks = rng.standard_normal((1, 1, 4, 2))
    x = np.repeat(blocks, s, axis=2)[:, :, :L]
    np.testing.assert_allclose(msgla_pool(x, s), blocks, rtol=1e-15, atol=0)
    held = msgla_hold(blocks, s, L)
    np.testing.assert_array_equal(held[:, :, :s - 1], 0.0)
    for t in range(s - 1, L):
        np.testing.assert_array_equal(held[:, :, t], blocks[:, :, (t + 1) // s - 1])


def test_fusion_weights_scale_each_group():
    """The output is linear in the weights, group by group: scaling one group's weights by c
    scales its heads by c and leaves the other group's heads unchanged."""
    q, k, v, g, w = rand_in(7, H=3, G=2)
    o, _ = msgla_fwd(q, k, v, g, [1, 2], [1, 2], w)
    w2 = w.copy()
    w2[..., 1] *= 3.0
    o2, _ = msgla_fwd(q, k, v, g, [1, 2], [1, 2], w2)
    np.testing.assert_array_equal(o2[:, :1], o[:, :1])
    np.testing.assert_allclose(o2[:, 1:], 3.0 * o[:, 1:], rtol=1e-14)
