"""fp64 step-by-step oracle for gated linear attention (GLA).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's CPU-baseline
leg, never by the product path.  It shares no code with the HIP library.

What is computed (per batch row b and head h, tokens t = 0..L-1):

    alpha_t = exp(g_t)                          (g_t in R^Dk: log forget gate per key channel)
    S_t     = Diag(alpha_t) S_{t-1} + k_t^T v_t (S in R^{Dk x Dv}, S_{-1} = h0 or 0)
    o_t     = q_t S_t                           (read after the update)
    ht      = S_{L-1}

Sources: the GLA visual companion ("Gated Linear Attention for Efficient Long Sequences",
cards "Core move" and "Step-by-step memory update") describes replacing softmax attention by
a gated update of a compressed matrix memory that the gate can keep, decay or overwrite; the
MS-GLA summary (section 2.1, "Linear Attention and Gated Linear Attention") says GLA's
forget gate is data dependent and scales the rows of the memory.  Readings taken where the
pages are silent: the output reads the state after the current token's write; the gate is
given in log space (alpha = exp(g)), one value per key channel, so Diag(alpha) scales rows;
no softmax-style scale is applied inside the operator; h0 = None means a zero state.

All inputs are upcast to float64 before any arithmetic; arrays have shape [B, H, L, D].
"""
from __future__ import annotations

from typing import Optional

import numpy as np

__all__ = ["gla_recurrent_fwd", "gla_recurrent_bwd", "gla_decode_step", "gla_chunkwise_fwd"]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def gla_recurrent_fwd(q, k, v, g, h0=None):
    """Token-by-token recurrence.  Returns (o [B,H,L,Dv], ht [B,H,Dk,Dv]) in float64."""
    q, k, v, g, h0 = map(_f64, (q, k, v, g, h0))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    S = np.zeros((B, H, Dk, Dv)) if h0 is None else h0.copy()
    o = np.empty((B, H, L, Dv))
    for t in range(L):
        alpha = np.exp(g[:, :, t, :])                                   # [B,H,Dk]
        S = alpha[..., None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        o[:, :, t, :] = (q[:, :, t, None, :] @ S)[:, :, 0, :]
    return o, S


def _segment_states(k, v, g, S_start, t0, t1):
    """States around tokens t0..t1-1: out[u] = state before token t0+u, out[u+1] = after it."""
    out = [S_start]
    S = S_start
    for t in range(t0, t1):
        S = np.exp(g[:, :, t, :])[..., None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        out.append(S)
    return out


def gla_recurrent_bwd(q, k, v, g, do, h0=None, dht=None, checkpoint: int = 64):
    """Reverse-mode gradient of sum(o*do) + sum(ht*dht) through the recurrence.

    Walks tokens from last to first carrying dS = dLoss/dS_t.  At token t:
        dS    += q_t^T do_t              (o_t = q_t S_t)
        dq_t   = S_t do_t^T
        dk_t   = dS v_t^T                (S_t contains k_t^T v_t)
        dv_t   = k_t dS
        dg_t   = alpha_t * rowsum(dS * S_{t-1})    (d alpha/d g = alpha)
        dS     = Diag(alpha_t) dS        (gradient handed to S_{t-1})
    and dh0 = dS after the walk.  States are recomputed per segment from checkpoints taken
    every `checkpoint` tokens in a forward sweep, which only bounds memory.
    Returns a dict with dq, dk, dv, dg [B,H,L,*] and dh0 [B,H,Dk,Dv], all float64.
    """
    q, k, v, g, do, h0, dht = map(_f64, (q, k, v, g, do, h0, dht))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    S0 = np.zeros((B, H, Dk, Dv)) if h0 is None else h0
    starts = list(range(0, L, checkpoint))
    ckpts = []
    S = S0
    for s in starts:
        ckpts.append(S)
        seg = _segment_states(k, v, g, S, s, min(s + checkpoint, L))
        S = seg[-1]
    dq = np.empty((B, H, L, Dk)); dk = np.empty((B, H, L, Dk))
    dv = np.empty((B, H, L, Dv)); dg = np.empty((B, H, L, Dk))
    dS = np.zeros((B, H, Dk, Dv)) if dht is None else dht.copy()
    for si in range(len(starts) - 1, -1, -1):
        t0 = starts[si]
        t1 = min(t0 + checkpoint, L)
        seg = _segment_states(k, v, g, ckpts[si], t0, t1)
        for t in range(t1 - 1, t0 - 1, -1):
            S_after, S_before = seg[t - t0 + 1], seg[t - t0]
            alpha = np.exp(g[:, :, t, :])
            dS = dS + q[:, :, t, :, None] * do[:, :, t, None, :]
            dq[:, :, t, :] = (S_after @ do[:, :, t, :, None])[..., 0]
            dk[:, :, t, :] = (dS @ v[:, :, t, :, None])[..., 0]
            dv[:, :, t, :] = (k[:, :, t, None, :] @ dS)[:, :, 0, :]
            dg[:, :, t, :] = alpha * np.sum(dS * S_before, axis=-1)
            dS = alpha[..., None] * dS
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dh0": dS}


def gla_decode_step(q, k, v, g, state):
    """One recurrent inference step on a single token per (batch, head).

    q, k, g [B,H,Dk]; v [B,H,Dv]; state [B,H,Dk,Dv].  Returns (o [B,H,Dv], new_state), float64.
    This is the O(1)-memory inference form of the same recurrence (MS-GLA summary, section 1:
    linear recurrent models give O(1) inference memory; GSA abstract: efficient recurrent
    inference).
    """
    q, k, v, g, S = map(_f64, (q, k, v, g, state))
    S = np.exp(g)[..., None] * S + k[..., :, None] * v[..., None, :]
    o = (q[..., None, :] @ S)[..., 0, :]
    return o, S


def gla_chunkwise_fwd(q, k, v, g, h0=None, C: int = 16):
    """fp64 chunkwise form, kept only to test that the method's result is independent of the
    chunk size and equals the recurrence.

    Sequence cut into chunks of C tokens (last one possibly shorter): states are passed from
    chunk to chunk, and inside a chunk all outputs are formed at once (MS-GLA summary, section
    2.1: sequential inter-chunk updates, parallel intra-chunk computation).  With b the
    chunk-local inclusive cumulative sum of g and Gamma its last row:
        O  = (Q * exp(b)) S_n + ((Q K^T with exp(b_r - b_c) per channel) masked to c <= r) V
        S_{n+1} = Diag(exp(Gamma)) S_n + (K * exp(Gamma - b))^T V
    The exponent differences are formed directly in float64 (no factorisation).
    """
    q, k, v, g, h0 = map(_f64, (q, k, v, g, h0))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    S = np.zeros((B, H, Dk, Dv)) if h0 is None else h0.copy()
    o = np.empty((B, H, L, Dv))
    for n0 in range(0, L, C):
        sl = slice(n0, min(n0 + C, L))
        Q, K, V = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        b = np.cumsum(g[:, :, sl], axis=2)                              # [B,H,c,Dk]
        c = b.shape[2]
        causal = np.tril(np.ones((c, c), dtype=bool))                   # c <= r
        diff = b[:, :, :, None, :] - b[:, :, None, :, :]                # [B,H,r,c,Dk]
        diff = np.where(causal[None, None, :, :, None], diff, -np.inf)
        A = np.einsum("bhri,bhci,bhrci->bhrc", Q, K, np.exp(diff))
        o[:, :, sl] = (Q * np.exp(b)) @ S + A @ V
        gamma = b[:, :, -1, :]                                          # [B,H,Dk]
        Kd = K * np.exp(gamma[:, :, None, :] - b)
        S = np.exp(gamma)[..., None] * S + np.swapaxes(Kd, -1, -2) @ V
    return o, S
