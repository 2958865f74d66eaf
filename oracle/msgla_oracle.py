"""fp64 oracle of the multi-scale GLA (MS-GLA) operator front end.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's CPU-baseline
leg, never by the product path.  It shares no code with the HIP library; its GLA step is the
token-by-token recurrence of gla_oracle.

The MS-GLA summary ("MS-GLA: Multi-Scale Gated Linear Attention ...": sections 3.1 to 3.4)
describes the layer as head groups, one per temporal scale s, each running GLA on a pooled
copy of the sequence, whose outputs are brought back to token resolution and fused:

  pooling (section 3.1): non-overlapping average pooling of blocks of s tokens; the sequence is
      right-padded and the padding is masked, so a trailing partial block averages only its
      real tokens; the pooled length is ceil(L / s).  Read here as pooling each of q, k, v and
      g of the group's heads (q, k, v are linear in the hidden state, so pooling them equals
      projecting the pooled state; the gates are pooled in the same way).
  branch (sections 3.2, 3.4): GLA on the pooled sequence, with the group's own heads.
  causal hold (section 3.3): a pooled block's output is used only once all of its tokens have
      been seen, then repeated: token t reads block j = floor((t + 1) / s) - 1, and zero while
      no block is complete (t + 1 < s).  For s = 1 this is the identity.
  fusion (section 3.3): weights computed by the caller from the unpooled hidden state (the
      learned router is outside the operator) scale each group's aligned output per token:
          o[b, h, t] = w[b, t, group(h)] * held_group(h)[b, h, t]
      The head groups stay side by side in o; the weighted sum over groups is completed by the
      output projection that follows, which is linear and partitioned by head group.

Head h belongs to the group i with heads[0] + ... + heads[i-1] <= h < heads[0] + ... + heads[i].
"""
from __future__ import annotations

import numpy as np

from .gla_oracle import gla_recurrent_fwd

__all__ = ["msgla_pool", "msgla_hold", "msgla_fwd"]


def msgla_pool(x, s: int):
    """Average over non-overlapping blocks of s tokens along axis 2 ([B, H, L, D]), the trailing
    partial block averaging only its real tokens.  Returns [B, H, ceil(L / s), D] float64."""
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[2]
    n = -(-L // s)
    out = np.empty(x.shape[:2] + (n,) + x.shape[3:])
    for j in range(n):
        out[:, :, j] = x[:, :, j * s:min((j + 1) * s, L)].mean(axis=2)
    return out


def msgla_hold(xp, s: int, L: int):
    """Causal hold of pooled outputs xp [B, H, n, D] back to L tokens: token t gets block
    floor((t + 1) / s) - 1, or zeros when no block is complete yet."""
    out = np.zeros(xp.shape[:2] + (L,) + xp.shape[3:])
    for t in range(L):
        j = (t + 1) // s - 1
        if j >= 0:
            out[:, :, t] = xp[:, :, j]
    return out


def msgla_fwd(q, k, v, g, scales, heads, w, h0=None):
    """MS-GLA forward.  q, k, g [B,H,L,Dk]; v [B,H,L,Dv]; scales and heads: one entry per head
    group (sum(heads) = H); w [B, L, len(scales)] fusion weights; h0 [B,H,Dk,Dv] or None, the
    initial state of every head's branch.  Returns (o [B,H,L,Dv], ht [B,H,Dk,Dv]) where ht is
    each branch's state after its last pooled token."""
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    w = np.asarray(w, dtype=np.float64)
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    assert sum(heads) == H and len(scales) == len(heads) == w.shape[-1]
    o = np.empty((B, H, L, Dv))
    ht = np.empty((B, H, Dk, Dv))
    h = 0
    for i, (s, nh) in enumerate(zip(scales, heads)):
        sel = slice(h, h + nh)
        pooled = [msgla_pool(a[:, sel], s) for a in (q, k, v, g)]
        op, ht[:, sel] = gla_recurrent_fwd(*pooled, None if h0 is None else np.asarray(h0)[:, sel])
        o[:, sel] = w[:, None, :, i, None] * msgla_hold(op, s, L)
        h += nh
    return o, ht
