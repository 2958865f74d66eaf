"""fp64 step-by-step oracle for gated slot attention (GSA).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's CPU-baseline
leg, never by the product path.  It shares no code with the HIP library.

GSA keeps m memory slots per head.  The GSA summaries ("Gated Slot Attention for Efficient
Linear-Time Sequence Modeling": abstract, and the research-map summary, "Approach") describe it
as ABC (bounded-memory control: slot memories written token by token and read through a
softmax over slots) with a data-dependent forget gate per slot, computable as two GLA passes
linked by a softmax.  This oracle evaluates the slot memories directly, token by token, not as
two passes, so that a two-pass implementation is checked against a different formulation:

    alpha_t = exp(g_t),  w_t = 1 - alpha_t = -expm1(g_t)        (g_t in R^m, one gate per slot)
    Kmem_t = Diag(alpha_t) Kmem_{t-1} + w_t^T k_t               (Kmem in R^{m x Dk})
    Vmem_t = Diag(alpha_t) Vmem_{t-1} + w_t^T v_t               (Vmem in R^{m x Dv})
    z_t = Kmem_t q_t^T,  p_t = softmax(z_t),  o_t = p_t Vmem_t

The read-out nonlinearity between the two memories is softmax by default.  The GSA summary's
ablations ("Measured effects": replacing the softmax) also run Swish, ReLU and ReLU^2 in its
place, or none; those variants are read as the function applied to each slot score alone,
with no normalisation over the slots (act = "swish": z * sigmoid(z); "relu": max(z, 0);
"relu2": max(z, 0)^2; "none": z).

Readings taken where the pages are silent: the slot write weight is the complement of the
forget gate (w = 1 - alpha), the same weights write keys and values; softmax temperature is 1
(max-subtracted, which is the same function); initial memories default to zero.  The states
exchanged with callers use the two-pass orientation: hk = Kmem^T [B,H,Dk,m], hv = Vmem
[B,H,m,Dv].
"""
from __future__ import annotations

import numpy as np

__all__ = ["gsa_recurrent_fwd", "gsa_recurrent_bwd", "gsa_decode_step", "ACTS"]

ACTS = ("softmax", "swish", "relu", "relu2", "none")


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _softmax(z):
    z = z - np.max(z, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def _sigmoid(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def _read(z, act):
    """Slot weights p from slot scores z (last axis = slots)."""
    if act == "softmax":
        return _softmax(z)
    if act == "swish":
        return z * _sigmoid(z)
    if act == "relu":
        return np.maximum(z, 0.0)
    if act == "relu2":
        return np.maximum(z, 0.0) ** 2
    if act == "none":
        return z.copy()
    raise ValueError(f"unknown read-out {act!r}")


def _read_bwd(z, p, dp, act):
    """dLoss/dz from dLoss/dp through the read-out."""
    if act == "softmax":
        return p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    if act == "swish":
        sg = _sigmoid(z)
        return dp * sg * (1.0 + z * (1.0 - sg))
    if act == "relu":
        return dp * (z > 0)
    if act == "relu2":
        return dp * 2.0 * np.maximum(z, 0.0)
    if act == "none":
        return dp.copy()
    raise ValueError(f"unknown read-out {act!r}")


def _init(hk0, hv0, B, H, Dk, Dv, m):
    Km = np.zeros((B, H, m, Dk)) if hk0 is None else np.swapaxes(hk0, -1, -2).copy()
    Vm = np.zeros((B, H, m, Dv)) if hv0 is None else hv0.copy()
    return Km, Vm


def _step(Km, Vm, k_t, v_t, g_t):
    a = np.exp(g_t)
    w = -np.expm1(g_t)
    Km = a[..., None] * Km + w[..., None] * k_t[:, :, None, :]
    Vm = a[..., None] * Vm + w[..., None] * v_t[:, :, None, :]
    return Km, Vm


def gsa_recurrent_fwd(q, k, v, g, hk0=None, hv0=None, act="softmax"):
    """Returns (o [B,H,L,Dv], hkt [B,H,Dk,m], hvt [B,H,m,Dv]) in float64."""
    q, k, v, g, hk0, hv0 = map(_f64, (q, k, v, g, hk0, hv0))
    B, H, L, Dk = q.shape
    Dv, m = v.shape[-1], g.shape[-1]
    Km, Vm = _init(hk0, hv0, B, H, Dk, Dv, m)
    o = np.empty((B, H, L, Dv))
    for t in range(L):
        Km, Vm = _step(Km, Vm, k[:, :, t], v[:, :, t], g[:, :, t])
        p = _read((Km @ q[:, :, t, :, None])[..., 0], act)               # [B,H,m]
        o[:, :, t] = (p[:, :, None, :] @ Vm)[:, :, 0, :]
    return o, np.swapaxes(Km, -1, -2), Vm


def gsa_recurrent_bwd(q, k, v, g, do, hk0=None, hv0=None, dhkt=None, dhvt=None,
                      checkpoint: int = 64, act="softmax"):
    """Reverse-mode gradient of sum(o*do) + sum(hkt*dhkt) + sum(hvt*dhvt).

    Walks tokens from last to first carrying dK = dLoss/dKmem_t and dV = dLoss/dVmem_t.
    At token t (memories after the write: Km, Vm; before it: Km', Vm'):
        dV  += p_t^T do_t;   dp = Vm do_t^T;   dz = p * (dp - <dp, p>)   (softmax backward;
                                                  the other read-outs: dz = f'(z) dp)
        dK  += dz^T q_t;     dq_t = dz Km
        dk_t = w_t dK;       dv_t = w_t dV
        dw   = rowsum(dK * k_t) + rowsum(dV * v_t)
        dalpha = rowsum(dK * Km') + rowsum(dV * Vm')
        dg_t = alpha * (dalpha - dw)               (alpha = e^g, w = 1 - e^g)
        dK, dV = Diag(alpha) dK, Diag(alpha) dV
    Returns dict dq, dk, dv, dg, dhk0 [B,H,Dk,m], dhv0 [B,H,m,Dv] (float64).
    """
    q, k, v, g, do, hk0, hv0, dhkt, dhvt = map(
        _f64, (q, k, v, g, do, hk0, hv0, dhkt, dhvt))
    B, H, L, Dk = q.shape
    Dv, m = v.shape[-1], g.shape[-1]
    Km, Vm = _init(hk0, hv0, B, H, Dk, Dv, m)
    starts = list(range(0, L, checkpoint))
    ckpts = []
    for s in starts:
        ckpts.append((Km, Vm))
        for t in range(s, min(s + checkpoint, L)):
            Km, Vm = _step(Km, Vm, k[:, :, t], v[:, :, t], g[:, :, t])
    dK = np.zeros((B, H, m, Dk)) if dhkt is None else np.swapaxes(dhkt, -1, -2).copy()
    dV = np.zeros((B, H, m, Dv)) if dhvt is None else dhvt.copy()
    dq = np.empty((B, H, L, Dk)); dk = np.empty((B, H, L, Dk))
    dv = np.empty((B, H, L, Dv)); dg = np.empty((B, H, L, m))
    for si in range(len(starts) - 1, -1, -1):
        t0, t1 = starts[si], min(starts[si] + checkpoint, L)
        seg = [ckpts[si]]
        for t in range(t0, t1):
            seg.append(_step(*seg[-1], k[:, :, t], v[:, :, t], g[:, :, t]))
        for t in range(t1 - 1, t0 - 1, -1):
            (Kb, Vb), (Ka, Va) = seg[t - t0], seg[t - t0 + 1]
            a = np.exp(g[:, :, t]); w = -np.expm1(g[:, :, t])
            z = (Ka @ q[:, :, t, :, None])[..., 0]
            p = _read(z, act)
            dV = dV + p[..., None] * do[:, :, t, None, :]
            dp = (Va @ do[:, :, t, :, None])[..., 0]
            dz = _read_bwd(z, p, dp, act)
            dK = dK + dz[..., None] * q[:, :, t, None, :]
            dq[:, :, t] = (dz[:, :, None, :] @ Ka)[:, :, 0, :]
            dk[:, :, t] = (w[:, :, None, :] @ dK)[:, :, 0, :]
            dv[:, :, t] = (w[:, :, None, :] @ dV)[:, :, 0, :]
            dw = np.sum(dK * k[:, :, t, None, :], axis=-1) + np.sum(dV * v[:, :, t, None, :], axis=-1)
            dalpha = np.sum(dK * Kb, axis=-1) + np.sum(dV * Vb, axis=-1)
            dg[:, :, t] = a * (dalpha - dw)
            dK = a[..., None] * dK
            dV = a[..., None] * dV
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg,
            "dhk0": np.swapaxes(dK, -1, -2), "dhv0": dV}


def gsa_decode_step(q, k, v, g, hk, hv, act="softmax"):
    """One recurrent inference step of GSA on a single token per (batch, head): the bounded
    slot memories make inference O(1) in memory per token (GSA abstract: efficient recurrent
    inference with a compact state; research-map summary, "Approach").

    q, k [B,H,Dk]; v [B,H,Dv]; g [B,H,m] slot log-gates; hk [B,H,Dk,m] (= Kmem^T);
    hv [B,H,m,Dv] (= Vmem).  Written slot by slot from the slot-memory definition:
        for each slot s:  Kmem[s] <- alpha_s Kmem[s] + w_s k,   Vmem[s] <- alpha_s Vmem[s] + w_s v,
                          z_s = <Kmem[s], q>
        p = softmax(z) (or the read-out act),  o = sum_s p_s Vmem[s].
    Returns (o [B,H,Dv], hk_new [B,H,Dk,m], hv_new [B,H,m,Dv]), float64.
    """
    q, k, v, g, hk, hv = map(_f64, (q, k, v, g, hk, hv))
    m = g.shape[-1]
    hk = hk.copy()
    hv = hv.copy()
    z = np.empty(g.shape)
    for s in range(m):
        a = np.exp(g[..., s])[..., None]
        w = -np.expm1(g[..., s])[..., None]
        hk[..., :, s] = a * hk[..., :, s] + w * k
        hv[..., s, :] = a * hv[..., s, :] + w * v
        z[..., s] = np.sum(hk[..., :, s] * q, axis=-1)
    p = _read(z, act)
    o = np.einsum("bhs,bhsd->bhd", p, hv)
    return o, hk, hv
