"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module draws random numbers and shapes them into the operator's inputs; it contains
none of the operator's arithmetic.  Every array is generated on the CPU in float32 from one
``numpy.random.Generator(PCG64(seed))`` per workload, in a fixed draw order, and, for bf16
workloads, rounded to bf16 (round to nearest, ties to even) while still stored as float32,
so that the oracle and the GPU path read bit-identical values.

Shapes and laws (readings of the pages' workloads; a token is one position of one batch row):

* q, k, v ~ N(0, 1); q is multiplied by Dk**-0.5 before rounding.
* gates g = log(alpha) = logsigmoid(x @ W) / 16, x ~ N(0, 1) of width 1024, W ~ N(0, 1/1024)
  (variance 1/1024) projected to H*Dk channels.  This gives per-token, per-key-channel,
  data-dependent forget gates as in the GLA summaries (MS-GLA summary, section 2.1: the gate
  scales the rows of the memory).
* long-sequence workload: 13 of 128 key channels per head (a seeded permutation, the same for
  every batch row and position) get +4 inside the logsigmoid, i.e. alpha close to 1.
* GSA slot gates: g = logsigmoid(N(0, 1)) / 16 per slot.
* initial states, where present, ~ N(0, 0.02**2) in float32.
* upstream gradients ~ N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "round_bf16", "logsigmoid", "GlaWorkload", "GsaWorkload", "DecodeWorkload",
    "GsaDecodeWorkload", "gla_inputs", "gsa_inputs", "decode_inputs", "gsa_decode_inputs", "WORKLOADS",
]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return them as float32.

    NaN stays NaN.  The bit pattern of every result has its low 16 bits clear, so the values
    convert to torch.bfloat16 exactly.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out).astype(np.float32)


def logsigmoid(x: np.ndarray) -> np.ndarray:
    """log(sigmoid(x)) = -log1p(exp(-x)), evaluated stably for both signs (input law only)."""
    x = np.asarray(x, dtype=np.float64)
    return (np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class GlaWorkload:
    name: str
    B: int
    H: int
    L: int
    Dk: int
    Dv: int
    C: int
    dtype: str            # "bf16" or "f32"
    seed: int
    h0: bool = False      # non-zero initial state
    gate_law: str = "proj"  # "proj" = logsigmoid(xW)/16, "iid" = logsigmoid(N(0,1))/16
    bias_frac: float = 0.0  # fraction of key channels per head biased toward alpha ~ 1


@dataclasses.dataclass(frozen=True)
class GsaWorkload:
    name: str
    B: int
    H: int
    L: int
    Dk: int
    Dv: int
    m: int
    C: int
    dtype: str
    seed: int
    h0: bool = False


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    T: int      # number of single-token steps
    B: int
    H: int
    Dk: int
    Dv: int
    dtype: str
    seed: int
    bias_frac: float = 0.1


@dataclasses.dataclass(frozen=True)
class GsaDecodeWorkload:
    name: str
    T: int      # number of single-token steps
    B: int
    H: int
    Dk: int
    Dv: int
    m: int
    dtype: str
    seed: int


# The workloads named by the measurement plan (sizes from the pages' model shapes: the 340M
# and 1.3B GLA layers, a 20K-token sequence, and GSA with 64 slots).
WORKLOADS = {
    "tiny_f32": GlaWorkload("tiny_f32", 1, 1, 64, 16, 16, 16, "f32", 1001, gate_law="iid"),
    "gla_340m": GlaWorkload("gla_340m", 8, 4, 2048, 128, 256, 64, "bf16", 1002),
    "gla_1p3b": GlaWorkload("gla_1p3b", 4, 4, 4096, 256, 512, 64, "bf16", 1003, h0=True),
    "gla_long": GlaWorkload("gla_long", 1, 4, 20480, 128, 256, 64, "bf16", 1004, bias_frac=0.1),
    "decode": DecodeWorkload("decode", 1024, 64, 4, 128, 256, "bf16", 1004),
    "gsa_340m": GsaWorkload("gsa_340m", 8, 4, 2048, 128, 128, 64, 64, "bf16", 1005),
    # the GSA layer with 128 slots (the GSA summary's slot-count ablation); chunk 32, the
    # largest at which the backward's kernels fit 128 slots
    "gsa_340m_m128": GsaWorkload("gsa_340m_m128", 8, 4, 2048, 128, 128, 128, 32, "bf16", 1007),
    # GSA recurrent inference at the GSA layer's dimensions with the decode batch
    "gsa_decode": GsaDecodeWorkload("gsa_decode", 1024, 64, 4, 128, 128, 64, "bf16", 1006),
}


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def _bias_mask(rng: np.random.Generator, H: int, Dk: int, frac: float) -> np.ndarray:
    """[H, Dk] 0/1 mask: round(frac*Dk) channels per head chosen by a seeded permutation."""
    n = int(round(frac * Dk))
    mask = np.zeros((H, Dk), dtype=np.float32)
    for h in range(H):
        mask[h, rng.permutation(Dk)[:n]] = 1.0
    return mask


def _proj_gates(rng: np.random.Generator, B: int, L: int, H: int, Dk: int,
                bias: Optional[np.ndarray]) -> np.ndarray:
    """g = logsigmoid(x W + 4*bias)/16 with x [B, L, 1024] ~ N(0,1), W ~ N(0, 1/1024)."""
    width = 1024
    g = np.empty((B, H, L, Dk), dtype=np.float32)
    W = (rng.standard_normal((width, H * Dk), dtype=np.float32) / np.float32(32.0))
    for b in range(B):  # one batch row at a time keeps the temporary small
        x = rng.standard_normal((L, width), dtype=np.float32)
        pre = (x @ W).reshape(L, H, Dk)
        if bias is not None:
            pre = pre + 4.0 * bias[None, :, :]
        g[b] = (logsigmoid(pre) / np.float32(16.0)).transpose(1, 0, 2)
    return g


def gla_inputs(w: GlaWorkload, *, with_grad: bool = True, B: Optional[int] = None,
               L: Optional[int] = None) -> dict:
    """Inputs of one GLA workload as float32 numpy arrays holding values exact in w.dtype.

    Returns q, k, g [B,H,L,Dk]; v [B,H,L,Dv]; h0 [B,H,Dk,Dv] or None; do [B,H,L,Dv] and
    dht [B,H,Dk,Dv] (None unless with_grad).  B and L may be overridden to draw a smaller
    instance of the same law (used by tests); the draw order stays q, k, v, gates, h0, do.
    """
    B = w.B if B is None else B
    L = w.L if L is None else L
    H, Dk, Dv = w.H, w.Dk, w.Dv
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal((B, H, L, Dk), dtype=np.float32) * np.float32(Dk ** -0.5)
    k = rng.standard_normal((B, H, L, Dk), dtype=np.float32)
    v = rng.standard_normal((B, H, L, Dv), dtype=np.float32)
    if w.gate_law == "iid":
        g = logsigmoid(rng.standard_normal((B, H, L, Dk), dtype=np.float32)) / np.float32(16.0)
    else:
        bias = _bias_mask(rng, H, Dk, w.bias_frac) if w.bias_frac > 0 else None
        g = _proj_gates(rng, B, L, H, Dk, bias)
    h0 = (rng.standard_normal((B, H, Dk, Dv), dtype=np.float32) * np.float32(0.02)
          if w.h0 else None)
    out = {
        "q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
        "g": _cast(g, w.dtype), "h0": h0, "do": None, "dht": None,
    }
    if with_grad:
        out["do"] = _cast(rng.standard_normal((B, H, L, Dv), dtype=np.float32), w.dtype)
        out["dht"] = rng.standard_normal((B, H, Dk, Dv), dtype=np.float32) * np.float32(0.02)
    return out


def gsa_inputs(w: GsaWorkload, *, with_grad: bool = True, B: Optional[int] = None,
               L: Optional[int] = None) -> dict:
    """Inputs of one GSA workload: q, k [B,H,L,Dk], v [B,H,L,Dv], g [B,H,L,m] slot log-gates,
    optional hk0 [B,H,Dk,m], hv0 [B,H,m,Dv], and do [B,H,L,Dv], dhkt, dhvt when with_grad."""
    B = w.B if B is None else B
    L = w.L if L is None else L
    H, Dk, Dv, m = w.H, w.Dk, w.Dv, w.m
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal((B, H, L, Dk), dtype=np.float32) * np.float32(Dk ** -0.5)
    k = rng.standard_normal((B, H, L, Dk), dtype=np.float32)
    v = rng.standard_normal((B, H, L, Dv), dtype=np.float32)
    g = logsigmoid(rng.standard_normal((B, H, L, m), dtype=np.float32)) / np.float32(16.0)
    hk0 = hv0 = None
    if w.h0:
        hk0 = rng.standard_normal((B, H, Dk, m), dtype=np.float32) * np.float32(0.02)
        hv0 = rng.standard_normal((B, H, m, Dv), dtype=np.float32) * np.float32(0.02)
    out = {"q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
           "g": _cast(g, w.dtype), "hk0": hk0, "hv0": hv0,
           "do": None, "dhkt": None, "dhvt": None}
    if with_grad:
        out["do"] = _cast(rng.standard_normal((B, H, L, Dv), dtype=np.float32), w.dtype)
        out["dhkt"] = rng.standard_normal((B, H, Dk, m), dtype=np.float32) * np.float32(0.02)
        out["dhvt"] = rng.standard_normal((B, H, m, Dv), dtype=np.float32) * np.float32(0.02)
    return out


def decode_inputs(w: DecodeWorkload, *, T: Optional[int] = None, B: Optional[int] = None) -> dict:
    """Pre-generated single-token stream: q, k, g [T,B,H,Dk], v [T,B,H,Dv]; state [B,H,Dk,Dv]
    float32 ~ N(0, 0.02**2).  Gates follow the long-sequence law (projected, 10% of channels
    biased toward alpha ~ 1)."""
    T = w.T if T is None else T
    B = w.B if B is None else B
    H, Dk, Dv = w.H, w.Dk, w.Dv
    rng = np.random.Generator(np.random.PCG64(w.seed + 100))
    q = rng.standard_normal((T, B, H, Dk), dtype=np.float32) * np.float32(Dk ** -0.5)
    k = rng.standard_normal((T, B, H, Dk), dtype=np.float32)
    v = rng.standard_normal((T, B, H, Dv), dtype=np.float32)
    bias = _bias_mask(rng, H, Dk, w.bias_frac)
    # gates: projection of a width-1024 token feature; batch rows play the role of positions
    g = np.empty((T, B, H, Dk), dtype=np.float32)
    W = rng.standard_normal((1024, H * Dk), dtype=np.float32) / np.float32(32.0)
    for t in range(T):
        x = rng.standard_normal((B, 1024), dtype=np.float32)
        pre = (x @ W).reshape(B, H, Dk) + 4.0 * bias[None]
        g[t] = logsigmoid(pre) / np.float32(16.0)
    state = rng.standard_normal((B, H, Dk, Dv), dtype=np.float32) * np.float32(0.02)
    return {"q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
            "g": _cast(g, w.dtype), "state": state}


def gsa_decode_inputs(w: GsaDecodeWorkload, *, T: Optional[int] = None, B: Optional[int] = None) -> dict:
    """Pre-generated single-token GSA stream: q, k [T,B,H,Dk], v [T,B,H,Dv], g [T,B,H,m] slot
    log-gates (the GSA law, logsigmoid(N(0, 1)) / 16); slot memories hk [B,H,Dk,m] and
    hv [B,H,m,Dv] float32 ~ N(0, 0.02**2)."""
    T = w.T if T is None else T
    B = w.B if B is None else B
    H, Dk, Dv, m = w.H, w.Dk, w.Dv, w.m
    rng = np.random.Generator(np.random.PCG64(w.seed + 100))
    q = rng.standard_normal((T, B, H, Dk), dtype=np.float32) * np.float32(Dk ** -0.5)
    k = rng.standard_normal((T, B, H, Dk), dtype=np.float32)
    v = rng.standard_normal((T, B, H, Dv), dtype=np.float32)
    g = logsigmoid(rng.standard_normal((T, B, H, m), dtype=np.float32)) / np.float32(16.0)
    hk = rng.standard_normal((B, H, Dk, m), dtype=np.float32) * np.float32(0.02)
    hv = rng.standard_normal((B, H, m, Dv), dtype=np.float32) * np.float32(0.02)
    return {"q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
            "g": _cast(g, w.dtype), "hk": hk, "hv": hv}
