"""Python binding of libgla_amd.so (include/gla.h): gated linear attention on MI355X.

Argument marshalling only.  Every step of the computation runs in the library's HIP kernels;
torch supplies device memory (outputs, workspace) and the current stream.  There is no CPU
or PyTorch fallback: if the library is missing or cannot be loaded every call raises.

Entry points (same names as the C ABI):
    gla_fwd(q, k, v, g, C=64, h0=None, output_final_state=True) -> (o, ht)
    gla_fwd_noalloc(q, k, v, g, C=64, h0=None, output_final_state=True) -> (o, ht)
        (gla_fwd on the library's fixed scratch buffer; no workspace allocation)
    gla_bwd(q, k, v, g, do, C=64, h0=None, dht=None, want_dh0=False) -> (dq, dk, dv, dg, dh0)
    gla_fwd_save(q, k, v, g, C=64, h0=None, output_final_state=True) -> (o, ht, saved)
    gla_bwd_saved(q, k, v, g, do, saved, C=64, h0=None, dht=None, want_dh0=False)
        -> (dq, dk, dv, dg, dh0)             (saved: what gla_fwd_save left for these inputs)
    gla_decode_step(q, k, v, g, state) -> o                     (state updated in place)
    gsa_fwd(q, k, v, g, C=64, hk0=None, hv0=None, output_final_state=True, act="softmax")
        -> (o, hkt, hvt)
    gsa_decode_step(q, k, v, g, hk, hv, act="softmax") -> o     (hk, hv updated in place)
    gsa_bwd(q, k, v, g, do, C=64, hk0=None, hv0=None, dhkt=None, dhvt=None, want_dh0=False,
            act="softmax") -> (dq, dk, dv, dg, dhk0, dhv0)
    (act: the read-out between GSA's passes, one of GSA_ACTS)
    msgla_fwd(q, k, v, g, scales, heads, w=None, C=64, h0=None, output_final_state=True)
        -> (o, ht)                         (multi-scale GLA over head groups; w [B,L,groups])
Layouts: q, k, g [B,H,L,Dk]; v, o, do [B,H,L,Dv] (all bf16 or all float32); states float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # imported first so the library binds to the HIP runtime torch already loaded

__all__ = [
    "lib", "lib_path", "GlaError", "gla_fwd", "gla_fwd_noalloc", "gla_bwd", "gla_fwd_save", "gla_bwd_saved", "gla_decode_step",
    "gsa_fwd", "gsa_bwd", "gsa_decode_step", "gla_saved_bytes", "gla_bwd_saved_workspace_bytes",
    "gla_fwd_workspace_bytes", "gla_bwd_workspace_bytes", "gsa_fwd_workspace_bytes",
    "gsa_bwd_workspace_bytes", "EXPORTED_SYMBOLS", "GSA_ACTS", "msgla_fwd", "msgla_fwd_workspace_bytes",
    "gsa_fwd_save", "gsa_bwd_saved", "gsa_saved_bytes", "gsa_bwd_saved_workspace_bytes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# GLA_AMD_LIB: another build of the same library (the host-AddressSanitizer one, for instance)
lib_path = os.environ.get("GLA_AMD_LIB") or os.path.join(_HERE, "libgla_amd.so")

GLA_F32, GLA_BF16 = 0, 1
_DT = {torch.float32: GLA_F32, torch.bfloat16: GLA_BF16}
# read-outs between GSA's two passes, in the order of gla.h's gsa_act values
GSA_ACTS = ("softmax", "swish", "relu", "relu2", "none")


def _act(act: str) -> int:
    if act not in GSA_ACTS:
        raise ValueError(f"act must be one of {GSA_ACTS}, not {act!r}")
    return GSA_ACTS.index(act)

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/gla.h
_SIGS = {
    "gla_abi_version": (_I, []),
    "gla_status_str": (ctypes.c_char_p, [_I]),
    "gla_fwd_workspace_bytes": (_Z, [_I] * 7),
    "gla_fwd": (_I, [_P] * 7 + [_I] * 7 + [_P, _Z, _P]),
    "gla_bwd_workspace_bytes": (_Z, [_I] * 7),
    "gla_bwd": (_I, [_P] * 12 + [_I] * 7 + [_P, _Z, _P]),
    "gla_fwd_noalloc_max_workspace_bytes": (_Z, []),
    "gla_fwd_noalloc": (_I, [_P] * 7 + [_I] * 7 + [_P]),
    "gla_fwd_profiled": (_I, [_P] * 7 + [_I] * 7 + [_P, _Z, _P, _P, _I]),
    "gla_bwd_profiled": (_I, [_P] * 12 + [_I] * 7 + [_P, _Z, _P, _P, _I]),
    "gla_bwd_launch_count": (_I, [_I] * 7),
    "gla_fwd_launch_count": (_I, [_I] * 8),
    "gla_saved_bytes": (_Z, [_I] * 7),
    "gla_bwd_saved_workspace_bytes": (_Z, [_I] * 7),
    "gla_fwd_save": (_I, [_P] * 7 + [_I] * 7 + [_P, _Z, _P, _P, _I]),
    "gla_bwd_saved": (_I, [_P] * 12 + [_I] * 7 + [_P, _Z, _P, _Z, _P, _P, _I]),
    "gla_decode_step": (_I, [_P] * 6 + [_I] * 5 + [_P]),
    "gsa_fwd_workspace_bytes": (_Z, [_I] * 8),
    "gsa_fwd": (_I, [_P] * 9 + [_I] * 9 + [_P, _Z, _P]),
    "gsa_bwd_workspace_bytes": (_Z, [_I] * 8),
    "gsa_bwd": (_I, [_P] * 15 + [_I] * 9 + [_P, _Z, _P]),
    "gsa_saved_bytes": (_Z, [_I] * 8),
    "gsa_bwd_saved_workspace_bytes": (_Z, [_I] * 8),
    "gsa_fwd_save": (_I, [_P] * 9 + [_I] * 9 + [_P, _Z, _P]),
    "gsa_bwd_saved": (_I, [_P] * 15 + [_I] * 9 + [_P, _Z, _P, _Z, _P]),
    "gsa_decode_step": (_I, [_P] * 7 + [_I] * 7 + [_P]),
    "msgla_fwd_workspace_bytes": (_Z, [_I] * 8 + [_P, _P]),
    "msgla_fwd": (_I, [_P] * 8 + [_I] * 8 + [_P, _P, _P, _Z, _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None


class GlaError(RuntimeError):
    """A non-zero gla_status returned by the library."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libgla_amd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(
                f"{lib_path} is missing: build it with `python -m linear_recurrent_sequence_gla_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != 0:
        raise GlaError(status, lib().gla_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _common(q, k, v, g, gate_width=None):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-d tensor [B,H,L,Dk]")
    if q.dtype not in _DT:
        raise TypeError("q, k, v, g must be torch.bfloat16 or torch.float32")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a HIP (cuda) device")
    B, H, L, Dk = q.shape
    Dv = v.shape[-1] if isinstance(v, torch.Tensor) else -1
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, H, L, Dk), dt, dev)
    _need(k, "k", (B, H, L, Dk), dt, dev)
    _need(v, "v", (B, H, L, Dv), dt, dev)
    _need(g, "g", (B, H, L, Dk if gate_width is None else g.shape[-1]), dt, dev)
    return B, H, L, Dk, Dv, dev, dt


def _workspace(nbytes: int, dev, workspace):
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace must be a tensor on {dev} of at least {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)


def gla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, dtype) -> int:
    return int(lib().gla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dtype]))


def gla_bwd_workspace_bytes(B, H, L, Dk, Dv, C, dtype) -> int:
    return int(lib().gla_bwd_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dtype]))


def gla_saved_bytes(B, H, L, Dk, Dv, C, dtype) -> int:
    return int(lib().gla_saved_bytes(B, H, L, Dk, Dv, C, _DT[dtype]))


def gla_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, C, dtype) -> int:
    return int(lib().gla_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dtype]))


def gsa_fwd_workspace_bytes(B, H, L, Dk, Dv, m, C, dtype) -> int:
    return int(lib().gsa_fwd_workspace_bytes(B, H, L, Dk, Dv, m, C, _DT[dtype]))


def gsa_bwd_workspace_bytes(B, H, L, Dk, Dv, m, C, dtype) -> int:
    return int(lib().gsa_bwd_workspace_bytes(B, H, L, Dk, Dv, m, C, _DT[dtype]))


def gla_fwd(q, k, v, g, C: int = 64, h0=None, output_final_state: bool = True, *,
            out=None, ht_out=None, workspace=None):
    """Chunkwise GLA forward.  Returns (o, ht) with ht None unless output_final_state."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, L, Dv), dtype=dt, device=dev)
    _need(o, "out", (B, H, L, Dv), dt, dev)
    ht = None
    if output_final_state:
        ht = ht_out if ht_out is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        _need(ht, "ht_out", (B, H, Dk, Dv), torch.float32, dev)
    L_ = lib()
    nbytes = L_.gla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gla_fwd(None, None, None, None, None, None, None, B, H, L, Dk, Dv, C, _DT[dt], None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    _check(L_.gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(o), _ptr(ht),
                      B, H, L, Dk, Dv, C, _DT[dt], _ptr(ws), ws.numel(), _stream(dev)))
    return o, ht


def gla_fwd_noalloc(q, k, v, g, C: int = 64, h0=None, output_final_state: bool = True, *,
                    out=None, ht_out=None):
    """gla_fwd whose scratch is the library's fixed per-device buffer: no workspace is
    allocated by the library (pass out / ht_out to allocate nothing here either).  Sizes whose
    forward workspace exceeds gla_fwd_noalloc_max_workspace_bytes() raise (GLA_ERR_SCRATCH)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, L, Dv), dtype=dt, device=dev)
    _need(o, "out", (B, H, L, Dv), dt, dev)
    ht = None
    if output_final_state:
        ht = ht_out if ht_out is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        _need(ht, "ht_out", (B, H, Dk, Dv), torch.float32, dev)
    _check(lib().gla_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(o), _ptr(ht),
                                 B, H, L, Dk, Dv, C, _DT[dt], _stream(dev)))
    return o, ht


def gla_bwd(q, k, v, g, do, C: int = 64, h0=None, dht=None, want_dh0: bool = False, *,
            workspace=None, outs=None):
    """Gradients of sum(o*do) + sum(ht*dht).  Returns (dq, dk, dv, dg, dh0-or-None)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g)
    _need(do, "do", (B, H, L, Dv), dt, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if dht is not None:
        _need(dht, "dht", (B, H, Dk, Dv), torch.float32, dev)
    if outs is None:
        dq = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dk = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dv = torch.empty((B, H, L, Dv), dtype=dt, device=dev)
        dg = torch.empty((B, H, L, Dk), dtype=torch.float32, device=dev)
        dh0 = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if want_dh0 else None
    else:
        dq, dk, dv, dg, dh0 = outs
    L_ = lib()
    nbytes = L_.gla_bwd_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gla_bwd(*([None] * 12), B, H, L, Dk, Dv, C, _DT[dt], None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    _check(L_.gla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(do), _ptr(dht),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dh0),
                      B, H, L, Dk, Dv, C, _DT[dt], _ptr(ws), ws.numel(), _stream(dev)))
    return dq, dk, dv, dg, dh0


def gla_fwd_save(q, k, v, g, C: int = 64, h0=None, output_final_state: bool = True, *,
                 out=None, ht_out=None, saved=None):
    """gla_fwd that also keeps the chunk operands and chunk-start states for gla_bwd_saved.
    Returns (o, ht, saved)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, L, Dv), dtype=dt, device=dev)
    _need(o, "out", (B, H, L, Dv), dt, dev)
    ht = None
    if output_final_state:
        ht = ht_out if ht_out is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        _need(ht, "ht_out", (B, H, Dk, Dv), torch.float32, dev)
    L_ = lib()
    nbytes = L_.gla_saved_bytes(B, H, L, Dk, Dv, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gla_fwd_save(*([None] * 7), B, H, L, Dk, Dv, C, _DT[dt], None, 0, None, None, 0))
    sv = _workspace(nbytes, dev, saved)
    _check(L_.gla_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(o), _ptr(ht),
                           B, H, L, Dk, Dv, C, _DT[dt], _ptr(sv), sv.numel(), _stream(dev), None, 0))
    return o, ht, sv


def gla_bwd_saved(q, k, v, g, do, saved, C: int = 64, h0=None, dht=None, want_dh0: bool = False, *,
                  workspace=None, outs=None):
    """gla_bwd reusing what gla_fwd_save left in `saved` for the same q, k, v, g, h0 and C."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g)
    _need(do, "do", (B, H, L, Dv), dt, dev)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if dht is not None:
        _need(dht, "dht", (B, H, Dk, Dv), torch.float32, dev)
    if outs is None:
        dq = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dk = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dv = torch.empty((B, H, L, Dv), dtype=dt, device=dev)
        dg = torch.empty((B, H, L, Dk), dtype=torch.float32, device=dev)
        dh0 = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if want_dh0 else None
    else:
        dq, dk, dv, dg, dh0 = outs
    L_ = lib()
    nbytes = L_.gla_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gla_bwd_saved(*([None] * 12), B, H, L, Dk, Dv, C, _DT[dt], None, 0, None, 0, None, None, 0))
    if not isinstance(saved, torch.Tensor) or saved.device != dev:
        raise ValueError(f"saved must be the tensor gla_fwd_save returned, on {dev}")
    ws = _workspace(nbytes, dev, workspace)
    _check(L_.gla_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(do), _ptr(dht),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dh0),
                            B, H, L, Dk, Dv, C, _DT[dt], _ptr(saved), saved.numel() * saved.element_size(),
                            _ptr(ws), ws.numel(), _stream(dev), None, 0))
    return dq, dk, dv, dg, dh0


def gla_decode_step(q, k, v, g, state, *, out=None):
    """One recurrent step: state <- Diag(exp g) state + k^T v (in place); returns o = q state.
    q, k, g [B,H,Dk]; v [B,H,Dv]; state [B,H,Dk,Dv] float32."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be [B,H,Dk]")
    if q.dtype not in _DT:
        raise TypeError("q, k, v, g must be torch.bfloat16 or torch.float32")
    B, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    Dv = v.shape[-1]
    for t, n, s in ((q, "q", (B, H, Dk)), (k, "k", (B, H, Dk)), (g, "g", (B, H, Dk)), (v, "v", (B, H, Dv))):
        _need(t, n, s, dt, dev)
    _need(state, "state", (B, H, Dk, Dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, Dv), dtype=dt, device=dev)
    _need(o, "out", (B, H, Dv), dt, dev)
    _check(lib().gla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state), _ptr(o),
                                 B, H, Dk, Dv, _DT[dt], _stream(dev)))
    return o


def gsa_decode_step(q, k, v, g, hk, hv, *, act: str = "softmax", out=None):
    """One GSA recurrent step: with a = exp(g), w = 1 - a per slot, hk <- hk Diag(a) + k^T w and
    hv <- Diag(a) hv + w^T v (in place); returns o = softmax(q hk) hv (or f(q hk) hv).
    q, k [B,H,Dk]; v [B,H,Dv]; g [B,H,m]; hk [B,H,Dk,m], hv [B,H,m,Dv] float32."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be [B,H,Dk]")
    if q.dtype not in _DT:
        raise TypeError("q, k, v, g must be torch.bfloat16 or torch.float32")
    B, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    Dv, m = v.shape[-1], g.shape[-1]
    for t, n, s in ((q, "q", (B, H, Dk)), (k, "k", (B, H, Dk)), (g, "g", (B, H, m)), (v, "v", (B, H, Dv))):
        _need(t, n, s, dt, dev)
    _need(hk, "hk", (B, H, Dk, m), torch.float32, dev)
    _need(hv, "hv", (B, H, m, Dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, Dv), dtype=dt, device=dev)
    _need(o, "out", (B, H, Dv), dt, dev)
    _check(lib().gsa_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(hk), _ptr(hv), _ptr(o),
                                 B, H, Dk, Dv, m, _DT[dt], _act(act), _stream(dev)))
    return o


def gsa_fwd(q, k, v, g, C: int = 64, hk0=None, hv0=None, output_final_state: bool = True, *,
            act: str = "softmax", workspace=None, out=None):
    """Gated slot attention forward; g [B,H,L,m].  Returns (o, hkt, hvt)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g, gate_width=True)
    m = g.shape[-1]
    if hk0 is not None:
        _need(hk0, "hk0", (B, H, Dk, m), torch.float32, dev)
    if hv0 is not None:
        _need(hv0, "hv0", (B, H, m, Dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, L, Dv), dtype=dt, device=dev)
    hkt = hvt = None
    if output_final_state:
        hkt = torch.empty((B, H, Dk, m), dtype=torch.float32, device=dev)
        hvt = torch.empty((B, H, m, Dv), dtype=torch.float32, device=dev)
    L_ = lib()
    nbytes = L_.gsa_fwd_workspace_bytes(B, H, L, Dk, Dv, m, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gsa_fwd(*([None] * 9), B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    _check(L_.gsa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(hk0), _ptr(hv0), _ptr(o), _ptr(hkt), _ptr(hvt),
                      B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), _ptr(ws), ws.numel(), _stream(dev)))
    return o, hkt, hvt


def gsa_bwd(q, k, v, g, do, C: int = 64, hk0=None, hv0=None, dhkt=None, dhvt=None,
            want_dh0: bool = False, *, act: str = "softmax", workspace=None, outs=None):
    """Gradients of sum(o*do) + sum(hkt*dhkt) + sum(hvt*dhvt).
    Returns (dq, dk, dv, dg, dhk0-or-None, dhv0-or-None)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g, gate_width=True)
    m = g.shape[-1]
    _need(do, "do", (B, H, L, Dv), dt, dev)
    for t, n, s in ((hk0, "hk0", (B, H, Dk, m)), (hv0, "hv0", (B, H, m, Dv)),
                    (dhkt, "dhkt", (B, H, Dk, m)), (dhvt, "dhvt", (B, H, m, Dv))):
        if t is not None:
            _need(t, n, s, torch.float32, dev)
    if outs is None:
        dq = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dk = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dv = torch.empty((B, H, L, Dv), dtype=dt, device=dev)
        dg = torch.empty((B, H, L, m), dtype=torch.float32, device=dev)
        dhk0 = torch.empty((B, H, Dk, m), dtype=torch.float32, device=dev) if want_dh0 else None
        dhv0 = torch.empty((B, H, m, Dv), dtype=torch.float32, device=dev) if want_dh0 else None
    else:
        dq, dk, dv, dg, dhk0, dhv0 = outs
    L_ = lib()
    nbytes = L_.gsa_bwd_workspace_bytes(B, H, L, Dk, Dv, m, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gsa_bwd(*([None] * 15), B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    _check(L_.gsa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(hk0), _ptr(hv0), _ptr(do), _ptr(dhkt), _ptr(dhvt),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dhk0), _ptr(dhv0),
                      B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), _ptr(ws), ws.numel(), _stream(dev)))
    return dq, dk, dv, dg, dhk0, dhv0


def gsa_saved_bytes(B, H, L, Dk, Dv, m, C, dtype) -> int:
    return int(lib().gsa_saved_bytes(B, H, L, Dk, Dv, m, C, _DT[dtype]))


def gsa_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, m, C, dtype) -> int:
    return int(lib().gsa_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, m, C, _DT[dtype]))


def gsa_fwd_save(q, k, v, g, C: int = 64, hk0=None, hv0=None, output_final_state: bool = True, *,
                 act: str = "softmax", saved=None, out=None):
    """gsa_fwd that also keeps the forward's intermediate tensors for gsa_bwd_saved.
    Returns (o, hkt, hvt, saved)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g, gate_width=True)
    m = g.shape[-1]
    if hk0 is not None:
        _need(hk0, "hk0", (B, H, Dk, m), torch.float32, dev)
    if hv0 is not None:
        _need(hv0, "hv0", (B, H, m, Dv), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, L, Dv), dtype=dt, device=dev)
    hkt = hvt = None
    if output_final_state:
        hkt = torch.empty((B, H, Dk, m), dtype=torch.float32, device=dev)
        hvt = torch.empty((B, H, m, Dv), dtype=torch.float32, device=dev)
    L_ = lib()
    nbytes = L_.gsa_saved_bytes(B, H, L, Dk, Dv, m, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gsa_fwd_save(*([None] * 9), B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), None, 0, None))
    sv = _workspace(nbytes, dev, saved)
    _check(L_.gsa_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(hk0), _ptr(hv0), _ptr(o), _ptr(hkt),
                           _ptr(hvt), B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), _ptr(sv), sv.numel(),
                           _stream(dev)))
    return o, hkt, hvt, sv


def gsa_bwd_saved(q, k, v, g, do, saved, C: int = 64, hk0=None, hv0=None, dhkt=None, dhvt=None,
                  want_dh0: bool = False, *, act: str = "softmax", workspace=None, outs=None):
    """gsa_bwd reusing what gsa_fwd_save left in `saved` for the same q, k, g, hk0, hv0, C and act.
    Returns (dq, dk, dv, dg, dhk0-or-None, dhv0-or-None)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g, gate_width=True)
    m = g.shape[-1]
    _need(do, "do", (B, H, L, Dv), dt, dev)
    for t, n, s in ((hk0, "hk0", (B, H, Dk, m)), (hv0, "hv0", (B, H, m, Dv)),
                    (dhkt, "dhkt", (B, H, Dk, m)), (dhvt, "dhvt", (B, H, m, Dv))):
        if t is not None:
            _need(t, n, s, torch.float32, dev)
    if outs is None:
        dq = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dk = torch.empty((B, H, L, Dk), dtype=dt, device=dev)
        dv = torch.empty((B, H, L, Dv), dtype=dt, device=dev)
        dg = torch.empty((B, H, L, m), dtype=torch.float32, device=dev)
        dhk0 = torch.empty((B, H, Dk, m), dtype=torch.float32, device=dev) if want_dh0 else None
        dhv0 = torch.empty((B, H, m, Dv), dtype=torch.float32, device=dev) if want_dh0 else None
    else:
        dq, dk, dv, dg, dhk0, dhv0 = outs
    L_ = lib()
    nbytes = L_.gsa_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, m, C, _DT[dt])
    if nbytes == 0:
        _check(L_.gsa_bwd_saved(*([None] * 15), B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), None, 0, None, 0,
                                None))
    if not isinstance(saved, torch.Tensor) or saved.device != dev:
        raise ValueError(f"saved must be the tensor gsa_fwd_save returned, on {dev}")
    ws = _workspace(nbytes, dev, workspace)
    _check(L_.gsa_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(hk0), _ptr(hv0), _ptr(do), _ptr(dhkt),
                            _ptr(dhvt), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dhk0), _ptr(dhv0),
                            B, H, L, Dk, Dv, m, C, _DT[dt], _act(act), _ptr(saved),
                            saved.numel() * saved.element_size(), _ptr(ws), ws.numel(), _stream(dev)))
    return dq, dk, dv, dg, dhk0, dhv0


def _groups(scales, heads):
    scales, heads = [int(x) for x in scales], [int(x) for x in heads]
    if len(scales) != len(heads):
        raise ValueError("scales and heads need one entry per head group")
    n = len(scales)
    return n, (ctypes.c_int * n)(*scales), (ctypes.c_int * n)(*heads)


def msgla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, dtype, scales, heads) -> int:
    n, sc, hd = _groups(scales, heads)
    return lib().msgla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dtype], n, sc, hd)


def msgla_fwd(q, k, v, g, scales, heads, w=None, C: int = 64, h0=None, output_final_state: bool = True, *,
              workspace=None, out=None):
    """Multi-scale GLA: head group i (heads[i] consecutive heads) runs GLA on its q, k, g, v
    average-pooled over blocks of scales[i] tokens; token t takes its group's pooled output of
    block (t+1)//s - 1 (zeros before the first block completes), times w[b, t, i].
    Returns (o [B,H,L,Dv], ht [B,H,Dk,Dv] or None)."""
    B, H, L, Dk, Dv, dev, dt = _common(q, k, v, g)
    n, sc, hd = _groups(scales, heads)
    if h0 is not None:
        _need(h0, "h0", (B, H, Dk, Dv), torch.float32, dev)
    if w is not None:
        _need(w, "w", (B, L, n), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, L, Dv), dtype=dt, device=dev)
    ht = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if output_final_state else None
    L_ = lib()
    nbytes = L_.msgla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, _DT[dt], n, sc, hd)
    if nbytes == 0:
        _check(L_.msgla_fwd(*([None] * 8), B, H, L, Dk, Dv, C, _DT[dt], n, sc, hd, None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    _check(L_.msgla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(w), _ptr(o), _ptr(ht),
                        B, H, L, Dk, Dv, C, _DT[dt], n, sc, hd, _ptr(ws), ws.numel(), _stream(dev)))
    return o, ht
