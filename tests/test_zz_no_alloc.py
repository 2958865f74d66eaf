"""gla_fwd_noalloc (the forward on the library's fixed scratch buffer) against gla_fwd, called
through the C ABI: two calls in a row, the second smaller than the first, each equal to
gla_fwd's outputs bit for bit (the same kernels on the same inputs) and to the fp64 oracle
within the bf16 bound; a third call with a segmented state walk; sizes beyond the buffer are
refused."""
import ctypes

import numpy as np
import pytest

import workloads as W
from oracle import gla_recurrent_fwd
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


def call_noalloc(lib, x, C, dt, h0):
    import torch
    q, k, v, g = (dev(x[n], dt) for n in ("q", "k", "v", "g"))
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    o = torch.full((B, H, L, Dv), float("nan"), dtype=q.dtype, device=q.device)
    ht = torch.full((B, H, Dk, Dv), float("nan"), dtype=torch.float32, device=q.device)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.gla_fwd_noalloc(P(q), P(k), P(v), P(g), P(h0), P(o), P(ht), B, H, L, Dk, Dv, C,
                             1 if dt == "bf16" else 0, stream)
    assert st == 0, lib.gla_status_str(st).decode()
    return (q, k, v, g), o, ht


# (B, H, L, Dk, Dv, C, dtype, h0): the first needs ~55 MB of the 64 MiB buffer, the second is
# smaller, the third takes the segmented state walk (few, long sequences)
CALLS = [(4, 4, 2048, 128, 256, 64, "bf16", True), (1, 2, 300, 64, 64, 64, "bf16", True),
         (1, 2, 2000, 64, 64, 64, "bf16", False)]


def test_noalloc_matches_gla_fwd(gla):
    import torch
    lib = gla.lib()
    assert lib.gla_fwd_workspace_bytes(*CALLS[0][:6], 1) <= lib.gla_fwd_noalloc_max_workspace_bytes()
    for i, (B, H, L, Dk, Dv, C, dt, with_h0) in enumerate(CALLS):
        w = W.GlaWorkload("noalloc", B, H, L, Dk, Dv, C, dt, 900 + i, h0=with_h0)
        x = W.gla_inputs(w, with_grad=False)
        h0 = dev(x["h0"])
        print(f"[noalloc call {i}] B={B} H={H} L={L} Dk={Dk} Dv={Dv} C={C} {dt} h0={with_h0}", flush=True)
        args, o, ht = call_noalloc(lib, x, C, dt, h0)
        o_ref, ht_ref = gla.gla_fwd(*args, C=C, h0=h0)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref), "gla_fwd_noalloc differs from gla_fwd"
        sel = (np.array([[0]]), np.array([[H - 1]]))
        ro, rh = gla_recurrent_fwd(*(x[n][sel] for n in ("q", "k", "v", "g")), None if x["h0"] is None else x["h0"][sel])
        assert_close("o", host(o)[sel], ro, dt)
        assert_close("ht", host(ht)[sel], rh, dt)


def test_noalloc_refuses_oversized(gla):
    """The 340M-layer batch needs more than the buffer: refused before anything is enqueued,
    outputs untouched."""
    import torch
    lib = gla.lib()
    w = W.WORKLOADS["gla_340m"]
    q, k, g = (torch.zeros(w.B, w.H, w.L, w.Dk, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    v, o = (torch.zeros(w.B, w.H, w.L, w.Dv, dtype=torch.bfloat16, device="cuda") for _ in range(2))
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.gla_fwd_noalloc(P(q), P(k), P(v), P(g), None, P(o), None, w.B, w.H, w.L, w.Dk, w.Dv, w.C, 1, None)
    torch.cuda.synchronize()
    assert st == 8, lib.gla_status_str(st).decode()
    assert not torch.any(o)
