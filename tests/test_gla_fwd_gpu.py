"""GPU parity of the GLA forward and decode (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import gla_decode_step as ref_decode
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


def run_fwd(gla, x, C, dtype, want_ht=True):
    o, ht = gla.gla_fwd(dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype), dev(x["g"], dtype),
                        C=C, h0=dev(x["h0"]), output_final_state=want_ht)
    return host(o), (host(ht) if ht is not None else None)


def check_fwd(gla, w, x, units=None):
    o, ht = run_fwd(gla, x, w.C, w.dtype)
    sel = (slice(None), slice(None)) if units is None else units
    h0 = None if x["h0"] is None else x["h0"][sel]
    ro, rh = gla_recurrent_fwd(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], h0)
    print(f"[{w.name}] B={w.B} H={w.H} L={x['q'].shape[2]} Dk={w.Dk} Dv={w.Dv} C={w.C} {w.dtype}", flush=True)
    assert_close("o", o[sel], ro, w.dtype)
    assert_close("ht", ht[sel], rh, w.dtype)


def test_tiny_fp32_config(gla):
    """The tiny fp32 workload: B=1, H=1, L=64, Dk=Dv=16, C=16, zero initial state."""
    w = W.WORKLOADS["tiny_f32"]
    check_fwd(gla, w, W.gla_inputs(w, with_grad=False))


SHAPES = [
    # (B, H, L, Dk, Dv, C, dtype, h0)
    (2, 2, 150, 64, 64, 64, "bf16", True),
    (1, 3, 200, 128, 256, 64, "bf16", False),
    (2, 1, 77, 16, 48, 16, "bf16", True),
    (1, 2, 130, 32, 80, 32, "bf16", True),
    (1, 2, 300, 128, 128, 128, "bf16", True),
    (1, 1, 129, 256, 512, 64, "bf16", True),
    (2, 4, 130, 256, 512, 64, "bf16", True),     # walk grid fills every CU at 64-row tiles
    (4, 4, 150, 128, 256, 64, "bf16", True),     # ... at 32-row tiles (smaller shapes: 16-row)
    (1, 1, 100, 256, 64, 32, "bf16", False),
    (1, 2, 1, 128, 64, 64, "bf16", True),       # single token
    (1, 2, 64, 128, 64, 64, "bf16", True),      # exactly one chunk
    (2, 2, 90, 48, 32, 16, "f32", True),
    (1, 2, 70, 128, 96, 64, "f32", True),
    (1, 1, 140, 64, 64, 64, "f32", False),
    (1, 1, 66, 256, 32, 32, "f32", True),
    (1, 2, 300, 64, 80, 128, "f32", True),      # fp32 with C=128: forward only
    # few sequences, many chunks: the state walk runs in parallel segments (4, 5 ragged, 2)
    (1, 2, 2000, 64, 64, 64, "bf16", True),
    (1, 1, 1500, 128, 96, 32, "bf16", True),
    (1, 2, 1100, 64, 80, 64, "f32", True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(gla, shape):
    B, H, L, Dk, Dv, C, dt, h0 = shape
    w = W.GlaWorkload("sweep", B, H, L, Dk, Dv, C, dt, 77 + L + Dk, h0=h0, gate_law="iid")
    check_fwd(gla, w, W.gla_inputs(w, with_grad=False))


# Enough sequences that the 32-column tiles give each CU of a 256-CU device a workgroup: the
# walk and the outputs run as one kernel, which keeps no states for gla_fwd
FUSED_SHAPES = [
    # (B, H, L, Dk, Dv, C, dtype, h0)
    (64, 4, 100, 128, 32, 64, "bf16", True),     # ragged last chunk
    (32, 4, 200, 112, 64, 64, "bf16", False),    # padded key rows, no initial state
    (64, 4, 150, 80, 32, 64, "bf16", True),      # 48 padded key rows
    (16, 4, 129, 128, 128, 64, "bf16", True),    # last chunk of one row (odd chunk count)
    (64, 4, 64, 128, 32, 64, "bf16", True),      # one chunk
    (64, 4, 1, 128, 32, 64, "bf16", True),       # one token
    (64, 4, 128, 128, 32, 64, "bf16", True),     # two chunks
]


@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_walk_output_shapes(gla, shape):
    B, H, L, Dk, Dv, C, dt, h0 = shape
    w = W.GlaWorkload("fused", B, H, L, Dk, Dv, C, dt, 91 + L + Dk, h0=h0, gate_law="iid")
    check_fwd(gla, w, W.gla_inputs(w, with_grad=False))


def test_fused_launch_count(gla):
    """gla_fwd_launch_count reports the fused walk-output kernel exactly where 32-column tiles
    give every compute unit a workgroup (and 64-column multiples when the states are kept)."""
    import torch
    lib = gla.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B, H, Dv, keep in ((8, 4, 256, 1), (8, 4, 256, 0), (64, 4, 32, 0), (64, 4, 32, 1), (1, 2, 256, 0)):
        fused = B * H * Dv // 32 >= cus and Dv % (64 if keep else 32) == 0
        assert lib.gla_fwd_launch_count(B, H, 2048, 128, Dv, 64, 1, keep) == (2 if fused else 3), (B, H, Dv, keep)
    assert lib.gla_fwd_launch_count(64, 4, 2048, 128, 256, 64, 0, 0) == 3      # fp32: never fused


def test_fused_profiled_events(gla):
    """gla_fwd_profiled on a fused shape: the same outputs as gla_fwd, and its events bracket
    the preparation and the fused kernel, with nothing between events[2] and events[3]."""
    import ctypes
    import torch
    lib = gla.lib()
    B, H, L, Dk, Dv, C = 64, 4, 100, 128, 32, 64
    if lib.gla_fwd_launch_count(B, H, L, Dk, Dv, C, 1, 0) != 2:
        pytest.skip("the fused walk-output kernel does not apply on this device")
    w = W.GlaWorkload("fused-ev", B, H, L, Dk, Dv, C, "bf16", 95, h0=True, gate_law="iid")
    x = W.gla_inputs(w, with_grad=False)
    q, k, v, g = (dev(x[n], "bf16") for n in ("q", "k", "v", "g"))
    h0 = dev(x["h0"])
    o_ref, ht_ref = gla.gla_fwd(q, k, v, g, C=C, h0=h0)
    o, ht = torch.empty_like(o_ref), torch.empty_like(ht_ref)
    ws = torch.empty(lib.gla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, 1), dtype=torch.uint8, device="cuda")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * 4)(*[e.cuda_event for e in evs])
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.gla_fwd_profiled(P(q), P(k), P(v), P(g), P(h0), P(o), P(ht), B, H, L, Dk, Dv, C, 1, P(ws), ws.numel(),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), handles, 4)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
    t = [evs[i].elapsed_time(evs[i + 1]) for i in range(3)]
    print(f"  prep {t[0] * 1e3:.1f} us, walk+out {t[1] * 1e3:.1f} us, after {t[2] * 1e3:.1f} us", flush=True)
    assert t[0] > 0 and t[1] > 0 and t[2] * 1e3 < 10.0      # nothing runs between events[2] and [3]


@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_chunk_size_independence(gla, C):
    """Same inputs, every chunk size: each result matches the oracle (and so each other)."""
    w = W.GlaWorkload("chunks", 1, 2, 333, 128, 64, C, "bf16", 5, h0=True)
    check_fwd(gla, w, W.gla_inputs(w, with_grad=False))


@pytest.mark.parametrize("gval", [0.0, -30.0, -3.0])
def test_extreme_gates(gla, gval):
    """g = 0 (ungated), g = -30 (memoryless; exercises the sub-chunked safe path), g = -3."""
    w = W.GlaWorkload("gates", 1, 2, 150, 64, 64, 64, "bf16", 9, h0=True)
    x = W.gla_inputs(w, with_grad=False)
    x["g"] = np.full_like(x["g"], gval)
    check_fwd(gla, w, x)


def test_mixed_safe_and_fast_chunks(gla):
    """Some chunks far beyond the span limit, others not, in one call."""
    w = W.GlaWorkload("mixed", 1, 2, 256, 64, 64, 64, "bf16", 10, h0=True)
    x = W.gla_inputs(w, with_grad=False)
    x["g"][:, :, 64:128] = -2.0
    x["g"][:, 1, 200:210, :7] = -40.0
    check_fwd(gla, w, x)


@pytest.mark.parametrize("C", [32, 64])
def test_mixed_safe_and_fast_chunks_wide_keys(gla, C):
    """As above with 256-channel keys, whose preparation kernel runs 512 threads (persistent at
    C = 64, one chunk per workgroup at C = 32), on both intra-chunk paths."""
    w = W.GlaWorkload("mixed-wide", 1, 2, 256, 256, 64, C, "bf16", 12, h0=True)
    x = W.gla_inputs(w, with_grad=False)
    x["g"][:, :, 64:128] = -2.0
    x["g"][:, 1, 200:210, :7] = -40.0
    check_fwd(gla, w, x)


def test_large_negative_gate_is_finite(gla):
    w = W.GlaWorkload("neg", 1, 1, 100, 32, 32, 32, "bf16", 11, h0=True)
    x = W.gla_inputs(w, with_grad=False)
    x["g"][:] = -1e4
    check_fwd(gla, w, x)


@pytest.mark.parametrize("name,units", [
    ("gla_340m", (np.array([0, 7]), np.array([0, 3]))),
    ("gla_1p3b", (np.array([2]), np.array([1]))),
    ("gla_long", (np.array([0]), np.array([2]))),
])
def test_full_size_configs_sampled(gla, name, units):
    """Full-size workloads, launched exactly as the benchmark does; the oracle checks sampled
    (batch, head) units (units are independent, so this is exact for those outputs)."""
    w = W.WORKLOADS[name]
    x = W.gla_inputs(w, with_grad=False)
    b, h = units
    check_fwd(gla, w, x, units=(b[:, None], h[None, :]))


@pytest.mark.parametrize("shape", [(1, 2, 2000, 64, 64, 64), (1, 4, 3000, 128, 256, 64)])
def test_segmented_walk_matches_plain_walk(gla, shape):
    """gla_fwd splits the state walk of few, long sequences into segments and adds the carried
    states afterwards; gla_fwd_save never splits.  Outputs and final states agree to rounding
    (the fixed-up states are rounded to bf16 twice)."""
    import torch
    B, H, L, Dk, Dv, C = shape
    w = W.GlaWorkload("seg", B, H, L, Dk, Dv, C, "bf16", 77, h0=True)
    x = W.gla_inputs(w, with_grad=False)
    q, k, v, g = (dev(x[n], "bf16") for n in ("q", "k", "v", "g"))
    h0 = dev(x["h0"])
    o1, ht1 = gla.gla_fwd(q, k, v, g, C=C, h0=h0)
    o2, ht2, _ = gla.gla_fwd_save(q, k, v, g, C=C, h0=h0)
    torch.cuda.synchronize()
    for name, a, b in (("o", o1, o2), ("ht", ht1, ht2)):
        a, b = host(a), host(b)
        e = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)
        print(f"  {name}: max|segmented - plain| / max|plain| = {e:.2e}", flush=True)
        assert e <= 1e-2, name


def test_deterministic(gla):
    import torch
    w = W.GlaWorkload("det", 2, 2, 500, 128, 256, 64, "bf16", 12, h0=True)
    x = W.gla_inputs(w, with_grad=False)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "g")]
    o1, h1 = gla.gla_fwd(*args, C=64, h0=dev(x["h0"]))
    o2, h2 = gla.gla_fwd(*args, C=64, h0=dev(x["h0"]))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_state_chaining(gla):
    """fwd over [0, L) equals fwd over [0, L1) then [L1, L) from the carried state, L1 unaligned."""
    w = W.GlaWorkload("chain", 1, 2, 300, 64, 64, 64, "bf16", 13, h0=True)
    x = W.gla_inputs(w, with_grad=False)
    L1 = 101
    full_o, full_h = run_fwd(gla, x, 64, "bf16")
    a = {n: (x[n][:, :, :L1] if n in "qkvg" else x[n]) for n in ("q", "k", "v", "g", "h0")}
    o1, h1 = run_fwd(gla, a, 64, "bf16")
    b = {n: x[n][:, :, L1:] for n in ("q", "k", "v", "g")}
    b["h0"] = h1.astype(np.float32)
    o2, h2 = run_fwd(gla, b, 64, "bf16")
    ro, rh = gla_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["h0"])
    assert_close("o chained", np.concatenate([o1, o2], axis=2), ro, "bf16")
    assert_close("ht chained", h2, rh, "bf16")


def test_decode_matches_oracle_and_forward(gla):
    """Decode steps: each step's output and the final state match the oracle's steps, and the
    T-step result equals the forward over the same T tokens."""
    import torch
    w = W.WORKLOADS["decode"]
    T = 40
    d = W.decode_inputs(w, T=T, B=8)
    state = dev(d["state"])
    S = d["state"].astype(np.float64)
    outs = []
    for t in range(T):
        o = gla.gla_decode_step(dev(d["q"][t], "bf16"), dev(d["k"][t], "bf16"), dev(d["v"][t], "bf16"),
                                dev(d["g"][t], "bf16"), state)
        ro, S = ref_decode(d["q"][t], d["k"][t], d["v"][t], d["g"][t], S)
        outs.append(host(o))
        assert_close(f"o[{t}]", host(o), ro, "bf16")
    assert_close("state", host(state), S, "bf16")
    # decode == forward over the same tokens (the forward sees [B,H,T,D])
    perm = lambda a: np.ascontiguousarray(np.transpose(a, (1, 2, 0, 3)))
    fo, fh = gla.gla_fwd(dev(perm(d["q"]), "bf16"), dev(perm(d["k"]), "bf16"), dev(perm(d["v"]), "bf16"),
                         dev(perm(d["g"]), "bf16"), C=16, h0=dev(d["state"]))
    torch.cuda.synchronize()
    assert_close("decode vs fwd o", np.stack(outs, axis=2), host(fo), "bf16")
    assert_close("decode vs fwd state", host(state), host(fh), "bf16")


def test_decode_full_size_sampled(gla):
    """The decode workload's full batch (64 x 4, Dk=128, Dv=256), a few steps, all units."""
    w = W.WORKLOADS["decode"]
    d = W.decode_inputs(w, T=3)
    state = dev(d["state"])
    S = d["state"].astype(np.float64)
    for t in range(3):
        o = gla.gla_decode_step(dev(d["q"][t], "bf16"), dev(d["k"][t], "bf16"), dev(d["v"][t], "bf16"),
                                dev(d["g"][t], "bf16"), state)
        ro, S = ref_decode(d["q"][t], d["k"][t], d["v"][t], d["g"][t], S)
        assert_close(f"o[{t}]", host(o), ro, "bf16")
    assert_close("state", host(state), S, "bf16")


def test_decode_fp32(gla):
    w = W.DecodeWorkload("dec32", 5, 2, 3, 48, 32, "f32", 21)
    d = W.decode_inputs(w)
    state = dev(d["state"])
    S = d["state"].astype(np.float64)
    for t in range(w.T):
        o = gla.gla_decode_step(dev(d["q"][t]), dev(d["k"][t]), dev(d["v"][t]), dev(d["g"][t]), state)
        ro, S = ref_decode(d["q"][t], d["k"][t], d["v"][t], d["g"][t], S)
        assert_close(f"o[{t}]", host(o), ro, "f32")
    assert_close("state", host(state), S, "f32")
