"""GPU parity of the GLA backward (through the C ABI) against the fp64 oracle's reverse sweep."""
import numpy as np
import pytest

import workloads as W
from oracle import gla_recurrent_bwd
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


def run_bwd(gla, x, C, dtype, with_dht=True, want_dh0=True):
    dt = dtype
    outs = gla.gla_bwd(dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt), dev(x["g"], dt), dev(x["do"], dt),
                       C=C, h0=dev(x["h0"]), dht=dev(x["dht"]) if with_dht else None, want_dh0=want_dh0)
    return [None if t is None else host(t) for t in outs]


def check_bwd(gla, w, x, units=None, with_dht=True):
    dq, dk, dv, dg, dh0 = run_bwd(gla, x, w.C, w.dtype, with_dht)
    sel = (slice(None), slice(None)) if units is None else units
    h0 = None if x["h0"] is None else x["h0"][sel]
    dht = x["dht"][sel] if with_dht else None
    ref = gla_recurrent_bwd(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], x["do"][sel], h0, dht)
    print(f"[{w.name}] B={w.B} H={w.H} L={x['q'].shape[2]} Dk={w.Dk} Dv={w.Dv} C={w.C} {w.dtype} "
          f"h0={x['h0'] is not None} dht={with_dht}", flush=True)
    assert_close("dq", dq[sel], ref["dq"], w.dtype)
    assert_close("dk", dk[sel], ref["dk"], w.dtype)
    assert_close("dv", dv[sel], ref["dv"], w.dtype)
    assert_close("dg", dg[sel], ref["dg"], w.dtype)
    assert_close("dh0", dh0[sel], ref["dh0"], w.dtype)


def test_tiny_fp32_config(gla):
    w = W.WORKLOADS["tiny_f32"]
    check_bwd(gla, w, W.gla_inputs(w))


SHAPES = [
    # (B, H, L, Dk, Dv, C, dtype, h0, dht)
    (2, 2, 150, 64, 64, 64, "bf16", True, True),
    (1, 3, 200, 128, 256, 64, "bf16", False, False),
    (2, 1, 77, 16, 48, 16, "bf16", True, True),
    (1, 2, 130, 32, 80, 32, "bf16", True, True),
    (1, 2, 300, 128, 128, 128, "bf16", True, True),
    (1, 1, 129, 256, 512, 64, "bf16", True, True),
    (2, 4, 130, 256, 512, 64, "bf16", True, True),   # 64-row walk tiles
    (4, 4, 150, 128, 256, 64, "bf16", True, True),   # 32-row walk tiles
    (1, 1, 100, 256, 64, 32, "bf16", False, True),
    (1, 2, 1, 128, 64, 64, "bf16", True, True),
    (1, 2, 64, 128, 64, 64, "bf16", True, False),
    (1, 1, 200, 64, 96, 128, "bf16", True, True),
    (2, 2, 90, 48, 32, 16, "f32", True, True),
    (1, 2, 70, 128, 96, 64, "f32", True, True),
    (1, 1, 140, 64, 64, 64, "f32", False, True),
    # chunk sizes whose tiles exceed a CU's LDS: the call runs at a smaller chunk (same result)
    (1, 2, 300, 256, 64, 128, "bf16", True, True),    # at C = 64
    (1, 2, 200, 64, 48, 128, "f32", True, True),      # the fp32 backward at C = 64
    (1, 1, 150, 256, 32, 64, "f32", True, True),      # fp32 with 256-channel keys at C = 32
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(gla, shape):
    B, H, L, Dk, Dv, C, dt, h0, dht = shape
    w = W.GlaWorkload("sweep", B, H, L, Dk, Dv, C, dt, 177 + L + Dk, h0=h0, gate_law="iid")
    check_bwd(gla, w, W.gla_inputs(w), with_dht=dht)


@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_chunk_size_independence(gla, C):
    w = W.GlaWorkload("chunks", 1, 2, 333, 128, 64, C, "bf16", 5, h0=True)
    check_bwd(gla, w, W.gla_inputs(w))


@pytest.mark.parametrize("gval", [0.0, -30.0, -3.0])
def test_extreme_gates(gla, gval):
    """g = 0, g = -30 and g = -3 (the last two take the exact intra-chunk path)."""
    w = W.GlaWorkload("gates", 1, 2, 150, 64, 64, 64, "bf16", 9, h0=True)
    x = W.gla_inputs(w)
    x["g"] = np.full_like(x["g"], gval)
    check_bwd(gla, w, x)


def test_mixed_safe_and_fast_chunks(gla):
    w = W.GlaWorkload("mixed", 1, 2, 256, 64, 64, 64, "bf16", 10, h0=True)
    x = W.gla_inputs(w)
    x["g"][:, :, 64:128] = -2.0
    x["g"][:, 1, 200:210, :7] = -40.0
    check_bwd(gla, w, x)


def test_mixed_safe_and_fast_chunks_wide_keys(gla):
    """256-channel keys (512-thread preparation, split key width in the chunk kernel, separate
    dv kernel) with chunks on both intra-chunk paths."""
    w = W.GlaWorkload("mixed-wide", 1, 2, 256, 256, 64, 64, "bf16", 13, h0=True)
    x = W.gla_inputs(w)
    x["g"][:, :, 64:128] = -2.0
    x["g"][:, 1, 200:210, :7] = -40.0
    check_bwd(gla, w, x)


@pytest.mark.parametrize("name,units,dht", [
    ("gla_340m", (np.array([0, 7]), np.array([1, 2])), False),
    ("gla_340m", (np.array([3]), np.array([0])), True),
    ("gla_1p3b", (np.array([1]), np.array([3])), True),
])
def test_full_size_configs_sampled(gla, name, units, dht):
    """Full-size workloads as the benchmark launches them; the oracle checks sampled units."""
    w = W.WORKLOADS[name]
    x = W.gla_inputs(w)
    b, h = units
    check_bwd(gla, w, x, units=(b[:, None], h[None, :]), with_dht=dht)


@pytest.mark.parametrize("shape", [
    # (B, H, L, Dk, Dv): just over 256 chunk tiles, a ragged last chunk
    (3, 3, 1850, 128, 64),      # 261 tiles of the whole-width kernel
    (2, 5, 1700, 64, 128),      # 270 tiles of the Dk = 64 kernel
], ids=lambda s: "x".join(map(str, s)))
def test_workgroups_with_several_tiles(gla, shape):
    """The chunk-gradient kernel's grid is persistent, one workgroup per CU: with more tiles
    than workgroups, some workgroups run a second tile, whose q, k and g they loaded during the
    first tile's epilogue, and the rest stop after one.  Every output is checked."""
    B, H, L, Dk, Dv = shape
    w = W.GlaWorkload(f"multi-tile-{Dk}", B, H, L, Dk, Dv, 64, "bf16", 77 + Dk, h0=True, gate_law="iid")
    check_bwd(gla, w, W.gla_inputs(w))


def test_deterministic(gla):
    import torch
    w = W.GlaWorkload("det", 2, 2, 500, 128, 256, 64, "bf16", 12, h0=True)
    x = W.gla_inputs(w)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "g", "do")]
    a = gla.gla_bwd(*args, C=64, h0=dev(x["h0"]), dht=dev(x["dht"]), want_dh0=True)
    b = gla.gla_bwd(*args, C=64, h0=dev(x["h0"]), dht=dev(x["dht"]), want_dh0=True)
    torch.cuda.synchronize()
    assert all(torch.equal(s, t) for s, t in zip(a, b))
