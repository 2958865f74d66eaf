"""A sweep of pseudo-random supported shapes through the GLA forward and backward (C ABI)
against the fp64 oracle.

The shapes come from a fixed generator: batch and head counts, sequence lengths with ragged
last chunks, key and value widths (multiples of 16), chunk sizes, dtypes, and present or
absent initial states and state gradients.  Between them they reach the walks' three tile
heights, the segmented forward walk (few sequences with many chunks), padded key widths and
value tiles, and both chunk-kernel forms.  Each case is sized so that the oracle finishes in
about a second."""
import numpy as np
import pytest

import workloads as W
from oracle import gla_recurrent_bwd, gla_recurrent_fwd
from tests.helpers import assert_close, dev, host

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, H = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 5]))
        Dk = int(rng.choice([16, 32, 48, 64, 96, 128, 160, 256]))
        Dv = int(rng.choice([16, 48, 64, 80, 128, 192, 256, 512]))
        C = int(rng.choice([16, 32, 64, 128]))
        dt = "f32" if rng.random() < 0.2 else "bf16"
        # lengths from one token to ~40 chunks, with ragged last chunks
        u = rng.random()
        L = 1 if u < 0.1 else int(rng.integers(2, 200)) if u < 0.5 else int(rng.integers(200, 40 * C + 1))
        if B * H * L * Dk * Dv > 6e7:              # keep the oracle to about a second
            continue
        out.append((B, H, L, Dk, Dv, C, dt, bool(rng.random() < 0.6), bool(rng.random() < 0.6), len(out)))
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def gla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_gla_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:7])))
def test_random_shape(gla, case):
    B, H, L, Dk, Dv, C, dt, h0, dht, i = case
    print(f"[sweep {i}] B={B} H={H} L={L} Dk={Dk} Dv={Dv} C={C} {dt} h0={h0} dht={dht}", flush=True)
    import torch
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    zeros = lambda d: torch.zeros(B, H, L, d, dtype=tdt, device="cuda")
    if gla.gla_fwd_workspace_bytes(B, H, L, Dk, Dv, C, tdt) == 0:
        # outside the tiles a CU's LDS holds: the library must refuse, not run
        with pytest.raises(gla.GlaError):
            gla.gla_fwd(zeros(Dk), zeros(Dk), zeros(Dv), zeros(Dk), C=C)
        return                                # refused, as it must be
    w = W.GlaWorkload(f"sweep{i}", B, H, L, Dk, Dv, C, dt, 3000 + i, h0=h0, gate_law="iid")
    x = W.gla_inputs(w)
    q, k, v, g = (dev(x[n], dt) for n in ("q", "k", "v", "g"))
    o, ht = gla.gla_fwd(q, k, v, g, C=C, h0=dev(x["h0"]))
    ro, rht = gla_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["h0"])
    assert_close("o", host(o), ro, dt)
    assert_close("ht", host(ht), rht, dt)
    if gla.gla_bwd_workspace_bytes(B, H, L, Dk, Dv, C, tdt) == 0:
        with pytest.raises(gla.GlaError):
            gla.gla_bwd(q, k, v, g, zeros(Dv), C=C)
        return
    outs = gla.gla_bwd(q, k, v, g, dev(x["do"], dt), C=C, h0=dev(x["h0"]), dht=dev(x["dht"]) if dht else None,
                       want_dh0=True)
    ref = gla_recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["do"], x["h0"], x["dht"] if dht else None)
    for name, got in zip(("dq", "dk", "dv", "dg", "dh0"), outs):
        assert_close(name, host(got), ref[name], dt)
