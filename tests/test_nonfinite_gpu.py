"""Non-finite inputs propagate to exactly the outputs that depend on them.

One NaN or +Inf is planted in q or in g of one (batch row, head) unit at one token and key
channel.  The fp64 oracle, run on the same inputs, marks which outputs depend on it (IEEE
arithmetic carries the NaN or Inf along every path that uses the value).

* Forward: the GPU's non-finite entries of o and ht are exactly the oracle's (for q: the
  token's output row; for g: every later output row and the channel's row of the final state).
* Backward: every entry the oracle marks is non-finite on the GPU too, and nothing outside the
  unit is.  Inside the unit the chunked form may mark more: masked score entries are zeros
  that the matrix cores multiply with the planted value (0 * NaN = NaN), where the
  token-by-token recurrence never forms that product.  For q, dq never depends on q and stays
  finite everywhere.
* Every other unit, and every entry finite on both sides, matches the oracle at the usual bound.
"""
import numpy as np
import pytest

import workloads as W
from oracle import gla_recurrent_bwd, gla_recurrent_fwd
from tests.helpers import TOL, dev, host

pytestmark = pytest.mark.gpu

B, H, L, DK, DV, C = 2, 2, 200, 64, 64, 64
UNIT = (1, 0)           # the (batch row, head) that holds the planted value
TOKEN, CHANNEL = 70, 5  # in the second chunk


@pytest.fixture(scope="module")
def gla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_gla_amd as m
    m.lib()
    return m


def planted(tensor, value):
    w = W.GlaWorkload("nonfinite", B, H, L, DK, DV, C, "bf16", 808, h0=True, gate_law="iid")
    x = W.gla_inputs(w)
    x[tensor] = x[tensor].copy()
    x[tensor][UNIT[0], UNIT[1], TOKEN, CHANNEL] = value
    return x


def oracle_fwd(x):
    with np.errstate(invalid="ignore", over="ignore"):
        return gla_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["h0"])


def oracle_bwd(x):
    with np.errstate(invalid="ignore", over="ignore"):
        return gla_recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["do"], x["h0"], x["dht"])


def compare_finite(name, got, ref, mask):
    """max |got - ref| / max |ref| over the entries in mask (finite on both sides)."""
    if not np.any(mask):
        return
    d = np.abs(got[mask] - ref[mask])
    scale = np.max(np.abs(ref[mask]))
    e = float(np.max(d) / scale) if d.size else 0.0
    print(f"  {name}: rel err on finite entries {e:.3e}", flush=True)
    assert e <= TOL["bf16"], name


def other_units(a):
    """Every (batch row, head) unit but the planted one."""
    keep = np.ones(a.shape[:2], dtype=bool)
    keep[UNIT] = False
    return a[keep]


@pytest.mark.parametrize("tensor,value", [("q", np.nan), ("q", np.inf), ("g", np.nan), ("g", np.inf)])
def test_forward_marks_exactly_the_dependent_outputs(gla, tensor, value):
    x = planted(tensor, value)
    o, ht = gla.gla_fwd(*(dev(x[n], "bf16") for n in ("q", "k", "v", "g")), C=C, h0=dev(x["h0"]))
    o, ht = host(o), host(ht)
    ro, rht = oracle_fwd(x)
    print(f"[nonfinite fwd] {tensor}={value}: oracle marks {np.sum(~np.isfinite(ro))} o and "
          f"{np.sum(~np.isfinite(rht))} ht entries", flush=True)
    assert np.sum(~np.isfinite(ro)) > 0
    for name, got, ref in (("o", o, ro), ("ht", ht, rht)):
        assert np.array_equal(~np.isfinite(got), ~np.isfinite(ref)), f"{name}: non-finite entries differ"
        compare_finite(name, got, ref, np.isfinite(ref))
    if tensor == "q":   # the token's output row only
        bad = np.argwhere(~np.isfinite(ro))
        assert set(map(tuple, bad[:, :3])) == {(UNIT[0], UNIT[1], TOKEN)}


@pytest.mark.parametrize("tensor", ["q", "g"])
def test_backward_propagates_within_the_unit(gla, tensor):
    x = planted(tensor, np.nan)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "g", "do")]
    grads = gla.gla_bwd(*args, C=C, h0=dev(x["h0"]), dht=dev(x["dht"]), want_dh0=True)
    ref = oracle_bwd(x)
    for name, t in zip(("dq", "dk", "dv", "dg", "dh0"), grads):
        got, r = host(t), ref[name]
        gbad, rbad = ~np.isfinite(got), ~np.isfinite(r)
        print(f"[nonfinite bwd] {tensor}=nan {name}: oracle {int(rbad.sum())}, gpu {int(gbad.sum())} "
              "non-finite", flush=True)
        assert np.all(gbad[rbad]), f"{name}: an entry that depends on the planted value is finite"
        assert not np.any(other_units(gbad)), f"{name}: non-finite outside the planted unit"
        if tensor == "q" and name == "dq":
            assert not np.any(gbad)
        compare_finite(name, got, r, ~gbad & ~rbad)
        compare_finite(name + " (other units)", other_units(got), other_units(r),
                       np.ones(other_units(r).shape, dtype=bool))
