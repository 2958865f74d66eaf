"""A sweep of pseudo-random supported GSA shapes through the forward and the backward, both
the recomputing entry points and the saved-activation path, against the fp64 oracle.

The shapes come from a fixed generator: batch and head counts, sequence lengths with ragged
last chunks, key and value widths, slot counts m (multiples of 16 up to 64), chunk sizes,
dtypes, read-outs, and present or absent initial memories and memory gradients; a second set
draws 80 to 128 slots, where some shapes support the forward only.  Each case
is sized so that the oracle finishes in about a second.  ReLU's derivative jumps at z = 0 and
the two sides compute z in different precision, so a ReLU case compares its backward only when
every score clears a margin (test_gsa_gpu.py checks the ReLU backward on inputs built for one)."""
import numpy as np
import pytest

import workloads as W
from oracle import gsa_recurrent_bwd, gsa_recurrent_fwd
from tests.helpers import assert_close, dev, host
from tests.test_gsa_gpu import slot_scores

pytestmark = pytest.mark.gpu

ACTS = ("softmax", "swish", "relu", "relu2", "none")


def _cases(n=16, seed=2028, ms=(16, 32, 48, 64)):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, H = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3]))
        Dk = int(rng.choice([16, 32, 64, 96, 128, 256]))
        Dv = int(rng.choice([16, 48, 64, 128, 256, 512]))
        m = int(rng.choice(list(ms)))
        C = int(rng.choice([16, 32, 64]))
        dt = "f32" if rng.random() < 0.2 else "bf16"
        u = rng.random()
        L = 1 if u < 0.1 else int(rng.integers(2, 120)) if u < 0.5 else int(rng.integers(120, 20 * C + 1))
        if B * H * L * (Dk + Dv) * m > 4e7:
            continue
        act = ACTS[int(rng.integers(0, len(ACTS)))]
        out.append((B, H, L, Dk, Dv, m, C, dt, act, bool(rng.random() < 0.6), bool(rng.random() < 0.6),
                    bool(rng.random() < 0.5), len(out)))
    return out


# slot counts up to 64, then beyond 64 (where C = 64 runs the forward only)
CASES = _cases() + [c[:-1] + (16 + c[-1],) for c in _cases(n=8, seed=2029, ms=(80, 96, 112, 128))]


@pytest.fixture(scope="module")
def gla():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_gla_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:9])))
def test_random_gsa_shape(gla, case):
    import torch
    B, H, L, Dk, Dv, m, C, dt, act, h0, dht, saved, i = case
    print(f"[gsa sweep {i}] B={B} H={H} L={L} Dk={Dk} Dv={Dv} m={m} C={C} {dt} act={act} h0={h0} dht={dht} "
          f"saved={saved}", flush=True)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    fwd_only = False
    if gla.gsa_bwd_workspace_bytes(B, H, L, Dk, Dv, m, C, tdt) == 0:
        z = lambda d: torch.zeros(B, H, L, d, dtype=tdt, device="cuda")
        with pytest.raises(gla.GlaError):
            gla.gsa_bwd(z(Dk), z(Dk), z(Dv), z(m), z(Dv), C=C)
        if gla.gsa_fwd_workspace_bytes(B, H, L, Dk, Dv, m, C, tdt) == 0:
            with pytest.raises(gla.GlaError):
                gla.gsa_fwd(z(Dk), z(Dk), z(Dv), z(m), C=C)
            return                            # refused, as it must be
        fwd_only, saved = True, False         # the forward alone is supported
    w = W.GsaWorkload(f"gsweep{i}", B, H, L, Dk, Dv, m, C, dt, 4000 + i, h0=h0)
    x = W.gsa_inputs(w)
    args = [dev(x[n], dt) for n in ("q", "k", "v", "g")]
    st = dict(C=C, hk0=dev(x["hk0"]), hv0=dev(x["hv0"]), act=act)
    if saved:
        o, hkt, hvt, sv = gla.gsa_fwd_save(*args, **st)
    else:
        o, hkt, hvt = gla.gsa_fwd(*args, **st)
    ro, rhk, rhv = gsa_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["hk0"], x["hv0"], act=act)
    assert_close("o", host(o), ro, dt)
    assert_close("hkt", host(hkt), rhk, dt)
    assert_close("hvt", host(hvt), rhv, dt)
    if fwd_only:
        return
    if act == "relu":
        margin = float(np.min(np.abs(slot_scores(x["q"], x["k"], x["g"], x["hk0"]))))
        print(f"  min |z| = {margin:.2e}", flush=True)
        if margin < 0.05:
            return
    dk_ = dict(dhkt=dev(x["dhkt"]) if dht else None, dhvt=dev(x["dhvt"]) if dht else None, want_dh0=True)
    do = dev(x["do"], dt)
    outs = gla.gsa_bwd_saved(*args, do, sv, **st, **dk_) if saved else gla.gsa_bwd(*args, do, **st, **dk_)
    rb = gsa_recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["do"], x["hk0"], x["hv0"],
                           x["dhkt"] if dht else None, x["dhvt"] if dht else None, act=act)
    for name, got in zip(("dq", "dk", "dv", "dg", "dhk0", "dhv0"), outs):
        assert_close(name, host(got), rb[name], dt)
