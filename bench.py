#!/usr/bin/env python3
"""Benchmark of the chunkwise GLA operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
    python bench.py --only {gla_1p3b,decode,gsa_decode,gsa,gsa_m128,msgla,long_fwd} [--steps K] [--warmup W]
        (one extra workload alone)

One step is one pass of the training hot path over one batch of the 340M-layer workload
(B=8, H=4, L=2048, Dk=128, Dv=256, chunk C=64, bf16 inputs, fp32 accumulation): the forward
(gla_fwd_save: chunk preparation + state walk, keeping the chunk operands and chunk-start
states) then the backward (gla_bwd_saved: reverse state walk + chunk gradients) on inputs
already resident in HBM, outputs and buffers preallocated.  The timed region is exactly K
steps between two device synchronisations; per-kernel durations come from HIP events the
library records at its own kernel boundaries on the same stream.

Prints ONE JSON line: tokens/s (B*L per step; mean over the timed region, with the median and
minimum of the per-step event durations beside it), % of bf16 MFMA peak at the algorithmic
flop count, the roofline of the dominant kernel, the fp64 oracle timed on this host's cores
on a bounded sample, and extra measurements of the other paths (the 1.3B-layer fwd+bwd, the
decode steps with their state in HBM and in the Infinity Cache, the long-sequence forward,
gated slot attention, multi-scale GLA).  Inputs are synthetic and seeded (see workloads/).

Helper mode (summaries of rocprofv3 output, written under profiles/):
    python bench.py --summarize-stats <kernel_stats.csv> --title T --cmd C --out F
    python bench.py --summarize-pmc <counter_collection.csv> --kernel K --calib-bytes N ...
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402  (seeded input generators; no operator arithmetic)

PEAK_BF16_FLOPS = 2516.6e12          # 256 CU x 2.4 GHz x 4096 flop/clk (dense bf16 MFMA)
PEAK_HBM_BYTES = 8.0e12              # HBM3E
WORKLOAD = "gla_340m"
METRIC = "GLA fwd+bwd tokens/s and % bf16 MFMA peak at H=4 Dk=128 Dv=256 L=2048"
CSRC = os.path.join(ROOT, "linear_recurrent_sequence_gla_amd", "csrc")
PMC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


# ----------------------------------------------------------------------------- accounting
def algorithmic(B, H, L, Dk, Dv, C, s=2, saved=True, h0=False):
    """Algorithmic flops and bytes of one forward and one backward (per token-head figures,
    times B*H*L token-heads).  Flops: the causal intra-chunk block incl. the diagonal, the
    inter-chunk output and the state update (forward); three times the intra work on the key
    side, twice on the value side, plus 2 Dk Dv each for the reverse state pass and the three
    inter-chunk gradient products (dq, dk, dv) for the backward, and 2 Dk Dv more when the
    backward recomputes the forward states (saved=False).  Bytes: each operator input and
    output once (q, k, g, v read, o written; + do read, dq, dk, dv written, dg written in
    fp32), plus 4 Dk Dv per (b,h) for each state read or written (ht always; h0 read by both
    passes when given)."""
    u = B * H * L
    ff = (C + 1) * (Dk + Dv) + 4 * Dk * Dv
    fb = 3 * (C + 1) * Dk + 2 * (C + 1) * Dv + (8 if saved else 10) * Dk * Dv
    bf = s * (3 * Dk + 2 * Dv)
    bb = s * (3 * Dk + 2 * Dv) + s * (2 * Dk + Dv) + 4 * Dk
    st = 4 * Dk * Dv * B * H
    return {"flops_fwd": u * ff, "flops_bwd": u * fb, "bytes_fwd": u * bf + st * (1 + h0),
            "bytes_bwd": u * bb + st * h0, "units": u}


def gsa_algorithmic(B, H, L, Dk, Dv, m, C, s=2):
    """GSA forward and backward as its two GLA passes: pass 1 with keys k (Dk) and values w
    (m), pass 2 with keys w (m) and values v (Dv), each counted with the GLA figures above
    (saved-activation backward); the read-out between them is O(m) per token and left out.
    Bytes: q, k, v, g read and o written (forward); q, k, v, g, do read, dq, dk, dv written,
    dg written in fp32 (backward)."""
    u = B * H * L
    fwd = lambda a, b: (C + 1) * (a + b) + 4 * a * b
    bwd = lambda a, b: 3 * (C + 1) * a + 2 * (C + 1) * b + 8 * a * b
    return {"flops_fwd": u * (fwd(Dk, m) + fwd(m, Dv)), "flops_bwd": u * (bwd(Dk, m) + bwd(m, Dv)),
            "bytes_fwd": u * s * (2 * Dk + m + 2 * Dv),
            "bytes_bwd": u * (s * (2 * Dk + m + 2 * Dv) + s * (2 * Dk + Dv) + 4 * m), "units": u}


def kernel_alg_bytes(B, H, L, Dk, Dv, s=2):
    """Per-launch algorithmic bytes of each kernel: the operator tensors it reads or writes,
    each counted once (per token-head figure x B*H*L).  Workspace traffic is design overhead
    and is not counted here (it shows up in the measured HBM traffic)."""
    u = B * H * L
    return {
        "fwd.prep": u * s * 3 * Dk,                            # q, k, g
        "fwd.walk": u * s * Dv,                                # v (states are workspace)
        "fwd.out": u * s * 2 * Dv,                             # v in, o out
        "fwd.walk_out": u * s * 2 * Dv,                        # v in, o out (walk and outputs fused)
        "bwd.prep": u * s * 3 * Dk,                            # q, k, g (self-contained backward)
        "bwd.walk_fwd": u * s * Dv,                            # v
        "bwd.walk_rev": u * s * Dv,                            # do
        "bwd.chunk": u * (s * (3 * Dk + 2 * Dv) + s * (2 * Dk + Dv) + 4 * Dk),  # all but h0/dh0
        "bwd.dv": u * s * 2 * Dv,                              # do in, dv out
    }


def csrc_hash():
    """Hash of the device-code sources (every kernel source; the host-only C-ABI layer in
    api.hip does not change what the counters measure)."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if os.path.basename(f) == "api.hip":
            continue
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- CPU baseline
def _oracle_unit(args):
    """fwd + bwd of the fp64 oracle on one (batch row, head) unit at full length."""
    q, k, v, g, do = args
    from oracle import gla_recurrent_bwd, gla_recurrent_fwd
    t0 = time.perf_counter()
    gla_recurrent_fwd(q, k, v, g)
    gla_recurrent_bwd(q, k, v, g, do)
    return time.perf_counter() - t0


def cpu_baseline(x, B, H, L, max_workers=16):
    """The oracle as it stands, on this host's cores: one task per (batch row, head) unit of
    the same 340M-shape batch, as many worker processes as the process may run on (its CPU
    affinity set, at most max_workers), one BLAS/OpenMP thread each.  Returns tokens/s of
    that batch."""
    import multiprocessing as mp
    workers = max(1, min(max_workers, B * H, len(os.sched_getaffinity(0))))
    units = [tuple(x[n][b:b + 1, h:h + 1] for n in ("q", "k", "v", "g", "do")) for b in range(B) for h in range(H)]
    saved = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for v in saved:
        os.environ[v] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            pool.map(_oracle_unit, units[:workers])          # warm the workers (imports)
            t0 = time.perf_counter()
            per = pool.map(_oracle_unit, units, chunksize=1)
            wall = time.perf_counter() - t0
    finally:
        for v, val in saved.items():
            if val is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = val
    return {"value": B * L / wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"the full 340M-shape batch (B={B}, H={H}, L={L}) fwd+bwd, {B * H} (batch row, head) "
                      f"units as tasks over {workers} worker processes (the CPU affinity set), fp64 NumPy, "
                      f"wall {wall:.1f} s, {float(np.sum(per)):.1f} s of CPU work "
                      f"(one unit on one core: {float(np.median(per)):.2f} s)"}


# ----------------------------------------------------------------------------- GPU legs
def _events(torch, n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()                                           # created on first record
    return evs


def _handles(evs):
    import ctypes
    arr = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    return arr


def _stats(vals_ms):
    """mean / median / min of a list of durations in ms, in us."""
    v = np.asarray(vals_ms, dtype=np.float64) * 1e3
    return {"mean": round(float(np.mean(v)), 2), "median": round(float(np.median(v)), 2),
            "min": round(float(np.min(v)), 2)}


def run_gla(torch, m, steps, warmup, name=WORKLOAD):
    """Training steps (gla_fwd_save then gla_bwd_saved) on one GLA workload.  Three timed
    passes over the same `steps` steps: the mean step time with nothing recorded between the
    steps (the headline: an event at each kernel boundary costs about 2.5 us of the stream's
    time, some 20 us per step); each step's duration, from an event before and after it; and
    each kernel's duration, from the HIP events the library records at its kernel boundaries
    on the launch stream."""
    import ctypes
    w = W.WORKLOADS[name]
    B, H, L, Dk, Dv, C = w.B, w.H, w.L, w.Dk, w.Dv, w.C
    x = W.gla_inputs(w)
    dt = torch.bfloat16
    # three resident copies of the inputs, used in rotation, so that a step's inputs are not
    # still in the 256 MB Infinity Cache from the step before
    d0 = {n: torch.from_numpy(x[n]).to("cuda", dt).contiguous() for n in ("q", "k", "v", "g", "do")}
    sets = [d0] + [{n: t.clone() for n, t in d0.items()} for _ in range(2)]
    h0 = torch.from_numpy(x["h0"]).cuda() if x["h0"] is not None else None
    o = torch.empty(B, H, L, Dv, device="cuda", dtype=dt)
    ht = torch.empty(B, H, Dk, Dv, device="cuda", dtype=torch.float32)
    dq = torch.empty(B, H, L, Dk, device="cuda", dtype=dt)
    dk = torch.empty_like(dq)
    dv = torch.empty(B, H, L, Dv, device="cuda", dtype=dt)
    dg = torch.empty(B, H, L, Dk, device="cuda", dtype=torch.float32)
    lib = m.lib()
    sv = torch.empty(lib.gla_saved_bytes(B, H, L, Dk, Dv, C, 1), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(lib.gla_bwd_saved_workspace_bytes(B, H, L, Dk, Dv, C, 1), dtype=torch.uint8, device="cuda")
    nb = lib.gla_bwd_launch_count(B, H, L, Dk, Dv, C, 1) - 2      # the saved backward skips two
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step(evf=None, evb=None, k=0):
        d = sets[k % len(sets)]
        m._check(lib.gla_fwd_save(P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(h0), P(o), P(ht),
                                  B, H, L, Dk, Dv, C, 1, P(sv), sv.numel(), stream, evf, 4 if evf else 0))
        m._check(lib.gla_bwd_saved(P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(h0), P(d["do"]), None,
                                   P(dq), P(dk), P(dv), P(dg), None, B, H, L, Dk, Dv, C, 1, P(sv), sv.numel(),
                                   P(wsb), wsb.numel(), stream, evb, 4 if evb else 0))

    for k in range(warmup):
        step(k=k)
    ms, step_ms = _timed_steps(torch, lambda k: step(k=k), steps, 0, indexed=True)
    ef = [_events(torch, 4) for _ in range(steps)]
    eb = [_events(torch, 4) for _ in range(steps)]                 # room for the most launches
    hf = [_handles(e) for e in ef]
    hb = [_handles(e) for e in eb]
    torch.cuda.synchronize()
    for k in range(steps):
        step(hf[k], hb[k], k)
    torch.cuda.synchronize()
    # the state walk and the chunk outputs run as one kernel where gla_fwd_launch_count says 2
    fused = lib.gla_fwd_launch_count(B, H, L, Dk, Dv, C, 1, 1) == 2
    names_f = ["fwd.prep", "fwd.walk_out"] if fused else ["fwd.prep", "fwd.walk", "fwd.out"]
    names_b = ["bwd.walk_rev", "bwd.chunk", "bwd.dv"][:nb]
    kt = {}
    for i, nme in enumerate(names_f):
        kt[nme] = [ef[k][i].elapsed_time(ef[k][i + 1]) for k in range(steps)]
    for i, nme in enumerate(names_b):
        kt[nme] = [eb[k][i].elapsed_time(eb[k][i + 1]) for k in range(steps)]
    return {"w": w, "x": x, "ms": ms, "step_ms": step_ms, "kernel_ms": kt}


def gla_summary(r):
    """Throughput, algorithmic TFLOP/s, % of the bf16 MFMA peak and the roofline of the
    dominant kernel for one run_gla result."""
    w = r["w"]
    B, H, L, Dk, Dv, C = w.B, w.H, w.L, w.Dk, w.Dv, w.C
    alg = algorithmic(B, H, L, Dk, Dv, C, saved=True, h0=w.h0)
    ms = r["ms"]
    tflops = (alg["flops_fwd"] + alg["flops_bwd"]) / (ms * 1e-3) / 1e12
    kmean = {k: float(np.mean(v)) for k, v in r["kernel_ms"].items()}
    dom = max(kmean, key=kmean.get)
    kb = kernel_alg_bytes(B, H, L, Dk, Dv)[dom]
    achieved = kb / (kmean[dom] * 1e-3) / 1e9
    return {
        "tokens_per_s": round(B * L / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(float(np.median(r["step_ms"])), 4),
        "ms_per_step_min": round(float(np.min(r["step_ms"])), 4),
        "tflops": round(tflops, 3),
        "pct_bf16_mfma_peak": round(100 * tflops * 1e12 / PEAK_BF16_FLOPS, 3),
        "pct_hbm_roofline_step": round(100 * (alg["bytes_fwd"] + alg["bytes_bwd"]) / (ms * 1e-3) / PEAK_HBM_BYTES, 3),
        "kernel_us": {k: _stats(v) for k, v in r["kernel_ms"].items()},
        "dominant": dom,
        "roofline": {"kernel": KERNEL_SYMBOLS[dom] + f" ({dom})", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                     "frac": round(achieved / (PEAK_HBM_BYTES / 1e9), 4),
                     "alg_bytes": kb, "avg_us": round(kmean[dom] * 1e3, 2)},
    }


def time_decode_chain(torch, run_all, states, T):
    """Times T decode steps (run_all launches them, updating `states` in place) two ways: launched
    one by one from Python, and captured once in a HIP graph and replayed, as a serving loop would
    run them.  The replay's states and outputs must equal the one-by-one launches bit for bit.
    Returns (us per step replayed, us per step launched one by one)."""
    init = [t.clone() for t in states]

    def reset():
        for t, t0 in zip(states, init):
            t.copy_(t0)

    outs = run_all()                                          # warm
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    run_all()
    e.record()
    torch.cuda.synchronize()
    us_eager = s.elapsed_time(e) * 1e3 / T
    reset()
    outs = run_all()
    torch.cuda.synchronize()
    ref = [t.clone() for t in list(states) + list(outs)]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            outs = run_all()
    torch.cuda.current_stream().wait_stream(cap)
    reset()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(list(states) + list(outs), ref)):
        raise RuntimeError("graph replay of the decode steps differs from launching them one by one")
    g.replay()                                                # warm
    torch.cuda.synchronize()
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) * 1e3 / T, us_eager


def decode_line(workload, T, nbytes, cold, warm, sets, state_mb):
    """cold: (us, us_eager) with the steps rotating over `sets` state copies (more bytes than the
    256 MB Infinity Cache, so each step's state comes from HBM); warm: the same steps on one
    state, which stays in the Infinity Cache."""
    us, us_eager = cold
    wus, _ = warm
    return {"workload": f"{workload}, {T} steps replayed as one HIP graph (bitwise equal to launching "
                        "them one by one)",
            "us_per_step": round(us, 3), "GBps": round(nbytes / us / 1e3, 1),
            "frac_hbm": round(nbytes / us / 1e3 / (PEAK_HBM_BYTES / 1e9), 4),
            "state_sets": sets,
            "note": f"steps rotate over {sets} copies of the {state_mb:.1f} MB state ({sets * state_mb:.0f} MB, more "
                    "than the 256 MB Infinity Cache), so every step reads and writes its state in HBM",
            "us_per_step_launched_one_by_one": round(us_eager, 3),
            "cache_resident": {"us_per_step": round(wus, 3), "GBps": round(nbytes / wus / 1e3, 1),
                               "note": "all steps on one state, which stays in the Infinity Cache: "
                                       "not an HBM figure"}}


def run_decode(torch, m, T=None, sets=12):
    """GLA decode steps on the decode workload (B=64, H=4, Dk=128, Dv=256), fp32 state updated in
    place; all of the workload's steps, rotating over `sets` states (cold) and on one (warm)."""
    w = W.WORKLOADS["decode"]
    T = w.T if T is None else T
    dd = W.decode_inputs(w, T=T)
    dt = torch.bfloat16
    qs, ks, vs, gs = (torch.from_numpy(dd[n]).to("cuda", dt) for n in ("q", "k", "v", "g"))
    st0 = torch.from_numpy(dd["state"]).to("cuda")
    o = torch.empty(w.B, w.H, w.Dv, device="cuda", dtype=dt)

    def chain(states):
        def run_all():
            for t in range(T):
                m.gla_decode_step(qs[t], ks[t], vs[t], gs[t], states[t % len(states)], out=o)
            return [o]
        return time_decode_chain(torch, run_all, states, T)

    cold = chain([st0.clone() for _ in range(sets)])
    warm = chain([st0.clone()])
    BH = w.B * w.H
    nbytes = BH * (2 * w.Dk * w.Dv * 4 + 2 * (3 * w.Dk + 2 * w.Dv))   # state in+out, q k g v o
    return decode_line(f"decode B={w.B} H={w.H} Dk={w.Dk} Dv={w.Dv} fp32 state", T, nbytes, cold, warm, sets,
                       BH * w.Dk * w.Dv * 4 / 1e6)


def run_gsa_decode(torch, m, T=None, sets=24):
    """GSA decode steps on the GSA decode workload (B=64, H=4, Dk=Dv=128, m=64), both fp32 slot
    memories updated in place; all steps, rotating over `sets` memory pairs (cold) and on one."""
    w = W.WORKLOADS["gsa_decode"]
    T = w.T if T is None else T
    dd = W.gsa_decode_inputs(w, T=T)
    dt = torch.bfloat16
    qs, ks, vs, gs = (torch.from_numpy(dd[n]).to("cuda", dt) for n in ("q", "k", "v", "g"))
    hk0 = torch.from_numpy(dd["hk"]).to("cuda")
    hv0 = torch.from_numpy(dd["hv"]).to("cuda")
    o = torch.empty(w.B, w.H, w.Dv, device="cuda", dtype=dt)

    def chain(n):
        hks = [hk0.clone() for _ in range(n)]
        hvs = [hv0.clone() for _ in range(n)]

        def run_all():
            for t in range(T):
                m.gsa_decode_step(qs[t], ks[t], vs[t], gs[t], hks[t % n], hvs[t % n], out=o)
            return [o]
        return time_decode_chain(torch, run_all, hks + hvs, T)

    cold = chain(sets)
    warm = chain(1)
    BH = w.B * w.H
    state = (w.Dk * w.m + w.m * w.Dv) * 4
    nbytes = BH * (2 * state + 2 * (2 * w.Dk + w.m + 2 * w.Dv))     # memories in+out, q k g v o
    return decode_line(f"gsa decode B={w.B} H={w.H} Dk={w.Dk} Dv={w.Dv} m={w.m} fp32 memories", T, nbytes,
                       cold, warm, sets, BH * state / 1e6)


def _timed_steps(torch, fn, steps, warmup, indexed=False):
    """The mean over one timed region of `steps` calls with nothing recorded between them, and
    each call's duration from a second pass with an event before and after every call (those
    events take stream time of their own, so they stay out of the mean).  With indexed, fn
    takes the call's index."""
    call = (lambda k: fn(k)) if indexed else (lambda k: fn())
    for k in range(warmup):
        call(k)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for k in range(steps):
        call(k)
    e.record()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k, (a, b) in enumerate(evs):
        a.record()
        call(k)
        b.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps, [a.elapsed_time(b) for a, b in evs]


def run_gsa(torch, m, steps=20, warmup=100, name="gsa_340m", read_outs=None):
    """GSA fwd+bwd at its workload: gsa_fwd_save then gsa_bwd_saved (the training-step form, as
    for GLA), with the recomputing gsa_fwd + gsa_bwd timed beside it, and (read_outs, by
    default for the 64-slot workload only) the same step with each element-wise read-out."""
    read_outs = (name == "gsa_340m") if read_outs is None else read_outs
    w = W.WORKLOADS[name]
    lib = m.lib()
    if lib.gsa_fwd_workspace_bytes(w.B, w.H, w.L, w.Dk, w.Dv, w.m, w.C, 1) == 0:
        return None
    x = W.gsa_inputs(w)
    dt = torch.bfloat16
    d = {n: torch.from_numpy(x[n]).to("cuda", dt).contiguous() for n in ("q", "k", "v", "g", "do")}
    args = (d["q"], d["k"], d["v"], d["g"])
    saved = torch.empty(m.gsa_saved_bytes(w.B, w.H, w.L, w.Dk, w.Dv, w.m, w.C, dt), dtype=torch.uint8,
                        device="cuda")
    ws = torch.empty(m.gsa_bwd_saved_workspace_bytes(w.B, w.H, w.L, w.Dk, w.Dv, w.m, w.C, dt),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty(w.B, w.H, w.L, w.Dv, device="cuda", dtype=dt)
    outs = (torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
            torch.empty(w.B, w.H, w.L, w.m, device="cuda"), None, None)

    def saved_step(act="softmax"):
        m.gsa_fwd_save(*args, C=w.C, output_final_state=False, act=act, saved=saved, out=o)
        m.gsa_bwd_saved(*args, d["do"], saved, C=w.C, act=act, workspace=ws, outs=outs)

    def recompute_step():
        m.gsa_fwd(*args, C=w.C)
        m.gsa_bwd(*args, d["do"], C=w.C)

    ms, per = _timed_steps(torch, saved_step, steps, warmup)
    ms_re, _ = _timed_steps(torch, recompute_step, steps, warmup)
    # the element-wise read-outs in place of the softmax (same saved-path step)
    acts = {a: round(_timed_steps(torch, lambda a=a: saved_step(a), steps, warmup)[0], 4)
            for a in m.GSA_ACTS if a != "softmax" and read_outs}
    alg = gsa_algorithmic(w.B, w.H, w.L, w.Dk, w.Dv, w.m, w.C)
    tflops = (alg["flops_fwd"] + alg["flops_bwd"]) / (ms * 1e-3) / 1e12
    nbytes = alg["bytes_fwd"] + alg["bytes_bwd"]
    return {"workload": f"gsa B={w.B} H={w.H} L={w.L} Dk={w.Dk} Dv={w.Dv} m={w.m} C={w.C} fwd+bwd "
                        "(gsa_fwd_save + gsa_bwd_saved)",
            "ms_per_step": round(ms, 4), "ms_per_step_median": round(float(np.median(per)), 4),
            "ms_per_step_min": round(float(np.min(per)), 4),
            "tokens_per_s": round(w.B * w.L / ms * 1e3, 1),
            "tflops": round(tflops, 3), "pct_bf16_mfma_peak": round(100 * tflops * 1e12 / PEAK_BF16_FLOPS, 3),
            "roofline_step": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 2),
                              "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                              "frac": round(nbytes / (ms * 1e-3) / PEAK_HBM_BYTES, 4), "alg_bytes": nbytes},
            "recomputing_ms_per_step": round(ms_re, 4), **({"read_out_ms_per_step": acts} if acts else {})}


def run_long_fwd(torch, m, steps=20, warmup=200):
    """The long-sequence forward (B=1, H=4, L=20480, Dk=128, Dv=256, C=64): few sequences, so
    the sequential state walk over 320 chunks sets the time."""
    import ctypes
    w = W.WORKLOADS["gla_long"]
    x = W.gla_inputs(w, with_grad=False)
    dt = torch.bfloat16
    d = {n: torch.from_numpy(x[n]).to("cuda", dt).contiguous() for n in ("q", "k", "v", "g")}
    lib = m.lib()
    ws = torch.empty(lib.gla_fwd_workspace_bytes(w.B, w.H, w.L, w.Dk, w.Dv, w.C, 1), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty(w.B, w.H, w.L, w.Dv, device="cuda", dtype=dt)
    ht = torch.empty(w.B, w.H, w.Dk, w.Dv, device="cuda", dtype=torch.float32)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    evs = [_events(torch, 4) for _ in range(steps)]
    hs = [_handles(e) for e in evs]

    def fwd(h=None):
        args = (P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), None, P(o), P(ht), w.B, w.H, w.L, w.Dk, w.Dv, w.C, 1,
                P(ws), ws.numel(), stream)
        m._check(lib.gla_fwd_profiled(*args, h, 4) if h else lib.gla_fwd(*args))

    ms, per = _timed_steps(torch, fwd, steps, warmup)   # no events recorded between kernels
    torch.cuda.synchronize()
    for k in range(steps):                              # each kernel's duration
        fwd(hs[k])
    torch.cuda.synchronize()
    fused = lib.gla_fwd_launch_count(w.B, w.H, w.L, w.Dk, w.Dv, w.C, 1, 0) == 2
    kt = {nme: [evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]
          for i, nme in enumerate(("prep", "walk_out") if fused else ("prep", "walk", "out"))}
    alg = algorithmic(w.B, w.H, w.L, w.Dk, w.Dv, w.C)
    tflops = alg["flops_fwd"] / (ms * 1e-3) / 1e12
    kmean = {k: float(np.mean(v)) for k, v in kt.items()}
    dom = max(kmean, key=kmean.get)
    u = w.B * w.H * w.L
    kbytes = {"prep": u * 2 * 3 * w.Dk, "walk": u * 2 * w.Dv + w.B * w.H * w.Dk * w.Dv * 4, "out": u * 2 * 2 * w.Dv,
              "walk_out": u * 2 * 2 * w.Dv + w.B * w.H * w.Dk * w.Dv * 4}
    ach = kbytes[dom] / (kmean[dom] * 1e-3) / 1e9
    return {"workload": f"gla_long forward B={w.B} H={w.H} L={w.L} Dk={w.Dk} Dv={w.Dv} C={w.C}, final state kept",
            "ms": round(ms, 4), "ms_median": round(float(np.median(per)), 4), "ms_min": round(float(np.min(per)), 4),
            "tokens_per_s": round(w.B * w.L / ms * 1e3, 1),
            "tflops": round(tflops, 3), "pct_bf16_mfma_peak": round(100 * tflops * 1e12 / PEAK_BF16_FLOPS, 3),
            "pct_hbm_roofline": round(100 * alg["bytes_fwd"] / (ms * 1e-3) / PEAK_HBM_BYTES, 3),
            "kernel_us": {k: _stats(v) for k, v in kt.items()},
            "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_BYTES / 1e9,
                         "unit": "GB/s", "frac": round(ach / (PEAK_HBM_BYTES / 1e9), 4), "alg_bytes": kbytes[dom]}}


def run_msgla(torch, m, steps=20, warmup=200):
    """MS-GLA {1, 2, 4} forward on the 340M-layer shape, head budget split 2/1/1, with fusion
    weights; plain gla_fwd on the same inputs is timed beside it."""
    w = W.WORKLOADS["gla_340m"]
    x = W.gla_inputs(w, with_grad=False)
    dt = torch.bfloat16
    d = {n: torch.from_numpy(x[n]).to("cuda", dt).contiguous() for n in ("q", "k", "v", "g")}
    wts = torch.full((w.B, w.L, 3), 1.0 / 3.0, device="cuda")
    scales, heads = [1, 2, 4], [2, 1, 1]
    ws = torch.empty(m.msgla_fwd_workspace_bytes(w.B, w.H, w.L, w.Dk, w.Dv, w.C, dt, scales, heads),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty(w.B, w.H, w.L, w.Dv, device="cuda", dtype=dt)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    ms = timed(lambda: m.msgla_fwd(d["q"], d["k"], d["v"], d["g"], scales, heads, wts, C=w.C,
                                   output_final_state=False, workspace=ws, out=o))
    ws2 = torch.empty(m.gla_fwd_workspace_bytes(w.B, w.H, w.L, w.Dk, w.Dv, w.C, dt), dtype=torch.uint8,
                      device="cuda")
    ms_gla = timed(lambda: m.gla_fwd(d["q"], d["k"], d["v"], d["g"], C=w.C, output_final_state=False, out=o,
                                     workspace=ws2))
    return {"workload": f"ms-gla scales (1,2,4) heads (2,1,1) B={w.B} H={w.H} L={w.L} Dk={w.Dk} Dv={w.Dv} "
                        f"C={w.C} forward",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.L / ms * 1e3, 1),
            "gla_fwd_ms_same_inputs": round(ms_gla, 4)}


# ----------------------------------------------------------------------------- summaries
def summarize_stats(path, title, cmd, out):
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Name"].startswith("_ZN3gla")]
    lines = [f"# {title}", "", "Command:", "", "```", cmd, "```", "",
             "The library's kernels only (the run's host-to-device input copies are left out); % is of "
             "the whole run's kernel time.", "",
             "| kernel | calls | avg (us) | total (us) | % |", "|---|---|---|---|---|"]
    for r in rows:
        nm = r["Name"]
        short = nm.split("(")[0]
        if len(short) > 70:
            short = short[:70] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def summarize_pmc(paths, kernel_sub, calib_sub, calib_bytes, cmd, out_json, out_md):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the kernels whose name contains kernel_sub,
    scaled by what the same counters read for a copy kernel of known size (calib_sub)."""
    import csv
    vals, every = {}, {}
    for p in paths:
        for r in csv.DictReader(open(p)):
            name, ctr, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            key = "kernel" if kernel_sub in name else ("calib" if calib_sub in name else None)
            if key:
                vals.setdefault((key, ctr), []).append(v)
            if name.startswith("_ZN3gla"):
                every.setdefault(name, {}).setdefault(ctr, []).append(v)
    res = {}
    for ctr, label in (("FETCH_SIZE", "read"), ("WRITE_SIZE", "write")):
        kk = vals.get(("kernel", ctr))
        cc = vals.get(("calib", ctr))
        if not kk or not cc:
            continue
        # the calibration copy is the run's largest copy dispatch (the others upload inputs)
        factor = calib_bytes / (np.max(cc) * 1024.0)          # known bytes / counted bytes
        res[label] = {"kib_per_dispatch": float(np.median(kk)), "calib_kib": float(np.max(cc)),
                      "scale": float(factor), "bytes": float(np.median(kk) * 1024.0 * factor)}
    summary = {"kernel": kernel_sub, "csrc_hash": csrc_hash(), "command": cmd, **res}
    if "read" in res and "write" in res:
        summary["traffic_bytes"] = res["read"]["bytes"] + res["write"]["bytes"]
    json.dump(summary, open(out_json, "w"), indent=1)
    lines = [f"# HBM traffic of `{kernel_sub}` (rocprofv3 counters)", "", "Commands:", "", "```", cmd, "```", "",
             f"Copy calibration: a plain device copy of {calib_bytes / 1e6:.1f} MB read + write.", "",
             "| counter | KiB/dispatch | copy KiB | scale | bytes/dispatch |", "|---|---|---|---|---|"]
    for label, r in res.items():
        lines.append(f"| {label} | {r['kib_per_dispatch']:.0f} | {r['calib_kib']:.0f} | {r['scale']:.3f} | "
                     f"{r['bytes'] / 1e6:.1f} MB |")
    if "read" in res and "write" in res:
        lines += ["", "Every kernel of the library in the same runs (scaled the same way):", "",
                  "| kernel | read MB | write MB |", "|---|---|---|"]
        for name, c in every.items():
            if "FETCH_SIZE" in c and "WRITE_SIZE" in c:
                rd = np.median(c["FETCH_SIZE"]) * 1024.0 * res["read"]["scale"] / 1e6
                wr = np.median(c["WRITE_SIZE"]) * 1024.0 * res["write"]["scale"] / 1e6
                lines.append(f"| `{name[:70]}` | {rd:.1f} | {wr:.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_mfma(paths, cmd, out, title):
    """Matrix-core counters per library kernel from rocprofv3 --pmc MfmaUtil MfmaFlopsBF16:
    busy share of the SIMDs' matrix cores, and executed bf16 MFMA flops over the dispatch's own
    duration (hi/lo operand splits count every MFMA they issue)."""
    import csv
    per = {}
    for p in paths:
        for r in csv.DictReader(open(p)):
            name = r["Kernel_Name"]
            if not name.startswith("_ZN3gla"):
                continue
            d = per.setdefault(name, {"dur": {}, "ctr": {}})
            did = r["Dispatch_Id"]
            d["dur"][did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            d["ctr"].setdefault(r["Counter_Name"], {})[did] = float(r["Counter_Value"])
    lines = [f"# {title}", "", "Command:", "", "```", cmd, "```", "",
             "MFMA busy: `MfmaUtil` (matrix-core busy cycles over active cycles of all SIMDs). "
             "Executed bf16 flops: `MfmaFlopsBF16` (512 per MFMA MOP), over each dispatch's duration in "
             f"the same run, against the {PEAK_BF16_FLOPS / 1e12:.0f} TFLOP/s dense bf16 peak. Medians over "
             "dispatches.", "",
             "| kernel | dispatches | avg (us) | MFMA busy % | executed bf16 TFLOP/s | % of peak |",
             "|---|---|---|---|---|---|"]
    for name, d in per.items():
        util = d["ctr"].get("MfmaUtil", {})
        fl = d["ctr"].get("MfmaFlopsBF16", {})
        ids = [i for i in d["dur"] if i in fl]
        if not ids:
            continue
        dur = float(np.median([d["dur"][i] for i in ids]))
        tf = float(np.median([fl[i] / d["dur"][i] for i in ids])) / 1e12
        u = float(np.median([util[i] for i in ids if i in util])) if util else float("nan")
        short = name.split("(")[0]
        short = short[:70] + "..." if len(short) > 70 else short
        lines.append(f"| `{short}` | {len(ids)} | {dur * 1e6:.1f} | {u:.1f} | {tf:.1f} | "
                     f"{100 * tf * 1e12 / PEAK_BF16_FLOPS:.2f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def traffic_for(kernel):
    """Counter-measured HBM bytes per launch of `kernel`, if taken on the current sources."""
    try:
        s = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if s.get("kernel") != kernel or s.get("csrc_hash") != csrc_hash():
        return None
    return s.get("traffic_bytes")


KERNEL_SYMBOLS = {"fwd.prep": "gla_prep_kernel", "fwd.walk": "walk_kernel", "fwd.out": "gla_fwd_out",
                  "fwd.walk_out": "walk_out_kernel",
                  "bwd.prep": "gla_prep_kernel",
                  "bwd.walk_fwd": "walk_kernel", "bwd.walk_rev": "walk_kernel", "bwd.chunk": "gla_bwd_chunk",
                  "bwd.dv": "gla_bwd_dv"}


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks ramp up over the first 10-15 ms of work after an idle spell: the default
    # warm-up (about 20 ms of steps at the 340M shape) lets the timed steps run at steady clocks
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--copy-calib-mb", type=float, default=0.0,
                    help="also run one plain device copy of this many MB (counter calibration)")
    ap.add_argument("--only", choices=["gla_1p3b", "decode", "gsa_decode", "gsa", "gsa_m128", "msgla", "long_fwd"],
                    help="run one extra workload alone and print its line (for profiling)")
    ap.add_argument("--summarize-stats")
    ap.add_argument("--summarize-pmc", nargs="+")
    ap.add_argument("--summarize-mfma", nargs="+")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--out", default="")
    ap.add_argument("--out-json", default="")
    ap.add_argument("--kernel", default="walk_reverse")
    ap.add_argument("--calib-kernel", default="copy")
    ap.add_argument("--calib-bytes", type=float, default=0.0)
    args = ap.parse_args()

    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.title, args.cmd, args.out)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.cmd, args.out, args.title)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.kernel, args.calib_kernel, args.calib_bytes, args.cmd,
                      args.out_json, args.out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the operator's work is per batch-row and head and "
              f"needs no communication); --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_recurrent_sequence_gla_amd as m
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    m.lib()

    if args.copy_calib_mb > 0:
        nb = int(args.copy_calib_mb * 1e6) // 16 * 16
        a = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.only:
        # one extra workload alone (for profiling it); prints its JSON object
        fns = {"decode": lambda: run_decode(torch, m), "gsa_decode": lambda: run_gsa_decode(torch, m),
               "long_fwd": lambda: run_long_fwd(torch, m, args.steps, args.warmup),
               "gsa": lambda: run_gsa(torch, m, args.steps, args.warmup),
               "gsa_m128": lambda: run_gsa(torch, m, args.steps, args.warmup, name="gsa_340m_m128"),
               "msgla": lambda: run_msgla(torch, m, args.steps, args.warmup),
               "gla_1p3b": lambda: c3_line(torch, m, args.steps, args.warmup)}
        print(json.dumps({args.only: fns[args.only]()}), flush=True)
        return

    r = run_gla(torch, m, args.steps, args.warmup)
    w = r["w"]
    B, H, L, Dk, Dv, C = w.B, w.H, w.L, w.Dk, w.Dv, w.C
    sm = gla_summary(r)
    roof = dict(sm["roofline"])
    roof["traffic"] = traffic_for(KERNEL_SYMBOLS[sm["dominant"]])
    out = {
        "metric": METRIC,
        "value": sm["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sm["ms_per_step"],
        "ms_per_step_median": sm["ms_per_step_median"],
        "ms_per_step_min": sm["ms_per_step_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: GLA fwd+bwd (forward keeps chunk operands and states for the "
                               f"backward), B={B} H={H} L={L} Dk={Dk} Dv={Dv} C={C}, bf16 inputs, fp32 "
                               "accumulation, no initial state",
                   "B": B, "H": H, "L": L, "Dk": Dk, "Dv": Dv, "C": C},
        "pct_bf16_mfma_peak": sm["pct_bf16_mfma_peak"],
        "tflops": sm["tflops"],
        "pct_hbm_roofline_step": sm["pct_hbm_roofline_step"],
        "kernel_us": sm["kernel_us"],
        "roofline": roof,
        "context": "the pages claim a standalone GLA layer beats FlashAttention-2 from about 1K tokens "
                   "(GLA visual companion, 'Episode thesis map'); they name no hardware or precision for it",
    }
    if not args.no_extras:
        ex = {"gla_1p3b": c3_line(torch, m, max(5, args.steps // 2), max(2, args.warmup // 2)),
              "decode": run_decode(torch, m), "gsa_decode": run_gsa_decode(torch, m),
              "long_fwd": run_long_fwd(torch, m)}
        g = run_gsa(torch, m)
        if g is not None:
            ex["gsa"] = g
        g = run_gsa(torch, m, name="gsa_340m_m128")
        if g is not None:
            ex["gsa_m128"] = g
        ex["msgla"] = run_msgla(torch, m)
        out["extras"] = ex
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(r["x"], B, H, L)
    print(json.dumps(out), flush=True)


def c3_line(torch, m, steps, warmup):
    """The 1.3B-layer shape (B=4, H=4, L=4096, Dk=256, Dv=512, C=64, initial state ~ N(0, 0.02^2)),
    fwd+bwd timed as the headline step is."""
    r = run_gla(torch, m, steps, warmup, name="gla_1p3b")
    w = r["w"]
    sm = gla_summary(r)
    sm.pop("dominant")
    return {"workload": f"gla_1p3b: GLA fwd+bwd B={w.B} H={w.H} L={w.L} Dk={w.Dk} Dv={w.Dv} C={w.C}, bf16, "
                        "non-zero initial state, final state kept", **sm}


if __name__ == "__main__":
    main()
