"""Benchmark of the Gated DeltaNet-2 forward on one MI355X.

A step is one chunked forward (every stage of the path: cumulative decay,
decay-absorbed operands, gated Gram and scores, WY solve, state propagation
and output) over one batch of the training-shape workload: B=8, H=16,
T=4096, d_k=d_v=128, bf16 inputs, fp32 state, chunk 64, per-channel gates.
Inputs are seeded synthetic tensors (gated_delta_rule_86_amd.inputs), already
resident in device memory when the timed region starts.

Prints one JSON line: tokens/s (B*T per step time), the roofline of the
dominant kernel (HIP events on the launch stream, algorithmic bytes per
launch), the fp64 CPU oracle on the host cores, and in "extra" the per-kernel
split, the MFMA fraction, the batched decode step (256 x 16 states,
1000 steps) in GB/s, the forward for each gate-width mix, the chunked
backward over the same batch and the long-context forward (one sequence of
65536 tokens, two-level scan beside one pass).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "tokens/s, GDN-2 chunked fwd H=16 d=128 T=4K; % MFMA peak; decode HBM GB/s"
NAMES = ("q", "k", "v", "b", "w", "g")


def algorithmic_flops_per_chunk(C: int, D: int) -> int:
    """Dense contractions the chunked method must do per (b, h, chunk), with
    the triangular structure exploited: gated Gram, scores, WY solve, W S,
    K^T Delta, Q~ S, P Delta."""
    return (C * (C - 1) * D + C * (C + 1) * D + C * (C - 1) * (D + D)
            + 6 * C * D * D + C * (C + 1) * D)


def staged_bytes(B, T, H, D, C, esz, bw, ww, gw, s0: bool, s_out: bool):
    """Algorithmic HBM bytes per launch of the two staged kernels: every
    operand read once and every result written once."""
    rows = B * T * H
    nrec = B * H * -(-T // C)
    inputs = rows * ((2 * D + D + bw + ww) * esz + gw * 4)      # q,k,v,b,w (dtype) + g fp32
    kt = 2 if esz == 2 else 1                                  # 16-token blocks per P fragment
    p_frags = sum(t // kt + 1 for t in range(C // 16))         # nonzero 1 KB fragments of P
    factors = nrec * (4 * C * D * esz + p_frags * 1024 + D * 4)  # -W, U~, K^T, Q~, P, gamma
    state = B * H * D * D * 4
    prep = inputs + factors
    st = factors + rows * D * esz + (state if s0 else 0) + (state if s_out else 0)
    minimum = inputs + rows * D * esz + (state if s0 else 0) + (state if s_out else 0)
    return prep, st, minimum


def backward_flops_per_chunk(C: int, D: int) -> int:
    """Dense contractions of the chunked backward per (b, h, chunk), with the
    triangular structure exploited.  Recomputed forward factors: gated Gram
    and scores, WY solve, Delta = U~ - W S.  Reverse scan: K^ Lam, P^T dO,
    Q~^T dO, W^T dDelta.  Chunk-local gradients: dO S^T, dDelta S^T,
    Delta Lam^T, dO Delta^T, dDelta U^T + dW E~^T, X^T dDelta, X^T dW,
    X^T dX X^T, and the four decay-weighted sums of dM and dP."""
    tri = C * (C + 1) * D                 # one lower-triangular C x C x D product
    dense = 2 * C * D * D                 # one C x D x D product
    recompute = C * (C - 1) * D + tri + C * (C - 1) * (D + D) + dense
    scan = 3 * dense + tri
    grads = 3 * dense + tri + 2 * tri + 2 * tri + 2 * C * C * C * 2 // 3 + 4 * tri
    return recompute + scan + grads


def backward_min_bytes(B, T, H, D, esz) -> int:
    """Fewest HBM bytes the backward can move: the forward's inputs, dO and
    the chunk-start states read once, the fp32 gradients written once."""
    rows = B * T * H
    nck = -(-T // 64)
    return rows * (5 * D * esz + D * 4 + D * esz + 6 * D * 4) + B * H * nck * D * D * 4


def bench_backward(torch, gdr2, lib, wl, d, steps: int, warmup: int):
    """The chunked backward over the same batch: a forward that records the
    chunk-start states (untimed), then `steps` backward calls."""
    from gated_delta_rule_86_amd.inputs import draw_cotangents

    cot = {n: t.cuda() for n, t in draw_cotangents(wl, 1.0).items()}
    x = [d[n] for n in NAMES]
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    _, _, ck = gdr2.forward(*x, S0=d["S0"], chunk=64, chunk_states=True)
    grads = tuple(torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in x)
    dS0 = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr2.backward_workspace_size(*x), dtype=torch.uint8, device="cuda")
    a = gdr2.bwd_args(*x, ck, cot["dO"], cot["dS_final"], grads, dS0, workspace=ws)
    # the forward as a training step runs it: o, S_final and the chunk-start states
    o = torch.empty_like(d["v"])
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    fws = torch.empty(gdr2.workspace_size(*x, chunk=64), dtype=torch.uint8, device="cuda")
    f = gdr2.fwd_args(*x, S0=d["S0"], o=o, S_out=S_out, chunk=64, workspace=fws, S_chunks=ck)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        assert lib.gdr2_forward_chunked(ctypes.byref(f), stream) == 0, lib.gdr2_last_error()
        assert lib.gdr2_backward_chunked(ctypes.byref(a), stream) == 0, lib.gdr2_last_error()
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(steps):
        lib.gdr2_forward_chunked(ctypes.byref(f), stream)
    e1.record()
    for _ in range(steps):
        lib.gdr2_backward_chunked(ctypes.byref(a), stream)
    e2.record()
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / steps
    ms = e1.elapsed_time(e2) / steps
    flops = backward_flops_per_chunk(64, D) * B * H * -(-T // 64)
    mb = backward_min_bytes(B, T, H, D, 2)
    out = {"workload": "train_4k backward: dq, dk, dv, db, dw, dg, dS0 from dO and dS_final, "
                       "chunk-start states from the forward", "steps": steps, "ms": round(ms, 4),
           "tokens_per_s": round(B * T / (ms * 1e-3), 1), "workspace_bytes": ws.numel(),
           "algorithmic_flops": flops,
           "mfma_frac_bf16_dense": round(flops / (ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 4),
           "min_bytes": mb, "hbm_frac_of_min_bytes": round(mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "forward_with_chunk_states_ms": round(fwd_ms, 4),
           "train_step_tokens_per_s": round(B * T / ((fwd_ms + ms) * 1e-3), 1)}
    del ws, fws, grads, dS0, ck, cot, o, S_out
    return out


def bench_gate_widths(torch, gdr2, lib, d, steps: int):
    """The forward at the same shape for each gate-width mix: per-channel
    (GDN-2), KDA (scalar erase and write gate, per-channel decay), GDN (all
    scalar), the two ablation variants (one scalar gate) and scalar decay
    with per-channel gates.  Width-1 gates are channel 0 of the same draw."""
    x = {n: d[n] for n in NAMES}
    mixes = [("gdn2_per_channel", False, False, False), ("kda_scalar_b_w", True, True, False),
             ("gdn_all_scalar", True, True, True), ("scalar_write", False, True, False),
             ("scalar_erase", True, False, False), ("scalar_decay", False, False, True)]
    B, T, H, D = x["q"].shape
    o = torch.empty_like(x["v"])
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for name, nb, nw, ng in mixes:
        b = x["b"][..., :1].contiguous() if nb else x["b"]
        w = x["w"][..., :1].contiguous() if nw else x["w"]
        g = x["g"][..., :1].contiguous() if ng else x["g"]
        args = (x["q"], x["k"], x["v"], b, w, g)
        ws = torch.empty(gdr2.workspace_size(*args, chunk=64), dtype=torch.uint8, device="cuda")
        a = gdr2.fwd_args(*args, S0=d["S0"], o=o, S_out=S_out, chunk=64, workspace=ws)
        for _ in range(20):       # each mix warms up on its own workspace (3 calls read ~10% slow)
            lib.gdr2_forward_chunked(ctypes.byref(a), stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            lib.gdr2_forward_chunked(ctypes.byref(a), stream)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out.append({"gates": name, "widths_b_w_g": [b.shape[-1], w.shape[-1], g.shape[-1]],
                    "ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1)})
        del ws
    return out


def bench_prologue(torch, gdr2, lib, d, steps: int):
    """The forward with the fused input prologue (q, k normalised per token,
    gates and decay activated inside the kernels) beside the plain forward,
    same inputs and shape."""
    x = [d[n] for n in NAMES]
    B, T, H, D = x[0].shape
    o = torch.empty_like(d["v"])
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr2.workspace_size(*x, chunk=64), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, bits in (("plain", 0), ("prologue_all", gdr2.PROLOGUE_NORM_QK | gdr2.PROLOGUE_GATES)):
        a = gdr2.fwd_args(*x, S0=d["S0"], o=o, S_out=S_out, chunk=64, workspace=ws, prologue=bits)
        for _ in range(20):
            lib.gdr2_forward_chunked(ctypes.byref(a), stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            lib.gdr2_forward_chunked(ctypes.byref(a), stream)
        e1.record()
        torch.cuda.synchronize()
        res[name + "_ms"] = round(e0.elapsed_time(e1) / steps, 4)
    # a separate normalisation / activation pass would read and write q, k,
    # b, w, g once more: 2 x (4 x 256 + 512) B per token-head at d = 128, bf16
    res["separate_pass_bytes_saved"] = 2 * B * T * H * (4 * D * 2 + D * 4)
    del ws
    return res


def host_cpu_info() -> dict:
    """The host this process runs on: the CPU model, how many cores the OS
    shows, how many this process may use, and OMP_NUM_THREADS."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "nproc_online": os.cpu_count(), "affinity_cores": affinity,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def bench_fused(torch, gdr2, lib, steps: int):
    """The fused forward (one kernel, no workspace) beside the staged one:
    at the training shape, and at d = 64 with B*H = 256 (sequences x heads
    filling the GPU), where the library's default takes it."""
    from gated_delta_rule_86_amd.inputs import WORKLOADS, draw

    out = {}
    stream = torch.cuda.current_stream().cuda_stream
    for label, wl in (("train_4k", WORKLOADS["train_4k"]), ("B16_H16_T4096_d64", WORKLOADS["train_4k"].with_(B=16, D=64))):
        d = {n: (None if t is None else t.cuda()) for n, t in draw(wl).items()}
        x = [d[n] for n in NAMES]
        o = torch.empty_like(d["v"])
        S_out = torch.empty((wl.B, wl.H, wl.D, wl.D), dtype=torch.float32, device="cuda")
        for algo in ("staged", "fused"):
            ws = torch.empty(max(gdr2.workspace_size(*x, chunk=wl.chunk, algo=algo), 16), dtype=torch.uint8,
                             device="cuda")
            a = gdr2.fwd_args(*x, S0=d["S0"], o=o, S_out=S_out, chunk=wl.chunk, workspace=ws, algo=algo)
            for _ in range(20):
                assert lib.gdr2_forward_chunked(ctypes.byref(a), stream) == 0, lib.gdr2_last_error()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                lib.gdr2_forward_chunked(ctypes.byref(a), stream)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            out[f"{label}_{algo}_ms"] = round(ms, 4)
            out[f"{label}_{algo}_tokens_per_s"] = round(wl.B * wl.T / (ms * 1e-3), 1)
            del ws
        del d, x, o, S_out
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, wl):
    """The fp64 oracle (as it stands) on the host cores over the whole
    workload batch: every (b, h) recurrence, OpenMP over them, with as many
    threads as this process is granted (OMP_NUM_THREADS when it is set --
    the share of the host that goes with one GPU -- else every core of the
    affinity set).  Also one recurrence on one thread, the per-core rate.
    Returns the baseline record and the oracle's (o, S_final)."""
    import oracle
    from gated_delta_rule_86_amd.inputs import select_heads, to_f64

    host = host_cpu_info()
    omp = host["OMP_NUM_THREADS"]
    granted = int(omp) if omp and omp.isdigit() and int(omp) > 0 else host["affinity_cores"]
    threads = max(1, min(granted, wl.B * wl.H))
    args = [to_f64(inp[n]) for n in NAMES]
    t0 = time.perf_counter()
    o_ref, S_ref = oracle.forward(*args, S0=to_f64(inp["S0"]), threads=threads)
    dt = time.perf_counter() - t0
    one = select_heads(inp, [(0, 0)])
    a1 = [to_f64(one[n]) for n in NAMES]
    t1 = time.perf_counter()
    oracle.forward(*a1, S0=to_f64(one["S0"]), threads=1)
    dt1 = time.perf_counter() - t1
    rec = {"value": wl.B * wl.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "seconds": dt,
           "sample": f"the whole batch: {wl.B * wl.H} (b,h) recurrences x T={wl.T}, fp64, "
                     f"{threads} OpenMP threads (OpenMP over the independent recurrences)",
           "single_thread": {"recurrence_tokens": wl.T, "seconds": dt1,
                             "token_heads_per_s": wl.T / dt1},
           **host}
    return rec, o_ref, S_ref


def bench_decode(torch, gdr2, lib, steps: int, warmup: int, sets: int = 1):
    """`steps` batched decode steps (256 sequences x 16 heads, one token
    each).  With sets > 1, that many independent state sets take turns (step
    i updates set i % sets), so the working set is sets x 268 MB: two or
    more exceed the 256 MB memory-side cache, and the state then streams
    from HBM.  Every call's status is checked."""
    from gated_delta_rule_86_amd.inputs import WORKLOADS, draw, draw_decode_tokens

    wl = WORKLOADS["decode"]
    base = draw(wl)["state"]
    states = [base.cuda() for _ in range(sets)]
    ring = []
    for s in range(8):                         # 8 token sets reused cyclically
        tok = {n: t.cuda() for n, t in draw_decode_tokens(wl, s).items() if t is not None}
        o = torch.empty((wl.B, wl.H, wl.D), dtype=tok["q"].dtype, device="cuda")
        ring.append([gdr2.decode_args(st, *(tok[n] for n in NAMES), o) for st in states])
        for a in ring[-1]:
            a._keep = (tok, o)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(warmup):
        assert lib.gdr2_decode_step(ctypes.byref(ring[i % 8][i % sets]), stream) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bad = 0
    e0.record()
    for i in range(steps):
        bad |= lib.gdr2_decode_step(ctypes.byref(ring[i % 8][i % sets]), stream)
    e1.record()
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError("gdr2_decode_step failed: " + lib.gdr2_last_error().decode())
    us = e0.elapsed_time(e1) * 1e3 / steps
    nstate = wl.B * wl.H
    byts = nstate * (2 * wl.D * wl.D * 4 + (5 * wl.D) * 2 + wl.D * 4 + wl.D * 2)
    del states, ring
    torch.cuda.empty_cache()
    return {"workload": "decode: 256 sequences x 16 heads, d=128, bf16 tokens, fp32 state",
            "state_sets": sets, "working_set_bytes": sets * nstate * wl.D * wl.D * 4,
            "steps": steps, "us_per_step": us, "algorithmic_bytes_per_step": byts,
            "GBps": byts / (us * 1e-6) / 1e9, "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def bench_long(torch, gdr2, lib, steps: int, warmup: int, algos=("auto", "staged"), stages=("all", "state"),
               backward: bool = True):
    """The long-context forward: one sequence of 65536 tokens, 16 heads,
    d = 128, bf16, S0 ~ N(0, 0.02^2).  One pass over the 1024 chunks runs only
    32 state workgroups; the library's default here is the two-level scan over
    chunk segments.  Both are timed, with the state stage alone, and the
    backward over the same sequence with its reverse scan either way."""
    from gated_delta_rule_86_amd.inputs import WORKLOADS, draw

    wl = WORKLOADS["long_64k"]
    inp = draw(wl)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    x = [d[n] for n in NAMES]
    o = torch.empty_like(d["v"])
    S_out = torch.empty((wl.B, wl.H, wl.D, wl.D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {"workload": "long_64k: B=1 H=16 T=65536 d=128 bf16, per-channel gates, chunk 64, S0"}
    for algo in algos:
        ws = torch.empty(gdr2.workspace_size(*x, chunk=64, algo=algo), dtype=torch.uint8, device="cuda")
        for stage in stages:
            a = gdr2.fwd_args(*x, S0=d["S0"], o=o, S_out=S_out, chunk=64, workspace=ws, stage=stage, algo=algo)
            for _ in range(warmup):
                assert lib.gdr2_forward_chunked(ctypes.byref(a), stream) == 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                lib.gdr2_forward_chunked(ctypes.byref(a), stream)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            key = ("segmented" if algo == "auto" else "one_pass") + ("" if stage == "all" else "_state_stage")
            res[key + "_ms"] = round(ms, 4)
            if stage == "all":
                res[key + "_tokens_per_s"] = round(wl.B * wl.T / (ms * 1e-3), 1)
        del ws
    if backward:
        # the backward over the same sequence (chunk-start states from the
        # forward): one reverse pass, and the two-level reverse scan
        from gated_delta_rule_86_amd.inputs import draw_cotangents
        cot = {n: t.cuda() for n, t in draw_cotangents(wl, 1.0).items() if t is not None}
        _, _, ck = gdr2.forward(*x, S0=d["S0"], chunk=64, chunk_states=True)
        for algo in algos:
            ws = torch.empty(gdr2.backward_workspace_size(*x, algo=algo), dtype=torch.uint8, device="cuda")
            grads = tuple(torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in x)
            dS0 = torch.empty_like(S_out)
            run = lambda: gdr2.backward(*x, S_chunks=ck, dO=cot["dO"], dS_final=cot["dS_final"], workspace=ws,
                                        grads=grads, dS0=dS0, algo=algo)
            for _ in range(2):
                run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                run()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            key = "backward_" + ("segmented" if algo == "auto" else "one_pass")
            res[key + "_ms"] = round(ms, 4)
            res[key + "_tokens_per_s"] = round(wl.B * wl.T / (ms * 1e-3), 1)
            del ws, grads, dS0
        del ck, cot
    del d, x, o, S_out
    torch.cuda.empty_cache()
    return res


COPY_BYTES = 1 << 30
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_train_4k.md")


def plain_copy(torch, reps: int = 3):
    """A plain device copy of COPY_BYTES: the achievable-bandwidth reference
    of this run, and the known-size kernel the HBM counters are scaled by."""
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x, y
    return {"bytes_moved": 2 * COPY_BYTES, "ms": round(ms, 4),
            "GBps": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}


def parity_errors(o, S, o_ref, S_ref) -> dict:
    """Normwise error per (b, h) slice, max over the slices: max |x - y| over
    the slice / max |y| over the slice, for o and for S_final."""
    import numpy as np

    def nw(x, y, btd):
        x = np.asarray(x, np.float64)
        y = np.asarray(y, np.float64)
        if btd:
            x, y = np.moveaxis(x, 2, 1), np.moveaxis(y, 2, 1)
        x = x.reshape(x.shape[0] * x.shape[1], -1)
        y = y.reshape(y.shape[0] * y.shape[1], -1)
        den = np.abs(y).max(axis=1)
        return float((np.abs(x - y).max(axis=1) / np.where(den == 0, 1.0, den)).max())

    return {"o": nw(o, o_ref, True), "S_final": nw(S, S_ref, False), "tolerance": 2e-2,
            "slices": int(o_ref.shape[0] * o_ref.shape[2]),
            "metric": "max over (b,h) slices of max|gpu - oracle| / max|oracle|, oracle fp64 on the same "
                      "bf16 inputs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50, help="untimed steps right before the timed ones")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-gate-widths", action="store_true", help="skip the gate-width sweep")
    ap.add_argument("--no-copy", action="store_true", help="skip the plain-copy bandwidth reference")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context forward")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-kernel comparison")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the training-shape forward legs (warm-up, timed loop, repeats, per-kernel split): "
                         "for a profile of the headline kernels alone")
    ap.add_argument("--long-only", action="store_true",
                    help="time only the long-context forward and print its JSON object (for a profile of "
                         "those kernels alone)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the training-shape backward (after the forward that records the "
                         "chunk-start states) and print its JSON object (for a profile of the backward "
                         "kernels alone)")
    args = ap.parse_args()
    if args.headline_only:
        args.no_decode = args.no_long = args.no_fused = args.no_gate_widths = args.no_backward = True
        args.no_copy = args.no_cpu_baseline = True
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards across GPUs without communication by (batch, head); "
              "only the one-GPU measurement is implemented)", file=sys.stderr)
        sys.exit(2)

    import statistics

    import torch

    from gated_delta_rule_86_amd import gdr2
    from gated_delta_rule_86_amd.inputs import WORKLOADS, draw

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib = gdr2.load_library()
    if args.long_only:
        # the library's default algorithm only, whole calls: one kernel of each kind per call
        res = bench_long(torch, gdr2, lib, args.steps, args.warmup, algos=("auto",), stages=("all",), backward=False)
        print(json.dumps({"long_context": res}), flush=True)
        return
    if args.backward_only:
        wl = WORKLOADS["train_4k"]
        d = {n: (None if t is None else t.cuda()) for n, t in draw(wl).items()}
        print(json.dumps({"backward": bench_backward(torch, gdr2, lib, wl, d, args.steps, args.warmup)}), flush=True)
        return
    K = args.steps
    extra = {}
    # Legs other than the headline run first: they are timed on their own,
    # and by the time the headline loop starts the GPU has been busy for
    # a while (its clocks have settled).  Their GPU time is reported.
    t_legs = time.perf_counter()
    if not args.no_decode:
        extra["decode"] = bench_decode(torch, gdr2, lib, args.decode_steps, 20, sets=1)
        # two and four independent state sets (537 MB, 1.07 GB): more than the
        # 256 MB memory-side cache holds, so the state streams from HBM
        extra["decode_hbm_working_set"] = [bench_decode(torch, gdr2, lib, args.decode_steps, 20, sets=n)
                                           for n in (2, 4)]
    if not args.no_long:
        extra["long_context"] = bench_long(torch, gdr2, lib, max(1, K // 2), 5)
    if not args.no_fused:
        extra["fused"] = bench_fused(torch, gdr2, lib, K)

    wl = WORKLOADS["train_4k"]
    inp = draw(wl)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    B, T, H, D, C = wl.B, wl.T, wl.H, wl.D, wl.chunk
    o = torch.empty((B, T, H, D), dtype=d["q"].dtype, device="cuda")
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    x = [d[n] for n in NAMES]
    if not args.no_gate_widths:
        extra["gate_widths"] = bench_gate_widths(torch, gdr2, lib, d, K)
        extra["prologue"] = bench_prologue(torch, gdr2, lib, d, K)
    if not args.no_backward:
        # one training step of the layer: the forward that also records the
        # chunk-start states, then the backward
        extra["backward"] = bench_backward(torch, gdr2, lib, wl, d, max(1, K // 2), 2)
    torch.cuda.synchronize()
    legs_s = time.perf_counter() - t_legs

    need = gdr2.workspace_size(*x, chunk=C)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    a_all = gdr2.fwd_args(*x, S0=d["S0"], o=o, S_out=S_out, chunk=C, workspace=ws)
    a_prep = gdr2.fwd_args(*x, S0=d["S0"], o=o, S_out=S_out, chunk=C, workspace=ws, stage="prep")
    a_state = gdr2.fwd_args(*x, S0=d["S0"], o=o, S_out=S_out, chunk=C, workspace=ws, stage="state")
    stream = torch.cuda.current_stream().cuda_stream

    def call(a):
        rc = lib.gdr2_forward_chunked(ctypes.byref(a), stream)
        if rc != 0:
            raise RuntimeError(lib.gdr2_last_error().decode())

    for _ in range(args.warmup):
        call(a_all)
    torch.cuda.synchronize()
    # The step: K whole forward calls (every kernel of the path, one API
    # call each), events only at the ends of the timed region.
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e_start.record()
    for i in range(K):
        call(a_all)
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = e_start.elapsed_time(e_end) / K
    o_gpu, S_gpu = o.float().cpu(), S_out.cpu()
    # The spread: five more loops of K steps, each timed like the headline
    # (events only at its ends), min and median of their per-step times.
    reps = [step_ms]
    for _ in range(5):
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record()
        for i in range(K):
            call(a_all)
        r1.record()
        torch.cuda.synchronize()
        reps.append(r0.elapsed_time(r1) / K)
    # The per-kernel split: the same K steps, each kernel bracketed by
    # events on the launch stream (a stage call per kernel).  The events
    # between kernels cost a little, so these durations sum to slightly
    # more than the step.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record()
        call(a_prep)
        ev[i][1].record()
        call(a_state)
        ev[i][2].record()
    torch.cuda.synchronize()
    prep_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    state_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    split_step_ms = ev[0][0].elapsed_time(ev[-1][2]) / K
    tokens = B * T
    value = tokens / (step_ms * 1e-3)

    esz = 2
    prep_b, state_b, min_b = staged_bytes(B, T, H, D, C, esz, D, D, D, d["S0"] is not None, True)
    flops = algorithmic_flops_per_chunk(C, D) * B * H * (T // C)
    kernels = {"gdr2_chunk_prep[b,w,g=d,d,d]": prep_ms, "gdr2_chunk_state": state_ms}
    own_bytes = {"gdr2_chunk_prep[b,w,g=d,d,d]": prep_b, "gdr2_chunk_state": state_b}
    dom = max(kernels, key=lambda n: kernels[n])
    dom_ms = kernels[dom]
    # Algorithmic bytes of the path: the minimum a single fused pass moves
    # (q, k, v, b, w in bf16 and g in fp32 read once, o in bf16 written once:
    # 2048 B per token-head at d = 128, plus S_final), charged to the
    # dominant kernel's launch -- the kernels' own workspace traffic is not
    # algorithmic.
    achieved = min_b / (dom_ms * 1e-3) / 1e9
    from gated_delta_rule_86_amd.rocprof_summary import read_traffic
    measured = read_traffic(TRAFFIC_SUMMARY) or {}
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured.get(dom), "kernel": dom,
                "kernel_avg_us": round(dom_ms * 1e3, 2),
                "algorithmic_bytes_per_launch": min_b,
                "algorithmic_bytes_basis": "2048 B per token-head (q,k,v,b,w bf16 and g fp32 read once, "
                                           "o bf16 written once) x 524288 token-heads + S_final",
                "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE of these kernel sources, "
                                   "profiles/hbm_traffic_train_4k.md") if measured.get(dom) else None}
    t_mem_min = min_b / (HBM_PEAK_GBS * 1e9)
    t_mfma_min = flops / (BF16_DENSE_PEAK_TFLOPS * 1e12)
    extra.update({
        "step_ms": round(step_ms, 4), "wall_ms_per_step": round(wall * 1e3 / K, 4),
        "step_ms_over_6_loops": {"min": round(min(reps), 4), "median": round(statistics.median(reps), 4),
                                 "max": round(max(reps), 4)},
        "host_seconds_of_gpu_work_before_timed_loop": round(legs_s, 2),
        "prep_ms": round(prep_ms, 4), "state_ms": round(state_ms, 4),
        "split_step_ms_with_events_between_kernels": round(split_step_ms, 4),
        "path_min_bytes": min_b,
        "path_roofline_frac": round(max(t_mem_min, t_mfma_min) / (step_ms * 1e-3), 4),
        "path_hbm_frac_of_min_bytes": round(min_b / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_own_bytes": {n: {"bytes": own_bytes[n], "GBps": round(own_bytes[n] / (kernels[n] * 1e-3) / 1e9, 1),
                                 "note": "the kernel's own reads and writes, workspace included"}
                             for n in kernels},
        "algorithmic_flops": flops,
        "mfma_frac_bf16_dense": round(flops / (step_ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 4),
        "pages_context": "38.0 Kt/s (2K) and 36.1 Kt/s (8K): whole-model GDN-2 training "
                         "throughput on unstated hardware; not comparable",
    })
    if measured:
        extra["hbm_traffic_bytes_per_launch"] = measured
        fwd_traffic = sum(measured.get(n, 0) for n in kernels)
        if all(n in measured for n in kernels):
            extra["path_counter_traffic_bytes"] = fwd_traffic
            extra["path_counter_traffic_over_min_bytes"] = round(fwd_traffic / min_b, 3)

    del d, x, o, S_out, ws
    torch.cuda.empty_cache()
    if not args.no_copy:
        extra["plain_copy"] = plain_copy(torch)
        pc = extra["plain_copy"]["GBps"]
        extra["step_frac_of_plain_copy_bw"] = round(min_b / (step_ms * 1e-3) / 1e9 / pc, 4)
    cpu = None
    if not args.no_cpu_baseline:
        cpu, o_ref, S_ref = cpu_baseline(inp, wl)
        extra["parity"] = parity_errors(o_gpu.numpy(), S_gpu.numpy(), o_ref, S_ref)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "train_4k: GDN-2 chunked forward B=8 H=16 T=4096 d_k=d_v=128, "
                               "per-channel gates, chunk 64, bf16 inputs, fp32 state",
                   "B": B, "T": T, "H": H, "d": D, "chunk": C, "algo": "staged"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
