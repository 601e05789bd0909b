"""GPU parity of the chunked forward against the fp64 oracle, through the C ABI
(gdr2_forward_chunked).  Tolerances (normwise per (batch, head) slice, for
o and for the final state): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with
fp32 state.  The oracle always sees exactly the quantised inputs the GPU
sees, upcast to fp64."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_86_amd import gdr2
from gated_delta_rule_86_amd.inputs import WORKLOADS, Workload, draw, select_heads, to_f64
from tests.parity import TOL, finite, normwise, oracle_forward, to_dev

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "b", "w", "g")


def gpu_forward(inp, chunk, **kw):
    d = to_dev(inp)
    o, S = gdr2.forward(*(d[n] for n in NAMES), S0=d.get("S0"), chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, S


def check(inp, chunk, dtype, label, **kw):
    o, S = gpu_forward(inp, chunk, **kw)
    o_ref, S_ref = oracle_forward(inp)
    eo = normwise(to_f64(o), o_ref)
    es = normwise(to_f64(S), S_ref, "state")
    print(f"{label}: o {eo:.2e}  S {es:.2e}", flush=True)
    assert finite(o) and finite(S)
    assert eo <= TOL[dtype], f"{label}: o error {eo:.3e}"
    assert es <= TOL[dtype], f"{label}: state error {es:.3e}"
    return eo, es


def test_tiny_f32_workload():
    """B=1 H=1 T=256 d=64 fp32, chunk 32: the whole workload against the oracle."""
    wl = WORKLOADS["tiny_f32"]
    check(draw(wl), wl.chunk, wl.dtype, "tiny_f32")


SMALL = [(dt, D, C) for dt in ("bf16", "f32") for D in (64, 128) for C in (32, 64)
         if not (dt == "f32" and D * C > 4096)]


@pytest.mark.parametrize("dtype,D,C", SMALL, ids=[f"{a}-d{b}-c{c}" for a, b, c in SMALL])
@pytest.mark.parametrize("T", [1, 15, 33, 64, 130])
def test_ragged_lengths(dtype, D, C, T):
    wl = Workload("small", "forward", 2, T, 2, D, dtype, "full", 0.05, C, 7 * T + D + C)
    check(draw(wl), C, dtype, f"{dtype} D={D} C={C} T={T}")


# The prep pass is persistent (one workgroup per CU, items visited with a
# stride of the grid size, last chunk first): head counts above the grid
# size, item counts that are not a multiple of it, and several chunks per
# sequence exercise every carry of that walk.
WALK_CASES = [
    # B, T, H
    (1, 64, 300),
    (2, 130, 200),
    (3, 100, 7),
]


@pytest.mark.parametrize("B,T,H", WALK_CASES, ids=[f"B{b}_T{t}_H{h}" for b, t, h in WALK_CASES])
def test_prep_item_walk(B, T, H):
    wl = Workload("walk", "forward", B, T, H, 64, "bf16", "full", 0.05, 64, 17 * H + T + B)
    check(draw(wl), 64, "bf16", f"walk B={B} T={T} H={H}")


WIDTH_CFGS = [("bf16", 128, 64), ("f32", 64, 32), ("bf16", 64, 32)]
WIDTH_MIXES = [(nb, nw, ng) for nb in (0, 1) for nw in (0, 1) for ng in (0, 1)]


@pytest.mark.parametrize("dtype,D,C", WIDTH_CFGS, ids=[f"{a}-d{b}-c{c}" for a, b, c in WIDTH_CFGS])
@pytest.mark.parametrize("mix", WIDTH_MIXES, ids=["b%s_w%s_g%s" % tuple("1" if x else "d" for x in m)
                                                  for m in WIDTH_MIXES])
def test_gate_widths(dtype, D, C, mix):
    """Every gate-width mix (b, w, g each of width 1 or d; each mix has its
    own compiled prep kernel): scalar gates broadcast, and the result must
    equal the oracle on the same (width-1) inputs."""
    wl = Workload("widths", "forward", 2, 100, 2, D, dtype, "full", 0.05, C, 55 + D + C)
    inp = draw(wl)
    for n, narrow in zip(("b", "w", "g"), mix):
        if narrow:
            inp[n] = inp[n][..., :1].contiguous()
    check(inp, C, dtype, f"widths {mix} {dtype} D={D} C={C}")


@pytest.mark.parametrize("g_const,g_scale", [(0.0, 1.0), (-80.0, 1.0), (None, 0.01), (-1e-4, 1.0)],
                         ids=["no_decay", "steep_decay", "weak_decay", "tiny_decay"])
def test_decay_extremes(g_const, g_scale):
    """g = 0 (no decay), g = -80 (every factor underflows; the block-span
    guard takes the exact path), g scaled by 0.01 (long memory)."""
    wl = Workload("decay", "forward", 1, 200, 2, 128, "bf16", "full", 0.05, 64, 77,
                  g_scale=g_scale, g_const=g_const)
    check(draw(wl), 64, "bf16", f"decay const={g_const} scale={g_scale}")


def test_steep_decay_f32():
    wl = Workload("decay32", "forward", 1, 100, 1, 64, "f32", "full", 0.05, 32, 78, g_const=-80.0)
    check(draw(wl), 32, "f32", "steep decay f32")


def test_inplace_state_and_chaining():
    """S_out may alias S0; running x[:T1] then x[T1:] from the state it ends
    in reproduces one call (within rounding)."""
    wl = Workload("chain", "forward", 2, 300, 2, 128, "bf16", "full", 0.05, 64, 31)
    inp = draw(wl)
    d = to_dev(inp)
    o_all, S_all = gdr2.forward(*(d[n] for n in NAMES), S0=d["S0"], chunk=64)
    S = d["S0"].clone()
    parts = []
    for lo, hi in ((0, 100), (100, 101), (101, 300)):
        sl = {n: d[n][:, lo:hi].contiguous() for n in NAMES}
        o, _ = gdr2.forward(*(sl[n] for n in NAMES), S0=S, S_out=S, chunk=64)
        parts.append(o)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp)
    assert normwise(to_f64(torch.cat(parts, 1)), o_ref) <= TOL["bf16"]
    assert normwise(to_f64(S), S_ref, "state") <= TOL["bf16"]
    assert normwise(to_f64(o_all), o_ref) <= TOL["bf16"]


def test_inplace_state_two_level_scan():
    """S_out aliasing S0 under the two-level scan: segment 0 starts from the
    span pass's copy of S0 while the last segment writes S_out in the same
    pass, so the result equals the out-of-place call bit for bit."""
    wl = Workload("inplace_seg", "forward", 1, 2000, 2, 128, "bf16", "full", 0.05, 64, 32, g_scale=0.05)
    d = to_dev(draw(wl))
    args = [d[n] for n in NAMES]
    o1, S1 = gdr2.forward(*args, S0=d["S0"], chunk=64, algo="segmented")
    S = d["S0"].clone()
    o2, S2 = gdr2.forward(*args, S0=S, S_out=S, chunk=64, algo="segmented")
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S)


def test_zero_length_copies_state():
    wl = Workload("t0", "forward", 2, 0, 3, 64, "bf16", "full", 0.05, 64, 5)
    inp = draw(wl)
    d = to_dev(inp)
    o, S = gdr2.forward(*(d[n] for n in NAMES), S0=d["S0"], chunk=64)
    torch.cuda.synchronize()
    assert o.shape[1] == 0 and torch.equal(S.cpu(), inp["S0"])
    o, S = gdr2.forward(*(d[n] for n in NAMES), S0=None, chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_deterministic_and_no_uninitialised_reads():
    """Two runs agree bit for bit (no atomics anywhere), and a workspace
    poisoned with NaN before the call leaves no NaN in the results."""
    wl = Workload("det", "forward", 2, 257, 3, 128, "bf16", "full", 0.05, 64, 8)
    inp = draw(wl)
    d = to_dev(inp)
    args = [d[n] for n in NAMES]
    need = gdr2.workspace_size(*args, chunk=64)
    ws = torch.full((need // 4,), float("nan"), device="cuda").view(torch.uint8)
    o1, S1 = gdr2.forward(*args, S0=d["S0"], chunk=64, workspace=ws)
    ws.view(torch.float32).fill_(float("nan"))
    o2, S2 = gdr2.forward(*args, S0=d["S0"], chunk=64, workspace=ws)
    torch.cuda.synchronize()
    assert finite(o1) and finite(S1)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_gdn_scalar_workload():
    """B=4 H=16 T=2048 d=128 bf16, scalar beta (erase = write) and scalar decay."""
    wl = WORKLOADS["gdn_scalar"]
    check(draw(wl), wl.chunk, wl.dtype, "gdn_scalar")


def _sampled(wl, pairs, label):
    inp = draw(wl)
    o, S = gpu_forward(inp, wl.chunk)
    assert finite(o) and finite(S)
    sub = select_heads(inp, pairs)
    o_ref, S_ref = oracle_forward(sub)
    o_gpu = torch.stack([o[b, :, h:h + 1] for b, h in pairs]).cpu()
    S_gpu = torch.stack([S[b, h:h + 1] for b, h in pairs]).cpu()
    eo = normwise(to_f64(o_gpu), o_ref)
    es = normwise(to_f64(S_gpu), S_ref, "state")
    print(f"{label} (heads {pairs}): o {eo:.2e}  S {es:.2e}", flush=True)
    assert eo <= TOL[wl.dtype] and es <= TOL[wl.dtype]
    return o_gpu, o_ref, wl


def test_train_4k_workload_sampled_heads():
    """The benchmark workload (B=8 H=16 T=4096 d=128 bf16, chunk 64) in the
    launch configuration the benchmark times; the oracle checks 6 of the 128
    independent (b, h) recurrences, first and last included."""
    _sampled(WORKLOADS["train_4k"], [(0, 0), (0, 15), (3, 7), (5, 2), (7, 0), (7, 15)], "train_4k")


def test_long_64k_workload_sampled_heads():
    """B=1 H=16 T=65536 with S0 ~ N(0, 0.02^2): 2 heads against the oracle,
    and the error per 64-token chunk over the 1024 chunks reported."""
    o_gpu, o_ref, wl = _sampled(WORKLOADS["long_64k"], [(0, 0), (0, 9)], "long_64k")
    x = to_f64(o_gpu)[:, :, 0]
    y = o_ref[:, :, 0]
    per_chunk = np.abs(x - y).reshape(2, -1, 64, 128).max(axis=(2, 3)) / np.abs(y).max(axis=(1, 2))[:, None]
    q = per_chunk.shape[1] // 4
    print("long_64k per-chunk error, quartile maxima:",
          [float(per_chunk[:, i * q:(i + 1) * q].max()) for i in range(4)], flush=True)


@pytest.mark.parametrize("algo", ["staged", "auto"])
def test_weak_decay_long_sequence(algo):
    """g scaled by 0.01: memory spans thousands of tokens, so the state carries
    the accumulated chunk updates; the error must not grow past tolerance.
    With 2 heads and 128 chunks, AUTO takes the two-level scan (on 256 CUs:
    32 segments of 4 chunks), whose segment products are far from zero here."""
    wl = Workload("weak", "forward", 1, 8192, 2, 128, "bf16", "full", 0.02, 64, 4321, g_scale=0.01)
    check(draw(wl), 64, "bf16", f"weak decay T=8192 {algo}", algo=algo)


# Two-level scan forced on small shapes.  Segment plans on 256 CUs:
# 4 segments of 3 chunks (the last of 2), one chunk per segment, 2 per
# segment with a 1-chunk tail, and so on.
SEG_CASES = [
    # name, B, T, H, D, dtype, chunk, S0 std, gates
    ("bf16_d128_c64_len3", 4, 647, 8, 128, "bf16", 64, 0.05, "full"),
    ("f32_d64_c32_len1", 1, 333, 2, 64, "f32", 32, 0.05, "full"),
    ("bf16_d64_c32_len2", 2, 2000, 3, 64, "bf16", 32, 0.02, "full"),
    ("f32_d128_c32_len1", 1, 500, 1, 128, "f32", 32, 0.0, "full"),
    ("bf16_d128_c32_len2", 1, 1500, 4, 128, "bf16", 32, 0.05, "scalar"),
    ("f32_d64_c64_len1", 1, 700, 3, 64, "f32", 64, 0.05, "full"),
    ("bf16_d128_c64_two_chunks", 1, 100, 1, 128, "bf16", 64, 0.05, "full"),
]


@pytest.mark.parametrize("name,B,T,H,D,dtype,chunk,s0,gates", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_segmented_matches_oracle(name, B, T, H, D, dtype, chunk, s0, gates):
    wl = Workload(name, "forward", B, T, H, D, dtype, gates, s0, chunk, 5000 + T)
    check(draw(wl), chunk, dtype, f"segmented {name}", algo="segmented")


def test_segmented_weak_decay_products():
    """g scaled by 0.005 over 40 chunks in 40 one-chunk segments: every segment
    start is a fold of many nearly undecayed chunk products."""
    wl = Workload("weak_seg", "forward", 1, 2560, 1, 64, "f32", "full", 0.05, 64, 4322, g_scale=0.005)
    check(draw(wl), 64, "f32", "segmented weak decay", algo="segmented")


def test_segmented_stage_split_and_determinism():
    """PREP then STATE equals one call bit for bit on the segmented path, and
    two calls agree bit for bit."""
    wl = Workload("seg_stages", "forward", 1, 1000, 2, 128, "bf16", "full", 0.05, 64, 13)
    d = to_dev(draw(wl))
    args = [d[n] for n in NAMES]
    o1, S1 = gdr2.forward(*args, S0=d["S0"], chunk=64, algo="segmented")
    o3, S3 = gdr2.forward(*args, S0=d["S0"], chunk=64, algo="segmented")
    ws = torch.empty(gdr2.workspace_size(*args, chunk=64, algo="segmented"), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    gdr2.forward(*args, S0=d["S0"], chunk=64, out=o2, S_out=S2, workspace=ws, stage="prep", algo="segmented")
    gdr2.forward(*args, S0=d["S0"], chunk=64, out=o2, S_out=S2, workspace=ws, stage="state", algo="segmented")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o1, o3) and torch.equal(S1, S3)


def test_stage_split_equals_one_call():
    """PREP then STATE as two calls gives bit for bit the one-call result."""
    wl = Workload("stages", "forward", 2, 200, 2, 128, "bf16", "full", 0.05, 64, 12)
    inp = draw(wl)
    d = to_dev(inp)
    args = [d[n] for n in NAMES]
    o1, S1 = gdr2.forward(*args, S0=d["S0"], chunk=64)
    ws = torch.empty(gdr2.workspace_size(*args, chunk=64), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    gdr2.forward(*args, S0=d["S0"], chunk=64, out=o2, S_out=S2, workspace=ws, stage="prep")
    gdr2.forward(*args, S0=d["S0"], chunk=64, out=o2, S_out=S2, workspace=ws, stage="state")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
