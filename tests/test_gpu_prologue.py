"""GPU parity of the fused input prologue (gdr2_prologue bits): raw q, k
normalised per token and raw gate pre-activations activated inside the
kernels, against the fp64 oracle applying oracle.prologue to the same raw
inputs (forward, chunk-start states, decode step and backward), normwise per
(batch, head) slice with the dtype's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from oracle import prologue as pro
from gated_delta_rule_86_amd import gdr2
from gated_delta_rule_86_amd.inputs import Workload, draw_cotangents, draw_raw, to_f64
from tests.parity import TOL, normwise, to_dev

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "b", "w", "g")
GRADS = ("dq", "dk", "dv", "db", "dw", "dg")

FWD_CASES = [
    # name, B, T, H, D, dtype, gates, S0 std, chunk, prologue bits
    ("f32_d64_c32_all", 1, 100, 2, 64, "f32", "full", 0.05, 32, pro.ALL),
    ("f32_d64_c64_norm", 2, 70, 1, 64, "f32", "full", 0.0, 64, pro.NORM_QK),
    ("f32_d128_c32_gates", 1, 64, 2, 128, "f32", "scalar", 0.02, 32, pro.GATES),
    ("bf16_d128_c64_all_ragged", 2, 150, 2, 128, "bf16", "full", 0.05, 64, pro.ALL),
    ("bf16_d128_c64_all_scalar", 1, 130, 3, 128, "bf16", "scalar", 0.0, 64, pro.ALL),
    ("bf16_d64_c32_norm", 1, 96, 2, 64, "bf16", "full", 0.05, 32, pro.NORM_QK),
]


def _inputs(wl, bits):
    """Raw projections for the prologue's bits; the parts a bit does not
    cover are brought into the recurrence's valid range here instead (unit
    keys without NORM_QK; gates in (0, 1) and log-decay <= 0 without GATES),
    so every case is a stable recurrence.  Casts back to the input dtype."""
    inp = draw_raw(wl)
    if not bits & pro.NORM_QK:
        k = inp["k"].double()
        inp["k"] = (k / k.norm(dim=-1, keepdim=True)).to(inp["k"].dtype)
    if not bits & pro.GATES:
        inp["b"] = torch.sigmoid(inp["b"].double()).to(inp["b"].dtype)
        inp["w"] = torch.sigmoid(inp["w"].double()).to(inp["w"].dtype)
        inp["g"] = (-torch.nn.functional.softplus(inp["g"].double())).float()
    return inp


def _fwd_check(name, wl, bits, chunk, algo="auto"):
    inp = _inputs(wl, bits)
    d = to_dev(inp)
    o, S, ck = gdr2.forward(*(d[n] for n in NAMES), S0=d["S0"], chunk=chunk, chunk_states=True, prologue=bits,
                            algo=algo)
    torch.cuda.synchronize()
    raw = [to_f64(inp[n]) for n in NAMES]
    o_ref, S_ref, ck_ref = oracle.forward_checkpoints(*raw, every=chunk, S0=to_f64(inp["S0"]), prologue=bits)
    B, H, NC = wl.B, wl.H, ck_ref.shape[2]
    eo, es = normwise(to_f64(o), o_ref, "btd"), normwise(to_f64(S), S_ref, "state")
    ec = normwise(to_f64(ck).reshape(B, H * NC, wl.D, wl.D), ck_ref.reshape(B, H * NC, wl.D, wl.D), "state")
    print(f"{name}: o {eo:.2e} S {es:.2e} chunk states {ec:.2e}", flush=True)
    tol = TOL[wl.dtype]
    assert eo <= tol and es <= tol and ec <= tol, f"{name}: {eo:.3e} {es:.3e} {ec:.3e}"


@pytest.mark.parametrize("algo", ["staged", "fused"])
@pytest.mark.parametrize("name,B,T,H,D,dtype,gates,s0,chunk,bits", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_prologue_matches_oracle(name, B, T, H, D, dtype, gates, s0, chunk, bits, algo):
    """Both forward algorithms (the fused one for bf16 only)."""
    if algo == "fused" and dtype != "bf16":
        pytest.skip("the fused kernel takes bf16 inputs only")
    _fwd_check(name, Workload(name, "forward", B, T, H, D, dtype, gates, s0, chunk, 801), bits, chunk, algo=algo)


@pytest.mark.parametrize("dtype,D,chunk", [("bf16", 128, 64), ("f32", 64, 32)])
def test_forward_prologue_two_level_scan(dtype, D, chunk):
    """The prologue under the two-level scan over chunk segments (the span
    pass reads the factors the prologue-fused prep kernel wrote)."""
    name = f"{dtype}_d{D}_c{chunk}_all_segmented"
    _fwd_check(name, Workload(name, "forward", 1, 700, 2, D, dtype, "full", 0.05, chunk, 802), pro.ALL, chunk,
               algo="segmented")


@pytest.mark.parametrize("algo", ["staged", "fused"])
def test_forward_prologue_steep_decay_exact_path(algo):
    """Decay pre-activation 80: log-decay -softplus(80) ~ -80 per token, so
    the chunk's factors take the exact pair-by-pair path, which reads the
    raw inputs again and must apply the prologue there too."""
    wl = Workload("steep_pro", "forward", 1, 80, 2, 128, "bf16", "full", 0.05, 64, 802, g_const=80.0)
    _fwd_check("steep_pro", wl, pro.ALL, 64, algo=algo)


def test_prologue_off_is_unchanged():
    """Bits 0 run the plain kernels: identical results to a call that never
    names the prologue."""
    wl = Workload("pro_off", "forward", 1, 100, 2, 128, "bf16", "full", 0.05, 64, 803)
    d = to_dev(_inputs(wl, 0))
    o1, S1 = gdr2.forward(*(d[n] for n in NAMES), S0=d["S0"], chunk=64)
    o2, S2 = gdr2.forward(*(d[n] for n in NAMES), S0=d["S0"], chunk=64, prologue=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype,D,gates", [("bf16", 128, "full"), ("f32", 64, "scalar")])
def test_decode_prologue_matches_oracle(dtype, D, gates):
    wl = Workload("dec_pro", "decode", 16, 1, 4, D, dtype, gates, 0.05, 0, 804)
    inp = draw_raw(wl)
    state = inp["state"].cuda()
    o = gdr2.decode_step(state, *(inp[n].cuda() for n in NAMES), prologue=pro.ALL)
    torch.cuda.synchronize()
    st64 = to_f64(inp["state"]).copy()
    o_ref = oracle.decode_step(st64, *(to_f64(inp[n]) for n in NAMES), prologue=pro.ALL)
    eo, es = normwise(to_f64(o), o_ref, "nd"), normwise(to_f64(state), st64, "state")
    print(f"decode {dtype} d{D} {gates}: o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


BWD_CASES = [
    ("f32_d64_all", 1, 100, 2, 64, "f32", "full", 0.05, pro.ALL),
    ("f32_d64_norm_scalar", 2, 64, 1, 64, "f32", "scalar", 0.0, pro.NORM_QK),
    ("bf16_d128_all_ragged", 2, 150, 2, 128, "bf16", "full", 0.05, pro.ALL),
    ("bf16_d128_gates_scalar", 1, 130, 2, 128, "bf16", "scalar", 0.0, pro.GATES),
]


@pytest.mark.parametrize("name,B,T,H,D,dtype,gates,s0,bits", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_prologue_matches_oracle(name, B, T, H, D, dtype, gates, s0, bits):
    wl = Workload(name, "forward", B, T, H, D, dtype, gates, s0, 64, 805)
    inp = _inputs(wl, bits)
    inp.update(draw_cotangents(wl, 1.0))
    d = to_dev(inp)
    args = [d[n] for n in NAMES]
    _, _, ck = gdr2.forward(*args, S0=d["S0"], chunk=64, chunk_states=True, prologue=bits)
    got = gdr2.backward(*args, S_chunks=ck, dO=d["dO"], dS_final=d["dS_final"], prologue=bits)
    torch.cuda.synchronize()
    ref = oracle.backward(*(to_f64(inp[n]) for n in NAMES), dO=to_f64(inp["dO"]), S0=to_f64(inp["S0"]),
                          dS_final=to_f64(inp["dS_final"]), prologue=bits)
    errs = {n: normwise(to_f64(got[n]), ref[n], "btd") for n in GRADS}
    errs["dS0"] = normwise(to_f64(got["dS0"]), ref["dS0"], "state")
    print(f"{name}: " + " ".join(f"{n} {e:.1e}" for n, e in errs.items()), flush=True)
    for n in GRADS:
        assert np.isfinite(to_f64(got[n])).all(), n
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, f"{name}: {bad}"
