"""Out-of-bounds writes: every output buffer (and the workspace) sits inside a
larger allocation whose guard zones before and after it hold a sentinel; after
the call the guards must be untouched and the outputs fully written (no
sentinel left inside).  One case per kernel family: the staged forward (its
one-pass and two-level-scan forms), the fused forward, the decode step and
the backward, on ragged shapes."""
import pytest
import torch

from gated_delta_rule_86_amd import gdr2
from gated_delta_rule_86_amd.inputs import Workload, draw, draw_cotangents, draw_decode_tokens
from tests.parity import to_dev

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "b", "w", "g")
GUARD = 4096          # elements on each side (a multiple of 16 bytes for every dtype)
SENT = {torch.float32: -7.25e33, torch.bfloat16: -7.25e33, torch.uint8: 0xA5}


class Guarded:
    """A tensor of `shape` inside a buffer with GUARD sentinel elements on
    either side."""

    def __init__(self, shape, dtype, fill_inside=True):
        n = 1
        for s in shape:
            n *= s
        self.n, self.dtype = n, dtype
        self.buf = torch.full((n + 2 * GUARD,), SENT[dtype], dtype=dtype, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(shape)
        if not fill_inside:
            self.t.zero_()

    def check(self, name, written=True):
        lo, hi = self.buf[:GUARD], self.buf[GUARD + self.n:]
        s = torch.tensor(SENT[self.dtype], dtype=self.dtype, device="cuda")
        assert bool((lo == s).all()), f"{name}: write before the buffer"
        assert bool((hi == s).all()), f"{name}: write after the buffer"
        if written and self.n:
            assert not bool((self.t == s).any()), f"{name}: part of the output not written"


@pytest.mark.parametrize("algo", ["staged", "segmented", "fused"])
@pytest.mark.parametrize("D,C", [(128, 64), (64, 32)])
def test_forward_writes_only_its_outputs(algo, D, C):
    wl = Workload("canary", "forward", 2, 333, 3, D, "bf16", "full", 0.05, C, 71)
    d = to_dev(draw(wl))
    x = [d[n] for n in NAMES]
    B, T, H = 2, 333, 3
    NC = -(-T // C)
    o = Guarded((B, T, H, D), torch.bfloat16)
    S = Guarded((B, H, D, D), torch.float32)
    ck = Guarded((B, H, NC, D, D), torch.float32)
    need = gdr2.workspace_size(*x, chunk=C, algo=algo)
    ws = Guarded((max(need, 16),), torch.uint8)
    gdr2.forward(*x, S0=d["S0"], chunk=C, algo=algo, out=o.t, S_out=S.t, chunk_states=ck.t,
                 workspace=ws.t if need else None)
    torch.cuda.synchronize()
    o.check("o")
    S.check("S_out")
    ck.check("S_chunks")
    ws.check("workspace", written=False)


def test_decode_writes_only_its_outputs():
    wl = Workload("canary_dec", "decode", 37, 1, 5, 128, "bf16", "full", 0.05, 0, 72)
    st = draw(wl)["state"]
    tok = {n: t.cuda() for n, t in draw_decode_tokens(wl, 0).items() if t is not None}
    state = Guarded(tuple(st.shape), torch.float32)
    state.t.copy_(st.cuda())
    o = Guarded((37, 5, 128), torch.bfloat16)
    gdr2.decode_step(state.t, *(tok[n] for n in NAMES), out=o.t)
    torch.cuda.synchronize()
    o.check("o")
    state.check("state")


@pytest.mark.parametrize("widths", [(0, 0, 0), (1, 1, 1)], ids=["per_channel", "scalar_gates"])
def test_backward_writes_only_its_outputs(widths):
    wl = Workload("canary_bwd", "forward", 2, 150, 3, 128, "bf16", "full", 0.05, 64, 73)
    inp = draw(wl)
    inp.update(draw_cotangents(wl, 0.5))
    for n, nar in zip(("b", "w", "g"), widths):
        if nar:
            inp[n] = inp[n][..., :1].contiguous()
    d = to_dev(inp)
    x = [d[n] for n in NAMES]
    _, _, ck = gdr2.forward(*x, S0=d["S0"], chunk=64, chunk_states=True)
    grads = [Guarded(tuple(t.shape), torch.float32) for t in x]
    dS0 = Guarded((2, 3, 128, 128), torch.float32)
    need = gdr2.backward_workspace_size(*x)
    ws = Guarded((need,), torch.uint8)
    gdr2.backward(*x, S_chunks=ck, dO=d["dO"], dS_final=d["dS_final"], grads=tuple(g.t for g in grads),
                  dS0=dS0.t, workspace=ws.t)
    torch.cuda.synchronize()
    for n, g in zip(("dq", "dk", "dv", "db", "dw", "dg"), grads):
        g.check(n)
    dS0.check("dS0")
    ws.check("workspace", written=False)
