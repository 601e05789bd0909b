"""gdr2_forward_chunked_noalloc (through the C ABI): the chunked forward whose
workspace is the library's static device scratch.  Its results must equal
gdr2_forward_chunked's (same kernels) bit for bit, on consecutive calls of
different sizes (the scratch keeps the previous call's contents), and
arguments needing more scratch than the library holds are refused before
any launch."""
import ctypes

import pytest
import torch

from gated_delta_rule_86_amd import gdr2
from gated_delta_rule_86_amd.inputs import Workload, draw
from tests.parity import TOL, normwise, oracle_forward, to_dev
from gated_delta_rule_86_amd.inputs import to_f64

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "b", "w", "g")


def _run(lib, entry, d, chunk, algo="auto"):
    B, T, H, D = d["q"].shape
    o = torch.full((B, T, H, D), float("nan"), dtype=d["q"].dtype, device="cuda")
    S = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    x = [d[n] for n in NAMES]
    ws = None
    if entry == "gdr2_forward_chunked":
        ws = torch.empty(max(gdr2.workspace_size(*x, chunk=chunk, algo=algo), 1), dtype=torch.uint8, device="cuda")
    a = gdr2.fwd_args(*x, S0=d.get("S0"), o=o, S_out=S, chunk=chunk, algo=algo, workspace=ws)
    stream = torch.cuda.current_stream().cuda_stream
    rc = getattr(lib, entry)(ctypes.byref(a), stream)
    assert rc == gdr2.OK, lib.gdr2_last_error()
    torch.cuda.synchronize()
    return o, S


CALLS = [
    # name, B, T, H, D, dtype, chunk, algo
    ("bf16_d128_c64", 2, 700, 4, 128, "bf16", 64, "staged"),
    ("bf16_d128_c64_smaller", 1, 200, 3, 128, "bf16", 64, "staged"),
    ("bf16_d64_c32_segmented", 1, 1500, 2, 64, "bf16", 32, "segmented"),
    ("f32_d64_c32_smallest", 1, 65, 1, 64, "f32", 32, "auto"),
]


def test_noalloc_equals_forward_on_consecutive_calls():
    lib = gdr2.load_library()
    for i, (name, B, T, H, D, dtype, C, algo) in enumerate(CALLS):
        print(f"noalloc call {i}: {name}", flush=True)
        inp = draw(Workload(name, "forward", B, T, H, D, dtype, "full", 0.05, C, 900 + i))
        d = to_dev(inp)
        o_ref, S_ref = _run(lib, "gdr2_forward_chunked", d, C, algo)
        o, S = _run(lib, "gdr2_forward_chunked_noalloc", d, C, algo)
        assert torch.equal(o, o_ref), name
        assert torch.equal(S, S_ref), name
        eo = normwise(to_f64(o), oracle_forward(inp)[0])
        assert eo <= TOL[dtype], (name, eo)


def test_noalloc_refuses_oversized_arguments():
    """The train_4k shape needs ~1.2 GB of workspace: refused with
    GDR2_ERR_WORKSPACE, nothing launched, outputs untouched."""
    lib = gdr2.load_library()
    B, T, H, D = 8, 4096, 16, 128
    q = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((B, T, H, D), dtype=torch.float32, device="cuda")
    o = torch.full_like(q, 7.0)
    S = torch.full((B, H, D, D), 7.0, device="cuda")
    a = gdr2.fwd_args(q, q, q, q, q, g, o=o, S_out=S, chunk=64, algo="staged")
    assert gdr2.workspace_size(q, q, q, q, q, g, chunk=64, algo="staged") > gdr2.NOALLOC_SCRATCH_BYTES
    rc = lib.gdr2_forward_chunked_noalloc(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == gdr2.ERR_WORKSPACE
    assert b"static scratch" in lib.gdr2_last_error()
    assert bool((o == 7.0).all()) and bool((S == 7.0).all())
