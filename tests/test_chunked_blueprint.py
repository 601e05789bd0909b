"""The chunkwise (WY) fp64 evaluation in oracle/chunked.py against the
sequential oracle: chunking is an exact reorganisation, so the two agree to
fp64 rounding for every chunk size, ragged tails included."""
import numpy as np
import pytest

import oracle
from oracle import chunked
from tests import oracle_pins as pins


@pytest.mark.parametrize("chunk", [1, 2, 7, 32, 64, 100, 128])
@pytest.mark.parametrize("widths", [(16, 12, 16), (1, 1, 1), (16, 1, 16)], ids=["full", "scalar", "mixed"])
def test_chunked_equals_sequential(chunk, widths):
    rng = np.random.default_rng(chunk * 7 + widths[0])
    bw, ww, gw = widths
    p = pins.rand_problem(rng, B=1, T=100, H=2, dk=16, dv=12, bw=bw, ww=ww, gw=gw)
    S0 = rng.standard_normal((1, 2, 16, 12)) * 0.3
    o_ref, S_ref = oracle.forward(**p, S0=S0)
    o, S = chunked.forward(**p, S0=S0, chunk=chunk)
    scale = max(np.abs(o_ref).max(), 1.0)
    assert np.abs(o - o_ref).max() / scale < 1e-12
    assert np.abs(S - S_ref).max() / max(np.abs(S_ref).max(), 1.0) < 1e-12


@pytest.mark.parametrize("g_const", [0.0, -80.0, -1e-3])
def test_chunked_decay_extremes(g_const):
    rng = np.random.default_rng(5)
    p = pins.rand_problem(rng, B=1, T=70, H=1, dk=8, dv=8)
    p["g"][:] = g_const
    S0 = rng.standard_normal((1, 1, 8, 8))
    o_ref, S_ref = oracle.forward(**p, S0=S0)
    o, S = chunked.forward(**p, S0=S0, chunk=32)
    assert np.abs(o - o_ref).max() < 1e-11 * max(1.0, np.abs(o_ref).max())
    assert np.abs(S - S_ref).max() < 1e-11 * max(1.0, np.abs(S_ref).max())


def test_chunk_intermediates_reproduce_the_update():
    """Delta rows are the per-token 'written minus read' vectors: feeding them
    back through S_t = D_t S_{t-1} + k_t delta_t^T replays the oracle's states."""
    rng = np.random.default_rng(9)
    p = pins.rand_problem(rng, B=1, T=20, H=1, dk=8, dv=6)
    S0 = rng.standard_normal((1, 1, 8, 6))
    _, _, kept = chunked.forward(**p, S0=S0, chunk=8, keep=True)
    S = S0[0, 0].copy()
    t = 0
    for c in kept[0]:
        for row in c["Delta"]:
            S = np.exp(p["g"][0, t, 0])[:, None] * S + np.outer(p["k"][0, t, 0], row)
            t += 1
        assert np.allclose(S, c["S_next"], atol=1e-12)
