"""The chunked backward blueprint (oracle/chunked.py, fp64 NumPy) against
the sequential fp64 oracle backward: the chunk-level reverse and the
per-chunk gradient formulas reproduce the token-by-token chain rule for any
chunk size, ragged lengths, initial and final-state gradients, and every
gate width."""
import numpy as np
import pytest

import oracle
from oracle import chunked
from tests import oracle_pins as pins

CASES = [(13, 4, None, None, None), (16, 8, 1, 1, 1), (7, 7, None, 1, None), (20, 6, 1, None, 1),
         (9, 16, None, None, None), (64, 16, None, None, None)]


@pytest.mark.parametrize("T,C,bw,ww,gw", CASES)
def test_chunked_backward_matches_sequential(T, C, bw, ww, gw):
    rng = np.random.default_rng(T * 100 + C)
    p = pins.rand_problem(rng, B=2, T=T, H=2, dk=5, dv=4, bw=bw, ww=ww, gw=gw)
    S0 = rng.standard_normal((2, 2, 5, 4))
    dO = rng.standard_normal((2, T, 2, 4))
    dSf = rng.standard_normal((2, 2, 5, 4))
    ref = oracle.backward(**p, dO=dO, S0=S0, dS_final=dSf)
    got = chunked.backward(**p, dO=dO, S0=S0, dS_final=dSf, chunk=C)
    for name in ref:
        err = np.abs(ref[name] - got[name]).max() / max(np.abs(ref[name]).max(), 1e-30)
        assert err < 1e-11, (name, err)
