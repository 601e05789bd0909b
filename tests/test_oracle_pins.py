"""The fp64 oracle against its pins (closed forms, special cases, brute
force, a hand-worked example); see tests/oracle_pins.py for each pin's source."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_pin(name):
    res = pins.ALL_PINS[name](oracle.load())
    assert res <= pins.TOL[name], f"{name}: residual {res:.3e} > {pins.TOL[name]:.1e}"


def test_thread_count_does_not_change_results():
    import numpy as np
    rng = np.random.default_rng(0)
    p = pins.rand_problem(rng, B=3, T=7, H=3)
    o1, S1 = oracle.forward(**p, threads=1)
    o4, S4 = oracle.forward(**p, threads=4)
    assert (o1 == o4).all() and (S1 == S4).all()


def test_empty_sequence_returns_initial_state():
    import numpy as np
    rng = np.random.default_rng(0)
    p = pins.rand_problem(rng, B=2, T=0, H=2)
    S0 = rng.standard_normal((2, 2, 6, 5))
    o, S = oracle.forward(**p, S0=S0)
    assert o.shape == (2, 0, 2, 5) and (S == S0).all()
