"""Plant plausible mistakes in a copy of the C oracle (on the CPU) and check
that the pins catch every one of them: evidence that the pins constrain each
part of the recurrence (decay, erase, write, readout, gate broadcasting)."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr2_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("erase_transposed",
     "r[j] += e * S[i * dv + j];", "r[j] += k[i] * S[i * dv + j];"),
    ("decay_dropped",
     "double d = exp(gw == 1 ? g[0] : g[i]);", "double d = 1.0;"),
    ("decay_sign",
     "double d = exp(gw == 1 ? g[0] : g[i]);", "double d = exp(-(gw == 1 ? g[0] : g[i]));"),
    ("decay_broadcast",
     "double d = exp(gw == 1 ? g[0] : g[i]);", "double d = exp(g[0]);"),
    ("erase_gate_ignored",
     "double e = (bw == 1 ? b[0] : b[i]) * k[i];", "double e = k[i];"),
    ("erase_gate_index",
     "double e = (bw == 1 ? b[0] : b[i]) * k[i];", "double e = (bw == 1 ? b[0] : b[0]) * k[i];"),
    ("write_gate_ignored",
     "double u = (ww == 1 ? w[0] : w[j]) * v[j];", "double u = v[j];"),
    ("write_gate_on_read",
     "S[i * dv + j] += k[i] * (u - r[j]);", "S[i * dv + j] += k[i] * (u - (ww == 1 ? w[0] : w[j]) * r[j]);"),
    ("erase_sign",
     "S[i * dv + j] += k[i] * (u - r[j]);", "S[i * dv + j] += k[i] * (u + r[j]);"),
    ("erase_dropped",
     "S[i * dv + j] += k[i] * (u - r[j]);", "S[i * dv + j] += k[i] * u;"),
    ("readout_uses_k",
     "o[j] += q[i] * S[i * dv + j];", "o[j] += k[i] * S[i * dv + j];"),
    ("readout_transposed",
     "o[j] += q[i] * S[i * dv + j];", "o[j] += q[j < dk ? j : 0] * S[i * dv + (i < dv ? i : 0)];"),
    # the backward sweep
    ("bwd_readout_uses_old_state",
     "acc += Sn[i * dv + j] * dot[j];", "acc += Sprev[i * dv + j] * dot[j];"),
    ("bwd_erase_read_sign", "de[i] = -acc;", "de[i] = acc;"),
    ("bwd_erase_outer_sign",
     "double dsp = Lam[i * dv + j] - e * c[j];", "double dsp = Lam[i * dv + j] + e * c[j];"),
    ("bwd_erase_outer_dropped",
     "double dsp = Lam[i * dv + j] - e * c[j];", "double dsp = Lam[i * dv + j];"),
    ("bwd_decay_not_propagated", "Lam[i * dv + j] = d * dsp;", "Lam[i * dv + j] = dsp;"),
    ("bwd_dg_uses_undecayed", "acc += dsp * Sp[i * dv + j];", "acc += dsp * Sprev[i * dv + j];"),
    ("bwd_dk_drops_read",
     "acc += Lam[i * dv + j] * (u - r[j]);", "acc += Lam[i * dv + j] * u;"),
    ("bwd_dv_drops_gate",
     "dvt[j] = c[j] * (ww == 1 ? wt[0] : wt[j]);", "dvt[j] = c[j];"),
    ("bwd_db_drops_key", "dbt[i] = de[i] * kt[i];", "dbt[i] = de[i];"),
]


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", str(src),
                    "-o", str(so), "-lm"], check=True)
    return oracle.load(str(so))


def _compile(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    so = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", str(src),
                    "-o", str(so), "-lm"], check=True)
    return oracle.load(str(so))


def _caught(lib):
    return [n for n, f in pins.ALL_PINS.items() if not f(lib) <= pins.TOL[n]]


def test_decay_after_erase_is_caught(tmp_path):
    # apply D_t after the erase and write instead of before: D_t((I - k e^T) S + k u^T)
    text = open(SRC).read()
    start = text.index("    /* S' = D_t S_{t-1}")
    end = text.index("    /* r = S'^T (b_t . k_t)")
    decay = text[start:end]
    ro = text.index("    /* o_t = S_t^T q_t. */")
    mutated = text[:start] + text[end:ro] + decay + text[ro:]
    assert _caught(_compile(tmp_path, "late_decay", mutated))


def test_readout_before_update_is_caught(tmp_path):
    # move the readout ahead of the update: o_t = S_{t-1}^T q_t (after decay)
    text = open(SRC).read()
    start = text.index("    /* r = S'^T (b_t . k_t)")
    ro = text.index("    /* o_t = S_t^T q_t. */")
    end = text.index("}\n", text.index("o[j] += q[i] * S[i * dv + j];"))
    readout = text[ro:end]
    mutated = text[:start] + readout + text[start:ro] + text[end:]
    assert _caught(_compile(tmp_path, "early_readout", mutated)), "early readout not caught"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    assert _caught(lib), f"mutant {name} passes every pin"   # NaN residuals count as caught
