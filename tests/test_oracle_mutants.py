"""Plant plausible mistakes in a copy of the C oracle (on the CPU) and check
that the pins catch every one of them: evidence that the pins constrain each
part of the recurrence (decay, erase, write, readout, gate broadcasting)."""
import os
import subprocess

import numpy as np
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


# Mistakes planted in the prologue (oracle/prologue.py), each of which must
# fail a prologue pin.
def _mut_norm_axis(q, k, b, w, g, flags):
    from oracle import prologue as pro
    q, k, b, w, g = (np.asarray(x, np.float64) for x in (q, k, b, w, g))
    if flags & pro.NORM_QK:                                   # over heads instead of channels
        q = q / np.sqrt((q * q).sum(-2, keepdims=True) + pro.NORM_EPS)
        k = k / np.sqrt((k * k).sum(-2, keepdims=True) + pro.NORM_EPS)
    if flags & pro.GATES:
        b, w, g = pro._sigmoid(b), pro._sigmoid(w), -pro._softplus(g)
    return q, k, b, w, g


def _mut_decay_sign(q, k, b, w, g, flags):
    from oracle import prologue as pro
    q, k, b, w, g = _ORIG_APPLY(q, k, b, w, g, flags & pro.NORM_QK)
    if flags & pro.GATES:
        b, w, g = pro._sigmoid(b), pro._sigmoid(w), pro._softplus(g)
    return q, k, b, w, g


def _mut_sigmoid_grad(q, k, b, w, g, flags, grads):
    out = _ORIG_BACKWARD(q, k, b, w, g, flags, grads)
    from oracle import prologue as pro
    if flags & pro.GATES:
        out["db"] = np.asarray(grads["db"]) * pro._sigmoid(np.asarray(b))
    return out


def _mut_norm_grad(q, k, b, w, g, flags, grads):
    out = _ORIG_BACKWARD(q, k, b, w, g, flags, grads)
    from oracle import prologue as pro
    if flags & pro.NORM_QK:                                   # Jacobian without the projection
        kk = np.asarray(k, np.float64)
        out["dk"] = np.asarray(grads["dk"]) / np.sqrt((kk * kk).sum(-1, keepdims=True) + pro.NORM_EPS)
    return out


from oracle import prologue as _prologue_mod  # noqa: E402

_ORIG_APPLY = _prologue_mod.apply
_ORIG_BACKWARD = _prologue_mod.backward
PROLOGUE_MUTANTS = [("norm_over_heads", "apply", _mut_norm_axis), ("decay_sign", "apply", _mut_decay_sign),
                    ("sigmoid_derivative", "backward", _mut_sigmoid_grad),
                    ("norm_jacobian_no_projection", "backward", _mut_norm_grad)]


@pytest.mark.parametrize("name,attr,fn", PROLOGUE_MUTANTS, ids=[m[0] for m in PROLOGUE_MUTANTS])
def test_prologue_mutant_is_caught(monkeypatch, name, attr, fn):
    monkeypatch.setattr(_prologue_mod, attr, fn)
    lib = oracle.load()
    failed = []
    for pin in ("prologue_normalised_retrieval", "prologue_gate_values", "prologue_finite_differences"):
        try:
            res = pins.ALL_PINS[pin](lib)
            if not res <= pins.TOL[pin]:
                failed.append(pin)
        except AssertionError:
            failed.append(pin)
    assert failed, f"prologue mutant {name} survived every prologue pin"
