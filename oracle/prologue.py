"""fp64 definition of the optional input prologue -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this package (see ``oracle/__init__.py``).

The page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리" (section
"Gated Delta Rule-2 업데이트 수식", symbol table) takes the key L2-normalised
and the erase and write gates in [0, 1], the decay as a channel-wise diagonal
in (0, 1).  The prologue maps raw per-token inputs to those quantities before
the recurrence, so a caller can hand over projections directly:

  NORM_QK  q <- q (sum_i q_i^2 + eps)^(-1/2), same for k, per token and head
           over the d_k channels (eps = 1e-6)
  GATES    b <- sigmoid(b), w <- sigmoid(w), and the log-decay
           g <- -softplus(g) = log sigmoid(-g)

The pages name no activation functions: the logistic sigmoid (range (0, 1))
and the log-sigmoid decay are readings, as is the epsilon.  Each is a plain
elementwise or per-row definition; ``apply`` performs it and ``backward``
is its chain rule, composed with the recurrence's own gradients.
"""
from __future__ import annotations

import numpy as np

NORM_QK = 1
GATES = 2
ALL = NORM_QK | GATES
NORM_EPS = 1e-6


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def apply(q, k, b, w, g, flags: int):
    """The prologue's outputs (fp64 arrays) for raw inputs and flag bits."""
    q, k, b, w, g = (np.asarray(x, np.float64) for x in (q, k, b, w, g))
    if flags & ~ALL:
        raise ValueError(f"unknown prologue bits {flags:#x}")
    if flags & NORM_QK:
        q = q / np.sqrt((q * q).sum(-1, keepdims=True) + NORM_EPS)
        k = k / np.sqrt((k * k).sum(-1, keepdims=True) + NORM_EPS)
    if flags & GATES:
        b, w, g = _sigmoid(b), _sigmoid(w), -_softplus(g)
    return q, k, b, w, g


def backward(q, k, b, w, g, flags: int, grads: dict) -> dict:
    """Gradients with respect to the raw inputs, from those with respect to
    the prologue's outputs (keys dq, dk, db, dw, dg; others pass through)."""
    q, k, b, w, g = (np.asarray(x, np.float64) for x in (q, k, b, w, g))
    out = dict(grads)
    if flags & NORM_QK:
        # y = x r, r = (|x|^2 + eps)^(-1/2):  dx = r (dy - y (y . dy))
        for name, x in (("dq", q), ("dk", k)):
            r = 1.0 / np.sqrt((x * x).sum(-1, keepdims=True) + NORM_EPS)
            y, dy = x * r, np.asarray(grads[name], np.float64)
            out[name] = r * (dy - y * (y * dy).sum(-1, keepdims=True))
    if flags & GATES:
        sb, sw = _sigmoid(b), _sigmoid(w)
        out["db"] = np.asarray(grads["db"]) * sb * (1.0 - sb)
        out["dw"] = np.asarray(grads["dw"]) * sw * (1.0 - sw)
        out["dg"] = -np.asarray(grads["dg"]) * _sigmoid(g)     # d/dx[-softplus(x)] = -sigmoid(x)
    return out
