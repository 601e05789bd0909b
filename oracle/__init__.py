"""fp64 CPU oracle for the Gated DeltaNet-2 recurrence -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never links, loads or
calls it, and the two share no code.

``gdr2_oracle.c`` holds the plain, sequential, token-by-token recurrence of the
page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리", section
"Gated Delta Rule-2 업데이트 수식":

    S_t = (I - k_t (b_t * k_t)^T) D_t S_{t-1} + k_t (w_t * v_t)^T,   o_t = S_t^T q_t

with D_t = diag(exp(g_t)).  This module is a ctypes wrapper around it
(argument marshalling only) plus the build step.  ``chunked.py`` holds the
chunkwise reorganisation of the same recurrence, checked against this one.

Pinning: every part of the recurrence is pinned by tests/test_oracle_pins.py
against closed forms, special cases that reduce to textbook routines, brute
force with explicit transition matrices, and a hand-worked example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from . import prologue as _pro

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr2_oracle.c")
_LIB = os.path.join(_HERE, "libgdr2_oracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_L = ctypes.c_long


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall",
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str | None = None):
    """Load (building first if absent) the oracle library; returns the CDLL.
    GDR2_ORACLE_LIB, when set, names another build of the same source to
    load instead (the sanitizer test runs the pins against an ASan/UBSan
    build this way)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            alt = os.environ.get("GDR2_ORACLE_LIB")
            if alt:
                _lib = _bind(ctypes.CDLL(alt))
            else:
                if not os.path.exists(_LIB):
                    build()
                _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    lib.gdr2_oracle_forward.restype = ctypes.c_int
    lib.gdr2_oracle_forward.argtypes = [_L, _L, _L, _L, _L, _D, _D, _D, _D, _L, _D, _L,
                                        _D, _L, _D, _D, _D, ctypes.c_int]
    lib.gdr2_oracle_forward_ckpt.restype = ctypes.c_int
    lib.gdr2_oracle_forward_ckpt.argtypes = [_L, _L, _L, _L, _L, _D, _D, _D, _D, _L, _D, _L,
                                             _D, _L, _D, _D, _D, _L, _D, ctypes.c_int]
    lib.gdr2_oracle_backward.restype = ctypes.c_int
    lib.gdr2_oracle_backward.argtypes = [_L, _L, _L, _L, _L, _D, _D, _D, _D, _L, _D, _L, _D, _L,
                                         _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, ctypes.c_int]
    lib.gdr2_oracle_decode.restype = ctypes.c_int
    lib.gdr2_oracle_decode.argtypes = [_L, _L, _L, _L, _D, _D, _D, _D, _L, _D, _L, _D, _L,
                                       _D, _D, ctypes.c_int]
    lib.gdr2_oracle_max_threads.restype = ctypes.c_int
    lib.gdr2_oracle_max_threads.argtypes = []
    return lib


def _f64(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


def _width(gate, full, name):
    wdt = gate.shape[-1]
    if wdt not in (1, full):
        raise ValueError(f"{name}: last dim must be 1 or {full}, got {wdt}")
    return wdt


def forward(q, k, v, b, w, g, S0=None, threads: int = 0, lib=None, prologue: int = 0):
    """Sequential fp64 forward.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; b: [B,T,H,1|dk]; w: [B,T,H,1|dv];
    g: [B,T,H,1|dk] (log-decay); S0: [B,H,dk,dv] or None (zeros).
    prologue: bits of oracle.prologue applied to the raw q, k, b, w, g first.
    Returns (o [B,T,H,dv], S_final [B,H,dk,dv]) as float64 arrays.
    """
    lib = lib or load()
    q, k, b, w, g = _pro.apply(q, k, b, w, g, prologue)
    q, k, v, b, w, g = (_f64(x) for x in (q, k, v, b, w, g))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and v.shape == (B, T, H, dv)
    bw, ww, gw = _width(b, dk, "b"), _width(w, dv, "w"), _width(g, dk, "g")
    assert b.shape[:3] == (B, T, H) and w.shape[:3] == (B, T, H) and g.shape[:3] == (B, T, H)
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None:
        assert s0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S = np.zeros((B, H, dk, dv), dtype=np.float64)
    rc = lib.gdr2_oracle_forward(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(b), bw,
                                 _ptr(w), ww, _ptr(g), gw, _ptr(s0), _ptr(o), _ptr(S),
                                 int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr2_oracle_forward failed ({rc})")
    return o, S


def forward_checkpoints(q, k, v, b, w, g, every: int, S0=None, threads: int = 0, lib=None,
                        prologue: int = 0):
    """Sequential fp64 forward that also records the state before every
    `every`-th token (a checkpoint at each segment boundary).

    Returns (o, S_final, S_ckpt [B,H,ceil(T/every),dk,dv]) as float64 arrays;
    S_ckpt[:, :, n] is the state before token n*every (S_ckpt[:, :, 0] = S0).
    """
    lib = lib or load()
    q, k, b, w, g = _pro.apply(q, k, b, w, g, prologue)
    q, k, v, b, w, g = (_f64(x) for x in (q, k, v, b, w, g))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bw, ww, gw = _width(b, dk, "b"), _width(w, dv, "w"), _width(g, dk, "g")
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S = np.zeros((B, H, dk, dv), dtype=np.float64)
    ck = np.zeros((B, H, -(-T // every), dk, dv), dtype=np.float64)
    rc = lib.gdr2_oracle_forward_ckpt(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(b), bw,
                                      _ptr(w), ww, _ptr(g), gw, _ptr(s0), _ptr(o), _ptr(S),
                                      int(every), _ptr(ck), int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr2_oracle_forward_ckpt failed ({rc})")
    return o, S, ck


def backward(q, k, v, b, w, g, dO, S0=None, dS_final=None, threads: int = 0, lib=None,
             prologue: int = 0):
    """Sequential fp64 gradients of a loss through the forward.

    dO: dL/do [B,T,H,dv]; dS_final: dL/dS_final [B,H,dk,dv] or None (zero).
    prologue: bits of oracle.prologue; the gradients are then with respect
    to the raw inputs (the prologue's chain rule is applied last).
    Returns a dict with dq, dk, dv, db, dw, dg (shaped like the inputs; a
    width-1 gate's gradient is summed over its channels) and dS0.
    """
    if prologue:
        raw = (q, k, b, w, g)
        pq, pk, pb, pw, pg = _pro.apply(*raw, prologue)
        grads = backward(pq, pk, v, pb, pw, pg, dO, S0=S0, dS_final=dS_final, threads=threads, lib=lib)
        return _pro.backward(*raw, prologue, grads)
    lib = lib or load()
    q, k, v, b, w, g, dO = (_f64(x) for x in (q, k, v, b, w, g, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bw, ww, gw = _width(b, dk, "b"), _width(w, dv, "w"), _width(g, dk, "g")
    assert dO.shape == (B, T, H, dv)
    s0 = None if S0 is None else _f64(S0)
    dsf = None if dS_final is None else _f64(dS_final)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "db": np.zeros_like(b), "dw": np.zeros_like(w), "dg": np.zeros_like(g),
           "dS0": np.zeros((B, H, dk, dv), dtype=np.float64)}
    rc = lib.gdr2_oracle_backward(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(b), bw,
                                  _ptr(w), ww, _ptr(g), gw, _ptr(s0), _ptr(dO), _ptr(dsf),
                                  *(_ptr(out[n]) for n in ("dq", "dk", "dv", "db", "dw", "dg", "dS0")),
                                  int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr2_oracle_backward failed ({rc})")
    return out


def decode_step(state, q, k, v, b, w, g, threads: int = 0, lib=None, prologue: int = 0):
    """One decode step, in place on ``state`` [N,H,dk,dv] (float64, contiguous).

    q, k: [N,H,dk]; v: [N,H,dv]; b: [N,H,1|dk]; w: [N,H,1|dv]; g: [N,H,1|dk].
    prologue: bits of oracle.prologue applied to the raw token inputs first.
    Returns o [N,H,dv].
    """
    lib = lib or load()
    q, k, b, w, g = _pro.apply(q, k, b, w, g, prologue)
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags["C_CONTIGUOUS"]):
        raise TypeError("state must be a C-contiguous float64 array (updated in place)")
    q, k, v, b, w, g = (_f64(x) for x in (q, k, v, b, w, g))
    N, H, dk, dv = state.shape
    assert q.shape == (N, H, dk) and k.shape == (N, H, dk) and v.shape == (N, H, dv)
    bw, ww, gw = _width(b, dk, "b"), _width(w, dv, "w"), _width(g, dk, "g")
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.gdr2_oracle_decode(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(b), bw,
                                _ptr(w), ww, _ptr(g), gw, _ptr(state), _ptr(o), int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr2_oracle_decode failed ({rc})")
    return o


def max_threads(lib=None) -> int:
    return int((lib or load()).gdr2_oracle_max_threads())
