"""Seeded synthetic inputs for the Gated DeltaNet-2 forward and decode step.

This module only draws random numbers and casts them; it holds none of the
recurrence's arithmetic.  Both the tests (for the fp64 oracle and the HIP
library) and the benchmark take their inputs from here.

The workloads follow the model shape of the page "Gated DeltaNet-2: 선형
어텐션에서 삭제와 쓰기 게이트 분리" (section "Gated Delta Rule-2 업데이트 수식":
16 heads, d_k = d_v = 128; training at sequence length 4K; throughput quoted
at 2K and 8K).  No dataset is used: the pages' text corpora are stood in for
by these random tensors.

Recipe (per workload, ``numpy.random.default_rng(seed)``):
  * draw order: q, k, v, erase gate, write gate, decay pre-activation x,
    then S0 / state; each drawn in full, fp64, row-major [B, T, H, D];
  * q, v ~ N(0, 1); k ~ N(0, 1) then L2-normalised per token in fp64;
  * per-channel gates b ~ U(0,1)^{d_k}, w ~ U(0,1)^{d_v};
    scalar gates: one beta ~ U(0,1) per (batch, token, head) used as both
    b and w (width 1) -- drawn in the erase-gate slot, nothing drawn for w;
  * log-decay g = -softplus(x) = -log1p(exp(x)), x ~ N(0,1), per key channel
    (or one per token-head for scalar decay), stored as float32;
  * q, k, v, b, w are cast to the workload dtype with round-to-nearest-even;
  * S0 ~ N(0, s0_std^2) (float32) when s0_std > 0, else None.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "forward" or "decode"
    B: int               # batch (decode: number of sequences N)
    T: int               # tokens per sequence (decode: 1)
    H: int
    D: int               # d_k = d_v
    dtype: str           # "f32" or "bf16"
    gates: str           # "full" (per channel) or "scalar"
    s0_std: float        # 0 -> no initial state
    chunk: int           # chunk size for the chunked forward (decode: 0)
    seed: int
    g_scale: float = 1.0  # multiplies g (stress variants); 1.0 for the standard workloads
    g_const: float | None = None  # overrides g with a constant (stress variants)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "forward", 1, 256, 1, 64, "f32", "full", 0.0, 32, 86_001),
    "gdn_scalar": Workload("gdn_scalar", "forward", 4, 2048, 16, 128, "bf16", "scalar", 0.0, 64, 86_002),
    "train_4k": Workload("train_4k", "forward", 8, 4096, 16, 128, "bf16", "full", 0.0, 64, 86_003),
    "long_64k": Workload("long_64k", "forward", 1, 65536, 16, 128, "bf16", "full", 0.02, 64, 86_004),
    "decode": Workload("decode", "decode", 256, 1, 16, 128, "bf16", "full", 0.05, 0, 86_005),
}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _softplus(x):
    return np.log1p(np.exp(x))


def draw(wl: Workload, seed: int | None = None) -> dict:
    """Draw one set of inputs; returns CPU torch tensors.

    Forward: q,k [B,T,H,D]; v [B,T,H,D]; b [B,T,H,1|D]; w [B,T,H,1|D];
    g float32 [B,T,H,1|D]; S0 float32 [B,H,D,D] or None.
    Decode: the same with T squeezed ([N,H,.]) and 'state' instead of 'S0'.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    shp = (B, T, H, D)
    q = rng.standard_normal(shp)
    k = rng.standard_normal(shp)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal(shp)
    if wl.gates == "full":
        b = rng.random(shp)
        w = rng.random(shp)
        x = rng.standard_normal(shp)
    elif wl.gates == "scalar":
        b = rng.random((B, T, H, 1))
        w = b
        x = rng.standard_normal((B, T, H, 1))
    else:
        raise ValueError(wl.gates)
    g = -_softplus(x) * wl.g_scale
    if wl.g_const is not None:
        g = np.full_like(g, wl.g_const)
    S0 = None
    if wl.s0_std > 0:
        S0 = rng.standard_normal((B, H, D, D)) * wl.s0_std
    dt = TORCH_DTYPES[wl.dtype]
    out = {n: torch.from_numpy(a).to(dt) for n, a in
           (("q", q), ("k", k), ("v", v), ("b", b), ("w", w))}
    out["g"] = torch.from_numpy(g).to(torch.float32)
    out["S0"] = None if S0 is None else torch.from_numpy(S0).to(torch.float32)
    if wl.kind == "decode":
        for n in ("q", "k", "v", "b", "w", "g"):
            out[n] = out[n][:, 0].contiguous()
        out["state"] = out.pop("S0")
    return out


def draw_decode_tokens(wl: Workload, step: int) -> dict:
    """Fresh tokens for decode step `step` (no state): same recipe as `draw`,
    seed wl.seed + 1000 * (step + 1)."""
    return draw(wl.with_(s0_std=0.0), seed=wl.seed + 1000 * (step + 1))


def draw_raw(wl: Workload, seed: int | None = None) -> dict:
    """Raw projections for the input prologue: q, k ~ N(0, 1) scaled per
    token by U(0.5, 3) (not normalised), erase / write gate and decay
    pre-activations ~ N(0, 1) (width 1 when wl.gates == "scalar"), cast like
    `draw`; S0 ~ N(0, s0_std^2).  Seed wl.seed + 700_000 unless given."""
    rng = np.random.default_rng(wl.seed + 700_000 if seed is None else seed)
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    shp = (B, T, H, D)
    q = rng.standard_normal(shp) * rng.uniform(0.5, 3.0, (B, T, H, 1))
    k = rng.standard_normal(shp) * rng.uniform(0.5, 3.0, (B, T, H, 1))
    v = rng.standard_normal(shp)
    gshape = shp if wl.gates == "full" else (B, T, H, 1)
    b = rng.standard_normal(gshape)
    w = rng.standard_normal(gshape)
    x = rng.standard_normal(gshape)
    if wl.g_const is not None:
        x = np.full_like(x, wl.g_const)
    S0 = rng.standard_normal((B, H, D, D)) * wl.s0_std if wl.s0_std > 0 else None
    dt = TORCH_DTYPES[wl.dtype]
    out = {n: torch.from_numpy(a).to(dt) for n, a in (("q", q), ("k", k), ("v", v), ("b", b), ("w", w))}
    out["g"] = torch.from_numpy(x).to(torch.float32)
    out["S0"] = None if S0 is None else torch.from_numpy(S0).to(torch.float32)
    if wl.kind == "decode":
        for n in ("q", "k", "v", "b", "w", "g"):
            out[n] = out[n][:, 0].contiguous()
        out["state"] = out.pop("S0")
    return out


def draw_cotangents(wl: Workload, dS_std: float = 1.0, seed: int | None = None) -> dict:
    """Seeded loss cotangents for the backward: dO ~ N(0,1) [B,T,H,D] in the
    workload dtype, dS_final ~ N(0, dS_std^2) float32 [B,H,D,D] (None when
    dS_std == 0).  Seed wl.seed + 500_000 unless given."""
    rng = np.random.default_rng(wl.seed + 500_000 if seed is None else seed)
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    dO = torch.from_numpy(rng.standard_normal((B, T, H, D))).to(TORCH_DTYPES[wl.dtype])
    dS = None
    if dS_std > 0:
        dS = torch.from_numpy(rng.standard_normal((B, H, D, D)) * dS_std).to(torch.float32)
    return {"dO": dO, "dS_final": dS}


def select_heads(inp: dict, pairs) -> dict:
    """Restrict forward inputs to the given (b, h) pairs, each as its own
    batch row of one head: every (b, h) recurrence is independent."""
    out = {}
    for n in ("q", "k", "v", "b", "w", "g"):
        out[n] = torch.stack([inp[n][b, :, h:h + 1] for b, h in pairs])
    S0 = inp.get("S0")
    out["S0"] = None if S0 is None else torch.stack([S0[b, h:h + 1] for b, h in pairs])
    for n in ("dO", "dS_final"):      # cotangents, when present
        t = inp.get(n)
        if t is not None:
            out[n] = torch.stack([t[b, :, h:h + 1] if n == "dO" else t[b, h:h + 1] for b, h in pairs])
    return out


def to_f64(t):
    """Exact upcast of a (quantised) CPU/GPU tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
