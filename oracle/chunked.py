"""Chunkwise (WY) evaluation of the Gated DeltaNet-2 recurrence in fp64 NumPy.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): it exists to give the
per-chunk intermediates of the chunked method a plain fp64 definition, so the
GPU stages can be checked one by one.  It is itself checked against the
sequential oracle (tests/test_chunked_blueprint.py).

Source: page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리",
section "효율적 구현" (efficient implementation): fixed-size chunks, and a WY
form that folds the cumulative per-channel decay into the rank-1 erase
factors.  The pages give no formulas for it; the form below is derived from
the update equation of section "Gated Delta Rule-2 업데이트 수식" by
unrolling it over one chunk (the derivation is in the function docstring).

Each step is a plain NumPy expression or library routine (einsum, a matmul,
a unit-lower-triangular solve); there is no further blocking or fusion.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _full(gate, width):
    return np.broadcast_to(gate, gate.shape[:-1] + (width,))


def chunk_step(S, q, k, v, b, w, g):
    """Advance one chunk of L tokens from chunk-start state S (dk x dv).

    Unrolling S_t = D_t S_{t-1} + k_t d_t^T with d_t = w_t*v_t - (D_t S_{t-1})^T e_t,
    e_t = b_t*k_t, over the chunk, with G_t = sum_{r<=t} g_r (per key channel):

      D_t S_{t-1} = diag(e^{G_t}) S + sum_{s<t} diag(e^{G_t-G_s}) k_s d_s^T
      => d_t + sum_{s<t} M[t,s] d_s = u_t - S^T (e_t*e^{G_t})
         M[t,s] = sum_i e_t[i] k_s[i] e^{G_t[i]-G_s[i]}
      => Delta = (I+M)^{-1} U - (I+M)^{-1} E~ S = U~ - W S
      o_t = S_t^T q_t = S^T (q_t*e^{G_t}) + sum_{s<=t} P[t,s] d_s,
         P[t,s] = sum_i q_t[i] k_s[i] e^{G_t[i]-G_s[i]}
      S_next = diag(e^{G_L}) S + K^T Delta,  K^[s] = k_s * e^{G_L-G_s}

    Inputs are [L, .] arrays with full-width gates.  Returns a dict with the
    chunk's intermediates and outputs.
    """
    L, dk = k.shape
    G = np.cumsum(g, axis=0)                                  # [L, dk]
    E = b * k                                                 # erase-weighted keys
    U = w * v                                                 # gated values
    Et = E * np.exp(G)
    Qt = q * np.exp(G)
    Kh = k * np.exp(G[-1][None, :] - G)
    diff = G[:, None, :] - G[None, :, :]                      # [t, s, i] = G_t - G_s
    lower = np.tril(np.ones((L, L), dtype=bool))
    decay = np.exp(np.where(lower[:, :, None], diff, -np.inf))
    M = np.einsum("ti,si,tsi->ts", E, k, decay) * np.tril(np.ones((L, L)), -1)
    P = np.einsum("ti,si,tsi->ts", q, k, decay)
    A = np.eye(L) + M
    W = solve_triangular(A, Et, lower=True, unit_diagonal=True)
    Ut = solve_triangular(A, U, lower=True, unit_diagonal=True)
    Delta = Ut - W @ S
    O = Qt @ S + P @ Delta
    gamma = np.exp(G[-1])
    S_next = gamma[:, None] * S + Kh.T @ Delta
    return dict(G=G, Et=Et, Qt=Qt, Kh=Kh, M=M, P=P, W=W, Ut=Ut, Delta=Delta,
                O=O, gamma=gamma, S_next=S_next)


def forward(q, k, v, b, w, g, S0=None, chunk: int = 64, keep=False):
    """Chunked forward over [B,T,H,.] inputs (any gate widths), fp64.

    Returns (o, S_final) and, with keep=True, a list per (b,h) of the per-chunk
    dicts from ``chunk_step`` (chunk-start states included as 'S').
    """
    q, k, v, b, w, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, b, w, g))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    b, w, g = _full(b, dk), _full(w, dv), _full(g, dk)
    o = np.zeros((B, T, H, dv))
    S_fin = np.zeros((B, H, dk, dv))
    kept = []
    for bi in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)[bi, h].copy()
            per = []
            for c0 in range(0, T, chunk):
                sl = slice(c0, min(T, c0 + chunk))
                r = chunk_step(S, q[bi, sl, h], k[bi, sl, h], v[bi, sl, h],
                               b[bi, sl, h], w[bi, sl, h], g[bi, sl, h])
                o[bi, sl, h] = r["O"]
                if keep:
                    r["S"] = S
                    per.append(r)
                S = r["S_next"]
            S_fin[bi, h] = S
            kept.append(per)
    return (o, S_fin, kept) if keep else (o, S_fin)


def chunk_backward(r, S, q, k, v, b, w, g, dO, Lam_end):
    """Gradients through one chunk (full-width gates), given the chunk's
    forward intermediates r (from ``chunk_step``), its start state S, the
    output gradient dO [L, dv] and the gradient Lam_end of the chunk-end state.

    Chunk level (exact reverse of the chunk form):
      dDelta = P^T dO + K^ Lam_end
      Lam_start = Q~^T dO + diag(gamma) Lam_end - W^T dDelta
      dQ~ = dO S^T, dP = tril(dO Delta^T), dK^ = Delta Lam_end^T,
      dgamma = rowsum(S * Lam_end), dU~ = dDelta, dW = -dDelta S^T
    WY factors (X = (I + M)^-1):
      dX = dU~ U^T + dW E~^T, dU = X^T dU~, dE~ = X^T dW,
      dM = strictly-lower(-X^T dX X^T)
    Decay-weighted Gram and scores (F[t,s,i] = e^{G_t[i]-G_s[i]}):
      dE[t] += sum_s dM[t,s] k_s * F[t,s],  dk[s] += sum_t dM[t,s] E_t * F[t,s]
      dq[t] += sum_s dP[t,s] k_s * F[t,s],  dk[s] += sum_t dP[t,s] q_t * F[t,s]
      dG[t] += E_t * dE_M[t] + q_t * dq_P[t];  dG[s] -= k_s * (dk_M[s] + dk_P[s])
    Decayed vectors: E~ = E e^G, Q~ = q e^G, K^ = k e^{G_L - G}, gamma = e^{G_L};
    G = cumsum(g) so dg is the reverse cumulative sum of dG.
    Returns (Lam_start, dict of dq, dk, dv, db, dw, dg [L, .]).
    """
    L, dk = k.shape
    G, Et, Qt, Kh, M, P, W, Ut, Delta, gamma = (r[n] for n in
                                                 ("G", "Et", "Qt", "Kh", "M", "P", "W", "Ut", "Delta", "gamma"))
    E = b * k
    U = w * v
    dDelta = P.T @ dO + Kh @ Lam_end
    Lam_start = Qt.T @ dO + gamma[:, None] * Lam_end - W.T @ dDelta
    dQt = dO @ S.T
    dP = np.tril(dO @ Delta.T)
    dKh = Delta @ Lam_end.T
    dgamma = (S * Lam_end).sum(axis=1)
    dUt = dDelta
    dW = -dDelta @ S.T
    X = np.linalg.inv(np.eye(L) + M)
    dX = dUt @ U.T + dW @ Et.T
    dU = X.T @ dUt
    dEt = X.T @ dW
    dM = np.tril(-X.T @ dX @ X.T, -1)
    diff = G[:, None, :] - G[None, :, :]
    lower = np.tril(np.ones((L, L), dtype=bool))
    F = np.exp(np.where(lower[:, :, None], diff, -np.inf))            # [t, s, i]
    dE_M = np.einsum("ts,si,tsi->ti", dM, k, F)
    dk_M = np.einsum("ts,ti,tsi->si", dM, E, F)
    dq_P = np.einsum("ts,si,tsi->ti", dP, k, F)
    dk_P = np.einsum("ts,ti,tsi->si", dP, q, F)
    dG = E * dE_M + q * dq_P - k * (dk_M + dk_P)
    eG = np.exp(G)
    dE = dE_M + dEt * eG
    dG += dEt * Et + dQt * Qt - dKh * Kh
    dGL = (dKh * Kh).sum(axis=0) + dgamma * gamma
    dG[-1] += dGL
    dq = dq_P + dQt * eG
    dkk = dk_M + dk_P + dKh * np.exp(G[-1][None, :] - G) + dE * b
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return Lam_start, dict(dq=dq, dk=dkk, dv=dU * w, db=dE * k, dw=dU * v, dg=dg)


def backward(q, k, v, b, w, g, dO, S0=None, dS_final=None, chunk: int = 64):
    """Chunked backward over [B,T,H,.] inputs (any gate widths), fp64:
    a forward that keeps each chunk's start state and intermediates, then a
    reverse sweep over chunks with ``chunk_backward``.  Returns a dict like
    the sequential oracle's backward (width-1 gates summed over channels)."""
    q, k, v, b, w, g, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, b, w, g, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bw, ww, gw = b.shape[-1], w.shape[-1], g.shape[-1]
    bf, wf, gf = _full(b, dk), _full(w, dv), _full(g, dk)
    _, _, kept = forward(q, k, v, b, w, g, S0=S0, chunk=chunk, keep=True)
    out = {n: np.zeros((B, T, H, wd)) for n, wd in
           (("dq", dk), ("dk", dk), ("dv", dv), ("db", dk), ("dw", dv), ("dg", dk))}
    dS0 = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for h in range(H):
            Lam = np.zeros((dk, dv)) if dS_final is None else np.asarray(dS_final, np.float64)[bi, h].copy()
            per = kept[bi * H + h]
            for n in range(len(per) - 1, -1, -1):
                sl = slice(n * chunk, min(T, (n + 1) * chunk))
                Lam, gr = chunk_backward(per[n], per[n]["S"], q[bi, sl, h], k[bi, sl, h], v[bi, sl, h],
                                         bf[bi, sl, h], wf[bi, sl, h], gf[bi, sl, h], dO[bi, sl, h], Lam)
                for name, val in gr.items():
                    out[name][bi, sl, h] = val
            dS0[bi, h] = Lam
    for name, wd in (("db", bw), ("dw", ww), ("dg", gw)):
        if wd == 1:
            out[name] = out[name].sum(axis=-1, keepdims=True)
    out["dS0"] = dS0
    return out
