"""Pins for the fp64 oracle: each function checks the oracle against something
other than itself and returns the worst residual found (0 = exact).

Sources (page titles and sections):
  [GDN2] "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리",
         section "Gated Delta Rule-2 업데이트 수식" (update equation, symbol
         table, the KDA / Gated DeltaNet special cases).
  [DeepMem] "[논문리뷰] Going Deeper With Memories", section 1 (key terms):
         its fast-weight memory is gated linear attention, the erase-free
         (b = 0) case of the update.
  [MC]   "Memory Caching(MC): ...", section "체크포인트를 캐싱할까, 독립
         압축기를 쓸까?": a segment resumes from the previous segment's state.

Every pin is written from mathematics the pages fix (closed forms, special
cases that reduce to textbook routines, invariants, brute force with explicit
matrices), never by calling the oracle's own code path twice.  The mutant test
(test_oracle_mutants.py) plants plausible mistakes in a copy of the C oracle
and checks that at least one pin here catches each of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_problem(rng, B=2, T=5, H=2, dk=6, dv=5, bw=None, ww=None, gw=None,
                 unit_k=True, g_lo=-1.5):
    bw = dk if bw is None else bw
    ww = dv if ww is None else ww
    gw = dk if gw is None else gw
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    b = rng.random((B, T, H, bw))
    w = rng.random((B, T, H, ww))
    g = rng.random((B, T, H, gw)) * g_lo
    return dict(q=q, k=k, v=v, b=b, w=w, g=g)


def _full(x, n):
    return np.broadcast_to(x, x.shape[:-1] + (n,))


def pin_retrieval_identity(lib, seed=1):
    """[GDN2] With |k_t| = 1 and b_t = 1 the erase removes exactly what k_t
    reads, so S_t^T k_t = w_t * v_t for ANY decay and previous state.  With
    w = 1 and D = I this is the plain delta rule's S_t^T k_t = v_t."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (bw, ww, gw) in ((6, 5, 6), (1, 1, 1), (6, 1, 1)):
        p = rand_problem(rng, T=1, bw=bw, ww=ww, gw=gw)
        p["b"] = np.ones_like(p["b"])
        S0 = rng.standard_normal((2, 2, 6, 5))
        _, S = oracle.forward(**p, S0=S0, lib=lib)
        got = np.einsum("bhij,bhi->bhj", S, p["k"][:, 0])
        want = _full(p["w"][:, 0], 5) * p["v"][:, 0]
        worst = max(worst, np.abs(got - want).max())
        # the spec form: b = w = 1, no decay, over several tokens
        p = rand_problem(rng, T=4)
        p["b"][:] = 1.0
        p["w"][:] = 1.0
        p["g"][:] = 0.0
        for t in range(4):
            sub = {n: a[:, : t + 1] for n, a in p.items()}
            _, S = oracle.forward(**sub, S0=S0, lib=lib)
            got = np.einsum("bhij,bhi->bhj", S, p["k"][:, t])
            worst = max(worst, np.abs(got - p["v"][:, t]).max())
    return worst


def pin_one_step_all_gates(lib, seed=2):
    """[GDN2] One step with all gates: with |k| = 1,
    S_t^T k_t = (D_t S_{t-1})^T ((1 - b_t) * k_t) + w_t * v_t.  Distinguishes
    the printed erase k (b*k)^T from its transpose (b*k) k^T."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (bw, ww, gw) in ((6, 5, 6), (1, 1, 1), (1, 5, 6)):
        p = rand_problem(rng, T=1, bw=bw, ww=ww, gw=gw)
        S0 = rng.standard_normal((2, 2, 6, 5))
        _, S = oracle.forward(**p, S0=S0, lib=lib)
        k = p["k"][:, 0]
        DS = np.exp(_full(p["g"][:, 0], 6))[..., None] * S0
        want = np.einsum("bhij,bhi->bhj", DS, (1 - _full(p["b"][:, 0], 6)) * k) \
            + _full(p["w"][:, 0], 5) * p["v"][:, 0]
        got = np.einsum("bhij,bhi->bhj", S, k)
        worst = max(worst, np.abs(got - want).max())
    return worst


def pin_explicit_matrices(lib, seed=3):
    """[GDN2] The equation as printed, with explicit d_k x d_k matrices,
    applied token by token (brute force), for non-unit keys, unequal d_k and
    d_v, and every gate width; also the readout o_t = S_t^T q_t."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (bw, ww, gw) in ((6, 5, 6), (1, 1, 1), (1, 5, 1), (6, 1, 6)):
        p = rand_problem(rng, B=1, T=4, H=2, unit_k=False, bw=bw, ww=ww, gw=gw)
        S0 = rng.standard_normal((1, 2, 6, 5))
        o, S = oracle.forward(**p, S0=S0, lib=lib)
        for h in range(2):
            St = S0[0, h].copy()
            for t in range(4):
                k = p["k"][0, t, h]
                e = _full(p["b"][0, t, h], 6) * k
                A = (np.eye(6) - np.outer(k, e)) @ np.diag(np.exp(_full(p["g"][0, t, h], 6)))
                St = A @ St + np.outer(k, _full(p["w"][0, t, h], 5) * p["v"][0, t, h])
                worst = max(worst, np.abs(o[0, t, h] - St.T @ p["q"][0, t, h]).max())
            worst = max(worst, np.abs(S[0, h] - St).max())
    return worst


def pin_transition_product(lib, seed=4):
    """Brute force, the other association: S_T = (A_T...A_1) S0 +
    sum_t (A_T...A_{t+1}) k_t u_t^T with A_t = (I - k_t e_t^T) D_t."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=1, T=6, H=1, dk=3, dv=4, unit_k=False)
    S0 = rng.standard_normal((1, 1, 3, 4))
    _, S = oracle.forward(**p, S0=S0, lib=lib)
    A = []
    for t in range(6):
        k = p["k"][0, t, 0]
        A.append((np.eye(3) - np.outer(k, p["b"][0, t, 0] * k)) @ np.diag(np.exp(p["g"][0, t, 0])))
    total = np.linalg.multi_dot(A[::-1]) @ S0[0, 0]
    for t in range(6):
        tail = np.eye(3)
        for r in range(t + 1, 6):
            tail = A[r] @ tail
        total += tail @ np.outer(p["k"][0, t, 0], p["w"][0, t, 0] * p["v"][0, t, 0])
    return np.abs(S[0, 0] - total).max()


def pin_linear_attention(lib, seed=5):
    """b = 0, w = 1, g = 0: no erase, no decay -- causal linear attention,
    S_T = S0 + K^T V and O = tril(Q K^T) V + Q S0 (matrix products)."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=2, T=9, H=2, unit_k=False)
    p["b"][:] = 0.0
    p["w"][:] = 1.0
    p["g"][:] = 0.0
    S0 = rng.standard_normal((2, 2, 6, 5))
    o, S = oracle.forward(**p, S0=S0, lib=lib)
    worst = 0.0
    for bi in range(2):
        for h in range(2):
            Q, K, V = p["q"][bi, :, h], p["k"][bi, :, h], p["v"][bi, :, h]
            worst = max(worst, np.abs(S[bi, h] - (S0[bi, h] + K.T @ V)).max())
            worst = max(worst, np.abs(o[bi, :, h] - (np.tril(Q @ K.T) @ V + Q @ S0[bi, h])).max())
    return worst


def pin_gated_linear_attention(lib, seed=6):
    """[DeepMem] b = 0: gated linear attention with per-key-channel decay.
    With G_t = sum_{r<=t} g_r:  o_t = S0^T (q_t e^{G_t}) +
    sum_{s<=t} (w_s v_s) sum_i q_t[i] k_s[i] e^{G_t[i]-G_s[i]}, and
    S_T = diag(e^{G_T}) S0 + sum_s diag(e^{G_T-G_s}) k_s (w_s v_s)^T."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=1, T=7, H=2, unit_k=False)
    p["b"][:] = 0.0
    S0 = rng.standard_normal((1, 2, 6, 5))
    o, S = oracle.forward(**p, S0=S0, lib=lib)
    worst = 0.0
    for h in range(2):
        q, k, g = p["q"][0, :, h], p["k"][0, :, h], p["g"][0, :, h]
        u = p["w"][0, :, h] * p["v"][0, :, h]
        G = np.cumsum(g, axis=0)
        dec = np.exp(G[:, None, :] - G[None, :, :])                     # [t, s, i]
        A = np.einsum("ti,si,tsi->ts", q, k, dec) * np.tril(np.ones((7, 7)))
        want_o = (q * np.exp(G)) @ S0[0, h] + A @ u
        want_S = np.exp(G[-1])[:, None] * S0[0, h] + (k * np.exp(G[-1] - G)).T @ u
        worst = max(worst, np.abs(o[0, :, h] - want_o).max(), np.abs(S[0, h] - want_S).max())
    return worst


def pin_gdn_special_cases(lib, seed=7):
    """[GDN2] Tying b = w = beta (scalar) gives KDA; a scalar decay alpha on top
    gives Gated DeltaNet.  Checked against those models' own update forms:
      GDN: S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
      KDA: S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T"""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for kind in ("gdn", "kda"):
        p = rand_problem(rng, B=1, T=6, H=2, bw=1, ww=1, gw=1 if kind == "gdn" else 6)
        p["w"] = p["b"].copy()
        S0 = rng.standard_normal((1, 2, 6, 5))
        o, S = oracle.forward(**p, S0=S0, lib=lib)
        for h in range(2):
            St = S0[0, h].copy()
            for t in range(6):
                k, v, q = p["k"][0, t, h], p["v"][0, t, h], p["q"][0, t, h]
                beta = p["b"][0, t, h, 0]
                alpha = np.exp(p["g"][0, t, h])
                if kind == "gdn":
                    St = alpha[0] * (St - beta * np.outer(k, k @ St)) + beta * np.outer(k, v)
                else:
                    St = alpha[:, None] * St
                    St = St - beta * np.outer(k, k @ St) + beta * np.outer(k, v)
                worst = max(worst, np.abs(o[0, t, h] - St.T @ q).max())
            worst = max(worst, np.abs(S[0, h] - St).max())
    return worst


def pin_zero_decay(lib, seed=8):
    """D_t = 0 (g = -inf) forgets everything: S_t = k_t (w_t v_t)^T and
    o_t = (w_t v_t)(k_t . q_t), whatever came before."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=1, T=3, H=2, unit_k=False)
    p["g"][:] = -np.inf
    S0 = rng.standard_normal((1, 2, 6, 5))
    o, S = oracle.forward(**p, S0=S0, lib=lib)
    u = p["w"] * p["v"]
    want_o = u * np.einsum("bthi,bthi->bth", p["k"], p["q"])[..., None]
    want_S = np.einsum("bhi,bhj->bhij", p["k"][:, -1], u[:, -1])
    return max(np.abs(o - want_o).max(), np.abs(S - want_S).max())


def pin_linearity_and_columns(lib, seed=9):
    """For fixed k, b, g the outputs are jointly linear in (S0, w*v); and the
    d_v columns evolve independently (permuting them permutes the outputs).
    Returns a relative residual."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=1, T=6, H=2)
    S0a, S0b = rng.standard_normal((2, 1, 2, 6, 5))
    va, vb = p["v"], rng.standard_normal(p["v"].shape)
    oa, Sa = oracle.forward(**{**p, "v": va}, S0=S0a, lib=lib)
    ob, Sb = oracle.forward(**{**p, "v": vb}, S0=S0b, lib=lib)
    oc, Sc = oracle.forward(**{**p, "v": va + 2.5 * vb}, S0=S0a + 2.5 * S0b, lib=lib)
    scale = max(np.abs(oc).max(), np.abs(Sc).max(), 1.0)
    worst = max(np.abs(oc - (oa + 2.5 * ob)).max(), np.abs(Sc - (Sa + 2.5 * Sb)).max()) / scale
    perm = rng.permutation(5)
    op, Sp = oracle.forward(**{**p, "v": va[..., perm], "w": p["w"][..., perm]},
                            S0=S0a[..., perm], lib=lib)
    worst = max(worst, np.abs(op - oa[..., perm]).max() / scale,
                np.abs(Sp - Sa[..., perm]).max() / scale)
    return worst


def pin_segment_chaining(lib, seed=10):
    """[MC] Running x[:T1] from S0 and then x[T1:] from the state it ends in
    reproduces one run over x (bit for bit: the same operations in the same
    order).  A missing S0 means a zero state."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=2, T=11, H=2)
    S0 = rng.standard_normal((2, 2, 6, 5))
    o, S = oracle.forward(**p, S0=S0, lib=lib)
    worst = 0.0
    for T1 in (0, 1, 4, 11):
        o1, S1 = oracle.forward(**{n: a[:, :T1] for n, a in p.items()}, S0=S0, lib=lib)
        o2, S2 = oracle.forward(**{n: a[:, T1:] for n, a in p.items()}, S0=S1, lib=lib)
        worst = max(worst, np.abs(np.concatenate([o1, o2], axis=1) - o).max(),
                    np.abs(S2 - S).max())
    oz, Sz = oracle.forward(**p, S0=np.zeros_like(S0), lib=lib)
    on, Sn = oracle.forward(**p, S0=None, lib=lib)
    worst = max(worst, np.abs(oz - on).max(), np.abs(Sz - Sn).max())
    return worst


def pin_hand_example(lib):
    """The hand-worked two-token example in tests/golden/hand_example_d2.json."""
    with open(os.path.join(GOLDEN, "hand_example_d2.json")) as f:
        ex = json.load(f)
    inp = ex["inputs"]
    arr = {}
    for n in ("q", "k", "v", "b", "w", "g"):
        rows = [[math.log(0.5) if x == "ln0.5" else float(x) for x in r] for r in inp[n]]
        arr[n] = np.array(rows)[None, :, None, :]            # [B=1, T=2, H=1, 2]
    o, S = oracle.forward(**arr, lib=lib)
    want_o = np.array(ex["expected"]["o"])
    want_S = np.array(ex["expected"]["S_final"])
    return max(np.abs(o[0, :, 0] - want_o).max(), np.abs(S[0, 0] - want_S).max())


def pin_decode_is_one_token(lib, seed=11):
    """The decode step is the update applied once per state: compared with the
    explicit matrix form for each (sequence, head)."""
    rng = np.random.default_rng(seed)
    N, H, dk, dv = 3, 2, 6, 5
    p = rand_problem(rng, B=N, T=1, H=H, unit_k=False)
    state = rng.standard_normal((N, H, dk, dv))
    want = state.copy()
    o = oracle.decode_step(state, *(p[n][:, 0] for n in ("q", "k", "v", "b", "w", "g")), lib=lib)
    worst = 0.0
    for n in range(N):
        for h in range(H):
            k = p["k"][n, 0, h]
            A = (np.eye(dk) - np.outer(k, p["b"][n, 0, h] * k)) @ np.diag(np.exp(p["g"][n, 0, h]))
            St = A @ want[n, h] + np.outer(k, p["w"][n, 0, h] * p["v"][n, 0, h])
            worst = max(worst, np.abs(state[n, h] - St).max(),
                        np.abs(o[n, h] - St.T @ p["q"][n, 0, h]).max())
    return worst


def pin_checkpoints_are_prefix_states(lib, seed=12):
    """[MC] The checkpoint at segment boundary n is the state a run over the
    first n*every tokens ends in (bit for bit), checkpoint 0 is S0, and the
    run's own outputs are unchanged by recording checkpoints."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=2, T=13, H=2)
    S0 = rng.standard_normal((2, 2, 6, 5))
    o, S = oracle.forward(**p, S0=S0, lib=lib)
    worst = 0.0
    for every in (1, 4, 13, 20):
        oc, Sc, ck = oracle.forward_checkpoints(**p, every=every, S0=S0, lib=lib)
        assert ck.shape[2] == -(-13 // every)
        worst = max(worst, np.abs(oc - o).max(), np.abs(Sc - S).max(), np.abs(ck[:, :, 0] - S0).max())
        for n in range(ck.shape[2]):
            _, Sn = oracle.forward(**{m: a[:, :n * every] for m, a in p.items()}, S0=S0, lib=lib)
            worst = max(worst, np.abs(ck[:, :, n] - Sn).max())
    return worst


def _loss(p, S0, dO, dSf, lib):
    o, S = oracle.forward(**p, S0=S0, lib=lib)
    return float((o * dO).sum() + (S * dSf).sum())


def pin_backward_finite_differences(lib, seed=13):
    """The backward against central finite differences of the loss
    L = <dO, o> + <dS_final, S_final> through the oracle forward, for every
    input (q, k, v, b, w, g, S0) and every gate width: an independent check
    of the chain rule (a dropped term, a wrong sign or a transposed operand
    in the backward changes some derivative by O(1))."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for bw, ww, gw in ((None, None, None), (1, 1, 1), (None, 1, None), (1, None, 1)):
        p = rand_problem(rng, B=1, T=6, H=2, dk=4, dv=3, bw=bw, ww=ww, gw=gw)
        S0 = rng.standard_normal((1, 2, 4, 3))
        dO = rng.standard_normal((1, 6, 2, 3))
        dSf = rng.standard_normal((1, 2, 4, 3))
        gr = oracle.backward(**p, dO=dO, S0=S0, dS_final=dSf, lib=lib)
        grads = {"q": gr["dq"], "k": gr["dk"], "v": gr["dv"], "b": gr["db"], "w": gr["dw"],
                 "g": gr["dg"], "S0": gr["dS0"]}
        h = 1e-6
        for name, an in grads.items():
            base = S0 if name == "S0" else p[name]
            fd = np.zeros_like(base)
            for idx in np.ndindex(base.shape):
                x = base.copy()
                x[idx] += h
                lp = _loss(p if name == "S0" else {**p, name: x}, x if name == "S0" else S0, dO, dSf, lib)
                x[idx] -= 2 * h
                lm = _loss(p if name == "S0" else {**p, name: x}, x if name == "S0" else S0, dO, dSf, lib)
                fd[idx] = (lp - lm) / (2 * h)
            worst = max(worst, float(np.abs(fd - an).max() / max(np.abs(fd).max(), 1.0)))
    return worst


def pin_backward_linear_attention(lib, seed=14):
    """b = 0, w = 1, g = 0 (plain linear attention, o_t = S0^T q_t +
    sum_{s<=t} (q_t . k_s) v_s): the closed-form gradients
    dq_t = S0 dO_t + sum_{s<=t} k_s (v_s . dO_t), dv_s = sum_{t>=s} (q_t . k_s) dO_t,
    dk_s = sum_{t>=s} q_t (v_s . dO_t), dS0 = sum_t q_t dO_t^T."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=2, T=7, H=2, dk=5, dv=4)
    p["b"] = np.zeros_like(p["b"])
    p["w"] = np.ones_like(p["w"])
    p["g"] = np.zeros_like(p["g"])
    S0 = rng.standard_normal((2, 2, 5, 4))
    dO = rng.standard_normal((2, 7, 2, 4))
    gr = oracle.backward(**p, dO=dO, S0=S0, lib=lib)
    q, k, v = p["q"], p["k"], p["v"]
    worst = 0.0
    for bi in range(2):
        for h in range(2):
            Q, K, V, G = q[bi, :, h], k[bi, :, h], v[bi, :, h], dO[bi, :, h]
            Lt = np.tril(np.ones((7, 7)))
            A = (Q @ K.T) * Lt                  # A[t,s] = q_t . k_s, s <= t
            dq = G @ S0[bi, h].T + ((G @ V.T) * Lt) @ K
            dv = A.T @ G
            dk = ((G @ V.T) * Lt).T @ Q
            dS0 = Q.T @ G
            worst = max(worst, np.abs(gr["dq"][bi, :, h] - dq).max(), np.abs(gr["dv"][bi, :, h] - dv).max(),
                        np.abs(gr["dk"][bi, :, h] - dk).max(), np.abs(gr["dS0"][bi, h] - dS0).max())
    return worst


def pin_prologue_normalised_retrieval(lib, seed=15):
    """[GDN2] takes the key L2-normalised.  With the prologue's NORM_QK bit a
    raw key of any length behaves as the unit key: b = 1 makes the erase
    remove exactly what the key reads, so S_t^T k^_t = w_t * v_t (up to the
    epsilon's relative 1e-6 / |k|^2), and the readout of q equals that of
    q / |q|.  Without the bit the identity fails for |k| != 1."""
    from oracle import prologue as pro
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, B=2, T=5, H=2, unit_k=False)
    p["k"] *= 3.0                     # |k| ~ 3 * sqrt(dk): far from unit length
    p["b"] = np.ones_like(p["b"])
    S0 = rng.standard_normal((2, 2, 6, 5))
    worst = 0.0
    for T in range(1, 6):
        sub = {m: a[:, :T] for m, a in p.items()}
        o, S = oracle.forward(**sub, S0=S0, lib=lib, prologue=pro.NORM_QK)
        kT = sub["k"][:, T - 1]
        kn = kT / np.sqrt((kT * kT).sum(-1, keepdims=True) + pro.NORM_EPS)
        lhs = np.einsum("bhij,bhi->bhj", S, kn)
        rhs = sub["w"][:, T - 1] * sub["v"][:, T - 1]
        worst = max(worst, np.abs(lhs - rhs).max() / 1e-6)      # scaled: a 1e-6 residual is the epsilon
        # readout of the raw q equals the readout through the normalised q
        qT = sub["q"][:, T - 1]
        qn = qT / np.sqrt((qT * qT).sum(-1, keepdims=True) + pro.NORM_EPS)
        worst = max(worst, np.abs(o[:, T - 1] - np.einsum("bhij,bhi->bhj", S, qn)).max() / 1e-12)
    _, S = oracle.forward(**p, S0=S0, lib=lib)                 # without the bit: no identity
    lhs = np.einsum("bhij,bhi->bhj", S, p["k"][:, -1] / np.linalg.norm(p["k"][:, -1], axis=-1, keepdims=True))
    assert np.abs(lhs - p["w"][:, -1] * p["v"][:, -1]).max() > 1e-3
    return worst


def pin_prologue_gate_values(lib, seed=16):
    """The GATES bit at points where the activations have closed forms:
    pre-activations 0 give b = w = 1/2 and decay exp(-ln 2) = 1/2; b, w
    pre-activations of -40 give gates of ~4e-18 and a decay pre-activation
    of -40 gives no decay (g ~ -4e-18).  Compared with the plain recurrence
    on those gate values."""
    from oracle import prologue as pro
    rng = np.random.default_rng(seed)
    worst = 0.0
    for bv, wv, gv, b_eff, w_eff, g_eff in ((0.0, 0.0, 0.0, 0.5, 0.5, -np.log(2.0)),
                                             (-40.0, 0.0, -40.0, 0.0, 0.5, 0.0),
                                             (0.0, -40.0, 0.0, 0.5, 0.0, -np.log(2.0))):
        p = rand_problem(rng, B=1, T=6, H=2)
        S0 = rng.standard_normal((1, 2, 6, 5))
        raw = {**p, "b": np.full_like(p["b"], bv), "w": np.full_like(p["w"], wv), "g": np.full_like(p["g"], gv)}
        eff = {**p, "b": np.full_like(p["b"], b_eff), "w": np.full_like(p["w"], w_eff),
               "g": np.full_like(p["g"], g_eff)}
        o1, S1 = oracle.forward(**raw, S0=S0, lib=lib, prologue=pro.GATES)
        o2, S2 = oracle.forward(**eff, S0=S0, lib=lib)
        worst = max(worst, np.abs(o1 - o2).max(), np.abs(S1 - S2).max())
    return worst


def pin_prologue_finite_differences(lib, seed=17):
    """The backward with the prologue (both bits, every gate width) against
    central finite differences of L = <dO, o> + <dS_final, S_final> through
    the prologue and the forward, in the raw inputs."""
    from oracle import prologue as pro
    rng = np.random.default_rng(seed)
    worst = 0.0
    for bw, ww, gw in ((None, None, None), (1, 1, 1), (1, None, 1)):
        p = rand_problem(rng, B=1, T=5, H=1, dk=4, dv=3, bw=bw, ww=ww, gw=gw, unit_k=False)
        p["b"] = rng.standard_normal(p["b"].shape)       # pre-activations
        p["w"] = rng.standard_normal(p["w"].shape)
        p["g"] = rng.standard_normal(p["g"].shape)
        S0 = rng.standard_normal((1, 1, 4, 3))
        dO = rng.standard_normal((1, 5, 1, 3))
        dSf = rng.standard_normal((1, 1, 4, 3))
        gr = oracle.backward(**p, dO=dO, S0=S0, dS_final=dSf, lib=lib, prologue=pro.ALL)

        def loss(pp):
            o, S = oracle.forward(**pp, S0=S0, lib=lib, prologue=pro.ALL)
            return float((o * dO).sum() + (S * dSf).sum())
        h = 1e-6
        for name in ("q", "k", "v", "b", "w", "g"):
            fd = np.zeros_like(p[name])
            for idx in np.ndindex(p[name].shape):
                x = p[name].copy()
                x[idx] += h
                lp = loss({**p, name: x})
                x[idx] -= 2 * h
                lm = loss({**p, name: x})
                fd[idx] = (lp - lm) / (2 * h)
            worst = max(worst, float(np.abs(fd - gr["d" + name]).max() / max(np.abs(fd).max(), 1.0)))
    return worst


ALL_PINS = {
    "retrieval_identity": pin_retrieval_identity,
    "one_step_all_gates": pin_one_step_all_gates,
    "explicit_matrices": pin_explicit_matrices,
    "transition_product": pin_transition_product,
    "linear_attention": pin_linear_attention,
    "gated_linear_attention": pin_gated_linear_attention,
    "gdn_special_cases": pin_gdn_special_cases,
    "zero_decay": pin_zero_decay,
    "linearity_and_columns": pin_linearity_and_columns,
    "segment_chaining": pin_segment_chaining,
    "hand_example": pin_hand_example,
    "decode_is_one_token": pin_decode_is_one_token,
    "checkpoints_are_prefix_states": pin_checkpoints_are_prefix_states,
    "backward_finite_differences": pin_backward_finite_differences,
    "backward_linear_attention": pin_backward_linear_attention,
    "prologue_normalised_retrieval": pin_prologue_normalised_retrieval,
    "prologue_gate_values": pin_prologue_gate_values,
    "prologue_finite_differences": pin_prologue_finite_differences,
}

# Residual bounds: fp64 arithmetic on O(1) values over a few tokens.
TOL = {name: 1e-12 for name in ALL_PINS}
TOL["segment_chaining"] = 0.0           # identical operations in identical order
TOL["checkpoints_are_prefix_states"] = 0.0
TOL["backward_finite_differences"] = 1e-7   # central differences, h = 1e-6, in fp64
TOL["prologue_finite_differences"] = 1e-7
TOL["prologue_normalised_retrieval"] = 1.0   # residuals scaled: epsilon-sized and rounding-sized
TOL["prologue_gate_values"] = 1e-12
TOL["hand_example"] = 1e-14
