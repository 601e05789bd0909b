/*
 * gdr2_oracle.c -- fp64 CPU oracle for the Gated DeltaNet-2 state recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP library is checked against.  Only the tests, the smoke entry point and
 * the CPU-baseline leg of the benchmark may load it; the library itself never
 * links, loads or calls it, and it shares no code with the library.
 *
 * Sources (cited by page title and section):
 *   [GDN2]  "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리"
 *           (juhoplayground.github.io), section "Gated Delta Rule-2 업데이트
 *           수식" (the update equation and its symbol table).
 *   [SDM]   "[논문리뷰] Sparse Delta Memory: Scaling the State of Linear RNNs
 *           through Sparsity", section 3 "Method & Key Results" (a learned
 *           initial memory M_0: the optional initial state S0 below).
 *   [MC]    "Memory Caching(MC): 길이에 따라 메모리가 커지는 RNN에 대한 연구",
 *           section "체크포인트를 캐싱할까, 독립 압축기를 쓸까?" (a segment
 *           starts from the previous segment's final state: S_final of one
 *           call is the S0 of the next).
 *
 * What is computed, for every (batch b, head h) independently, strictly one
 * token after another (this is the plain definition; nothing is blocked,
 * fused or reordered):
 *
 *   [GDN2, update equation]
 *     S_t = (I - k_t (b_t . k_t)^T) D_t S_{t-1} + k_t (w_t . v_t)^T
 *   with S_t a d_k x d_v matrix, D_t = diag(exp(g_t)) a per-key-channel
 *   decay given as its logarithm g_t, b_t a per-key-channel erase gate,
 *   w_t a per-value-channel write gate ('.' is the elementwise product).
 *   Expanding the product in the order printed (decay first, then erase):
 *     S'  = D_t S_{t-1}
 *     r   = S'^T (b_t . k_t)           (what the erase removes, per value ch.)
 *     S_t = S' + k_t (w_t . v_t - r)^T
 *   Readout (the pages give none; the standard linear-attention convention):
 *     o_t = S_t^T q_t                  (after the update, no scaling)
 *
 * Gate widths: b has width 1 or d_k, w width 1 or d_v, g width 1 or d_k.
 * A width-1 gate is one scalar per (token, head), broadcast over its channels
 * ([GDN2, update equation]: tying b = w to one scalar gives KDA, and a scalar
 * decay on top gives Gated DeltaNet).
 *
 * Layouts (all row-major, contiguous, float64):
 *   q, k    [B, T, H, d_k]        v        [B, T, H, d_v]
 *   b       [B, T, H, bw]         w        [B, T, H, ww]
 *   g       [B, T, H, gw]         o        [B, T, H, d_v]
 *   S0, S_out [B, H, d_k, d_v]    (S0 may be NULL: zero initial state;
 *                                  S_out may be NULL or equal to S0)
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC -std=c11 gdr2_oracle.c -lm
 * (no -ffast-math, no intrinsics).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence for one head, in place on S (d_k x d_v). */
static void gdr2_token(long dk, long dv, double *S, double *r,
                       const double *q, const double *k, const double *v,
                       const double *b, long bw, const double *w, long ww,
                       const double *g, long gw, double *o)
{
    long i, j;
    /* S' = D_t S_{t-1}: row i (key channel i) is scaled by exp(g_t[i]). */
    for (i = 0; i < dk; ++i) {
        double d = exp(gw == 1 ? g[0] : g[i]);
        for (j = 0; j < dv; ++j)
            S[i * dv + j] *= d;
    }
    /* r = S'^T (b_t . k_t): the old memory read through the erase-weighted key. */
    for (j = 0; j < dv; ++j)
        r[j] = 0.0;
    for (i = 0; i < dk; ++i) {
        double e = (bw == 1 ? b[0] : b[i]) * k[i];
        for (j = 0; j < dv; ++j)
            r[j] += e * S[i * dv + j];
    }
    /* S_t = S' - k_t r^T + k_t (w_t . v_t)^T. */
    for (i = 0; i < dk; ++i) {
        for (j = 0; j < dv; ++j) {
            double u = (ww == 1 ? w[0] : w[j]) * v[j];
            S[i * dv + j] += k[i] * (u - r[j]);
        }
    }
    /* o_t = S_t^T q_t. */
    for (j = 0; j < dv; ++j)
        o[j] = 0.0;
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            o[j] += q[i] * S[i * dv + j];
}

/*
 * The forward.  every > 0 and S_ckpt non-NULL also record checkpoints
 * ([MC], section "체크포인트를 캐싱할까, 독립 압축기를 쓸까?": the memory
 * at segment boundaries): S_ckpt [B, H, ceil(T/every), d_k, d_v] receives
 * the state before token n*every, for every n (entry 0 is the initial state).
 * Returns 0 on success, -1 on bad arguments, -2 when memory runs out.
 * threads <= 0 keeps the OpenMP default.
 */
static int forward_impl(long B, long T, long H, long dk, long dv,
                        const double *q, const double *k, const double *v,
                        const double *b, long bw, const double *w, long ww,
                        const double *g, long gw, const double *S0,
                        double *o, double *S_out, long every, double *S_ckpt, int threads)
{
    long bh, n_bh = B * H;
    int failed = 0;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (!(bw == 1 || bw == dk) || !(ww == 1 || ww == dv) || !(gw == 1 || gw == dk))
        return -1;
    if (T > 0 && (!q || !k || !v || !b || !w || !g || !o))
        return -1;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif

#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
    for (bh = 0; bh < n_bh; ++bh) {
        long bi = bh / H, h = bh % H, t;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !r) {
            free(S);
            free(r);
            failed = 1;
            continue;
        }
        if (S0)
            memcpy(S, S0 + bh * dk * dv, sizeof(double) * (size_t)(dk * dv));
        else
            memset(S, 0, sizeof(double) * (size_t)(dk * dv));
        for (t = 0; t < T; ++t) {
            long row = (bi * T + t) * H + h; /* token row in [B, T, H, .] */
            if (S_ckpt && t % every == 0) {
                long nck = (T + every - 1) / every;
                memcpy(S_ckpt + (bh * nck + t / every) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
            }
            gdr2_token(dk, dv, S, r,
                       q + row * dk, k + row * dk, v + row * dv,
                       b + row * bw, bw, w + row * ww, ww,
                       g + row * gw, gw, o + row * dv);
        }
        if (S_out)
            memcpy(S_out + bh * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
        free(r);
    }
    return failed ? -2 : 0;
}

int gdr2_oracle_forward(long B, long T, long H, long dk, long dv,
                        const double *q, const double *k, const double *v,
                        const double *b, long bw, const double *w, long ww,
                        const double *g, long gw, const double *S0,
                        double *o, double *S_out, int threads)
{
    return forward_impl(B, T, H, dk, dv, q, k, v, b, bw, w, ww, g, gw, S0, o, S_out, 0, NULL, threads);
}

int gdr2_oracle_forward_ckpt(long B, long T, long H, long dk, long dv,
                             const double *q, const double *k, const double *v,
                             const double *b, long bw, const double *w, long ww,
                             const double *g, long gw, const double *S0,
                             double *o, double *S_out, long every, double *S_ckpt, int threads)
{
    if (every <= 0 || !S_ckpt)
        return -1;
    return forward_impl(B, T, H, dk, dv, q, k, v, b, bw, w, ww, g, gw, S0, o, S_out, every, S_ckpt, threads);
}

/*
 * Gradients of a scalar loss L through the forward, given dO = dL/do
 * [B, T, H, d_v] and dS_final = dL/dS_T [B, H, d_k, d_v] (NULL: zero).
 * Outputs dq, dk [B,T,H,d_k], dv [B,T,H,d_v], db [B,T,H,bw], dw [B,T,H,ww],
 * dg [B,T,H,gw] and dS0 [B,H,d_k,d_v] (dS0 may be NULL).  A width-1 gate's
 * gradient is the sum over the channels it is broadcast to.
 *
 * The reverse sweep walks the same per-token steps as gdr2_token backwards
 * (chain rule, one step at a time), with Lam = dL/dS_t:
 *   o_t = S_t^T q_t              ->  dq_t = S_t dO_t,  Lam += q_t dO_t^T
 *   S_t = S' + k_t (u - r)^T     ->  c = Lam^T k_t (= dL/du = -dL/dr),
 *                                    dk_t += Lam (u - r),  dS' = Lam
 *   u = w_t . v_t                ->  dw = c . v_t,  dv = c . w_t
 *   r = S'^T e,  e = b_t . k_t   ->  de = -S' c,  dS' += -e c^T
 *                                    db = de . k_t,  dk_t += de . b_t
 *   S' = D_t S_{t-1}             ->  dg_t[i] = sum_j dS'[i,j] S'[i,j],
 *                                    Lam_{t-1} = D_t dS'
 * S_{t-1} for the sweep comes from a stored copy of every state.
 * Returns 0, -1 (bad arguments) or -2 (out of memory).
 */
int gdr2_oracle_backward(long B, long T, long H, long dk, long dv,
                         const double *q, const double *k, const double *v,
                         const double *b, long bw, const double *w, long ww,
                         const double *g, long gw, const double *S0,
                         const double *dO, const double *dS_final,
                         double *dq, double *dk_out, double *dv_out, double *db,
                         double *dw, double *dg, double *dS0, int threads)
{
    long bh, n_bh = B * H;
    int failed = 0;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (!(bw == 1 || bw == dk) || !(ww == 1 || ww == dv) || !(gw == 1 || gw == dk))
        return -1;
    if (T > 0 && (!q || !k || !v || !b || !w || !g || !dO || !dq || !dk_out || !dv_out || !db ||
                  !dw || !dg))
        return -1;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif

#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
    for (bh = 0; bh < n_bh; ++bh) {
        long bi = bh / H, h = bh % H, t, i, j;
        const size_t ss = (size_t)(dk * dv);
        double *St = (double *)malloc(sizeof(double) * ss * (size_t)(T + 1)); /* S_0 .. S_T */
        double *Lam = (double *)malloc(sizeof(double) * ss);
        double *Sp = (double *)malloc(sizeof(double) * ss);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        double *c = (double *)malloc(sizeof(double) * (size_t)dv);
        double *de = (double *)malloc(sizeof(double) * (size_t)dk);
        double *ot = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!St || !Lam || !Sp || !r || !c || !de || !ot) {
            free(St); free(Lam); free(Sp); free(r); free(c); free(de); free(ot);
            failed = 1;
            continue;
        }
        /* forward, keeping every state */
        if (S0)
            memcpy(St, S0 + bh * ss, sizeof(double) * ss);
        else
            memset(St, 0, sizeof(double) * ss);
        for (t = 0; t < T; ++t) {
            long row = (bi * T + t) * H + h;
            memcpy(St + (t + 1) * ss, St + t * ss, sizeof(double) * ss);
            gdr2_token(dk, dv, St + (t + 1) * ss, r, q + row * dk, k + row * dk, v + row * dv,
                       b + row * bw, bw, w + row * ww, ww, g + row * gw, gw, ot);
        }
        /* reverse sweep */
        if (dS_final)
            memcpy(Lam, dS_final + bh * ss, sizeof(double) * ss);
        else
            memset(Lam, 0, sizeof(double) * ss);
        for (t = T - 1; t >= 0; --t) {
            long row = (bi * T + t) * H + h;
            const double *qt = q + row * dk, *kt = k + row * dk, *vt = v + row * dv;
            const double *bt = b + row * bw, *wt = w + row * ww, *gt = g + row * gw;
            const double *dot = dO + row * dv;
            const double *Sn = St + (t + 1) * ss, *Sprev = St + t * ss;
            double *dqt = dq + row * dk, *dkt = dk_out + row * dk, *dvt = dv_out + row * dv;
            double *dbt = db + row * bw, *dwt = dw + row * ww, *dgt = dg + row * gw;
            /* readout */
            for (i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (j = 0; j < dv; ++j)
                    acc += Sn[i * dv + j] * dot[j];
                dqt[i] = acc;
                for (j = 0; j < dv; ++j)
                    Lam[i * dv + j] += qt[i] * dot[j];
            }
            /* recompute S' = D_t S_{t-1} and r = S'^T e */
            for (i = 0; i < dk; ++i) {
                double d = exp(gw == 1 ? gt[0] : gt[i]);
                for (j = 0; j < dv; ++j)
                    Sp[i * dv + j] = d * Sprev[i * dv + j];
            }
            for (j = 0; j < dv; ++j)
                r[j] = 0.0;
            for (i = 0; i < dk; ++i) {
                double e = (bw == 1 ? bt[0] : bt[i]) * kt[i];
                for (j = 0; j < dv; ++j)
                    r[j] += e * Sp[i * dv + j];
            }
            /* write term: c = Lam^T k, dk = Lam (u - r) */
            for (j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (i = 0; i < dk; ++i)
                    acc += Lam[i * dv + j] * kt[i];
                c[j] = acc;
            }
            for (i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (j = 0; j < dv; ++j) {
                    double u = (ww == 1 ? wt[0] : wt[j]) * vt[j];
                    acc += Lam[i * dv + j] * (u - r[j]);
                }
                dkt[i] = acc;
            }
            /* u = w . v */
            if (ww == 1) {
                double acc = 0.0;
                for (j = 0; j < dv; ++j)
                    acc += c[j] * vt[j];
                dwt[0] = acc;
            } else {
                for (j = 0; j < dv; ++j)
                    dwt[j] = c[j] * vt[j];
            }
            for (j = 0; j < dv; ++j)
                dvt[j] = c[j] * (ww == 1 ? wt[0] : wt[j]);
            /* erase read: de = -S' c; e = b . k */
            for (i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (j = 0; j < dv; ++j)
                    acc += Sp[i * dv + j] * c[j];
                de[i] = -acc;
            }
            if (bw == 1) {
                double acc = 0.0;
                for (i = 0; i < dk; ++i)
                    acc += de[i] * kt[i];
                dbt[0] = acc;
            } else {
                for (i = 0; i < dk; ++i)
                    dbt[i] = de[i] * kt[i];
            }
            for (i = 0; i < dk; ++i)
                dkt[i] += de[i] * (bw == 1 ? bt[0] : bt[i]);
            /* dS' = Lam - e c^T; dg; Lam_{t-1} = D dS' */
            if (gw == 1)
                dgt[0] = 0.0;
            for (i = 0; i < dk; ++i) {
                double e = (bw == 1 ? bt[0] : bt[i]) * kt[i];
                double d = exp(gw == 1 ? gt[0] : gt[i]);
                double acc = 0.0;
                for (j = 0; j < dv; ++j) {
                    double dsp = Lam[i * dv + j] - e * c[j];
                    acc += dsp * Sp[i * dv + j];
                    Lam[i * dv + j] = d * dsp;
                }
                if (gw == 1)
                    dgt[0] += acc;
                else
                    dgt[i] = acc;
            }
        }
        if (dS0)
            memcpy(dS0 + bh * ss, Lam, sizeof(double) * ss);
        free(St); free(Lam); free(Sp); free(r); free(c); free(de); free(ot);
    }
    return failed ? -2 : 0;
}

/*
 * One decode step for N independent sequences x H heads: the same token
 * update applied once per state, in place on state [N, H, d_k, d_v].
 * Token inputs are [N, H, .] (one token each); o is [N, H, d_v].
 */
int gdr2_oracle_decode(long N, long H, long dk, long dv,
                       const double *q, const double *k, const double *v,
                       const double *b, long bw, const double *w, long ww,
                       const double *g, long gw, double *state, double *o,
                       int threads)
{
    if (!state)
        return -1;
    /* A decode step is a forward over T = 1 that starts from and ends in state. */
    return gdr2_oracle_forward(N, 1, H, dk, dv, q, k, v, b, bw, w, ww, g, gw,
                               state, o, state, threads);
}

int gdr2_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
