// gdr2_backward.hip -- chunked backward of the Gated DeltaNet-2 recurrence
// (page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리": gradients
// of the update of section "Gated Delta Rule-2 업데이트 수식" through the
// chunked form of section "효율적 구현").
//
// Given dO = dL/do and dS_T = dL/dS_final, and the chunk-start states S_n
// the forward recorded (S_chunks), the gradients follow the chunk form
// (G = in-chunk cumulative log-decay, natural units here; E = b*k, U = w*v):
//   chunk level, in reverse:  dDelta = P^T dO + K^ Lam,
//                             Lam_start = Q~^T dO + diag(gamma) Lam - W^T dDelta
//   per chunk:  Delta = U~ - W S, dQ~ = dO S^T, dP = tril(dO Delta^T),
//               dK^ = Delta Lam^T, dgamma = rowsum(S * Lam), dW = -dDelta S^T
//   WY factors (X = (I + M)^-1):  dX = dDelta U^T + dW E~^T,
//               dU = X^T dDelta, dE~ = X^T dW, dM = strict_tril(-X^T dX X^T)
//   decay-weighted Gram / scores, F[t,s,i] = e^{G_t[i] - G_s[i]}:
//               dE_M[t] = sum_s dM[t,s] k_s F,  dk_M[s] = sum_t dM[t,s] E_t F,
//               dq_P[t] = sum_s dP[t,s] k_s F,  dk_P[s] = sum_t dP[t,s] q_t F
//   and the decayed vectors E~ = E e^G, Q~ = q e^G, K^ = k e^{G_L - G},
//   gamma = e^{G_L}; dg is the reverse cumulative sum of dG within a chunk.
//
// Kernels (all fp32 arithmetic; intermediates in a fp32 workspace, one
// record per (sequence, head, chunk)):
//   bwd_prep   one workgroup per chunk: G, E, U, E~, Q~, K^, gamma; M and P
//              pair by pair (every exponent is G_t - G_s for s <= t, so no
//              factor exceeds 1 for decays); X by substitution; W, U~.
//   bwd_dout   dO rows of every chunk into the workspace (zero past T).
//   bwd_scan   per (sequence, head, 32 value columns): the state gradient
//              through the chunks in reverse (columns evolve independently),
//              recording Lam at every chunk end and dDelta.
//   bgemm      batched C = alpha op(A) op(B) + beta C0 over all chunks (LDS
//              tiles, 64x64 per workgroup) for the products above.
//   bwd_decay  per chunk: the decay-weighted sums, dG, dg and the input
//              gradients.
#include "gdr2_device.h"
#include "gdr2_internal.h"

#include <algorithm>

namespace gdr2 {
namespace {

constexpr int BC = 64;           // chunk of the backward
constexpr int NTB = 256;         // threads per workgroup

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t a64(size_t x) { return (x + 63) & ~size_t(63); }

// Workspace: fp32 arrays of nrec records each.  Offsets count floats (each
// array starts on a 256-byte boundary); `total` is in bytes.
struct BwdLayout {
    int64_t nrec;
    // [C][D] per record
    size_t G, E, U, Et, Qt, Kh, W, Ut, Del, dDel, dQt, dKh, dW, dU, dEt, dO;
    // [C][C] per record
    size_t P, X, dP, dX, T1, dM;
    // [D] per record
    size_t gam;
    // [D][D] per record: state gradient at every chunk end
    size_t Lam;
    size_t total;
};

BwdLayout bwd_layout(int64_t B, int64_t H, int64_t T, int D)
{
    BwdLayout L;
    L.nrec = B * H * cdiv(T, BC);
    const size_t cd = a64((size_t)L.nrec * BC * D), cc = a64((size_t)L.nrec * BC * BC);
    const size_t dd = a64((size_t)L.nrec * D * D), d1 = a64((size_t)L.nrec * D);
    size_t o = 0;
    size_t* cds[] = {&L.G, &L.E, &L.U, &L.Et, &L.Qt, &L.Kh, &L.W, &L.Ut, &L.Del, &L.dDel, &L.dQt, &L.dKh,
                     &L.dW, &L.dU, &L.dEt, &L.dO};
    for (size_t* p : cds) {
        *p = o;
        o += cd;
    }
    size_t* ccs[] = {&L.P, &L.X, &L.dP, &L.dX, &L.T1, &L.dM};
    for (size_t* p : ccs) {
        *p = o;
        o += cc;
    }
    L.gam = o;
    o += d1;
    L.Lam = o;
    o += dd;
    L.total = o * sizeof(float);
    return L;
}

struct BwdArgs {
    const void *q, *k, *v, *b, *w;
    const float* g;
    const void* dO;
    const float* S_chunks;
    const float* dS_final;
    float *dq, *dk, *dv, *db, *dw, *dg, *dS0;
    int bw, ww, gw;
    int64_t T, H, NC, nrec;
    float* ws;           // workspace base (fp32)
    BwdLayout L;
};

__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const bf16* p, int64_t i) { return (float)p[i]; }

struct Rec {
    int64_t bh, n, row0;   // row0: element row of token 0 of the chunk in [B,T,H,.]
    int L;
};

__device__ __forceinline__ Rec rec_of(int64_t r, int64_t NC, int64_t T, int64_t H)
{
    Rec x;
    x.bh = r / NC;
    x.n = r - x.bh * NC;
    const int64_t b = x.bh / H, h = x.bh - b * H, t0 = x.n * BC;
    x.row0 = (b * T + t0) * H + h;
    x.L = (int)min((int64_t)BC, T - t0);
    return x;
}

// ---------------------------------------------------------------------------
// bwd_prep: one workgroup per chunk record.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_prep_kernel(BwdArgs a)
{
    // Rows of the [C][D] tiles are padded to LD floats so that lanes walking
    // down a column hit distinct LDS banks in the pairwise loops.
    constexpr int C = BC, LD = D + 1;
    extern __shared__ __align__(16) float sm[];
    float* sG = sm;                 // [C][LD] cumulative log-decay
    float* sE = sG + C * LD;        // [C][LD] e = b*k, later u
    float* sK = sE + C * LD;        // [C][LD] k, later E~
    float* sQ = sK + C * LD;        // [C][LD] q, later X [C][C]
    float* sM = sQ + C * LD;        // [C][C] M
    const int64_t r = blockIdx.x;
    const Rec rc = rec_of(r, a.NC, a.T, a.H);
    const int tid = threadIdx.x;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* b = (const E*)a.b;
    const E* w = (const E*)a.w;
    float* ws = a.ws;
    const size_t cdo = (size_t)r * C * D, cco = (size_t)r * C * C;

    // raw rows (zero past the chunk's valid length)
    for (int e = tid; e < C * D; e += NTB) {
        const int t = e / D, i = e % D, l = t * LD + i;
        float gv = 0.f, kv = 0.f, qv = 0.f, bv = 0.f, uv = 0.f;
        if (t < rc.L) {
            const int64_t row = rc.row0 + (int64_t)t * a.H;
            gv = a.g[a.gw == 1 ? row : row * D + i];
            kv = ldf(k, row * D + i);
            qv = ldf(q, row * D + i);
            bv = ldf(b, a.bw == 1 ? row : row * D + i);
            uv = ldf(w, a.ww == 1 ? row : row * D + i) * ldf(v, row * D + i);
        }
        sG[l] = gv;
        sK[l] = kv;
        sQ[l] = qv;
        sE[l] = bv * kv;
        ws[a.L.E + cdo + e] = bv * kv;
        ws[a.L.U + cdo + e] = uv;
    }
    __syncthreads();
    // cumulative sum over the chunk, per channel
    for (int i = tid; i < D; i += NTB) {
        float acc = 0.f;
        for (int t = 0; t < C; ++t) {
            acc += sG[t * LD + i];
            sG[t * LD + i] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < C * D; e += NTB) {
        const int t = e / D, i = e % D, l = t * LD + i;
        const float G = sG[l], GL = sG[(C - 1) * LD + i], eg = expf(G);
        ws[a.L.G + cdo + e] = G;
        ws[a.L.Et + cdo + e] = sE[l] * eg;
        ws[a.L.Qt + cdo + e] = sQ[l] * eg;
        ws[a.L.Kh + cdo + e] = sK[l] * expf(GL - G);
        if (t == 0)
            ws[a.L.gam + (size_t)r * D + i] = expf(GL);
    }
    // M (strictly lower) and P (lower), pair by pair; every exponent is
    // G_t - G_s with s <= t
    for (int e = tid; e < C * C; e += NTB) {
        const int t = e / C, s = e % C;
        float m = 0.f, p = 0.f;
        if (s <= t) {
            for (int i = 0; i < D; ++i) {
                const float f = expf(sG[t * LD + i] - sG[s * LD + i]) * sK[s * LD + i];
                m += sE[t * LD + i] * f;
                p += sQ[t * LD + i] * f;
            }
        }
        sM[e] = s < t ? m : 0.f;
        ws[a.L.P + cco + e] = p;
    }
    __syncthreads();
    // X = (I + M)^-1 by forward substitution, one column per thread (into sQ)
    float* sX = sQ;
    if (tid < C) {
        const int j = tid;
        for (int rr = 0; rr < C; ++rr) {
            float acc = rr == j ? 1.f : 0.f;
            for (int c = j; c < rr; ++c)
                acc -= sM[rr * C + c] * sX[c * C + j];
            sX[rr * C + j] = acc;
        }
    }
    // E~ into sK, u into sE
    for (int e = tid; e < C * D; e += NTB) {
        const int l = (e / D) * LD + e % D;
        sK[l] = sE[l] * expf(sG[l]);
        sE[l] = ws[a.L.U + cdo + e];
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += NTB)
        ws[a.L.X + cco + e] = sX[e];
    // W = X E~, U~ = X u (X is lower triangular)
    for (int e = tid; e < C * D; e += NTB) {
        const int t = e / D, i = e % D;
        float wv = 0.f, uv = 0.f;
        for (int s = 0; s <= t; ++s) {
            const float x = sX[t * C + s];
            wv += x * sK[s * LD + i];
            uv += x * sE[s * LD + i];
        }
        ws[a.L.W + cdo + e] = wv;
        ws[a.L.Ut + cdo + e] = uv;
    }
}

// dO rows of every chunk as fp32 [C][D] records (zero past T).
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_dout_kernel(BwdArgs a)
{
    const int64_t r = blockIdx.x;
    const Rec rc = rec_of(r, a.NC, a.T, a.H);
    const E* dO = (const E*)a.dO;
    float* out = a.ws + a.L.dO + (size_t)r * BC * D;
    for (int e = threadIdx.x; e < BC * D; e += NTB) {
        const int t = e / D, j = e % D;
        out[e] = t < rc.L ? ldf(dO, (rc.row0 + (int64_t)t * a.H) * D + j) : 0.f;
    }
}

// ---------------------------------------------------------------------------
// bwd_scan: state gradient through the chunks in reverse, per (sequence,
// head, 32 value columns).  Lam [D][32] lives in LDS.
// ---------------------------------------------------------------------------
constexpr int SV = 32;   // value columns per workgroup

template <int D>
__global__ __launch_bounds__(NTB) void bwd_scan_kernel(BwdArgs a)
{
    constexpr int C = BC;
    extern __shared__ __align__(16) float sm[];
    float* sLam = sm;                // [D][SV]
    float* sdO = sLam + D * SV;      // [C][SV]
    float* sdD = sdO + C * SV;       // [C][SV]
    float* sP = sdD + C * SV;        // [C][C]
    float* sKh = sP + C * C;         // [C][D]
    float* sQt = sKh + C * D;        // [C][D]
    float* sW = sQt + C * D;         // [C][D]
    float* sGam = sW + C * D;        // [D]
    const int NS = D / SV;
    const int64_t bh = blockIdx.x / NS;
    const int c0 = (int)(blockIdx.x % NS) * SV;
    const int tid = threadIdx.x;
    float* ws = a.ws;

    for (int e = tid; e < D * SV; e += NTB) {
        const int i = e / SV, j = e % SV;
        sLam[e] = a.dS_final ? a.dS_final[(bh * D + i) * D + c0 + j] : 0.f;
    }
    for (int64_t n = a.NC - 1; n >= 0; --n) {
        const int64_t r = bh * a.NC + n;
        const size_t cdo = (size_t)r * C * D, cco = (size_t)r * C * C;
        __syncthreads();
        for (int e = tid; e < C * SV; e += NTB)
            sdO[e] = ws[a.L.dO + cdo + (e / SV) * D + c0 + e % SV];
        for (int e = tid; e < C * C; e += NTB)
            sP[e] = ws[a.L.P + cco + e];
        for (int e = tid; e < C * D; e += NTB) {
            sKh[e] = ws[a.L.Kh + cdo + e];
            sQt[e] = ws[a.L.Qt + cdo + e];
            sW[e] = ws[a.L.W + cdo + e];
        }
        for (int e = tid; e < D; e += NTB)
            sGam[e] = ws[a.L.gam + (size_t)r * D + e];
        __syncthreads();
        // the state gradient at this chunk's end
        for (int e = tid; e < D * SV; e += NTB)
            ws[a.L.Lam + (size_t)r * D * D + (e / SV) * D + c0 + e % SV] = sLam[e];
        // dDelta = P^T dO + K^ Lam
        for (int e = tid; e < C * SV; e += NTB) {
            const int s = e / SV, j = e % SV;
            float acc = 0.f;
            for (int t = s; t < C; ++t)
                acc += sP[t * C + s] * sdO[t * SV + j];
            for (int i = 0; i < D; ++i)
                acc += sKh[s * D + i] * sLam[i * SV + j];
            sdD[e] = acc;
            ws[a.L.dDel + cdo + s * D + c0 + j] = acc;
        }
        __syncthreads();
        // Lam_start = Q~^T dO + gamma Lam - W^T dDelta
        float nl[D * SV / NTB];
#pragma unroll
        for (int u = 0; u < D * SV / NTB; ++u) {
            const int e = u * NTB + tid, i = e / SV, j = e % SV;
            float acc = sGam[i] * sLam[e];
            for (int t = 0; t < C; ++t)
                acc += sQt[t * D + i] * sdO[t * SV + j] - sW[t * D + i] * sdD[t * SV + j];
            nl[u] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < D * SV / NTB; ++u)
            sLam[u * NTB + tid] = nl[u];
    }
    __syncthreads();
    if (a.dS0)
        for (int e = tid; e < D * SV; e += NTB)
            a.dS0[(bh * D + e / SV) * D + c0 + e % SV] = sLam[e];
}

// ---------------------------------------------------------------------------
// bgemm: Cz = alpha * op(Az) * op(Bz) + beta * C0z for every record z.
// op(X) is X or X^T of a row-major matrix with leading dimension ld.  M, N,
// K are multiples of 64 / 16.  mask: 0 none, 1 keep n <= m, 2 keep n < m.
// ---------------------------------------------------------------------------
struct GemmOp {
    const float* p;
    int64_t bs;      // elements between records
    int ld;
    int trans;
};

__global__ __launch_bounds__(NTB) void bgemm_kernel(int M, int N, int K, GemmOp A, GemmOp B, float* Cp,
                                                    int64_t cbs, int ldc, float alpha, float beta,
                                                    const float* C0, int64_t c0bs, int mask)
{
    __shared__ float sA[16][64 + 4];   // [k][m]
    __shared__ float sB[16][64 + 4];   // [k][n]
    const int tiles_n = N / 64, tiles = (M / 64) * tiles_n;
    const int64_t z = blockIdx.x / tiles;
    const int tile = (int)(blockIdx.x - z * tiles);
    const int m0 = (tile / tiles_n) * 64, n0 = (tile % tiles_n) * 64;
    const int tid = threadIdx.x, tm = tid / 16, tn = tid % 16;
    const float* Ap = A.p + z * A.bs;
    const float* Bp = B.p + z * B.bs;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        for (int e = tid; e < 16 * 64; e += NTB) {
            int kk, mm;
            if (A.trans) {             // op(A)(m, k) = A[k][m]: read rows of A
                kk = e / 64; mm = e % 64;
                sA[kk][mm] = Ap[(int64_t)(k0 + kk) * A.ld + m0 + mm];
            } else {                   // A[m][k]
                mm = e / 16; kk = e % 16;
                sA[kk][mm] = Ap[(int64_t)(m0 + mm) * A.ld + k0 + kk];
            }
            int nn;
            if (B.trans) {             // op(B)(k, n) = B[n][k]
                nn = e / 16; kk = e % 16;
                sB[kk][nn] = Bp[(int64_t)(n0 + nn) * B.ld + k0 + kk];
            } else {                   // B[k][n]
                kk = e / 64; nn = e % 64;
                sB[kk][nn] = Bp[(int64_t)(k0 + kk) * B.ld + n0 + nn];
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = sA[kk][tm * 4 + i];
                bv[i] = sB[kk][tn * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] += av[i] * bv[j];
        }
        __syncthreads();
    }
    float* Cz = Cp + z * cbs;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + tm * 4 + i, n = n0 + tn * 4 + j;
            float val = alpha * acc[i][j];
            if (C0)
                val += beta * C0[z * c0bs + (int64_t)m * ldc + n];
            if ((mask == 1 && n > m) || (mask == 2 && n >= m))
                val = 0.f;
            Cz[(int64_t)m * ldc + n] = val;
        }
}

// ---------------------------------------------------------------------------
// bwd_decay: per chunk, the decay-weighted sums and the input gradients.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_decay_kernel(BwdArgs a)
{
    constexpr int C = BC;
    extern __shared__ __align__(16) float sm[];
    float* sG = sm;                 // [C][D]
    float* sE = sG + C * D;         // [C][D] e
    float* sK = sE + C * D;         // [C][D] k
    float* sQ = sK + C * D;         // [C][D] q, later dG
    float* sGL = sQ + C * D;        // [D] dG_L
    const int64_t r = blockIdx.x;
    const Rec rc = rec_of(r, a.NC, a.T, a.H);
    const int tid = threadIdx.x;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* b = (const E*)a.b;
    const E* w = (const E*)a.w;
    const float* ws = a.ws;
    const size_t cdo = (size_t)r * C * D, cco = (size_t)r * C * C;
    const float* dM = ws + a.L.dM + cco;
    const float* dP = ws + a.L.dP + cco;

    for (int e = tid; e < C * D; e += NTB) {
        const int t = e / D;
        float kv = 0.f, qv = 0.f;
        if (t < rc.L) {
            const int64_t row = rc.row0 + (int64_t)t * a.H;
            kv = ldf(k, row * D + e % D);
            qv = ldf(q, row * D + e % D);
        }
        sG[e] = ws[a.L.G + cdo + e];
        sE[e] = ws[a.L.E + cdo + e];
        sK[e] = kv;
        sQ[e] = qv;
    }
    // dG_L = sum_s dK^ K^ + dgamma gamma, with dgamma = rowsum(S * Lam)
    for (int i = tid; i < D; i += NTB) {
        const float* S = a.S_chunks + (size_t)r * D * D + (size_t)i * D;
        const float* Lam = ws + a.L.Lam + (size_t)r * D * D + (size_t)i * D;
        float dgam = 0.f;
        for (int j = 0; j < D; ++j)
            dgam += S[j] * Lam[j];
        float acc = dgam * ws[a.L.gam + (size_t)r * D + i];
        for (int s = 0; s < C; ++s)
            acc += ws[a.L.dKh + cdo + s * D + i] * ws[a.L.Kh + cdo + s * D + i];
        sGL[i] = acc;
    }
    __syncthreads();
    // per (row, channel): the four decay-weighted sums
    constexpr int PER = C * D / NTB;
    float dEm[PER], dqp[PER], dkm[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = u * NTB + tid, t = e / D, i = e % D;
        const float Gt = sG[e];
        float a1 = 0.f, a2 = 0.f, b1 = 0.f;
        for (int s = 0; s <= t; ++s) {           // as the later token t
            const float f = expf(Gt - sG[s * D + i]) * sK[s * D + i];
            a1 += (s < t ? dM[t * C + s] : 0.f) * f;
            a2 += dP[t * C + s] * f;
        }
        for (int t2 = t; t2 < C; ++t2) {          // as the earlier token (s = t)
            const float f = expf(sG[t2 * D + i] - Gt);
            b1 += ((t2 > t ? dM[t2 * C + t] * sE[t2 * D + i] : 0.f) + dP[t2 * C + t] * sQ[t2 * D + i]) * f;
        }
        dEm[u] = a1;
        dqp[u] = a2;
        dkm[u] = b1;
    }
    __syncthreads();
    // dG into sQ (q is read again from the inputs below)
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = u * NTB + tid, t = e / D, i = e % D;
        const float kv = sK[e];
        const int64_t row = rc.row0 + (int64_t)t * a.H;
        const float qv = t < rc.L ? ldf(q, row * D + i) : 0.f;
        float dG = sE[e] * dEm[u] + qv * dqp[u] - kv * dkm[u];
        dG += ws[a.L.dEt + cdo + e] * ws[a.L.Et + cdo + e] + ws[a.L.dQt + cdo + e] * ws[a.L.Qt + cdo + e] -
              ws[a.L.dKh + cdo + e] * ws[a.L.Kh + cdo + e];
        if (t == rc.L - 1)
            dG += sGL[i];
        sQ[e] = dG;
    }
    __syncthreads();
    // dg: reverse cumulative sum over the chunk, per channel
    for (int i = tid; i < D; i += NTB) {
        float acc = 0.f;
        for (int t = C - 1; t >= 0; --t) {
            acc += sQ[t * D + i];
            sQ[t * D + i] = acc;
        }
    }
    __syncthreads();
    // input gradients for valid rows; width-1 gates sum over channels
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = u * NTB + tid, t = e / D, i = e % D;
        if (t >= rc.L)
            continue;
        const int64_t row = rc.row0 + (int64_t)t * a.H, off = row * D + i;
        const float G = sG[e], GL = sG[(C - 1) * D + i], eg = expf(G);
        const float bv = ldf(b, a.bw == 1 ? row : off);
        const float dE = dEm[u] + ws[a.L.dEt + cdo + e] * eg;
        const float dU = ws[a.L.dU + cdo + e];
        a.dq[off] = dqp[u] + ws[a.L.dQt + cdo + e] * eg;
        a.dk[off] = dkm[u] + ws[a.L.dKh + cdo + e] * expf(GL - G) + dE * bv;
        a.dv[off] = dU * ldf(w, a.ww == 1 ? row : off);
        const float dbv = dE * sK[e], dwv = dU * ldf(v, off), dgv = sQ[e];
        if (a.bw == 1)
            atomicAdd(a.db + row, dbv);
        else
            a.db[off] = dbv;
        if (a.ww == 1)
            atomicAdd(a.dw + row, dwv);
        else
            a.dw[off] = dwv;
        if (a.gw == 1)
            atomicAdd(a.dg + row, dgv);
        else
            a.dg[off] = dgv;
    }
}

__global__ void zero_kernel(float* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

hipError_t zero_fill(float* p, int64_t n, hipStream_t s)
{
    if (!p || n <= 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 4096);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t gemm(hipStream_t s, int64_t nrec, int M, int N, int K, GemmOp A, GemmOp B, float* Cp,
                int64_t cbs, int ldc, float alpha, float beta = 0.f, const float* C0 = nullptr,
                int64_t c0bs = 0, int mask = 0)
{
    const int64_t blocks = nrec * (M / 64) * (N / 64);
    hipLaunchKernelGGL(bgemm_kernel, dim3((unsigned)blocks), dim3(NTB), 0, s, M, N, K, A, B, Cp,
                       cbs, ldc, alpha, beta, C0, c0bs, mask);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_backward_t(const gdr2_bwd_args& x, hipStream_t s)
{
    constexpr int C = BC;
    BwdArgs a;
    a.q = x.q; a.k = x.k; a.v = x.v; a.b = x.b; a.w = x.w; a.g = x.g; a.dO = x.dO;
    a.S_chunks = x.S_chunks; a.dS_final = x.dS_final;
    a.dq = x.dq; a.dk = x.dk; a.dv = x.dv; a.db = x.db; a.dw = x.dw; a.dg = x.dg; a.dS0 = x.dS0;
    a.bw = x.b_width; a.ww = x.w_width; a.gw = x.g_width;
    a.T = x.T; a.H = x.H; a.NC = cdiv(x.T, C);
    a.L = bwd_layout(x.B, x.H, x.T, D);
    a.nrec = a.L.nrec;
    a.ws = static_cast<float*>(x.workspace);
    const int64_t nrec = a.nrec, rows = x.B * x.T * x.H;
    hipError_t e;
    // width-1 gate gradients accumulate over channels
    if (a.bw == 1 && (e = zero_fill(a.db, rows, s)) != hipSuccess) return e;
    if (a.ww == 1 && (e = zero_fill(a.dw, rows, s)) != hipSuccess) return e;
    if (a.gw == 1 && (e = zero_fill(a.dg, rows, s)) != hipSuccess) return e;

    const size_t lds_prep = (size_t)(4 * C * (D + 1) + C * C) * 4;
    const size_t lds_scan = (size_t)(D * SV + 2 * C * SV + C * C + 3 * C * D + D) * 4;
    const size_t lds_decay = (size_t)(4 * C * D + D) * 4;
    // more than 64 KiB of dynamic LDS must be requested per kernel
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_prep_kernel<E, D>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_prep)) != hipSuccess ||
        (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_scan_kernel<D>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_scan)) != hipSuccess ||
        (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_decay_kernel<E, D>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_decay)) != hipSuccess)
        return e;

    hipLaunchKernelGGL((bwd_prep_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), lds_prep, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dout_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_scan_kernel<D>), dim3((unsigned)(x.B * x.H * (D / SV))), dim3(NTB), lds_scan, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    float* ws = a.ws;
    const BwdLayout& L = a.L;
    const int64_t CD = (int64_t)C * D, CC = (int64_t)C * C, DD = (int64_t)D * D;
    auto op = [&](size_t off, int64_t bs, int ld, int tr) { return GemmOp{ws + off, bs, ld, tr}; };
    const GemmOp Sop{x.S_chunks, DD, D, 0}, SopT{x.S_chunks, DD, D, 1};
    // Delta = U~ - W S
    if ((e = gemm(s, nrec, C, D, D, op(L.W, CD, D, 0), Sop, ws + L.Del, CD, D, -1.f, 1.f, ws + L.Ut, CD)) != hipSuccess) return e;
    // dQ~ = dO S^T, dW = -dDelta S^T
    if ((e = gemm(s, nrec, C, D, D, op(L.dO, CD, D, 0), SopT, ws + L.dQt, CD, D, 1.f)) != hipSuccess) return e;
    if ((e = gemm(s, nrec, C, D, D, op(L.dDel, CD, D, 0), SopT, ws + L.dW, CD, D, -1.f)) != hipSuccess) return e;
    // dK^ = Delta Lam^T
    if ((e = gemm(s, nrec, C, D, D, op(L.Del, CD, D, 0), op(L.Lam, DD, D, 1), ws + L.dKh, CD, D, 1.f)) != hipSuccess) return e;
    // dP = tril(dO Delta^T)
    if ((e = gemm(s, nrec, C, C, D, op(L.dO, CD, D, 0), op(L.Del, CD, D, 1), ws + L.dP, CC, C, 1.f, 0.f, nullptr, 0, 1)) != hipSuccess) return e;
    // dX = dDelta U^T + dW E~^T
    if ((e = gemm(s, nrec, C, C, D, op(L.dDel, CD, D, 0), op(L.U, CD, D, 1), ws + L.dX, CC, C, 1.f)) != hipSuccess) return e;
    if ((e = gemm(s, nrec, C, C, D, op(L.dW, CD, D, 0), op(L.Et, CD, D, 1), ws + L.dX, CC, C, 1.f, 1.f, ws + L.dX, CC)) != hipSuccess) return e;
    // dU = X^T dDelta, dE~ = X^T dW
    if ((e = gemm(s, nrec, C, D, C, op(L.X, CC, C, 1), op(L.dDel, CD, D, 0), ws + L.dU, CD, D, 1.f)) != hipSuccess) return e;
    if ((e = gemm(s, nrec, C, D, C, op(L.X, CC, C, 1), op(L.dW, CD, D, 0), ws + L.dEt, CD, D, 1.f)) != hipSuccess) return e;
    // dM = strict_tril(-X^T dX X^T)
    if ((e = gemm(s, nrec, C, C, C, op(L.dX, CC, C, 0), op(L.X, CC, C, 1), ws + L.T1, CC, C, 1.f)) != hipSuccess) return e;
    if ((e = gemm(s, nrec, C, C, C, op(L.X, CC, C, 1), op(L.T1, CC, C, 0), ws + L.dM, CC, C, -1.f, 0.f, nullptr, 0, 2)) != hipSuccess) return e;

    hipLaunchKernelGGL((bwd_decay_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), lds_decay, s, a);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(const gdr2_bwd_args& a)
{
    if (a.B * a.H * a.T == 0)
        return 0;
    return bwd_layout(a.B, a.H, a.T, (int)a.Dk).total;
}

hipError_t launch_backward(const gdr2_bwd_args& a, hipStream_t stream)
{
    if (a.T == 0) {   // no tokens: dS0 = dS_final
        const int64_t n = a.B * a.H * a.Dk * a.Dv;
        if (!a.dS0 || a.dS0 == a.dS_final)
            return hipSuccess;
        return a.dS_final ? launch_state_copy(a.dS_final, a.dS0, n, stream) : zero_fill(a.dS0, n, stream);
    }
    if (a.dtype == GDR2_BF16)
        return a.Dk == 128 ? launch_backward_t<bf16, 128>(a, stream) : launch_backward_t<bf16, 64>(a, stream);
    return a.Dk == 128 ? launch_backward_t<float, 128>(a, stream) : launch_backward_t<float, 64>(a, stream);
}

}  // namespace gdr2
