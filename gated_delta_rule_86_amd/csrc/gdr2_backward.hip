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
    // scan operand fragments (ScanFrags), rec_bytes per record
    size_t SF;
    size_t total;
};

BwdLayout bwd_layout(int64_t B, int64_t H, int64_t T, int D, size_t rec_bytes)
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
    L.SF = o;
    o += a64((size_t)L.nrec * rec_bytes / 4);
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
    int64_t T, H, NC, nrec, nbh;
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
// Operands of the reverse scan, in MFMA fragment order and the input
// precision E.  A 1 KB fragment holds 16 rows x KB contraction indices: lane
// l keeps row l%16 and, inside the KB block, k = 4(l/16)..+3 (bf16: also
// 16+4(l/16)..+3), 16 contiguous bytes per lane -- what Mma<E>::load reads
// from a row-major matrix, so an accumulator tile is directly a B operand.
// Per chunk record:
//   K   K^      rows s (C/16 tiles)           x k = key channel (D/KB steps)
//   P   P^T     rows s                        x k = token (C/KB steps; the
//               part below the diagonal is stored as zeros)
//   Q   Q~^T    rows = key channel (D/16)     x k = token
//   W   -W^T    same
//   O   dO^T    rows = value column (D/16)    x k = token
// ---------------------------------------------------------------------------
template <typename E, int D>
struct ScanFrags {
    static constexpr int KB = Mma<E>::KB, KT = KB / 16, NB = BC / 16;
    static constexpr int NKS = D / KB, NKC = BC / KB, DT = D / 16;
    static constexpr size_t FRAG = 1024;
    static constexpr size_t K_BYTES = (size_t)NB * NKS * FRAG;    // C*D*sizeof(E)
    static constexpr size_t P_BYTES = (size_t)NB * NKC * FRAG;    // C*C*sizeof(E)
    static constexpr size_t T_BYTES = (size_t)DT * NKC * FRAG;    // C*D*sizeof(E)
    static constexpr size_t OFF_K = 0, OFF_P = K_BYTES, OFF_Q = OFF_P + P_BYTES, OFF_W = OFF_Q + T_BYTES,
                            OFF_O = OFF_W + T_BYTES, REC = OFF_O + T_BYTES;
    static constexpr int NFRAG = (int)(REC / FRAG);
    static_assert(K_BYTES == (size_t)BC * D * sizeof(E), "fragment size");
    static_assert(REC == (size_t)(4 * BC * D + BC * BC) * sizeof(E), "record size used for the workspace");
};

// Contraction index held in slot j (0 .. 16/sizeof(E)-1) by lane group gq.
template <typename E> __device__ __forceinline__ int slot_k(int gq, int j);
template <> __device__ __forceinline__ int slot_k<bf16>(int gq, int j) { return (j < 4 ? 0 : 12) + 4 * gq + j; }
template <> __device__ __forceinline__ int slot_k<float>(int gq, int j) { return 4 * gq + j; }

// One workgroup per chunk record: the fp32 rows the prep kernel and the dO
// copy wrote, re-laid into fragments.  Item (fragment, lane) -> 16 bytes.
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_frag_kernel(BwdArgs a)
{
    typedef ScanFrags<E, D> F;
    constexpr int C = BC, NV = 16 / (int)sizeof(E);
    const int64_t r = blockIdx.x;
    const float* ws = a.ws;
    const size_t cdo = (size_t)r * C * D, cco = (size_t)r * C * C;
    unsigned char* out = reinterpret_cast<unsigned char*>(a.ws + a.L.SF) + (size_t)r * F::REC;
    for (int it = threadIdx.x; it < F::NFRAG * 64; it += NTB) {
        const int f = it / 64, lane = it % 64, gq = lane / 16, rl = lane % 16;
        const float* src;
        int row, m;
        int64_t rs, ks;            // element (row, k) at src[row * rs + k * ks]
        float sign = 1.f;
        if (f < F::NB * F::NKS) {                       // K^ [s][i]
            row = 16 * (f / F::NKS) + rl; m = f % F::NKS;
            src = ws + a.L.Kh + cdo; rs = D; ks = 1;
        } else if (f < F::NB * (F::NKS + F::NKC)) {     // P^T [s][t] = P[t][s]
            const int g = f - F::NB * F::NKS;
            row = 16 * (g / F::NKC) + rl; m = g % F::NKC;
            src = ws + a.L.P + cco; rs = 1; ks = C;
        } else {                                        // Q~^T, -W^T, dO^T: [i][t] = X[t][i]
            const int g = f - F::NB * (F::NKS + F::NKC), which = g / (F::DT * F::NKC), h = g % (F::DT * F::NKC);
            row = 16 * (h / F::NKC) + rl; m = h % F::NKC;
            src = ws + cdo + (which == 0 ? a.L.Qt : which == 1 ? a.L.W : a.L.dO);
            sign = which == 1 ? -1.f : 1.f;
            rs = 1; ks = D;
        }
        float x[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j)
            x[j] = sign * src[row * rs + (int64_t)(m * F::KB + slot_k<E>(gq, j)) * ks];
        unsigned char* dst = out + (size_t)f * F::FRAG + lane * 16;
        if constexpr (sizeof(E) == 2) {
            *reinterpret_cast<bf16x8*>(dst) = Mma<bf16>::pack(f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]});
        } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_scan: the state gradient through the chunks in reverse, per (sequence,
// head) and BV value columns (16 per wave; columns evolve independently).
// Lam (the gradient at the current chunk end) stays in MFMA accumulators;
// per chunk:
//   dDelta = K^ Lam + P^T dO,   Lam <- diag(gamma) Lam + Q~^T dO - W^T dDelta
// and Lam (before the update) and dDelta go to the workspace in fp32.  A
// chunk's fragments are copied global -> LDS with global_load_lds (no
// register staging), double buffered when two buffers fit.
// ---------------------------------------------------------------------------
template <typename E, int D>
struct ScanShape {
    typedef ScanFrags<E, D> F;
    static constexpr int BV = 64, NS = D / BV;
    static constexpr size_t O_SLICE = (size_t)(BV / 16) * F::NKC * F::FRAG;
    static constexpr size_t OFF_O = F::OFF_O, OFF_G = OFF_O + O_SLICE, BUF = OFF_G + (size_t)D * 4;
    static constexpr int NBUF = 2 * BUF <= 160 * 1024 ? 2 : 1;
    static_assert(F::OFF_O % 1024 == 0 && O_SLICE % 1024 == 0, "whole fragments");
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// BYTES (a multiple of 1 KB) global -> LDS, 16 bytes per lane per
// instruction; instruction j belongs to wave j % 4.
template <size_t BYTES>
__device__ __forceinline__ void copy_frags(const unsigned char* g, unsigned char* l, int wave, int lane)
{
    constexpr int NINST = (int)(BYTES / 1024);
#pragma unroll
    for (int j = wave; j < NINST; j += NTB / 64)
        __builtin_amdgcn_global_load_lds(g + j * 1024 + lane * 16, (lds_void*)(l + j * 1024), 16, 0, 0);
}

template <typename E, int D>
__device__ __forceinline__ void scan_fetch(const BwdArgs& a, int64_t r, int slice, unsigned char* buf, int wave,
                                           int lane)
{
    typedef ScanShape<E, D> S;
    typedef ScanFrags<E, D> F;
    const unsigned char* rec = reinterpret_cast<const unsigned char*>(a.ws + a.L.SF) + (size_t)r * F::REC;
    copy_frags<F::OFF_O>(rec, buf, wave, lane);
    copy_frags<S::O_SLICE>(rec + F::OFF_O + slice * S::O_SLICE, buf + S::OFF_O, wave, lane);
    if (wave == NTB / 64 - 1 && lane < D / 4)
        __builtin_amdgcn_global_load_lds(a.ws + a.L.gam + (size_t)r * D + lane * 4, (lds_void*)(buf + S::OFF_G), 16,
                                         0, 0);
}

template <typename E, int D>
__device__ __forceinline__ void scan_chunk(const BwdArgs& a, const unsigned char* buf, f32x4* lam, int64_t r,
                                           int col, int lane, int wave)
{
    typedef ScanShape<E, D> S;
    typedef ScanFrags<E, D> F;
    typedef Mma<E> MM;
    typedef typename MM::Frag Frag;
    constexpr int NB = F::NB, NKS = F::NKS, NKC = F::NKC, KT = F::KT, DT = F::DT;
    const int gq = lane >> 4;
    const unsigned char* fl = buf + lane * 16;
    auto frag = [&](size_t off, int i) -> Frag { return *reinterpret_cast<const Frag*>(fl + off + (size_t)i * 1024); };
    const float* sGam = reinterpret_cast<const float*>(buf + S::OFF_G);

    // the gradient at this chunk's end, for the per-chunk products
    float* lo = a.ws + a.L.Lam + (size_t)r * D * D;
#pragma unroll
    for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lo[(16 * kt + 4 * gq + i) * D + col] = lam[kt][i];

    Frag LB[NKS], OB[NKC];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        LB[ks] = MM::from_acc(&lam[ks * KT]);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        OB[kc] = frag(S::OFF_O, wave * NKC + kc);

    // dDelta = K^ Lam + P^T dO  (P^T is upper triangular: k-steps from the diagonal)
    f32x4 dd[NB];
#pragma unroll
    for (int st = 0; st < NB; ++st)
        dd[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int st = 0; st < NB; ++st)
            dd[st] = MM::mma(frag(F::OFF_K, st * NKS + ks), LB[ks], dd[st]);
#pragma unroll
    for (int st = 0; st < NB; ++st)
#pragma unroll
        for (int kc = st / KT; kc < NKC; ++kc)
            dd[st] = MM::mma(frag(F::OFF_P, st * NKC + kc), OB[kc], dd[st]);
    float* dq = a.ws + a.L.dDel + (size_t)r * BC * D;
#pragma unroll
    for (int st = 0; st < NB; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dq[(16 * st + 4 * gq + i) * D + col] = dd[st][i];

    // Lam <- diag(gamma) Lam + Q~^T dO - W^T dDelta  (the W fragments hold -W^T)
    Frag DB[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        DB[kc] = MM::from_acc(&dd[kc * KT]);
#pragma unroll
    for (int kt = 0; kt < DT; ++kt)
        lam[kt] = lam[kt] * *reinterpret_cast<const f32x4*>(sGam + 16 * kt + 4 * gq);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int kt = 0; kt < DT; ++kt) {
            lam[kt] = MM::mma(frag(F::OFF_Q, kt * NKC + kc), OB[kc], lam[kt]);
            lam[kt] = MM::mma(frag(F::OFF_W, kt * NKC + kc), DB[kc], lam[kt]);
        }
}

template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_scan_kernel(BwdArgs a)
{
    typedef ScanShape<E, D> S;
    constexpr int DT = D / 16;
    __shared__ __align__(16) unsigned char buf0[S::BUF];
    __shared__ __align__(16) unsigned char buf1[S::NBUF == 2 ? S::BUF : 16];
    // workgroup -> ((b,h), column slice); the slices of one (b,h) share
    // blockIdx % 8, i.e. one XCD and its L2
    const int64_t bx = blockIdx.x, grp = bx / (8 * S::NS);
    const int within = (int)(bx % (8 * S::NS)), slice = within / 8;
    const int64_t bh = grp * 8 + within % 8;
    if (bh >= a.nbh)
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4;
    const int col = slice * S::BV + 16 * wave + (lane & 15);
    const int64_t rec0 = bh * a.NC;

    f32x4 lam[DT];
#pragma unroll
    for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lam[kt][i] = a.dS_final ? a.dS_final[(bh * D + 16 * kt + 4 * gq + i) * D + col] : 0.f;

    scan_fetch<E, D>(a, rec0 + a.NC - 1, slice, buf0, wave, lane);
    if constexpr (S::NBUF == 2) {
        for (int64_t n = a.NC - 1; n >= 0; n -= 2) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0; everyone is done with buf1
            if (n >= 1)
                scan_fetch<E, D>(a, rec0 + n - 1, slice, buf1, wave, lane);
            scan_chunk<E, D>(a, buf0, lam, rec0 + n, col, lane, wave);
            if (n == 0)
                break;
            wait_copies();
            __syncthreads();          // chunk n - 1 is in buf1; everyone is done with buf0
            if (n >= 2)
                scan_fetch<E, D>(a, rec0 + n - 2, slice, buf0, wave, lane);
            scan_chunk<E, D>(a, buf1, lam, rec0 + n - 1, col, lane, wave);
        }
    } else {
        for (int64_t n = a.NC - 1; n >= 0; --n) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0
            scan_chunk<E, D>(a, buf0, lam, rec0 + n, col, lane, wave);
            __syncthreads();          // everyone is done with buf0
            if (n >= 1)
                scan_fetch<E, D>(a, rec0 + n - 1, slice, buf0, wave, lane);
        }
    }
    if (a.dS0) {
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.dS0[(bh * D + 16 * kt + 4 * gq + i) * D + col] = lam[kt][i];
    }
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
// bwd_decay: per chunk and block of DC key channels, the decay-weighted sums
// and the input gradients.  Every channel is independent here, so one
// workgroup takes DC channels of one chunk; thread (row group, channel) owns
// the rows t = rg + 8m of its channel.
// ---------------------------------------------------------------------------
constexpr int DC = 32;                 // channels per decay workgroup
constexpr int LC = DC + 1;             // padded LDS row

template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_decay_kernel(BwdArgs a)
{
    constexpr int C = BC, NRG = NTB / DC, RPT = C / NRG;
    extern __shared__ __align__(16) float sm[];
    float* sG = sm;                 // [C][LC] cumulative log-decay
    float* sE = sG + C * LC;        // [C][LC] e = b*k
    float* sK = sE + C * LC;        // [C][LC] k
    float* sQ = sK + C * LC;        // [C][LC] q
    float* sdG = sQ + C * LC;       // [C][LC] dG, then dg
    float* sdM = sdG + C * LC;      // [C][C]
    float* sdP = sdM + C * C;       // [C][C]
    float* sGL = sdP + C * C;       // [DC] dG_L
    const int64_t r = blockIdx.x / (D / DC);
    const int i0 = (int)(blockIdx.x % (D / DC)) * DC;
    const Rec rc = rec_of(r, a.NC, a.T, a.H);
    const int tid = threadIdx.x, il = tid % DC, rg = tid / DC, i = i0 + il;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* b = (const E*)a.b;
    const E* w = (const E*)a.w;
    const float* ws = a.ws;
    const size_t cdo = (size_t)r * C * D, cco = (size_t)r * C * C;

    for (int e = tid; e < C * DC; e += NTB) {
        const int t = e / DC, c = e % DC, l = t * LC + c;
        const size_t x = cdo + (size_t)t * D + i0 + c;
        float kv = 0.f, qv = 0.f;
        if (t < rc.L) {
            const int64_t row = rc.row0 + (int64_t)t * a.H;
            kv = ldf(k, row * D + i0 + c);
            qv = ldf(q, row * D + i0 + c);
        }
        sG[l] = ws[a.L.G + x];
        sE[l] = ws[a.L.E + x];
        sK[l] = kv;
        sQ[l] = qv;
    }
    for (int e = tid; e < C * C; e += NTB) {
        sdM[e] = ws[a.L.dM + cco + e];
        sdP[e] = ws[a.L.dP + cco + e];
    }
    // dG_L = sum_s dK^ K^ + dgamma gamma, with dgamma = rowsum(S * Lam)
    if (tid < DC) {
        const float* S = a.S_chunks + (size_t)r * D * D + (size_t)i * D;
        const float* Lam = ws + a.L.Lam + (size_t)r * D * D + (size_t)i * D;
        float dgam = 0.f;
        for (int j = 0; j < D; ++j)
            dgam += S[j] * Lam[j];
        float acc = dgam * ws[a.L.gam + (size_t)r * D + i];
        for (int s = 0; s < C; ++s)
            acc += ws[a.L.dKh + cdo + s * D + i] * ws[a.L.Kh + cdo + s * D + i];
        sGL[il] = acc;
    }
    __syncthreads();
    for (int m = 0; m < RPT; ++m) {
        const int t = rg + NRG * m, l = t * LC + il;
        const float Gt = sG[l];
        // as the later token t: sum over s <= t
        float dEm = 0.f, dqp = 0.f;
        for (int s = 0; s <= t; ++s) {
            const float f = expf(Gt - sG[s * LC + il]) * sK[s * LC + il];
            dEm += sdM[t * C + s] * f;       // dM is strictly lower: dM[t][t] = 0
            dqp += sdP[t * C + s] * f;
        }
        // as the earlier token: sum over t2 >= t
        float dkm = 0.f;
        for (int t2 = t; t2 < C; ++t2) {
            const float f = expf(sG[t2 * LC + il] - Gt);
            dkm += (sdM[t2 * C + t] * sE[t2 * LC + il] + sdP[t2 * C + t] * sQ[t2 * LC + il]) * f;
        }
        const size_t x = cdo + (size_t)t * D + i;
        const float eg = expf(Gt), dEt = ws[a.L.dEt + x], dQt = ws[a.L.dQt + x];
        const float dKh = ws[a.L.dKh + x], Kh = ws[a.L.Kh + x];
        float dG = sE[l] * dEm + sQ[l] * dqp - sK[l] * dkm + dEt * ws[a.L.Et + x] + dQt * ws[a.L.Qt + x] -
                   dKh * Kh;
        if (t == rc.L - 1)
            dG += sGL[il];
        sdG[l] = dG;
        if (t < rc.L) {
            const int64_t row = rc.row0 + (int64_t)t * a.H, off = row * D + i;
            const float GL = sG[(C - 1) * LC + il];
            const float bv = ldf(b, a.bw == 1 ? row : off);
            const float dE = dEm + dEt * eg;
            const float dU = ws[a.L.dU + x];
            a.dq[off] = dqp + dQt * eg;
            a.dk[off] = dkm + dKh * expf(GL - Gt) + dE * bv;
            a.dv[off] = dU * ldf(w, a.ww == 1 ? row : off);
            const float dbv = dE * sK[l], dwv = dU * ldf(v, off);
            if (a.bw == 1)
                atomicAdd(a.db + row, dbv);
            else
                a.db[off] = dbv;
            if (a.ww == 1)
                atomicAdd(a.dw + row, dwv);
            else
                a.dw[off] = dwv;
        }
    }
    __syncthreads();
    // dg: reverse cumulative sum over the chunk, per channel
    if (tid < DC) {
        float acc = 0.f;
        for (int t = C - 1; t >= 0; --t) {
            acc += sdG[t * LC + tid];
            sdG[t * LC + tid] = acc;
        }
    }
    __syncthreads();
    for (int m = 0; m < RPT; ++m) {
        const int t = rg + NRG * m;
        if (t >= rc.L)
            continue;
        const int64_t row = rc.row0 + (int64_t)t * a.H;
        const float dgv = sdG[t * LC + il];
        if (a.gw == 1)
            atomicAdd(a.dg + row, dgv);
        else
            a.dg[row * D + i] = dgv;
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
    a.L = bwd_layout(x.B, x.H, x.T, D, ScanFrags<E, D>::REC);
    a.nbh = x.B * x.H;
    a.nrec = a.L.nrec;
    a.ws = static_cast<float*>(x.workspace);
    const int64_t nrec = a.nrec, rows = x.B * x.T * x.H;
    hipError_t e;
    // width-1 gate gradients accumulate over channels
    if (a.bw == 1 && (e = zero_fill(a.db, rows, s)) != hipSuccess) return e;
    if (a.ww == 1 && (e = zero_fill(a.dw, rows, s)) != hipSuccess) return e;
    if (a.gw == 1 && (e = zero_fill(a.dg, rows, s)) != hipSuccess) return e;

    const size_t lds_prep = (size_t)(4 * C * (D + 1) + C * C) * 4;
    const size_t lds_decay = (size_t)(5 * C * LC + 2 * C * C + DC) * 4;
    // more than 64 KiB of dynamic LDS must be requested per kernel
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_prep_kernel<E, D>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_prep)) != hipSuccess ||
        (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_decay_kernel<E, D>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_decay)) != hipSuccess)
        return e;

    hipLaunchKernelGGL((bwd_prep_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), lds_prep, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dout_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_frag_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        const int64_t groups = cdiv(a.nbh, 8) * 8 * ScanShape<E, D>::NS;
        hipLaunchKernelGGL((bwd_scan_kernel<E, D>), dim3((unsigned)groups), dim3(NTB), 0, s, a);
    }
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

    hipLaunchKernelGGL((bwd_decay_kernel<E, D>), dim3((unsigned)(nrec * (D / DC))), dim3(NTB), lds_decay, s, a);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(const gdr2_bwd_args& a)
{
    if (a.B * a.H * a.T == 0)
        return 0;
    const size_t esz = a.dtype == GDR2_BF16 ? 2 : 4;
    const size_t rec = (size_t)(4 * BC * a.Dk + BC * BC) * esz;   // ScanFrags<E, D>::REC
    return bwd_layout(a.B, a.H, a.T, (int)a.Dk, rec).total;
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
