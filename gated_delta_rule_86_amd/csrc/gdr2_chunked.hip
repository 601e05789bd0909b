// gdr2_chunked.hip -- chunked forward of the Gated DeltaNet-2 recurrence
// (page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리": the update
// of section "Gated Delta Rule-2 업데이트 수식"; fixed-size chunks and a WY
// form that absorbs the cumulative channel decay into the erase factors,
// section "효율적 구현").
//
// Chunk form used here (derived from the update; L tokens, chunk-start state
// S, G_t = sum_{r<=t} g_r per key channel, e_t = b_t*k_t, u_t = w_t*v_t):
//   M[t,s] = sum_i e_t[i] k_s[i] 2^(G_t[i]-G_s[i])   s <  t   (strictly lower)
//   P[t,s] = sum_i q_t[i] k_s[i] 2^(G_t[i]-G_s[i])   s <= t
//   X = (I + M)^-1,  W = X (e*2^G),  U~ = X u
//   Delta = U~ - W S,  O = (q*2^G) S + P Delta,
//   S_next = diag(2^G_L) S + K^T Delta,   K^_s = k_s*2^(G_L-G_s)
// (G is kept in log2 units, so every decay factor is one v_exp_f32.)
//
// Two kernels:
//   chunk_prep  (every chunk of every sequence in parallel): the cumulative
//               decay, the gated Gram M and scores P (MFMA), X by blocked
//               substitution, W and U~ (MFMA).  It writes -W, U~, K^, Q~ =
//               q*2^G, P and gamma = 2^G_L per chunk to the workspace.
//   chunk_state (one workgroup per (sequence, head, 64 value columns); the
//               value columns of S evolve independently, so they split
//               exactly): walks the chunks in order with the fp32 state in
//               MFMA accumulators; Delta, O and the state update are MFMAs
//               whose B operands are the accumulators themselves.
//
// Decay absorption without overflow.  Factors are taken relative to the
// cumulative decay at 16-token block boundaries Gb[J] = G at the last token
// of block J (Gb[-1] = 0):
//   alpha_t = 2^(G_t - Gb[blk(t)-1]) <= 1,   beta_s = 2^(Gb[blk(s)] - G_s) <= 1
//   tile (I,J), J < I:  2^(G_t-G_s) = alpha_t * 2^(Gb[I-1]-Gb[J]) * beta_s,
//                       every factor <= 1 (underflow is the true limit);
//   tile (I,I):         the middle factor is 2^(span of block I) >= 1.
// The diagonal tiles are exact while the span of every 16-token block stays
// below kSpanMax (log2 units); a chunk that exceeds it recomputes its
// diagonal tiles pair by pair from the raw inputs (slow, exact).
#include "gdr2_device.h"
#include "gdr2_internal.h"

#include <algorithm>

namespace gdr2 {
namespace {

constexpr int NT = 256;            // threads per workgroup (4 waves)
constexpr float kSpanMax = 80.f;   // log2 units per 16-token block

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// Workspace: per chunk record (sequence, head, chunk), element type E:
//   Wn [C][D] = -W,  Ut [C][D] = U~,  Kh [C][D] = K^,  Qt [C][D] = Q~,
//   P [C][C],  gam [D] fp32.   Records are ordered (b*H + h)*NC + n.
// ---------------------------------------------------------------------------
struct Layout {
    int64_t nrec;
    size_t wn, ut, kh, qt, p, gam, total;
};

Layout staged_layout(int64_t B, int64_t H, int64_t T, int D, int C, int esz)
{
    Layout L;
    L.nrec = B * H * ceil_div(T, C);
    const size_t mat = al256((size_t)L.nrec * C * D * esz);
    const size_t pm = al256((size_t)L.nrec * C * C * esz);
    const size_t gm = al256((size_t)L.nrec * D * 4);
    L.wn = 0;
    L.ut = mat;
    L.kh = 2 * mat;
    L.qt = 3 * mat;
    L.p = 4 * mat;
    L.gam = 4 * mat + pm;
    L.total = 4 * mat + pm + gm;
    return L;
}

struct PrepArgs {
    const void *q, *k, *v, *b, *w;
    const float* g;
    int bw, ww, gw;
    int64_t T, H, NC, nrec;
    void *Wn, *Ut, *Kh, *Qt, *P;
    float* gam;
};

struct StateArgs {
    const void *Wn, *Ut, *Kh, *Qt, *P;
    const float* gam;
    const float* S0;
    float* S_out;
    void* o;
    int64_t T, H, NC, nbh;
};

template <typename E, int D, int C>
struct PrepShape {
    static constexpr int NB = C / 16;
    static constexpr int VEC = 16 / (int)sizeof(E);      // elements per 16-byte access
    static constexpr int NLD = C * D / (NT * VEC);        // 16-byte loads per thread per [C][D]
    static constexpr int NLDG = C * D / (NT * 4);         // fp32 g loads per thread
    static constexpr int LDA = D + 16 / (int)sizeof(E);   // [C][D] operands in LDS
    static constexpr int LDT = C + 16 / (int)sizeof(E);   // [D][C] operands in LDS
    static constexpr int LDM = C + 4;                     // fp32 [C][C] (M, X)
    static constexpr size_t R1 = cmax((size_t)C * D * 4, 2 * (size_t)D * LDT * sizeof(E));
    static constexpr size_t R2 = cmax(3 * (size_t)C * LDA * sizeof(E),
                                      ((size_t)C * LDM + (NB > 1 ? NB - 1 : 1) * 256) * 4);
    static constexpr size_t R3 = cmax((size_t)C * LDM * 4, (size_t)4 * D * 4);
    static constexpr size_t R4 = ((size_t)NB * NB * D + 2 * (size_t)NB * D) * 4;
    static constexpr size_t SMEM = al256(R1) + al256(R2) + al256(R3) + al256(R4) + 256;
    static_assert(C * D % (NT * VEC) == 0 && C * D % (NT * 4) == 0, "tile / thread mismatch");
    static_assert(NT % D == 0 && C % (NT / D) == 0, "cumsum mapping");
};

// Raw inputs of one chunk as loaded from HBM (bit patterns of E, or fp32 g).
template <typename E, int D, int C>
struct PrepRegs {
    typedef PrepShape<E, D, C> S;
    u32x4 k[S::NLD], q[S::NLD], b[S::NLD], v[S::NLD], w[S::NLD];
    f32x4 g[S::NLDG];
};

template <typename E>
__device__ __forceinline__ void unpack(const u32x4& r, float* out);
template <>
__device__ __forceinline__ void unpack<bf16>(const u32x4& r, float* out)
{
    const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        out[i] = (float)v[i];
}
template <>
__device__ __forceinline__ void unpack<float>(const u32x4& r, float* out)
{
    out[0] = __uint_as_float(r[0]);
    out[1] = __uint_as_float(r[1]);
    out[2] = __uint_as_float(r[2]);
    out[3] = __uint_as_float(r[3]);
}

template <typename E>
__device__ __forceinline__ u32x4 pack_vec(const float* x);
template <>
__device__ __forceinline__ u32x4 pack_vec<bf16>(const float* x)
{
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = (bf16)x[i];
    return __builtin_bit_cast(u32x4, v);
}
template <>
__device__ __forceinline__ u32x4 pack_vec<float>(const float* x)
{
    return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                 __float_as_uint(x[3])};
}

__device__ __forceinline__ u32x4 ldg16(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Chunk record -> (first token row, valid length).  Token row r of the chunk
// is the element offset ((b*T + t0 + r)*H + h) of [B,T,H,.] tensors.
struct ChunkPos {
    int64_t row0;     // (b*T + t0)*H + h
    int64_t H;        // row stride in tokens
    int L;            // valid tokens
};

__device__ __forceinline__ ChunkPos chunk_pos(int64_t rec, int64_t NC, int64_t T, int64_t H, int C)
{
    const int64_t bh = rec / NC, n = rec - bh * NC;
    const int64_t b = bh / H, h = bh - b * H;
    const int64_t t0 = n * C;
    ChunkPos p;
    p.row0 = (b * T + t0) * H + h;
    p.H = H;
    p.L = (int)min((int64_t)C, T - t0);
    return p;
}

template <typename E, int D, int C>
__device__ __forceinline__ void prep_load_gates(const PrepArgs& a, const ChunkPos& cp,
                                                PrepRegs<E, D, C>& R, int tid)
{
    typedef PrepShape<E, D, C> S;
#pragma unroll
    for (int j = 0; j < S::NLDG; ++j) {
        const int e = (j * NT + tid) * 4, t = e / D, c = e % D;
        f32x4 val = {0.f, 0.f, 0.f, 0.f};
        if (t < cp.L) {
            const int64_t row = cp.row0 + (int64_t)t * cp.H;
            if (a.gw == 1) {
                const float s = a.g[row];
                val = f32x4{s, s, s, s};
            } else {
                val = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.g + row * D + c));
            }
        }
        R.g[j] = val;
    }
}

template <typename E>
__device__ __forceinline__ u32x4 splat_bits(const E* p);
template <>
__device__ __forceinline__ u32x4 splat_bits<bf16>(const bf16* p)
{
    const unsigned short s = *reinterpret_cast<const unsigned short*>(p);
    const unsigned int w = (unsigned int)s | ((unsigned int)s << 16);
    return u32x4{w, w, w, w};
}
template <>
__device__ __forceinline__ u32x4 splat_bits<float>(const float* p)
{
    const unsigned int w = __float_as_uint(*p);
    return u32x4{w, w, w, w};
}

template <typename E, int D, int C>
__device__ __forceinline__ void prep_load_tokens(const PrepArgs& a, const ChunkPos& cp,
                                                 PrepRegs<E, D, C>& R, int tid)
{
    typedef PrepShape<E, D, C> S;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* b = (const E*)a.b;
    const E* w = (const E*)a.w;
#pragma unroll
    for (int j = 0; j < S::NLD; ++j) {
        const int e = (j * NT + tid) * S::VEC, t = e / D, c = e % D;
        const u32x4 z = {0u, 0u, 0u, 0u};
        R.k[j] = R.q[j] = R.b[j] = R.v[j] = R.w[j] = z;
        if (t < cp.L) {
            const int64_t row = cp.row0 + (int64_t)t * cp.H;
            R.k[j] = ldg16(k + row * D + c);
            R.q[j] = ldg16(q + row * D + c);
            R.v[j] = ldg16(v + row * D + c);
            R.b[j] = a.bw == 1 ? splat_bits<E>(b + row) : ldg16(b + row * D + c);
            R.w[j] = a.ww == 1 ? splat_bits<E>(w + row) : ldg16(w + row * D + c);
        }
    }
}

// ---------------------------------------------------------------------------
// chunk_prep: one workgroup per CU, looping over chunk records with the next
// chunk's inputs prefetched into registers while the current one computes.
// ---------------------------------------------------------------------------
template <typename E, int D, int C>
__global__ __launch_bounds__(NT, 1) void chunk_prep_kernel(PrepArgs a)
{
    typedef PrepShape<E, D, C> S;
    typedef Mma<E> MM;
    constexpr int NB = S::NB, VEC = S::VEC, LDA = S::LDA, LDT = S::LDT, LDM = S::LDM;

    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* r1 = smem;
    unsigned char* r2 = r1 + al256(S::R1);
    unsigned char* r3 = r2 + al256(S::R2);
    unsigned char* r4 = r3 + al256(S::R3);
    int* sFlag = reinterpret_cast<int*>(r4 + al256(S::R4));
    float* sG = reinterpret_cast<float*>(r1);            // [C][D]  (phases 1-4)
    E* sEtT = reinterpret_cast<E*>(r1);                  // [D][LDT] (phase 6)
    E* sUT = sEtT + D * LDT;                             // [D][LDT] (phase 6)
    E* sEa = reinterpret_cast<E*>(r2);                   // [C][LDA] e*alpha
    E* sQa = sEa + C * LDA;                              // [C][LDA] q*alpha
    E* sKb = sQa + C * LDA;                              // [C][LDA] k*beta
    float* sX = reinterpret_cast<float*>(r2);            // [C][LDM] (phases 5-6)
    float* sY = sX + C * LDM;                            // [NB-1][16][16]
    float* sM = reinterpret_cast<float*>(r3);            // [C][LDM]
    float* sPart = reinterpret_cast<float*>(r3);         // [NT/D][D] (phase 2)
    float* sF = reinterpret_cast<float*>(r4);            // [NB][NB][D] 2^(Gb[I-1]-Gb[J])
    float* sE0 = sF + NB * NB * D;                       // [NB][D] 2^Gb[J-1]
    float* sEl = sE0 + NB * D;                           // [NB][D] 2^(Gb[NB-1]-Gb[J])

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    PrepRegs<E, D, C> R;
    int64_t rec = blockIdx.x;
    if (rec >= a.nrec)
        return;
    {
        const ChunkPos cp = chunk_pos(rec, a.NC, a.T, a.H, C);
        prep_load_gates(a, cp, R, tid);
        prep_load_tokens(a, cp, R, tid);
    }

    for (; rec < a.nrec; rec += gridDim.x) {
        const ChunkPos cp = chunk_pos(rec, a.NC, a.T, a.H, C);
        const int64_t next = rec + gridDim.x;
        const ChunkPos np = chunk_pos(next < a.nrec ? next : rec, a.NC, a.T, a.H, C);
        E* gWn = (E*)a.Wn + rec * C * D;
        E* gUt = (E*)a.Ut + rec * C * D;
        E* gKh = (E*)a.Kh + rec * C * D;
        E* gQt = (E*)a.Qt + rec * C * D;
        E* gP = (E*)a.P + rec * C * C;
        float* gGam = a.gam + rec * D;

        __syncthreads();  // the previous chunk is done with every LDS region
        // Phase 1: log-decay into LDS (natural log -> log2 units).
#pragma unroll
        for (int j = 0; j < S::NLDG; ++j) {
            const int e = (j * NT + tid) * 4;
            *reinterpret_cast<f32x4*>(sG + e) = R.g[j] * kLog2e;
        }
        if (tid == 0)
            *sFlag = 0;
        if (next < a.nrec)
            prep_load_gates(a, np, R, tid);
        __syncthreads();

        // Phase 2: inclusive prefix sum over the chunk's tokens, per channel.
        {
            constexpr int P = NT / D, RP = C / P;
            const int i = tid % D, p = tid / D;
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                acc += sG[(p * RP + r) * D + i];
                sG[(p * RP + r) * D + i] = acc;
            }
            sPart[p * D + i] = acc;
            __syncthreads();
            float off = 0.f;
            for (int pp = 0; pp < p; ++pp)
                off += sPart[pp * D + i];
            if (p > 0) {
#pragma unroll
                for (int r = 0; r < RP; ++r)
                    sG[(p * RP + r) * D + i] += off;
            }
        }
        __syncthreads();
        // Block-boundary tables, gamma, and the span guard.
        for (int e = tid; e < NB * NB * D; e += NT) {
            const int i = e % D, IJ = e / D, I = IJ / NB, J = IJ % NB;
            if (J > I)
                continue;
            const float gprev = I > 0 ? sG[(16 * I - 1) * D + i] : 0.f;
            const float gj = sG[(16 * J + 15) * D + i];
            sF[e] = fast_exp2(gprev - gj);
            if (I == J) {
                if (gprev - gj > kSpanMax)
                    *sFlag = 1;
                sE0[J * D + i] = fast_exp2(gprev);
                sEl[J * D + i] = fast_exp2(sG[(C - 1) * D + i] - gj);
                if (J == NB - 1)
                    gGam[i] = fast_exp2(gj);
            }
        }
        __syncthreads();

        // Phase 3: decay-absorbed operands.
        u32x4 rEt[S::NLD], rU[S::NLD];
#pragma unroll
        for (int j = 0; j < S::NLD; ++j) {
            const int e = (j * NT + tid) * VEC, t = e / D, c = e % D, blk = t >> 4;
            float kk[VEC], qq[VEC], bb[VEC], vv[VEC], ww[VEC];
            unpack<E>(R.k[j], kk);
            unpack<E>(R.q[j], qq);
            unpack<E>(R.b[j], bb);
            unpack<E>(R.v[j], vv);
            unpack<E>(R.w[j], ww);
            float ea[VEC], qa[VEC], kb[VEC], qt[VEC], kh[VEC], et[VEC], uu[VEC];
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                const int i = c + x;
                const float G = sG[t * D + i];
                const float Gp = blk > 0 ? sG[(16 * blk - 1) * D + i] : 0.f;
                const float Gc = sG[(16 * blk + 15) * D + i];
                const float al = fast_exp2(G - Gp);
                const float be = fast_exp2(Gc - G);
                const float e0 = sE0[blk * D + i];
                ea[x] = bb[x] * kk[x] * al;
                qa[x] = qq[x] * al;
                kb[x] = kk[x] * be;
                qt[x] = qa[x] * e0;
                kh[x] = kb[x] * sEl[blk * D + i];
                et[x] = ea[x] * e0;
                uu[x] = ww[x] * vv[x];
            }
            *reinterpret_cast<u32x4*>(sEa + t * LDA + c) = pack_vec<E>(ea);
            *reinterpret_cast<u32x4*>(sQa + t * LDA + c) = pack_vec<E>(qa);
            *reinterpret_cast<u32x4*>(sKb + t * LDA + c) = pack_vec<E>(kb);
            *reinterpret_cast<u32x4*>(gQt + t * D + c) = pack_vec<E>(qt);
            *reinterpret_cast<u32x4*>(gKh + t * D + c) = pack_vec<E>(kh);
            rEt[j] = pack_vec<E>(et);
            rU[j] = pack_vec<E>(uu);
        }
        if (next < a.nrec)
            prep_load_tokens(a, np, R, tid);
        __syncthreads();

        // Phase 4: gated Gram M (-> LDS) and scores P (-> workspace), MFMA.
        const bool guard = *sFlag != 0;
        {
            constexpr int NTASK = NB * (NB + 1);
            for (int tau = wave; tau < NTASK; tau += NT / 64) {
                const int kind = tau & 1, pair = tau >> 1;
                int I = 0;
                while ((I + 1) * (I + 2) / 2 <= pair)
                    ++I;
                const int J = pair - I * (I + 1) / 2;
                if (guard && I == J)
                    continue;
                const E* A = (kind ? sQa : sEa) + 16 * I * LDA;
                const E* Bm = sKb + 16 * J * LDA;
                const float* f = sF + (I * NB + J) * D;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < D; k0 += MM::KB)
                    acc = MM::mma(MM::load(A + k0, LDA, lane), MM::load_scaled(Bm + k0, LDA, f + k0, lane), acc);
                const int r0 = 16 * I + 4 * (lane >> 4), s = 16 * J + (lane & 15);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int r = r0 + ii;
                    if (kind == 0)
                        sM[r * LDM + s] = s < r ? acc[ii] : 0.f;
                    else
                        gP[r * C + s] = from_f32<E>(s <= r ? acc[ii] : 0.f);
                }
            }
            // P is lower triangular: zero the tiles above the diagonal.
            for (int e = tid; e < C * C; e += NT) {
                const int r = e / C, s = e % C;
                if ((s >> 4) > (r >> 4))
                    gP[e] = from_f32<E>(0.f);
            }
        }
        if (guard) {
            // Exact diagonal tiles for a chunk whose decay is too steep for the
            // block-factored form: every pair from the raw inputs.
            __syncthreads();
            const E* q = (const E*)a.q;
            const E* k = (const E*)a.k;
            const E* b = (const E*)a.b;
            for (int e = tid; e < NB * 256; e += NT) {
                const int I = e >> 8, r = 16 * I + ((e >> 4) & 15), s = 16 * I + (e & 15);
                float m = 0.f, p = 0.f;
                if (s <= r && r < cp.L && s < cp.L) {
                    const int64_t rr = cp.row0 + (int64_t)r * cp.H, rs = cp.row0 + (int64_t)s * cp.H;
                    for (int i = 0; i < D; ++i) {
                        const float dec = fast_exp2(sG[r * D + i] - sG[s * D + i]);
                        const float ks = to_f32(k[rs * D + i]) * dec;
                        const float br = to_f32(a.bw == 1 ? b[rr] : b[rr * D + i]);
                        m += br * to_f32(k[rr * D + i]) * ks;
                        p += to_f32(q[rr * D + i]) * ks;
                    }
                }
                sM[r * LDM + s] = s < r ? m : 0.f;
                gP[r * C + s] = from_f32<E>(p);
            }
        }
        __syncthreads();

        // Phase 5: X = (I + M)^-1.  Diagonal 16x16 blocks by forward
        // substitution (one lane per column), then the blocks below the
        // diagonal level by level: X_IJ = -X_II sum_{J<=K<I} M_IK X_KJ.
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, s = e % C;
            if ((s >> 4) > (r >> 4))
                sX[r * LDM + s] = 0.f;
        }
        if (wave == 0 && (lane >> 4) < NB) {
            const int I = lane >> 4, j = lane & 15;
            const float* m = sM + 16 * I * LDM + 16 * I;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == j ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < r; ++c)
                    acc -= m[r * LDM + c] * x[c];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sX[(16 * I + r) * LDM + 16 * I + j] = x[r];
        }
        __syncthreads();
        for (int d = 1; d < NB; ++d) {
            const int nblk = NB - d;
            for (int e = tid; e < nblk * 256; e += NT) {
                const int I = d + (e >> 8), J = I - d, r = (e >> 4) & 15, c = e & 15;
                float y = 0.f;
                for (int K = J; K < I; ++K) {
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        y += sM[(16 * I + r) * LDM + 16 * K + s] * sX[(16 * K + s) * LDM + 16 * J + c];
                }
                sY[e] = y;
            }
            __syncthreads();
            for (int e = tid; e < nblk * 256; e += NT) {
                const int I = d + (e >> 8), J = I - d, r = (e >> 4) & 15, c = e & 15;
                float x = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    x -= sX[(16 * I + r) * LDM + 16 * I + m] * sY[(e >> 8) * 256 + m * 16 + c];
                sX[(16 * I + r) * LDM + 16 * J + c] = x;
            }
            __syncthreads();
        }

        // Phase 6: W = X (e*2^G) and U~ = X u, with the right-hand sides
        // stored transposed so their B fragments are contiguous along tokens.
#pragma unroll
        for (int j = 0; j < S::NLD; ++j) {
            const int e = (j * NT + tid) * VEC, t = e / D, c = e % D;
            float et[VEC], uu[VEC];
            unpack<E>(rEt[j], et);
            unpack<E>(rU[j], uu);
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                sEtT[(c + x) * LDT + t] = from_f32<E>(et[x]);
                sUT[(c + x) * LDT + t] = from_f32<E>(uu[x]);
            }
        }
        __syncthreads();
        {
            constexpr int NTILE = NB * (D / 16);
            for (int tau = wave; tau < 2 * NTILE; tau += NT / 64) {
                const int kind = tau / NTILE, rem = tau % NTILE, mt = rem / (D / 16), nt = rem % (D / 16);
                const E* Bm = (kind ? sUT : sEtT) + 16 * nt * LDT;
                const float* A = sX + 16 * mt * LDM;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 0; k0 < 16 * (mt + 1); k0 += MM::KB)
                    acc = MM::mma(MM::load(A + k0, LDM, lane), MM::load(Bm + k0, LDT, lane), acc);
                const int r0 = 16 * mt + 4 * (lane >> 4), col = 16 * nt + (lane & 15);
                E* out = kind ? gUt : gWn;
                const float sg = kind ? 1.f : -1.f;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    out[(r0 + ii) * D + col] = from_f32<E>(sg * acc[ii]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// chunk_state: carries the fp32 state through the chunks of one sequence and
// head, BV value columns per workgroup (16 per wave), and writes o.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, int BV>
struct StateShape {
    static constexpr int NB = C / 16;
    static constexpr int VEC = 16 / (int)sizeof(E);
    static constexpr int NS = D / BV;                     // column slices per (b,h)
    static constexpr int LDA = D + 16 / (int)sizeof(E);   // sW, sQ  [C][LDA]
    static constexpr int LDT = C + 16 / (int)sizeof(E);   // sKT [D][LDT], sP [C][LDT]
    static constexpr int LDU = BV + 16 / (int)sizeof(E);  // sU  [C][LDU]
    static constexpr int NLD = C * D / (NT * VEC);
    static constexpr int NLDP = (C * C + NT * VEC - 1) / (NT * VEC);
    static constexpr int NLDU = (C * BV + NT * VEC - 1) / (NT * VEC);
    static constexpr size_t SMEM = al256((size_t)C * LDA * sizeof(E)) * 2 +
                                   al256((size_t)D * LDT * sizeof(E)) +
                                   al256((size_t)C * LDT * sizeof(E)) +
                                   al256((size_t)C * LDU * sizeof(E)) + al256((size_t)D * 4);
    static_assert(BV == 16 * (NT / 64), "one 16-column tile per wave");
    static_assert(C * D % (NT * VEC) == 0, "tile / thread mismatch");
};

template <typename E, int D, int C, int BV>
struct StateRegs {
    typedef StateShape<E, D, C, BV> S;
    u32x4 w[S::NLD], q[S::NLD], kh[S::NLD], p[S::NLDP], u[S::NLDU];
    f32x4 gam;
};

template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_load(const StateArgs& a, int64_t rec, int slice,
                                           StateRegs<E, D, C, BV>& R, int tid)
{
    typedef StateShape<E, D, C, BV> S;
    const E* Wn = (const E*)a.Wn + rec * C * D;
    const E* Qt = (const E*)a.Qt + rec * C * D;
    const E* Kh = (const E*)a.Kh + rec * C * D;
    const E* P = (const E*)a.P + rec * C * C;
    const E* Ut = (const E*)a.Ut + rec * C * D;
#pragma unroll
    for (int j = 0; j < S::NLD; ++j) {
        const int e = (j * NT + tid) * S::VEC;
        R.w[j] = *reinterpret_cast<const u32x4*>(Wn + e);
        R.q[j] = *reinterpret_cast<const u32x4*>(Qt + e);
        R.kh[j] = *reinterpret_cast<const u32x4*>(Kh + e);
    }
#pragma unroll
    for (int j = 0; j < S::NLDP; ++j) {
        const int e = (j * NT + tid) * S::VEC;
        if (e < C * C)
            R.p[j] = *reinterpret_cast<const u32x4*>(P + e);
    }
#pragma unroll
    for (int j = 0; j < S::NLDU; ++j) {
        const int e = (j * NT + tid) * S::VEC;
        if (e < C * BV) {
            const int t = e / BV, c = e % BV;
            R.u[j] = *reinterpret_cast<const u32x4*>(Ut + t * D + slice * BV + c);
        }
    }
    if (tid < D / 4)
        R.gam = *reinterpret_cast<const f32x4*>(a.gam + rec * D + tid * 4);
}

template <typename E, int D, int C, int BV>
__global__ __launch_bounds__(NT, 1) void chunk_state_kernel(StateArgs a)
{
    typedef StateShape<E, D, C, BV> S;
    typedef Mma<E> MM;
    constexpr int NB = S::NB, VEC = S::VEC, LDA = S::LDA, LDT = S::LDT, LDU = S::LDU;
    constexpr int KTS = D / 16;          // k-tiles of the state rows
    constexpr int NKS = D / MM::KB;      // MFMA steps over the state rows
    constexpr int NKC = C / MM::KB;      // MFMA steps over the chunk's tokens

    extern __shared__ __align__(16) unsigned char smem[];
    E* sW = reinterpret_cast<E*>(smem);
    E* sQ = reinterpret_cast<E*>(smem + al256((size_t)C * LDA * sizeof(E)));
    E* sKT = reinterpret_cast<E*>(smem + 2 * al256((size_t)C * LDA * sizeof(E)));
    E* sP = reinterpret_cast<E*>((unsigned char*)sKT + al256((size_t)D * LDT * sizeof(E)));
    E* sU = reinterpret_cast<E*>((unsigned char*)sP + al256((size_t)C * LDT * sizeof(E)));
    float* sGam = reinterpret_cast<float*>((unsigned char*)sU + al256((size_t)C * LDU * sizeof(E)));

    // Workgroup -> (sequence*head, column slice).  The NS slices of one
    // (b,h) read the same chunk records: give them the same blockIdx % 8 so
    // they land on the same XCD and share its L2.
    const int64_t x = blockIdx.x;
    const int64_t grp = x / (8 * S::NS);
    const int within = (int)(x % (8 * S::NS));
    const int slice = within / 8;
    const int64_t bh = grp * 8 + within % 8;
    if (bh >= a.nbh)
        return;
    const int64_t b = bh / a.H, h = bh - b * a.H;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gq = lane >> 4, cl = lane & 15;
    const int col = slice * BV + 16 * wave + cl;     // this lane's state / output column

    f32x4 St[KTS];
    {
        const float* s0 = a.S0 ? a.S0 + bh * D * D : nullptr;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                St[kt][i] = s0 ? s0[(16 * kt + 4 * gq + i) * D + col] : 0.f;
    }

    StateRegs<E, D, C, BV> R;
    const int64_t rec0 = bh * a.NC;
    state_load(a, rec0, slice, R, tid);
    E* o = (E*)a.o;

    for (int64_t n = 0; n < a.NC; ++n) {
        __syncthreads();  // previous chunk done reading LDS
#pragma unroll
        for (int j = 0; j < S::NLD; ++j) {
            const int e = (j * NT + tid) * VEC, t = e / D, c = e % D;
            *reinterpret_cast<u32x4*>(sW + t * LDA + c) = R.w[j];
            *reinterpret_cast<u32x4*>(sQ + t * LDA + c) = R.q[j];
            float kv[VEC];
            unpack<E>(R.kh[j], kv);
#pragma unroll
            for (int xx = 0; xx < VEC; ++xx)
                sKT[(c + xx) * LDT + t] = from_f32<E>(kv[xx]);
        }
#pragma unroll
        for (int j = 0; j < S::NLDP; ++j) {
            const int e = (j * NT + tid) * VEC;
            if (e < C * C)
                *reinterpret_cast<u32x4*>(sP + (e / C) * LDT + e % C) = R.p[j];
        }
#pragma unroll
        for (int j = 0; j < S::NLDU; ++j) {
            const int e = (j * NT + tid) * VEC;
            if (e < C * BV)
                *reinterpret_cast<u32x4*>(sU + (e / BV) * LDU + e % BV) = R.u[j];
        }
        if (tid < D / 4)
            *reinterpret_cast<f32x4*>(sGam + tid * 4) = R.gam;
        if (n + 1 < a.NC)
            state_load(a, rec0 + n + 1, slice, R, tid);
        __syncthreads();

        // B operands from the chunk-start state.
        typename MM::Frag SB[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            SB[ks] = MM::from_acc(&St[ks * MM::KT]);

        // Delta = U~ - W S  (W is stored negated).
        f32x4 dl[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dl[mt][i] = to_f32(sU[(16 * mt + 4 * gq + i) * LDU + 16 * wave + cl]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                dl[mt] = MM::mma(MM::load(sW + 16 * mt * LDA + ks * MM::KB, LDA, lane), SB[ks], dl[mt]);
        }
        typename MM::Frag DB[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            DB[kc] = MM::from_acc(&dl[kc * MM::KT]);

        // O = Q~ S + P Delta  (P is lower triangular: skip all-zero steps).
        f32x4 ot[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            ot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                ot[mt] = MM::mma(MM::load(sQ + 16 * mt * LDA + ks * MM::KB, LDA, lane), SB[ks], ot[mt]);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                if (kc * MM::KT <= mt)
                    ot[mt] = MM::mma(MM::load(sP + 16 * mt * LDT + kc * MM::KB, LDT, lane), DB[kc], ot[mt]);
        }

        // S <- diag(gamma) S + K^T Delta.
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(sGam + 16 * kt + 4 * gq);
            St[kt] = St[kt] * gm;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                St[kt] = MM::mma(MM::load(sKT + 16 * kt * LDT + kc * MM::KB, LDT, lane), DB[kc], St[kt]);
        }

        // Store this chunk's outputs (valid rows only).
        const int64_t t0 = n * C;
        const int L = (int)min((int64_t)C, a.T - t0);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * gq + i;
                if (r < L)
                    o[((b * a.T + t0 + r) * a.H + h) * D + col] = from_f32<E>(ot[mt][i]);
            }
    }

    if (a.S_out) {
        float* so = a.S_out + bh * D * D;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[(16 * kt + 4 * gq + i) * D + col] = St[kt][i];
    }
}

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

int cu_count()
{
    static int counts[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (counts[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        counts[dev] = n;
    }
    return counts[dev];
}

template <typename E, int D, int C>
hipError_t launch_staged_t(const gdr2_fwd_args& a, hipStream_t stream)
{
    constexpr int BV = 64;
    typedef PrepShape<E, D, C> PS;
    typedef StateShape<E, D, C, BV> SS;
    const Layout L = staged_layout(a.B, a.H, a.T, D, C, (int)sizeof(E));
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);

    PrepArgs pa;
    pa.q = a.q; pa.k = a.k; pa.v = a.v; pa.b = a.b; pa.w = a.w; pa.g = a.g;
    pa.bw = a.b_width; pa.ww = a.w_width; pa.gw = a.g_width;
    pa.T = a.T; pa.H = a.H; pa.NC = ceil_div(a.T, C); pa.nrec = L.nrec;
    pa.Wn = ws + L.wn; pa.Ut = ws + L.ut; pa.Kh = ws + L.kh; pa.Qt = ws + L.qt; pa.P = ws + L.p;
    pa.gam = reinterpret_cast<float*>(ws + L.gam);

    static const hipError_t attr1 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&chunk_prep_kernel<E, D, C>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)PS::SMEM);
    static const hipError_t attr2 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&chunk_state_kernel<E, D, C, BV>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)SS::SMEM);
    if (attr1 != hipSuccess)
        return attr1;
    if (attr2 != hipSuccess)
        return attr2;

    const int64_t grid1 = std::min<int64_t>(L.nrec, (int64_t)cu_count());
    hipLaunchKernelGGL((chunk_prep_kernel<E, D, C>), dim3((unsigned)grid1), dim3(NT), PS::SMEM, stream, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;

    StateArgs sa;
    sa.Wn = pa.Wn; sa.Ut = pa.Ut; sa.Kh = pa.Kh; sa.Qt = pa.Qt; sa.P = pa.P; sa.gam = pa.gam;
    sa.S0 = a.S0; sa.S_out = a.S_out; sa.o = a.o;
    sa.T = a.T; sa.H = a.H; sa.NC = pa.NC; sa.nbh = a.B * a.H;
    const int64_t grid2 = ceil_div(sa.nbh, 8) * 8 * SS::NS;
    hipLaunchKernelGGL((chunk_state_kernel<E, D, C, BV>), dim3((unsigned)grid2), dim3(NT), SS::SMEM, stream, sa);
    return hipGetLastError();
}

}  // namespace

size_t staged_workspace_bytes(const gdr2_fwd_args& a)
{
    if (a.B * a.H * a.T == 0)
        return 0;
    return staged_layout(a.B, a.H, a.T, (int)a.Dk, a.chunk, a.dtype == GDR2_BF16 ? 2 : 4).total;
}

hipError_t launch_forward_staged(const gdr2_fwd_args& a, hipStream_t stream)
{
    const int D = (int)a.Dk, C = a.chunk;
    if (a.dtype == GDR2_BF16) {
        if (D == 128)
            return C == 64 ? launch_staged_t<bf16, 128, 64>(a, stream) : launch_staged_t<bf16, 128, 32>(a, stream);
        return C == 64 ? launch_staged_t<bf16, 64, 64>(a, stream) : launch_staged_t<bf16, 64, 32>(a, stream);
    }
    if (D == 128)
        return launch_staged_t<float, 128, 32>(a, stream);
    return C == 64 ? launch_staged_t<float, 64, 64>(a, stream) : launch_staged_t<float, 64, 32>(a, stream);
}

hipError_t launch_state_copy(const float* src, float* dst, int64_t n, hipStream_t stream)
{
    const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), 4096);
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError();
}

}  // namespace gdr2
