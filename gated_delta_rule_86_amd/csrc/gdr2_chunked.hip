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
//   Wn [C][D] = -W,  Ut [C][D] = U~,  Kh [D][C] = K^ transposed,  Qt [C][D] = Q~,
//   P [C][C],  gam [D] fp32.   Records are ordered (b*H + h)*NC + n.
//   Wn, Qt, Kh and P (the A operands of the state kernel) store their
//   contraction dimension in MFMA k-order (perm_chunk); U~ is plain.
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

// ---------------------------------------------------------------------------
// chunk_prep: 512 threads (8 waves), one workgroup per CU, looping over chunk
// records with the next chunk's inputs prefetched into registers while the
// current one computes.
//
// Decay references.  A chunk is split into halves of 32 tokens; Gh(t) is the
// cumulative log2-decay at the end of the previous half (0 for the first).
//   E~_t = e_t 2^G_t,  Q~_t = q_t 2^G_t            (chunk reference, <= |e|,|q|)
//   Kr_s = k_s 2^(Gh(s) - G_s)                      (own half's reference)
//   E^_t = e_t 2^(G_t - Gh(t)),  Q^_t likewise       (second half only)
// A 16x16 tile (I, J) of M (or P) with both blocks in the same half is
// E^_I Kr_J^T (E~ in the first half), and with I in the second half and J in
// the first it is E~_I Kr_J^T: each product equals the wanted
// e_t k_s 2^(G_t - G_s) with no factor above 2^(half span).  The half span is
// guarded by kSpanMax; a chunk beyond it takes an exact pair-by-pair path for
// its same-half tiles.
//
// WY solve.  [W | U~] = (I + M)^-1 [E~ | u] by blocked forward substitution
// over the four 16-row blocks:  R_I = RHS_I - sum_{J<I} M_IJ [W|U~]_J,
// [W|U~]_I = X_II R_I, with X_II = (I + M_II)^-1 from a 16-lane substitution.
// Each wave owns 32 columns of the right-hand side and keeps its solved blocks
// in MFMA accumulators, which are the B operands of the next blocks.
// ---------------------------------------------------------------------------
constexpr int NTP = 512;           // threads of the prep kernel
constexpr int NWP = NTP / 64;      // its waves

template <typename E, int D, int C>
struct PrepShape {
    static constexpr int NB = C / 16;                       // 16-token blocks
    static constexpr int NH = C / 32;                       // 32-token halves
    static constexpr int VEC = 16 / (int)sizeof(E);         // elements per 16-byte access
    static constexpr int NLD = (C * D + NTP * VEC - 1) / (NTP * VEC);  // [C][D] loads per thread
    static constexpr int NLDG = (C * D + NTP * 4 - 1) / (NTP * 4);     // fp32 g loads per thread
    static constexpr int LDA = D + 16 / (int)sizeof(E);     // [rows][D] E arrays in LDS
    static constexpr int LDC = C + 16 / (int)sizeof(E);     // [C][C] E arrays (P, -M)
    static constexpr int LDX = 20;                          // fp32 16x16 blocks
    static constexpr int PARTS = NTP / D;                   // prefix-sum parts per channel
    static constexpr size_t SZ_G = (size_t)C * D * 4;
    static constexpr size_t SZ_A = (size_t)C * LDA * sizeof(E);
    static constexpr size_t SZ_AH = (size_t)(C - 32) * LDA * sizeof(E);
    static constexpr size_t SZ_CC = (size_t)C * LDC * sizeof(E);
    static constexpr size_t SZ_BLK = (size_t)NB * 16 * LDX * 4;
    static constexpr size_t OFF_G = 0;                             // sG
    static constexpr size_t OFF_E = OFF_G + al256(SZ_G);           // sE  (E~, then -W)
    static constexpr size_t OFF_Q = OFF_E + al256(SZ_A);           // sQ  (Q~)
    static constexpr size_t OFF_KR = OFF_Q + al256(SZ_A);          // sKr
    static constexpr size_t OFF_U = OFF_KR + al256(SZ_A);          // sU  (u, then U~)
    static constexpr size_t OFF_EH = OFF_U + al256(SZ_A);          // sEh (second half)
    static constexpr size_t OFF_QH = OFF_EH + al256(SZ_AH);        // sQh (second half)
    static constexpr size_t OFF_MB = OFF_QH + al256(SZ_AH);        // sMb (-M below the diagonal blocks)
    static constexpr size_t OFF_P = OFF_MB + al256(SZ_CC);         // sP  (scores)
    static constexpr size_t OFF_MD = OFF_P + al256(SZ_CC);         // sMd (-M diagonal blocks, fp32)
    static constexpr size_t OFF_XD = OFF_MD + al256(SZ_BLK);       // sXd (X_II, fp32)
    static constexpr size_t OFF_T = OFF_XD + al256(SZ_BLK);        // tables [NH][D] + partials
    static constexpr size_t SZ_T = ((size_t)NH * D + (size_t)PARTS * D) * 4;
    static constexpr size_t OFF_FLAG = OFF_T + al256(SZ_T);
    static constexpr size_t SMEM = OFF_FLAG + 256;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(C == 32 || C == 64, "chunk");
    static_assert(D % VEC == 0 && NTP % D == 0 && C % PARTS == 0, "shape");
    static_assert((2 * D) % (NWP * 16) == 0, "right-hand-side columns per wave");
};

// Raw inputs of one chunk as loaded (bit patterns; width-1 gates keep their
// scalar in element 0 and are broadcast when used).
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

// 16 bytes of E as a vector.
template <typename E> struct VecOf;
template <> struct VecOf<bf16> { typedef bf16x8 T; };
template <> struct VecOf<float> { typedef f32x4 T; };

// The scalar held in element 0 of a width-1 gate's raw bits.
template <typename E>
__device__ __forceinline__ float scalar0(const u32x4& r);
template <>
__device__ __forceinline__ float scalar0<bf16>(const u32x4& r)
{
    return __uint_as_float(r[0] << 16);
}
template <>
__device__ __forceinline__ float scalar0<float>(const u32x4& r)
{
    return __uint_as_float(r[0]);
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
__device__ __forceinline__ void stg16(void* p, u32x4 v)
{
    *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ u32x4 lds16(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void sts16(void* p, u32x4 v)
{
    *reinterpret_cast<u32x4*>(p) = v;
}

// MFMA k-order of the state kernel's A operands (bf16): within every block of
// 32 elements along k, physical 16-byte chunk g holds logical elements
// 4g..4g+3 and 16+4g..16+4g+3 -- exactly the k values lane group g of a
// 16x16x32 MFMA takes from accumulator-layout B operands -- so a fragment is
// one 16-byte LDS read.  fp32 operands are already in that order (identity).
// perm_chunk: the 16 bytes of physical chunk pc, gathered from a row held in
// logical order.
template <typename E>
__device__ __forceinline__ u32x4 perm_chunk(const E* row, int pc);
template <>
__device__ __forceinline__ u32x4 perm_chunk<bf16>(const bf16* row, int pc)
{
    const bf16* p = row + 32 * (pc >> 2) + 4 * (pc & 3);
    const unsigned int* lo = reinterpret_cast<const unsigned int*>(p);
    const unsigned int* hi = reinterpret_cast<const unsigned int*>(p + 16);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
template <>
__device__ __forceinline__ u32x4 perm_chunk<float>(const float* row, int pc)
{
    return *reinterpret_cast<const u32x4*>(row + 4 * pc);
}
// Logical index of element u of physical chunk pc (the same order).
template <typename E>
__device__ __forceinline__ int perm_index(int pc, int u)
{
    if (sizeof(E) == 4)
        return 4 * pc + u;
    return 32 * (pc >> 2) + 4 * (pc & 3) + (u < 4 ? u : 12 + u);
}

// Bits of one element, for width-1 gates.
template <typename E>
__device__ __forceinline__ unsigned int ld_bits(const E* p);
template <>
__device__ __forceinline__ unsigned int ld_bits<bf16>(const bf16* p)
{
    return *reinterpret_cast<const unsigned short*>(p);
}
template <>
__device__ __forceinline__ unsigned int ld_bits<float>(const float* p)
{
    return __float_as_uint(*p);
}

// Chunk record -> position.  Token row r of the chunk is element offset
// ((b*T + t0 + r)*H + h) of the [B,T,H,.] tensors.
struct ChunkPos {
    int64_t row0;     // (b*T + t0)*H + h
    int L;            // valid tokens (>= 1)
};

__device__ __forceinline__ ChunkPos chunk_pos(int64_t rec, int64_t NC, int64_t T, int64_t H, int C)
{
    const int64_t bh = rec / NC, n = rec - bh * NC;
    const int64_t b = bh / H, h = bh - b * H;
    const int64_t t0 = n * C;
    ChunkPos p;
    p.row0 = (b * T + t0) * H + h;
    p.L = (int)min((int64_t)C, T - t0);
    return p;
}

// Issue the loads of one chunk.  Rows past the valid length re-read the last
// valid row (always in bounds) and are zeroed where they are used, so no load
// sits under a per-lane branch.  FULL: every gate has full width, and the
// load sequence is straight-line code.
template <bool FULL, typename E, int D, int C>
__device__ __forceinline__ void prep_load_gates(const PrepArgs& a, const ChunkPos& cp,
                                                PrepRegs<E, D, C>& R, int tid)
{
    typedef PrepShape<E, D, C> S;
#pragma unroll
    for (int j = 0; j < S::NLDG; ++j) {
        const int e = (j * NTP + tid) * 4, t = min(e / D, cp.L - 1), c = e % D;
        const int64_t row = cp.row0 + (int64_t)t * a.H;
        if (e < C * D) {
            if (FULL || a.gw != 1)
                R.g[j] = __builtin_bit_cast(f32x4, ldg16(a.g + row * D + c));
            else
                R.g[j][0] = a.g[row];
        }
    }
}

template <bool FULL, typename E, int D, int C>
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
        const int e = (j * NTP + tid) * S::VEC, t = min(e / D, cp.L - 1), c = e % D;
        const int64_t row = cp.row0 + (int64_t)t * a.H, off = row * D + c;
        if (e < C * D) {
            R.k[j] = ldg16(k + off);
            R.q[j] = ldg16(q + off);
            R.v[j] = ldg16(v + off);
            if (FULL) {
                R.b[j] = ldg16(b + off);
                R.w[j] = ldg16(w + off);
            }
        }
    }
    if (!FULL) {
#pragma unroll
        for (int j = 0; j < S::NLD; ++j) {
            const int e = (j * NTP + tid) * S::VEC, t = min(e / D, cp.L - 1), c = e % D;
            const int64_t row = cp.row0 + (int64_t)t * a.H, off = row * D + c;
            if (e < C * D) {
                if (a.bw == 1)
                    R.b[j][0] = ld_bits<E>(b + row);
                else
                    R.b[j] = ldg16(b + off);
                if (a.ww == 1)
                    R.w[j][0] = ld_bits<E>(w + row);
                else
                    R.w[j] = ldg16(w + off);
            }
        }
    }
}

// A operand of X_II (16x16, fp32 in LDS) for one bf16 MFMA step of k = 32:
// the second k-tile is zero.  fp32 MFMA steps are k = 16 and need no padding.
template <typename E> struct XiiFrag;
template <> struct XiiFrag<bf16> {
    static __device__ __forceinline__ Mma<bf16>::Frag load(const float* p, int ld, int lane) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(p + (lane & 15) * ld + 4 * (lane >> 4));
        return Mma<bf16>::pack(lo, f32x4{0.f, 0.f, 0.f, 0.f});
    }
};
template <> struct XiiFrag<float> {
    static __device__ __forceinline__ Mma<float>::Frag load(const float* p, int ld, int lane) {
        return Mma<float>::load(p, ld, lane);
    }
};

template <bool FULL, typename E, int D, int C>
__global__ __launch_bounds__(NTP) void chunk_prep_kernel(PrepArgs a)
{
    typedef PrepShape<E, D, C> S;
    typedef Mma<E> MM;
    constexpr int NB = S::NB, NH = S::NH, VEC = S::VEC, LDA = S::LDA, LDC = S::LDC, LDX = S::LDX;

    extern __shared__ __align__(16) unsigned char smem[];
    float* sG = reinterpret_cast<float*>(smem + S::OFF_G);     // [C][D] cumulative log2-decay
    E* sE = reinterpret_cast<E*>(smem + S::OFF_E);             // [C][LDA] E~, then -W
    E* sQ = reinterpret_cast<E*>(smem + S::OFF_Q);             // [C][LDA] Q~
    E* sKr = reinterpret_cast<E*>(smem + S::OFF_KR);           // [C][LDA] Kr
    E* sU = reinterpret_cast<E*>(smem + S::OFF_U);             // [C][LDA] u, then U~
    E* sEh = reinterpret_cast<E*>(smem + S::OFF_EH);           // [C-32][LDA] E^ (rows 32..)
    E* sQh = reinterpret_cast<E*>(smem + S::OFF_QH);           // [C-32][LDA] Q^ (rows 32..)
    E* sMb = reinterpret_cast<E*>(smem + S::OFF_MB);           // [C][LDC] -M, blocks below the diagonal
    E* sP = reinterpret_cast<E*>(smem + S::OFF_P);             // [C][LDC] P
    float* sMd = reinterpret_cast<float*>(smem + S::OFF_MD);   // [NB][16][LDX] -M_II
    float* sXd = reinterpret_cast<float*>(smem + S::OFF_XD);   // [NB][16][LDX] X_II
    float* sFk = reinterpret_cast<float*>(smem + S::OFF_T);    // [NH][D] 2^(G_last - Gh)
    float* sPart = sFk + NH * D;                               // [PARTS][D]
    int* sFlag = reinterpret_cast<int*>(smem + S::OFF_FLAG);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gq = lane >> 4, cl = lane & 15;
    PrepRegs<E, D, C> R;
    int64_t rec = blockIdx.x;
    if (rec >= a.nrec)
        return;
    {
        const ChunkPos cp = chunk_pos(rec, a.NC, a.T, a.H, C);
        prep_load_gates<FULL>(a, cp, R, tid);
        prep_load_tokens<FULL>(a, cp, R, tid);
    }

    for (; rec < a.nrec; rec += gridDim.x) {
        const ChunkPos cp = chunk_pos(rec, a.NC, a.T, a.H, C);
        const int64_t next = rec + gridDim.x;
        const ChunkPos np = chunk_pos(next < a.nrec ? next : rec, a.NC, a.T, a.H, C);
        E* gWn = (E*)a.Wn + rec * C * D;
        E* gUt = (E*)a.Ut + rec * C * D;
        E* gKt = (E*)a.Kh + rec * C * D;
        E* gQt = (E*)a.Qt + rec * C * D;
        E* gP = (E*)a.P + rec * C * C;
        float* gGam = a.gam + rec * D;
        const int bw = FULL ? D : a.bw, ww = FULL ? D : a.ww, gw = FULL ? D : a.gw;

        __syncthreads();  // the previous chunk is done with every LDS region
        // Phase 1: log-decay into LDS in log2 units (padding rows: 0).
#pragma unroll
        for (int j = 0; j < S::NLDG; ++j) {
            const int e = (j * NTP + tid) * 4;
            if (e < C * D) {
                f32x4 gv = R.g[j];
                if (gw == 1)
                    gv = f32x4{gv[0], gv[0], gv[0], gv[0]};
                *reinterpret_cast<f32x4*>(sG + e) = (e / D < cp.L) ? gv * kLog2e : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (tid == 0)
            *sFlag = 0;
        if (next < a.nrec)
            prep_load_gates<FULL>(a, np, R, tid);
        __syncthreads();

        // Phase 2: inclusive prefix sum over the chunk's tokens, per channel.
        {
            constexpr int RP = C / S::PARTS;
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
#pragma unroll
            for (int pp = 0; pp < S::PARTS - 1; ++pp)
                off += pp < p ? sPart[pp * D + i] : 0.f;
#pragma unroll
            for (int r = 0; r < RP; ++r)
                sG[(p * RP + r) * D + i] += off;
        }
        __syncthreads();

        // Phase 3: decay-referenced operands, as 16-byte LDS rows.
        if (tid < NH * D) {
            const int h = tid / D, i = tid % D;
            const float gl = sG[(C - 1) * D + i];
            const float gh = h ? sG[31 * D + i] : 0.f;
            sFk[tid] = fast_exp2(gl - gh);
            if (h == 0)
                gGam[i] = fast_exp2(gl);
        }
#pragma unroll
        for (int j = 0; j < S::NLD; ++j) {
            const int e = (j * NTP + tid) * VEC;
            if (e >= C * D)
                continue;
            const int t = e / D, c = e % D, h = t >> 5;
            const bool valid = t < cp.L;
            float kk[VEC], qq[VEC], bb[VEC], vv[VEC], ww_[VEC];
            unpack<E>(R.k[j], kk);
            unpack<E>(R.q[j], qq);
            unpack<E>(R.v[j], vv);
            unpack<E>(R.b[j], bb);
            unpack<E>(R.w[j], ww_);
            const float bs = scalar0<E>(R.b[j]), ws = scalar0<E>(R.w[j]);
            const float* Gt = sG + t * D + c;
            const float* Gh = sG + 31 * D + c;
            typename VecOf<E>::T ve, vq, vk, vu, veh, vqh;
            bool steep = false;
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                const float kx = valid ? kk[x] : 0.f;
                const float qx = valid ? qq[x] : 0.f;
                const float bx = bw == 1 ? bs : bb[x];
                const float wx = valid ? (ww == 1 ? ws : ww_[x]) : 0.f;
                const float G = Gt[x];
                const float gh = h ? Gh[x] : 0.f;
                const float d2 = G - gh;                  // <= 0 for decays g <= 0
                steep |= fabsf(d2) > kSpanMax || G > kSpanMax;
                const float e2g = fast_exp2(G);
                const float ekr = fast_exp2(-d2);
                const float ex = bx * kx;
                ve[x] = from_f32<E>(ex * e2g);
                vq[x] = from_f32<E>(qx * e2g);
                vk[x] = from_f32<E>(kx * ekr);
                vu[x] = from_f32<E>(wx * vv[x]);
                if (h) {
                    const float eh = fast_exp2(d2);
                    veh[x] = from_f32<E>(ex * eh);
                    vqh[x] = from_f32<E>(qx * eh);
                }
            }
            if (steep)
                *sFlag = 1;
            sts16(sE + t * LDA + c, __builtin_bit_cast(u32x4, ve));
            sts16(sQ + t * LDA + c, __builtin_bit_cast(u32x4, vq));
            sts16(sKr + t * LDA + c, __builtin_bit_cast(u32x4, vk));
            sts16(sU + t * LDA + c, __builtin_bit_cast(u32x4, vu));
            if (h) {
                sts16(sEh + (t - 32) * LDA + c, __builtin_bit_cast(u32x4, veh));
                sts16(sQh + (t - 32) * LDA + c, __builtin_bit_cast(u32x4, vqh));
            }
        }
        if (next < a.nrec)
            prep_load_tokens<FULL>(a, np, R, tid);
        __syncthreads();

        // Phase 4: tiles of M (-> -M in sMb / sMd) and P (-> sP), MFMA; then
        // K^ = Kr * 2^(G_last - Gh) leaves transposed ([D][C], tokens
        // contiguous: the layout in which it is an A operand of the state
        // update), VEC lanes per row of K^T.
        const bool guard = *sFlag != 0;
        {
            constexpr int NTILE = NB * (NB + 1) / 2;
            const int kind = wave / 4, sub = wave % 4;
#pragma unroll
            for (int r = 0; r < (NTILE + 3) / 4; ++r) {
                const int tile = sub + 4 * r;
                if (tile >= NTILE)
                    break;
                int I = 0;
                while ((I + 1) * (I + 2) / 2 <= tile)
                    ++I;
                const int J = tile - I * (I + 1) / 2;
                const bool same_half = (I >> 1) == (J >> 1);
                if (guard)
                    break;
                const E* A = (I >= 2 && same_half) ? (kind ? sQh : sEh) + (16 * I - 32) * LDA
                                                   : (kind ? sQ : sE) + 16 * I * LDA;
                const E* Bm = sKr + 16 * J * LDA;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < D; k0 += MM::KB)
                    acc = MM::mma(MM::load(A + k0, LDA, lane), MM::load(Bm + k0, LDA, lane), acc);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int rr = 16 * I + 4 * gq + ii, s = 16 * J + cl;
                    if (kind == 0) {
                        const float m = s < rr ? -acc[ii] : 0.f;
                        if (I == J)
                            sMd[(I * 16 + 4 * gq + ii) * LDX + cl] = m;
                        sMb[rr * LDC + s] = from_f32<E>(I == J ? 0.f : m);
                    } else {
                        sP[rr * LDC + s] = from_f32<E>(s <= rr ? acc[ii] : 0.f);
                    }
                }
            }
            // Tiles above the block diagonal are zero in both.
            for (int e = tid; e < C * C; e += NTP) {
                const int rr = e / C, s = e % C;
                if ((s >> 4) > (rr >> 4)) {
                    sP[rr * LDC + s] = from_f32<E>(0.f);
                    sMb[rr * LDC + s] = from_f32<E>(0.f);
                }
            }
            for (int e = tid; e < D * (C / VEC); e += NTP) {
                const int tg = e % (C / VEC), i = e / (C / VEC);
                float x[VEC];
                if (!guard) {
                    const float f = sFk[((tg * VEC) >> 5) * D + i];
#pragma unroll
                    for (int u = 0; u < VEC; ++u)
                        x[u] = to_f32(sKr[perm_index<E>(tg, u) * LDA + i]) * f;
                } else {
                    // steep decay: K^ = k 2^(G_last - G) directly from the inputs
                    const E* k = (const E*)a.k;
                    const float gl = sG[(C - 1) * D + i];
#pragma unroll
                    for (int u = 0; u < VEC; ++u) {
                        const int t = perm_index<E>(tg, u);
                        const float kv = t < cp.L ? to_f32(k[(cp.row0 + (int64_t)t * a.H) * D + i]) : 0.f;
                        x[u] = kv * fast_exp2(gl - sG[t * D + i]);
                    }
                }
                stg16(gKt + i * C + tg * VEC, pack_vec<E>(x));
            }
        }
        if (guard) {
            // Exact tiles for a chunk whose decay is too steep for the
            // referenced form: every pair s <= t from the raw inputs.
            __syncthreads();
            const E* q = (const E*)a.q;
            const E* k = (const E*)a.k;
            const E* b = (const E*)a.b;
            for (int e = tid; e < C * C; e += NTP) {
                const int rr = e / C, s = e % C;
                float m = 0.f, p = 0.f;
                if (s <= rr && rr < cp.L) {
                    const int64_t xr = cp.row0 + (int64_t)rr * a.H, xs = cp.row0 + (int64_t)s * a.H;
                    for (int i = 0; i < D; ++i) {
                        const float dec = fast_exp2(sG[rr * D + i] - sG[s * D + i]);
                        const float ks = to_f32(k[xs * D + i]) * dec;
                        const float br = to_f32(bw == 1 ? b[xr] : b[xr * D + i]);
                        m += br * to_f32(k[xr * D + i]) * ks;
                        p += to_f32(q[xr * D + i]) * ks;
                    }
                }
                const float mn = s < rr ? -m : 0.f;
                if ((rr >> 4) == (s >> 4))
                    sMd[((rr >> 4) * 16 + (rr & 15)) * LDX + (s & 15)] = mn;
                sMb[rr * LDC + s] = from_f32<E>((rr >> 4) == (s >> 4) ? 0.f : mn);
                sP[rr * LDC + s] = from_f32<E>(p);
            }
        }
        __syncthreads();

        // Phase 5: wave 0 inverts the diagonal blocks by forward substitution
        // (one lane per column, fp32); the other waves write P out.
        if (wave == 0) {
            if (gq < NB) {
                const float* m = sMd + gq * 16 * LDX;
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = r == cl ? 1.f : 0.f;
#pragma unroll
                    for (int c2 = 0; c2 < r; ++c2)
                        acc += m[r * LDX + c2] * x[c2];
                    x[r] = acc;
                    // keep each row's LDS reads next to their use (bounded registers)
                    __asm__ __volatile__("" ::: "memory");
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sXd[(gq * 16 + r) * LDX + cl] = x[r];
            }
        } else {
            for (int e = tid - 64; e < C * (C / VEC); e += NTP - 64) {
                const int rr = e / (C / VEC), cg = e % (C / VEC);
                stg16(gP + rr * C + cg * VEC, perm_chunk<E>(sP + rr * LDC, cg));
            }
            for (int e = tid - 64; e < C * (D / VEC); e += NTP - 64) {
                const int rr = e / (D / VEC), cg = e % (D / VEC);
                stg16(gQt + rr * D + cg * VEC, perm_chunk<E>(sQ + rr * LDA, cg));
            }
        }
        __syncthreads();

        // Phase 6: blocked substitution for [W | U~], 2D/8 right-hand-side
        // columns per wave (waves 0-3: E~ -> W, waves 4-7: u -> U~), solved
        // blocks kept as MFMA accumulators.
        {
            constexpr int NCT = 2 * D / NWP / 16;     // 16-column tiles per wave
            E* rhs = wave < NWP / 2 ? sE : sU;
            const int c0 = 16 * NCT * (wave % (NWP / 2));
            f32x4 sol[NCT][NB];
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int I = 0; I < NB; ++I)
                    sol[n][I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 res[NCT];
#pragma unroll
                for (int n = 0; n < NCT; ++n) {
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        res[n][ii] = to_f32(rhs[(16 * I + 4 * gq + ii) * LDA + c0 + 16 * n + cl]);
                }
#pragma unroll
                for (int kk = 0; kk < I; kk += MM::KT) {
                    const typename MM::Frag am = MM::load(sMb + 16 * I * LDC + 16 * kk, LDC, lane);
#pragma unroll
                    for (int n = 0; n < NCT; ++n)
                        res[n] = MM::mma(am, MM::from_acc(&sol[n][kk]), res[n]);
                }
                const typename MM::Frag ax = XiiFrag<E>::load(sXd + I * 16 * LDX, LDX, lane);
#pragma unroll
                for (int n = 0; n < NCT; ++n) {
                    const f32x4 pair[2] = {res[n], res[n]};
                    sol[n][I] = MM::mma(ax, MM::from_acc(pair), f32x4{0.f, 0.f, 0.f, 0.f});
                }
            }
            const float sg = wave < NWP / 2 ? -1.f : 1.f;   // W leaves negated
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        rhs[(16 * I + 4 * gq + ii) * LDA + c0 + 16 * n + cl] = from_f32<E>(sg * sol[n][I][ii]);
        }
        __syncthreads();
        for (int e = tid; e < C * (D / VEC); e += NTP) {
            const int rr = e / (D / VEC), cg = e % (D / VEC);
            stg16(gWn + rr * D + cg * VEC, perm_chunk<E>(sE + rr * LDA, cg));
            stg16(gUt + rr * D + cg * VEC, lds16(sU + rr * LDA + cg * VEC));
        }
    }
}

// ---------------------------------------------------------------------------
// chunk_state: carries the fp32 state through the chunks of one sequence and
// head, BV value columns per workgroup (16 per wave), and writes o.
//
// The factors of a chunk (-W, Q~, K^T, P, this slice of U~, gamma) are copied
// from the workspace straight into LDS with global_load_lds_dwordx4 (no
// register staging), double buffered: the copy of chunk n + 1 is in flight
// while chunk n computes.  The two buffers are separate static LDS objects so
// that reads of one are never ordered behind the copies into the other.
// Rows are padded by 16 bytes (one extra copy slot per row, filled with a
// harmless duplicate) so that fragment reads of 16 consecutive rows hit 16
// different bank groups.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, int BV>
struct StateShape {
    static constexpr int NB = C / 16;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int VEC = 16 / ES;
    static constexpr int NS = D / BV;                       // column slices per (b,h)
    static constexpr int LDA = D + VEC;                     // W, Q~ rows (elements)
    static constexpr int LDT = C + VEC;                     // K^T, P rows
    static constexpr int LDU = BV + VEC;                    // U~ slice rows
    static constexpr int LDO = 16 + VEC;                    // per-wave output staging rows
    static constexpr int OFF_W = 0;                         // element offsets in one buffer
    static constexpr int OFF_Q = OFF_W + C * LDA;
    static constexpr int OFF_KT = OFF_Q + C * LDA;
    static constexpr int OFF_P = OFF_KT + D * LDT;
    static constexpr int OFF_U = OFF_P + C * LDT;
    static constexpr int OFF_G = OFF_U + C * LDU;           // gamma: D floats
    static constexpr int BUF = OFF_G + D * 4 / ES;          // elements per buffer
    static constexpr size_t SZ_O = (size_t)(NT / 64) * C * LDO * ES;
    // double buffering when two buffers fit (every bf16 shape); else one
    static constexpr int NBUF = 2 * (size_t)BUF * ES + SZ_O <= 160 * 1024 ? 2 : 1;
    static constexpr size_t SMEM = NBUF * (size_t)BUF * ES + SZ_O;
    static_assert(BV == 16 * (NT / 64), "one 16-column tile per wave");
    static_assert(SMEM <= 160 * 1024, "LDS budget");
};

typedef __attribute__((address_space(3))) void lds_void;

// Copy R rows of RB bytes (global rows GS bytes apart) into LDS rows of
// RB + 16 bytes, 16 bytes per lane per instruction, instructions spread over
// the waves (instruction j belongs to wave j % 4).  Copy slot s of the tile
// is LDS byte 16*s; the last slot of each row is padding and receives a
// duplicate of the row's first 16 bytes.  The per-lane source offsets are the
// same for every chunk and are computed once.
template <int R, int RB>
struct TileCopy {
    static constexpr int SPR = RB / 16 + 1, TOTAL = R * SPR, NINST = (TOTAL + 63) / 64;
    static constexpr int PER_WAVE = (NINST + NT / 64 - 1) / (NT / 64);
    int off[PER_WAVE];     // source byte offset, or -1 where the lane has no slot
    __device__ __forceinline__ void init(int64_t gs, int wave, int lane) {
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u) {
            const int j = u * (NT / 64) + wave, sl = j * 64 + lane;
            const int row = sl / SPR, c = sl % SPR;
            off[u] = (j < NINST && sl < TOTAL) ? (int)(row * gs + (c == SPR - 1 ? 0 : c * 16)) : -1;
        }
    }
    __device__ __forceinline__ void issue(const unsigned char* g, unsigned char* l, int wave) const {
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u) {
            const int j = u * (NT / 64) + wave;
            // wave-uniform except in a partial last instruction
            if (j < NINST && (TOTAL % 64 == 0 || off[u] >= 0))
                __builtin_amdgcn_global_load_lds(g + off[u], (lds_void*)(l + j * 64 * 16), 16, 0, 0);
        }
    }
};

template <typename E, int D, int C, int BV>
struct StateCopies {
    TileCopy<C, D * (int)sizeof(E)> wq;     // -W and Q~ (same shape)
    TileCopy<D, C * (int)sizeof(E)> kt;     // K^T
    TileCopy<C, C * (int)sizeof(E)> p;      // P
    TileCopy<C, BV * (int)sizeof(E)> u;     // this slice of U~
    __device__ __forceinline__ void init(int wave, int lane) {
        constexpr int ES = (int)sizeof(E);
        wq.init(D * ES, wave, lane);
        kt.init(C * ES, wave, lane);
        p.init(C * ES, wave, lane);
        u.init(D * ES, wave, lane);
    }
};

template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_fetch(const StateArgs& a, const StateCopies<E, D, C, BV>& cp,
                                            int64_t rec, int slice, E* buf, int wave, int lane)
{
    typedef StateShape<E, D, C, BV> S;
    constexpr int ES = S::ES;
    unsigned char* l = reinterpret_cast<unsigned char*>(buf);
    cp.wq.issue((const unsigned char*)((const E*)a.Wn + rec * C * D), l + S::OFF_W * ES, wave);
    cp.wq.issue((const unsigned char*)((const E*)a.Qt + rec * C * D), l + S::OFF_Q * ES, wave);
    cp.kt.issue((const unsigned char*)((const E*)a.Kh + rec * C * D), l + S::OFF_KT * ES, wave);
    cp.p.issue((const unsigned char*)((const E*)a.P + rec * C * C), l + S::OFF_P * ES, wave);
    cp.u.issue((const unsigned char*)((const E*)a.Ut + rec * C * D + slice * BV), l + S::OFF_U * ES, wave);
    // gamma: D floats, one unpadded row
    if (wave == 0 && lane < D / 4)
        __builtin_amdgcn_global_load_lds(a.gam + rec * D + lane * 4, (lds_void*)(l + S::OFF_G * ES), 16, 0, 0);
}

// Scheduling hint for a phase of N MFMAs fed from LDS: issue the first
// group of fragment reads, then alternate one MFMA with one more read, so
// reads run ahead of the MFMAs that consume them.
template <int N>
__device__ __forceinline__ void sched_pipeline()
{
    constexpr int AHEAD = N < 8 ? N : 8;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);   // DS reads
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // DS reads
    }
}

// s_waitcnt vmcnt(0): every global->LDS copy this wave issued has landed.
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One chunk from buffer `buf`: Delta = U~ - W S, O = Q~ S + P Delta,
// S <- diag(gamma) S + K^T Delta; O goes out through the wave's staging rows.
template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_store_o(const StateArgs& a, const E* sOw, int64_t b, int64_t h,
                                             int slice, int64_t n, int lane, int wave);

template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_compute(const StateArgs& a, const E* buf, E* sOw, f32x4* St,
                                              int64_t b, int64_t h, int slice, int64_t n,
                                              int lane, int wave)
{
    typedef StateShape<E, D, C, BV> S;
    typedef Mma<E> MM;
    constexpr int NB = S::NB, VEC = S::VEC, LDA = S::LDA, LDT = S::LDT, LDU = S::LDU, LDO = S::LDO;
    constexpr int NKS = D / MM::KB;      // MFMA steps over the state rows
    constexpr int NKC = C / MM::KB;      // MFMA steps over the chunk's tokens
    constexpr int KTS = D / 16;
    const int gq = lane >> 4, cl = lane & 15;
    const E* sW = buf + S::OFF_W;
    const E* sQ = buf + S::OFF_Q;
    const E* sKT = buf + S::OFF_KT;
    const E* sP = buf + S::OFF_P;
    const E* sU = buf + S::OFF_U;
    const float* sGam = reinterpret_cast<const float*>(buf + S::OFF_G);

    typename MM::Frag SB[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        SB[ks] = MM::from_acc(&St[ks * MM::KT]);

    // Delta = U~ - W S  (W is stored negated).  Each phase reads all of its
    // A fragments before its MFMAs so LDS latency overlaps.
    f32x4 dl[NB];
    {
        typename MM::Frag aw[NB][NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                aw[mt][ks] = MM::load_perm(sW + 16 * mt * LDA + ks * MM::KB, LDA, lane);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dl[mt][i] = to_f32(sU[(16 * mt + 4 * gq + i) * LDU + 16 * wave + cl]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                dl[mt] = MM::mma(aw[mt][ks], SB[ks], dl[mt]);
        sched_pipeline<NB * NKS>();
    }
    typename MM::Frag DB[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        DB[kc] = MM::from_acc(&dl[kc * MM::KT]);
    // the previous chunk's outputs leave while this one computes
    if (n > 0)
        state_store_o<E, D, C, BV>(a, sOw, b, h, slice, n - 1, lane, wave);

    // O = Q~ S + P Delta  (P is lower triangular: skip all-zero steps).
    f32x4 ot[NB];
    {
        typename MM::Frag aq[NB][NKS], ap[NB][NKC];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                aq[mt][ks] = MM::load_perm(sQ + 16 * mt * LDA + ks * MM::KB, LDA, lane);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                if (kc * MM::KT <= mt)
                    ap[mt][kc] = MM::load_perm(sP + 16 * mt * LDT + kc * MM::KB, LDT, lane);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
            ot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                ot[mt] = MM::mma(aq[mt][ks], SB[ks], ot[mt]);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                if (kc * MM::KT <= mt)
                    ot[mt] = MM::mma(ap[mt][kc], DB[kc], ot[mt]);
        sched_pipeline<NB * NKS>();
    }

    // S <- diag(gamma) S + K^T Delta.
    {
        typename MM::Frag ak[KTS][NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int kt = 0; kt < KTS; ++kt)
                ak[kt][kc] = MM::load_perm(sKT + 16 * kt * LDT + kc * MM::KB, LDT, lane);
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
            St[kt] = St[kt] * *reinterpret_cast<const f32x4*>(sGam + 16 * kt + 4 * gq);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int kt = 0; kt < KTS; ++kt)
                St[kt] = MM::mma(ak[kt][kc], DB[kc], St[kt]);
        sched_pipeline<KTS * NKC>();
    }

    // O: into this wave's staging rows; written out during the next chunk.
#pragma unroll
    for (int mt = 0; mt < NB; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sOw[(16 * mt + 4 * gq + i) * LDO + cl] = from_f32<E>(ot[mt][i]);
}

// 16-byte stores of one wave's 16 staged output columns of chunk n.
template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_store_o(const StateArgs& a, const E* sOw, int64_t b, int64_t h,
                                             int slice, int64_t n, int lane, int wave)
{
    typedef StateShape<E, D, C, BV> S;
    constexpr int VEC = S::VEC, LDO = S::LDO, CPR = 16 / VEC;   // 16-byte pieces per staged row
    const int64_t t0 = n * C;
    const int L = (int)min((int64_t)C, a.T - t0);
    E* o = (E*)a.o;
#pragma unroll
    for (int e = lane; e < C * CPR; e += 64) {
        const int r = e / CPR, cg = e % CPR;
        if (r < L)
            *reinterpret_cast<u32x4*>(o + ((b * a.T + t0 + r) * a.H + h) * D + slice * BV + 16 * wave + cg * VEC) =
                *reinterpret_cast<const u32x4*>(sOw + r * LDO + cg * VEC);
    }
}

template <typename E, int D, int C, int BV>
__global__ __launch_bounds__(NT) void chunk_state_kernel(StateArgs a)
{
    typedef StateShape<E, D, C, BV> S;
    constexpr int KTS = D / 16;
    __shared__ __align__(16) E buf0[S::BUF];
    __shared__ __align__(16) E buf1[S::NBUF == 2 ? S::BUF : 1];
    __shared__ __align__(16) E sO[(NT / 64) * C * S::LDO];

    // Workgroup -> (sequence*head, column slice).  The NS slices of one
    // (b,h) read the same chunk records: give them the same blockIdx % 8 so
    // they land on the same XCD and share its L2.
    const int64_t bx = blockIdx.x;
    const int64_t grp = bx / (8 * S::NS);
    const int within = (int)(bx % (8 * S::NS));
    const int slice = within / 8;
    const int64_t bh = grp * 8 + within % 8;
    if (bh >= a.nbh)
        return;
    const int64_t b = bh / a.H, h = bh - b * a.H, rec0 = bh * a.NC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4, cl = lane & 15;
    const int col = slice * BV + 16 * wave + cl;     // this lane's state column
    E* sOw = sO + wave * C * S::LDO;

    f32x4 St[KTS];
    {
        const float* s0 = a.S0 ? a.S0 + bh * D * D : nullptr;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                St[kt][i] = s0 ? s0[(16 * kt + 4 * gq + i) * D + col] : 0.f;
    }

    StateCopies<E, D, C, BV> cp;
    cp.init(wave, lane);
    state_fetch<E, D, C, BV>(a, cp, rec0, slice, buf0, wave, lane);
    if (S::NBUF == 2) {
        for (int64_t n = 0; n < a.NC; n += 2) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0; everyone is done with buf1
            if (n + 1 < a.NC)
                state_fetch<E, D, C, BV>(a, cp, rec0 + n + 1, slice, buf1, wave, lane);
            state_compute<E, D, C, BV>(a, buf0, sOw, St, b, h, slice, n, lane, wave);
            if (n + 1 >= a.NC)
                break;
            wait_copies();
            __syncthreads();          // chunk n + 1 is in buf1; everyone is done with buf0
            if (n + 2 < a.NC)
                state_fetch<E, D, C, BV>(a, cp, rec0 + n + 2, slice, buf0, wave, lane);
            state_compute<E, D, C, BV>(a, buf1, sOw, St, b, h, slice, n + 1, lane, wave);
        }
    } else {
        for (int64_t n = 0; n < a.NC; ++n) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0
            state_compute<E, D, C, BV>(a, buf0, sOw, St, b, h, slice, n, lane, wave);
            __syncthreads();          // everyone is done with buf0
            if (n + 1 < a.NC)
                state_fetch<E, D, C, BV>(a, cp, rec0 + n + 1, slice, buf0, wave, lane);
        }
    }

    state_store_o<E, D, C, BV>(a, sOw, b, h, slice, a.NC - 1, lane, wave);

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
        reinterpret_cast<const void*>(&chunk_prep_kernel<true, E, D, C>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)PS::SMEM);
    static const hipError_t attr1g = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&chunk_prep_kernel<false, E, D, C>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)PS::SMEM);
    static const hipError_t attr2 = hipSuccess;
    if (attr1 != hipSuccess)
        return attr1;
    if (attr1g != hipSuccess)
        return attr1g;
    if (attr2 != hipSuccess)
        return attr2;

    if (a.stage != GDR2_STAGE_STATE) {
        const int64_t grid1 = std::min<int64_t>(L.nrec, (int64_t)cu_count());
        const bool full = a.b_width == D && a.w_width == D && a.g_width == D;
        if (full)
            hipLaunchKernelGGL((chunk_prep_kernel<true, E, D, C>), dim3((unsigned)grid1), dim3(NTP), PS::SMEM, stream, pa);
        else
            hipLaunchKernelGGL((chunk_prep_kernel<false, E, D, C>), dim3((unsigned)grid1), dim3(NTP), PS::SMEM, stream, pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.stage == GDR2_STAGE_PREP)
            return e;
    }

    StateArgs sa;
    sa.Wn = pa.Wn; sa.Ut = pa.Ut; sa.Kh = pa.Kh; sa.Qt = pa.Qt; sa.P = pa.P; sa.gam = pa.gam;
    sa.S0 = a.S0; sa.S_out = a.S_out; sa.o = a.o;
    sa.T = a.T; sa.H = a.H; sa.NC = pa.NC; sa.nbh = a.B * a.H;
    const int64_t grid2 = ceil_div(sa.nbh, 8) * 8 * SS::NS;
    hipLaunchKernelGGL((chunk_state_kernel<E, D, C, BV>), dim3((unsigned)grid2), dim3(NT), 0, stream, sa);
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
