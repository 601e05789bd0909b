// gdr2_chunk_common.h -- the intra-chunk machinery shared by the staged
// prep kernel (gdr2_chunked.hip) and the fused forward (gdr2_fused.hip):
// MFMA tiles in the state kernel's operand order, the lane mapping of one
// chunk's token rows, the prefetch of a chunk's inputs, and the phases that
// turn one chunk's inputs into its WY factors (cumulative log-decay,
// decay-referenced operands, gated Gram M and scores P, the inverse of I + M,
// the K^T fragments, -W and U~).  Each phase writes its results through
// pointers, so one kernel can send them to the workspace and another keep
// them in LDS.
//
// Chunk form (page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트
// 분리", update of section "Gated Delta Rule-2 업데이트 수식", organised in
// fixed-size chunks as in section "효율적 구현"; L tokens, chunk-start state
// S, G_t = sum_{r<=t} g_r per key channel in log2 units, e_t = b_t*k_t,
// u_t = w_t*v_t):
//   M[t,s] = sum_i e_t[i] k_s[i] 2^(G_t[i]-G_s[i])   s <  t   (strictly lower)
//   P[t,s] = sum_i q_t[i] k_s[i] 2^(G_t[i]-G_s[i])   s <= t
//   X = (I + M)^-1,  W = X (e*2^G),  U~ = X u
//   Delta = U~ - W S,  O = (q*2^G) S + P Delta,
//   S_next = diag(2^G_L) S + K^T Delta,   K^_s = k_s*2^(G_L-G_s)
#pragma once

#include "gdr2_device.h"
#include "gdr2_internal.h"

namespace gdr2 {
namespace {

constexpr float kSpanMax = 80.f;   // largest decay exponent (log2) a factor may carry

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// 16x16x16 products in the accumulator-compatible k order: lane l holds
// k = 4*(l/16) .. 4*(l/16)+3 of a 16-deep contraction, for A (row l%16) and
// B (column l%16) alike -- an accumulator tile is directly a B operand.
// bf16: v_mfma_f32_16x16x16_bf16; fp32: four v_mfma_f32_16x16x4f32.
// ---------------------------------------------------------------------------
template <typename E> struct Mma16;
template <> struct Mma16<bf16> {
    typedef bf16x4 Frag;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ Frag pack(f32x4 x) {
        Frag f;
        f[0] = (bf16)x[0]; f[1] = (bf16)x[1]; f[2] = (bf16)x[2]; f[3] = (bf16)x[3];
        return f;
    }
    static __device__ __forceinline__ Frag load(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    }
};
template <> struct Mma16<float> {
    typedef f32x4 Frag;
    static __device__ __forceinline__ Frag pack(f32x4 x) { return x; }
    static __device__ __forceinline__ Frag load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) { return Mma<float>::mma(a, b, c); }
};

// A full-width fragment (KT 16-blocks along k) from KT accumulator tiles.
template <typename E> __device__ __forceinline__ typename Mma<E>::Frag frag_of(const f32x4* t);
template <> __device__ __forceinline__ Mma<bf16>::Frag frag_of<bf16>(const f32x4* t) { return Mma<bf16>::pack(t[0], t[1]); }
template <> __device__ __forceinline__ Mma<float>::Frag frag_of<float>(const f32x4* t) { return t[0]; }

// ---------------------------------------------------------------------------
// Fragment geometry of one chunk record.
//   -W  [T][m]: rows t = 16T + l%16, k = key channels (m-th KB block)
//   Q~  [T][m]: same
//   K^T [c][m]: rows = key channels 16c + l%16, k = tokens (m-th KB block)
//   P   [T][m] for m*KT <= T only (the rest of P is zero above the diagonal)
//   U~  [n][T]: accumulator tiles, rows = tokens 16T.., columns 16n..
// Within a KB block, lane group g = l/16 holds k = 4g..4g+3 (and, for bf16,
// 16+4g..16+4g+3 in its upper four slots).
// ---------------------------------------------------------------------------
template <typename E, int D, int C>
struct Frags {
    static constexpr int KB = Mma<E>::KB, KT = KB / 16;
    static constexpr int NB = C / 16;
    static constexpr int NKS = D / KB;               // k-steps over key channels
    static constexpr int NKC = C / KB;               // k-steps over tokens
    static constexpr int FRAG = 1024;
    static constexpr int TILE_U = 64 * 4 * (int)sizeof(E);
    static constexpr int p_count(int T) { return T / KT + 1; }
    static constexpr int p_offset(int T) { return T == 0 ? 0 : p_offset(T - 1) + p_count(T - 1); }
    static constexpr int NP = p_offset(NB);
    static constexpr size_t W_BYTES = (size_t)NB * NKS * FRAG;       // = C*D*sizeof(E)
    static constexpr size_t K_BYTES = (size_t)(D / 16) * NKC * FRAG;  // = C*D*sizeof(E)
    static constexpr size_t P_BYTES = (size_t)NP * FRAG;
    static constexpr size_t U_BYTES = (size_t)NB * (D / 16) * TILE_U; // = C*D*sizeof(E)
    static_assert(W_BYTES == (size_t)C * D * sizeof(E) && K_BYTES == W_BYTES && U_BYTES == W_BYTES, "sizes");
};

// Workspace: per record (sequence, head, chunk) in the order (b*H + h)*NC + n,

// Inputs of the intra-chunk phases.
struct PrepIn {
    const void *q, *k, *v, *b, *w;
    const float* g;
    int bw, ww, gw;
    int pro;                  // prologue bits (normalise q, k; activate gates)
    int64_t B, T, H, NC;
};

// ---------------------------------------------------------------------------
// Small element helpers.
// ---------------------------------------------------------------------------
template <typename E>
__device__ __forceinline__ void unpack(const u32x4& r, float* out);
template <>
__device__ __forceinline__ void unpack<bf16>(const u32x4& r, float* out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(r[i] << 16);
        out[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void unpack<float>(const u32x4& r, float* out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        out[i] = __uint_as_float(r[i]);
}

// A width-1 gate's value from its raw bits, zero-extended to 32 bits.
template <typename E> __device__ __forceinline__ float gate_bits(unsigned int u);
template <> __device__ __forceinline__ float gate_bits<bf16>(unsigned int u) { return __uint_as_float(u << 16); }
template <> __device__ __forceinline__ float gate_bits<float>(unsigned int u) { return __uint_as_float(u); }

template <typename E> __device__ __forceinline__ u32x4 pack_vec(const float* x);
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
    return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
}

__device__ __forceinline__ u32x4 ldg16(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void sts16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Position of logical k index `col` inside its fragment row (see Frags).
template <typename E> __device__ __forceinline__ int kpos(int col);
template <> __device__ __forceinline__ int kpos<bf16>(int col)
{
    const int c = col & 31;
    return (col & ~31) + 8 * ((c & 15) >> 2) + (c & 3) + 4 * (c >> 4);
}
template <> __device__ __forceinline__ int kpos<float>(int col) { return col; }


// Prologue activations (logistic sigmoid; log-decay -softplus(x) = log sigmoid(-x)).
// (v_exp, v_log, v_rcp: about 1 ulp each; log(1 + e) loses e < 6e-8 absolute,
// far below the decay's own rounding)
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float neg_softplus(float x) { return -(fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)))); }
constexpr float kNormEps = 1e-6f;

// s_waitcnt lgkmcnt(0) with a compiler barrier: LDS writes of this wave are
// complete before any later LDS read of it (lanes exchange data this way).
__device__ __forceinline__ void lds_fence_wave()
{
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workgroup barrier that orders LDS data only: this wave's LDS operations
// have completed, then s_barrier.  (__syncthreads() also waits for every
// outstanding global access, including loads still being prefetched.)
__device__ __forceinline__ void lds_barrier()
{
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(0): every global->LDS copy this wave issued has landed.
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Inclusive-scan step: the value of the lane `d` below within the 16-lane row.
template <int d>
__device__ __forceinline__ float dpp_shr(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + d, 0xF, 0xF, true));
}

// Work item -> chunk.  The persistent prep kernel visits items in the order
// (chunk taken last to first, sequence, head) with the head fastest (see
// ItemWalk), so the workgroups in flight together read whole token rows: the
// H heads of a token are one contiguous run of H*D elements of the
// [B,T,H,.] inputs.  Token row r of the chunk is element offset
// ((b*T + t0 + r)*H + h); the chunk's record in the workspace is

// One chunk of one (sequence, head): token row r of the chunk is element
// offset ((b*T + t0 + r)*H + h) of the [B,T,H,.] inputs.
struct ChunkPos {
    int64_t rec;      // workspace record (b*H + h)*NC + n (staged path)
    int64_t row0;     // (b*T + t0)*H + h
    int L;            // valid tokens (>= 1)
};

constexpr int NTP = 512;           // threads of the prep and fused kernels
constexpr int NWP = NTP / 64;      // their waves

// Lane mapping of one chunk's [C][D] token rows over the 8 waves: each lane
// owns VEC key channels (one 16-byte access) of TPL consecutive tokens; LPC
// lanes share a channel group.
template <typename E, int D, int C>
struct PrepGeom {
    typedef Frags<E, D, C> F;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int VEC = 16 / ES;                      // elements per 16-byte access
    static constexpr int NB = C / 16, NH = C / 32;
    static constexpr int NCG = D / VEC;                      // 16-byte chunks per row
    static constexpr int NWB0 = C * D / VEC / 64;
    static constexpr int NWB = NWB0 < NWP ? NWB0 : NWP;      // waves of phases A and B
    static constexpr int TW = C / NWB;                       // tokens per wave
    static constexpr int LPC = 64 / NCG;                     // lanes sharing a channel group
    static constexpr int TPL = TW / LPC;                     // tokens per lane
    static constexpr int LDM = C + 4;                        // rows of M (elements)
    static constexpr int LDXP = C + VEC;                     // rows of X (elements)
    static constexpr int LDX = 20;                           // rows of fp32 16x16 blocks
    static constexpr size_t ROWB = (size_t)D * ES;
    // LDS of the phases, bytes (the caller places the arrays)
    static constexpr size_t SZ_ROWS = (size_t)C * ROWB;                       // E^, Q^, Kr [C][D]
    static constexpr size_t SZ_HALF = (size_t)(NH - 1) * 32 * ROWB;           // E~, Q~ second half
    static constexpr size_t SZ_M = al256((size_t)C * LDM * ES);
    static constexpr size_t SZ_MD = (size_t)NB * 16 * LDX * 4;
    static constexpr size_t SZ_X = al256((size_t)C * LDXP * ES);
    static constexpr size_t SZ_TOT = (size_t)NWB * D * 4;
    static constexpr size_t SZ_FK = (size_t)NH * D * 4;
    static constexpr size_t SZ_RN = (size_t)2 * C * 4;
    static constexpr size_t SZ_G = (size_t)C * D * 4;                        // raw g (static LDS)
    static_assert(C == 32 || C == 64, "chunk");
    static_assert(64 % NCG == 0 && NCG >= 8 && TPL >= 1 && TW == LPC * TPL, "lane mapping");
    static_assert(NWB == NWP || NH == 1, "halves need every wave in phase B");
};

}  // namespace

// The kernel's dynamic LDS (every extern __shared__ array of a kernel names
// the same base).
extern __shared__ __align__(16) unsigned char dyn_lds[];

namespace {

// LDS arrays of the phases, at the byte offsets OFF_* of the kernel's layout
// L in its dynamic LDS (compile-time offsets, so every access is an LDS
// address with a constant offset).  U holds UC value columns per row
// (u_lo .. u_lo + UC - 1); the others full rows of D.  G (the raw or
// cumulative log-decay) and BW (width-1 b and w of the chunk, [2][C] words)
// are the kernel's static LDS arrays.
template <typename E, typename L>
struct PrepLds {
    float* G;
    unsigned int* BW;
    template <typename T> static __device__ __forceinline__ T* at(size_t off) { return reinterpret_cast<T*>(dyn_lds + off); }
    static __device__ __forceinline__ E* Eh() { return at<E>(L::OFF_EH); }
    static __device__ __forceinline__ E* Qh() { return at<E>(L::OFF_QH); }
    static __device__ __forceinline__ E* Kr() { return at<E>(L::OFF_KR); }
    static __device__ __forceinline__ E* U() { return at<E>(L::OFF_U); }
    static __device__ __forceinline__ E* E2() { return at<E>(L::OFF_E2); }
    static __device__ __forceinline__ E* Q2() { return at<E>(L::OFF_Q2); }
    static __device__ __forceinline__ E* M() { return at<E>(L::OFF_M); }
    static __device__ __forceinline__ E* X() { return at<E>(L::OFF_X); }
    static __device__ __forceinline__ float* Md() { return at<float>(L::OFF_MD); }
    static __device__ __forceinline__ float* Xc() { return at<float>(L::OFF_XC); }
    static __device__ __forceinline__ float* Tot() { return at<float>(L::OFF_TOT); }
    static __device__ __forceinline__ float* Fk() { return at<float>(L::OFF_FK); }
    static __device__ __forceinline__ float* Rn() { return at<float>(L::OFF_RN); }
    static __device__ __forceinline__ int* Flag() { return at<int>(L::OFF_FLAG); }
};

// Row swizzle of the [rows][D] operand arrays: 16-byte chunk j of row r
// sits at chunk j ^ (r & SWZ_MASK), with the mask as wide as the row allows
// up to 15, so the 16 rows that one 16-lane group of a fragment read touches
// land on distinct banks.
template <typename E, int D>
constexpr int swz_mask()
{
    constexpr int NCG = D * (int)sizeof(E) / 16;   // 16-byte chunks per row
    return (NCG < 16 ? NCG : 16) - 1;
}

// Element offset of element `col` of row `r` in a swizzled [rows][D] array.
template <typename E, int D>
__device__ __forceinline__ int swz(int r, int col)
{
    constexpr int VEC = 16 / (int)sizeof(E);
    return r * D + (((col / VEC) ^ (r & swz_mask<E, D>())) * VEC) + (col % VEC);
}

// Raw inputs of one lane's TPL tokens (bit patterns; width-1 gates are not
// held here but copied to LDS by prep_copy_bw).
template <typename E, int D, int C>
struct PrepRegs {
    typedef PrepGeom<E, D, C> S;
    u32x4 k[S::TPL], q[S::TPL], v[S::TPL], b[S::TPL], w[S::TPL];
};

// Issue the token loads of one chunk for tokens t0.. of this lane, channels
// c0...  Rows past the valid length re-read the last valid row (in bounds)
// and are zeroed where they are used, so no load sits under a per-lane branch.
// PART: 0 = k, 1 = q, 2 = v, 3 = b, 4 = w (issued at different points of
// the previous chunk, so no wave stalls on a full memory queue).
template <int PART, int WB, int WW, typename E, int D, int C>
__device__ __forceinline__ void prep_load(const PrepIn& a, const ChunkPos& cp, PrepRegs<E, D, C>& R,
                                          int t0, int c0)
{
    typedef PrepGeom<E, D, C> S;
#pragma unroll
    for (int j = 0; j < S::TPL; ++j) {
        const int t = min(t0 + j, cp.L - 1);
        const int64_t row = cp.row0 + (int64_t)t * a.H, off = row * D + c0;
        if (PART == 0)
            R.k[j] = ldg16((const E*)a.k + off);
        if (PART == 1)
            R.q[j] = ldg16((const E*)a.q + off);
        if (PART == 2)
            R.v[j] = ldg16((const E*)a.v + off);
        if (PART == 3 && (WB == 0 ? a.bw != 1 : WB != 1))
            R.b[j] = ldg16((const E*)a.b + off);
        if (PART == 4 && (WW == 0 ? a.ww != 1 : WW != 1))
            R.w[j] = ldg16((const E*)a.w + off);
    }
}

// Copy one chunk's log-decay rows straight into LDS (global_load_lds, no
// registers): [C][D] fp32, or C floats for a width-1 gate.  Rows past the
// valid length repeat the last valid row and are zeroed by the reader.
template <int WG, typename E, int D, int C>
__device__ __forceinline__ void prep_copy_g(const PrepIn& a, const ChunkPos& cp, unsigned char* sGraw,
                                            int wave, int lane)
{
    typedef __attribute__((address_space(3))) void lds_t;
    if (WG == 0 ? a.gw != 1 : WG != 1) {
        constexpr int NI = C * D * 4 / 1024;
        for (int j = wave; j < NI; j += NWP) {
            const int byte = j * 1024 + lane * 16, t = min(byte / (D * 4), cp.L - 1), col = (byte % (D * 4)) / 4;
            __builtin_amdgcn_global_load_lds(a.g + (cp.row0 + (int64_t)t * a.H) * D + col,
                                             (lds_t*)(sGraw + j * 1024), 16, 0, 0);
        }
    } else if (wave == 0 && lane < C) {
        __builtin_amdgcn_global_load_lds(a.g + cp.row0 + (int64_t)min(lane, cp.L - 1) * a.H, (lds_t*)sGraw, 4, 0, 0);
    }
}

// One element per lane from global memory into the 32-bit LDS word `lane` of
// dst (zero-extended), without a register.
template <typename E> __device__ __forceinline__ void copy_elem_lds(const E* src, unsigned int* dst);
template <>
__device__ __forceinline__ void copy_elem_lds<bf16>(const bf16* src, unsigned int* dst)
{
    typedef __attribute__((address_space(3))) void lds_t;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_t*)dst, 2, 0, 0);
}
template <>
__device__ __forceinline__ void copy_elem_lds<float>(const float* src, unsigned int* dst)
{
    typedef __attribute__((address_space(3))) void lds_t;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_t*)dst, 4, 0, 0);
}

// Copy one chunk's width-1 erase and write gates straight into LDS
// (global_load_lds, one element per lane): token t's bits land
// zero-extended in 32-bit word t of sBW (b) and of sBW + C (w), so no lane
// spends a register load on a scalar that 16 lanes share.  Rows past the
// valid length repeat the last valid row.
template <int WB, int WW, typename E, int D, int C>
__device__ __forceinline__ void prep_copy_bw(const PrepIn& a, const ChunkPos& cp, unsigned int* sBW,
                                             int wave, int lane)
{
    const bool nb = WB == 0 ? a.bw == 1 : WB == 1, nw = WW == 0 ? a.ww == 1 : WW == 1;
    if (lane < C) {
        const int64_t row = cp.row0 + (int64_t)min(lane, cp.L - 1) * a.H;
        if (nb && wave == 1)
            copy_elem_lds<E>((const E*)a.b + row, sBW);
        if (nw && wave == 2)
            copy_elem_lds<E>((const E*)a.w + row, sBW + C);
    }
}

// Phase B for one lane: decay-referenced operands of its tokens into LDS.
// VALID: every token of the chunk is valid (no zeroing needed).  u = w v is
// stored only for the value columns u_lo .. u_lo + UC - 1 (rows of UC).
template <bool VALID, bool SECOND, bool PRO, int UC, typename E, int D, int C, typename SL>
__device__ __forceinline__ float prep_operands(const PrepRegs<E, D, C>& R, const float (*G)[16 / sizeof(E)],
                                               const float* gh, int bw, int ww, int L, int t0, int c0,
                                               const SL& s, int u_lo, int pro)
{
    typedef PrepGeom<E, D, C> S;
    constexpr int VEC = S::VEC;
    const unsigned int* sBW = s.BW;
    const bool own_u = UC == D || (unsigned)(c0 - u_lo) < (unsigned)UC;
    float fh[VEC];
    if (SECOND) {
#pragma unroll
        for (int x = 0; x < VEC; ++x)
            fh[x] = fast_exp2(gh[x]);
    }
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < S::TPL; ++j) {
        // one output array at a time keeps few values live
        const int t = t0 + j;
        const bool valid = VALID || t < L;
        const int o = swz<E, D>(t, c0);
        const int o2 = SECOND ? swz<E, D>(t - 32, c0) : 0;
        float eh[VEC], d[VEC], kk[VEC], tmp[VEC], tmp2[VEC];
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
            const float g = G[j][x];
            d[x] = SECOND ? g - gh[x] : g;
            mx = fmaxf(mx, fmaxf(fabsf(d[x]), g));
        }
        unpack<E>(R.k[j], kk);
        if constexpr (PRO) {
            // prologue: unit L2 norm per token over the row, whose channel
            // groups sit in the lanes lane % LPC + LPC * m
            if (pro & GDR2_PROLOGUE_NORM_QK) {
                float ss = 0.f;
#pragma unroll
                for (int x = 0; x < VEC; ++x)
                    ss += kk[x] * kk[x];
#pragma unroll
                for (int m = S::LPC; m < 64; m <<= 1)
                    ss += __shfl_xor(ss, m);
                const float rk = rsqrtf(ss + kNormEps);
#pragma unroll
                for (int x = 0; x < VEC; ++x)
                    kk[x] *= rk;
                if (c0 == 0)
                    s.Rn()[t] = rk;
            }
        }
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
            kk[x] = valid ? kk[x] : 0.f;
            tmp[x] = kk[x] * fast_exp2(-d[x]);
            eh[x] = fast_exp2(d[x]);
        }
        sts16(s.Kr() + o, pack_vec<E>(tmp));
        __builtin_amdgcn_sched_barrier(0);
        {
            float bb[VEC];
            unpack<E>(R.b[j], bb);
            float bs = bw == 1 ? gate_bits<E>(sBW[t]) : 0.f;
            if constexpr (PRO) {
                if (pro & GDR2_PROLOGUE_GATES) {
                    bs = sigm(bs);
#pragma unroll
                    for (int x = 0; x < VEC; ++x)
                        bb[x] = sigm(bb[x]);
                }
            }
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                tmp[x] = (bw == 1 ? bs : bb[x]) * kk[x] * eh[x];
                if (SECOND)
                    tmp2[x] = tmp[x] * fh[x];
            }
        }
        sts16(s.Eh() + o, pack_vec<E>(tmp));
        if (SECOND)
            sts16(s.E2() + o2, pack_vec<E>(tmp2));
        __builtin_amdgcn_sched_barrier(0);
        {
            float qq[VEC];
            unpack<E>(R.q[j], qq);
            if constexpr (PRO) {
                if (pro & GDR2_PROLOGUE_NORM_QK) {
                    float ss = 0.f;
#pragma unroll
                    for (int x = 0; x < VEC; ++x)
                        ss += qq[x] * qq[x];
#pragma unroll
                    for (int m = S::LPC; m < 64; m <<= 1)
                        ss += __shfl_xor(ss, m);
                    const float rq = rsqrtf(ss + kNormEps);
#pragma unroll
                    for (int x = 0; x < VEC; ++x)
                        qq[x] *= rq;
                    if (c0 == 0)
                        s.Rn()[C + t] = rq;
                }
            }
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                tmp[x] = (valid ? qq[x] : 0.f) * eh[x];
                if (SECOND)
                    tmp2[x] = tmp[x] * fh[x];
            }
        }
        sts16(s.Qh() + o, pack_vec<E>(tmp));
        if (SECOND)
            sts16(s.Q2() + o2, pack_vec<E>(tmp2));
        __builtin_amdgcn_sched_barrier(0);
        if (own_u) {
            float vv[VEC], wv[VEC];
            unpack<E>(R.v[j], vv);
            unpack<E>(R.w[j], wv);
            float ws = ww == 1 ? gate_bits<E>(sBW[C + t]) : 0.f;
            if constexpr (PRO) {
                if (pro & GDR2_PROLOGUE_GATES) {
                    ws = sigm(ws);
#pragma unroll
                    for (int x = 0; x < VEC; ++x)
                        wv[x] = sigm(wv[x]);
                }
            }
#pragma unroll
            for (int x = 0; x < VEC; ++x)
                tmp[x] = (valid ? (ww == 1 ? ws : wv[x]) : 0.f) * vv[x];
            sts16(s.U() + swz<E, UC>(t, c0 - u_lo), pack_vec<E>(tmp));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return mx;
}

// 16 bytes of a swizzled row array as a full-width fragment: logical chunk
// ch (k-values VEC*ch ..) of row r.
template <typename E, int D>
__device__ __forceinline__ typename Mma<E>::Frag row_frag(const E* base, int r, int ch)
{
    constexpr int VEC = 16 / (int)sizeof(E);
    return *reinterpret_cast<const typename Mma<E>::Frag*>(base + r * D + ((ch ^ (r & swz_mask<E, D>())) * VEC));
}

// Four consecutive elements (col a multiple of 4) of a swizzled row array.
template <typename E, int D>
__device__ __forceinline__ typename Mma16<E>::Frag row4(const E* base, int r, int col)
{
    return Mma16<E>::load(base + swz<E, D>(r, col));
}

// Identity B operand of the 16x16x16 transposes: element (k = 4gq + i, n = cl).
template <typename E>
__device__ __forceinline__ typename Mma16<E>::Frag identity16(int gq, int cl)
{
    f32x4 id;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        id[i] = (4 * gq + i == cl) ? 1.f : 0.f;
    return Mma16<E>::pack(id);
}

// ---------------------------------------------------------------------------
// Phase A: cumulative log2-decay of this lane's TPL tokens, in registers.
// The prefix sum runs within the lane, across the LPC lanes sharing the
// channels (DPP row shifts); each wave's totals go to s.Tot() for phase B.
// Only waves < NWB call it.
// ---------------------------------------------------------------------------
template <int WG, bool PRO, typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_cumsum(const PrepIn& a, const SL& s, int L, int t0, int c0, int lpc,
                                            int wave, float (&G)[PrepGeom<E, D, C>::TPL][16 / sizeof(E)],
                                            float (&excl)[16 / sizeof(E)])
{
    typedef PrepGeom<E, D, C> S;
    constexpr int VEC = S::VEC;
    const int gw = WG ? WG : a.gw;
    const bool full_chunk = L == C;
#pragma unroll
    for (int j = 0; j < S::TPL; ++j) {
        const bool valid = full_chunk || t0 + j < L;
        const bool act = PRO && (a.pro & GDR2_PROLOGUE_GATES);
        if (gw == 1) {
            float gv = s.G[t0 + j];
            if (act)
                gv = neg_softplus(gv);
#pragma unroll
            for (int x = 0; x < VEC; ++x)
                G[j][x] = valid ? gv * kLog2e : 0.f;
        } else {
#pragma unroll
            for (int x4 = 0; x4 < VEC / 4; ++x4) {
                f32x4 gv = *reinterpret_cast<const f32x4*>(s.G + (t0 + j) * D + c0 + 4 * x4);
                if (act) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        gv[i] = neg_softplus(gv[i]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    G[j][4 * x4 + i] = valid ? gv[i] * kLog2e : 0.f;
            }
        }
    }
#pragma unroll
    for (int j = 1; j < S::TPL; ++j)
#pragma unroll
        for (int x = 0; x < VEC; ++x)
            G[j][x] += G[j - 1][x];
    float inc[VEC];
#pragma unroll
    for (int x = 0; x < VEC; ++x)
        inc[x] = G[S::TPL - 1][x];
    if (S::LPC > 1) {
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
            const float y = dpp_shr<1>(inc[x]);
            inc[x] += lpc >= 1 ? y : 0.f;
        }
    }
    if (S::LPC > 2) {
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
            const float y = dpp_shr<2>(inc[x]);
            inc[x] += lpc >= 2 ? y : 0.f;
        }
    }
    if (S::LPC > 4) {
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
            const float y = dpp_shr<4>(inc[x]);
            inc[x] += lpc >= 4 ? y : 0.f;
        }
    }
#pragma unroll
    for (int x = 0; x < VEC; ++x)
        excl[x] = inc[x] - G[S::TPL - 1][x];
    if (lpc == S::LPC - 1) {
#pragma unroll
        for (int x4 = 0; x4 < VEC / 4; ++x4)
            *reinterpret_cast<f32x4*>(s.Tot() + wave * D + c0 + 4 * x4) =
                f32x4{inc[4 * x4], inc[4 * x4 + 1], inc[4 * x4 + 2], inc[4 * x4 + 3]};
    }
}

// ---------------------------------------------------------------------------
// Phase B: the chunk-level offsets from the wave totals (G becomes the
// cumulative decay from the chunk start; gh the decay at the half boundary),
// gamma = 2^G_L and the K^ factors 2^(G_L - Gh) per half into s.Fk() (gamma
// also to gam_out when it is given), then the decay-referenced operands.
// Sets *s.Flag() when a factor would exceed 2^kSpanMax.  Only waves < NWB.
// ---------------------------------------------------------------------------
template <bool PRO, int UC, typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_offsets_operands(const PrepIn& a, const PrepRegs<E, D, C>& R, const SL& s,
                                                      int L, int t0, int c0, int lpc, int wave, bool second,
                                                      float (&G)[PrepGeom<E, D, C>::TPL][16 / sizeof(E)],
                                                      const float (&excl)[16 / sizeof(E)], float* gam_out,
                                                      int u_lo, int bw, int ww)
{
    typedef PrepGeom<E, D, C> S;
    constexpr int VEC = S::VEC, NH = S::NH;
    float gh[VEC], off[VEC];
#pragma unroll
    for (int x = 0; x < VEC; ++x)
        off[x] = gh[x] = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < S::NWB - 1; ++w2) {
        if (w2 < wave) {
#pragma unroll
            for (int x4 = 0; x4 < VEC / 4; ++x4) {
                const f32x4 tv = *reinterpret_cast<const f32x4*>(s.Tot() + w2 * D + c0 + 4 * x4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    off[4 * x4 + i] += tv[i];
            }
        }
        if (NH == 2 && w2 == S::NWB / 2 - 1) {
#pragma unroll
            for (int x = 0; x < VEC; ++x)
                gh[x] = off[x];
        }
    }
#pragma unroll
    for (int j = 0; j < S::TPL; ++j)
#pragma unroll
        for (int x = 0; x < VEC; ++x)
            G[j][x] += off[x] + excl[x];
    if (wave == S::NWB - 1 && lpc == S::LPC - 1) {
        // the chunk's last token: gamma and the K^ factors per half
        float f0[VEC], f1[VEC];
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
            const float gl = G[S::TPL - 1][x];
            f0[x] = fast_exp2(gl);
            f1[x] = fast_exp2(gl - gh[x]);
        }
#pragma unroll
        for (int x4 = 0; x4 < VEC / 4; ++x4) {
            const f32x4 v0 = f32x4{f0[4 * x4], f0[4 * x4 + 1], f0[4 * x4 + 2], f0[4 * x4 + 3]};
            *reinterpret_cast<f32x4*>(s.Fk() + c0 + 4 * x4) = v0;
            if (gam_out)
                *reinterpret_cast<f32x4*>(gam_out + c0 + 4 * x4) = v0;
            if (NH == 2)
                *reinterpret_cast<f32x4*>(s.Fk() + D + c0 + 4 * x4) =
                    f32x4{f1[4 * x4], f1[4 * x4 + 1], f1[4 * x4 + 2], f1[4 * x4 + 3]};
        }
    }
    float mx;
    const bool full_chunk = L == C;
    if (second)
        mx = full_chunk ? prep_operands<true, true, PRO, UC, E, D, C>(R, G, gh, bw, ww, L, t0, c0, s, u_lo, a.pro)
                        : prep_operands<false, true, PRO, UC, E, D, C>(R, G, gh, bw, ww, L, t0, c0, s, u_lo, a.pro);
    else
        mx = full_chunk ? prep_operands<true, false, PRO, UC, E, D, C>(R, G, gh, bw, ww, L, t0, c0, s, u_lo, a.pro)
                        : prep_operands<false, false, PRO, UC, E, D, C>(R, G, gh, bw, ww, L, t0, c0, s, u_lo, a.pro);
    if (mx > kSpanMax)
        *s.Flag() = 1;
}

// ---------------------------------------------------------------------------
// Phase C1 (no steep decay): M tiles into s.M() / s.Md() (waves 0 .. NWP/2-1, as
// transposed products so each lane holds four consecutive columns of one
// row) and the P fragments (the other waves; their accumulators are the
// fragments) to dP, fragment f at dP + f KB + 16 lane.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_gram(const SL& s, unsigned char* dP, int wave, int lane)
{
    typedef PrepGeom<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef Mma16<E> M16;
    constexpr int NB = S::NB, NH = S::NH, LDM = S::LDM, LDX = S::LDX;
    constexpr int KT = F::KT, NKS = F::NKS, NP = F::NP;
    const int gq = lane >> 4, cl = lane & 15;
    if (wave < NWP / 2) {
        constexpr int NTM = NB * (NB + 1) / 2;
        for (int tile = wave; tile < NTM; tile += NWP / 2) {
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= tile)
                ++I;
            const int J = tile - I * (I + 1) / 2;
            const bool same = NH == 1 || (I >> 1) == (J >> 1);
            const E* Bs = same ? s.Eh() : s.E2();
            const int rb = same ? 16 * I + cl : 16 * I - 32 + cl;
            // every fragment of the tile is read before its first MFMA
            typename MM::Frag fa[NKS], fb[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                fa[ks] = row_frag<E, D>(s.Kr(), 16 * J + cl, 4 * ks + gq);
                fb[ks] = row_frag<E, D>(Bs, rb, 4 * ks + gq);
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                acc = MM::mma(fa[ks], fb[ks], acc);
            // lane: M[16I + cl][16J + 4gq + i]
            if (J < I) {
                *reinterpret_cast<typename M16::Frag*>(s.M() + (16 * I + cl) * LDM + 16 * J + 4 * gq) = M16::pack(acc);
            } else {
                f32x4 m;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    m[i] = 4 * gq + i < cl ? acc[i] : 0.f;
                *reinterpret_cast<f32x4*>(s.Md() + (16 * I + cl) * LDX + 4 * gq) = m;
            }
        }
    } else {
        for (int f = wave - NWP / 2; f < NP; f += NWP / 2) {
            int I = 0;
            while (I + 1 < NB && F::p_offset(I + 1) <= f)
                ++I;
            const int m = f - F::p_offset(I);
            // the k-tiles J = KT m + kt of one step share their half, so the
            // Q rows (B operand) serve both; every fragment of the step is read
            // before its first MFMA (a k-tile above the diagonal reads row
            // block I and its product is discarded)
            const bool same = NH == 1 || (I >> 1) == ((KT * m) >> 1);
            const E* Bs = same ? s.Qh() : s.Q2();
            const int rb = same ? 16 * I + cl : 16 * I - 32 + cl;
            typename MM::Frag fa[KT][NKS], fb[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                fb[ks] = row_frag<E, D>(Bs, rb, 4 * ks + gq);
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
                    fa[kt][ks] = row_frag<E, D>(s.Kr(), 16 * min(KT * m + kt, I) + cl, 4 * ks + gq);
            }
            f32x4 acc[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
                    acc[kt] = MM::mma(fa[kt][ks], fb[ks], acc[kt]);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int J = KT * m + kt;
                if (J > I) {
                    acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                } else if (J == I) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[kt][i] = 4 * gq + i <= cl ? acc[kt][i] : 0.f;
                }
            }
            stg16(dP + f * F::FRAG + lane * 16, __builtin_bit_cast(u32x4, frag_of<E>(acc)));
        }
    }
}

// ---------------------------------------------------------------------------
// Phase C1, exact path for a chunk with steep decay: M, P (straight into
// its fragments at dP, zeros above the diagonal) and K^ (unscaled, into the
// Kr rows) pair by pair from the raw inputs, with G over the raw rows in
// s.G (phase A has read them all).  Every thread calls it; it ends with a
// barrier after the last read of s.G.
// ---------------------------------------------------------------------------
template <bool PRO, typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_exact(const PrepIn& a, const ChunkPos& cp, const SL& s, unsigned char* dP,
                                           bool ab, int t0, int c0, int bw,
                                           const float (&G)[PrepGeom<E, D, C>::TPL][16 / sizeof(E)])
{
    typedef PrepGeom<E, D, C> S;
    typedef Frags<E, D, C> F;
    constexpr int NB = S::NB, VEC = S::VEC, LDM = S::LDM, LDX = S::LDX, KB = F::KB, NP = F::NP;
    const int tid = threadIdx.x;
    if (ab) {
#pragma unroll
        for (int j = 0; j < S::TPL; ++j)
#pragma unroll
            for (int x4 = 0; x4 < VEC / 4; ++x4)
                *reinterpret_cast<f32x4*>(s.G + (t0 + j) * D + c0 + 4 * x4) =
                    f32x4{G[j][4 * x4], G[j][4 * x4 + 1], G[j][4 * x4 + 2], G[j][4 * x4 + 3]};
    }
    __syncthreads();
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* b = (const E*)a.b;
    // prologue: per-token 1/|k|, 1/|q| from phase B, sigmoid on b
    const float* sRn = s.Rn();
    const bool pn = PRO && (a.pro & GDR2_PROLOGUE_NORM_QK), pg = PRO && (a.pro & GDR2_PROLOGUE_GATES);
    const float* sG = s.G;
    // M, every pair s < t
    for (int e = tid; e < C * C; e += NTP) {
        const int t = e / C, u = e % C;
        if (u >= t)
            continue;
        float m = 0.f;
        if (t < cp.L) {
            const int64_t xr = cp.row0 + (int64_t)t * a.H, xs = cp.row0 + (int64_t)u * a.H;
            for (int i = 0; i < D; ++i) {
                float br = to_f32(bw == 1 ? b[xr] : b[xr * D + i]);
                if (pg)
                    br = sigm(br);
                m += br * to_f32(k[xr * D + i]) * to_f32(k[xs * D + i]) * fast_exp2(sG[t * D + i] - sG[u * D + i]);
            }
            if (pn)
                m *= sRn[t] * sRn[u];
        }
        if ((t >> 4) == (u >> 4))
            s.Md()[t * LDX + (u & 15)] = m;
        else
            s.M()[t * LDM + u] = from_f32<E>(m);
    }
    // P, straight into its fragments (zeros above the diagonal)
    E* gP = reinterpret_cast<E*>(dP);
    for (int e = tid; e < NP * 16 * KB; e += NTP) {
        const int f = e / (16 * KB), r = (e / KB) % 16, kk = e % KB;
        int I = 0;
        while (I + 1 < NB && F::p_offset(I + 1) <= f)
            ++I;
        const int m = f - F::p_offset(I);
        const int t = 16 * I + r, u = KB * m + kk;
        float p = 0.f;
        if (u <= t && t < cp.L) {
            const int64_t xr = cp.row0 + (int64_t)t * a.H, xs = cp.row0 + (int64_t)u * a.H;
            for (int i = 0; i < D; ++i)
                p += to_f32(q[xr * D + i]) * to_f32(k[xs * D + i]) * fast_exp2(sG[t * D + i] - sG[u * D + i]);
            if (pn)
                p *= sRn[C + t] * sRn[u];
        }
        // lane (g, r) holds k = 4g..4g+3 of each 16-block of the fragment
        const int k16 = kk & 15, slot = 4 * (kk >> 4) + (k16 & 3);
        gP[f * (F::FRAG / sizeof(E)) + ((k16 >> 2) * 16 + r) * (16 / sizeof(E)) + slot] = from_f32<E>(p);
    }
    // K^ = k 2^(G_L - G) into the Kr rows (used below unscaled)
    for (int e = tid; e < C * D; e += NTP) {
        const int t = e / D, i = e % D;
        float kh = 0.f;
        if (t < cp.L)
            kh = to_f32(k[(cp.row0 + (int64_t)t * a.H) * D + i]) * fast_exp2(sG[(C - 1) * D + i] - sG[t * D + i]) *
                 (pn ? sRn[t] : 1.f);
        s.Kr()[swz<E, D>(t, i)] = from_f32<E>(kh);
    }
    __syncthreads();   // every read of G is done
}

// ---------------------------------------------------------------------------
// Phase C2, wave 0: X = (I + M)^-1 into s.X() (fragment k order).  The 16x16
// diagonal blocks by lane-per-column substitution (fp32), then
// X_IJ = -X_II sum_K M_IK X_KJ block by block on MFMA with the earlier blocks
// kept as accumulators.  Entries of s.X() above the diagonal are not written
// (the caller keeps them zero).
// ---------------------------------------------------------------------------
template <typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_inverse(const SL& s, int lane)
{
    typedef PrepGeom<E, D, C> S;
    typedef Mma16<E> M16;
    constexpr int NB = S::NB, LDM = S::LDM, LDXP = S::LDXP, LDX = S::LDX;
    const int gq = lane >> 4, cl = lane & 15;
    if (gq < NB) {
        // column cl of X_gq,gq by forward substitution
        const float* m = s.Md() + gq * 16 * LDX;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc0 = r == cl ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
            for (int c = 0; c + 1 < r; c += 2) {
                acc0 -= m[r * LDX + c] * x[c];
                acc1 -= m[r * LDX + c + 1] * x[c + 1];
            }
            if (r & 1)
                acc0 -= m[r * LDX + r - 1] * x[r - 1];
            x[r] = acc0 + acc1;
        }
        float* xc = s.Xc() + (gq * 16 + cl) * LDX;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<f32x4*>(xc + 4 * r4) = f32x4{x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]};
    }
    lds_fence_wave();
    f32x4 Xt[NB][NB];
    typename M16::Frag nx[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        // accumulator tile X_II[4gq + i][cl]
        Xt[I][I] = *reinterpret_cast<const f32x4*>(s.Xc() + (16 * I + cl) * LDX + 4 * gq);
        // A operand -X_II[cl][4gq + i]
        f32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            t[i] = -s.Xc()[(16 * I + 4 * gq + i) * LDX + cl];
        nx[I] = M16::pack(t);
    }
#pragma unroll
    for (int d = 1; d < NB; ++d) {
#pragma unroll
        for (int I = d; I < NB; ++I) {
            const int J = I - d;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int K = J; K < I; ++K)
                y = M16::mma(M16::load(s.M() + (16 * I + cl) * LDM + 16 * K + 4 * gq), M16::pack(Xt[K][J]), y);
            Xt[I][J] = M16::mma(nx[I], M16::pack(y), f32x4{0.f, 0.f, 0.f, 0.f});
        }
    }
    // X into LDS rows in fragment k order
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int J = 0; J <= I; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s.X()[(16 * I + 4 * gq + i) * LDXP + kpos<E>(16 * J + cl)] = from_f32<E>(Xt[I][J][i]);
}

// ---------------------------------------------------------------------------
// Phase C2, one K^T fragment (channel block c, token step m) from the Kr
// rows by identity transposes, scaled by the K^ factor of its half (1 on the
// exact path, whose Kr rows hold K^ already); the accumulators are the
// fragment.  Returns it as 16 bytes per lane.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, typename SL>
__device__ __forceinline__ u32x4 prep_kt_frag(const SL& s, int c, int m, bool guard,
                                              const typename Mma16<E>::Frag& ident, int lane)
{
    typedef PrepGeom<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma16<E> M16;
    constexpr int KT = F::KT, NH = S::NH;
    const int gq = lane >> 4, cl = lane & 15;
    f32x4 acc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        const int tb = KT * m + kt;
        acc[kt] = M16::mma(row4<E, D>(s.Kr(), 16 * tb + cl, 16 * c + 4 * gq), ident, f32x4{0.f, 0.f, 0.f, 0.f});
        const float f = guard ? 1.f : s.Fk()[(NH == 2 ? (tb >> 1) : 0) * D + 16 * c + cl];
        acc[kt] = acc[kt] * f;
    }
    return __builtin_bit_cast(u32x4, frag_of<E>(acc));
}

// The X fragments of phase D: row block T, token step m (m*KT <= T), from s.X().
template <typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_x_frags(const SL& s, typename Mma<E>::Frag* xf, int lane)
{
    typedef PrepGeom<E, D, C> S;
    typedef Frags<E, D, C> F;
    constexpr int NB = S::NB, LDXP = S::LDXP, VEC = S::VEC, KB = F::KB, KT = F::KT;
    const int gq = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int T = 0; T < NB; ++T)
#pragma unroll
        for (int m = 0; m <= T / KT; ++m)
            xf[F::p_offset(T) + m] =
                *reinterpret_cast<const typename Mma<E>::Frag*>(s.X() + (16 * T + cl) * LDXP + KB * m + VEC * gq);
}

// ---------------------------------------------------------------------------
// Phase D, -W: for key-channel step m2, W^T = E~^T X^T gives the -W
// fragments (T, m2) of every token block T in registers; each goes to
// dW + (T NKS + m2) KB + 16 lane.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_w(const SL& s, const typename Mma<E>::Frag* xf, int m2,
                                       unsigned char* dW, const typename Mma16<E>::Frag& ident, int lane)
{
    typedef PrepGeom<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef Mma16<E> M16;
    constexpr int NB = S::NB, NH = S::NH, KT = F::KT, NKS = F::NKS, NKC = F::NKC;
    const int gq = lane >> 4, cl = lane & 15;
    // E~^T fragments of channel blocks KT*m2.., every token step
    typename MM::Frag ea[KT][NKC];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        const int cb = KT * m2 + kt;
#pragma unroll
        for (int m = 0; m < NKC; ++m) {
            f32x4 tt[KT];
#pragma unroll
            for (int k2 = 0; k2 < KT; ++k2) {
                const int tb = KT * m + k2;
                const bool sec = NH == 2 && tb >= 2;
                tt[k2] = M16::mma(row4<E, D>(sec ? s.E2() : s.Eh(), sec ? 16 * tb - 32 + cl : 16 * tb + cl, 16 * cb + 4 * gq),
                                  ident, f32x4{0.f, 0.f, 0.f, 0.f});
            }
            ea[kt][m] = frag_of<E>(tt);
        }
    }
#pragma unroll
    for (int T = 0; T < NB; ++T) {
        f32x4 wt[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            wt[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m <= T / KT; ++m)
                wt[kt] = MM::mma(ea[kt][m], xf[F::p_offset(T) + m], wt[kt]);
            wt[kt] = -wt[kt];
        }
        stg16(dW + (T * NKS + m2) * F::FRAG + lane * 16, __builtin_bit_cast(u32x4, frag_of<E>(wt)));
    }
}

// ---------------------------------------------------------------------------
// Phase D, U~ = X u for value tile n of the UC columns in s.U(): the
// accumulator tiles of every token block T into ut[T].
// ---------------------------------------------------------------------------
template <int UC, typename E, int D, int C, typename SL>
__device__ __forceinline__ void prep_u_tile(const SL& s, const typename Mma<E>::Frag* xf, int n, f32x4* ut,
                                            const typename Mma16<E>::Frag& ident, int lane)
{
    typedef PrepGeom<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef Mma16<E> M16;
    constexpr int NB = S::NB, KT = F::KT, NKC = F::NKC;
    const int gq = lane >> 4, cl = lane & 15;
    typename MM::Frag ub[NKC];
#pragma unroll
    for (int m = 0; m < NKC; ++m) {
        f32x4 tt[KT];
#pragma unroll
        for (int k2 = 0; k2 < KT; ++k2)
            tt[k2] = M16::mma(row4<E, UC>(s.U(), 16 * (KT * m + k2) + cl, 16 * n + 4 * gq), ident,
                              f32x4{0.f, 0.f, 0.f, 0.f});
        ub[m] = frag_of<E>(tt);
    }
#pragma unroll
    for (int T = 0; T < NB; ++T) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m <= T / KT; ++m)
            acc = MM::mma(xf[F::p_offset(T) + m], ub[m], acc);
        ut[T] = acc;
    }
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

}  // namespace
}  // namespace gdr2
