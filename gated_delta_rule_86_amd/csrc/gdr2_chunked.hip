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
// Two kernels joined by a workspace:
//   chunk_prep  (every chunk of every sequence in parallel) writes -W, U~,
//               K^T, Q~ = q*2^G, P and gamma = 2^G_L per chunk;
//   chunk_state (one workgroup per (sequence, head, 64 value columns); the
//               value columns of S evolve independently, so they split
//               exactly) walks the chunks in order with the fp32 state in
//               MFMA accumulators.
// With few sequences x heads and many chunks, a two-level scan over chunk
// segments replaces the one pass (chunk_span, span_fold, then chunk_state
// per segment; see the section on it below).
//
// The workspace holds every factor in MFMA operand order.  A "fragment" is
// one A operand tile of the state kernel -- 16 rows x KB k-values (KB = 32
// for bf16, 16 for fp32), 16 bytes per lane, 1 KB -- stored lane-major; U~ is
// stored as accumulator tiles (4 values per lane).  The prep kernel produces
// each fragment in registers and writes it with one coalesced 16-byte store
// per lane; the state kernel copies a chunk's fragments into LDS linearly and
// reads each one with a single conflict-free 16-byte LDS read per lane.
#include "gdr2_device.h"
#include "gdr2_internal.h"

#include <algorithm>

namespace gdr2 {
namespace {

constexpr int NT = 256;            // threads of the state kernel (4 waves)
constexpr float kSpanMax = 80.f;   // largest decay exponent (log2) a factor may carry

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
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
// arrays -W, U~, K^T, Q~ (C*D elements each), P (NP fragments), gamma (D fp32).
struct Layout {
    int64_t nrec;
    size_t wn, ut, kh, qt, p, gam, span, total;
};

int p_frags(int C, int es)
{
    const int KT = es == 2 ? 2 : 1;
    int n = 0;
    for (int T = 0; T < C / 16; ++T)
        n += T / KT + 1;
    return n;
}

// nseg > 1 adds the segment area of the two-level scan: per (sequence, head)
// and per segment but the last, two D x D fp32 matrices (the segment's chunk
// product, then its local state).
Layout staged_layout(int64_t B, int64_t H, int64_t T, int D, int C, int esz, int64_t nseg)
{
    Layout L;
    L.nrec = B * H * ceil_div(T, C);
    const size_t mat = al256((size_t)L.nrec * C * D * esz);
    const size_t pm = al256((size_t)L.nrec * p_frags(C, esz) * 1024);
    const size_t gm = al256((size_t)L.nrec * D * 4);
    L.wn = 0;
    L.ut = mat;
    L.kh = 2 * mat;
    L.qt = 3 * mat;
    L.p = 4 * mat;
    L.gam = 4 * mat + pm;
    L.span = 4 * mat + pm + gm;
    L.total = L.span + (nseg > 1 ? al256((size_t)(B * H) * (nseg - 1) * 2 * D * D * 4) : 0);
    return L;
}

struct PrepArgs {
    const void *q, *k, *v, *b, *w;
    const float* g;
    int bw, ww, gw;
    int pro;                  // prologue bits (normalise q, k; activate gates)
    int64_t B, T, H, NC, nrec;
    void *Wn, *Ut, *Kh, *Qt, *P;
    float* gam;
};

struct StateArgs {
    const void *Wn, *Ut, *Kh, *Qt, *P;
    const float* gam;
    const float* S0;
    float* S_out;
    float* S_chunks;          // optional: the state at the start of every chunk
    void* o;
    int64_t T, H, NC, nbh;
    int64_t nseg, seg_len;    // chunk segments of the two-level scan (1, NC: one pass)
    float* span;              // segment area (nseg > 1)
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

// s_waitcnt lgkmcnt(0) with a compiler barrier: LDS writes of this wave are
// complete before any later LDS read of it (lanes exchange data this way).
// Prologue activations (logistic sigmoid; log-decay -softplus(x) = log sigmoid(-x)).
// (v_exp, v_log, v_rcp: about 1 ulp each; log(1 + e) loses e < 6e-8 absolute,
// far below the decay's own rounding)
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float neg_softplus(float x) { return -(fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)))); }
constexpr float kNormEps = 1e-6f;

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

// Work item -> chunk.  Items run in (sequence, chunk, head) order, so the
// workgroups in flight together read whole token rows: the H heads of a
// token are one contiguous run of H*D elements of the [B,T,H,.] inputs.
// Token row r of the chunk is element offset ((b*T + t0 + r)*H + h); the
// chunk's record in the workspace is (b*H + h)*NC + n.
struct ChunkPos {
    int64_t rec;      // workspace record
    int64_t row0;     // (b*T + t0)*H + h
    int L;            // valid tokens (>= 1)
};

// Walks the items blockIdx.x, blockIdx.x + gridDim.x, ... with carries, so
// the loop divides only once.  Item i is (m, b, h) with the head fastest and
// m = NC - 1 - n slowest: the chunks are visited last to first, so the
// records written last -- the ones the memory-side cache still holds when
// the state pass starts -- are the early chunks that pass reads first.
struct ItemWalk {
    int64_t m, b, h;          // current item, m = NC - 1 - n
    int64_t dm, db, dh;       // one step of gridDim.x items
    __device__ __forceinline__ void init(int64_t i, int64_t step, int64_t B, int64_t H)
    {
        const int64_t mb = i / H, sm = step / H;
        h = i - mb * H;
        b = mb % B;
        m = mb / B;
        dh = step - sm * H;
        db = sm % B;
        dm = sm / B;
    }
    __device__ __forceinline__ void advance(int64_t B, int64_t H)
    {
        h += dh;
        const int64_t ch = h >= H;
        h -= ch * H;
        b += db + ch;
        const int64_t cb = b >= B;
        b -= cb * B;
        m += dm + cb;
    }
    __device__ __forceinline__ ChunkPos pos(int64_t NC, int64_t T, int64_t H, int C) const
    {
        const int64_t n = NC - 1 - m, t0 = n * C;
        ChunkPos p;
        p.rec = (b * H + h) * NC + n;
        p.row0 = (b * T + t0) * H + h;
        p.L = (int)min((int64_t)C, T - t0);
        return p;
    }
};

// ---------------------------------------------------------------------------
// chunk_prep: 512 threads (8 waves), one workgroup per CU, looping over chunk
// records; the next chunk's inputs are loaded into registers while the
// current one computes.  Per chunk:
//
//  A  Cumulative log-decay, in registers.  Each lane owns VEC key channels of
//     TPL consecutive tokens (its 16-byte loads); the prefix sum runs within
//     the lane, across the LPC lanes sharing the channels (DPP row shifts) and
//     across waves through a small table of wave totals.
//  B  Decay-referenced operands, written to LDS rows (16-byte chunks XOR-
//     swizzled by row so fragment reads are conflict-free).  A chunk is split
//     into halves of 32 tokens; Gh is the cumulative decay at the end of the
//     first half (0 for tokens of the first half):
//        E^ = e 2^(G-Gh),  Q^ = q 2^(G-Gh),  Kr = k 2^(Gh-G),  u = w v,
//        second half also E~ = e 2^G, Q~ = q 2^G (chunk reference).
//     A tile of M (or P) with both 16-token blocks in one half is E^ Kr^T,
//     one across the halves is E~ Kr^T; both equal e_t k_s 2^(G_t-G_s) and no
//     factor exceeds 2^(half span).  A chunk whose exponents exceed kSpanMax
//     takes an exact pair-by-pair path for M, P and K^ instead.
//  C1 M tiles (transposed products, so each lane holds four consecutive
//     columns of one row) into LDS; P fragments straight to the workspace.
//  C2 One wave inverts I + M: the 16x16 diagonal blocks by lane-per-column
//     substitution (fp32), then X_IJ = -X_II sum_K M_IK X_KJ block by block
//     on MFMA with the earlier blocks kept as accumulators.  Meanwhile the
//     other waves form the K^T and Q~ fragments (transposes are MFMAs with an
//     identity operand, exact in bf16).
//  D  W^T = E~^T X^T gives the -W fragments in registers; U~ = X u gives the
//     U~ accumulator tiles.  Both go straight to the workspace.
// ---------------------------------------------------------------------------
constexpr int NTP = 512;           // threads of the prep kernel
constexpr int NWP = NTP / 64;      // its waves

template <typename E, int D, int C>
struct PrepShape {
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
    static constexpr size_t OFF_EH = 0;                              // E^ [C][D]
    static constexpr size_t OFF_QH = OFF_EH + C * ROWB;              // Q^ [C][D]
    static constexpr size_t OFF_KR = OFF_QH + C * ROWB;              // Kr [C][D] (exact path: K^)
    static constexpr size_t OFF_U = OFF_KR + C * ROWB;               // u  [C][D]
    static constexpr size_t OFF_E2 = OFF_U + C * ROWB;               // E~ [C-32][D] second half
    static constexpr size_t OFF_Q2 = OFF_E2 + (NH - 1) * 32 * ROWB;  // Q~ [C-32][D] second half
    static constexpr size_t OFF_M = al256(OFF_Q2 + (NH - 1) * 32 * ROWB);       // M [C][LDM], blocks below the diagonal
    static constexpr size_t OFF_MD = al256(OFF_M + (size_t)C * LDM * ES);       // M_II fp32 [NB][16][LDX]
    static constexpr size_t OFF_XC = OFF_MD + (size_t)NB * 16 * LDX * 4;        // X_II fp32, column j as row j
    static constexpr size_t OFF_X = al256(OFF_XC + (size_t)NB * 16 * LDX * 4);  // X [C][LDXP] in fragment k order
    static constexpr size_t OFF_TOT = al256(OFF_X + (size_t)C * LDXP * ES);     // wave totals [NWB][D]
    static constexpr size_t OFF_FK = OFF_TOT + (size_t)NWB * D * 4;             // 2^(G_L - Gh) [NH][D]
    static constexpr size_t OFF_RN = OFF_FK + (size_t)NH * D * 4;               // prologue: 1/|k|, 1/|q| [2][C]
    static constexpr size_t OFF_FLAG = OFF_RN + (size_t)2 * C * 4;
    static constexpr size_t SMEM = OFF_FLAG + 16;                               // dynamic LDS
    // raw g [C][D] (exact path: G) lives in its own static LDS object, so the
    // compiler knows the asynchronous copies into it touch nothing else
    static constexpr size_t SZ_G = (size_t)C * D * 4;
    static_assert(SMEM + SZ_G + 2 * C * 4 <= 160 * 1024, "LDS budget");   // + width-1 b, w
    static_assert(C == 32 || C == 64, "chunk");
    static_assert(64 % NCG == 0 && NCG >= 8 && TPL >= 1 && TW == LPC * TPL, "lane mapping");
    static_assert(NWB == NWP || NH == 1, "halves need every wave in phase B");
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
    typedef PrepShape<E, D, C> S;
    u32x4 k[S::TPL], q[S::TPL], v[S::TPL], b[S::TPL], w[S::TPL];
};

// Issue the token loads of one chunk for tokens t0.. of this lane, channels
// c0...  Rows past the valid length re-read the last valid row (in bounds)
// and are zeroed where they are used, so no load sits under a per-lane branch.
// PART: 0 = k, 1 = q, 2 = v, 3 = b, 4 = w (issued at different points of
// the previous chunk, so no wave stalls on a full memory queue).
template <int PART, int WB, int WW, typename E, int D, int C>
__device__ __forceinline__ void prep_load(const PrepArgs& a, const ChunkPos& cp, PrepRegs<E, D, C>& R,
                                          int t0, int c0)
{
    typedef PrepShape<E, D, C> S;
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
__device__ __forceinline__ void prep_copy_g(const PrepArgs& a, const ChunkPos& cp, unsigned char* sGraw,
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
__device__ __forceinline__ void prep_copy_bw(const PrepArgs& a, const ChunkPos& cp, unsigned int* sBW,
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
// VALID: every token of the chunk is valid (no zeroing needed).
template <bool VALID, bool SECOND, bool PRO, typename E, int D, int C>
__device__ __forceinline__ float prep_operands(const PrepRegs<E, D, C>& R, const float (*G)[16 / sizeof(E)],
                                               const float* gh, int bw, int ww, int L, int t0, int c0,
                                               unsigned char* smem, const unsigned int* sBW, int pro)
{
    typedef PrepShape<E, D, C> S;
    constexpr int VEC = S::VEC;
    E* sEh = reinterpret_cast<E*>(smem + S::OFF_EH);
    E* sQh = reinterpret_cast<E*>(smem + S::OFF_QH);
    E* sKr = reinterpret_cast<E*>(smem + S::OFF_KR);
    E* sU = reinterpret_cast<E*>(smem + S::OFF_U);
    E* sE2 = reinterpret_cast<E*>(smem + S::OFF_E2);
    E* sQ2 = reinterpret_cast<E*>(smem + S::OFF_Q2);
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
                    reinterpret_cast<float*>(smem + S::OFF_RN)[t] = rk;
            }
        }
#pragma unroll
        for (int x = 0; x < VEC; ++x) {
            kk[x] = valid ? kk[x] : 0.f;
            tmp[x] = kk[x] * fast_exp2(-d[x]);
            eh[x] = fast_exp2(d[x]);
        }
        sts16(sKr + o, pack_vec<E>(tmp));
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
        sts16(sEh + o, pack_vec<E>(tmp));
        if (SECOND)
            sts16(sE2 + o2, pack_vec<E>(tmp2));
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
                        reinterpret_cast<float*>(smem + S::OFF_RN)[C + t] = rq;
                }
            }
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                tmp[x] = (valid ? qq[x] : 0.f) * eh[x];
                if (SECOND)
                    tmp2[x] = tmp[x] * fh[x];
            }
        }
        sts16(sQh + o, pack_vec<E>(tmp));
        if (SECOND)
            sts16(sQ2 + o2, pack_vec<E>(tmp2));
        __builtin_amdgcn_sched_barrier(0);
        {
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
        }
        sts16(sU + o, pack_vec<E>(tmp));
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

// Gate widths WB, WW, WG: 1 or D fixed at compile time, 0 = read from the
// arguments (one variant serves every mix).
template <int WB, int WW, int WG, bool PRO, typename E, int D, int C>
__global__ __launch_bounds__(NTP) void chunk_prep_kernel(PrepArgs a)
{
    typedef PrepShape<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef Mma16<E> M16;
    constexpr int NB = S::NB, NH = S::NH, VEC = S::VEC, LDM = S::LDM, LDXP = S::LDXP, LDX = S::LDX;
    constexpr int KB = F::KB, KT = F::KT, NKS = F::NKS, NKC = F::NKC, NP = F::NP;

    extern __shared__ __align__(16) unsigned char smem[];
    E* sEh = reinterpret_cast<E*>(smem + S::OFF_EH);
    E* sQh = reinterpret_cast<E*>(smem + S::OFF_QH);
    E* sKr = reinterpret_cast<E*>(smem + S::OFF_KR);
    E* sU = reinterpret_cast<E*>(smem + S::OFF_U);
    E* sE2 = reinterpret_cast<E*>(smem + S::OFF_E2);
    E* sQ2 = reinterpret_cast<E*>(smem + S::OFF_Q2);
    E* sM = reinterpret_cast<E*>(smem + S::OFF_M);
    float* sMd = reinterpret_cast<float*>(smem + S::OFF_MD);
    float* sXc = reinterpret_cast<float*>(smem + S::OFF_XC);
    E* sX = reinterpret_cast<E*>(smem + S::OFF_X);
    float* sTot = reinterpret_cast<float*>(smem + S::OFF_TOT);
    float* sFk = reinterpret_cast<float*>(smem + S::OFF_FK);
    int* sFlag = reinterpret_cast<int*>(smem + S::OFF_FLAG);
    __shared__ __align__(16) float sG[C * D];
    __shared__ __align__(16) unsigned int sBW[2 * C];   // width-1 b and w of the chunk

    const int wave = threadIdx.x >> 6;
    const bool ab = wave < S::NWB;              // waves of phases A and B
    const bool second = NH == 2 && wave >= S::NWB / 2;
    const int bw = WB ? WB : a.bw, ww = WW ? WW : a.ww, gw = WG ? WG : a.gw;

    // X: the blocks above the diagonal that fragments cover stay zero
    for (int e = threadIdx.x; e < C * LDXP; e += NTP)
        sX[e] = from_f32<E>(0.f);

    // Token inputs: two register sets, Rn receives chunk n+1 while chunk n
    // computes from R, so every token load is issued a whole chunk ahead of
    // its use.  The log-decay goes straight to LDS (sG), issued as soon as
    // the previous chunk's rows have been read.
    PrepRegs<E, D, C> R, Rn;
    int64_t it = blockIdx.x;
    if (it >= a.nrec)
        return;
    ItemWalk walk;
    walk.init(it, gridDim.x, a.B, a.H);
    {
        const int lane = threadIdx.x & 63;
        const ChunkPos cp0 = walk.pos(a.NC, a.T, a.H, C);
        const int t0 = wave * S::TW + (lane % S::LPC) * S::TPL, c0 = (lane / S::LPC) * VEC;
        prep_copy_g<WG, E, D, C>(a, cp0, reinterpret_cast<unsigned char*>(sG), wave, lane);
        prep_copy_bw<WB, WW, E, D, C>(a, cp0, sBW, wave, lane);
        if (ab) {
            prep_load<0, WB, WW>(a, cp0, Rn, t0, c0);
            prep_load<1, WB, WW>(a, cp0, Rn, t0, c0);
            prep_load<2, WB, WW>(a, cp0, Rn, t0, c0);
            prep_load<3, WB, WW>(a, cp0, Rn, t0, c0);
            prep_load<4, WB, WW>(a, cp0, Rn, t0, c0);
        }
    }

    for (; it < a.nrec; it += gridDim.x) {
        // Lane indices are rederived every chunk from an opaque copy of the
        // thread id, so the compiler does not keep every lane-dependent
        // address of the loop body live across iterations.
        int tid = threadIdx.x;
        __asm__ __volatile__("" : "+v"(tid));
        const int lane = tid & 63, gq = lane >> 4, cl = lane & 15;
        const int cgp = lane / S::LPC, lpc = lane % S::LPC;
        const int t0 = wave * S::TW + lpc * S::TPL, c0 = cgp * VEC;
        wait_copies();
        __syncthreads();   // B0: this chunk's g rows are in LDS, its tokens in Rn
        R = Rn;
        const ChunkPos cp = walk.pos(a.NC, a.T, a.H, C);
        walk.advance(a.B, a.H);
        const int64_t next = it + gridDim.x;
        const bool pre = ab && next < a.nrec;   // this lane prefetches tokens
        const ChunkPos np = walk.pos(a.NC, a.T, a.H, C);
        if (pre) {
            prep_load<0, WB, WW>(a, np, Rn, t0, c0);
            prep_load<1, WB, WW>(a, np, Rn, t0, c0);
        }
        // identity B operand of the transposes: element (k = 4gq + i, n = cl)
        typename M16::Frag ident;
        {
            f32x4 id;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                id[i] = (4 * gq + i == cl) ? 1.f : 0.f;
            ident = M16::pack(id);
        }
        const int64_t rec = cp.rec;
        const bool full_chunk = cp.L == C;

        // ---- A: cumulative log2-decay in registers -------------------------
        float G[S::TPL][VEC];
        float excl[VEC];
        if (ab) {
#pragma unroll
            for (int j = 0; j < S::TPL; ++j) {
                const bool valid = full_chunk || t0 + j < cp.L;
                const bool act = PRO && (a.pro & GDR2_PROLOGUE_GATES);
                if (gw == 1) {
                    float gv = sG[t0 + j];
                    if (act)
                        gv = neg_softplus(gv);
#pragma unroll
                    for (int x = 0; x < VEC; ++x)
                        G[j][x] = valid ? gv * kLog2e : 0.f;
                } else {
#pragma unroll
                    for (int x4 = 0; x4 < VEC / 4; ++x4) {
                        f32x4 gv = *reinterpret_cast<const f32x4*>(sG + (t0 + j) * D + c0 + 4 * x4);
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
                    *reinterpret_cast<f32x4*>(sTot + wave * D + c0 + 4 * x4) =
                        f32x4{inc[4 * x4], inc[4 * x4 + 1], inc[4 * x4 + 2], inc[4 * x4 + 3]};
            }
        }
        if (tid == 0)
            *sFlag = 0;
        lds_barrier();   // B1: wave totals; the previous chunk is done with LDS
        if (pre)
            prep_load<2, WB, WW>(a, np, Rn, t0, c0);

        // ---- B: decay-referenced operands ----------------------------------
        float gh[VEC];
        if (ab) {
            float off[VEC];
#pragma unroll
            for (int x = 0; x < VEC; ++x)
                off[x] = gh[x] = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < S::NWB - 1; ++w2) {
                if (w2 < wave) {
#pragma unroll
                    for (int x4 = 0; x4 < VEC / 4; ++x4) {
                        const f32x4 tv = *reinterpret_cast<const f32x4*>(sTot + w2 * D + c0 + 4 * x4);
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
                    *reinterpret_cast<f32x4*>(sFk + c0 + 4 * x4) = v0;
                    *reinterpret_cast<f32x4*>(a.gam + rec * D + c0 + 4 * x4) = v0;
                    if (NH == 2)
                        *reinterpret_cast<f32x4*>(sFk + D + c0 + 4 * x4) =
                            f32x4{f1[4 * x4], f1[4 * x4 + 1], f1[4 * x4 + 2], f1[4 * x4 + 3]};
                }
            }
            float mx;
            if (second)
                mx = full_chunk ? prep_operands<true, true, PRO, E, D, C>(R, G, gh, bw, ww, cp.L, t0, c0, smem, sBW, a.pro)
                                : prep_operands<false, true, PRO, E, D, C>(R, G, gh, bw, ww, cp.L, t0, c0, smem, sBW, a.pro);
            else
                mx = full_chunk ? prep_operands<true, false, PRO, E, D, C>(R, G, gh, bw, ww, cp.L, t0, c0, smem, sBW, a.pro)
                                : prep_operands<false, false, PRO, E, D, C>(R, G, gh, bw, ww, cp.L, t0, c0, smem, sBW, a.pro);
            if (mx > kSpanMax)
                *sFlag = 1;
            if (pre)
                prep_load<3, WB, WW>(a, np, Rn, t0, c0);
        }
        lds_barrier();   // B2: operands in LDS
        if (next < a.nrec)   // phase B has read this chunk's width-1 gates
            prep_copy_bw<WB, WW, E, D, C>(a, np, sBW, wave, lane);

        E* gP = (E*)a.P + rec * (F::P_BYTES / sizeof(E));
        if (pre)
            prep_load<4, WB, WW>(a, np, Rn, t0, c0);
        const bool guard = *sFlag != 0;
        if (!guard) {
            if (next < a.nrec)
                prep_copy_g<WG, E, D, C>(a, np, reinterpret_cast<unsigned char*>(sG), wave, lane);
            // ---- C1: M tiles (waves 0-3) and P fragments (waves 4-7) -------
            if (wave < NWP / 2) {
                constexpr int NTM = NB * (NB + 1) / 2;
                for (int tile = wave; tile < NTM; tile += NWP / 2) {
                    int I = 0;
                    while ((I + 1) * (I + 2) / 2 <= tile)
                        ++I;
                    const int J = tile - I * (I + 1) / 2;
                    const bool same = NH == 1 || (I >> 1) == (J >> 1);
                    const E* Bs = same ? sEh : sE2;
                    const int rb = same ? 16 * I + cl : 16 * I - 32 + cl;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        acc = MM::mma(row_frag<E, D>(sKr, 16 * J + cl, 4 * ks + gq),
                                      row_frag<E, D>(Bs, rb, 4 * ks + gq), acc);
                    // lane: M[16I + cl][16J + 4gq + i]
                    if (J < I) {
                        *reinterpret_cast<typename M16::Frag*>(sM + (16 * I + cl) * LDM + 16 * J + 4 * gq) =
                            M16::pack(acc);
                    } else {
                        f32x4 m;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            m[i] = 4 * gq + i < cl ? acc[i] : 0.f;
                        *reinterpret_cast<f32x4*>(sMd + (16 * I + cl) * LDX + 4 * gq) = m;
                    }
                }
            } else {
                for (int f = wave - NWP / 2; f < NP; f += NWP / 2) {
                    int I = 0;
                    while (I + 1 < NB && F::p_offset(I + 1) <= f)
                        ++I;
                    const int m = f - F::p_offset(I);
                    f32x4 acc[KT];
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) {
                        const int J = KT * m + kt;
                        acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (J > I)
                            continue;
                        const bool same = NH == 1 || (I >> 1) == (J >> 1);
                        const E* Bs = same ? sQh : sQ2;
                        const int rb = same ? 16 * I + cl : 16 * I - 32 + cl;
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks)
                            acc[kt] = MM::mma(row_frag<E, D>(sKr, 16 * J + cl, 4 * ks + gq),
                                              row_frag<E, D>(Bs, rb, 4 * ks + gq), acc[kt]);
                        if (J == I) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[kt][i] = 4 * gq + i <= cl ? acc[kt][i] : 0.f;
                        }
                    }
                    stg16(reinterpret_cast<unsigned char*>(gP) + f * F::FRAG + lane * 16,
                          __builtin_bit_cast(u32x4, frag_of<E>(acc)));
                }
            }
        } else {
            // ---- exact path for a chunk with steep decay -------------------
            // G over the raw rows in sG (phase A has read them all)
            if (ab) {
#pragma unroll
                for (int j = 0; j < S::TPL; ++j)
#pragma unroll
                    for (int x4 = 0; x4 < VEC / 4; ++x4)
                        *reinterpret_cast<f32x4*>(sG + (t0 + j) * D + c0 + 4 * x4) =
                            f32x4{G[j][4 * x4], G[j][4 * x4 + 1], G[j][4 * x4 + 2], G[j][4 * x4 + 3]};
            }
            __syncthreads();
            const E* q = (const E*)a.q;
            const E* k = (const E*)a.k;
            const E* b = (const E*)a.b;
            // prologue: per-token 1/|k|, 1/|q| from phase B, sigmoid on b
            const float* sRn = reinterpret_cast<const float*>(smem + S::OFF_RN);
            const bool pn = PRO && (a.pro & GDR2_PROLOGUE_NORM_QK), pg = PRO && (a.pro & GDR2_PROLOGUE_GATES);
            // M, every pair s < t
            for (int e = tid; e < C * C; e += NTP) {
                const int t = e / C, s = e % C;
                if (s >= t)
                    continue;
                float m = 0.f;
                if (t < cp.L) {
                    const int64_t xr = cp.row0 + (int64_t)t * a.H, xs = cp.row0 + (int64_t)s * a.H;
                    for (int i = 0; i < D; ++i) {
                        float br = to_f32(bw == 1 ? b[xr] : b[xr * D + i]);
                        if (pg)
                            br = sigm(br);
                        m += br * to_f32(k[xr * D + i]) * to_f32(k[xs * D + i]) *
                             fast_exp2(sG[t * D + i] - sG[s * D + i]);
                    }
                    if (pn)
                        m *= sRn[t] * sRn[s];
                }
                if ((t >> 4) == (s >> 4))
                    sMd[t * LDX + (s & 15)] = m;
                else
                    sM[t * LDM + s] = from_f32<E>(m);
            }
            // P, straight into its fragments (zeros above the diagonal)
            for (int e = tid; e < NP * 16 * KB; e += NTP) {
                const int f = e / (16 * KB), r = (e / KB) % 16, kk = e % KB;
                int I = 0;
                while (I + 1 < NB && F::p_offset(I + 1) <= f)
                    ++I;
                const int m = f - F::p_offset(I);
                const int t = 16 * I + r, s = KB * m + kk;
                float p = 0.f;
                if (s <= t && t < cp.L) {
                    const int64_t xr = cp.row0 + (int64_t)t * a.H, xs = cp.row0 + (int64_t)s * a.H;
                    for (int i = 0; i < D; ++i)
                        p += to_f32(q[xr * D + i]) * to_f32(k[xs * D + i]) * fast_exp2(sG[t * D + i] - sG[s * D + i]);
                    if (pn)
                        p *= sRn[C + t] * sRn[s];
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
                sKr[swz<E, D>(t, i)] = from_f32<E>(kh);
            }
            __syncthreads();   // every read of G is done
            if (next < a.nrec)
                prep_copy_g<WG, E, D, C>(a, np, reinterpret_cast<unsigned char*>(sG), wave, lane);
        }
        lds_barrier();   // B3: M in LDS

        // ---- C2: X = (I + M)^-1 (wave 0); K^T and Q~ fragments (others) --
        if (wave == 0) {
            if (gq < NB) {
                // column cl of X_gq,gq by forward substitution
                const float* m = sMd + gq * 16 * LDX;
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
                float* xc = sXc + (gq * 16 + cl) * LDX;
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
                Xt[I][I] = *reinterpret_cast<const f32x4*>(sXc + (16 * I + cl) * LDX + 4 * gq);
                // A operand -X_II[cl][4gq + i]
                f32x4 t;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    t[i] = -sXc[(16 * I + 4 * gq + i) * LDX + cl];
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
                        y = M16::mma(M16::load(sM + (16 * I + cl) * LDM + 16 * K + 4 * gq), M16::pack(Xt[K][J]), y);
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
                        sX[(16 * I + 4 * gq + i) * LDXP + kpos<E>(16 * J + cl)] = from_f32<E>(Xt[I][J][i]);
        } else {
            constexpr int NK = (D / 16) * NKC, NQ = NB * NKS;
            E* gKh = (E*)a.Kh + rec * (F::K_BYTES / sizeof(E));
            E* gQt = (E*)a.Qt + rec * (F::W_BYTES / sizeof(E));
            for (int task = wave - 1; task < NK + NQ; task += NWP - 1) {
                if (task < NK) {
                    // K^T fragment (channel block c, token step m)
                    const int c = task / NKC, m = task % NKC;
                    f32x4 acc[KT];
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) {
                        const int tb = KT * m + kt;
                        acc[kt] = M16::mma(row4<E, D>(sKr, 16 * tb + cl, 16 * c + 4 * gq), ident,
                                           f32x4{0.f, 0.f, 0.f, 0.f});
                        const float f = guard ? 1.f : sFk[(NH == 2 ? (tb >> 1) : 0) * D + 16 * c + cl];
                        acc[kt] = acc[kt] * f;
                    }
                    stg16(reinterpret_cast<unsigned char*>(gKh) + task * F::FRAG + lane * 16,
                          __builtin_bit_cast(u32x4, frag_of<E>(acc)));
                } else {
                    // Q~ fragment (token block T, channel step m)
                    const int fq = task - NK, T = fq / NKS, m = fq % NKS;
                    const bool sec = NH == 2 && T >= 2;
                    const E* src = sec ? sQ2 : sQh;
                    const int r = sec ? 16 * T - 32 + cl : 16 * T + cl;
                    u32x4 v;
                    if constexpr (sizeof(E) == 2) {
                        const u32x2 lo = __builtin_bit_cast(u32x2, row4<E, D>(src, r, KB * m + 4 * gq));
                        const u32x2 hi = __builtin_bit_cast(u32x2, row4<E, D>(src, r, KB * m + 16 + 4 * gq));
                        v = u32x4{lo[0], lo[1], hi[0], hi[1]};
                    } else {
                        v = __builtin_bit_cast(u32x4, row4<E, D>(src, r, KB * m + 4 * gq));
                    }
                    stg16(reinterpret_cast<unsigned char*>(gQt) + fq * F::FRAG + lane * 16, v);
                }
            }
        }
        lds_barrier();   // B4: X in LDS

        // ---- D: -W fragments (waves 0-3), U~ tiles (waves 4-7) ------------
        {
            typename MM::Frag xf[NP];
#pragma unroll
            for (int T = 0; T < NB; ++T)
#pragma unroll
                for (int m = 0; m <= T / KT; ++m)
                    xf[F::p_offset(T) + m] =
                        *reinterpret_cast<const typename MM::Frag*>(sX + (16 * T + cl) * LDXP + KB * m + VEC * gq);
            if (wave < NWP / 2) {
                E* gWn = (E*)a.Wn + rec * (F::W_BYTES / sizeof(E));
                for (int m2 = wave; m2 < NKS; m2 += NWP / 2) {
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
                                tt[k2] = M16::mma(row4<E, D>(sec ? sE2 : sEh, sec ? 16 * tb - 32 + cl : 16 * tb + cl,
                                                             16 * cb + 4 * gq),
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
                        stg16(reinterpret_cast<unsigned char*>(gWn) + (T * NKS + m2) * F::FRAG + lane * 16,
                              __builtin_bit_cast(u32x4, frag_of<E>(wt)));
                    }
                }
            } else {
                E* gUt = (E*)a.Ut + rec * (F::U_BYTES / sizeof(E));
                for (int n = wave - NWP / 2; n < D / 16; n += NWP / 2) {
                    typename MM::Frag ub[NKC];
#pragma unroll
                    for (int m = 0; m < NKC; ++m) {
                        f32x4 tt[KT];
#pragma unroll
                        for (int k2 = 0; k2 < KT; ++k2)
                            tt[k2] = M16::mma(row4<E, D>(sU, 16 * (KT * m + k2) + cl, 16 * n + 4 * gq), ident,
                                              f32x4{0.f, 0.f, 0.f, 0.f});
                        ub[m] = frag_of<E>(tt);
                    }
#pragma unroll
                    for (int T = 0; T < NB; ++T) {
                        f32x4 ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int m = 0; m <= T / KT; ++m)
                            ut = MM::mma(xf[F::p_offset(T) + m], ub[m], ut);
                        E* dst = gUt + (n * NB + T) * (F::TILE_U / sizeof(E)) + lane * 4;
                        *reinterpret_cast<typename Mma16<E>::Frag*>(dst) = M16::pack(ut);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// chunk_state: carries the fp32 state through the chunks of one sequence and
// head, BV value columns per workgroup (16 per wave), and writes o.
//
// A chunk's fragments (-W, Q~, K^T, P, this slice's U~ tiles, gamma) are
// copied from the workspace straight into LDS with global_load_lds_dwordx4
// (no register staging), double buffered: the copy of chunk n + 1 is in
// flight while chunk n computes.  The two buffers are separate static LDS
// objects so that reads of one are never ordered behind the copies into the
// other.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, int BV>
struct StateShape {
    typedef Frags<E, D, C> F;
    static constexpr int NB = C / 16;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int VEC = 16 / ES;
    static constexpr int NS = D / BV;                       // column slices per (b,h)
    static constexpr int NTU = BV / 16;                     // value tiles per slice
    static constexpr int LDO = 16 + VEC;                    // per-wave output staging rows
    static constexpr size_t U_SLICE = (size_t)NTU * NB * F::TILE_U;
    static constexpr size_t OFF_W = 0;                      // byte offsets in one buffer
    static constexpr size_t OFF_Q = OFF_W + F::W_BYTES;
    static constexpr size_t OFF_KT = OFF_Q + F::W_BYTES;
    static constexpr size_t OFF_P = OFF_KT + F::K_BYTES;
    static constexpr size_t OFF_U = OFF_P + F::P_BYTES;
    static constexpr size_t OFF_G = OFF_U + U_SLICE;        // gamma: D floats
    static constexpr size_t BUF = OFF_G + (size_t)D * 4;
    static constexpr size_t SZ_O = (size_t)(NT / 64) * C * LDO * ES;
    // double buffering when two buffers fit; else one
    static constexpr int NBUF = 2 * BUF + SZ_O <= 160 * 1024 ? 2 : 1;
    static constexpr size_t SMEM = NBUF * BUF + SZ_O;
    static_assert(BV == 16 * (NT / 64), "one 16-column tile per wave");
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(U_SLICE % 1024 == 0, "U~ slice copies");
};

typedef __attribute__((address_space(3))) void lds_void;

// Copy BYTES (a multiple of 1 KB) from global to LDS, 16 bytes per lane per
// instruction; instruction j belongs to wave j % 4.
template <size_t BYTES>
__device__ __forceinline__ void copy_linear(const unsigned char* g, unsigned char* l, int wave, int lane)
{
    constexpr int NINST = (int)(BYTES / 1024);
#pragma unroll
    for (int j = wave; j < NINST; j += NT / 64)
        __builtin_amdgcn_global_load_lds(g + j * 1024 + lane * 16, (lds_void*)(l + j * 1024), 16, 0, 0);
}

template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_fetch(const StateArgs& a, int64_t rec, int slice, unsigned char* buf,
                                            int wave, int lane)
{
    typedef StateShape<E, D, C, BV> S;
    typedef Frags<E, D, C> F;
    copy_linear<F::W_BYTES>((const unsigned char*)a.Wn + rec * F::W_BYTES, buf + S::OFF_W, wave, lane);
    copy_linear<F::W_BYTES>((const unsigned char*)a.Qt + rec * F::W_BYTES, buf + S::OFF_Q, wave, lane);
    copy_linear<F::K_BYTES>((const unsigned char*)a.Kh + rec * F::K_BYTES, buf + S::OFF_KT, wave, lane);
    copy_linear<F::P_BYTES>((const unsigned char*)a.P + rec * F::P_BYTES, buf + S::OFF_P, wave, lane);
    copy_linear<S::U_SLICE>((const unsigned char*)a.Ut + rec * F::U_BYTES + slice * S::U_SLICE, buf + S::OFF_U,
                            wave, lane);
    // gamma: D floats
    if (wave == (NT / 64) - 1 && lane < D / 4)
        __builtin_amdgcn_global_load_lds(a.gam + rec * D + lane * 4, (lds_void*)(buf + S::OFF_G), 16, 0, 0);
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


template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_store_o(const StateArgs& a, const E* sOw, int64_t b, int64_t h,
                                             int slice, int64_t n, int lane, int wave);

// The state at the start of chunk n (this lane's column, its 4 rows per
// tile) into the checkpoint output.
template <int D>
__device__ __forceinline__ void state_emit(const StateArgs& a, const f32x4* St, int64_t bh, int64_t n,
                                           int gq, int col)
{
    constexpr int KTS = D / 16;
    float* dst = a.S_chunks + (bh * a.NC + n) * D * D;
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[(16 * kt + 4 * gq + i) * D + col] = St[kt][i];
}

// One chunk from buffer `buf`: Delta = U~ - W S, O = Q~ S + P Delta,
// S <- diag(gamma) S + K^T Delta; O goes out through the wave's staging rows.
template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_compute(const StateArgs& a, const unsigned char* buf, E* sOw, f32x4* St,
                                              int64_t b, int64_t h, int slice, int64_t n, bool store_prev,
                                              int lane, int wave)
{
    typedef StateShape<E, D, C, BV> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef typename MM::Frag Frag;
    constexpr int NB = S::NB, LDO = S::LDO, KT = F::KT, NKS = F::NKS, NKC = F::NKC;
    constexpr int KTS = D / 16;
    const int gq = lane >> 4, cl = lane & 15;
    const unsigned char* fl = buf + lane * 16;
    auto frag = [&](size_t off, int i) -> Frag { return *reinterpret_cast<const Frag*>(fl + off + i * F::FRAG); };
    const float* sGam = reinterpret_cast<const float*>(buf + S::OFF_G);

    Frag SB[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        SB[ks] = MM::from_acc(&St[ks * KT]);

    // Delta = U~ - W S  (W is stored negated).  Each phase reads all of its
    // A fragments before its MFMAs so LDS latency overlaps.
    f32x4 dl[NB];
    {
        Frag aw[NB][NKS];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                aw[mt][ks] = frag(S::OFF_W, mt * NKS + ks);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            const E* u = reinterpret_cast<const E*>(buf + S::OFF_U + (wave * NB + mt) * F::TILE_U) + lane * 4;
            dl[mt] = f32x4{to_f32(u[0]), to_f32(u[1]), to_f32(u[2]), to_f32(u[3])};
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                dl[mt] = MM::mma(aw[mt][ks], SB[ks], dl[mt]);
        sched_pipeline<NB * NKS>();
    }
    Frag DB[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        DB[kc] = MM::from_acc(&dl[kc * KT]);
    // the previous chunk's outputs leave while this one computes
    if (store_prev)
        state_store_o<E, D, C, BV>(a, sOw, b, h, slice, n - 1, lane, wave);

    // O = Q~ S + P Delta  (P is lower triangular: only stored steps).
    f32x4 ot[NB];
    {
        Frag aq[NB][NKS], ap[F::NP];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                aq[mt][ks] = frag(S::OFF_Q, mt * NKS + ks);
#pragma unroll
        for (int i = 0; i < F::NP; ++i)
            ap[i] = frag(S::OFF_P, i);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
            ot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                ot[mt] = MM::mma(aq[mt][ks], SB[ks], ot[mt]);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int kc = 0; kc <= mt / KT; ++kc)
                ot[mt] = MM::mma(ap[F::p_offset(mt) + kc], DB[kc], ot[mt]);
        sched_pipeline<NB * NKS>();
    }

    // S <- diag(gamma) S + K^T Delta.
    {
        Frag ak[KTS][NKC];
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                ak[kt][kc] = frag(S::OFF_KT, kt * NKC + kc);
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
    __shared__ __align__(16) unsigned char buf0[S::BUF];
    __shared__ __align__(16) unsigned char buf1[S::NBUF == 2 ? S::BUF : 16];
    __shared__ __align__(16) E sO[(NT / 64) * C * S::LDO];

    // Workgroup -> (sequence*head, chunk segment, column slice).  The NS
    // slices of one segment read the same chunk records: give them the same
    // blockIdx % 8 so they land on the same XCD and share its L2.
    const int64_t bx = blockIdx.x;
    const int64_t grp = bx / (8 * S::NS);
    const int within = (int)(bx % (8 * S::NS));
    const int slice = within / 8;
    const int64_t unit = grp * 8 + within % 8;       // (b*H + h) * nseg + segment
    if (unit >= a.nbh * a.nseg)
        return;
    const int64_t bh = unit / a.nseg, seg = unit - bh * a.nseg;
    const int64_t b = bh / a.H, h = bh - b * a.H, rec0 = bh * a.NC;
    const int64_t n0 = seg * a.seg_len, n1 = min(a.NC, n0 + a.seg_len);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4, cl = lane & 15;
    const int col = slice * BV + 16 * wave + cl;     // this lane's state column
    E* sOw = sO + wave * C * S::LDO;

    // start state: S0 (or zero) for the first segment -- with segments, the
    // span pass's copy of it, as S_out may be S0 -- else the one the segment
    // fold left in the local-state half of the previous segment
    const float* s0 = seg > 0   ? a.span + ((bh * (a.nseg - 1) + seg - 1) * 2 + 1) * D * D
                      : !a.S0   ? nullptr
                      : a.nseg > 1 ? a.span + bh * (a.nseg - 1) * 2 * D * D
                                   : a.S0 + bh * D * D;
    f32x4 St[KTS];
    if (s0) {
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                St[kt][i] = s0[(16 * kt + 4 * gq + i) * D + col];
    } else {
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
            St[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    state_fetch<E, D, C, BV>(a, rec0 + n0, slice, buf0, wave, lane);
    if (S::NBUF == 2) {
        for (int64_t n = n0; n < n1; n += 2) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0; everyone is done with buf1
            if (n + 1 < n1)
                state_fetch<E, D, C, BV>(a, rec0 + n + 1, slice, buf1, wave, lane);
            if (a.S_chunks)
                state_emit<D>(a, St, bh, n, gq, col);
            state_compute<E, D, C, BV>(a, buf0, sOw, St, b, h, slice, n, n > n0, lane, wave);
            if (n + 1 >= n1)
                break;
            wait_copies();
            __syncthreads();          // chunk n + 1 is in buf1; everyone is done with buf0
            if (n + 2 < n1)
                state_fetch<E, D, C, BV>(a, rec0 + n + 2, slice, buf0, wave, lane);
            if (a.S_chunks)
                state_emit<D>(a, St, bh, n + 1, gq, col);
            state_compute<E, D, C, BV>(a, buf1, sOw, St, b, h, slice, n + 1, true, lane, wave);
        }
    } else {
        for (int64_t n = n0; n < n1; ++n) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0
            if (a.S_chunks)
                state_emit<D>(a, St, bh, n, gq, col);
            state_compute<E, D, C, BV>(a, buf0, sOw, St, b, h, slice, n, n > n0, lane, wave);
            __syncthreads();          // everyone is done with buf0
            if (n + 1 < n1)
                state_fetch<E, D, C, BV>(a, rec0 + n + 1, slice, buf0, wave, lane);
        }
    }

    state_store_o<E, D, C, BV>(a, sOw, b, h, slice, n1 - 1, lane, wave);

    if (a.S_out && n1 == a.NC) {
        float* so = a.S_out + bh * D * D;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[(16 * kt + 4 * gq + i) * D + col] = St[kt][i];
    }
}

// ---------------------------------------------------------------------------
// Two-level scan over the chunks, for few (sequence, head) pairs and many
// chunks, where one pass over the chunks would leave most CUs idle.  A chunk
// step is affine in the state: S_next = A S + B with A = diag(gamma) - K^T W
// and B = K^T U~.  The chunks of a sequence are cut into nseg segments of
// seg_len chunks (the last may be shorter):
//   span  every segment but the last, in parallel: the product of its
//         chunks' A (carried from the identity, as D more state columns)
//         and its local state (carried from zero; from S0 for segment 0,
//         which then holds the true state at the start of segment 1);
//   fold  per (sequence, head), over the segments in order: start of
//         segment j+1 = (product of segment j) (start of segment j) + (local
//         state of segment j), in fp32, written over the local state;
//   state the chunk pass above, every segment in parallel from its start.
// The span pass runs the same chunk step as the state pass without the
// outputs, so it needs only -W, K^T, gamma (and U~ for local-state columns).
// ---------------------------------------------------------------------------
template <typename E, int D, int C>
struct SpanShape {
    typedef Frags<E, D, C> F;
    static constexpr size_t OFF_W = 0;
    static constexpr size_t OFF_KT = OFF_W + F::W_BYTES;
    static constexpr size_t OFF_G = OFF_KT + F::K_BYTES;
    static constexpr size_t BUF = OFF_G + (size_t)D * 4;
    static_assert(2 * BUF <= 80 * 1024, "two workgroups per CU");
};

// Four U~ values of one accumulator tile, held raw until they are used so
// that the load of the next chunk's values stays in flight.
template <typename E> struct Quad;
template <> struct Quad<bf16> {
    typedef u32x2 Raw;
    static __device__ __forceinline__ Raw load(const bf16* p) { return *reinterpret_cast<const u32x2*>(p); }
    static __device__ __forceinline__ f32x4 cvt(Raw r) {
        return f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u),
                     __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xffff0000u)};
    }
};
template <> struct Quad<float> {
    typedef f32x4 Raw;
    static __device__ __forceinline__ Raw load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ f32x4 cvt(Raw r) { return r; }
};

template <typename E, int D, int C>
__device__ __forceinline__ void span_fetch(const StateArgs& a, int64_t rec, unsigned char* buf, int wave, int lane)
{
    typedef SpanShape<E, D, C> S;
    typedef Frags<E, D, C> F;
    copy_linear<F::W_BYTES>((const unsigned char*)a.Wn + rec * F::W_BYTES, buf + S::OFF_W, wave, lane);
    copy_linear<F::K_BYTES>((const unsigned char*)a.Kh + rec * F::K_BYTES, buf + S::OFF_KT, wave, lane);
    if (wave == (NT / 64) - 1 && lane < D / 4)
        __builtin_amdgcn_global_load_lds(a.gam + rec * D + lane * 4, (lds_void*)(buf + S::OFF_G), 16, 0, 0);
}

// One chunk step without outputs: Delta = U~ - W X, X <- diag(gamma) X + K^T Delta.
template <typename E, int D, int C>
__device__ __forceinline__ void span_compute(const unsigned char* buf, const f32x4* uc, f32x4* St, int lane)
{
    typedef SpanShape<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef typename MM::Frag Frag;
    constexpr int NB = F::NB, KT = F::KT, NKS = F::NKS, NKC = F::NKC, KTS = D / 16;
    const int gq = lane >> 4;
    const unsigned char* fl = buf + lane * 16;
    auto frag = [&](size_t off, int i) -> Frag { return *reinterpret_cast<const Frag*>(fl + off + i * F::FRAG); };
    const float* sGam = reinterpret_cast<const float*>(buf + S::OFF_G);

    Frag SB[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        SB[ks] = MM::from_acc(&St[ks * KT]);
    f32x4 dl[NB];
    {
        Frag aw[NB][NKS];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                aw[mt][ks] = frag(S::OFF_W, mt * NKS + ks);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
            dl[mt] = uc[mt];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < NB; ++mt)
                dl[mt] = MM::mma(aw[mt][ks], SB[ks], dl[mt]);
        sched_pipeline<NB * NKS>();
    }
    Frag DB[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        DB[kc] = MM::from_acc(&dl[kc * KT]);
    {
        Frag ak[KTS][NKC];
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                ak[kt][kc] = frag(S::OFF_KT, kt * NKC + kc);
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
}

// Workgroup -> (sequence*head, segment j < nseg - 1, column slice): slices
// 0 .. NS-1 carry the chunk product's columns, NS .. 2NS-1 the local state's.
template <typename E, int D, int C, int BV>
__global__ __launch_bounds__(NT, 2) void chunk_span_kernel(StateArgs a)
{
    typedef SpanShape<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Quad<E> Q;
    constexpr int NS = D / BV, NB = F::NB, KTS = D / 16;
    constexpr size_t U_SLICE = (size_t)(BV / 16) * NB * F::TILE_U;
    __shared__ __align__(16) unsigned char buf[2][S::BUF];

    const int64_t bx = blockIdx.x;
    const int64_t grp = bx / (8 * 2 * NS);
    const int within = (int)(bx % (8 * 2 * NS));
    const int slice = within / 8;
    const int64_t unit = grp * 8 + within % 8;       // (b*H + h) * (nseg - 1) + j
    const int64_t nspan = a.nseg - 1;
    if (unit >= a.nbh * nspan)
        return;
    const int64_t bh = unit / nspan, j = unit - bh * nspan;
    const bool local = slice >= NS;
    if (j == 0 && !local)
        return;                                      // segment 0 needs no product
    const int vs = local ? slice - NS : slice;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4, cl = lane & 15;
    const int col = vs * BV + 16 * wave + cl;

    f32x4 St[KTS];
    if (local && j == 0 && a.S0) {
        const float* s0 = a.S0 + bh * D * D;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                St[kt][i] = s0[(16 * kt + 4 * gq + i) * D + col];
        // a copy of S0 in entry 0's product half (segment 0 has no product):
        // the state pass starts segment 0 from it, since S_out may be S0 and
        // the last segment writes S_out in that same pass
        float* c0 = a.span + bh * nspan * 2 * D * D;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                c0[(16 * kt + 4 * gq + i) * D + col] = St[kt][i];
    } else {
        const float one = local ? 0.f : 1.f;    // identity for the product, zero for the local state
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                St[kt][i] = 16 * kt + 4 * gq + i == col ? one : 0.f;
    }

    const int64_t rec0 = bh * a.NC + j * a.seg_len;
    // this lane's U~ values: value tile (vs, wave), row tiles 0 .. NB-1
    const E* ub = reinterpret_cast<const E*>((const unsigned char*)a.Ut + vs * U_SLICE +
                                             (size_t)wave * NB * F::TILE_U) + lane * 4;
    typename Q::Raw ur[NB];
    span_fetch<E, D, C>(a, rec0, buf[0], wave, lane);
    if (local) {
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
            ur[mt] = Q::load(ub + rec0 * (F::U_BYTES / sizeof(E)) + mt * (F::TILE_U / sizeof(E)));
    }
    for (int64_t i = 0; i < a.seg_len; ++i) {
        wait_copies();
        __syncthreads();              // chunk i is in buf[i&1]; everyone is done with the other
        f32x4 uc[NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
            uc[mt] = local ? Q::cvt(ur[mt]) : f32x4{0.f, 0.f, 0.f, 0.f};
        if (i + 1 < a.seg_len) {
            const int64_t rec = rec0 + i + 1;
            span_fetch<E, D, C>(a, rec, buf[(i + 1) & 1], wave, lane);
            if (local) {
#pragma unroll
                for (int mt = 0; mt < NB; ++mt)
                    ur[mt] = Q::load(ub + rec * (F::U_BYTES / sizeof(E)) + mt * (F::TILE_U / sizeof(E)));
            }
        }
        span_compute<E, D, C>(buf[i & 1], uc, St, lane);
    }

    float* dst = a.span + ((bh * nspan + j) * 2 + (local ? 1 : 0)) * D * D;
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[(16 * kt + 4 * gq + i) * D + col] = St[kt][i];
}

// Start states of segments 2 .. nseg-1, in order: for j = 1 .. nseg-2,
// X <- Pi_j X + L_j (X starts as the true state at the start of segment 1,
// which the span pass left in L_0), written over L_j.  Workgroup ->
// (sequence*head, 16 state columns); the D/16 workgroups of one (b,h) share
// blockIdx % 8 (one XCD, one L2 for the products they all read).  fp32 MFMA:
// wave w computes row tiles NRT*w .. NRT*w+NRT-1 of Pi_j X with X's column
// tiles as B operands straight from accumulator layout; the new X goes
// round through LDS so that every wave holds all of it.  The operands of
// the next two folds are in flight while one fold computes.
template <int D>
struct FoldOps {
    static constexpr int KTS = D / 16, NRT = KTS / 4;
    f32x4 A[NRT][KTS];      // rows of Pi_j: (row tile, 16-wide k block)
    f32x4 L[NRT];           // L_j at this lane's output positions
};

template <int D>
__device__ __forceinline__ void fold_load(FoldOps<D>& op, const float* base, int64_t j, int wave, int lane, int col)
{
    typedef Mma<float> MM;
    constexpr int KTS = FoldOps<D>::KTS, NRT = FoldOps<D>::NRT;
    const float* Pi = base + j * 2 * D * D;
    const float* L = Pi + D * D;
    const int gq = lane >> 4;
#pragma unroll
    for (int r = 0; r < NRT; ++r) {
        const int mt = wave * NRT + r;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
            op.A[r][kt] = MM::load(Pi + 16 * mt * D + 16 * kt, D, lane);
#pragma unroll
        for (int x = 0; x < 4; ++x)
            op.L[r][x] = L[(16 * mt + 4 * gq + x) * D + col];
    }
}

template <int D>
__device__ __forceinline__ void fold_step(const FoldOps<D>& op, f32x4* X, f32x4 (*sX)[64], float* base, int64_t j,
                                          int wave, int lane, int col)
{
    typedef Mma<float> MM;
    constexpr int KTS = FoldOps<D>::KTS, NRT = FoldOps<D>::NRT;
    const int gq = lane >> 4;
    f32x4 acc[NRT];
#pragma unroll
    for (int r = 0; r < NRT; ++r)
        acc[r] = op.L[r];
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
        for (int r = 0; r < NRT; ++r)
            acc[r] = MM::mma(op.A[r][kt], MM::from_acc(&X[kt]), acc[r]);
    float* L = base + (j * 2 + 1) * D * D;
#pragma unroll
    for (int r = 0; r < NRT; ++r) {
        const int mt = wave * NRT + r;
#pragma unroll
        for (int x = 0; x < 4; ++x)
            L[(16 * mt + 4 * gq + x) * D + col] = acc[r][x];
        sX[mt][lane] = acc[r];
    }
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt)
        X[kt] = sX[kt][lane];
    __syncthreads();              // sX is rewritten by the next fold
}

template <int D>
__global__ __launch_bounds__(256) void span_fold_kernel(float* span, int64_t nbh, int64_t nseg)
{
    constexpr int KTS = D / 16, NCB = D / 16;
    static_assert(KTS % 4 == 0, "row tiles split over 4 waves");
    __shared__ __align__(16) f32x4 sX[KTS][64];
    const int64_t bx = blockIdx.x;
    const int64_t grp = bx / (8 * NCB);
    const int within = (int)(bx % (8 * NCB));
    const int cb = within / 8;
    const int64_t bh = grp * 8 + within % 8;
    if (bh >= nbh)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, gq = lane >> 4, cl = lane & 15;
    const int col = cb * 16 + cl;
    const int64_t nspan = nseg - 1;
    float* base = span + bh * nspan * 2 * D * D;

    f32x4 X[KTS];
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
        for (int x = 0; x < 4; ++x)
            X[kt][x] = base[D * D + (16 * kt + 4 * gq + x) * D + col];
    FoldOps<D> op0, op1;
    if (nspan > 1)
        fold_load<D>(op0, base, 1, wave, lane, col);
    if (nspan > 2)
        fold_load<D>(op1, base, 2, wave, lane, col);
    for (int64_t j = 1; j < nspan; j += 2) {
        fold_step<D>(op0, X, sX, base, j, wave, lane, col);
        if (j + 2 < nspan)
            fold_load<D>(op0, base, j + 2, wave, lane, col);
        if (j + 1 >= nspan)
            break;
        fold_step<D>(op1, X, sX, base, j + 1, wave, lane, col);
        if (j + 3 < nspan)
            fold_load<D>(op1, base, j + 3, wave, lane, col);
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

template <int WB, int WW, int WG, bool PRO, typename E, int D, int C>
hipError_t launch_prep(const PrepArgs& pa, int64_t grid, hipStream_t stream)
{
    typedef PrepShape<E, D, C> PS;
    // more than 64 KiB of dynamic LDS: requested once per variant and device
    // (the attribute belongs to the device current at the call)
    static int done[64] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || !done[dev]) {
        const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&chunk_prep_kernel<WB, WW, WG, PRO, E, D, C>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)PS::SMEM);
        if (attr != hipSuccess)
            return attr;
        if (dev >= 0 && dev < 64)
            done[dev] = 1;
    }
    hipLaunchKernelGGL((chunk_prep_kernel<WB, WW, WG, PRO, E, D, C>), dim3((unsigned)grid), dim3(NTP), PS::SMEM,
                       stream, pa);
    return hipSuccess;
}

// Segments of the two-level scan.  One pass runs B*H*D/64 workgroups for NC
// chunk steps each; nseg segments run about twice the chunk steps in all but
// only ~2*NC/nseg in sequence, so they pay when the one pass fills less than
// a quarter of the CUs.  AUTO cuts the chunks into as many segments as one
// wave of state workgroups fills the CUs with (at least 4 chunks each);
// SEGMENTED always uses at least two.
struct SegPlan {
    int64_t nseg, len;
};

SegPlan seg_plan(const gdr2_fwd_args& a)
{
    SegPlan p;
    segment_plan(a.algo, ceil_div(a.T, a.chunk), a.B * a.H * (a.Dk / 64), &p.nseg, &p.len);
    return p;
}

template <typename E, int D, int C>
hipError_t launch_staged_t(const gdr2_fwd_args& a, hipStream_t stream)
{
    constexpr int BV = 64;
    typedef PrepShape<E, D, C> PS;
    typedef StateShape<E, D, C, BV> SS;
    const SegPlan sp = seg_plan(a);
    const Layout L = staged_layout(a.B, a.H, a.T, D, C, (int)sizeof(E), sp.nseg);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);

    PrepArgs pa;
    pa.q = a.q; pa.k = a.k; pa.v = a.v; pa.b = a.b; pa.w = a.w; pa.g = a.g;
    pa.bw = a.b_width; pa.ww = a.w_width; pa.gw = a.g_width; pa.pro = a.prologue;
    pa.B = a.B; pa.T = a.T; pa.H = a.H; pa.NC = ceil_div(a.T, C); pa.nrec = L.nrec;
    pa.Wn = ws + L.wn; pa.Ut = ws + L.ut; pa.Kh = ws + L.kh; pa.Qt = ws + L.qt; pa.P = ws + L.p;
    pa.gam = reinterpret_cast<float*>(ws + L.gam);

    if (a.stage != GDR2_STAGE_STATE) {
        const int64_t grid1 = std::min<int64_t>(L.nrec, (int64_t)cu_count());
        // one compile-time variant per gate-width mix; with the prologue, the
        // per-channel mix has its own variant and the others share the one
        // that reads the widths at run time
        const int code = (a.b_width == 1 ? 4 : 0) | (a.w_width == 1 ? 2 : 0) | (a.g_width == 1 ? 1 : 0);
        hipError_t e0 = hipSuccess;
        if (a.prologue != 0) {
            e0 = code == 0 ? launch_prep<D, D, D, true, E, D, C>(pa, grid1, stream)
                           : launch_prep<0, 0, 0, true, E, D, C>(pa, grid1, stream);
        } else {
            switch (code) {
            case 0: e0 = launch_prep<D, D, D, false, E, D, C>(pa, grid1, stream); break;
            case 1: e0 = launch_prep<D, D, 1, false, E, D, C>(pa, grid1, stream); break;
            case 2: e0 = launch_prep<D, 1, D, false, E, D, C>(pa, grid1, stream); break;
            case 3: e0 = launch_prep<D, 1, 1, false, E, D, C>(pa, grid1, stream); break;
            case 4: e0 = launch_prep<1, D, D, false, E, D, C>(pa, grid1, stream); break;
            case 5: e0 = launch_prep<1, D, 1, false, E, D, C>(pa, grid1, stream); break;
            case 6: e0 = launch_prep<1, 1, D, false, E, D, C>(pa, grid1, stream); break;
            default: e0 = launch_prep<1, 1, 1, false, E, D, C>(pa, grid1, stream); break;
            }
        }
        if (e0 != hipSuccess)
            return e0;
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.stage == GDR2_STAGE_PREP)
            return e;
    }

    StateArgs sa;
    sa.Wn = pa.Wn; sa.Ut = pa.Ut; sa.Kh = pa.Kh; sa.Qt = pa.Qt; sa.P = pa.P; sa.gam = pa.gam;
    sa.S0 = a.S0; sa.S_out = a.S_out; sa.S_chunks = a.S_chunks; sa.o = a.o;
    sa.T = a.T; sa.H = a.H; sa.NC = pa.NC; sa.nbh = a.B * a.H;
    sa.nseg = sp.nseg; sa.seg_len = sp.len;
    sa.span = sp.nseg > 1 ? reinterpret_cast<float*>(ws + L.span) : nullptr;
    if (sp.nseg > 1) {
        const int64_t gs = ceil_div(sa.nbh * (sp.nseg - 1), 8) * 8 * 2 * SS::NS;
        hipLaunchKernelGGL((chunk_span_kernel<E, D, C, BV>), dim3((unsigned)gs), dim3(NT), 0, stream, sa);
        if (sp.nseg > 2)
            hipLaunchKernelGGL((span_fold_kernel<D>), dim3((unsigned)(ceil_div(sa.nbh, 8) * 8 * (D / 16))), dim3(256),
                               0, stream, sa.span, sa.nbh, sp.nseg);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return e;
    }
    const int64_t grid2 = ceil_div(sa.nbh * sp.nseg, 8) * 8 * SS::NS;
    hipLaunchKernelGGL((chunk_state_kernel<E, D, C, BV>), dim3((unsigned)grid2), dim3(NT), 0, stream, sa);
    return hipGetLastError();
}

}  // namespace

int device_cu_count() { return cu_count(); }

void segment_plan(int algo, int64_t NC, int64_t wgs, int64_t* nseg, int64_t* len)
{
    *nseg = 1;
    *len = NC;
    if (algo == GDR2_ALGO_STAGED || NC < 2 || wgs <= 0)
        return;
    const int64_t fill = (int64_t)cu_count() / wgs;
    int64_t n;
    if (algo == GDR2_ALGO_SEGMENTED) {
        n = std::max<int64_t>(2, std::min(fill, NC));
    } else {
        n = std::min(fill, NC / 4);
        if (n < 4)
            return;
    }
    *len = ceil_div(NC, n);
    *nseg = ceil_div(NC, *len);
}

hipError_t launch_span_fold(float* span, int64_t nbh, int64_t nseg, int D, hipStream_t stream)
{
    const unsigned grid = (unsigned)(ceil_div(nbh, 8) * 8 * (D / 16));
    if (D == 128)
        hipLaunchKernelGGL((span_fold_kernel<128>), dim3(grid), dim3(256), 0, stream, span, nbh, nseg);
    else
        hipLaunchKernelGGL((span_fold_kernel<64>), dim3(grid), dim3(256), 0, stream, span, nbh, nseg);
    return hipGetLastError();
}

size_t staged_workspace_bytes(const gdr2_fwd_args& a)
{
    if (a.B * a.H * a.T == 0)
        return 0;
    return staged_layout(a.B, a.H, a.T, (int)a.Dk, a.chunk, a.dtype == GDR2_BF16 ? 2 : 4, seg_plan(a).nseg).total;
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
