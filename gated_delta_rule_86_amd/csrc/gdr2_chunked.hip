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
#include "gdr2_chunk_common.h"

#include <algorithm>

namespace gdr2 {
namespace {

constexpr int NT = 256;            // threads of the state kernel (4 waves)

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


struct PrepArgs : PrepIn {
    int64_t nrec;
    void *Wn, *Ut, *Kh, *Qt, *P;
    float* gam;
};

struct StateArgs {
    const void *Wn, *Ut, *Kh, *Qt, *P;
    const float* gam;
    const float* S0;
    float* S_out;
    float* S_chunks;          // optional: the state at the start of every ck_every-th chunk
    void* o;
    int64_t T, H, NC, nbh;
    int ck_every;             // chunks per requested chunk (> 1: evaluated in smaller chunks)
    int64_t NCK;              // entries of S_chunks per (b, h): ceil(NC / ck_every)
    int64_t nseg, seg_len;    // chunk segments of the two-level scan (1, NC: one pass)
    float* span;              // segment area (nseg > 1)
};

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
template <typename E, int D, int C>
struct PrepShape : PrepGeom<E, D, C> {
    typedef PrepGeom<E, D, C> G;
    static constexpr size_t OFF_EH = 0;                                   // E^ [C][D]
    static constexpr size_t OFF_QH = OFF_EH + G::SZ_ROWS;                 // Q^ [C][D]
    static constexpr size_t OFF_KR = OFF_QH + G::SZ_ROWS;                 // Kr [C][D] (exact path: K^)
    static constexpr size_t OFF_U = OFF_KR + G::SZ_ROWS;                  // u  [C][D]
    static constexpr size_t OFF_E2 = OFF_U + G::SZ_ROWS;                  // E~ [C-32][D] second half
    static constexpr size_t OFF_Q2 = OFF_E2 + G::SZ_HALF;                 // Q~ [C-32][D] second half
    static constexpr size_t OFF_M = al256(OFF_Q2 + G::SZ_HALF);           // M [C][LDM], blocks below the diagonal
    static constexpr size_t OFF_MD = al256(OFF_M + G::SZ_M);              // M_II fp32 [NB][16][LDX]
    static constexpr size_t OFF_XC = OFF_MD + G::SZ_MD;                   // X_II fp32, column j as row j
    static constexpr size_t OFF_X = al256(OFF_XC + G::SZ_MD);             // X [C][LDXP] in fragment k order
    static constexpr size_t OFF_TOT = al256(OFF_X + G::SZ_X);             // wave totals [NWB][D]
    static constexpr size_t OFF_FK = OFF_TOT + G::SZ_TOT;                 // 2^(G_L - Gh) [NH][D]
    static constexpr size_t OFF_RN = OFF_FK + G::SZ_FK;                   // prologue: 1/|k|, 1/|q| [2][C]
    static constexpr size_t OFF_FLAG = OFF_RN + G::SZ_RN;
    static constexpr size_t SMEM = OFF_FLAG + 16;                         // dynamic LDS
    // raw g [C][D] (exact path: G) lives in its own static LDS object, so the
    // compiler knows the asynchronous copies into it touch nothing else
    static_assert(SMEM + G::SZ_G + 2 * C * 4 <= 160 * 1024, "LDS budget");   // + width-1 b, w
};

// Gate widths WB, WW, WG: 1 or D fixed at compile time, 0 = read from the
// arguments (one variant serves every mix).
template <int WB, int WW, int WG, bool PRO, typename E, int D, int C>
__global__ __launch_bounds__(NTP) void chunk_prep_kernel(PrepArgs a)
{
    typedef PrepShape<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef Mma16<E> M16;
    constexpr int NB = S::NB, NH = S::NH, VEC = S::VEC, LDXP = S::LDXP;
    constexpr int KB = F::KB, NKS = F::NKS, NKC = F::NKC, NP = F::NP;

    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ __align__(16) float sG[C * D];
    __shared__ __align__(16) unsigned int sBW[2 * C];   // width-1 b and w of the chunk
    PrepLds<E, S> s;
    s.G = sG;
    s.BW = sBW;

    const int wave = threadIdx.x >> 6;
    const bool ab = wave < S::NWB;              // waves of phases A and B
    const bool second = NH == 2 && wave >= S::NWB / 2;
    const int bw = WB ? WB : a.bw, ww = WW ? WW : a.ww;

    // X: the blocks above the diagonal that fragments cover stay zero
    for (int e = threadIdx.x; e < C * LDXP; e += NTP)
        s.X()[e] = from_f32<E>(0.f);

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
        const typename M16::Frag ident = identity16<E>(gq, cl);
        const int64_t rec = cp.rec;

        // ---- A: cumulative log2-decay in registers -------------------------
        float G[S::TPL][VEC];
        float excl[VEC];
        if (ab)
            prep_cumsum<WG, PRO, E, D, C>(a, s, cp.L, t0, c0, lpc, wave, G, excl);
        if (tid == 0)
            *s.Flag() = 0;
        lds_barrier();   // B1: wave totals; the previous chunk is done with LDS

        // ---- B: decay-referenced operands ----------------------------------
        if (ab) {
            prep_offsets_operands<PRO, D, E, D, C>(a, R, s, cp.L, t0, c0, lpc, wave, second, G, excl,
                                                   a.gam + rec * D, 0, bw, ww);
        }
        if (pre) {
            prep_load<2, WB, WW>(a, np, Rn, t0, c0);
            prep_load<3, WB, WW>(a, np, Rn, t0, c0);
        }
        lds_barrier();   // B2: operands in LDS
        if (next < a.nrec)   // phase B has read this chunk's width-1 gates
            prep_copy_bw<WB, WW, E, D, C>(a, np, sBW, wave, lane);

        unsigned char* gP = (unsigned char*)a.P + rec * F::P_BYTES;
        if (pre)
            prep_load<4, WB, WW>(a, np, Rn, t0, c0);
        const bool guard = __builtin_amdgcn_readfirstlane(*s.Flag()) != 0;   // wave-uniform
        if (!guard) {
            if (next < a.nrec)
                prep_copy_g<WG, E, D, C>(a, np, reinterpret_cast<unsigned char*>(sG), wave, lane);
            // ---- C1: M tiles (waves 0-3) and P fragments (waves 4-7) -------
            prep_gram<E, D, C>(s, gP, wave, lane);
        } else {
            // ---- exact path for a chunk with steep decay -------------------
            prep_exact<PRO, E, D, C>(a, cp, s, gP, ab, t0, c0, bw, G);
            if (next < a.nrec)
                prep_copy_g<WG, E, D, C>(a, np, reinterpret_cast<unsigned char*>(sG), wave, lane);
        }
        lds_barrier();   // B3: M in LDS

        // ---- C2: X = (I + M)^-1 (wave 0); K^T and Q~ fragments (others) --
        if (wave == 0) {
            prep_inverse<E, D, C>(s, lane);
        } else {
            constexpr int NK = (D / 16) * NKC, NQ = NB * NKS;
            unsigned char* gKh = (unsigned char*)a.Kh + rec * F::K_BYTES;
            unsigned char* gQt = (unsigned char*)a.Qt + rec * F::W_BYTES;
            for (int task = wave - 1; task < NK + NQ; task += NWP - 1) {
                if (task < NK) {
                    // K^T fragment (channel block c, token step m)
                    stg16(gKh + task * F::FRAG + lane * 16,
                          prep_kt_frag<E, D, C>(s, task / NKC, task % NKC, guard, ident, lane));
                } else {
                    // Q~ fragment (token block T, channel step m)
                    const int fq = task - NK, T = fq / NKS, m = fq % NKS;
                    const bool sec = NH == 2 && T >= 2;
                    const E* src = sec ? s.Q2() : s.Qh();
                    const int r = sec ? 16 * T - 32 + cl : 16 * T + cl;
                    u32x4 v;
                    if constexpr (sizeof(E) == 2) {
                        const u32x2 lo = __builtin_bit_cast(u32x2, row4<E, D>(src, r, KB * m + 4 * gq));
                        const u32x2 hi = __builtin_bit_cast(u32x2, row4<E, D>(src, r, KB * m + 16 + 4 * gq));
                        v = u32x4{lo[0], lo[1], hi[0], hi[1]};
                    } else {
                        v = __builtin_bit_cast(u32x4, row4<E, D>(src, r, KB * m + 4 * gq));
                    }
                    stg16(gQt + fq * F::FRAG + lane * 16, v);
                }
            }
        }
        lds_barrier();   // B4: X in LDS

        // ---- D: -W fragments (waves 0-3), U~ tiles (waves 4-7) ------------
        {
            typename MM::Frag xf[NP];
            prep_x_frags<E, D, C>(s, xf, lane);
            if (wave < NWP / 2) {
                unsigned char* gWn = (unsigned char*)a.Wn + rec * F::W_BYTES;
                for (int m2 = wave; m2 < NKS; m2 += NWP / 2)
                    prep_w<E, D, C>(s, xf, m2, gWn, ident, lane);
            } else {
                E* gUt = (E*)a.Ut + rec * (F::U_BYTES / sizeof(E));
                for (int n = wave - NWP / 2; n < D / 16; n += NWP / 2) {
                    f32x4 ut[NB];
                    prep_u_tile<D, E, D, C>(s, xf, n, ut, ident, lane);
#pragma unroll
                    for (int T = 0; T < NB; ++T) {
                        E* dst = gUt + (n * NB + T) * (F::TILE_U / sizeof(E)) + lane * 4;
                        *reinterpret_cast<typename Mma16<E>::Frag*>(dst) = M16::pack(ut[T]);
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
    static constexpr size_t U_SLICE = (size_t)NTU * NB * F::TILE_U;
    static constexpr size_t OFF_W = 0;                      // byte offsets in one buffer
    static constexpr size_t OFF_Q = OFF_W + F::W_BYTES;
    static constexpr size_t OFF_KT = OFF_Q + F::W_BYTES;
    static constexpr size_t OFF_P = OFF_KT + F::K_BYTES;
    static constexpr size_t OFF_U = OFF_P + F::P_BYTES;
    static constexpr size_t OFF_G = OFF_U + U_SLICE;        // gamma: D floats
    static constexpr size_t BUF = OFF_G + (size_t)D * 4;
    // double buffering when two buffers fit; else one
    static constexpr int NBUF = 2 * BUF <= 160 * 1024 ? 2 : 1;
    static constexpr size_t SMEM = NBUF * BUF;
    static_assert(BV == 16 * (NT / 64), "one 16-column tile per wave");
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(U_SLICE % 1024 == 0, "U~ slice copies");
};

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

// Four output values of one lane (consecutive value columns of one token)
// in the output dtype: 8 bytes for bf16, 16 for fp32.
template <typename E> struct OQuad;
template <> struct OQuad<bf16> {
    typedef bf16x4 T;
    static __device__ __forceinline__ T pack(f32x4 v) { return T{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]}; }
};
template <> struct OQuad<float> {
    typedef f32x4 T;
    static __device__ __forceinline__ T pack(f32x4 v) { return v; }
};

template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_store_o(const StateArgs& a, const typename OQuad<E>::T* oq, int64_t b,
                                             int64_t h, int slice, int64_t n, int lane, int wave);

// The state at the start of chunk n (this lane's column, its 4 rows per
// tile) into the checkpoint output, when n starts a requested chunk.
template <int D>
__device__ __forceinline__ void state_emit(const StateArgs& a, const f32x4* St, int64_t bh, int64_t n,
                                           int gq, int col)
{
    constexpr int KTS = D / 16;
    if (n % a.ck_every)
        return;
    float* dst = a.S_chunks + (bh * a.NCK + n / a.ck_every) * D * D;
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[(16 * kt + 4 * gq + i) * D + col] = St[kt][i];
}

// One chunk from buffer `buf`: Delta = U~ - W S, O = Q~ S + P Delta,
// S <- diag(gamma) S + K^T Delta.  O is formed transposed (O^T = S^T Q~^T +
// Delta^T P^T: the same fragments with the MFMA operands swapped, since an
// A and a B fragment share one lane layout), so each lane ends with four
// consecutive value columns of one token; they stay in `oq` and are stored
// from registers during the next chunk.  No LDS is written here, so no
// write can wait behind the copy into the other buffer.
template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_compute(const StateArgs& a, const unsigned char* buf,
                                              typename OQuad<E>::T* oq, f32x4* St, int64_t b, int64_t h, int slice,
                                              int64_t n, bool store_prev, int lane, int wave)
{
    typedef StateShape<E, D, C, BV> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef typename MM::Frag Frag;
    constexpr int NB = S::NB, KT = F::KT, NKS = F::NKS, NKC = F::NKC;
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
        state_store_o<E, D, C, BV>(a, oq, b, h, slice, n - 1, lane, wave);

    // O^T = S^T Q~^T + Delta^T P^T  (P is lower triangular: only stored steps).
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
                ot[mt] = MM::mma(SB[ks], aq[mt][ks], ot[mt]);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int kc = 0; kc <= mt / KT; ++kc)
                ot[mt] = MM::mma(DB[kc], ap[F::p_offset(mt) + kc], ot[mt]);
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

    // O: kept in registers, written out during the next chunk.
#pragma unroll
    for (int mt = 0; mt < NB; ++mt)
        oq[mt] = OQuad<E>::pack(ot[mt]);
}

// The outputs of chunk n held in `oq` (tile mt: token 16 mt + lane % 16,
// value columns 4 (lane / 16) .. + 3 of this wave's 16); tokens past the end
// of a ragged last chunk are not stored.
template <typename E, int D, int C, int BV>
__device__ __forceinline__ void state_store_o(const StateArgs& a, const typename OQuad<E>::T* oq, int64_t b,
                                             int64_t h, int slice, int64_t n, int lane, int wave)
{
    constexpr int NB = C / 16;
    const int gq = lane >> 4, cl = lane & 15;
    const int64_t t0 = n * C;
    const int L = (int)min((int64_t)C, a.T - t0);
    E* o = (E*)a.o + ((b * a.T + t0 + cl) * a.H + h) * D + slice * BV + 16 * wave + 4 * gq;
    const int64_t tile = (int64_t)16 * a.H * D;    // 16 tokens
#pragma unroll
    for (int mt = 0; mt < NB; ++mt)
        if (16 * mt + cl < L)
            *reinterpret_cast<typename OQuad<E>::T*>(o + mt * tile) = oq[mt];
}

template <typename E, int D, int C, int BV>
__global__ __launch_bounds__(NT) void chunk_state_kernel(StateArgs a)
{
    typedef StateShape<E, D, C, BV> S;
    constexpr int KTS = D / 16;
    __shared__ __align__(16) unsigned char buf0[S::BUF];
    __shared__ __align__(16) unsigned char buf1[S::NBUF == 2 ? S::BUF : 16];

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
    typename OQuad<E>::T oq[S::NB];                   // the previous chunk's outputs

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
            state_compute<E, D, C, BV>(a, buf0, oq, St, b, h, slice, n, n > n0, lane, wave);
            if (n + 1 >= n1)
                break;
            wait_copies();
            __syncthreads();          // chunk n + 1 is in buf1; everyone is done with buf0
            if (n + 2 < n1)
                state_fetch<E, D, C, BV>(a, rec0 + n + 2, slice, buf0, wave, lane);
            if (a.S_chunks)
                state_emit<D>(a, St, bh, n + 1, gq, col);
            state_compute<E, D, C, BV>(a, buf1, oq, St, b, h, slice, n + 1, true, lane, wave);
        }
    } else {
        for (int64_t n = n0; n < n1; ++n) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0
            if (a.S_chunks)
                state_emit<D>(a, St, bh, n, gq, col);
            state_compute<E, D, C, BV>(a, buf0, oq, St, b, h, slice, n, n > n0, lane, wave);
            __syncthreads();          // everyone is done with buf0
            if (n + 1 < n1)
                state_fetch<E, D, C, BV>(a, rec0 + n + 1, slice, buf0, wave, lane);
        }
    }

    state_store_o<E, D, C, BV>(a, oq, b, h, slice, n1 - 1, lane, wave);

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

// The chunk size the staged kernels evaluate in.  fp32 chunks of 64 tokens
// at d = 128 do not fit the prep kernel's LDS; since the chunked form is
// exact for every chunk size, they are evaluated as chunks of 32 (the
// requested chunk only fixes where S_chunks samples the state).
int eval_chunk(const gdr2_fwd_args& a)
{
    return (a.dtype == GDR2_F32 && a.Dk * a.chunk > 4096) ? 32 : a.chunk;
}

SegPlan seg_plan(const gdr2_fwd_args& a)
{
    SegPlan p;
    segment_plan(a.algo, ceil_div(a.T, eval_chunk(a)), a.B * a.H * (a.Dk / 64), &p.nseg, &p.len);
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
    sa.ck_every = a.chunk / C;
    sa.NCK = ceil_div(a.T, a.chunk);
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

// AUTO takes the fused kernel where it has no repeated work and fills the
// GPU: d = 64 (one workgroup per (sequence, head) covers every value column)
// with at least as many (sequence, head) pairs as compute units.  At d = 128
// each head's two value-column workgroups would both form the chunk's
// factors, which are compute-bound, and the staged kernels are faster
// (training shape: 0.46 against 0.63 ms); with fewer pairs than compute units
// the staged prep's parallelism over chunks wins.
int forward_algo(const gdr2_fwd_args& a)
{
    if (a.algo == GDR2_ALGO_FUSED)
        return GDR2_ALGO_FUSED;
    if (a.algo == GDR2_ALGO_AUTO && a.stage == GDR2_STAGE_ALL && fused_supported(a) && a.Dk == 64 &&
        a.B * a.H >= (int64_t)cu_count() && seg_plan(a).nseg == 1)
        return GDR2_ALGO_FUSED;
    return GDR2_ALGO_STAGED;
}

size_t staged_workspace_bytes(const gdr2_fwd_args& a)
{
    if (a.B * a.H * a.T == 0 || forward_algo(a) == GDR2_ALGO_FUSED)
        return 0;
    return staged_layout(a.B, a.H, a.T, (int)a.Dk, eval_chunk(a), a.dtype == GDR2_BF16 ? 2 : 4, seg_plan(a).nseg).total;
}

hipError_t launch_forward_staged(const gdr2_fwd_args& a, hipStream_t stream)
{
    const int D = (int)a.Dk, C = a.chunk;
    if (a.dtype == GDR2_BF16) {
        if (D == 128)
            return C == 64 ? launch_staged_t<bf16, 128, 64>(a, stream) : launch_staged_t<bf16, 128, 32>(a, stream);
        return C == 64 ? launch_staged_t<bf16, 64, 64>(a, stream) : launch_staged_t<bf16, 64, 32>(a, stream);
    }
    if (D == 128)   // chunk 64 is evaluated as chunks of 32 (eval_chunk)
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
