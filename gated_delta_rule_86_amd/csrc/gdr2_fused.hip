// gdr2_fused.hip -- the chunked forward of the Gated DeltaNet-2 recurrence
// as one kernel (page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트
// 분리": the update of section "Gated Delta Rule-2 업데이트 수식", in the
// fixed-size chunks and WY form of section "효율적 구현", whose kernels are
// fused).  The chunk form and the intra-chunk phases are those of
// gdr2_chunk_common.h.
//
// One workgroup of 8 waves per (sequence, head, 64 value columns) walks the
// chunks of its sequence in order.  Per chunk it forms the WY factors in LDS
// (every wave: cumulative decay, decay-referenced operands, M and P, the
// inverse of I + M, the K^T and -W fragments; the last 4 waves also the U~
// tiles of their 16 value columns, kept in registers) and then advances the
// fp32 state, held in the MFMA accumulators of those 4 waves:
//   Delta = U~ - W S,   O = Q~ S + P Delta,   S <- diag(gamma) S + K^T Delta.
// Nothing per chunk goes through HBM: the inputs are read once (the next
// chunk's rows are in flight during the current chunk) and o is written
// once.  The two column slices of a head recompute the same factors; they
// share an XCD (blockIdx % 8), so the second one's input reads hit its L2.
#include "gdr2_chunk_common.h"

#include <algorithm>

namespace gdr2 {
namespace {

struct FusedArgs : PrepIn {
    const float* S0;
    float* S_out;
    float* S_chunks;          // optional: the state at the start of every chunk
    void* o;
    int64_t nbh;
};

template <typename E, int D, int C>
struct FusedShape : PrepGeom<E, D, C> {
    typedef PrepGeom<E, D, C> G;
    typedef Frags<E, D, C> F;
    static constexpr int BV = 64;                            // value columns per workgroup
    static constexpr int NSL = D / BV;                       // workgroups per (b, h)
    static constexpr int NSW = BV / 16;                      // state waves, one 16-column tile each
    static constexpr int W0 = NWP - NSW;                     // the first state wave
    static constexpr int LDO = 16 + G::VEC;                  // output staging rows (elements)
    static constexpr size_t SZ_U = al256((size_t)C * BV * G::ES);
    static constexpr size_t SZ_O = (size_t)NSW * C * LDO * G::ES;
    static constexpr size_t SZ_MT = G::SZ_M > G::SZ_TOT ? G::SZ_M : G::SZ_TOT;
    static constexpr bool O_ALIAS = SZ_O <= SZ_U + G::SZ_HALF;
    static constexpr size_t OFF_EH = 0;                                  // E^ [C][D]
    static constexpr size_t OFF_QH = OFF_EH + G::SZ_ROWS;                // Q^ [C][D] (rows < 32: Q~)
    static constexpr size_t OFF_KR = OFF_QH + G::SZ_ROWS;                // Kr [C][D]; then -W fragments
    static constexpr size_t OFF_U = OFF_KR + G::SZ_ROWS;                 // u [C][BV]; with E~: o staging
    static constexpr size_t OFF_E2 = OFF_U + SZ_U;                       // E~ second half
    static constexpr size_t OFF_Q2 = OFF_E2 + G::SZ_HALF;                // Q~ second half
    static constexpr size_t OFF_M = al256(OFF_Q2 + G::SZ_HALF);          // wave totals (A -> B), then M
    static constexpr size_t OFF_TOT = OFF_M;
    static constexpr size_t OFF_MD = al256(OFF_M + SZ_MT);               // M_II fp32
    static constexpr size_t OFF_XC = OFF_MD + G::SZ_MD;                  // X_II fp32
    static constexpr size_t OFF_X = al256(OFF_XC + G::SZ_MD);            // X [C][LDXP]
    static constexpr size_t OFF_P = al256(OFF_X + G::SZ_X);              // P fragments
    static constexpr size_t OFF_KT = OFF_P + F::P_BYTES;                 // K^T fragments
    static constexpr size_t OFF_FK = OFF_KT + F::K_BYTES;                // gamma [D], 2^(G_L - Gh) [D]
    static constexpr size_t OFF_RN = OFF_FK + G::SZ_FK;                  // prologue 1/|k|, 1/|q|
    static constexpr size_t OFF_FLAG = OFF_RN + G::SZ_RN;
    static constexpr size_t OFF_O = O_ALIAS ? OFF_U : al256(OFF_FLAG + 16);
    static constexpr size_t SMEM = O_ALIAS ? OFF_FLAG + 16 : OFF_O + SZ_O;
    static_assert(SMEM + G::SZ_G + 2 * C * 4 <= 160 * 1024, "LDS budget");
    static_assert(F::W_BYTES <= G::SZ_ROWS, "-W fragments fit the Kr rows");
    static_assert(D % BV == 0 && NSW <= NWP / 2, "value slices");
};

// The chunk n of (b, h).
__device__ __forceinline__ ChunkPos fused_pos(const FusedArgs& a, int64_t b, int64_t h, int64_t n, int C)
{
    const int64_t t0 = n * C;
    ChunkPos p;
    p.rec = 0;
    p.row0 = (b * a.T + t0) * a.H + h;
    p.L = (int)min((int64_t)C, a.T - t0);
    return p;
}

// One chunk of the state recurrence for one 16-column tile (col0 ..
// col0 + 15) from the factors in LDS: Delta = U~ - W S (U~ in ut, W stored
// negated), O = Q~ S + P Delta, S <- diag(gamma) S + K^T Delta; O leaves
// through the wave's staging rows with 16-byte stores.
template <typename E, int D, int C>
__device__ __forceinline__ void fused_state_step(const FusedArgs& a, const PrepLds<E, FusedShape<E, D, C>>& s, const unsigned char* sW,
                                                 const unsigned char* sKT, const unsigned char* sP, E* sOw,
                                                 f32x4* St, const f32x4* ut, const ChunkPos& cp, int col0, int lane)
{
    typedef FusedShape<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef typename MM::Frag Frag;
    constexpr int NB = S::NB, NH = S::NH, KT = F::KT, KB = F::KB, NKS = F::NKS, NKC = F::NKC, LDO = S::LDO;
    constexpr int KTS = D / 16;
    const int gq = lane >> 4, cl = lane & 15;
    auto frag = [&](const unsigned char* base, int i) -> Frag {
        return *reinterpret_cast<const Frag*>(base + i * F::FRAG + lane * 16);
    };
    // Q~ as an A fragment (rows 16 mt.., key channels KB ks..), read from
    // the operand rows in the accumulator k order
    auto qfrag = [&](int mt, int ks) -> Frag {
        const bool sec = NH == 2 && mt >= 2;
        const E* src = sec ? s.Q2() : s.Qh();
        const int r = sec ? 16 * mt - 32 + cl : 16 * mt + cl;
        if constexpr (sizeof(E) == 2) {
            const typename Mma16<E>::Frag lo = row4<E, D>(src, r, KB * ks + 4 * gq);
            const typename Mma16<E>::Frag hi = row4<E, D>(src, r, KB * ks + 16 + 4 * gq);
            Frag f;
            f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
            f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
            return f;
        } else {
            return row4<E, D>(src, r, KB * ks + 4 * gq);
        }
    };

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
                aw[mt][ks] = frag(sW, mt * NKS + ks);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
            dl[mt] = ut[mt];
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

    f32x4 ot[NB];
    {
        Frag aq[NB][NKS], ap[F::NP];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                aq[mt][ks] = qfrag(mt, ks);
#pragma unroll
        for (int i = 0; i < F::NP; ++i)
            ap[i] = frag(sP, i);
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
    }

    {
        Frag ak[KTS][NKC];
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                ak[kt][kc] = frag(sKT, kt * NKC + kc);
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
            St[kt] = St[kt] * *reinterpret_cast<const f32x4*>(s.Fk() + 16 * kt + 4 * gq);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int kt = 0; kt < KTS; ++kt)
                St[kt] = MM::mma(ak[kt][kc], DB[kc], St[kt]);
        sched_pipeline<KTS * NKC>();
    }

    // O: this wave's 16 columns through its staging rows, then 16-byte stores
#pragma unroll
    for (int mt = 0; mt < NB; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sOw[(16 * mt + 4 * gq + i) * LDO + cl] = from_f32<E>(ot[mt][i]);
    lds_fence_wave();
    constexpr int VEC = S::VEC, CPR = 16 / VEC;   // 16-byte pieces per staged row
    E* o = (E*)a.o;
#pragma unroll
    for (int e = lane; e < C * CPR; e += 64) {
        const int r = e / CPR, cg = e % CPR;
        if (r < cp.L)
            *reinterpret_cast<u32x4*>(o + (cp.row0 + (int64_t)r * a.H) * D + col0 + cg * VEC) =
                *reinterpret_cast<const u32x4*>(sOw + r * LDO + cg * VEC);
    }
}

// Gate widths WB, WW, WG: 1 or D fixed at compile time, 0 = read from the
// arguments (one variant serves every mix).
template <int WB, int WW, int WG, bool PRO, typename E, int D, int C>
__global__ __launch_bounds__(NTP) void chunk_fused_kernel(FusedArgs a)
{
    typedef FusedShape<E, D, C> S;
    typedef Frags<E, D, C> F;
    typedef Mma<E> MM;
    typedef Mma16<E> M16;
    constexpr int NB = S::NB, NH = S::NH, VEC = S::VEC, LDXP = S::LDXP, BV = S::BV, NSL = S::NSL;
    constexpr int NKS = F::NKS, NKC = F::NKC, NP = F::NP, KTS = D / 16;

    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ __align__(16) float sG[C * D];
    __shared__ __align__(16) unsigned int sBW[2 * C];   // width-1 b and w of the chunk
    PrepLds<E, S> s;
    s.G = sG;
    s.BW = sBW;
    unsigned char* sW = smem + S::OFF_KR;      // -W fragments over the Kr rows (after C2)
    unsigned char* sKT = smem + S::OFF_KT;
    unsigned char* sP = smem + S::OFF_P;

    // workgroup -> (b*H + h, value slice); the NSL slices of one (b, h)
    // compute the same factors from the same inputs: same blockIdx % 8, so
    // they run on one XCD and share its L2
    const int64_t bx = blockIdx.x;
    const int64_t grp = bx / (8 * NSL);
    const int within = (int)(bx % (8 * NSL));
    const int slice = within / 8;
    const int64_t bh = grp * 8 + within % 8;
    if (bh >= a.nbh)
        return;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    const int wave = threadIdx.x >> 6;
    const bool ab = wave < S::NWB;              // waves of phases A and B
    const bool second = NH == 2 && wave >= S::NWB / 2;
    const bool sw = wave >= S::W0;              // state waves
    const int tile = wave - S::W0;              // their 16-column tile
    const int col0 = slice * BV + 16 * tile;
    const int bw = WB ? WB : a.bw, ww = WW ? WW : a.ww;
    E* sOw = reinterpret_cast<E*>(smem + S::OFF_O) + (sw ? tile : 0) * C * S::LDO;

    // X: the blocks above the diagonal that fragments cover stay zero
    for (int e = threadIdx.x; e < C * LDXP; e += NTP)
        s.X()[e] = from_f32<E>(0.f);

    // the start state, this lane's column, 4 rows per accumulator tile
    f32x4 St[KTS];
    {
        const int lane = threadIdx.x & 63, gq = lane >> 4, cl = lane & 15;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
            St[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sw && a.S0) {
            const float* s0 = a.S0 + bh * D * D;
#pragma unroll
            for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    St[kt][i] = s0[(16 * kt + 4 * gq + i) * D + col0 + cl];
        }
    }

    // chunk 0's inputs: g and width-1 gates straight to LDS, tokens to R
    PrepRegs<E, D, C> R;
    {
        const int lane = threadIdx.x & 63;
        const ChunkPos cp0 = fused_pos(a, b, h, 0, C);
        const int t0 = wave * S::TW + (lane % S::LPC) * S::TPL, c0 = (lane / S::LPC) * VEC;
        prep_copy_g<WG, E, D, C>(a, cp0, reinterpret_cast<unsigned char*>(sG), wave, lane);
        prep_copy_bw<WB, WW, E, D, C>(a, cp0, sBW, wave, lane);
        if (ab) {
            prep_load<0, WB, WW>(a, cp0, R, t0, c0);
            prep_load<1, WB, WW>(a, cp0, R, t0, c0);
            prep_load<2, WB, WW>(a, cp0, R, t0, c0);
            prep_load<3, WB, WW>(a, cp0, R, t0, c0);
            prep_load<4, WB, WW>(a, cp0, R, t0, c0);
        }
    }

    for (int64_t n = 0; n < a.NC; ++n) {
        // Lane indices are rederived every chunk from an opaque copy of the
        // thread id, so the compiler does not keep every lane-dependent
        // address of the loop body live across iterations.
        int tid = threadIdx.x;
        __asm__ __volatile__("" : "+v"(tid));
        const int lane = tid & 63, gq = lane >> 4, cl = lane & 15;
        const int cgp = lane / S::LPC, lpc = lane % S::LPC;
        const int t0 = wave * S::TW + lpc * S::TPL, c0 = cgp * VEC;
        wait_copies();
        __syncthreads();   // B0: this chunk's g rows are in LDS, its tokens in R; the last chunk is done
        const ChunkPos cp = fused_pos(a, b, h, n, C);
        const bool more = n + 1 < a.NC;
        const ChunkPos np = fused_pos(a, b, h, more ? n + 1 : n, C);
        const typename M16::Frag ident = identity16<E>(gq, cl);

        // ---- A: cumulative log2-decay in registers -------------------------
        float G[S::TPL][VEC];
        float excl[VEC];
        if (ab)
            prep_cumsum<WG, PRO, E, D, C>(a, s, cp.L, t0, c0, lpc, wave, G, excl);
        if (tid == 0)
            *s.Flag() = 0;
        lds_barrier();   // B1: wave totals

        // ---- B: decay-referenced operands; the next chunk's tokens ---------
        if (ab) {
            prep_offsets_operands<PRO, BV, E, D, C>(a, R, s, cp.L, t0, c0, lpc, wave, second, G, excl, nullptr,
                                                    slice * BV, bw, ww);
            if (more) {
                prep_load<0, WB, WW>(a, np, R, t0, c0);
                prep_load<1, WB, WW>(a, np, R, t0, c0);
                prep_load<2, WB, WW>(a, np, R, t0, c0);
                prep_load<3, WB, WW>(a, np, R, t0, c0);
                prep_load<4, WB, WW>(a, np, R, t0, c0);
            }
        }
        lds_barrier();   // B2: operands in LDS
        if (more)        // phase B has read this chunk's width-1 gates
            prep_copy_bw<WB, WW, E, D, C>(a, np, sBW, wave, lane);
        const bool guard = *s.Flag() != 0;
        if (!guard) {
            if (more)
                prep_copy_g<WG, E, D, C>(a, np, reinterpret_cast<unsigned char*>(sG), wave, lane);
            // ---- C1: M tiles (waves 0-3) and P fragments (waves 4-7) -------
            prep_gram<E, D, C>(s, sP, wave, lane);
        } else {
            // ---- exact path for a chunk with steep decay -------------------
            prep_exact<PRO, E, D, C>(a, cp, s, sP, ab, t0, c0, bw, G);
            if (more)
                prep_copy_g<WG, E, D, C>(a, np, reinterpret_cast<unsigned char*>(sG), wave, lane);
        }
        lds_barrier();   // B3: M and P in LDS

        // ---- C2: X = (I + M)^-1 (wave 0); K^T fragments (others) ----------
        if (wave == 0) {
            prep_inverse<E, D, C>(s, lane);
        } else {
            constexpr int NK = (D / 16) * NKC;
            for (int task = wave - 1; task < NK; task += NWP - 1)
                sts16(sKT + task * F::FRAG + lane * 16, prep_kt_frag<E, D, C>(s, task / NKC, task % NKC, guard, ident, lane));
        }
        lds_barrier();   // B4: X and K^T in LDS; the Kr rows are free

        // ---- D: -W fragments (waves 0-3) into LDS ------------------------
        if (wave < NWP / 2) {
            typename MM::Frag xf[NP];
            prep_x_frags<E, D, C>(s, xf, lane);
            for (int m2 = wave; m2 < NKS; m2 += NWP / 2)
                prep_w<E, D, C>(s, xf, m2, sW, ident, lane);
        }
        lds_barrier();   // B5: -W in LDS

        // ---- the state recurrence over this chunk (waves 4-7): U~ = X u for
        // the wave's 16 columns (X stays in LDS until the next chunk's C2),
        // then the state step
        if (sw) {
            f32x4 ut[NB];
            {
                typename MM::Frag xf[NP];
                prep_x_frags<E, D, C>(s, xf, lane);
                prep_u_tile<BV, E, D, C>(s, xf, tile, ut, ident, lane);
            }
            if (a.S_chunks) {
                float* dst = a.S_chunks + (bh * a.NC + n) * D * D;
#pragma unroll
                for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[(16 * kt + 4 * gq + i) * D + col0 + cl] = St[kt][i];
            }
            fused_state_step<E, D, C>(a, s, sW, sKT, sP, sOw, St, ut, cp, col0, lane);
        }
    }

    if (sw && a.S_out) {
        const int lane = threadIdx.x & 63, gq = lane >> 4, cl = lane & 15;
        float* so = a.S_out + bh * D * D;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[(16 * kt + 4 * gq + i) * D + col0 + cl] = St[kt][i];
    }
}

template <int WB, int WW, int WG, bool PRO, typename E, int D, int C>
hipError_t launch_fused_v(const FusedArgs& fa, int64_t grid, hipStream_t stream)
{
    typedef FusedShape<E, D, C> FS;
    // more than 64 KiB of dynamic LDS: requested once per variant and device
    static int done[64] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || !done[dev]) {
        const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&chunk_fused_kernel<WB, WW, WG, PRO, E, D, C>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)FS::SMEM);
        if (attr != hipSuccess)
            return attr;
        if (dev >= 0 && dev < 64)
            done[dev] = 1;
    }
    hipLaunchKernelGGL((chunk_fused_kernel<WB, WW, WG, PRO, E, D, C>), dim3((unsigned)grid), dim3(NTP), FS::SMEM,
                       stream, fa);
    return hipGetLastError();
}

template <typename E, int D, int C>
hipError_t launch_fused_t(const gdr2_fwd_args& a, hipStream_t stream)
{
    typedef FusedShape<E, D, C> FS;
    FusedArgs fa;
    fa.q = a.q; fa.k = a.k; fa.v = a.v; fa.b = a.b; fa.w = a.w; fa.g = a.g;
    fa.bw = a.b_width; fa.ww = a.w_width; fa.gw = a.g_width; fa.pro = a.prologue;
    fa.B = a.B; fa.T = a.T; fa.H = a.H; fa.NC = ceil_div(a.T, C);
    fa.S0 = a.S0; fa.S_out = a.S_out; fa.S_chunks = a.S_chunks; fa.o = a.o;
    fa.nbh = a.B * a.H;
    const int64_t grid = ceil_div(fa.nbh, 8) * 8 * FS::NSL;
    // one compile-time variant per gate-width mix; with the prologue, the
    // per-channel mix has its own variant and the others share the one that
    // reads the widths at run time
    const int code = (a.b_width == 1 ? 4 : 0) | (a.w_width == 1 ? 2 : 0) | (a.g_width == 1 ? 1 : 0);
    if (a.prologue != 0)
        return code == 0 ? launch_fused_v<D, D, D, true, E, D, C>(fa, grid, stream)
                         : launch_fused_v<0, 0, 0, true, E, D, C>(fa, grid, stream);
    switch (code) {
    case 0: return launch_fused_v<D, D, D, false, E, D, C>(fa, grid, stream);
    case 1: return launch_fused_v<D, D, 1, false, E, D, C>(fa, grid, stream);
    case 2: return launch_fused_v<D, 1, D, false, E, D, C>(fa, grid, stream);
    case 3: return launch_fused_v<D, 1, 1, false, E, D, C>(fa, grid, stream);
    case 4: return launch_fused_v<1, D, D, false, E, D, C>(fa, grid, stream);
    case 5: return launch_fused_v<1, D, 1, false, E, D, C>(fa, grid, stream);
    case 6: return launch_fused_v<1, 1, D, false, E, D, C>(fa, grid, stream);
    default: return launch_fused_v<1, 1, 1, false, E, D, C>(fa, grid, stream);
    }
}

}  // namespace

bool fused_supported(const gdr2_fwd_args& a)
{
    return a.dtype == GDR2_BF16 && (a.Dk == 64 || a.Dk == 128) && (a.chunk == 32 || a.chunk == 64);
}

hipError_t launch_forward_fused(const gdr2_fwd_args& a, hipStream_t stream)
{
    const int D = (int)a.Dk, C = a.chunk;
    if (D == 128)
        return C == 64 ? launch_fused_t<bf16, 128, 64>(a, stream) : launch_fused_t<bf16, 128, 32>(a, stream);
    return C == 64 ? launch_fused_t<bf16, 64, 64>(a, stream) : launch_fused_t<bf16, 64, 32>(a, stream);
}

}  // namespace gdr2
