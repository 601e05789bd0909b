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
// Kernels (fp32 accumulation; with bf16 inputs the matrix-core operands are
// bf16, as in the forward; intermediates in a workspace of one record per
// (sequence, head, chunk)):
//   bwd_prep   persistent, one workgroup per CU, a chunk record at a time
//              (the next record's input rows in flight): G, U, E~, gamma; M
//              and P as 16x16 blocks through block-referenced rows (fp32
//              MFMA; bf16 inputs: three-pass bf16 products); X by blocks; W,
//              U~ likewise; and the scan's K^, P^T, Q~^T, -W^T operands in
//              MFMA fragment order.
//   bwd_dout   (fp32 inputs) dO rows of every chunk into the workspace (zero
//              past T); the other kernels read dO from the input.
//   bwd_frag   (fp32 inputs) the scan's dO^T fragments; with bf16 inputs the
//              scan copies the dO rows itself.
//   bwd_span   (few sequences x heads, many chunks) per chunk segment: the
//              segment's transition product and local gradient, for the
//              two-level reverse scan.
//   bwd_scan   per (sequence, head, chunk segment, 64 value columns): the
//              state gradient through the chunks in reverse (columns evolve
//              independently), recording Lam at every chunk end and dDelta
//              (in the input dtype).
//   bwd_sgrad  the state products per chunk.  bf16 inputs: persistent, every
//              operand read once and staged in LDS in bf16, Delta kept on
//              chip, then dM (the WY-factor product through dX and T1, also
//              on chip); fp32 inputs: chained 64x64 fp32 MFMA tiles through
//              memory.
//   bwd_xgrad  (fp32 inputs) the WY-factor products dU, dE~, dM as chained
//              tiles; bf16 inputs form dM in bwd_sgrad and dU, dE~ in
//              bwd_decay.
//   bwd_decay  per chunk and 32 channels: (bf16) dU and dE~ on its channels,
//              the decay-weighted sums, dG, dg and the input gradients.
//   bwd_gate_sum  width-1 gates: the channel groups' partial sums in order.
//   bwd_norm   the prologue's normalisation, backwards (when asked for).
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
    size_t G, U, Et, W, Ut, Del, dDel, dQt, dKh, dW, dU, dEt, dO;
    // [C][C] per record (X in the input dtype: bf16 inputs take it only as
    // a bf16 matrix-core operand after bwd_prep)
    size_t X, dP, dX, T1, dM;
    // [D] per record
    size_t gam;
    // [2][C] per record: prologue 1/|k|, 1/|q| of every token
    size_t RN;
    // [D][D] per record: state gradient at every chunk end, in the input
    // dtype (bf16 inputs: the precision of every product that takes it)
    size_t Lam;
    // scan operand fragments (ScanFrags), rec_bytes per record
    size_t SF;
    // two-level scan (nseg > 1): per (b,h) and segment but the first, a
    // chunk product and a local gradient, D x D fp32 each
    size_t span;
    // width-1 gates (narrow): per record, token and key-channel group of the
    // decay kernel, that group's partial sums of db, dw and dg
    // ([3][nrec*C][D/DC]); bwd_gate_sum adds the groups in order
    size_t GP;
    size_t total;
};

constexpr int DC = 32;                 // channels per decay workgroup

// fp32 inputs (wide) run the chained-tile state and WY-factor kernels
// through Delta, dU, dE~, dO, dX and the product T1 in memory; for bf16
// inputs the fused kernels keep them on chip (dU and dE~ are formed in
// bwd_decay) and those arrays are absent (their offsets are 0, never used).
BwdLayout bwd_layout(int64_t B, int64_t H, int64_t T, int D, size_t rec_bytes, int64_t nseg, bool narrow, bool wide)
{
    BwdLayout L;
    L.nrec = B * H * cdiv(T, BC);
    const size_t cd = a64((size_t)L.nrec * BC * D), cc = a64((size_t)L.nrec * BC * BC);
    const size_t dd = a64((size_t)L.nrec * D * D), d1 = a64((size_t)L.nrec * D);
    size_t o = 0;
    L.Del = L.dU = L.dEt = L.dO = L.dX = L.T1 = 0;
    size_t* cds[] = {&L.G, &L.U, &L.Et, &L.W, &L.Ut, &L.dDel, &L.dQt, &L.dKh, &L.dW, &L.Del, &L.dU, &L.dEt, &L.dO};
    for (int x = 0; x < (wide ? 13 : 9); ++x) {
        *cds[x] = o;
        o += cd;
    }
    L.X = o;                            // in the input dtype
    o += wide ? cc : a64((size_t)L.nrec * BC * BC / 2);
    size_t* ccs[] = {&L.dP, &L.dM, &L.dX, &L.T1};
    for (int x = 0; x < (wide ? 4 : 2); ++x) {
        *ccs[x] = o;
        o += cc;
    }
    L.gam = o;
    o += d1;
    L.RN = o;
    o += a64((size_t)L.nrec * 2 * BC);
    L.Lam = o;
    o += wide ? dd : a64((size_t)L.nrec * D * D / 2);
    L.SF = o;
    o += a64((size_t)L.nrec * rec_bytes / 4);
    L.span = o;
    if (nseg > 1)
        o += a64((size_t)(B * H) * (nseg - 1) * 2 * D * D);
    L.GP = o;
    if (narrow)
        o += a64((size_t)3 * L.nrec * BC * (D / DC));
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
    int pro;             // prologue bits
    int64_t T, H, NC, nrec, nbh;
    int64_t nseg, seg_len;   // chunk segments of the reverse scan (1, NC: one pass)
    float* ws;           // workspace base (fp32)
    BwdLayout L;
};

__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const bf16* p, int64_t i) { return (float)p[i]; }

struct Rec {
    int64_t bh, n, row0;   // row0: element row of token 0 of the chunk in [B,T,H,.]
    int L;
};

// Valid tokens of chunk n of a sequence.
__device__ __forceinline__ int chunk_len(const BwdArgs& a, int64_t n) { return (int)min((int64_t)BC, a.T - n * BC); }

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
    // dO^T (fp32 inputs only: with bf16 inputs the scan reads the dO rows
    // from the input and forms its fragments in LDS)
    static constexpr bool HAS_O = sizeof(E) == 4;
    static constexpr size_t OFF_K = 0, OFF_P = K_BYTES, OFF_Q = OFF_P + P_BYTES, OFF_W = OFF_Q + T_BYTES,
                            OFF_O = OFF_W + T_BYTES, REC = OFF_O + (HAS_O ? T_BYTES : 0);
    static constexpr int NFRAG = (int)(REC / FRAG);
    static_assert(K_BYTES == (size_t)BC * D * sizeof(E), "fragment size");
    static_assert(REC == (size_t)((HAS_O ? 4 : 3) * BC * D + BC * BC) * sizeof(E), "record size used for the workspace");
};

// Byte offset of element (row, k) in an array of such fragments whose
// 16-row blocks hold nk fragments each (KB k-values per fragment).  Four
// consecutive k from a multiple of 4 are contiguous.
template <typename E>
__device__ __forceinline__ size_t frag_at(int row, int k, int nk)
{
    constexpr int KB = Mma<E>::KB;
    const int f = (row >> 4) * nk + k / KB, lane = (row & 15) + 16 * ((k & 15) >> 2);
    const int j = (k & 3) + 4 * ((k % KB) >> 4);
    return (size_t)f * 1024 + (size_t)lane * 16 + (size_t)j * sizeof(E);
}

// ---------------------------------------------------------------------------
// bwd_prep: one workgroup (NTP threads) per chunk record at a time
// (persistent, one workgroup per CU).
//   1. raw rows into LDS, 4 channels per item; G = cumulative log-decay;
//      G, E~, gamma, U and the K^, Q~^T fragments written out
//   2. M (strictly lower) and P (lower) by 16x16 token blocks on fp32 MFMA,
//      through rows re-referenced to their block (every factor <= 1 below
//      the diagonal, <= e^kDiagSpan on it); steeper diagonal blocks pair by
//      pair, and every pair by its own exponential under growth
//   3. X = (I + M)^-1 by 16x16 blocks in one wave: diagonal blocks by
//      substitution (a column per lane), the rest by
//      X_ij = -X_ii sum_{k=j}^{i-1} M_ik X_kj on fp32 MFMA, one block diagonal
//      at a time; meanwhile the other waves stage E~ and U for step 4
//   4. W = X E~, U~ = X U as 16x16 fp32 MFMA tiles, one wave per tile
// ---------------------------------------------------------------------------
constexpr int NTP = 512;         // threads of the prep kernel
// Largest decay span (natural log units) over one 16-token block for which
// the pairs inside the block go through block-referenced rows: every factor
// then stays within e^{+-kDiagSpan}, far inside fp32's range.
constexpr float kDiagSpan = 60.f;

template <int D>
struct BwdPrepShape {
    static constexpr int C = BC, LD = D + 4, LDM = C + 4;
    static constexpr int OFF_G = 0, OFF_E = C * LD, OFF_K = 2 * C * LD, OFF_Q = 3 * C * LD, OFF_M = 4 * C * LD;
    static constexpr int OFF_CF = OFF_M + C * LDM;           // block-pair decay factors [10][D]
    static constexpr int FLOATS = OFF_CF + 10 * D;
    static constexpr size_t SMEM = (size_t)FLOATS * 4;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(C * LDM <= C * LD && 3 * 256 <= C * LD && C * C <= C * LD,
                  "X fits in the q area; the block products and the partial P in the k area");
};

// This wave's LDS accesses have completed (a wave-local LDS fence).
__device__ __forceinline__ void lds_fence_wave() { __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// s_barrier once this wave's LDS accesses have completed.  Unlike
// __syncthreads() it does not wait for the wave's outstanding global stores,
// so a workgroup that only exchanges data through LDS lets them drain.
__device__ __forceinline__ void lds_barrier() { __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup-wide OR of v through one LDS word per wave (slots[NW], used by
// one call site only), with lds_barrier.
template <int NW>
__device__ __forceinline__ int lds_barrier_or(int v, int* slots)
{
    const int any = __ballot(v) != 0;
    if ((threadIdx.x & 63) == 0)
        slots[threadIdx.x >> 6] = any;
    lds_barrier();
    int r = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        r |= slots[w];
    return r;
}

__device__ __forceinline__ f32x4 ld4s(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// An fp32 product on the bf16 matrix cores in three passes: every operand is
// split into a bf16 head and a bf16 tail (hi = x rounded to bf16, |x - hi| <=
// 2^-8 |x|; lo = x - hi rounded to bf16, off by at most 2^-16 |x|), and
// a b ~ lo_a hi_b + hi_a lo_b + hi_a hi_b, whose dropped term lo_a lo_b is at
// most 2^-16 of the product: errors of order 1e-5 relative, against 4e-3 for
// one bf16 pass, in far fewer cycles than the fp32 MFMA (three 16x16x32 bf16
// products against eight 16x16x4 fp32 ones per 32 k).
struct Split {
    Mma<bf16>::Frag hi, lo;
};
__device__ __forceinline__ Split bf_split(f32x4 a, f32x4 b)
{
    Split s;
    s.hi = Mma<bf16>::pack(a, b);
    f32x4 ra, rb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ra[j] = a[j] - (float)s.hi[j];
        rb[j] = b[j] - (float)s.hi[4 + j];
    }
    s.lo = Mma<bf16>::pack(ra, rb);
    return s;
}
__device__ __forceinline__ f32x4 mma3(const Split& a, const Split& b, f32x4 c)
{
    c = Mma<bf16>::mma(a.lo, b.hi, c);
    c = Mma<bf16>::mma(a.hi, b.lo, c);
    return Mma<bf16>::mma(a.hi, b.hi, c);
}
// The operands in Mma<bf16>'s fragment order from fp32 LDS: rows (lane % 16)
// at k = 4 (lane / 16).. and 16 + 4 (lane / 16).. (scaled elementwise along k
// by f[k], f -> k0, when f is given), or a k-major matrix's column lane % 16
// at those k.
__device__ __forceinline__ Split split_rows(const float* p, int ld, int lane, const float* f = nullptr)
{
    const int c = 4 * (lane >> 4);
    const float* s = p + (lane & 15) * ld + c;
    f32x4 a = ld4s(s), b = ld4s(s + 16);
    if (f) {
        a = a * ld4s(f + c);
        b = b * ld4s(f + c + 16);
    }
    return bf_split(a, b);
}
__device__ __forceinline__ Split split_kn(const float* p, int ld, int lane)
{
    const float* s = p + 4 * (lane >> 4) * ld + (lane & 15);
    return bf_split(f32x4{s[0], s[ld], s[2 * ld], s[3 * ld]}, f32x4{s[16 * ld], s[17 * ld], s[18 * ld], s[19 * ld]});
}


// Prologue activations (logistic sigmoid; log-decay -softplus(x) = log sigmoid(-x)).
__device__ __forceinline__ float bsigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float bneg_softplus(float x) { return -(fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)))); }
__device__ __forceinline__ f32x4 bsigm4(f32x4 x) { return f32x4{bsigm(x[0]), bsigm(x[1]), bsigm(x[2]), bsigm(x[3])}; }
constexpr float kNormEps = 1e-6f;
__device__ __forceinline__ void st4s(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Four consecutive channels of a gate of width 1 or D at element row `row`.
template <typename T>
__device__ __forceinline__ f32x4 gate4(const T* p, int width, int64_t row, int i)
{
    if (width == 1) {
        const float x = to_f32(p[row]);
        return f32x4{x, x, x, x};
    }
    return load4(p + row * (int64_t)width + i);
}

// Four consecutive elements in their storage type, converted at use.
template <typename T> struct Raw4;
template <> struct Raw4<float> {
    typedef f32x4 V;
    static __device__ __forceinline__ f32x4 cvt(V v) { return v; }
};
template <> struct Raw4<bf16> {
    typedef bf16x4 V;
    static __device__ __forceinline__ f32x4 cvt(V v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }
};
template <typename T>
__device__ __forceinline__ typename Raw4<T>::V ld_raw4(const T* p) { return *reinterpret_cast<const typename Raw4<T>::V*>(p); }
__device__ __forceinline__ f32x4 bcast4(float x) { return f32x4{x, x, x, x}; }

// bwd_prep step 1 for one gate-width mix (B1, W1, G1: b, w, g of width 1),
// in two parts so that a record's loads can be in flight while the
// previous record is processed.  prep_rows_load issues every load of this
// thread's items (token t, 4 channels) into `raw`; rows past the valid
// length re-read the last valid row.  prep_rows_use then writes the chunk's
// raw rows to LDS (G, k, q, e = b*k) and U = w*v to the workspace, zeroing
// rows past the valid length; e and u of every item stay in keepE, keepU
// for step 3.  It returns whether a valid log-decay is positive.
template <bool B1, bool W1, bool G1, typename E, int D>
struct PrepRaw {
    static constexpr int NIT = BC * (D / 4) / NTP;
    static_assert(BC * (D / 4) % NTP == 0, "whole items per thread");
    typename Raw4<E>::V rk[NIT], rq[NIT], rv[NIT], rb[NIT], rw[NIT];
    f32x4 rg[NIT];
    E sb[NIT], sw[NIT];
    float sg[NIT];
};

template <bool B1, bool W1, bool G1, typename E, int D>
__device__ __forceinline__ void prep_rows_load(const BwdArgs& a, const Rec& rc, int tid, PrepRaw<B1, W1, G1, E, D>& x)
{
    constexpr int Q4 = D / 4, NIT = PrepRaw<B1, W1, G1, E, D>::NIT;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* b = (const E*)a.b;
    const E* w = (const E*)a.w;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int e4 = tid + it * NTP, t = e4 / Q4, i = 4 * (e4 % Q4);
        const int64_t row = rc.row0 + (int64_t)min(t, rc.L - 1) * a.H;
        x.rk[it] = ld_raw4(k + row * D + i);
        x.rq[it] = ld_raw4(q + row * D + i);
        x.rv[it] = ld_raw4(v + row * D + i);
        if (B1)
            x.sb[it] = b[row];
        else
            x.rb[it] = ld_raw4(b + row * D + i);
        if (W1)
            x.sw[it] = w[row];
        else
            x.rw[it] = ld_raw4(w + row * D + i);
        if (G1)
            x.sg[it] = a.g[row];
        else
            x.rg[it] = load4(a.g + row * D + i);
    }
}

template <bool B1, bool W1, bool G1, typename E, int D>
__device__ __forceinline__ int prep_rows_use(const BwdArgs& a, const Rec& rc, int64_t r, int tid, float* sm,
                                             float* sRN, f32x4* keepE, f32x4* keepU, f32x4* keepK,
                                             const PrepRaw<B1, W1, G1, E, D>& x)
{
    typedef BwdPrepShape<D> PS;
    typedef Raw4<E> R;
    constexpr int C = BC, LD = PS::LD, Q4 = D / 4, NIT = PrepRaw<B1, W1, G1, E, D>::NIT;
    float* ws = a.ws;
    int growth = 0;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int e4 = tid + it * NTP, t = e4 / Q4, i = 4 * (e4 % Q4), l = t * LD + i;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 gv = G1 ? bcast4(x.sg[it]) : x.rg[it];
        f32x4 kv = R::cvt(x.rk[it]), qv = R::cvt(x.rq[it]);
        f32x4 bv = B1 ? bcast4(to_f32(x.sb[it])) : R::cvt(x.rb[it]);
        f32x4 wv = W1 ? bcast4(to_f32(x.sw[it])) : R::cvt(x.rw[it]);
        if (a.pro & GDR2_PROLOGUE_GATES) {
            bv = bsigm4(bv);
            wv = bsigm4(wv);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                gv[j] = bneg_softplus(gv[j]);
        }
        f32x4 ev = bv, uv = wv * R::cvt(x.rv[it]);
        if (t >= rc.L) {
            gv = zero;
            kv = zero;
            qv = zero;
            ev = zero;
            uv = zero;
        }
        growth |= (gv[0] > 0.f) | (gv[1] > 0.f) | (gv[2] > 0.f) | (gv[3] > 0.f);
        if (a.pro & GDR2_PROLOGUE_NORM_QK) {
            // unit L2 norm per token: the Q4 items of a row are Q4 consecutive lanes
            float sk = kv[0] * kv[0] + kv[1] * kv[1] + kv[2] * kv[2] + kv[3] * kv[3];
            float sq = qv[0] * qv[0] + qv[1] * qv[1] + qv[2] * qv[2] + qv[3] * qv[3];
#pragma unroll
            for (int m = 1; m < Q4; m <<= 1) {
                sk += __shfl_xor(sk, m);
                sq += __shfl_xor(sq, m);
            }
            const float rkn = rsqrtf(sk + kNormEps), rqn = rsqrtf(sq + kNormEps);
            kv = kv * rkn;
            qv = qv * rqn;
            if (i == 0) {
                ws[a.L.RN + (size_t)r * 2 * C + t] = rkn;
                ws[a.L.RN + (size_t)r * 2 * C + C + t] = rqn;
                sRN[t] = rkn;
            }
        }
        ev = ev * kv;
        st4s(sm + PS::OFF_G + l, gv);
        st4s(sm + PS::OFF_K + l, kv);
        st4s(sm + PS::OFF_Q + l, qv);
        st4s(sm + PS::OFF_E + l, ev);
        keepE[it] = ev;
        keepK[it] = kv;
        keepU[it] = uv;
    }
    return growth;
}

template <typename E, int D, int MIX>
__global__ __launch_bounds__(NTP) void bwd_prep_kernel(BwdArgs a)
{
    constexpr bool B1 = MIX & 4, W1 = MIX & 2, G1 = MIX & 1;   // gates of width 1
    typedef BwdPrepShape<D> PS;
    constexpr int C = BC, LD = PS::LD, LDM = PS::LDM, Q4 = D / 4;
    extern __shared__ __align__(16) float sm[];
    float* sG = sm + PS::OFF_G;     // [C][LD] cumulative log-decay (natural units)
    float* sE = sm + PS::OFF_E;     // [C][LD] e = b*k, later E~
    float* sK = sm + PS::OFF_K;     // [C][LD] k, later partial P, block products and u
    float* sQ = sm + PS::OFF_Q;     // [C][LD] q, later X [C][LDM]
    float* sM = sm + PS::OFF_M;     // [C][LDM] M
    __shared__ int sOr[2 * (NTP / 64)];
    __shared__ float sRN[2 * C];    // prologue: 1/|k|, 1/|q| per token
    float* ws = a.ws;
    typedef ScanFrags<E, D> SF;
    // persistent: records blockIdx.x, + gridDim.x, ... (the grid is at most
    // nrec), each record's input rows loaded while the previous record is
    // processed; barriers wait for LDS only, so a record's stores drain
    // during the next
    PrepRaw<B1, W1, G1, E, D> raw;
    prep_rows_load<B1, W1, G1, E, D>(a, rec_of(blockIdx.x, a.NC, a.T, a.H), threadIdx.x, raw);
    for (int64_t r = blockIdx.x; r < a.nrec; r += gridDim.x) {
        // the thread index, opaque to the compiler in each iteration: no
        // address derived from it is hoisted out of the loop to occupy a
        // register throughout
        int tid = threadIdx.x;
        __asm__ __volatile__("" : "+v"(tid));
        const Rec rc = rec_of(r, a.NC, a.T, a.H);
        const size_t cdo = (size_t)r * C * D, cco = (size_t)r * C * C;
        // the scan's operand fragments of this record (K^, P^T, Q~^T, -W^T; the
        // frag pass adds dO^T for fp32 inputs), in the input dtype
        unsigned char* sfr = reinterpret_cast<unsigned char*>(ws + a.L.SF) + (size_t)r * SF::REC;
        auto pT = [&](int s_, int t) -> E* {            // P^T[s][t] = P[t][s]
            return reinterpret_cast<E*>(sfr + SF::OFF_P + frag_at<E>(s_, t, SF::NKC));
        };

        // 1. raw rows (zero past the chunk's valid length), 4 channels per item,
        // once every wave is done with the previous record's LDS (the next
        // record's loads are issued in step 3)
        constexpr int NIT1 = C * Q4 / NTP;
        f32x4 keepE[NIT1], keepU[NIT1], keepK[NIT1];  // e = b k, u = w v and k of this thread's items, for step 3
        lds_barrier();
        int growth = prep_rows_use<B1, W1, G1, E, D>(a, rc, r, tid, sm, sRN, keepE, keepU, keepK, raw);
        growth = lds_barrier_or<NTP / 64>(growth, sOr);
        {
            // cumulative sum over the chunk per channel: thread (group gi, channel
            // i) scans its TPG consecutive tokens, then adds the earlier groups'
            // totals (through the M area, free until step 2)
            constexpr int NG = NTP / D, TPG = C / NG;
            static_assert(NTP % D == 0 && C % NG == 0, "whole token groups");
            const int i = tid % D, gi = tid / D;
            float* sTot = sM;
            float v[TPG];
#pragma unroll
            for (int m = 0; m < TPG; ++m)
                v[m] = sG[(gi * TPG + m) * LD + i];
#pragma unroll
            for (int m = 1; m < TPG; ++m)
                v[m] += v[m - 1];
            sTot[gi * D + i] = v[TPG - 1];
            lds_barrier();
            float off = 0.f;
            for (int g2 = 0; g2 < gi; ++g2)
                off += sTot[g2 * D + i];
#pragma unroll
            for (int m = 0; m < TPG; ++m)
                sG[(gi * TPG + m) * LD + i] = v[m] + off;
        }
        lds_barrier();
        // (G, E~, U, gamma and K^ are written in step 3, while one wave inverts)
        // Q~ = q e^G into the scan's Q~^T fragments (row = channel, k = token):
        // an item is one channel at 4 consecutive tokens, read from the raw
        // rows before step 2 re-references them
        for (int e = tid; e < D * (C / 4); e += NTP) {
            const int i = e % D, t0 = 4 * (e / D);
            f32x4 qv;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                qv[j] = sQ[(t0 + j) * LD + i] * __expf(sG[(t0 + j) * LD + i]);
            store4(reinterpret_cast<E*>(sfr + SF::OFF_Q + frag_at<E>(i, t0, SF::NKC)), qv);
        }

        // 2. M (strictly lower) and P (lower).
        if (!growth) {
            // Decays only.  The rows are re-referenced to their 16-token block in
            // place,  E^ = e e^{G - G_16T},  Q^ = q e^{G - G_16T},  K- = k e^{G_16T+15 - G},
            // so the block (T, S), S <= T, is  M_TS = (E^_T c_TS) K-_S^T  (and P
            // with Q^), c_TS = e^{G_16T - G_16S+15}: <= 1 below the diagonal,
            // e^{span of block T} on it.  A block whose span exceeds kDiagSpan in
            // some channel sends the diagonal blocks pair by pair (2a) instead.
            float* sCf = sm + PS::OFF_CF;
            int steep = 0;
            for (int e = tid; e < (C / 16) * D; e += NTP) {
                const int T = e / D, i = e % D;
                steep |= sG[16 * T * LD + i] - sG[(16 * T + 15) * LD + i] > kDiagSpan;
            }
            steep = lds_barrier_or<NTP / 64>(steep, sOr + NTP / 64);
            // 2a. (steep) the diagonal 16x16 blocks pair by pair, from the raw rows
            for (int e = steep ? tid : 4 * 136; e < 4 * 136; e += NTP) {
                const int blk = e / 136, pr = e % 136;
                int rr = 0;
                while ((rr + 1) * (rr + 2) / 2 <= pr)
                    ++rr;
                const int cc = pr - rr * (rr + 1) / 2, t = 16 * blk + rr, s_ = 16 * blk + cc;
                float m = 0.f, p = 0.f;
                for (int i = 0; i < D; ++i) {
                    const float f = __expf(sG[t * LD + i] - sG[s_ * LD + i]) * sK[s_ * LD + i];
                    m += sE[t * LD + i] * f;
                    p += sQ[t * LD + i] * f;
                }
                sM[t * LDM + s_] = cc < rr ? m : 0.f;
                *pT(s_, t) = from_f32<E>(p);
                if (cc < rr) {
                    sM[s_ * LDM + t] = 0.f;
                    *pT(t, s_) = from_f32<E>(0.f);
                }
            }
            lds_barrier();
            // 2b. re-referenced rows, and c_TS (pairs 0..5 below the diagonal in
            // the order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2); 6 + T on it)
            for (int e4 = tid; e4 < C * Q4; e4 += NTP) {
                const int t = e4 / Q4, i = 4 * (e4 % Q4), l = t * LD + i, T = t / 16;
                const f32x4 G = ld4s(sG + l), G0 = ld4s(sG + 16 * T * LD + i), G1 = ld4s(sG + (16 * T + 15) * LD + i);
                f32x4 fa, fb;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    fa[j] = __expf(G[j] - G0[j]);
                    fb[j] = __expf(G1[j] - G[j]);
                }
                st4s(sE + l, ld4s(sE + l) * fa);
                st4s(sQ + l, ld4s(sQ + l) * fa);
                st4s(sK + l, ld4s(sK + l) * fb);
            }
            for (int e = tid; e < 10 * D; e += NTP) {
                const int pi = e / D, i = e % D;
                const int T = pi < 1 ? 1 : pi < 3 ? 2 : pi < 6 ? 3 : pi - 6;
                const int S = pi < 6 ? pi - (T * (T - 1)) / 2 : T;
                sCf[e] = __expf(sG[16 * T * LD + i] - sG[(16 * S + 15) * LD + i]);
            }
            lds_barrier();
            // 2c. the block products in fp32 precision (fp32 MFMA for fp32
            // inputs; three-pass bf16 MFMA, mma3, for bf16 inputs), one wave per
            // block pair (M and P share the K- fragments); each wave also
            // clears the mirrored block above the diagonal
            {
                typedef Mma<float> MF;
                const int wave = tid >> 6, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
                for (int pi = wave; pi < (steep ? 6 : 10); pi += NTP / 64) {
                    const int T = pi < 1 ? 1 : pi < 3 ? 2 : pi < 6 ? 3 : pi - 6;
                    const int S = pi < 6 ? pi - (T * (T - 1)) / 2 : T;
                    const float* cf = sCf + pi * D;
                    f32x4 m = {0.f, 0.f, 0.f, 0.f}, p = m;
                    if constexpr (sizeof(E) == 2) {
#pragma unroll
                        for (int k0 = 0; k0 < D; k0 += Mma<bf16>::KB) {
                            const Split kb = split_rows(sK + 16 * S * LD + k0, LD, lane);
                            m = mma3(split_rows(sE + 16 * T * LD + k0, LD, lane, cf + k0), kb, m);
                            p = mma3(split_rows(sQ + 16 * T * LD + k0, LD, lane, cf + k0), kb, p);
                        }
                    } else {
#pragma unroll 4
                        for (int k0 = 0; k0 < D; k0 += MF::KB) {
                            const MF::Frag kb = MF::load(sK + 16 * S * LD + k0, LD, lane);
                            m = MF::mma(MF::load_scaled(sE + 16 * T * LD + k0, LD, cf + k0, lane), kb, m);
                            p = MF::mma(MF::load_scaled(sQ + 16 * T * LD + k0, LD, cf + k0, lane), kb, p);
                        }
                    }
                    f32x4 pv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * T + 4 * gq + i, s_ = 16 * S + cl;
                        sM[t * LDM + s_] = s_ < t ? m[i] : 0.f;
                        pv[i] = s_ <= t ? p[i] : 0.f;
                        if (S < T) {
                            const int ta = 16 * S + 4 * gq + i, sa = 16 * T + cl;   // the block (S, T)
                            sM[ta * LDM + sa] = 0.f;
                        }
                    }
                    // the accumulator column is a P^T fragment row: 4 consecutive tokens
                    store4(pT(16 * S + cl, 16 * T + 4 * gq), pv);
                    if (S < T)
                        store4(pT(16 * T + cl, 16 * S + 4 * gq), f32x4{0.f, 0.f, 0.f, 0.f});
                }
            }
            lds_barrier();
        } else {
            // Some log-decay > 0 (growth): factors could exceed 1, so every
            // pair takes its own exponential.  4x4 token blocks on and below the
            // diagonal; two threads (channel halves) per block.
            float m[4][4] = {}, p[4][4] = {};
            const int half = tid / 136, bid = tid % 136;
            int tb = 0;
            while ((tb + 1) * (tb + 2) / 2 <= bid)
                ++tb;
            const int sb = bid - tb * (tb + 1) / 2, t0 = 4 * tb, s0 = 4 * sb;
            if (tid < 272) {
                for (int i = half * (D / 2); i < (half + 1) * (D / 2); ++i) {
                    float gt[4], et[4], qt[4], gs[4], ks[4];
        #pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        gt[x] = sG[(t0 + x) * LD + i];
                        et[x] = sE[(t0 + x) * LD + i];
                        qt[x] = sQ[(t0 + x) * LD + i];
                        gs[x] = sG[(s0 + x) * LD + i];
                        ks[x] = sK[(s0 + x) * LD + i];
                    }
        #pragma unroll
                    for (int x = 0; x < 4; ++x)
        #pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            const float f = __expf(gt[x] - gs[y]) * ks[y];
                            m[x][y] += et[x] * f;
                            p[x][y] += qt[x] * f;
                        }
                }
            }
            lds_barrier();                  // q and k rows are no longer read
            float* sPp = sK;                  // [C][C] partial P of the second half
            if (tid >= 136 && tid < 272) {
        #pragma unroll
                for (int x = 0; x < 4; ++x)
        #pragma unroll
                    for (int y = 0; y < 4; ++y) {
                        sM[(t0 + x) * LDM + s0 + y] = m[x][y];
                        sPp[(t0 + x) * C + s0 + y] = p[x][y];
                    }
            }
            lds_barrier();
            if (tid < 136) {
                f32x4 pv[4];                  // pv[y][x] = P[t0 + x][s0 + y]
        #pragma unroll
                for (int x = 0; x < 4; ++x)
        #pragma unroll
                    for (int y = 0; y < 4; ++y) {
                        const int t = t0 + x, s_ = s0 + y;
                        const float mm = m[x][y] + sM[t * LDM + s_], pp = p[x][y] + sPp[t * C + s_];
                        sM[t * LDM + s_] = s_ < t ? mm : 0.f;
                        pv[y][x] = s_ <= t ? pp : 0.f;
                    }
        #pragma unroll
                for (int y = 0; y < 4; ++y)
                    store4(pT(s0 + y, t0), pv[y]);
                if (sb != tb) {               // the mirrored block above the diagonal is zero
        #pragma unroll
                    for (int x = 0; x < 4; ++x) {
        #pragma unroll
                        for (int y = 0; y < 4; ++y)
                            sM[(s0 + y) * LDM + t0 + x] = 0.f;
                        store4(pT(t0 + x, s0), f32x4{0.f, 0.f, 0.f, 0.f});
                    }
                }
            }
            lds_barrier();

        }

        // 3. X = (I + M)^-1 into the q area (wave 0), after every thread has
        // staged E~ = e e^G and u of its step-1 items for step 4 (the k and E
        // areas held re-referenced rows until now) and written G, E~, U,
        // gamma and K^ out: those stores drain while wave 0 inverts
        float* sX = sQ;
        float* sU = sK;
#pragma unroll
        for (int it = 0; it < NIT1; ++it) {
            const int e4 = tid + it * NTP, t = e4 / Q4, i = 4 * (e4 % Q4), l = t * LD + i;
            const size_t x = cdo + (size_t)t * D + i;
            const f32x4 G = ld4s(sG + l);
            f32x4 ev = keepE[it];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ev[j] *= __expf(G[j]);
            st4s(sE + l, ev);
            st4s(sU + l, keepU[it]);
            st4s(ws + a.L.G + x, G);
            store4(reinterpret_cast<E*>(ws + a.L.Et) + x, ev);
            store4(reinterpret_cast<E*>(ws + a.L.U) + x, keepU[it]);
            // K^ straight into the scan's fragments (row = token, k = channel)
            const f32x4 GL = ld4s(sG + (C - 1) * LD + i);
            f32x4 kd;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kd[j] = __expf(GL[j] - G[j]);
            store4(reinterpret_cast<E*>(sfr + SF::OFF_K + frag_at<E>(t, i, SF::NKS)), keepK[it] * kd);
            if (t == 0) {
                f32x4 gm;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    gm[j] = __expf(GL[j]);
                st4s(ws + a.L.gam + (size_t)r * D + i, gm);
            }
        }
        // the next record's input rows (the last record re-reads itself):
        // waves 1-7 issue theirs now, while wave 0 inverts, and wave 0 after;
        // at the start of the next record they would queue behind this one's
        // step-4 stores
        // (the wave test is made wave-uniform: as a per-lane test the two
        // branches run one after the other, and wave 0's inverse then waits
        // for registers the other branch's loads write)
        const Rec rnext = rec_of(std::min<int64_t>(r + gridDim.x, a.nrec - 1), a.NC, a.T, a.H);
        const bool w0 = __builtin_amdgcn_readfirstlane(tid) < 64;
        if (!w0)
            prep_rows_load<B1, W1, G1, E, D>(a, rnext, tid, raw);
        if (w0) {
            typedef Mma<float> MF;
            const int lane = tid, gq = lane >> 4, cl = lane & 15;
            {
                // column cl of the diagonal block X_gq,gq by forward substitution
                // (unit diagonal), then zeros for the blocks right of it
                const float* m = sM + 16 * gq * LDM + 16 * gq;
                float x[16];
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    // two interleaved partial sums: half the dependent chain
                    float acc0 = rr == cl ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
                    for (int c = 0; c + 1 < rr; c += 2) {
                        acc0 -= m[rr * LDM + c] * x[c];
                        acc1 -= m[rr * LDM + c + 1] * x[c + 1];
                    }
                    if (rr & 1)
                        acc0 -= m[rr * LDM + rr - 1] * x[rr - 1];
                    x[rr] = acc0 + acc1;
                }
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    sX[(16 * gq + rr) * LDM + 16 * gq + cl] = x[rr];
                    for (int J = gq + 1; J < C / 16; ++J)
                        sX[(16 * gq + rr) * LDM + 16 * J + cl] = 0.f;
                }
            }
            lds_fence_wave();
            // X_IJ = -X_II sum_{K=J}^{I-1} M_IK X_KJ, one block diagonal at a
            // time, the blocks held in registers: an accumulator tile (rows
            // 4 gq + i of column cl) is also the B operand of the next
            // products, so nothing goes through LDS until the end
            constexpr int NB = C / 16;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 Xt[NB][NB];
            MF::Frag xa[NB];                 // X_II as A operands
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                Xt[I][I] = MF::load_kn(sX + 16 * I * LDM + 16 * I, LDM, lane);
                xa[I] = MF::load(sX + 16 * I * LDM + 16 * I, LDM, lane);
            }
#pragma unroll
            for (int dg = 1; dg < NB; ++dg) {
#pragma unroll
                for (int I = dg; I < NB; ++I) {
                    const int J = I - dg;
                    f32x4 y = zero;
#pragma unroll
                    for (int K = J; K < I; ++K)
                        y = MF::mma(MF::load(sM + 16 * I * LDM + 16 * K, LDM, lane), Xt[K][J], y);
                    Xt[I][J] = -MF::mma(xa[I], MF::from_acc(&y), zero);
                }
            }
#pragma unroll
            for (int I = 1; I < NB; ++I)
#pragma unroll
                for (int J = 0; J < I; ++J)
#pragma unroll
                    for (int x4 = 0; x4 < 4; ++x4)
                        sX[(16 * I + 4 * gq + x4) * LDM + 16 * J + cl] = Xt[I][J][x4];
            prep_rows_load<B1, W1, G1, E, D>(a, rnext, tid, raw);
        }
        lds_barrier();
        for (int e4 = tid; e4 < C * C / 4; e4 += NTP) {
            const int t = e4 / (C / 4), c4 = 4 * (e4 % (C / 4));
            store4(reinterpret_cast<E*>(ws + a.L.X) + cco + (size_t)t * C + c4, ld4s(sX + t * LDM + c4));
        }

        // 4. W = X E~, U~ = X u
        {
            // 16x16 output tiles on fp32 MFMA, one wave per tile: A = rows of X
            // (lower triangular, so tile row T needs k-tiles 0..T), B = the
            // columns of E~ or u
            // Each tile goes out through a per-wave 16 x 20 LDS patch (in the
            // M area, free by now) as row pieces of 4, one vector store per lane.
            typedef Mma<float> MF;
            const int wave = tid >> 6, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
            constexpr int NTD = D / 16, NPER = (C / 16) * NTD, LP = 20;
            static_assert((NTP / 64) * 16 * LP <= C * LDM, "the patches fit in the M area");
            float* patch = sM + wave * 16 * LP;
            const int pr = lane >> 2, pc = 4 * (lane & 3);   // this lane's row piece of a tile
            // bf16 inputs: X's bf16 head and tail, split once for every tile
            // (the three-pass A operands), in the G area (free since step 3)
            constexpr int LXS = C + 4;    // rows of 136 bytes: 8-byte pieces stay aligned
            bf16* sXh = reinterpret_cast<bf16*>(sG);
            bf16* sXl = sXh + C * LXS;
            if constexpr (sizeof(E) == 2) {
                static_assert(2 * C * LXS * 2 <= C * LD * 4 && C * C / 8 % NTP == 0, "the split X fits the G area");
#pragma unroll
                for (int e = tid; e < C * C / 8; e += NTP) {
                    const int t = e / (C / 8), c8 = 8 * (e % (C / 8));
                    const Split sp = bf_split(ld4s(sX + t * LDM + c8), ld4s(sX + t * LDM + c8 + 4));
                    *reinterpret_cast<bf16x4*>(sXh + t * LXS + c8) = bf16x4{sp.hi[0], sp.hi[1], sp.hi[2], sp.hi[3]};
                    *reinterpret_cast<bf16x4*>(sXh + t * LXS + c8 + 4) = bf16x4{sp.hi[4], sp.hi[5], sp.hi[6], sp.hi[7]};
                    *reinterpret_cast<bf16x4*>(sXl + t * LXS + c8) = bf16x4{sp.lo[0], sp.lo[1], sp.lo[2], sp.lo[3]};
                    *reinterpret_cast<bf16x4*>(sXl + t * LXS + c8 + 4) = bf16x4{sp.lo[4], sp.lo[5], sp.lo[6], sp.lo[7]};
                }
                lds_barrier();
            }
            for (int tile = wave; tile < 2 * NPER; tile += NTP / 64) {
                const int which = tile / NPER, T = (tile % NPER) / NTD, c = tile % NTD;
                const float* src = which == 0 ? sE : sU;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (sizeof(E) == 2) {
                    // three-pass bf16 products, 32 tokens per step (X is zero
                    // above its diagonal)
                    for (int k0 = 0; k0 < 16 * (T + 1); k0 += Mma<bf16>::KB)
                        acc = mma3(Split{Mma<bf16>::load(sXh + 16 * T * LXS + k0, LXS, lane),
                                         Mma<bf16>::load(sXl + 16 * T * LXS + k0, LXS, lane)},
                                   split_kn(src + k0 * LD + 16 * c, LD, lane), acc);
                } else {
                    for (int kk = 0; kk <= T; ++kk)
                        acc = MF::mma(MF::load(sX + 16 * T * LDM + 16 * kk, LDM, lane),
                                      MF::load_kn(src + 16 * kk * LD + 16 * c, LD, lane), acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    patch[(4 * gq + i) * LP + cl] = acc[i];
                const f32x4 row4 = ld4s(patch + pr * LP + pc);
                const size_t o = cdo + (size_t)(16 * T + pr) * D + 16 * c + pc;
                if (which == 0) {
                    store4(reinterpret_cast<E*>(ws + a.L.W) + o, row4);
                    // and -W^T for the scan: the accumulator column is a fragment row
                    store4(reinterpret_cast<E*>(sfr + SF::OFF_W + frag_at<E>(16 * c + cl, 16 * T + 4 * gq, SF::NKC)), -acc);
                } else {
                    st4s(ws + a.L.Ut + o, row4);
                }
            }
        }
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


// Contraction index held in slot j (0 .. 16/sizeof(E)-1) by lane group gq.
template <typename E> __device__ __forceinline__ int slot_k(int gq, int j);
template <> __device__ __forceinline__ int slot_k<bf16>(int gq, int j) { return (j < 4 ? 0 : 12) + 4 * gq + j; }
template <> __device__ __forceinline__ int slot_k<float>(int gq, int j) { return 4 * gq + j; }

// fp32 inputs: one workgroup per chunk record: the dO^T fragments of the
// scan (rows = value columns, k = tokens), read from the input rows, zero
// past the valid length.  bwd_prep writes the record's other fragments.
// Item (fragment, lane) -> 16 bytes.  (bf16 inputs: the scan copies the dO
// rows itself, scan_fetch and o_frag.)
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_frag_kernel(BwdArgs a)
{
    typedef ScanFrags<E, D> F;
    constexpr int NV = 16 / (int)sizeof(E), NOF = F::DT * F::NKC;
    const int64_t r = blockIdx.x;
    const Rec rc = rec_of(r, a.NC, a.T, a.H);
    const E* dOin = (const E*)a.dO;
    unsigned char* out = reinterpret_cast<unsigned char*>(a.ws + a.L.SF) + (size_t)r * F::REC + F::OFF_O;
    for (int it = threadIdx.x; it < NOF * 64; it += NTB) {
        const int f = it / 64, lane = it % 64, gq = lane / 16;
        const int row = 16 * (f / F::NKC) + lane % 16, m = f % F::NKC;
        float x[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int t = m * F::KB + slot_k<E>(gq, j);
            x[j] = t < rc.L ? to_f32(dOin[(rc.row0 + (int64_t)min(t, rc.L - 1) * a.H) * D + row]) : 0.f;
        }
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
// and Lam (before the update) and dDelta go to the workspace in the input
// dtype (bf16 inputs: the precision in which every later product takes
// them; the fp32 accumulators carry on unrounded).  A chunk's fragments are
// copied global -> LDS with global_load_lds (no register staging), double
// buffered when two buffers fit; with bf16 inputs the dO rows of the
// workgroup's value columns are copied the same way, straight from the
// input, and the dO fragments are read out of them.
// ---------------------------------------------------------------------------
template <typename E, int D>
struct ScanShape {
    typedef ScanFrags<E, D> F;
    static constexpr int BV = 64, NS = D / BV;
    static constexpr size_t O_SLICE = (size_t)(BV / 16) * F::NKC * F::FRAG;
    static constexpr size_t OFF_O = F::OFF_O, OFF_G = OFF_O + O_SLICE, BUF = OFF_G + (size_t)D * 4;
    static constexpr int NBUF = 2 * BUF <= 160 * 1024 ? 2 : 1;
    static_assert(F::OFF_O % 1024 == 0 && O_SLICE % 1024 == 0, "whole fragments");
    // bf16: Lam and dDelta leave through workgroup patches in LDS ([D] and
    // [BC] rows of the BV columns, rows padded by 16 bytes) as 16-byte row
    // pieces, 2 BV bytes per row, instead of one 2-byte store per element
    static constexpr bool PATCH = sizeof(E) == 2;
    static constexpr int PLD = (int)sizeof(E) * BV + 16;
    static constexpr size_t PATCH_L = PATCH ? (size_t)D * PLD : 0, PATCH_D = PATCH ? (size_t)BC * PLD : 0;
    static_assert(!PATCH || (NBUF == 2 && 2 * BUF + PATCH_L + PATCH_D <= 160 * 1024), "LDS budget");
    static_assert(!PATCH || 2 * BV == 8 * 16, "eight 16-byte pieces per row");
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
    if constexpr (F::HAS_O) {
        copy_frags<S::O_SLICE>(rec + F::OFF_O + slice * S::O_SLICE, buf + S::OFF_O, wave, lane);
    } else {
        // the chunk's dO rows, columns BV*slice.., as [BC][BV] rows of 2*BV
        // bytes: instruction j copies rows 8j..8j+7 (lane: row 8j + lane/8,
        // bytes 16 (lane % 8)..); rows past the valid length re-read the last
        // valid row (o_frag zeroes those tokens)
        static_assert(2 * S::BV == 128 && S::O_SLICE == (size_t)BC * 2 * S::BV, "8 rows per 1 KB instruction");
        const Rec rc = rec_of(r, a.NC, a.T, a.H);
        const unsigned char* dO = reinterpret_cast<const unsigned char*>(a.dO) + (slice * S::BV + 8 * (lane & 7)) * sizeof(E);
#pragma unroll
        for (int j = wave; j < BC / 8; j += NTB / 64) {
            const int t = min(8 * j + (lane >> 3), rc.L - 1);
            __builtin_amdgcn_global_load_lds(dO + (rc.row0 + (int64_t)t * a.H) * D * sizeof(E),
                                             (lds_void*)(buf + S::OFF_O + j * 1024), 16, 0, 0);
        }
    }
    if (wave == NTB / 64 - 1 && lane < D / 4)
        __builtin_amdgcn_global_load_lds(a.ws + a.L.gam + (size_t)r * D + lane * 4, (lds_void*)(buf + S::OFF_G), 16,
                                         0, 0);
}

// The dO operand fragment kc (k = tokens KB kc.., n = the wave's 16 value
// columns) of a chunk in buf: fp32 inputs, as the frag pass stored it; bf16
// inputs, read out of the dO rows scan_fetch copied, zero at tokens >= L.
template <typename E, int D>
__device__ __forceinline__ typename Mma<E>::Frag o_frag(const unsigned char* buf, int kc, int wave, int lane, int L)
{
    typedef ScanShape<E, D> S;
    typedef ScanFrags<E, D> F;
    typedef typename Mma<E>::Frag Frag;
    if constexpr (F::HAS_O) {
        return *reinterpret_cast<const Frag*>(buf + S::OFF_O + (size_t)(wave * F::NKC + kc) * 1024 + lane * 16);
    } else {
        const E* sO = reinterpret_cast<const E*>(buf + S::OFF_O) + 16 * wave + (lane & 15);
        Frag f;
#pragma unroll
        for (int j = 0; j < 16 / (int)sizeof(E); ++j) {
            const int t = kc * F::KB + slot_k<E>(lane >> 4, j);
            f[j] = t < L ? sO[t * S::BV] : (E)0.f;
        }
        return f;
    }
}

// bf16: rows [nrows][BV] of the patch (written, then an lds_barrier) to
// memory at dst (row stride D elements), 16 bytes per lane and instruction.
template <typename E, int D, int NROWS>
__device__ __forceinline__ void patch_rows_out(const unsigned char* patch, E* dst, int tid)
{
    typedef ScanShape<E, D> S;
#pragma unroll
    for (int p = tid; p < NROWS * 8; p += NTB) {
        const int row = p >> 3, c = p & 7;
        *reinterpret_cast<uint4*>(dst + (size_t)row * D + 8 * c) =
            *reinterpret_cast<const uint4*>(patch + (size_t)row * S::PLD + 16 * c);
    }
}

template <typename E, int D>
__device__ __forceinline__ void scan_chunk(const BwdArgs& a, const unsigned char* buf, f32x4* lam, int64_t r,
                                           int col, int lane, int wave, int L, unsigned char* patch)
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
    E* lo = reinterpret_cast<E*>(a.ws + a.L.Lam) + (size_t)r * D * D;
    const int pc = 16 * wave + (lane & 15);    // the lane's column within the workgroup's BV
    if constexpr (S::PATCH) {
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<E*>(patch + (size_t)(16 * kt + 4 * gq + i) * S::PLD + 2 * pc) = from_f32<E>(lam[kt][i]);
        lds_barrier();
        patch_rows_out<E, D, D>(patch, lo + (col - pc), 64 * wave + lane);
    } else {
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lo[(16 * kt + 4 * gq + i) * D + col] = from_f32<E>(lam[kt][i]);
    }

    Frag LB[NKS], OB[NKC];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        LB[ks] = MM::from_acc(&lam[ks * KT]);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        OB[kc] = o_frag<E, D>(buf, kc, wave, lane, L);

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
    E* dq = reinterpret_cast<E*>(a.ws + a.L.dDel) + (size_t)r * BC * D;   // in the input dtype
    if constexpr (S::PATCH) {
        unsigned char* pd = patch + S::PATCH_L;
#pragma unroll
        for (int st = 0; st < NB; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<E*>(pd + (size_t)(16 * st + 4 * gq + i) * S::PLD + 2 * pc) = from_f32<E>(dd[st][i]);
        lds_barrier();
        patch_rows_out<E, D, BC>(pd, dq + (col - pc), 64 * wave + lane);
    } else {
#pragma unroll
        for (int st = 0; st < NB; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dq[(16 * st + 4 * gq + i) * D + col] = from_f32<E>(dd[st][i]);
    }

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
    __shared__ __align__(16) unsigned char patch[S::PATCH ? S::PATCH_L + S::PATCH_D : 16];
    // workgroup -> ((b,h), chunk segment, column slice); the slices of one
    // segment share blockIdx % 8, i.e. one XCD and its L2
    const int64_t bx = blockIdx.x, grp = bx / (8 * S::NS);
    const int within = (int)(bx % (8 * S::NS)), slice = within / 8;
    const int64_t unit = grp * 8 + within % 8;       // (b*H + h) * nseg + segment
    if (unit >= a.nbh * a.nseg)
        return;
    const int64_t bh = unit / a.nseg, seg = unit - bh * a.nseg;
    const int64_t n0 = seg * a.seg_len, n1 = min(a.NC, n0 + a.seg_len);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4;
    const int col = slice * S::BV + 16 * wave + (lane & 15);
    const int64_t rec0 = bh * a.NC;

    // the gradient at the segment's end: dS_final (or zero) for the last
    // segment, else what the segment fold left for it (the null test
    // outside the loads, so that they are all in flight at once)
    // (with segments, the last one starts from the span pass's copy of
    // dS_final, as dS0 may be dS_final)
    const float* l0 = seg < a.nseg - 1 ? a.ws + a.L.span + ((bh * (a.nseg - 1) + (a.nseg - 2 - seg)) * 2 + 1) * D * D
                      : !a.dS_final    ? nullptr
                      : a.nseg > 1     ? a.ws + a.L.span + bh * (a.nseg - 1) * 2 * D * D
                                       : a.dS_final + bh * D * D;
    f32x4 lam[DT];
    if (l0) {
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lam[kt][i] = l0[(16 * kt + 4 * gq + i) * D + col];
    } else {
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
            lam[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    scan_fetch<E, D>(a, rec0 + n1 - 1, slice, buf0, wave, lane);
    if constexpr (S::NBUF == 2) {
        for (int64_t n = n1 - 1; n >= n0; n -= 2) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0; everyone is done with buf1
            if (n - 1 >= n0)
                scan_fetch<E, D>(a, rec0 + n - 1, slice, buf1, wave, lane);
            scan_chunk<E, D>(a, buf0, lam, rec0 + n, col, lane, wave, chunk_len(a, n), patch);
            if (n == n0)
                break;
            wait_copies();
            __syncthreads();          // chunk n - 1 is in buf1; everyone is done with buf0
            if (n - 2 >= n0)
                scan_fetch<E, D>(a, rec0 + n - 2, slice, buf0, wave, lane);
            scan_chunk<E, D>(a, buf1, lam, rec0 + n - 1, col, lane, wave, chunk_len(a, n - 1), patch);
        }
    } else {
        for (int64_t n = n1 - 1; n >= n0; --n) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0
            scan_chunk<E, D>(a, buf0, lam, rec0 + n, col, lane, wave, chunk_len(a, n), patch);
            __syncthreads();          // everyone is done with buf0
            if (n - 1 >= n0)
                scan_fetch<E, D>(a, rec0 + n - 1, slice, buf0, wave, lane);
        }
    }
    if (a.dS0 && seg == 0) {
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.dS0[(bh * D + 16 * kt + 4 * gq + i) * D + col] = lam[kt][i];
    }
}

// ---------------------------------------------------------------------------
// Two-level reverse scan, the mirror of the forward's: in reverse the chunk
// step is affine in the gradient,
//   Lam_prev = (diag(gamma) - W^T K^) Lam + (Q~^T - W^T P^T) dO,
// and the chunks are cut into nseg segments of seg_len chunks.
// bwd_span_kernel runs every segment but the first, in parallel, from its
// end: the product of its chunks' transitions (carried from the identity as
// D more columns) and its local gradient (from zero; the last segment from
// dS_final, so that one is the true gradient at its start).  Entry e holds
// segment nseg-1-e, so the segment fold (X = L_0, X <- Pi_e X + L_e) leaves
// in the local half of entry e the gradient at the end of segment nseg-2-e,
// where bwd_scan_kernel starts that segment.
// ---------------------------------------------------------------------------
template <bool LOCAL, typename E, int D>
__device__ __forceinline__ void span_scan_chunk(const unsigned char* buf, f32x4* lam, int lane, int wave, int L)
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

    Frag LB[NKS], OB[NKC];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        LB[ks] = MM::from_acc(&lam[ks * KT]);
    if (LOCAL) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            OB[kc] = o_frag<E, D>(buf, kc, wave, lane, L);
    }
    // dDelta = K^ X (+ P^T dO for the local columns)
    f32x4 dd[NB];
#pragma unroll
    for (int st = 0; st < NB; ++st)
        dd[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int st = 0; st < NB; ++st)
            dd[st] = MM::mma(frag(F::OFF_K, st * NKS + ks), LB[ks], dd[st]);
    if (LOCAL) {
#pragma unroll
        for (int st = 0; st < NB; ++st)
#pragma unroll
            for (int kc = st / KT; kc < NKC; ++kc)
                dd[st] = MM::mma(frag(F::OFF_P, st * NKC + kc), OB[kc], dd[st]);
    }
    // X <- diag(gamma) X (+ Q~^T dO) - W^T dDelta
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
            if (LOCAL)
                lam[kt] = MM::mma(frag(F::OFF_Q, kt * NKC + kc), OB[kc], lam[kt]);
            lam[kt] = MM::mma(frag(F::OFF_W, kt * NKC + kc), DB[kc], lam[kt]);
        }
}

template <bool LOCAL, typename E, int D>
__device__ __forceinline__ void span_scan_run(const BwdArgs& a, unsigned char* buf0, unsigned char* buf1, f32x4* lam,
                                              int64_t rec0, int64_t n0, int64_t n1, int slice, int lane, int wave)
{
    typedef ScanShape<E, D> S;
    scan_fetch<E, D>(a, rec0 + n1 - 1, slice, buf0, wave, lane);
    if constexpr (S::NBUF == 2) {
        for (int64_t n = n1 - 1; n >= n0; n -= 2) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0; everyone is done with buf1
            if (n - 1 >= n0)
                scan_fetch<E, D>(a, rec0 + n - 1, slice, buf1, wave, lane);
            span_scan_chunk<LOCAL, E, D>(buf0, lam, lane, wave, chunk_len(a, n));
            if (n == n0)
                break;
            wait_copies();
            __syncthreads();          // chunk n - 1 is in buf1; everyone is done with buf0
            if (n - 2 >= n0)
                scan_fetch<E, D>(a, rec0 + n - 2, slice, buf0, wave, lane);
            span_scan_chunk<LOCAL, E, D>(buf1, lam, lane, wave, chunk_len(a, n - 1));
        }
    } else {
        for (int64_t n = n1 - 1; n >= n0; --n) {
            wait_copies();
            __syncthreads();          // chunk n is in buf0
            span_scan_chunk<LOCAL, E, D>(buf0, lam, lane, wave, chunk_len(a, n));
            __syncthreads();          // everyone is done with buf0
            if (n - 1 >= n0)
                scan_fetch<E, D>(a, rec0 + n - 1, slice, buf0, wave, lane);
        }
    }
}

// Workgroup -> ((b,h), entry e < nseg - 1, column slice): slices 0 .. NS-1
// carry the product's columns, NS .. 2NS-1 the local gradient's.
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_span_kernel(BwdArgs a)
{
    typedef ScanShape<E, D> S;
    constexpr int DT = D / 16, NS = S::NS;
    __shared__ __align__(16) unsigned char buf0[S::BUF];
    __shared__ __align__(16) unsigned char buf1[S::NBUF == 2 ? S::BUF : 16];
    const int64_t bx = blockIdx.x, grp = bx / (8 * 2 * NS);
    const int within = (int)(bx % (8 * 2 * NS)), slice = within / 8;
    const int64_t unit = grp * 8 + within % 8;       // (b*H + h) * (nseg - 1) + e
    const int64_t nspan = a.nseg - 1;
    if (unit >= a.nbh * nspan)
        return;
    const int64_t bh = unit / nspan, e = unit - bh * nspan, seg = a.nseg - 1 - e;
    const bool local = slice >= NS;
    if (e == 0 && !local)
        return;                                      // the last segment needs no product
    const int vs = local ? slice - NS : slice;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4;
    const int col = vs * S::BV + 16 * wave + (lane & 15);
    const int64_t n0 = seg * a.seg_len, n1 = min(a.NC, n0 + a.seg_len), rec0 = bh * a.NC;

    f32x4 lam[DT];
    if (local && e == 0 && a.dS_final) {
        const float* l0 = a.dS_final + bh * D * D;
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lam[kt][i] = l0[(16 * kt + 4 * gq + i) * D + col];
        // a copy of dS_final in entry 0's product half (the last segment has
        // no product): the scan starts the last segment from it, since dS0
        // may be dS_final and segment 0 writes dS0 in that same pass
        float* c0 = a.ws + a.L.span + bh * nspan * 2 * D * D;
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                c0[(16 * kt + 4 * gq + i) * D + col] = lam[kt][i];
    } else {
        const float one = local ? 0.f : 1.f;    // identity for the product, zero for the local gradient
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lam[kt][i] = 16 * kt + 4 * gq + i == col ? one : 0.f;
    }
    if (local)
        span_scan_run<true, E, D>(a, buf0, buf1, lam, rec0, n0, n1, vs, lane, wave);
    else
        span_scan_run<false, E, D>(a, buf0, buf1, lam, rec0, n0, n1, vs, lane, wave);

    float* dst = a.ws + a.L.span + ((bh * nspan + e) * 2 + (local ? 1 : 0)) * D * D;
#pragma unroll
    for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[(16 * kt + 4 * gq + i) * D + col] = lam[kt][i];
}

// ---------------------------------------------------------------------------
// Tile products of the chunk-local gradient (fp32 MFMA).  op(X) is X or X^T
// of a row-major matrix; every dimension is a multiple of 64 (M, N) or 16 (K).
// ---------------------------------------------------------------------------
// One row-major matrix operand of a tile product, already offset to its
// record: element (r, c) at p[r * ld + c]; trans = 1 reads it as X^T.
struct Mat {
    const float* p;
    int ld;
    int trans;
};

// One 64x64 tile of C = alpha (op(A1) op(B1) + op(A2) op(B2)) + beta C0 at
// rows m0.., columns n0.. of the record (the second product is skipped when
// K2 == 0).  All NTB threads take part: wave (wm, wn) owns a 32x32 quarter
// = 2x2 MFMA tiles, and each KB-deep k slab is staged in fp32 as sA[m][k]
// and sB[n][k] (rows padded to KB + 4 floats), the layout MM::load reads;
// with MM = Mma<bf16> the operands are rounded to bf16 as they are loaded
// into the MFMA (fp32 accumulation).  mask: 0 none, 1 keep n <= m, 2 keep
// n < m.
template <typename MM>
__device__ __forceinline__ void gemm_tile(float* sA, float* sB, int m0, int n0, int K1, Mat A1, Mat B1, int K2,
                                          Mat A2, Mat B2, float* Cz, int ldc, float alpha, float beta,
                                          const float* C0z, int mask)
{
    constexpr int KB = MM::KB, LS = KB + 4, NV = KB / 16;     // float4 per thread per operand slab
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
    // this thread's float4s of a slab: along k (row-major operand) or along m / n
    const int ra = tid / 4, ka = 4 * (tid % 4);      // 64 rows x 4 float4 along k, per 16 of k
    const int kb = tid / 16, ca = 4 * (tid % 16);    // 16 k-rows x 16 float4 along m / n
    // as a [row][k] source: A is "k along columns" when not transposed; B is
    // when transposed (op(B)(k, n) = B[n][k])
    auto fetch = [&](const float* p, int ld, bool k_cols, int r0, int k0, int v) -> f32x4 {
        return k_cols ? *reinterpret_cast<const f32x4*>(p + (int64_t)(r0 + ra) * ld + k0 + 16 * v + ka)
                      : *reinterpret_cast<const f32x4*>(p + (int64_t)(k0 + 16 * v + kb) * ld + r0 + ca);
    };
    auto stage = [&](float* sX, bool k_cols, f32x4 x, int v) {
        if (k_cols) {
            *reinterpret_cast<f32x4*>(sX + ra * LS + 16 * v + ka) = x;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sX[(ca + j) * LS + 16 * v + kb] = x[j];
        }
    };
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int seg = 0; seg < 2; ++seg) {
        const int K = seg == 0 ? K1 : K2;
        if (K == 0)
            break;
        const Mat A = seg == 0 ? A1 : A2, B = seg == 0 ? B1 : B2;
        const bool ak = A.trans == 0, bk = B.trans != 0;
        f32x4 va[NV], vb[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            va[v] = fetch(A.p, A.ld, ak, m0, 0, v);
            vb[v] = fetch(B.p, B.ld, bk, n0, 0, v);
        }
        for (int k0 = 0; k0 < K; k0 += KB) {
            __syncthreads();
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                stage(sA, ak, va[v], v);
                stage(sB, bk, vb[v], v);
            }
            __syncthreads();
            if (k0 + KB < K) {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    va[v] = fetch(A.p, A.ld, ak, m0, k0 + KB, v);
                    vb[v] = fetch(B.p, B.ld, bk, n0, k0 + KB, v);
                }
            }
            typename MM::Frag fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = MM::load(sA + (wm + 16 * i) * LS, LS, lane);
                fb[i] = MM::load(sB + (wn + 16 * i) * LS, LS, lane);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = MM::mma(fa[i], fb[j], acc[i][j]);
        }
    }
    const int gq = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int m = m0 + wm + 16 * i + 4 * gq + x, n = n0 + wn + 16 * j + cl;
                float val = alpha * acc[i][j][x];
                if (C0z)
                    val += beta * C0z[(int64_t)m * ldc + n];
                if ((mask == 1 && n > m) || (mask == 2 && n >= m))
                    val = 0.f;
                Cz[(int64_t)m * ldc + n] = val;
            }
}

// Results of one tile product are read by the next one in the same
// workgroup: complete the stores and meet at a barrier.
__device__ __forceinline__ void tile_done()
{
    __threadfence_block();
    __syncthreads();
}

// The products of the chunk-local gradient that involve the states, one
// workgroup per chunk record (S = the chunk-start state, Lam = dL/dS at its
// end):  Delta = U~ - W S,  dQ~ = dO S^T,  dW = -dDelta S^T,
// dK^ = Delta Lam^T,  dP = tril(dO Delta^T).
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_sgrad_kernel(BwdArgs a)
{
    constexpr int C = BC, NT = D / 64, LS = Mma<E>::KB + 4;
    __shared__ __align__(16) float sA[64 * LS];
    __shared__ __align__(16) float sB[64 * LS];
    const int64_t r = blockIdx.x;
    float* ws = a.ws;
    const size_t cd = (size_t)r * C * D, cc = (size_t)r * C * C, dd = (size_t)r * D * D;
    const Mat S{a.S_chunks + dd, D, 0}, St{a.S_chunks + dd, D, 1}, Lt{ws + a.L.Lam + dd, D, 1};
    const Mat W{ws + a.L.W + cd, D, 0}, dO{ws + a.L.dO + cd, D, 0}, dDel{ws + a.L.dDel + cd, D, 0};
    const Mat Del{ws + a.L.Del + cd, D, 0}, Delt{ws + a.L.Del + cd, D, 1}, none{nullptr, 0, 0};
    for (int nt = 0; nt < NT; ++nt)
        gemm_tile<Mma<E>>(sA, sB, 0, 64 * nt, D, W, S, 0, none, none, ws + a.L.Del + cd, D, -1.f, 1.f, ws + a.L.Ut + cd, 0);
    for (int nt = 0; nt < NT; ++nt) {
        gemm_tile<Mma<E>>(sA, sB, 0, 64 * nt, D, dO, St, 0, none, none, ws + a.L.dQt + cd, D, 1.f, 0.f, nullptr, 0);
        gemm_tile<Mma<E>>(sA, sB, 0, 64 * nt, D, dDel, St, 0, none, none, ws + a.L.dW + cd, D, -1.f, 0.f, nullptr, 0);
    }
    tile_done();                        // Delta complete
    for (int nt = 0; nt < NT; ++nt)
        gemm_tile<Mma<E>>(sA, sB, 0, 64 * nt, D, Del, Lt, 0, none, none, ws + a.L.dKh + cd, D, 1.f, 0.f, nullptr, 0);
    gemm_tile<Mma<E>>(sA, sB, 0, 0, D, dO, Delt, 0, none, none, ws + a.L.dP + cc, C, 1.f, 0.f, nullptr, 1);
}

// A 16x16 MFMA accumulator tile (lane l: rows 4(l/16)..+3 of column l%16)
// regrouped through a per-wave LDS patch of PATCH_LD-float rows into row
// pieces: lane l gets row l/4, columns 4(l%4)..+3, so that the tile leaves
// as one vector store per lane.  Within a wave the patch accesses run in
// order, so one patch serves tile after tile.
constexpr int PATCH_LD = 20;
constexpr int PATCH_FLOATS = 16 * PATCH_LD;
__device__ __forceinline__ f32x4 tile_rows(float* patch, f32x4 acc, int lane)
{
    const int gq = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        patch[(4 * gq + i) * PATCH_LD + cl] = acc[i];
    return *reinterpret_cast<const f32x4*>(patch + (lane >> 2) * PATCH_LD + 4 * (lane & 3));
}

// bf16 inputs: the same state products with every operand read from memory
// once (the tile version above re-reads S, W, dO and Delta from memory for
// each product, since a chunk's operands do not stay in cache), and then the
// WY-factor product dM that bwd_xgrad forms for fp32 inputs:
//   dX = dDelta U^T + dW E~^T,  T1 = dX X^T,  dM = strict_tril(-X^T T1)
// with dW, dX and T1 kept on chip (dU = X^T dDelta and dE~ = X^T dW are
// formed where they are used, in bwd_decay).  CG waves per 16 token rows:
// wave w owns the rows 16 (w % 4).. and a 1/CG share of the output columns
// of every product; its row operands W, dO and dDelta come straight from
// memory as A fragments; S (as S and S^T), Lam and Delta are staged in LDS
// in bf16, the precision of every MFMA operand here, and afterwards, in the
// same area, X and X^T, U, E~, the dW rows, dX and T1^T.  Delta never
// leaves the workgroup.
template <int D>
struct SgradShape {
    static constexpr int C = BC, LDB = D + 8;   // bf16 rows padded by 16 bytes: conflict-free fragment reads
    static constexpr int LDG = D / 4 + 1;         // fp32 row of the dgamma partial sums
    static constexpr size_t S_OFF = 0, ST_OFF = S_OFF + (size_t)D * LDB, L_OFF = ST_OFF + (size_t)D * LDB,
                            DEL_OFF = L_OFF + (size_t)D * LDB, ELEMS = DEL_OFF + (size_t)C * LDB;
    static constexpr int LX = C + 8;
    static constexpr size_t X_OFF = 0, XT_OFF = X_OFF + (size_t)C * LX, U_OFF = XT_OFF + (size_t)C * LX,
                            ET_OFF = U_OFF + (size_t)C * LDB, DW_OFF = ET_OFF + (size_t)C * LDB,
                            DX_OFF = DW_OFF + (size_t)C * LDB, T1T_OFF = DX_OFF + (size_t)C * LX,
                            X_END = T1T_OFF + (size_t)C * LX;
    static constexpr size_t AREA = ELEMS > X_END ? ELEMS : X_END;   // bf16 elements of the staging area
    static constexpr int CG = 2;                     // waves (column groups) per 16 token rows
    static constexpr int NTH = CG * 64 * (C / 16);   // threads
    static constexpr size_t PG_OFF = AREA * 2;       // bytes: the dgamma partial sums
    static constexpr size_t PATCH_OFF = PG_OFF + (size_t)D * LDG * 4;   // bytes: per-wave output patches
    static constexpr size_t SMEM = PATCH_OFF + (size_t)(NTH / 64) * PATCH_FLOATS * 4;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert((D / 16) % CG == 0 && (C / 16) % CG == 0, "whole tiles per column group");
};

template <int D>
__global__ __launch_bounds__(SgradShape<D>::NTH) void bwd_sgrad_bf16_kernel(BwdArgs a)
{
    typedef SgradShape<D> SH;
    typedef Mma<bf16> MM;
    typedef MM::Frag Frag;
    constexpr int C = BC, LDB = SH::LDB, NKS = D / MM::KB, NT = D / 16, NTH = SH::NTH, NH = NT / SH::CG;
    extern __shared__ __align__(16) bf16 sb[];
    bf16* sS = sb + SH::S_OFF;       // S[i][j]
    bf16* sSt = sb + SH::ST_OFF;     // S^T[j][i]
    bf16* sL = sb + SH::L_OFF;       // Lam[i][j]
    bf16* sDel = sb + SH::DEL_OFF;   // Delta[t][j]
    float* sPg = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(sb) + SH::PG_OFF);   // [D][LDG] partial sums of dgamma
    // after the state products: the dM operands
    bf16* sX = sb + SH::X_OFF;       // X[t][s]
    bf16* sXt = sb + SH::XT_OFF;     // X^T[s][t]
    bf16* sU = sb + SH::U_OFF;       // U[s][j]
    bf16* sEt = sb + SH::ET_OFF;     // E~[s][i]
    bf16* sDW = sb + SH::DW_OFF;     // dW[t][i]
    bf16* sdX = sb + SH::DX_OFF;     // dX[t][u]
    bf16* sT1t = sb + SH::T1T_OFF;   // T1^T[s][u]
    float* ws = a.ws;
    const int tid0 = threadIdx.x, wave = tid0 >> 6;
    float* patch = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(sb) + SH::PATCH_OFF) + wave * PATCH_FLOATS;
    const int rw = wave & 3, t0 = 16 * rw, n0 = (wave >> 2) * NH;   // row block; first of its NH column tiles
    // S and Lam of a record as pieces of 4 columns, loaded one record ahead
    // of their use.  Piece (wave, it) of a lane: u = NIT wave + it picks 4
    // rows 4 (u / NCH).. and 64 columns 64 (u % NCH)..; the lane quad q =
    // lane / 4 takes the columns 4q.. of them, and lane r = lane % 4 the row
    // 4 (u / NCH) + r.  A quad so holds a 4x4 block, which it transposes
    // across its lanes for S^T: 8-byte LDS writes instead of 2-byte ones
    // (the global reads stay 256-byte row pieces).
    constexpr int NIT = D * D / 4 / NTH, NCH = D / 64;
    static_assert(D * D / 4 % NTH == 0 && D % 64 == 0 && NIT * (NTH / 64) == (D / 4) * NCH, "whole pieces per lane");
    auto piece = [&](int it, int ln, int& i, int& j) {
        const int u = wave * NIT + it;
        i = 4 * (u / NCH) + (ln & 3);
        j = 64 * (u % NCH) + 4 * (ln >> 2);
    };
    f32x4 s4r[NIT];
    bf16x4 l4r[NIT];
    auto load_sl = [&](int64_t rr) {
        const float* S = a.S_chunks + (size_t)rr * D * D;
        const bf16* Lam = reinterpret_cast<const bf16*>(ws + a.L.Lam) + (size_t)rr * D * D;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            int i, j;
            piece(it, tid0 & 63, i, j);
            s4r[it] = *reinterpret_cast<const f32x4*>(S + (size_t)i * D + j);
            l4r[it] = *reinterpret_cast<const bf16x4*>(Lam + (size_t)i * D + j);
        }
    };
    // persistent: records blockIdx.x, + gridDim.x, ... (the grid is at most
    // nrec); the next record's S and Lam are in flight while this one's
    // products run, and barriers wait for LDS only, so the stores of a
    // record drain during the next.  Every global load is issued on every
    // path (the last prefetch re-reads the last record, rows past the valid
    // length read row 0 and are zeroed), which keeps the compiler's waits
    // for a load from also waiting for every later one.
    load_sl(blockIdx.x);
    for (int64_t r = blockIdx.x; r < a.nrec; r += gridDim.x) {
        // the lane index, opaque to the compiler in each iteration: no LDS
        // or memory address derived from it is hoisted out of the loop to
        // occupy a register throughout
        int lane = tid0 & 63;
        __asm__ __volatile__("" : "+v"(lane));
        const int tid = 64 * wave + lane, gq = lane >> 4, cl = lane & 15;
        const size_t cd = (size_t)r * C * D, cc = (size_t)r * C * C;
        const bf16* W = reinterpret_cast<const bf16*>(ws + a.L.W) + cd + (size_t)t0 * D;
        const bf16* dDel = reinterpret_cast<const bf16*>(ws + a.L.dDel) + cd + (size_t)t0 * D;
        // dO rows from the input (row t0 + lane % 16 of the chunk; zero past the
        // valid length)
        const Rec rc = rec_of(r, a.NC, a.T, a.H);
        const bool dorow = t0 + cl < rc.L;
        const bf16* dOr = (const bf16*)a.dO + (rc.row0 + (int64_t)(dorow ? t0 + cl : 0) * a.H) * D + 4 * gq;
        auto load_dO = [&](int ks) -> Frag {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(dOr + ks * MM::KB);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(dOr + ks * MM::KB + 16);
            const bf16 z = (bf16)0.f;
            Frag f;
            f[0] = dorow ? lo[0] : z; f[1] = dorow ? lo[1] : z; f[2] = dorow ? lo[2] : z; f[3] = dorow ? lo[3] : z;
            f[4] = dorow ? hi[0] : z; f[5] = dorow ? hi[1] : z; f[6] = dorow ? hi[2] : z; f[7] = dorow ? hi[3] : z;
            return f;
        };
        const size_t orow = cd + (size_t)(t0 + 4 * gq) * D + cl;   // output element (row 4gq, column cl) of the wave
        const size_t prow = cd + (size_t)(t0 + (lane >> 2)) * D + 4 * (lane & 3);   // the lane's row piece (tile_rows)
        // this wave's global operands of the products below, loaded first so
        // that they arrive while S and Lam are staged
        Frag pW[NKS], pD[NKS], pO[NKS];
        float pU[NH][4];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            pW[ks] = MM::load(W + ks * MM::KB, D, lane);
            pD[ks] = MM::load(dDel + ks * MM::KB, D, lane);
            pO[ks] = load_dO(ks);
        }
#pragma unroll
        for (int nt = 0; nt < NH; ++nt)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                pU[nt][x] = ws[a.L.Ut + orow + (size_t)x * D + 16 * (n0 + nt)];
        // staging also forms dgamma_i = sum_j S[i][j] Lam[i][j] in fp32 (Lam as
        // the scan stored it, in bf16; partial sums of 4 through LDS); gamma
        // becomes gamma * dgamma, the chunk-end term of dG_L that bwd_decay
        // adds (the scan has used gamma)
        const float gam_i = ws[a.L.gam + (size_t)r * D + tid % D];   // used by the threads tid < D
        // the staging below waits for S and Lam only: keep it after the
        // loads above, whose issue the wait then does not hold up
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();                   // the previous record's products are done with LDS
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            int i, j;
            piece(it, lane, i, j);
            const f32x4 s4 = s4r[it];
            const bf16x4 lv = l4r[it];
            bf16x4 sv, tv;
            f32x4 l4;
            // S^T[j + r][i - r ..]: this lane's column of the quad's 4x4 block
            const f32x4 st = quad_transpose(s4, lane & 3);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                sv[x] = (bf16)s4[x];
                tv[x] = (bf16)st[x];
                l4[x] = (float)lv[x];
            }
            *reinterpret_cast<bf16x4*>(sSt + (j + (lane & 3)) * LDB + (i - (lane & 3))) = tv;
            *reinterpret_cast<bf16x4*>(sS + i * LDB + j) = sv;
            *reinterpret_cast<bf16x4*>(sL + i * LDB + j) = lv;
            sPg[i * SH::LDG + j / 4] = s4[0] * l4[0] + s4[1] * l4[1] + s4[2] * l4[2] + s4[3] * l4[3];
        }
        load_sl(std::min<int64_t>(r + gridDim.x, a.nrec - 1));
        lds_barrier();
        if (tid < D) {
            float dg = 0.f;
#pragma unroll 8
            for (int c = 0; c < D / 4; ++c)
                dg += sPg[tid * SH::LDG + c];
            ws[a.L.gam + (size_t)r * D + tid] = gam_i * dg;
        }


        // Delta = U~ - W S   (k = i: B fragments from S^T)
        {
            f32x4 p[NH];
#pragma unroll
            for (int nt = 0; nt < NH; ++nt)
                p[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int nt = 0; nt < NH; ++nt)
                    p[nt] = MM::mma(pW[ks], MM::load(sSt + 16 * (n0 + nt) * LDB + ks * MM::KB, LDB, lane), p[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < NH; ++nt)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float dl = pU[nt][x] - p[nt][x];
                    sDel[(t0 + 4 * gq + x) * LDB + 16 * (n0 + nt) + cl] = (bf16)dl;
                }
        }
        // dQ~ = dO S^T,  dW = -dDelta S^T   (k = j: B fragments from S); the
        // dW tiles stay in registers for the dM phase
        f32x4 w[NH];
        {
            f32x4 q[NH];
#pragma unroll
            for (int nt = 0; nt < NH; ++nt)
                q[nt] = w[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int nt = 0; nt < NH; ++nt) {
                    const Frag bs = MM::load(sS + 16 * (n0 + nt) * LDB + ks * MM::KB, LDB, lane);
                    q[nt] = MM::mma(pO[ks], bs, q[nt]);
                    w[nt] = MM::mma(pD[ks], bs, w[nt]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NH; ++nt) {
                st4s(ws + a.L.dQt + prow + 16 * (n0 + nt), tile_rows(patch, q[nt], lane));
                store4(reinterpret_cast<bf16*>(ws + a.L.dW) + prow + 16 * (n0 + nt), tile_rows(patch, -w[nt], lane));
            }
        }
        lds_barrier();                   // every wave's Delta rows are in LDS
        // dK^ = Delta Lam^T   (A: this wave's Delta rows; k = j: B fragments from Lam)
        {
            f32x4 k[NH];
#pragma unroll
            for (int nt = 0; nt < NH; ++nt)
                k[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const Frag ad = MM::load(sDel + t0 * LDB + ks * MM::KB, LDB, lane);
#pragma unroll
                for (int nt = 0; nt < NH; ++nt)
                    k[nt] = MM::mma(ad, MM::load(sL + 16 * (n0 + nt) * LDB + ks * MM::KB, LDB, lane), k[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < NH; ++nt)
                st4s(ws + a.L.dKh + prow + 16 * (n0 + nt), tile_rows(patch, k[nt], lane));
        }
        // dP = tril(dO Delta^T)   (k = j: B fragments from the Delta rows s);
        // blocks above the diagonal are zero
        {
            constexpr int SBH = C / 16 / SH::CG;   // token blocks per column group
            const int s0 = (wave >> 2) * SBH;
            f32x4 pp[SBH];
#pragma unroll
            for (int sbk = 0; sbk < SBH; ++sbk)
                pp[sbk] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (s0 <= rw) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                    for (int sbk = 0; sbk < SBH; ++sbk)
                        if (s0 + sbk <= rw)
                            pp[sbk] = MM::mma(pO[ks], MM::load(sDel + 16 * (s0 + sbk) * LDB + ks * MM::KB, LDB, lane),
                                              pp[sbk]);
                }
            }
#pragma unroll
            for (int sbk = 0; sbk < SBH; ++sbk) {
                f32x4 m;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int t = t0 + 4 * gq + x, s_ = 16 * (s0 + sbk) + cl;
                    m[x] = s_ <= t ? pp[sbk][x] : 0.f;
                }
                st4s(ws + a.L.dP + cc + (size_t)(t0 + (lane >> 2)) * C + 16 * (s0 + sbk) + 4 * (lane & 3),
                     tile_rows(patch, m, lane));
            }
        }

        // the dM phase's operands from memory:
        // X, U and E~ rows (bf16), 4 elements per item
        constexpr int NXI = C * C / 4 / NTH, NUI = C * D / 4 / NTH;
        static_assert(C * C / 4 % NTH == 0 && C * D / 4 % NTH == 0, "whole items per thread");
        bf16x4 xr[NXI], ur[NUI], er[NUI];
        {
            const bf16x4* Xg = reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(ws + a.L.X) + cc);
            const bf16x4* Ug = reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(ws + a.L.U) + cd);
            const bf16x4* Eg = reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(ws + a.L.Et) + cd);
#pragma unroll
            for (int it = 0; it < NXI; ++it)
                xr[it] = Xg[tid + it * NTH];
#pragma unroll
            for (int it = 0; it < NUI; ++it) {
                ur[it] = Ug[tid + it * NTH];
                er[it] = Eg[tid + it * NTH];
            }
        }
        // dM = strict_tril(-X^T T1), T1 = dX X^T, dX = dDelta U^T + dW E~^T,
        // in the staging area once every wave is done with S, Lam and Delta
        constexpr int LX = SH::LX, KB = MM::KB;
        const int hf = wave >> 2;        // this wave's column blocks 2 hf, 2 hf + 1 of the C x C products
        lds_barrier();
#pragma unroll
        for (int it = 0; it < NXI; ++it) {
            const int e = tid + it * NTH, t = e / (C / 4), c = 4 * (e % (C / 4));
            const bf16x4 xv = xr[it];
#pragma unroll
            for (int y = 0; y < 4; ++y)
                sXt[(c + y) * LX + t] = xv[y];
            *reinterpret_cast<bf16x4*>(sX + t * LX + c) = xv;
        }
#pragma unroll
        for (int it = 0; it < NUI; ++it) {
            const int e = tid + it * NTH, t = e / (D / 4), j = 4 * (e % (D / 4));
            *reinterpret_cast<bf16x4*>(sU + t * LDB + j) = ur[it];
            *reinterpret_cast<bf16x4*>(sEt + t * LDB + j) = er[it];
        }
#pragma unroll
        for (int nt = 0; nt < NH; ++nt)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                sDW[(t0 + 4 * gq + x) * LDB + 16 * (n0 + nt) + cl] = (bf16)(-w[nt][x]);
        lds_barrier();
        {
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const Frag ad = pD[ks];                                // this wave's dDelta rows, kept
                const Frag aw = MM::load(sDW + t0 * LDB + ks * KB, LDB, lane);
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int sbk = 2 * hf + n;
                    acc[n] = MM::mma(ad, MM::load(sU + 16 * sbk * LDB + ks * KB, LDB, lane), acc[n]);
                    acc[n] = MM::mma(aw, MM::load(sEt + 16 * sbk * LDB + ks * KB, LDB, lane), acc[n]);
                }
            }
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    sdX[(t0 + 4 * gq + x) * LX + 16 * (2 * hf + n) + cl] = (bf16)acc[n][x];
        }
        lds_barrier();                   // dX complete
        {
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < C / KB; ++ks) {
                const Frag ad = MM::load(sdX + t0 * LX + ks * KB, LX, lane);
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[n] = MM::mma(ad, MM::load(sX + 16 * (2 * hf + n) * LX + ks * KB, LX, lane), acc[n]);
            }
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    sT1t[(16 * (2 * hf + n) + cl) * LX + t0 + 4 * gq + x] = (bf16)acc[n][x];
        }
        lds_barrier();                   // T1 complete
        {
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < C / KB; ++ks) {
                const Frag ax = MM::load(sXt + t0 * LX + ks * KB, LX, lane);
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    if (2 * hf + n <= rw)
                        acc[n] = MM::mma(ax, MM::load(sT1t + 16 * (2 * hf + n) * LX + ks * KB, LX, lane), acc[n]);
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                f32x4 m;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int t = t0 + 4 * gq + x, s_ = 16 * (2 * hf + n) + cl;
                    m[x] = s_ < t ? -acc[n][x] : 0.f;
                }
                st4s(ws + a.L.dM + cc + (size_t)(t0 + (lane >> 2)) * C + 16 * (2 * hf + n) + 4 * (lane & 3),
                     tile_rows(patch, m, lane));
            }
        }
    }
}

// fp32 inputs: the products through the WY factor X = (I + M)^-1, one
// workgroup per chunk record:  dX = dDelta U^T + dW E~^T,  dM = strict_tril(-X^T dX X^T),
// dU = X^T dDelta,  dE~ = X^T dW.
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_xgrad_kernel(BwdArgs a)
{
    constexpr int C = BC, NT = D / 64, LS = Mma<E>::KB + 4;
    __shared__ __align__(16) float sA[64 * LS];
    __shared__ __align__(16) float sB[64 * LS];
    const int64_t r = blockIdx.x;
    float* ws = a.ws;
    const size_t cd = (size_t)r * C * D, cc = (size_t)r * C * C;
    const Mat dDel{ws + a.L.dDel + cd, D, 0}, dW{ws + a.L.dW + cd, D, 0};
    const Mat Ut{ws + a.L.U + cd, D, 1}, Ett{ws + a.L.Et + cd, D, 1};
    const Mat Xt{ws + a.L.X + cc, C, 1}, dX{ws + a.L.dX + cc, C, 0}, T1{ws + a.L.T1 + cc, C, 0}, none{nullptr, 0, 0};
    gemm_tile<Mma<E>>(sA, sB, 0, 0, D, dDel, Ut, D, dW, Ett, ws + a.L.dX + cc, C, 1.f, 0.f, nullptr, 0);
    for (int nt = 0; nt < NT; ++nt) {
        gemm_tile<Mma<E>>(sA, sB, 0, 64 * nt, C, Xt, dDel, 0, none, none, ws + a.L.dU + cd, D, 1.f, 0.f, nullptr, 0);
        gemm_tile<Mma<E>>(sA, sB, 0, 64 * nt, C, Xt, dW, 0, none, none, ws + a.L.dEt + cd, D, 1.f, 0.f, nullptr, 0);
    }
    tile_done();                        // dX complete
    gemm_tile<Mma<E>>(sA, sB, 0, 0, C, dX, Xt, 0, none, none, ws + a.L.T1 + cc, C, 1.f, 0.f, nullptr, 0);
    tile_done();                        // T1 complete
    gemm_tile<Mma<E>>(sA, sB, 0, 0, C, Xt, T1, 0, none, none, ws + a.L.dM + cc, C, -1.f, 0.f, nullptr, 2);
}

// ---------------------------------------------------------------------------
// bwd_decay: per chunk and block of DC key channels, the decay-weighted sums
// and the input gradients.  Every channel is independent here, so one
// workgroup takes DC channels of one chunk; thread (row group rg, channel)
// owns the RPT consecutive tokens t = RPT*rg + m of its channel.  One pass
// over the partner token u serves both sums of every owned token:
//   u <= t:  f = e^{G_t - G_u};  dE_M[t] += dM[t,u] k_u f,  dq_P[t] += dP[t,u] k_u f
//   u >= t:  f = e^{G_u - G_t};  dk[t]   += (dM[u,t] e_u + dP[u,t] q_u) f
// (dM is strictly lower, so the u == t terms of dM vanish.)
// ---------------------------------------------------------------------------
constexpr int LC = DC + 1;             // padded LDS row of the per-channel arrays
constexpr int LPC = BC + 4;            // padded LDS row of dM and dP (16-byte aligned)

// bwd_decay's up-front loads for one gate-width mix (B1, W1: b, w of width
// 1): this thread's items (token t, 4 channels from i0) of the input rows
// and of dE~, dQ~, dK^, dU.  Every load is issued before any is used; rows
// past the valid length re-read the last valid row and are zeroed here.
template <bool B1, bool W1, typename E, int D, int NIT>
__device__ __forceinline__ void decay_loads(const BwdArgs& a, const Rec& rc, int64_t r, int tid, int i0, f32x4* xk,
                                            f32x4* xq, f32x4* xb, f32x4* xw, f32x4* xv, f32x4* xdEt, f32x4* xdQt,
                                            f32x4* xdKh, f32x4* xdU, float* xrk, float* xrq, f32x4* xG)
{
    typedef Raw4<E> R;
    constexpr int C = BC;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* b = (const E*)a.b;
    const E* w = (const E*)a.w;
    const float* ws = a.ws;
    const size_t cdo = (size_t)r * C * D;
    typename R::V rk[NIT], rq[NIT], rv[NIT], rb[NIT], rw[NIT];
    E sb[NIT], sw[NIT];
#pragma unroll
    for (int p = 0; p < NIT; ++p) {
        const int e4 = tid + p * NTB, t = e4 / (DC / 4), c = 4 * (e4 % (DC / 4));
        const size_t x = cdo + (size_t)t * D + i0 + c;
        const int64_t row = rc.row0 + (int64_t)min(t, rc.L - 1) * a.H;
        rk[p] = ld_raw4(k + row * D + i0 + c);
        rq[p] = ld_raw4(q + row * D + i0 + c);
        rv[p] = ld_raw4(v + row * D + i0 + c);
        if (B1)
            sb[p] = b[row];
        else
            rb[p] = ld_raw4(b + row * D + i0 + c);
        if (W1)
            sw[p] = w[row];
        else
            rw[p] = ld_raw4(w + row * D + i0 + c);
        xrk[p] = xrq[p] = 1.f;
        if (a.pro & GDR2_PROLOGUE_NORM_QK) {
            xrk[p] = ws[a.L.RN + (size_t)r * 2 * C + t];
            xrq[p] = ws[a.L.RN + (size_t)r * 2 * C + C + t];
        }
        if constexpr (sizeof(E) == 4) {   // bf16: formed in the decay kernel (decay_wy_slices)
            xdEt[p] = *reinterpret_cast<const f32x4*>(ws + a.L.dEt + x);
            xdU[p] = *reinterpret_cast<const f32x4*>(ws + a.L.dU + x);
        }
        xdQt[p] = *reinterpret_cast<const f32x4*>(ws + a.L.dQt + x);
        xdKh[p] = *reinterpret_cast<const f32x4*>(ws + a.L.dKh + x);
        xG[p] = *reinterpret_cast<const f32x4*>(ws + a.L.G + x);
    }
#pragma unroll
    for (int p = 0; p < NIT; ++p) {
        const int t = (tid + p * NTB) / (DC / 4);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const bool valid = t < rc.L;
        xk[p] = valid ? R::cvt(rk[p]) : z;
        xq[p] = valid ? R::cvt(rq[p]) : z;
        xv[p] = valid ? R::cvt(rv[p]) : z;
        xb[p] = valid ? (B1 ? bcast4(to_f32(sb[p])) : R::cvt(rb[p])) : z;
        xw[p] = valid ? (W1 ? bcast4(to_f32(sw[p])) : R::cvt(rw[p])) : z;
        if (!valid)
            xrk[p] = xrq[p] = 1.f;
    }
}

// bf16 inputs: dU = X^T dDelta and dE~ = X^T dW on a decay workgroup's DC
// channels (X = (I + M)^-1; bwd_sgrad forms dM), straight into the
// thread's items (token t, 4 channels) as the decay kernel uses them.  Four
// waves; wave w owns the token rows 16w..  X^T and the group's columns of
// dDelta and dW are staged in LDS transposed, in bf16 (the MFMA operands'
// precision), in the area the decay kernel fills only afterwards.
template <int D>
struct DecayWY {
    static constexpr int C = BC, LX = C + 8;                 // bf16 rows padded by 16 bytes
    static constexpr size_t XT = 0, DDT = XT + (size_t)C * LX, DWT = DDT + (size_t)DC * LX,
                            END = DWT + (size_t)DC * LX;     // bf16 elements
    static constexpr size_t OU = (END * 2 + 15) / 16 * 4;   // float offset of the dU, dE~ outputs [C][LC]
    static constexpr size_t BYTES = OU * 4 + 2 * (size_t)C * LC * 4;
};

template <int D, int NIT>
__device__ __forceinline__ void decay_wy_slices(const BwdArgs& a, int64_t r, int i0, int tid, float* scratch,
                                                f32x4* xdEt, f32x4* xdU)
{
    typedef DecayWY<D> WY;
    typedef Mma<bf16> MM;
    typedef MM::Frag Frag;
    constexpr int C = BC, LX = WY::LX, KB = MM::KB, NJ = DC / 16;
    static_assert(NTB == 256 && C == 64 && DC == 32, "four waves, one 16-token block each; 4x4 staging blocks");
    bf16* sx = reinterpret_cast<bf16*>(scratch);
    bf16* sXt = sx + WY::XT;       // X^T[s][t]
    bf16* sDdT = sx + WY::DDT;     // dDelta^T[j][t], the group's channels j
    bf16* sDwT = sx + WY::DWT;     // dW^T[i][t]
    float* sOU = scratch + WY::OU; // dU[t][j], the group's channels
    float* sOE = sOU + C * LC;     // dE~[t][i]
    const float* ws = a.ws;
    const size_t cd = (size_t)r * C * D, cc = (size_t)r * C * C;
    const bf16* Xg = reinterpret_cast<const bf16*>(ws + a.L.X) + cc;
    const bf16* dDel = reinterpret_cast<const bf16*>(ws + a.L.dDel) + cd;
    const bf16* dW = reinterpret_cast<const bf16*>(ws + a.L.dW) + cd;
    const int lane = tid & 63, wave = tid >> 6, gq = lane >> 4, cl = lane & 15, t0 = 16 * wave;

    // X^T: one 4x4 block of X per thread (rows 4bi.., columns 4bj..),
    // transposed in registers.  dDelta^T (threads 0-127) and dW^T (128-255):
    // one 4x4 block each, tokens 4ti.., the group's channels 4jj..
    {
        const int bi = tid >> 4, bj = tid & 15;
        const int half = tid >> 7, e = tid & 127, ti = e >> 3, jj = e & 7;
        const bf16* src = half ? dW : dDel;
        bf16x4 x4[4], d4[4];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            x4[y] = *reinterpret_cast<const bf16x4*>(Xg + (4 * bi + y) * C + 4 * bj);
            d4[y] = *reinterpret_cast<const bf16x4*>(src + (size_t)(4 * ti + y) * D + i0 + 4 * jj);
        }
        bf16* dst = half ? sDwT : sDdT;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            *reinterpret_cast<bf16x4*>(sXt + (4 * bj + x) * LX + 4 * bi) = bf16x4{x4[0][x], x4[1][x], x4[2][x], x4[3][x]};
            *reinterpret_cast<bf16x4*>(dst + (4 * jj + x) * LX + 4 * ti) = bf16x4{d4[0][x], d4[1][x], d4[2][x], d4[3][x]};
        }
    }
    lds_barrier();
    f32x4 au[NJ], ae[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
        au[jt] = ae[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C / KB; ++ks) {
        const Frag fx = MM::load(sXt + t0 * LX + ks * KB, LX, lane);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            au[jt] = MM::mma(fx, MM::load(sDdT + 16 * jt * LX + ks * KB, LX, lane), au[jt]);
            ae[jt] = MM::mma(fx, MM::load(sDwT + 16 * jt * LX + ks * KB, LX, lane), ae[jt]);
        }
    }
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            sOU[(t0 + 4 * gq + x) * LC + 16 * jt + cl] = au[jt][x];
            sOE[(t0 + 4 * gq + x) * LC + 16 * jt + cl] = ae[jt][x];
        }
    lds_barrier();
#pragma unroll
    for (int p = 0; p < NIT; ++p) {
        const int e4 = tid + p * NTB, t = e4 / (DC / 4), c = 4 * (e4 % (DC / 4)), l = t * LC + c;
        xdU[p] = f32x4{sOU[l], sOU[l + 1], sOU[l + 2], sOU[l + 3]};
        xdEt[p] = f32x4{sOE[l], sOE[l + 1], sOE[l + 2], sOE[l + 3]};
    }
    lds_barrier();                       // the scratch is free for the row arrays
}

template <typename E, int D>
__global__ __launch_bounds__(NTB, 2) void bwd_decay_kernel(BwdArgs a)
{
    constexpr int C = BC, NRG = NTB / DC, RPT = C / NRG;
    static_assert(RPT == 8, "two 16-byte reads cover a thread's tokens");
    static_assert(NTB / 64 == C / 16, "one wave per 16-token block in the block sums");
    extern __shared__ __align__(16) float sm[];
    float* sdM = sm;                // [C][LPC]
    float* sdP = sdM + C * LPC;     // [C][LPC]
    float* sG = sdP + C * LPC;      // [C][LC] cumulative log-decay
    float* sE = sG + C * LC;        // [C][LC] e = b*k
    float* sK = sE + C * LC;        // [C][LC] k
    float* sQ = sK + C * LC;        // [C][LC] q
    float* sdG = sQ + C * LC;       // [C][LC] dG, then dg
    float* sGL = sdG + C * LC;      // [DC] dG_L
    // width-1 gates, in the epilogue (e, k and q rows are no longer read
    // then): per-thread partials of db and dw [C][DC/4], per-channel dg [C][DC]
    float* sRb = sE;
    float* sRw = sRb + C * (DC / 4);
    float* sRg = sRw + C * (DC / 4);
    static_assert(2 * C * (DC / 4) + C * DC <= 3 * C * LC, "partials fit the e, k, q rows");
    __shared__ int sOr[2 * (NTB / 64)];
    // workgroup -> (chunk record, channel group): the D/DC groups of a
    // record share blockIdx % 8, i.e. one XCD, so the dM and dP they all
    // stage come from HBM once and from that XCD's L2 after
    constexpr int NCG = D / DC;
    const int64_t bx = blockIdx.x, grp = bx / (8 * NCG);
    const int within = (int)(bx % (8 * NCG));
    const int64_t r = grp * 8 + within % 8;
    if (r >= a.nrec)
        return;
    const int i0 = (within / 8) * DC;
    const Rec rc = rec_of(r, a.NC, a.T, a.H);
    const int tid = threadIdx.x, il = tid % DC, rg = tid / DC, i = i0 + il, t0 = RPT * rg;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* b = (const E*)a.b;
    const E* w = (const E*)a.w;
    const float* ws = a.ws;
    const size_t cdo = (size_t)r * C * D, cco = (size_t)r * C * C;

    // This thread's items (token t, 4 channels) of the row arrays: every
    // global operand of the staging and of the epilogue is loaded here, up
    // front, so those loads overlap everything up to the epilogue.
    constexpr int NIT = C * DC / 4 / NTB;
    static_assert(NIT * NTB == C * DC / 4, "whole items per thread");
    f32x4 xk[NIT], xq[NIT], xb[NIT], xw[NIT], xv[NIT], xdEt[NIT], xdQt[NIT], xdKh[NIT], xdU[NIT];
    float xrk[NIT], xrq[NIT];
    f32x4 xG[NIT];
    switch ((a.bw == 1 ? 2 : 0) | (a.ww == 1 ? 1 : 0)) {
    case 0: decay_loads<false, false, E, D, NIT>(a, rc, r, tid, i0, xk, xq, xb, xw, xv, xdEt, xdQt, xdKh, xdU, xrk, xrq, xG); break;
    case 1: decay_loads<false, true, E, D, NIT>(a, rc, r, tid, i0, xk, xq, xb, xw, xv, xdEt, xdQt, xdKh, xdU, xrk, xrq, xG); break;
    case 2: decay_loads<true, false, E, D, NIT>(a, rc, r, tid, i0, xk, xq, xb, xw, xv, xdEt, xdQt, xdKh, xdU, xrk, xrq, xG); break;
    default: decay_loads<true, true, E, D, NIT>(a, rc, r, tid, i0, xk, xq, xb, xw, xv, xdEt, xdQt, xdKh, xdU, xrk, xrq, xG); break;
    }
    // dM, dP loads in flight before any LDS use
    constexpr int NMP = C * C / 4 / NTB;
    static_assert(C * C / 4 % NTB == 0, "whole items per thread");
    f32x4 rM[NMP], rP[NMP];
#pragma unroll
    for (int it = 0; it < NMP; ++it) {
        const int e = tid + it * NTB, t = e / (C / 4), c = 4 * (e % (C / 4));
        rM[it] = *reinterpret_cast<const f32x4*>(ws + a.L.dM + cco + t * C + c);
        rP[it] = *reinterpret_cast<const f32x4*>(ws + a.L.dP + cco + t * C + c);
    }
    if constexpr (sizeof(E) == 2) {
        static_assert(DecayWY<D>::BYTES <= (size_t)(2 * C * LPC + 5 * C * LC + DC) * 4, "the scratch fits");
        decay_wy_slices<D, NIT>(a, r, i0, tid, sm, xdEt, xdU);
    }
#pragma unroll
    for (int p = 0; p < NIT; ++p) {
        // k, q normalised and b activated under the prologue; e = b k as
        // bwd_prep forms it
        xk[p] = xk[p] * xrk[p];
        xq[p] = xq[p] * xrq[p];
        if (a.pro & GDR2_PROLOGUE_GATES)
            xb[p] = bsigm4(xb[p]);
        const int e4 = tid + p * NTB, t = e4 / (DC / 4), c = 4 * (e4 % (DC / 4)), l = t * LC + c;
        const f32x4 gv = xG[p];
        const f32x4 ev = xb[p] * xk[p];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sG[l + j] = gv[j];
            sE[l + j] = ev[j];
            sK[l + j] = xk[p][j];
            sQ[l + j] = xq[p][j];
            sdG[l + j] = xdKh[p][j];     // for dG_L below (sdG is free until the main loop)
        }
    }
#pragma unroll
    for (int it = 0; it < NMP; ++it) {
        const int e = tid + it * NTB, t = e / (C / 4), c = 4 * (e % (C / 4));
        *reinterpret_cast<f32x4*>(sdM + t * LPC + c) = rM[it];
        *reinterpret_cast<f32x4*>(sdP + t * LPC + c) = rP[it];
    }
    lds_barrier();
    // dG_L = sum_s dK^ K^ + dgamma gamma, with dgamma = rowsum(S * Lam) and
    // K^ = k e^{G_L - G} recomputed from the rows in LDS: every thread sums
    // its share (D / NRG state columns, RPT tokens) of its channel, then the
    // NRG partial sums of a channel are added up
    {
        float acc = 0.f;
        if constexpr (sizeof(E) == 2) {
            // bf16 inputs: bwd_sgrad_bf16 left gamma * dgamma in gam
            acc = rg == 0 ? ws[a.L.gam + (size_t)r * D + i] : 0.f;
        } else {
            constexpr int JPT = D / NRG;
            const float* S = a.S_chunks + (size_t)r * D * D + (size_t)i * D + rg * JPT;
            const float* Lam = ws + a.L.Lam + (size_t)r * D * D + (size_t)i * D + rg * JPT;
#pragma unroll
            for (int j = 0; j < JPT; j += 4) {
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(S + j), l4 = *reinterpret_cast<const f32x4*>(Lam + j);
                acc += s4[0] * l4[0] + s4[1] * l4[1] + s4[2] * l4[2] + s4[3] * l4[3];
            }
            acc *= ws[a.L.gam + (size_t)r * D + i];
        }
        const float GL = sG[(C - 1) * LC + il];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int l = (t0 + m) * LC + il;
            acc += sdG[l] * (sK[l] * __expf(GL - sG[l]));     // dK^ staged above
        }
        lds_barrier();                  // every thread has read its dK^ rows
        sdG[rg * LC + il] = acc;        // sdG is free until the main loop
    }
    lds_barrier();
    if (tid < DC) {
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < NRG; ++g)
            acc += sdG[g * LC + tid];
        sGL[tid] = acc;
    }

    // growth (some G_t > G_t-1, i.e. a log-decay > 0) anywhere in these
    // channels: every pair takes its own exponential
    int grow = 0;
    for (int e = tid; e < (C - 1) * DC; e += NTB) {
        const int t = e / DC + 1, c = e % DC;
        grow |= sG[t * LC + c] > sG[(t - 1) * LC + c];
    }
    grow = lds_barrier_or<NTB / 64>(grow, sOr);

    // a 16-token block whose decay spans more than kDiagSpan in some channel:
    // the diagonal blocks take the pair-by-pair pass below
    int steep = 0;
    for (int e = tid; e < (C / 16) * DC; e += NTB) {
        const int T = e / DC, c = e % DC;
        steep |= sG[16 * T * LC + c] - sG[(16 * T + 15) * LC + c] > kDiagSpan;
    }
    steep = lds_barrier_or<NTB / 64>(steep, sOr + NTB / 64);
    const bool pairwise = grow || steep;

    float Gt[RPT], dEm[RPT], dqp[RPT], dkm[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        Gt[m] = sG[(t0 + m) * LC + il];
        dEm[m] = dqp[m] = dkm[m] = 0.f;
    }
    // the partner tokens u of the pair-by-pair pass: all of them (growth), or
    // only the 16-token block of the thread's rows (steep blocks)
    const int u_lo = grow ? 0 : (t0 / 16) * 16, u_hi = !pairwise ? u_lo : grow ? C : u_lo + 16;
    for (int u0 = u_lo; u0 < u_hi; u0 += 4) {
        f32x4 rM[RPT], rP[RPT];          // dM[t, u0..u0+3], dP[t, u0..u0+3]
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            rM[m] = *reinterpret_cast<const f32x4*>(sdM + (t0 + m) * LPC + u0);
            rP[m] = *reinterpret_cast<const f32x4*>(sdP + (t0 + m) * LPC + u0);
        }
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
            const int u = u0 + uu;
            const float Gu = sG[u * LC + il], ku = sK[u * LC + il], eu = sE[u * LC + il], qu = sQ[u * LC + il];
            // dM[u, t0..t0+7], dP[u, t0..t0+7]
            const f32x4 cM0 = *reinterpret_cast<const f32x4*>(sdM + u * LPC + t0);
            const f32x4 cM1 = *reinterpret_cast<const f32x4*>(sdM + u * LPC + t0 + 4);
            const f32x4 cP0 = *reinterpret_cast<const f32x4*>(sdP + u * LPC + t0);
            const f32x4 cP1 = *reinterpret_cast<const f32x4*>(sdP + u * LPC + t0 + 4);
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int t = t0 + m;
                const float d = Gt[m] - Gu;
                const float f = __expf(u <= t ? d : -d);
                const float w1 = u <= t ? f * ku : 0.f, w2 = u >= t ? f : 0.f;
                dEm[m] += rM[m][uu] * w1;
                dqp[m] += rP[m][uu] * w1;
                const float cm = m < 4 ? cM0[m & 3] : cM1[m & 3], cp = m < 4 ? cP0[m & 3] : cP1[m & 3];
                dkm[m] += (cm * eu + cp * qu) * w2;
            }
        }
    }
    // the three sums go to LDS (the dM / dP area) for the epilogue, which
    // takes four channels per item
    float* sEm = sdM;                    // [C][LC] dE_M
    float* sQp = sEm + C * LC;           // [C][LC] dq_P
    float* sKm = sQp + C * LC;           // [C][LC] dk_M + dk_P
    if (!grow) {
        // Decays only.  The rows are re-referenced in place to their 16-token
        // block,  E^ = e e^{G - G_16T},  Q^ = q e^{G - G_16T},  K- = k e^{G_16T+15 - G},
        // so with c_TS = e^{G_16T - G_16S+15} (<= 1 below the diagonal,
        // e^{span of block T} <= e^kDiagSpan on it), for blocks S <= T:
        //   dE_M[t] = e^{G_t - G_16T} sum_S c_TS sum_{s in S} dM[t,s] K-_s     (dq_P with dP)
        //   dk[s]   = e^{G_16S+15 - G_s} sum_T c_TS sum_{t in T} (dM[t,s] E^_t + dP[t,s] Q^_t)
        // block by block on fp32 MFMA; wave w takes token block w, as the
        // later token and as the earlier one.  Steep diagonal blocks came
        // from the pass above.  The epilogue reads the raw rows again.
        float* sCf = sdG;                // [10][DC] c_TS: the pairs S < T, then the diagonal
        lds_barrier();                   // the pass above is done with the raw rows
        for (int e = tid; e < C * DC; e += NTB) {
            const int t = e / DC, c = e % DC, l = t * LC + c, T = t / 16;
            const float G = sG[l];
            const float fa = __expf(G - sG[16 * T * LC + c]), fb = __expf(sG[(16 * T + 15) * LC + c] - G);
            sE[l] *= fa;
            sQ[l] *= fa;
            sK[l] *= fb;
        }
        for (int e = tid; e < 10 * DC; e += NTB) {
            const int pi = e / DC, c = e % DC;
            const int T = pi < 1 ? 1 : pi < 3 ? 2 : pi < 6 ? 3 : pi - 6;
            const int S = pi < 6 ? pi - (T * (T - 1)) / 2 : T;
            sCf[e] = __expf(sG[16 * T * LC + c] - sG[(16 * S + 15) * LC + c]);
        }
        lds_barrier();
        typedef Mma<float> MF;
        constexpr int NCT = DC / 16;
        const int wave = tid >> 6, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 aE[NCT], aQ[NCT], aK[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            aE[ct] = aQ[ct] = aK[ct] = zero;
        for (int S = 0; S <= wave; ++S) {            // as the later token (T = wave)
            if (S == wave && steep)
                continue;
            const int pi = S < wave ? wave * (wave - 1) / 2 + S : 6 + wave;
            const MF::Frag am = MF::load(sdM + 16 * wave * LPC + 16 * S, LPC, lane);
            const MF::Frag ap = MF::load(sdP + 16 * wave * LPC + 16 * S, LPC, lane);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const MF::Frag kb = MF::load_kn(sK + 16 * S * LC + 16 * ct, LC, lane);
                const float c = sCf[pi * DC + 16 * ct + cl];
                aE[ct] += c * MF::mma(am, kb, zero);
                aQ[ct] += c * MF::mma(ap, kb, zero);
            }
        }
        for (int T = wave; T < C / 16; ++T) {        // as the earlier token (S = wave)
            if (T == wave && steep)
                continue;
            const int pi = wave < T ? T * (T - 1) / 2 + wave : 6 + T;
            // dM[t][s], dP[t][s] with s as the row: rows s of block S, k = t of block T
            const MF::Frag am = MF::load_kn(sdM + 16 * T * LPC + 16 * wave, LPC, lane);
            const MF::Frag ap = MF::load_kn(sdP + 16 * T * LPC + 16 * wave, LPC, lane);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 z = MF::mma(am, MF::load_kn(sE + 16 * T * LC + 16 * ct, LC, lane), zero);
                z = MF::mma(ap, MF::load_kn(sQ + 16 * T * LC + 16 * ct, LC, lane), z);
                aK[ct] += sCf[pi * DC + 16 * ct + cl] * z;
            }
        }
        lds_barrier();                   // dM and dP no longer read
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int t = 16 * wave + 4 * gq + x, c = 16 * ct + cl, l = t * LC + c;
                const float G = sG[l];
                const float fa = __expf(G - sG[16 * wave * LC + c]), fb = __expf(sG[(16 * wave + 15) * LC + c] - G);
                sEm[l] = fa * aE[ct][x];
                sQp[l] = fa * aQ[ct][x];
                sKm[l] = fb * aK[ct][x];
            }
        if (steep) {
            lds_barrier();
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int l = (t0 + m) * LC + il;
                sEm[l] += dEm[m];
                sQp[l] += dqp[m];
                sKm[l] += dkm[m];
            }
        }
    } else {
        lds_barrier();                   // dM and dP no longer read
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int l = (t0 + m) * LC + il;
            sEm[l] = dEm[m];
            sQp[l] = dqp[m];
            sKm[l] = dkm[m];
        }
    }
    lds_barrier();
#pragma unroll
    for (int p = 0; p < NIT; ++p) {
        const int e4 = tid + p * NTB, t = e4 / (DC / 4), c = 4 * (e4 % (DC / 4)), l = t * LC + c;
        const f32x4 dEt = xdEt[p], dQt = xdQt[p], dKh = xdKh[p], dU = xdU[p];
        // raw rows (LDS may hold the re-referenced ones), held since the
        // start: k and q normalised and b activated under the prologue, e = b k
        const f32x4 kr = xk[p], qr = xq[p], bv = xb[p];
        const f32x4 bd = (a.pro & GDR2_PROLOGUE_GATES) ? bv * (f32x4{1.f, 1.f, 1.f, 1.f} - bv)
                                                       : f32x4{1.f, 1.f, 1.f, 1.f};   // d(activation)/d(raw)
        const f32x4 ev = bv * kr;
        f32x4 dq, dk, dE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // E~ = E e^G, Q~ = q e^G, K^ = k e^{G_L - G}, recomputed exactly as
            // bwd_prep forms them
            const float G = sG[l + j], eg = __expf(G), kd = __expf(sG[(C - 1) * LC + c + j] - G);
            float dG = ev[j] * sEm[l + j] + qr[j] * sQp[l + j] - kr[j] * sKm[l + j] + dEt[j] * (ev[j] * eg) +
                       dQt[j] * (qr[j] * eg) - dKh[j] * (kr[j] * kd);
            if (t == rc.L - 1)
                dG += sGL[c + j];
            sdG[l + j] = dG;
            dE[j] = sEm[l + j] + dEt[j] * eg;
            dq[j] = sQp[l + j] + dQt[j] * eg;
            dk[j] = sKm[l + j] + dKh[j] * kd;
        }
        if (t < rc.L) {
            const int64_t row = rc.row0 + (int64_t)t * a.H, off = row * D + i0 + c;
            f32x4 wv = xw[p], wd = {1.f, 1.f, 1.f, 1.f};
            // prologue gates: the activated values, and d(activation)/d(raw)
            if (a.pro & GDR2_PROLOGUE_GATES) {
                wv = bsigm4(wv);
                wd = wv * (f32x4{1.f, 1.f, 1.f, 1.f} - wv);
            }
            const f32x4 vv = xv[p], kv = kr;
            *reinterpret_cast<f32x4*>(a.dq + off) = dq;
            *reinterpret_cast<f32x4*>(a.dk + off) = dk + dE * bv;
            *reinterpret_cast<f32x4*>(a.dv + off) = dU * wv;
            const f32x4 dbv = dE * kv * bd, dwv = dU * vv * wd;
            if (a.bw == 1)
                sRb[e4] = (dbv[0] + dbv[1]) + (dbv[2] + dbv[3]);
            else
                *reinterpret_cast<f32x4*>(a.db + off) = dbv;
            if (a.ww == 1)
                sRw[e4] = (dwv[0] + dwv[1]) + (dwv[2] + dwv[3]);
            else
                *reinterpret_cast<f32x4*>(a.dw + off) = dwv;
        }
    }
    lds_barrier();
    // width-1 erase / write gate: this group's DC channels summed per token
    // in channel order (the groups are added in order by bwd_gate_sum, so
    // the result does not depend on scheduling)
    if ((a.bw == 1 || a.ww == 1) && tid < rc.L) {
        constexpr int NP4 = DC / 4;
        float sb = 0.f, sw = 0.f;
#pragma unroll
        for (int j = 0; j < NP4; ++j) {
            sb += sRb[tid * NP4 + j];
            sw += sRw[tid * NP4 + j];
        }
        const size_t gi = ((size_t)r * C + tid) * (D / DC) + i0 / DC;
        const size_t np = (size_t)a.nrec * C * (D / DC);
        if (a.bw == 1)
            a.ws[a.L.GP + gi] = sb;
        if (a.ww == 1)
            a.ws[a.L.GP + np + gi] = sw;
    }
    // dg: reverse cumulative sum over the chunk, per channel: each thread
    // scans its RPT tokens, then adds the later row groups' totals
    float vg[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        vg[m] = sdG[(t0 + m) * LC + il];
#pragma unroll
    for (int m = RPT - 2; m >= 0; --m)
        vg[m] += vg[m + 1];
    lds_barrier();                       // every thread has its dG rows
    sdG[rg * LC + il] = vg[0];
    lds_barrier();
    {
        float off = 0.f;
        for (int g2 = rg + 1; g2 < NRG; ++g2)
            off += sdG[g2 * LC + il];
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            vg[m] += off;
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int t = t0 + m;
        if (t >= rc.L)
            continue;
        const int64_t row = rc.row0 + (int64_t)t * a.H;
        float dgv = vg[m];
        if (a.pro & GDR2_PROLOGUE_GATES)      // d/dx[-softplus(x)] = -sigmoid(x)
            dgv *= -bsigm(a.g[a.gw == 1 ? row : row * D + i]);
        if (a.gw == 1)
            sRg[t * DC + il] = dgv;
        else
            a.dg[row * D + i] = dgv;
    }
    if (a.gw == 1) {
        // width-1 decay: this group's channels summed per token in order
        lds_barrier();
        if (tid < rc.L) {
            float sg = 0.f;
            for (int j = 0; j < DC; ++j)
                sg += sRg[tid * DC + j];
            const size_t np = (size_t)a.nrec * C * (D / DC);
            a.ws[a.L.GP + 2 * np + ((size_t)r * C + tid) * (D / DC) + i0 / DC] = sg;
        }
    }
}

// Width-1 gate gradients: the partial sums the D/DC decay workgroups of a
// chunk left per token, added in group order (one thread per token).
template <int D>
__global__ __launch_bounds__(NTB) void bwd_gate_sum_kernel(BwdArgs a)
{
    constexpr int C = BC, NG = D / DC;
    const int64_t e = (int64_t)blockIdx.x * NTB + threadIdx.x;
    const int64_t r = e / C;
    const int t = (int)(e - r * C);
    if (r >= a.nrec)
        return;
    const Rec rc = rec_of(r, a.NC, a.T, a.H);
    if (t >= rc.L)
        return;
    const int64_t row = rc.row0 + (int64_t)t * a.H;
    const size_t np = (size_t)a.nrec * C * NG;
    const float* gp = a.ws + a.L.GP + (size_t)e * NG;
    float* outs[3] = {a.bw == 1 ? a.db : nullptr, a.ww == 1 ? a.dw : nullptr, a.gw == 1 ? a.dg : nullptr};
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        if (!outs[x])
            continue;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NG; ++j)
            s += gp[x * np + j];
        outs[x][row] = s;
    }
}

// The prologue's normalisation, backwards: with y = x r, r = (|x|^2 + eps)^-1/2,
// dx = r (dy - y (y . dy)), in place on dq and dk.  A row (token, head) of D
// channels is D/4 consecutive threads, 4 channels each.
template <typename E, int D>
__global__ __launch_bounds__(NTB) void bwd_norm_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                       float* __restrict__ dq, float* __restrict__ dk,
                                                       int64_t rows)
{
    constexpr int TPR = D / 4, RPB = NTB / TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = 4 * (threadIdx.x % TPR);
    const bool ok = row < rows;
    const int64_t off = (ok ? row : 0) * D + c;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const E* x = which == 0 ? q : k;
        float* dx = which == 0 ? dq : dk;
        const f32x4 xv = load4(x + off);
        const f32x4 dy = ok ? *reinterpret_cast<const f32x4*>(dx + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        float ss = xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3];
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1)
            ss += __shfl_xor(ss, m);
        const float rn = rsqrtf(ss + kNormEps);
        const f32x4 y = xv * rn;
        float yd = y[0] * dy[0] + y[1] * dy[1] + y[2] * dy[2] + y[3] * dy[3];
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1)
            yd += __shfl_xor(yd, m);
        if (ok)
            *reinterpret_cast<f32x4*>(dx + off) = rn * (dy - y * yd);
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

// bwd_prep for one gate-width mix (more than 64 KiB of dynamic LDS must be
// requested per kernel)
template <typename E, int D, int MIX>
hipError_t launch_prep(int64_t grid, size_t lds, hipStream_t s, const BwdArgs& a)
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_prep_kernel<E, D, MIX>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((bwd_prep_kernel<E, D, MIX>), dim3((unsigned)grid), dim3(NTP), lds, s, a);
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
    a.bw = x.b_width; a.ww = x.w_width; a.gw = x.g_width; a.pro = x.prologue;
    a.T = x.T; a.H = x.H; a.NC = cdiv(x.T, C);
    a.nbh = x.B * x.H;
    segment_plan(x.algo, a.NC, a.nbh * ScanShape<E, D>::NS, &a.nseg, &a.seg_len);
    const bool narrow = a.bw == 1 || a.ww == 1 || a.gw == 1;
    a.L = bwd_layout(x.B, x.H, x.T, D, ScanFrags<E, D>::REC, a.nseg, narrow, sizeof(E) == 4);
    a.nrec = a.L.nrec;
    a.ws = static_cast<float*>(x.workspace);
    const int64_t nrec = a.nrec, rows = x.B * x.T * x.H;
    hipError_t e;

    const size_t lds_prep = BwdPrepShape<D>::SMEM;
    const size_t lds_decay = (size_t)(2 * C * LPC + 5 * C * LC + DC) * 4;
    // more than 64 KiB of dynamic LDS must be requested per kernel
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_decay_kernel<E, D>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_decay)) != hipSuccess)
        return e;
    if constexpr (sizeof(E) == 2) {
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_sgrad_bf16_kernel<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)SgradShape<D>::SMEM)) !=
            hipSuccess)
            return e;
    }

    {
        // persistent, one workgroup per compute unit (its LDS allows no more)
        const int64_t grid = std::min<int64_t>(nrec, (int64_t)device_cu_count());
        switch ((a.bw == 1 ? 4 : 0) | (a.ww == 1 ? 2 : 0) | (a.gw == 1 ? 1 : 0)) {
        case 0: e = launch_prep<E, D, 0>(grid, lds_prep, s, a); break;
        case 1: e = launch_prep<E, D, 1>(grid, lds_prep, s, a); break;
        case 2: e = launch_prep<E, D, 2>(grid, lds_prep, s, a); break;
        case 3: e = launch_prep<E, D, 3>(grid, lds_prep, s, a); break;
        case 4: e = launch_prep<E, D, 4>(grid, lds_prep, s, a); break;
        case 5: e = launch_prep<E, D, 5>(grid, lds_prep, s, a); break;
        case 6: e = launch_prep<E, D, 6>(grid, lds_prep, s, a); break;
        default: e = launch_prep<E, D, 7>(grid, lds_prep, s, a); break;
        }
        if (e != hipSuccess) return e;
    }
    if constexpr (sizeof(E) == 4) {   // the fp32 state products read dO as zero-padded records
        hipLaunchKernelGGL((bwd_dout_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (ScanFrags<E, D>::HAS_O) {   // bf16: the scan reads the dO rows itself
        hipLaunchKernelGGL((bwd_frag_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.nseg > 1) {
        const int64_t groups = cdiv(a.nbh * (a.nseg - 1), 8) * 8 * 2 * ScanShape<E, D>::NS;
        hipLaunchKernelGGL((bwd_span_kernel<E, D>), dim3((unsigned)groups), dim3(NTB), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (a.nseg > 2 && (e = launch_span_fold(a.ws + a.L.span, a.nbh, a.nseg, D, s)) != hipSuccess) return e;
    }
    {
        const int64_t groups = cdiv(a.nbh * a.nseg, 8) * 8 * ScanShape<E, D>::NS;
        hipLaunchKernelGGL((bwd_scan_kernel<E, D>), dim3((unsigned)groups), dim3(NTB), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    if constexpr (sizeof(E) == 2) {
        // persistent, one workgroup per compute unit (its LDS allows no more)
        const int64_t grid = std::min<int64_t>(nrec, (int64_t)device_cu_count());
        hipLaunchKernelGGL((bwd_sgrad_bf16_kernel<D>), dim3((unsigned)grid), dim3(SgradShape<D>::NTH),
                           SgradShape<D>::SMEM, s, a);
    } else {
        hipLaunchKernelGGL((bwd_sgrad_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // bf16: dM is formed in bwd_sgrad_bf16, dU and dE~ in bwd_decay
    if constexpr (sizeof(E) == 4) {
        hipLaunchKernelGGL((bwd_xgrad_kernel<E, D>), dim3((unsigned)nrec), dim3(NTB), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    hipLaunchKernelGGL((bwd_decay_kernel<E, D>), dim3((unsigned)(cdiv(nrec, 8) * 8 * (D / DC))), dim3(NTB), lds_decay, s,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (narrow) {
        hipLaunchKernelGGL((bwd_gate_sum_kernel<D>), dim3((unsigned)cdiv(nrec * C, NTB)), dim3(NTB), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.pro & GDR2_PROLOGUE_NORM_QK) {
        constexpr int RPB = NTB / (D / 4);
        hipLaunchKernelGGL((bwd_norm_kernel<E, D>), dim3((unsigned)cdiv(rows, RPB)), dim3(NTB), 0, s,
                           (const E*)x.q, (const E*)x.k, x.dq, x.dk, rows);
    }
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(const gdr2_bwd_args& a)
{
    if (a.B * a.H * a.T == 0)
        return 0;
    const size_t esz = a.dtype == GDR2_BF16 ? 2 : 4;
    const size_t rec = (size_t)((esz == 4 ? 4 : 3) * BC * a.Dk + BC * BC) * esz;   // ScanFrags<E, D>::REC
    int64_t nseg, len;
    segment_plan(a.algo, cdiv(a.T, BC), a.B * a.H * (a.Dk / 64), &nseg, &len);
    const bool narrow = a.b_width == 1 || a.w_width == 1 || a.g_width == 1;
    return bwd_layout(a.B, a.H, a.T, (int)a.Dk, rec, nseg, narrow, esz == 4).total;
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
