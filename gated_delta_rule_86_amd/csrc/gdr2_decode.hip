// gdr2_decode.hip -- one batched recurrent decode step (pure recurrent mode of
// the page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트 분리",
// section "개요"; the update of section "Gated Delta Rule-2 업데이트 수식").
//
// Per state (sequence n, head h), with d = exp(g), e = b*k, u = w*v:
//   r   = (D S)^T e            = sum_i d_i e_i S[i,:]
//   S'  = D S + k (u - r)^T
//   o   = S'^T q               = sum_i d_i q_i S[i,:] + (q.k) (u - r)
// The last line is the same readout expanded, so S is streamed from HBM once
// (read), both column reductions are formed from the registers that hold it,
// and S' is written back in place: 2 x 4 x Dk x Dv bytes of state traffic,
// the whole cost of the step.  The state stays fp32.
//
// One 256-thread workgroup per state, four or five resident per CU (see
// decode_lds_pad).  Thread t owns the 4-column group
// cg = t % (Dv/4) and the rows rg, rg + RG, ... with rg = t / (Dv/4): every
// wave reads or writes whole 512-byte rows with 16-byte lanes, so each state
// tile moves in fully coalesced dwordx4 transactions.
#include "gdr2_device.h"
#include "gdr2_internal.h"

namespace gdr2 {

// Prologue activations (logistic sigmoid; log-decay -softplus(x) = log sigmoid(-x)).
__device__ __forceinline__ float dec_sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float dec_neg_softplus(float x) { return -(fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)))); }

// PRO: the input prologue (gdr2_prologue bits in `pro`) is applied to the
// token vectors before the update.
template <int D, typename T, bool PRO>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ b, const T* __restrict__ w, const float* __restrict__ g,
    int bw, int ww, int gw, float* __restrict__ state, T* __restrict__ o, int pro)
{
    constexpr int CG = D / 4;       // column groups (4 fp32 each)
    constexpr int RG = 256 / CG;    // row groups
    constexpr int RPT = D / RG;     // rows per thread
    constexpr int NW = 256 / 64;    // waves

    const int64_t s = blockIdx.x;   // state index n*H + h
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    float* S = state + s * (int64_t)D * D;

    // 1) Issue every state load first; nothing below depends on them until
    //    the reductions.
    f32x4 st[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        st[r] = load4_nt(S + (int64_t)(rg + RG * r) * D + cg * 4);

    // 2) Token vectors (one token per state) into LDS, in fp32.
    __shared__ float s_d[D], s_de[D], s_dq[D], s_k[D], s_u[D];
    __shared__ float s_qk[NW];
    __shared__ f32x4 s_red_r[NW][CG], s_red_a[NW][CG];
    float qk = 0.f;
    float rk = 1.f, rq = 1.f;                 // prologue: 1/|k|, 1/|q|
    if constexpr (PRO) {
        if (pro & GDR2_PROLOGUE_NORM_QK) {
            __shared__ float s_ss[2][NW];
            float sk = 0.f, sq = 0.f;
            if (tid < D) {
                const float ki = to_f32(k[s * D + tid]), qi = to_f32(q[s * D + tid]);
                sk = ki * ki;
                sq = qi * qi;
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                sk += __shfl_xor(sk, off);
                sq += __shfl_xor(sq, off);
            }
            if ((tid & 63) == 0) {
                s_ss[0][tid >> 6] = sk;
                s_ss[1][tid >> 6] = sq;
            }
            __syncthreads();
            sk = sq = 0.f;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                sk += s_ss[0][wv];
                sq += s_ss[1][wv];
            }
            rk = rsqrtf(sk + 1e-6f);
            rq = rsqrtf(sq + 1e-6f);
        }
    }
    if (tid < D) {
        const int i = tid;
        float gi = g[s * gw + (gw == 1 ? 0 : i)];
        float bi = to_f32(b[s * bw + (bw == 1 ? 0 : i)]);
        float wi = to_f32(w[s * ww + (ww == 1 ? 0 : i)]);
        if constexpr (PRO) {
            if (pro & GDR2_PROLOGUE_GATES) {
                gi = dec_neg_softplus(gi);
                bi = dec_sigm(bi);
                wi = dec_sigm(wi);
            }
        }
        const float di = fast_exp2(gi * kLog2e);
        const float ki = to_f32(k[s * D + i]) * rk;
        const float qi = to_f32(q[s * D + i]) * rq;
        s_d[i] = di;
        s_de[i] = di * bi * ki;
        s_dq[i] = di * qi;
        s_k[i] = ki;
        const float vi = to_f32(v[s * D + i]);
        s_u[i] = wi * vi;
        qk = qi * ki;
    }
    // q.k: reduce inside each wave, then across waves through LDS.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        qk += __shfl_xor(qk, off);
    if ((tid & 63) == 0)
        s_qk[tid >> 6] = qk;
    __syncthreads();

    // 3) Partial column reductions over this thread's rows.
    f32x4 racc = {0.f, 0.f, 0.f, 0.f}, aacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + RG * r;
        racc += s_de[i] * st[r];
        aacc += s_dq[i] * st[r];
    }
    // 4) Across the row groups of one wave (lanes that share cg) ...
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            racc[c] += __shfl_xor(racc[c], off);
            aacc[c] += __shfl_xor(aacc[c], off);
        }
    }
    const int wave = tid >> 6, lane = tid & 63;
    if (lane < CG) {
        s_red_r[wave][cg] = racc;
        s_red_a[wave][cg] = aacc;
    }
    __syncthreads();
    // ... then across waves.
    f32x4 rj = s_red_r[0][cg];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv)
        rj += s_red_r[wv][cg];
    const f32x4 uj = *reinterpret_cast<const f32x4*>(&s_u[cg * 4]);
    const f32x4 du = uj - rj;

    // 5) S' = D S + k (u - r)^T, written back in place.
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + RG * r;
        const f32x4 nv = s_d[i] * st[r] + s_k[i] * du;
        store4_nt(S + (int64_t)(rg + RG * r) * D + cg * 4, nv);
    }

    // 6) o = (D S)^T q + (q.k)(u - r), by the first row group.
    if (rg == 0) {
        f32x4 aj = s_red_a[0][cg];
#pragma unroll
        for (int wv = 1; wv < NW; ++wv)
            aj += s_red_a[wv][cg];
        float qk_all = 0.f;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv)
            qk_all += s_qk[wv];
        store4(o + s * D + cg * 4, aj + qk_all * du);
    }
}

// Dynamic LDS the launch asks for (and leaves unused) to hold the kernel to
// four resident workgroups per CU instead of the five its registers allow at
// d = 128 (90-94 VGPRs per lane): taken when the n states then fill whole
// rounds of workgroups over the CUs better than at five, so the last round
// does not run on a partly idle chip (256 x 16 states on 256 CUs: exactly
// four rounds at four per CU, against 3.2 at five).
static size_t decode_lds_pad(int64_t n, int D)
{
    constexpr size_t kPad = 32768;   // with the kernel's ~6.7 KB: 4 x 39.5 KB fit in 160 KB, 5 do not
    if (D != 128)
        return 0;
    const int64_t cus = device_cu_count();
    if (n <= 4 * cus)
        return 0;                    // one round either way
    auto fill = [&](int64_t per_cu) {
        const int64_t slots = cus * per_cu, rounds = (n + slots - 1) / slots;
        return (double)n / (double)(rounds * slots);
    };
    return fill(4) > fill(5) ? kPad : 0;
}

template <int D, typename T>
static hipError_t launch_decode_t(const gdr2_decode_args& a, hipStream_t stream)
{
    const int64_t n = a.N * a.H;
    const size_t pad = decode_lds_pad(n, D);
    if (a.prologue != 0)
        hipLaunchKernelGGL((decode_step_kernel<D, T, true>), dim3((unsigned)n), dim3(256), pad, stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.b,
                           (const T*)a.w, a.g, a.b_width, a.w_width, a.g_width, a.state,
                           (T*)a.o, a.prologue);
    else
        hipLaunchKernelGGL((decode_step_kernel<D, T, false>), dim3((unsigned)n), dim3(256), pad, stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.b,
                           (const T*)a.w, a.g, a.b_width, a.w_width, a.g_width, a.state,
                           (T*)a.o, 0);
    return hipGetLastError();
}

hipError_t launch_decode(const gdr2_decode_args& a, hipStream_t stream)
{
    if (a.Dk == 128)
        return a.dtype == GDR2_BF16 ? launch_decode_t<128, bf16>(a, stream)
                                    : launch_decode_t<128, float>(a, stream);
    return a.dtype == GDR2_BF16 ? launch_decode_t<64, bf16>(a, stream)
                                : launch_decode_t<64, float>(a, stream);
}

}  // namespace gdr2
