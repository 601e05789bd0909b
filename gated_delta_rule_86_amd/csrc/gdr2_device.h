// gdr2_device.h -- small device helpers shared by the gfx950 kernels:
// element loads/stores for fp32 and bf16, exp2, and the MFMA tile wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr2 {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// v_cvt_pk_bf16_f32: round to nearest even.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// The value of the lane whose index differs in bit M (M = 1 or 2) within
// its group of four lanes (a DPP quad permutation).
template <int M>
__device__ __forceinline__ float dpp_quad_xor(float v)
{
    static_assert(M == 1 || M == 2, "quad lanes");
    constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
}

// 4x4 transpose across the four lanes of a quad (two exchange rounds): lane
// j = lane % 4 holds v[i] = X[i][j] on entry and X[j][c] in v[c] on return.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 v, int j)
{
    const bool b1 = (j >> 1) & 1, b0 = j & 1;
    float y0 = dpp_quad_xor<2>(b1 ? v[0] : v[2]), y1 = dpp_quad_xor<2>(b1 ? v[1] : v[3]);
    if (b1) {
        v[0] = y0;
        v[1] = y1;
    } else {
        v[2] = y0;
        v[3] = y1;
    }
    y0 = dpp_quad_xor<1>(b0 ? v[0] : v[1]);
    y1 = dpp_quad_xor<1>(b0 ? v[2] : v[3]);
    if (b0) {
        v[0] = y0;
        v[2] = y1;
    } else {
        v[1] = y0;
        v[3] = y1;
    }
    return v;
}

// 2^x on the transcendental unit (v_exp_f32).  Inputs here are <= 0 or
// bounded; large negative inputs flush to 0, which is the intended limit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load 4 consecutive elements (16-byte or 8-byte aligned) as fp32.
__device__ __forceinline__ f32x4 load4(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ f32x4 load4(const bf16* p) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

__device__ __forceinline__ void store4(float* p, f32x4 v) {
    *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0];
    o[1] = (bf16)v[1];
    o[2] = (bf16)v[2];
    o[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4*>(p) = o;
}

// Streaming (non-temporal) 16-byte access for data touched exactly once.
__device__ __forceinline__ f32x4 load4_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store4_nt(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

}  // namespace gdr2

namespace gdr2 {

// ---------------------------------------------------------------------------
// MFMA tiles.  Every product below is a 16 x 16 output tile held in the
// accumulator layout of the 16x16 MFMA family: lane l owns rows 4*(l/16)+i
// (i = 0..3) of column l%16.
//
// The contraction index k of one MFMA may be assigned to (lane group, slot)
// in any order as long as the A and B operands agree, because the hardware
// sums over it.  We pick the order that makes an accumulator tile directly
// usable as a B operand: lane group gq = l/16 holds k = 4gq..4gq+3 of each
// 16-row k-tile.  For bf16 (v_mfma_f32_16x16x32_bf16, 8 k per lane) one MFMA
// covers two 16-row k-tiles: slots 0..3 from the first, 4..7 from the second.
// For fp32 (v_mfma_f32_16x16x4f32, 1 k per lane) one 16-row k-tile takes four
// MFMAs, slot i of every lane in the i-th.
//
// An A operand stored row-major in memory (k contiguous, leading dimension
// ld) is read by lane l from row l%16, columns 4gq.. and (bf16) 16+4gq...
// A B operand stored with its n index as the row (k contiguous) is read the
// same way.
// ---------------------------------------------------------------------------
template <typename E> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int KB = 32;   // k per step
    static constexpr int KT = 2;    // 16-row k-tiles per step
    typedef bf16x8 Frag;

    static __device__ __forceinline__ Frag pack(f32x4 lo, f32x4 hi) {
        Frag f;
        f[0] = (bf16)lo[0]; f[1] = (bf16)lo[1]; f[2] = (bf16)lo[2]; f[3] = (bf16)lo[3];
        f[4] = (bf16)hi[0]; f[5] = (bf16)hi[1]; f[6] = (bf16)hi[2]; f[7] = (bf16)hi[3];
        return f;
    }
    // p -> element (row0, k0) of a row-major bf16 matrix.
    static __device__ __forceinline__ Frag load(const bf16* p, int ld, int lane) {
        const bf16* s = p + (lane & 15) * ld + 4 * (lane >> 4);
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(s);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(s + 16);
        Frag f;
        f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
        f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
        return f;
    }
    // Fragment from storage in MFMA k-order (see perm_chunk): one 16-byte read.
    static __device__ __forceinline__ Frag load_perm(const bf16* p, int ld, int lane) {
        return *reinterpret_cast<const bf16x8*>(p + (lane & 15) * ld + 8 * (lane >> 4));
    }
    // Same, from fp32 storage (rounded to bf16).
    static __device__ __forceinline__ Frag load(const float* p, int ld, int lane) {
        const float* s = p + (lane & 15) * ld + 4 * (lane >> 4);
        return pack(*reinterpret_cast<const f32x4*>(s), *reinterpret_cast<const f32x4*>(s + 16));
    }
    // bf16 storage scaled elementwise along k by fp32 factors f[k] (f -> k0).
    static __device__ __forceinline__ Frag load_scaled(const bf16* p, int ld, const float* f, int lane) {
        const int c = 4 * (lane >> 4);
        const bf16* s = p + (lane & 15) * ld + c;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(s);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(s + 16);
        const f32x4 flo = *reinterpret_cast<const f32x4*>(f + c);
        const f32x4 fhi = *reinterpret_cast<const f32x4*>(f + c + 16);
        f32x4 a = {(float)lo[0] * flo[0], (float)lo[1] * flo[1], (float)lo[2] * flo[2], (float)lo[3] * flo[3]};
        f32x4 b = {(float)hi[0] * fhi[0], (float)hi[1] * fhi[1], (float)hi[2] * fhi[2], (float)hi[3] * fhi[3]};
        return pack(a, b);
    }
    // B operand from a matrix stored k-major (row = k, n contiguous): lane l
    // gathers column l%16 at rows 4gq..4gq+3 and 16+4gq..16+4gq+3.
    static __device__ __forceinline__ Frag load_kn(const bf16* p, int ld, int lane) {
        const bf16* s = p + 4 * (lane >> 4) * ld + (lane & 15);
        Frag f;
        f[0] = s[0]; f[1] = s[ld]; f[2] = s[2 * ld]; f[3] = s[3 * ld];
        f[4] = s[16 * ld]; f[5] = s[17 * ld]; f[6] = s[18 * ld]; f[7] = s[19 * ld];
        return f;
    }
    // B operand from accumulator tiles t[0], t[1] (two consecutive k-tiles).
    static __device__ __forceinline__ Frag from_acc(const f32x4* t) { return pack(t[0], t[1]); }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KB = 16;
    static constexpr int KT = 1;
    typedef f32x4 Frag;

    static __device__ __forceinline__ Frag load(const float* p, int ld, int lane) {
        return *reinterpret_cast<const f32x4*>(p + (lane & 15) * ld + 4 * (lane >> 4));
    }
    static __device__ __forceinline__ Frag load_perm(const float* p, int ld, int lane) {
        return load(p, ld, lane);
    }
    static __device__ __forceinline__ Frag load_scaled(const float* p, int ld, const float* f, int lane) {
        const int c = 4 * (lane >> 4);
        return *reinterpret_cast<const f32x4*>(p + (lane & 15) * ld + c) *
               *reinterpret_cast<const f32x4*>(f + c);
    }
    static __device__ __forceinline__ Frag load_kn(const float* p, int ld, int lane) {
        const float* s = p + 4 * (lane >> 4) * ld + (lane & 15);
        return Frag{s[0], s[ld], s[2 * ld], s[3 * ld]};
    }
    static __device__ __forceinline__ Frag from_acc(const f32x4* t) { return t[0]; }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
};

}  // namespace gdr2
