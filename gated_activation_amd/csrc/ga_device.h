// Device-side building blocks shared by the gated-activation kernels (gfx950,
// wave64): element-type traits for 16-byte vectors, the wavefront and
// workgroup sum, and the fp32 activation functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// 16-byte global loads and stores.  Every input byte is read once and every
// output byte written once, so the nontemporal forms (streaming hint on the
// cache policy) are the default; NT = false gives the plain forms.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4 *p) {
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return uint4{v.x, v.y, v.z, v.w};
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st16(uint4 *p, const uint4 &v) {
    if constexpr (NT) {
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(p));
    } else {
        *p = v;
    }
}

// The same 16 bytes at any address aligned to the element size.  gfx950 runs
// global memory in unaligned-access mode; the compiler emits one 16-byte
// access for these (the type only lowers the alignment it may assume).
typedef u32x4 u32x4_a2 __attribute__((aligned(2)));

template <typename S>
__device__ __forceinline__ uint4 ldu16(const S *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a2 *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}

template <typename S>
__device__ __forceinline__ void stu16(S *p, const uint4 &v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_a2 *>(p));
}

// ---------------------------------------------------------------------------
// Element traits.  A 16-byte vector holds PER16 elements; unpack widens them
// to fp32, pack rounds fp32 to the element type (ties to even; gfx950 has a
// two-lane convert for both 16-bit types).
// ---------------------------------------------------------------------------
template <int DT> struct Elem;

template <> struct Elem<DT_F32> {
    using storage = uint32_t;
    static constexpr int PER16 = 4;
    static __device__ __forceinline__ void unpack(const uint4 &v, float (&f)[4]) {
        f[0] = __builtin_bit_cast(float, v.x);
        f[1] = __builtin_bit_cast(float, v.y);
        f[2] = __builtin_bit_cast(float, v.z);
        f[3] = __builtin_bit_cast(float, v.w);
    }
    static __device__ __forceinline__ uint4 pack(const float (&f)[4]) {
        return uint4{__builtin_bit_cast(uint32_t, f[0]), __builtin_bit_cast(uint32_t, f[1]),
                     __builtin_bit_cast(uint32_t, f[2]), __builtin_bit_cast(uint32_t, f[3])};
    }
    static __device__ __forceinline__ float to_f32(storage s) { return __builtin_bit_cast(float, s); }
    static __device__ __forceinline__ storage from_f32(float f) { return __builtin_bit_cast(uint32_t, f); }
    // The value an fp32 tensor holds: the number itself.
    static __device__ __forceinline__ float round(float f) { return f; }
};

template <> struct Elem<DT_BF16> {
    using storage = uint16_t;
    static constexpr int PER16 = 8;
    // bf16 is the top half of an fp32: widening is a shift / mask.
    static __device__ __forceinline__ void unpack2(uint32_t w, float &lo, float &hi) {
        lo = __builtin_bit_cast(float, w << 16);
        hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    }
    static __device__ __forceinline__ void unpack(const uint4 &v, float (&f)[8]) {
        unpack2(v.x, f[0], f[1]);
        unpack2(v.y, f[2], f[3]);
        unpack2(v.z, f[4], f[5]);
        unpack2(v.w, f[6], f[7]);
    }
    static __device__ __forceinline__ uint4 pack(const float (&f)[8]) {
        return uint4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
    }
    static __device__ __forceinline__ float to_f32(storage s) {
        return __builtin_bit_cast(float, (uint32_t)s << 16);
    }
    static __device__ __forceinline__ storage from_f32(float f) {
        return (storage)(pack2(f, 0.0f) & 0xFFFFu);
    }
    // The value a bf16 tensor would hold: round to nearest even and widen.
    static __device__ __forceinline__ float round(float f) {
        return __builtin_bit_cast(float, pack2(f, 0.0f) << 16);
    }
};

template <> struct Elem<DT_F16> {
    using storage = uint16_t;
    static constexpr int PER16 = 8;
    static __device__ __forceinline__ void unpack2(uint32_t w, float &lo, float &hi) {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        lo = (float)h.x;
        hi = (float)h.y;
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
    }
    static __device__ __forceinline__ void unpack(const uint4 &v, float (&f)[8]) {
        unpack2(v.x, f[0], f[1]);
        unpack2(v.y, f[2], f[3]);
        unpack2(v.z, f[4], f[5]);
        unpack2(v.w, f[6], f[7]);
    }
    static __device__ __forceinline__ uint4 pack(const float (&f)[8]) {
        return uint4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
    }
    static __device__ __forceinline__ float to_f32(storage s) {
        return (float)__builtin_bit_cast(_Float16, s);
    }
    static __device__ __forceinline__ storage from_f32(float f) {
        return (storage)(pack2(f, 0.0f) & 0xFFFFu);
    }
    // The value an fp16 tensor would hold: round to nearest even and widen.
    static __device__ __forceinline__ float round(float f) { return (float)(_Float16)f; }
};

// ---------------------------------------------------------------------------
// Reductions.  The wavefront sum pairs lanes symmetrically (xor 1, xor 2,
// half-row mirror, row mirror: all DPP, fused into the adds), so every lane of
// a 16-lane row holds the same row sum; the four row sums are then read into
// scalar registers and added in a fixed order.  The result is bit-identical on
// every lane and does not depend on scheduling.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v);  // row_half_mirror
    v += dpp_move<0x140>(v);  // row_mirror
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Sum over a workgroup of WAVES wavefronts.  `slots` is LDS of WAVES floats
// that no other thread reads or writes for the rest of this workgroup's
// lifetime (each call site passes its own); wave partials are combined in
// wave order, so the result is identical on every thread.
template <int WAVES>
__device__ __forceinline__ float block_sum(float v, float *slots) {
    v = wave_sum(v);
    if constexpr (WAVES == 1) {
        return v;
    } else {
        if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
        __syncthreads();
        float t = slots[0];
#pragma unroll
        for (int i = 1; i < WAVES; ++i) t += slots[i];
        return t;
    }
}

// ---------------------------------------------------------------------------
// Activations in fp32.
//
// tanh GELU: 0.5 s (1 + tanh w) = s / (1 + e^(-2w)) with
// w = sqrt(2/pi) (s + 0.044715 s^3).  In base 2, e^(-2w) = 2^(-s (A + B s^2)),
// A = 2 sqrt(2/pi) / ln 2, B = 0.044715 A.  For s >= 0 the exponent is <= 0
// and at s = 0 the result is exactly 0; for s << 0 the power overflows to +inf
// and the result is -0, the function's limit.
// ---------------------------------------------------------------------------
constexpr float GELU_A = 2.302208198144325f;
constexpr float GELU_B = 0.1029432395800235f;
constexpr float LOG2_E = 1.4426950408889634f;

__device__ __forceinline__ float gelu_tanh(float s) {
    const float t = s * __builtin_fmaf(GELU_B, s * s, GELU_A);
    return s * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t));
}

// erfc(a) for a >= 0 by Abramowitz & Stegun 7.1.26 (Hastings' rational
// approximation): erfc(a) = t (c1 + t (c2 + t (c3 + t (c4 + t c5)))) e^(-a^2),
// t = 1 / (1 + p a), absolute error below 1.5e-7.
__device__ __forceinline__ float erfc_nonneg(float a) {
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, a, 1.0f));
    float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
    poly = __builtin_fmaf(poly, t, 1.421413741f);
    poly = __builtin_fmaf(poly, t, -0.284496736f);
    poly = __builtin_fmaf(poly, t, 0.254829592f);
    return poly * t * __builtin_amdgcn_exp2f(-a * a * LOG2_E);
}

// Exact GELU, x Phi(x) = 0.5 x erfc(-x / sqrt 2).  With a = |x| / sqrt 2:
// x < 0 gives 0.5 x erfc(a) (no cancellation), x >= 0 gives
// x (1 - 0.5 erfc(a)) since erfc(-a) = 2 - erfc(a).
__device__ __forceinline__ float gelu_erf(float x) {
    const float c = erfc_nonneg(__builtin_fabsf(x) * 0.70710678118654752f);
    return x < 0.0f ? 0.5f * x * c : x * __builtin_fmaf(-0.5f, c, 1.0f);
}

// silu(x) = x / (1 + e^-x); for x << 0 the power overflows to +inf and the
// result is -0, for x >> 0 it underflows to 0 and the result is x.
__device__ __forceinline__ float silu(float x) {
    const float e = __builtin_amdgcn_exp2f(-x * LOG2_E);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Row mean and variance from the workgroup sums.
//
// The default form avoids IEEE division: r = 1/n from the hardware reciprocal
// (within 1 ulp), q0 = sum * r is then within 1.5 ulp of sum / n, so the
// residual sum - q0 * n is exact in one fma, and q0 + residual * r lands on
// sum / n itself whenever that quotient is a float.  A row of one repeated
// value therefore gets exactly that value as its mean, hence a variance of
// exactly 0; any other mean is within about half an ulp.  The variance is
// the sum times r (within 1.5 ulp) and the std the hardware square root
// (within 1 ulp): both far inside the error of the fp32 sums themselves.
// The round-trip form keeps IEEE division and square root, as the tensor
// composition it reproduces does.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float div_count(float sum, float n, float r) {
    const float q0 = sum * r;
    return __builtin_fmaf(__builtin_fmaf(-q0, n, sum), r, q0);
}

template <bool RT>
__device__ __forceinline__ float row_mean(float sum, float n) {
    if constexpr (RT) {
        return sum / n;
    } else {
        return div_count(sum, n, __builtin_amdgcn_rcpf(n));
    }
}

template <bool RT>
__device__ __forceinline__ float row_var(float sq_sum, float n) {
    if constexpr (RT) {
        return sq_sum / n;
    } else {
        return sq_sum * __builtin_amdgcn_rcpf(n);
    }
}

// The cutoff from the row's fp32 mean and variance.  RT (round-trip form):
// every intermediate is rounded to the element type as a tensor of that type
// would hold it -- mean, std, z, z * std, mean + z * std.  Contraction is off
// there: the compiler narrows these fp16 steps to half precision and would
// otherwise fuse z * std + mean into one fma, dropping a rounding.
template <typename E, bool RT>
__device__ __forceinline__ float sparse_cutoff(float mean, float var, float z) {
    if constexpr (RT) {
#pragma clang fp contract(off)
        const float zs = E::round(E::round(z) * E::round(__builtin_sqrtf(var)));
        return E::round(E::round(mean) + zs);
    } else {
        return __builtin_fmaf(z, __builtin_amdgcn_sqrtf(var), mean);
    }
}

// gelu_tanh(relu(g - cut)) * up; RT rounds g - cut and the GELU output to the
// element type (the final rounding is the store's).
template <typename E, bool RT>
__device__ __forceinline__ float sparse_apply(float g, float cut, float up) {
    if constexpr (RT) {
#pragma clang fp contract(off)
        const float s = __builtin_fmaxf(E::round(g - cut), 0.0f);
        return E::round(gelu_tanh(s)) * up;
    } else {
        return gelu_tanh(__builtin_fmaxf(g - cut, 0.0f)) * up;
    }
}

// Chan, Golub and LeVeque's pairwise update: fold the partial statistics
// (n_b, mean_b, M2_b) of one chunk of a row into (n_a, mean_a, M2_a), where
// M2 is the sum of squared deviations from the chunk's own mean.
__device__ __forceinline__ void chan_combine(float &n_a, float &mean_a, float &m2_a, float n_b,
                                             float mean_b, float m2_b) {
    const float n = n_a + n_b;
    const float delta = mean_b - mean_a;
    const float w = n_b * __builtin_amdgcn_rcpf(n);
    mean_a = __builtin_fmaf(delta, w, mean_a);
    m2_a = m2_a + m2_b + delta * delta * n_a * w;
    n_a = n;
}

__device__ __forceinline__ int32_t clamp_live(const int32_t *live, int32_t rows) {
    const int32_t n = *live;
    return n < 0 ? 0 : (n > rows ? rows : n);
}

}  // namespace ga
