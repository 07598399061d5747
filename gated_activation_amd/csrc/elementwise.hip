// Elementwise activations for gfx950: silu_and_mul_bounded, gelu_and_mul
// (tanh and erf forms) and the bounded squared ReLU, plus the
// streaming-ceiling kernel.
//
// silu_and_mul_bounded (Megatron-LM PR 6328, "Size MoE activation kernel grid
// to the row count", section What changed and why): silu(gate) * up over the
// live rows of a capture-sized MoE buffer in[M, 2d].  The live count sits in
// device memory and is read by every workgroup; the grid comes from the
// capacity M and the device's compute-unit count, never from the live count,
// so a launch recorded in a graph stays valid as the count changes.
// Workgroups whose first item lies past the live region exit at once.  The
// same page (Scope and risks) names the squared-ReLU activation as sharing
// that pattern: here relu(x)^2 over the live rows of in[M, d] (not gated).
// gelu_and_mul is the non-sparse GELU-and-multiply whose tanh and exact forms
// the vLLM page ("[Performance] Add Triton kernel for Gemma3n sparse GELU",
// Purpose) selects by "approximation mode"; its live count is optional.
//
// The live region of the output is one contiguous range of n * d elements,
// so items are numbered flat over it: item j lies in row j / items_per_row.
// Each workgroup step covers SILU_BLOCK * PL consecutive items and the grid
// strides over the region, which keeps every lane busy whatever d is (the
// Megatron page's lesson: a grid that is too small for the machine starves it).
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

template <int ACT>
__device__ __forceinline__ float activation(float x) {
    if constexpr (ACT == OP_SILU_MUL) {
        return silu(x);
    } else if constexpr (ACT == OP_GELU_TANH_MUL) {
        return gelu_tanh(x);
    } else if constexpr (ACT == OP_GELU_ERF_MUL) {
        return gelu_erf(x);
    } else {
        const float r = __builtin_fmaxf(x, 0.0f);
        return r * r;
    }
}

constexpr bool op_gated(int op) { return op != OP_SQUARED_RELU; }

// 16-byte items; nvec = vectors per (half) row.  Gated ops read in[M, 2d]
// (gate, then up), the others in[M, d].  live == nullptr means all M rows.
template <int DT, int PL, int OP, bool NONTEMP = true>
__global__ __launch_bounds__(SILU_BLOCK) void act_vec_kernel(
    const uint4 *__restrict__ in, uint4 *__restrict__ out, int32_t M, uint32_t nvec,
    const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    constexpr int PER = E::PER16;
    constexpr uint32_t CHUNK = SILU_BLOCK * PL;
    constexpr bool GATED = op_gated(OP);
    const uint32_t rows = live != nullptr ? (uint32_t)clamp_live(live, M) : (uint32_t)M;
    const uint32_t total = rows * nvec;
    const uint32_t step = gridDim.x * CHUNK;
    for (uint32_t base = blockIdx.x * CHUNK + threadIdx.x; base < total; base += step) {
        uint4 gv[PL], uv[PL];
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) {
                if constexpr (GATED) {
                    const uint32_t row = j / nvec;
                    const size_t off = (size_t)row * 2 * nvec + (j - row * nvec);
                    gv[k] = ld16<NONTEMP>(in + off);
                    uv[k] = ld16<NONTEMP>(in + off + nvec);
                } else {
                    gv[k] = ld16<NONTEMP>(in + j);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) {
                float g[PER], y[PER];
                E::unpack(gv[k], g);
                if constexpr (GATED) {
                    float u[PER];
                    E::unpack(uv[k], u);
#pragma unroll
                    for (int e = 0; e < PER; ++e) y[e] = activation<OP>(g[e]) * u[e];
                } else {
#pragma unroll
                    for (int e = 0; e < PER; ++e) y[e] = activation<OP>(g[e]);
                }
                st16<NONTEMP>(out + j, E::pack(y));
            }
        }
    }
}

// Single-element items: any d, any alignment natural to the type.
template <int DT, int PL, int OP>
__global__ __launch_bounds__(SILU_BLOCK) void act_elem_kernel(
    const typename Elem<DT>::storage *__restrict__ in, typename Elem<DT>::storage *__restrict__ out,
    int32_t M, uint32_t d, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    constexpr uint32_t CHUNK = SILU_BLOCK * PL;
    constexpr bool GATED = op_gated(OP);
    const uint32_t rows = live != nullptr ? (uint32_t)clamp_live(live, M) : (uint32_t)M;
    const uint32_t total = rows * d;
    const uint32_t step = gridDim.x * CHUNK;
    for (uint32_t base = blockIdx.x * CHUNK + threadIdx.x; base < total; base += step) {
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) {
                if constexpr (GATED) {
                    const uint32_t row = j / d;
                    const size_t off = (size_t)row * 2 * d + (j - row * d);
                    out[j] = E::from_f32(activation<OP>(E::to_f32(in[off])) * E::to_f32(in[off + d]));
                } else {
                    out[j] = E::from_f32(activation<OP>(E::to_f32(in[j])));
                }
            }
        }
    }
}

// Rows off 16-byte alignment (a shifted base, or d * element size not a
// multiple of 16).  The live region of the output is contiguous, so its
// 16-byte vectors are numbered flat over it and every one but the region's
// last is written whole: vector j holds output elements [PER j, PER j + PER),
// each vector one 16-byte access at the element's own alignment (gfx950 runs
// global memory in unaligned-access mode).  A vector inside one row reads its
// gate and up as one 16-byte access each, one that straddles a row boundary a
// third for the next row's up; the region's partial last vector, and every
// vector when d is below 16 bytes, go element by element.
template <int DT, int PL, int OP>
__global__ __launch_bounds__(SILU_BLOCK) void act_una_kernel(
    const typename Elem<DT>::storage *__restrict__ in, typename Elem<DT>::storage *__restrict__ out,
    int32_t M, uint32_t d, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    using S = typename E::storage;
    constexpr int PER = E::PER16;
    constexpr uint32_t CHUNK = SILU_BLOCK * PL;
    constexpr bool GATED = op_gated(OP);
    const uint32_t rows = live != nullptr ? (uint32_t)clamp_live(live, M) : (uint32_t)M;
    const uint32_t total = rows * d;  // live output elements
    const uint32_t nitems = (total + PER - 1) / PER;
    const uint32_t step = gridDim.x * CHUNK;
    for (uint32_t base = blockIdx.x * CHUNK + threadIdx.x; base < nitems; base += step) {
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j >= nitems) continue;
            const uint32_t e0 = j * PER;
            const bool full = e0 + PER <= total;
            float g[PER], u[PER], y[PER];
            if constexpr (GATED) {
                const uint32_t row = e0 / d;
                const uint32_t c0 = e0 - row * d;
                if (full && d >= (uint32_t)PER) {
                    // gate[row][c0..] and up[row][c0..]; a vector that runs
                    // past the row (d >= PER: into the next row only) takes
                    // its gate tail from the same 16 bytes as up (they run
                    // on into the next row's gate) and its up tail from the
                    // next row, at the same column.
                    const size_t off = (size_t)row * 2 * d + c0;
                    const uint4 gw = ldu16(in + off), mw = ldu16(in + off + d);
                    E::unpack(gw, g);
                    E::unpack(mw, u);
                    if (c0 + PER > d) {
                        const uint4 bw = ldu16(in + off + 2 * (size_t)d);
                        float m[PER], b[PER];
                        E::unpack(mw, m);
                        E::unpack(bw, b);
                        const uint32_t k = d - c0;  // elements of the vector in this row
#pragma unroll
                        for (int e = 0; e < PER; ++e) {
                            g[e] = (uint32_t)e < k ? g[e] : m[e];
                            u[e] = (uint32_t)e < k ? u[e] : b[e];
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < PER; ++e) {
                        const uint32_t i = e0 + e;
                        g[e] = 0.0f;
                        u[e] = 0.0f;
                        if (i < total) {
                            const uint32_t r = i / d;
                            const size_t off = (size_t)r * 2 * d + (i - r * d);
                            g[e] = E::to_f32(in[off]);
                            u[e] = E::to_f32(in[off + d]);
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < PER; ++e) y[e] = activation<OP>(g[e]) * u[e];
            } else {
                if (full) {
                    E::unpack(ldu16(in + e0), g);
                } else {
#pragma unroll
                    for (int e = 0; e < PER; ++e) g[e] = e0 + e < total ? E::to_f32(in[e0 + e]) : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < PER; ++e) y[e] = activation<OP>(g[e]);
            }
            const uint4 o = E::pack(y);
            if (full) {
                stu16(out + e0, o);
            } else {
                const uint32_t w[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int e = 0; e < PER; ++e) {
                    if (e0 + e < total) {
                        if constexpr (PER == 4) out[e0 + e] = (S)w[e];
                        else out[e0 + e] = (S)(w[e >> 1] >> ((e & 1) * 16));
                    }
                }
            }
        }
    }
}

// Streaming ceiling with the same access pattern: read both halves of each
// row 16 bytes at a time, write their XOR.
template <bool NONTEMP = true>
__global__ __launch_bounds__(SILU_BLOCK) void xor_rows_kernel(const uint4 *__restrict__ in,
                                                              uint4 *__restrict__ out, int32_t rows,
                                                              uint32_t nvec) {
    constexpr int PL = 2;
    constexpr uint32_t CHUNK = SILU_BLOCK * PL;
    const uint32_t total = (uint32_t)rows * nvec;
    const uint32_t step = gridDim.x * CHUNK;
    for (uint32_t base = blockIdx.x * CHUNK + threadIdx.x; base < total; base += step) {
        uint4 a[PL], b[PL];
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) {
                const uint32_t row = j / nvec;
                const size_t off = (size_t)row * 2 * nvec + (j - row * nvec);
                a[k] = ld16<NONTEMP>(in + off);
                b[k] = ld16<NONTEMP>(in + off + nvec);
            }
        }
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) st16<NONTEMP>(out + j, uint4{a[k].x ^ b[k].x, a[k].y ^ b[k].y, a[k].z ^ b[k].z, a[k].w ^ b[k].w});
        }
    }
}

namespace {

// Index [op][path (vector, element, unaligned vector)][dtype][per-lane index].
#define GA_AV(OP, DT) \
    { (const void *)&act_vec_kernel<DT, 1, OP>, (const void *)&act_vec_kernel<DT, 2, OP>, \
      (const void *)&act_vec_kernel<DT, 4, OP> }
#define GA_AE(OP, DT) \
    { (const void *)&act_elem_kernel<DT, 1, OP>, (const void *)&act_elem_kernel<DT, 2, OP>, \
      (const void *)&act_elem_kernel<DT, 4, OP> }
#define GA_AU(OP, DT) \
    { (const void *)&act_una_kernel<DT, 1, OP>, (const void *)&act_una_kernel<DT, 2, OP>, \
      (const void *)&act_una_kernel<DT, 4, OP> }
#define GA_AOP(OP) \
    { {GA_AV(OP, DT_F32), GA_AV(OP, DT_F16), GA_AV(OP, DT_BF16)}, \
      {GA_AE(OP, DT_F32), GA_AE(OP, DT_F16), GA_AE(OP, DT_BF16)}, \
      {GA_AU(OP, DT_F32), GA_AU(OP, DT_F16), GA_AU(OP, DT_BF16)} }
const void *const kAct[OP_COUNT][3][3][3] = {GA_AOP(OP_SILU_MUL), GA_AOP(OP_GELU_TANH_MUL),
                                             GA_AOP(OP_GELU_ERF_MUL), GA_AOP(OP_SQUARED_RELU)};
#undef GA_AV
#undef GA_AE
#undef GA_AU
#undef GA_AOP

int pl_index(int pl) { return pl == 1 ? 0 : pl == 2 ? 1 : pl == 4 ? 2 : -1; }

}  // namespace

bool act_available(int op, int path, int dtype, int per_lane) {
    return op >= 0 && op < OP_COUNT && path >= 0 && path <= 2 && dtype >= 0 && dtype <= 2 &&
           pl_index(per_lane) >= 0;
}

hipError_t launch_act(int op, int path, int dtype, int per_lane, int64_t grid, const void *in, void *out,
                      int32_t M, uint32_t nitems_row, const int32_t *live, hipStream_t stream) {
    if (!act_available(op, path, dtype, per_lane)) return hipErrorInvalidValue;
    const void *fn = kAct[op][path][dtype][pl_index(per_lane)];
    const void *a_in = in;
    void *a_out = out;
    void *args[] = {&a_in, &a_out, &M, &nitems_row, &live};
    return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(SILU_BLOCK), args, 0, stream);
}

hipError_t launch_xor_rows(int64_t grid, const void *in, void *out, int32_t rows, uint32_t nvec_row,
                           hipStream_t stream) {
    const void *a_in = in;
    void *a_out = out;
    void *args[] = {&a_in, &a_out, &rows, &nvec_row};
    return hipLaunchKernel((const void *)&xor_rows_kernel<true>, dim3((uint32_t)grid), dim3(SILU_BLOCK), args,
                           0, stream);
}

}  // namespace ga
