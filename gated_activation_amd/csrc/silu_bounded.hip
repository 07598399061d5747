// silu_and_mul_bounded for gfx950, and the streaming-ceiling kernel.
//
// The op (Megatron-LM PR 6328, "Size MoE activation kernel grid to the row
// count", section What changed and why): an elementwise silu(gate) * up over
// the live rows of a capture-sized MoE buffer in[M, 2d].  The live count sits
// in device memory and is read by every workgroup; the grid comes from the
// capacity M and the device's compute-unit count, never from the live count,
// so a launch recorded in a graph stays valid as the count changes.
// Workgroups whose first item lies past the live region exit at once.
//
// The live region of the output is one contiguous range of n * d elements,
// so items are numbered flat over it: item j lies in row j / items_per_row.
// Each workgroup step covers SILU_BLOCK * PL consecutive items and the grid
// strides over the region, which keeps every lane busy whatever d is (the
// pages' lesson: a grid that is too small for the machine starves it).
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

// 16-byte items; nvec = vectors per half row.
template <int DT, int PL, bool NONTEMP = true>
__global__ __launch_bounds__(SILU_BLOCK) void silu_bounded_vec_kernel(
    const uint4 *__restrict__ in, uint4 *__restrict__ out, int32_t M, uint32_t nvec,
    const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    constexpr int PER = E::PER16;
    constexpr uint32_t CHUNK = SILU_BLOCK * PL;
    const uint32_t total = (uint32_t)clamp_live(live, M) * nvec;
    const uint32_t step = gridDim.x * CHUNK;
    for (uint32_t base = blockIdx.x * CHUNK + threadIdx.x; base < total; base += step) {
        uint4 gv[PL], uv[PL];
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) {
                const uint32_t row = j / nvec;
                const size_t off = (size_t)row * 2 * nvec + (j - row * nvec);
                gv[k] = ld16<NONTEMP>(in + off);
                uv[k] = ld16<NONTEMP>(in + off + nvec);
            }
        }
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) {
                float g[PER], u[PER], y[PER];
                E::unpack(gv[k], g);
                E::unpack(uv[k], u);
#pragma unroll
                for (int e = 0; e < PER; ++e) y[e] = silu(g[e]) * u[e];
                st16<NONTEMP>(out + j, E::pack(y));
            }
        }
    }
}

// Single-element items: any d, any alignment natural to the type.
template <int DT, int PL>
__global__ __launch_bounds__(SILU_BLOCK) void silu_bounded_elem_kernel(
    const typename Elem<DT>::storage *__restrict__ in, typename Elem<DT>::storage *__restrict__ out,
    int32_t M, uint32_t d, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    constexpr uint32_t CHUNK = SILU_BLOCK * PL;
    const uint32_t total = (uint32_t)clamp_live(live, M) * d;
    const uint32_t step = gridDim.x * CHUNK;
    for (uint32_t base = blockIdx.x * CHUNK + threadIdx.x; base < total; base += step) {
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const uint32_t j = base + k * SILU_BLOCK;
            if (j < total) {
                const uint32_t row = j / d;
                const size_t off = (size_t)row * 2 * d + (j - row * d);
                out[j] = E::from_f32(silu(E::to_f32(in[off])) * E::to_f32(in[off + d]));
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
    constexpr int PL = 4;
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

#define GA_SV(DT) \
    { (const void *)&silu_bounded_vec_kernel<DT, 1>, (const void *)&silu_bounded_vec_kernel<DT, 2>, \
      (const void *)&silu_bounded_vec_kernel<DT, 4> }
#define GA_SE(DT) \
    { (const void *)&silu_bounded_elem_kernel<DT, 1>, (const void *)&silu_bounded_elem_kernel<DT, 2>, \
      (const void *)&silu_bounded_elem_kernel<DT, 4> }
const void *const kSilu[2][3][3] = {{GA_SV(DT_F32), GA_SV(DT_F16), GA_SV(DT_BF16)},
                                    {GA_SE(DT_F32), GA_SE(DT_F16), GA_SE(DT_BF16)}};
#undef GA_SV
#undef GA_SE

int pl_index(int pl) { return pl == 1 ? 0 : pl == 2 ? 1 : pl == 4 ? 2 : -1; }

}  // namespace

bool silu_available(int path, int dtype, int per_lane) {
    return (path == 0 || path == 1) && dtype >= 0 && dtype <= 2 && pl_index(per_lane) >= 0;
}

hipError_t launch_silu(int path, int dtype, int per_lane, int64_t grid, const void *in, void *out,
                       int32_t M, uint32_t nitems_row, const int32_t *live, hipStream_t stream) {
    if (!silu_available(path, dtype, per_lane)) return hipErrorInvalidValue;
    const void *fn = kSilu[path][dtype][pl_index(per_lane)];
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
