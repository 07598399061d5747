// gelu_and_mul_sparse for gfx950.
//
// The op (vLLM PR 48498, "[Performance] Add Triton kernel for Gemma3n sparse
// GELU", section Purpose): for each row of in[T, 2d] = [gate | up],
//   mean = sum(gate) / d,  std = sqrt(sum((gate - mean)^2) / d)   (population)
//   cut  = mean + z * std
//   out  = gelu_tanh(max(gate - cut, 0)) * up,  rounded once to the element type.
//
// One workgroup owns one row.  Its WAVES wavefronts load the whole gate row
// into registers once (16-byte loads, consecutive lanes on consecutive
// vectors), issue the loads of the up row right behind them so they are in
// flight while the two reductions run, reduce the sum, then the sum of
// squared deviations from the staged registers (two-pass: no E[x^2] - E[x]^2
// cancellation), and finally apply and store 16 bytes per vector.  HBM sees
// each input byte once and each output byte once.  Nothing here is a
// contraction, so there is no MFMA; the kernel is bound by HBM bandwidth.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

// Vector path: d * sizeof(elem) % 16 == 0 and 16-byte aligned bases.
// nvec = 16-byte vectors per half row.  Lane t holds vectors t, t + NT, ...
// UP selects when the up row is loaded: 0 = right behind the gate (in flight
// during both reductions), 1 = after the statistics, all vectors at once,
// 2 = after the statistics, UPCHUNK vectors at a time (fewer registers, so
// more rows resident per compute unit).
// RT: round-trip form (intermediates rounded to the element type).
template <int DT, int WAVES, int VPL, bool NONTEMP = true, int UP = 0, int UPCHUNK = 2, bool RT = false>
__global__ __launch_bounds__(WAVES * 64) void gelu_sparse_vec_kernel(
    const uint4 *__restrict__ in, uint4 *__restrict__ out, int32_t T, int32_t d, int32_t nvec,
    float z, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    constexpr int NT = WAVES * 64;
    constexpr int PER = E::PER16;
    __shared__ float red[2][WAVES];

    const int32_t r = (int32_t)blockIdx.x;
    if (live != nullptr && r >= clamp_live(live, T)) return;  // uniform per workgroup

    const uint4 *grow = in + (size_t)r * 2 * (size_t)nvec;
    const uint4 *urow = grow + nvec;
    uint4 *orow = out + (size_t)r * (size_t)nvec;
    const int t = (int)threadIdx.x;

    uint4 gv[VPL], uv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int j = k * NT + t;
        gv[k] = j < nvec ? ld16<NONTEMP>(grow + j) : uint4{0u, 0u, 0u, 0u};
    }
    if constexpr (UP == 0) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int j = k * NT + t;
            uv[k] = j < nvec ? ld16<NONTEMP>(urow + j) : uint4{0u, 0u, 0u, 0u};
        }
    }

    // Row mean (vectors past the row end were loaded as zeros).
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float f[PER];
        E::unpack(gv[k], f);
#pragma unroll
        for (int e = 0; e < PER; ++e) s += f[e];
    }
    const float mean = row_mean<RT>(block_sum<WAVES>(s, red[0]), (float)d);

    // Population variance from the staged row.
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        if (k * NT + t < nvec) {
            float f[PER];
            E::unpack(gv[k], f);
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float dv = f[e] - mean;
                q = __builtin_fmaf(dv, dv, q);
            }
        }
    }
    const float var = row_var<RT>(block_sum<WAVES>(q, red[1]), (float)d);
    const float cut = sparse_cutoff<E, RT>(mean, var, z);

    if constexpr (UP == 1) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int j = k * NT + t;
            uv[k] = j < nvec ? ld16<NONTEMP>(urow + j) : uint4{0u, 0u, 0u, 0u};
        }
    }

    // Apply and store.
    constexpr int CH = UP == 2 ? (UPCHUNK < VPL ? UPCHUNK : VPL) : VPL;
#pragma unroll
    for (int k0 = 0; k0 < VPL; k0 += CH) {
        if constexpr (UP == 2) {
#pragma unroll
            for (int k = k0; k < k0 + CH; ++k) {
                const int j = k * NT + t;
                uv[k] = j < nvec ? ld16<NONTEMP>(urow + j) : uint4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int k = k0; k < k0 + CH; ++k) {
            const int j = k * NT + t;
            if (j < nvec) {
                float g[PER], u[PER], y[PER];
                E::unpack(gv[k], g);
                E::unpack(uv[k], u);
#pragma unroll
                for (int e = 0; e < PER; ++e) y[e] = sparse_apply<E, RT>(g[e], cut, u[e]);
                st16<NONTEMP>(orow + j, E::pack(y));
            }
        }
    }
}

// Element path: any d and any alignment natural to the type.  Lane t holds
// elements t, t + NT, ... of the gate row as fp32; up is read in the apply
// loop.
template <int DT, int WAVES, int EPL, bool RT = false>
__global__ __launch_bounds__(WAVES * 64) void gelu_sparse_elem_kernel(
    const typename Elem<DT>::storage *__restrict__ in, typename Elem<DT>::storage *__restrict__ out,
    int32_t T, int32_t d, float z, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    using S = typename E::storage;
    constexpr int NT = WAVES * 64;
    __shared__ float red[2][WAVES];

    const int32_t r = (int32_t)blockIdx.x;
    if (live != nullptr && r >= clamp_live(live, T)) return;

    const S *grow = in + (size_t)r * 2 * (size_t)d;
    const S *urow = grow + d;
    S *orow = out + (size_t)r * (size_t)d;
    const int t = (int)threadIdx.x;

    float g[EPL];
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        const int i = k * NT + t;
        g[k] = i < d ? E::to_f32(grow[i]) : 0.0f;
        s += g[k];
    }
    const float mean = row_mean<RT>(block_sum<WAVES>(s, red[0]), (float)d);

    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        if (k * NT + t < d) {
            const float dv = g[k] - mean;
            q = __builtin_fmaf(dv, dv, q);
        }
    }
    const float var = row_var<RT>(block_sum<WAVES>(q, red[1]), (float)d);
    const float cut = sparse_cutoff<E, RT>(mean, var, z);

#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        const int i = k * NT + t;
        if (i < d) {
            const float y = sparse_apply<E, RT>(g[k], cut, E::to_f32(urow[i]));
            orow[i] = E::from_f32(y);
        }
    }
}

// ---------------------------------------------------------------------------
// Launch tables: every (dtype, waves, per-lane) combination is compiled ahead
// of time; the host picks one.
// ---------------------------------------------------------------------------
namespace {

using GeluVecFn = void (*)(const uint4 *, uint4 *, int32_t, int32_t, int32_t, float, const int32_t *);

// Index [round trip][dtype][up_late][log2 waves][log2 vectors per lane]; late
// up loads go one vector at a time.
#define GA_GV(RT, DT, U, W)                                                                            \
    { &gelu_sparse_vec_kernel<DT, W, 1, true, U, 1, RT>, &gelu_sparse_vec_kernel<DT, W, 2, true, U, 1, RT>, \
      &gelu_sparse_vec_kernel<DT, W, 4, true, U, 1, RT>, &gelu_sparse_vec_kernel<DT, W, 8, true, U, 1, RT> }
#define GA_GVU(RT, DT, U) \
    { GA_GV(RT, DT, U, 1), GA_GV(RT, DT, U, 2), GA_GV(RT, DT, U, 4), GA_GV(RT, DT, U, 8), GA_GV(RT, DT, U, 16) }
#define GA_GVD(RT, DT) { GA_GVU(RT, DT, 0), GA_GVU(RT, DT, 2) }
const GeluVecFn kGeluVec[2][3][2][5][4] = {
    {GA_GVD(false, DT_F32), GA_GVD(false, DT_F16), GA_GVD(false, DT_BF16)},
    {GA_GVD(true, DT_F32), GA_GVD(true, DT_F16), GA_GVD(true, DT_BF16)}};
#undef GA_GV
#undef GA_GVU
#undef GA_GVD

#define GA_GE(RT, DT, W)                                                                           \
    { (const void *)&gelu_sparse_elem_kernel<DT, W, 4, RT>, (const void *)&gelu_sparse_elem_kernel<DT, W, 16, RT>, \
      (const void *)&gelu_sparse_elem_kernel<DT, W, 64, RT> }
#define GA_GED(RT, DT) { GA_GE(RT, DT, 1), GA_GE(RT, DT, 4), GA_GE(RT, DT, 16) }
const void *const kGeluElem[2][3][3][3] = {
    {GA_GED(false, DT_F32), GA_GED(false, DT_F16), GA_GED(false, DT_BF16)},
    {GA_GED(true, DT_F32), GA_GED(true, DT_F16), GA_GED(true, DT_BF16)}};
#undef GA_GE
#undef GA_GED

int log2_exact(int v) {
    if (v <= 0 || v > 1024) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return (1 << l) == v ? l : -1;
}

int vec_index(int waves, int vpl, int *wi, int *vi) {
    *wi = log2_exact(waves);
    *vi = log2_exact(vpl);
    return (*wi >= 0 && *wi <= 4 && *vi >= 0 && *vi <= 3) ? 0 : -1;
}

int elem_index(int waves, int epl, int *wi, int *ei) {
    *wi = waves == 1 ? 0 : waves == 4 ? 1 : waves == 16 ? 2 : -1;
    *ei = epl == 4 ? 0 : epl == 16 ? 1 : epl == 64 ? 2 : -1;
    return (*wi >= 0 && *ei >= 0) ? 0 : -1;
}

}  // namespace

bool gelu_vec_available(int dtype, int waves, int vpl, int up_late) {
    int wi, vi;
    return dtype >= 0 && dtype <= 2 && (up_late == 0 || up_late == 1) &&
           vec_index(waves, vpl, &wi, &vi) == 0;
}

bool gelu_elem_available(int dtype, int waves, int epl) {
    int wi, ei;
    return dtype >= 0 && dtype <= 2 && elem_index(waves, epl, &wi, &ei) == 0;
}

hipError_t launch_gelu_vec(int dtype, int waves, int vpl, int up_late, bool round_trip, int64_t grid,
                           const void *in, void *out, int32_t T, int32_t d, int32_t nvec, float z,
                           const int32_t *live, hipStream_t stream) {
    int wi, vi;
    if (!gelu_vec_available(dtype, waves, vpl, up_late) || vec_index(waves, vpl, &wi, &vi) != 0)
        return hipErrorInvalidValue;
    const GeluVecFn fn = kGeluVec[round_trip ? 1 : 0][dtype][up_late][wi][vi];
    const uint4 *a_in = static_cast<const uint4 *>(in);
    uint4 *a_out = static_cast<uint4 *>(out);
    void *args[] = {&a_in, &a_out, &T, &d, &nvec, &z, &live};
    return hipLaunchKernel((const void *)fn, dim3((uint32_t)grid), dim3(waves * 64), args, 0, stream);
}

hipError_t launch_gelu_elem(int dtype, int waves, int epl, bool round_trip, int64_t grid, const void *in,
                            void *out, int32_t T, int32_t d, float z, const int32_t *live, hipStream_t stream) {
    int wi, ei;
    if (!gelu_elem_available(dtype, waves, epl) || elem_index(waves, epl, &wi, &ei) != 0)
        return hipErrorInvalidValue;
    const void *fn = kGeluElem[round_trip ? 1 : 0][dtype][wi][ei];
    const void *a_in = in;
    void *a_out = out;
    void *args[] = {&a_in, &a_out, &T, &d, &z, &live};
    return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(waves * 64), args, 0, stream);
}

}  // namespace ga
