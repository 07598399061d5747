// gelu_and_mul_sparse for rows that are not 16-byte aligned (gfx950).
//
// The op is the one of gelu_sparse.hip (vLLM PR 48498, "[Performance] Add
// Triton kernel for Gemma3n sparse GELU", section Purpose).  This path takes
// rows whose gate, up or output start is not on a 16-byte boundary: a base
// pointer offset by a few elements, or d * element size not a multiple of 16
// (then every row starts at a different offset).  The layout of the work is
// that of the vector path: vector j of a stream is its elements
// [PER j, PER j + PER), PER = 16 bytes / element size, and lane t of the
// workgroup owns vectors t, t + NT, ...  Each vector still moves as one
// 16-byte access, at the element's own 2- or 4-byte alignment: gfx950 runs
// global memory in unaligned-access mode (the compiler emits exactly these
// accesses for any under-aligned 16-byte load or store on this target), and
// a wavefront's 64 consecutive vectors cover one contiguous 1 KiB span.
//
// Only the row's last vector can be partial (d % PER elements).  It is read
// as a whole 16-byte access when those 16 bytes lie inside the input buffer
// (the gate's tail runs into the same row's up, up's into the next row), the
// elements past the row zeroed; otherwise, and for every output tail,
// element by element.
#include "ga_device.h"
#include "ga_internal.h"
#include "ga_unaligned.h"

namespace ga {

// Lane t holds gate vectors t, t + NT, ... (VPL of them, VPL * NT >= the
// row's vectors).  RT: round-trip form.  UPLATE: load the up vectors one at a
// time after the statistics (fewer registers, more rows resident) instead of
// all of them with the gate.
template <int DT, int WAVES, int VPL, bool RT = false, bool UPLATE = false>
__global__ __launch_bounds__(WAVES * 64) void gelu_sparse_unaligned_kernel(
    const typename Elem<DT>::storage *__restrict__ in, typename Elem<DT>::storage *__restrict__ out, int32_t T,
    int32_t d, float z, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    using S = typename E::storage;
    constexpr int NT = WAVES * 64;
    constexpr int PER = E::PER16;
    __shared__ float red[2][WAVES];

    const int32_t r = (int32_t)blockIdx.x;
    if (live != nullptr && r >= clamp_live(live, T)) return;  // uniform per workgroup

    const size_t row0 = (size_t)r * 2 * (size_t)d;
    const S *grow = in + row0;
    const S *urow = grow + d;
    S *orow = out + (size_t)r * (size_t)d;
    const int32_t t = (int32_t)threadIdx.x;
    const int32_t nfull = d / PER, tail = d - nfull * PER;
    const int32_t nvec = nfull + (tail > 0 ? 1 : 0);
    const size_t total = (size_t)T * 2 * (size_t)d;
    const size_t last = (size_t)nfull * PER + PER;  // end of the last vector, in elements from a stream's start
    const bool gspill = row0 + last <= total;
    const bool uspill = row0 + (size_t)d + last <= total;

    constexpr int NUV = UPLATE ? 1 : VPL;
    uint4 gv[VPL], uv[NUV];
#pragma unroll
    for (int k = 0; k < VPL; ++k) gv[k] = load_vec<E>(grow, k * NT + t, nfull, tail, gspill);
    if constexpr (!UPLATE) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) uv[k] = load_vec<E>(urow, k * NT + t, nfull, tail, uspill);
    }

    // Row mean (elements past the row were loaded as zeros).
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float f[PER];
        E::unpack(gv[k], f);
#pragma unroll
        for (int e = 0; e < PER; ++e) s += f[e];
    }
    const float mean = row_mean<RT>(block_sum<WAVES>(s, red[0]), (float)d);

    // Population variance from the staged row; only the lane holding the
    // partial last vector tests elements.
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t j = k * NT + t;
        float f[PER];
        E::unpack(gv[k], f);
        if (j < nfull) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float dv = f[e] - mean;
                q = __builtin_fmaf(dv, dv, q);
            }
        } else if (j == nfull) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float dv = e < tail ? f[e] - mean : 0.0f;
                q = __builtin_fmaf(dv, dv, q);
            }
        }
    }
    const float var = row_var<RT>(block_sum<WAVES>(q, red[1]), (float)d);
    const float cut = sparse_cutoff<E, RT>(mean, var, z);

    // Apply and store.
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t j = k * NT + t;
        if (j < nvec) {
            uint4 u4;
            if constexpr (UPLATE) u4 = load_vec<E>(urow, j, nfull, tail, uspill);
            else u4 = uv[k];
            float g[PER], u[PER], y[PER];
            E::unpack(gv[k], g);
            E::unpack(u4, u);
#pragma unroll
            for (int e = 0; e < PER; ++e) y[e] = sparse_apply<E, RT>(g[e], cut, u[e]);
            store_vec<E>(orow, j, nfull, tail, E::pack(y));
        }
    }
}

// ---------------------------------------------------------------------------
// Launch table: [round trip][up late][dtype][log2 waves][vectors per lane - 1].
// ---------------------------------------------------------------------------
namespace {

#define GA_UK(RT, UL, DT, W, V) (const void *)&gelu_sparse_unaligned_kernel<DT, W, V, RT, UL>
#define GA_UA(RT, UL, DT, W)                                                                                 \
    { GA_UK(RT, UL, DT, W, 1), GA_UK(RT, UL, DT, W, 2), GA_UK(RT, UL, DT, W, 3), GA_UK(RT, UL, DT, W, 4), \
      GA_UK(RT, UL, DT, W, 5), GA_UK(RT, UL, DT, W, 6), GA_UK(RT, UL, DT, W, 7), GA_UK(RT, UL, DT, W, 8) }
#define GA_UAD(RT, UL, DT) \
    { GA_UA(RT, UL, DT, 1), GA_UA(RT, UL, DT, 2), GA_UA(RT, UL, DT, 4), GA_UA(RT, UL, DT, 8), GA_UA(RT, UL, DT, 16) }
#define GA_UAU(RT, UL) { GA_UAD(RT, UL, DT_F32), GA_UAD(RT, UL, DT_F16), GA_UAD(RT, UL, DT_BF16) }
const void *const kGeluUnaligned[2][2][3][5][8] = {{GA_UAU(false, false), GA_UAU(false, true)},
                                                    {GA_UAU(true, false), GA_UAU(true, true)}};
#undef GA_UK
#undef GA_UA
#undef GA_UAD
#undef GA_UAU

int waves_index(int waves) {
    return waves == 1 ? 0 : waves == 2 ? 1 : waves == 4 ? 2 : waves == 8 ? 3 : waves == 16 ? 4 : -1;
}

}  // namespace

bool gelu_unaligned_available(int dtype, int waves, int vpl, int up_late) {
    return dtype >= 0 && dtype <= 2 && waves_index(waves) >= 0 && vpl >= 1 && vpl <= 8 &&
           (up_late == 0 || up_late == 1);
}

hipError_t launch_gelu_unaligned(int dtype, int waves, int vpl, int up_late, bool round_trip, int64_t grid,
                                 const void *in, void *out, int32_t T, int32_t d, float z, const int32_t *live,
                                 hipStream_t stream) {
    if (!gelu_unaligned_available(dtype, waves, vpl, up_late)) return hipErrorInvalidValue;
    const void *fn = kGeluUnaligned[round_trip ? 1 : 0][up_late][dtype][waves_index(waves)][vpl - 1];
    const void *a_in = in;
    void *a_out = out;
    void *args[] = {&a_in, &a_out, &T, &d, &z, &live};
    return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(waves * 64), args, 0, stream);
}

}  // namespace ga
