// gelu_and_mul_sparse for few rows: each row's output shared by REP
// workgroups that each compute the row's statistics themselves.
//
// Same op as gelu_sparse.hip (vLLM PR 48498, "[Performance] Add Triton kernel
// for Gemma3n sparse GELU", section Purpose).  With few rows, one workgroup
// per row leaves most compute units idle and puts the row's whole apply pass
// (about 14 VALU instructions per element) on one compute unit, where it
// dominates the call.  Here REP workgroups share a row: each loads the whole
// gate row and reduces it exactly as the one-row kernel with the same
// geometry does, so all of them derive the same mean, std and cutoff, bit
// for bit, with no exchange between them; each then loads up for, applies to
// and stores only its REP-th share of the row's vectors.  Against the split
// path (gelu_sparse_split.hip), which exchanges partial statistics through
// device memory, this trades the exchange's round trip for REP reads of the
// gate row and the statistics' arithmetic done REP times.
//
// Block b serves row r = (b / (8 REP)) * 8 + b % 8 and share s = (b / 8) % REP:
// the REP workgroups of a row have block indices congruent modulo 8, and the
// dispatcher deals consecutive workgroups to the eight XCDs in turn, so they
// normally share an XCD and its L2 and HBM sees the row's gate about once.
// The grid is rounded up to whole groups of 8 rows; blocks past the last row
// exit at once.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

template <int DT, int WAVES, int VPL, int REP>
__global__ __launch_bounds__(WAVES * 64) void gelu_sparse_rep_kernel(
    const uint4 *__restrict__ in, uint4 *__restrict__ out, int32_t T, int32_t d, int32_t nvec,
    float z, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    constexpr int NT = WAVES * 64;
    constexpr int PER = E::PER16;
    __shared__ float red[2][WAVES];

    const int32_t b = (int32_t)blockIdx.x;
    const int32_t r = (b / (8 * REP)) * 8 + b % 8;
    const int32_t s = (b / 8) % REP;
    if (r >= T) return;
    if (live != nullptr && r >= clamp_live(live, T)) return;  // uniform per workgroup

    const uint4 *grow = in + (size_t)r * 2 * (size_t)nvec;
    const uint4 *urow = grow + nvec;
    uint4 *orow = out + (size_t)r * (size_t)nvec;
    const int t = (int)threadIdx.x;
    // This workgroup's share of the row: vectors [lo, hi).
    const int lo = (int)((int64_t)s * nvec / REP), hi = (int)((int64_t)(s + 1) * nvec / REP);

    uint4 gv[VPL], uv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int j = k * NT + t;
        gv[k] = j < nvec ? ld16<true>(grow + j) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int j = k * NT + t;
        uv[k] = (j >= lo && j < hi) ? ld16<true>(urow + j) : uint4{0u, 0u, 0u, 0u};
    }

    // Row mean and variance over the whole row, as the one-row kernel does.
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float f[PER];
        E::unpack(gv[k], f);
#pragma unroll
        for (int e = 0; e < PER; ++e) sum += f[e];
    }
    const float mean = row_mean<false>(block_sum<WAVES>(sum, red[0]), (float)d);
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
    const float var = row_var<false>(block_sum<WAVES>(q, red[1]), (float)d);
    const float cut = sparse_cutoff<E, false>(mean, var, z);

    // Apply and store this workgroup's share.
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int j = k * NT + t;
        if (j >= lo && j < hi) {
            float g[PER], u[PER], y[PER];
            E::unpack(gv[k], g);
            E::unpack(uv[k], u);
#pragma unroll
            for (int e = 0; e < PER; ++e) y[e] = sparse_apply<E, false>(g[e], cut, u[e]);
            st16<true>(orow + j, E::pack(y));
        }
    }
}

namespace {

using RepFn = void (*)(const uint4 *, uint4 *, int32_t, int32_t, int32_t, float, const int32_t *);

// Index [dtype][log2 waves][log2 vectors per lane][log2 REP - 1]: waves 1..16,
// vectors per lane 1, 2, 4, 8, REP 2, 4, 8.
#define GA_GR(DT, W, V) \
    { &gelu_sparse_rep_kernel<DT, W, V, 2>, &gelu_sparse_rep_kernel<DT, W, V, 4>, &gelu_sparse_rep_kernel<DT, W, V, 8> }
#define GA_GRW(DT, W) { GA_GR(DT, W, 1), GA_GR(DT, W, 2), GA_GR(DT, W, 4), GA_GR(DT, W, 8) }
#define GA_GRD(DT) { GA_GRW(DT, 1), GA_GRW(DT, 2), GA_GRW(DT, 4), GA_GRW(DT, 8), GA_GRW(DT, 16) }
const RepFn kGeluRep[3][5][4][3] = {GA_GRD(DT_F32), GA_GRD(DT_F16), GA_GRD(DT_BF16)};
#undef GA_GR
#undef GA_GRW
#undef GA_GRD

int ilog2_pow2(int v, int max_log) {
    for (int l = 0; l <= max_log; ++l)
        if ((1 << l) == v) return l;
    return -1;
}

}  // namespace

bool gelu_rep_available(int dtype, int waves, int vec_per_lane, int rep) {
    return dtype >= 0 && dtype <= 2 && ilog2_pow2(waves, 4) >= 0 && ilog2_pow2(vec_per_lane, 3) >= 0 &&
           ilog2_pow2(rep, 3) >= 1;
}

int64_t gelu_rep_grid(int64_t T, int rep) { return (T + 7) / 8 * 8 * rep; }

hipError_t launch_gelu_rep(int dtype, int waves, int vec_per_lane, int rep, const void *in, void *out, int32_t T,
                           int32_t d, int32_t nvec, float z, const int32_t *live, hipStream_t stream) {
    if (!gelu_rep_available(dtype, waves, vec_per_lane, rep)) return hipErrorInvalidValue;
    const RepFn fn = kGeluRep[dtype][ilog2_pow2(waves, 4)][ilog2_pow2(vec_per_lane, 3)][ilog2_pow2(rep, 3) - 1];
    const uint4 *a_in = static_cast<const uint4 *>(in);
    uint4 *a_out = static_cast<uint4 *>(out);
    void *args[] = {&a_in, &a_out, &T, &d, &nvec, &z, &live};
    return hipLaunchKernel((const void *)fn, dim3((uint32_t)gelu_rep_grid(T, rep)), dim3(waves * 64), args, 0,
                           stream);
}

}  // namespace ga
