// gelu_and_mul_sparse for short rows (gfx950): several rows per wavefront.
//
// The op is the one of gelu_sparse.hip (vLLM PR 48498, "[Performance] Add
// Triton kernel for Gemma3n sparse GELU", section Purpose).  With one
// workgroup of at least one 64-lane wavefront per row, a row of up to 32
// 16-byte vectors (d <= 256 bf16) leaves most lanes idle.  Here a group of
// G = 4, 8, 16 or 32 consecutive lanes owns a row: its lanes hold the row's
// 16-byte vectors (lane l of the group: vectors l, l + G, ...), reduce within
// the group with DPP moves (quad permutes, half-row and row mirrors, and one
// cross-row exchange for 32 lanes), and store their own vectors.  A 256-lane
// workgroup covers 256 / G consecutive rows, so the loads of neighbouring
// rows form one contiguous stream.  The up row is loaded with the gate.
// Rows off 16-byte alignment (UNA) keep the same layout with unaligned
// 16-byte vectors (ga_unaligned.h): only a row's last vector can be partial,
// and only its lane tests elements in the statistics.
#include "ga_device.h"
#include "ga_internal.h"
#include "ga_unaligned.h"

namespace ga {

namespace {

// Sum over each aligned group of G lanes, the same value in every lane of the
// group.  The mirrors pair lane i with its partner in the other quad (half
// row) and in the other half row (row), which after the previous steps hold
// the other half's sum; the last step exchanges the two rows of 32 lanes.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32, "group of 4, 8, 16 or 32 lanes");
    v += dpp_move<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);  // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp_move<0x141>(v);  // row_half_mirror
    if constexpr (G >= 16) v += dpp_move<0x140>(v);  // row_mirror
    if constexpr (G >= 32) v += __shfl_xor(v, 16, 32);
    return v;
}

}  // namespace

// G lanes per row, VPL 16-byte vectors per lane (G * VPL >= nvec, the row's
// vectors including a partial last one).  UNA: rows off 16-byte alignment.
template <int DT, int G, int VPL, bool RT = false, bool UNA = false>
__global__ __launch_bounds__(ROWS_BLOCK) void gelu_sparse_rows_kernel(
    const void *__restrict__ in_, void *__restrict__ out_, int32_t T, int32_t d, int32_t nvec, float z,
    const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    using S = typename E::storage;
    constexpr int PER = E::PER16;
    constexpr int RPB = ROWS_BLOCK / G;

    const int32_t n = live != nullptr ? clamp_live(live, T) : T;
    const int64_t r0 = (int64_t)blockIdx.x * RPB;
    if (r0 >= n) return;  // uniform per workgroup
    const int32_t t = (int32_t)threadIdx.x;
    const int64_t r = r0 + t / G;
    const int32_t l = t % G;
    // A group past the last row runs the reductions on zeros (its lanes
    // only exchange values among themselves) and stores nothing.
    const bool valid = r < n;
    const int32_t nfull = UNA ? d / PER : nvec, tail = UNA ? d - nfull * PER : 0;

    // Aligned rows: 16-byte vector pointers.  Unaligned rows: element
    // pointers, and whether the 16 bytes of a partial last vector lie inside
    // the input buffer.
    const uint4 *grow = nullptr, *urow = nullptr;
    uint4 *orow = nullptr;
    const S *gs = nullptr, *us = nullptr;
    S *os = nullptr;
    bool gspill = false, uspill = false;
    if constexpr (UNA) {
        const size_t row0 = (size_t)r * 2 * (size_t)d, total = (size_t)T * 2 * (size_t)d;
        const size_t last = (size_t)nfull * PER + PER;
        gs = static_cast<const S *>(in_) + row0;
        us = gs + d;
        os = static_cast<S *>(out_) + (size_t)r * (size_t)d;
        gspill = row0 + last <= total;
        uspill = row0 + (size_t)d + last <= total;
    } else {
        grow = static_cast<const uint4 *>(in_) + (size_t)r * 2 * (size_t)nvec;
        urow = grow + nvec;
        orow = static_cast<uint4 *>(out_) + (size_t)r * (size_t)nvec;
    }

    uint4 gv[VPL], uv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t j = k * G + l;
        if constexpr (UNA) gv[k] = valid ? load_vec<E>(gs, j, nfull, tail, gspill) : uint4{0u, 0u, 0u, 0u};
        else gv[k] = (valid && j < nvec) ? ld16<true>(grow + j) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t j = k * G + l;
        if constexpr (UNA) uv[k] = valid ? load_vec<E>(us, j, nfull, tail, uspill) : uint4{0u, 0u, 0u, 0u};
        else uv[k] = (valid && j < nvec) ? ld16<true>(urow + j) : uint4{0u, 0u, 0u, 0u};
    }

    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float g[PER];
        E::unpack(gv[k], g);
#pragma unroll
        for (int e = 0; e < PER; ++e) s += g[e];
    }
    const float mean = row_mean<RT>(group_sum<G>(s), (float)d);

    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t j = k * G + l;
        float g[PER];
        E::unpack(gv[k], g);
        if (j < nfull) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float dv = g[e] - mean;
                q = __builtin_fmaf(dv, dv, q);
            }
        } else if (UNA && j == nfull) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float dv = e < tail ? g[e] - mean : 0.0f;
                q = __builtin_fmaf(dv, dv, q);
            }
        }
    }
    const float var = row_var<RT>(group_sum<G>(q), (float)d);
    const float cut = sparse_cutoff<E, RT>(mean, var, z);

    if (!valid) return;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t j = k * G + l;
        if (j < nvec) {
            float g[PER], u[PER], y[PER];
            E::unpack(gv[k], g);
            E::unpack(uv[k], u);
#pragma unroll
            for (int e = 0; e < PER; ++e) y[e] = sparse_apply<E, RT>(g[e], cut, u[e]);
            if constexpr (UNA) store_vec<E>(os, j, nfull, tail, E::pack(y));
            else st16<true>(orow + j, E::pack(y));
        }
    }
}

// ---------------------------------------------------------------------------
// Launch table.
// ---------------------------------------------------------------------------
namespace {

#define GA_RW(UNA, RT, DT, G)                                                                 \
    { (const void *)&gelu_sparse_rows_kernel<DT, G, 1, RT, UNA>,                            \
      (const void *)&gelu_sparse_rows_kernel<DT, G, 2, RT, UNA>,                            \
      (const void *)&gelu_sparse_rows_kernel<DT, G, 4, RT, UNA> }
#define GA_RWD(UNA, RT, DT) \
    { GA_RW(UNA, RT, DT, 4), GA_RW(UNA, RT, DT, 8), GA_RW(UNA, RT, DT, 16), GA_RW(UNA, RT, DT, 32) }
#define GA_RWU(UNA) \
    { {GA_RWD(UNA, false, DT_F32), GA_RWD(UNA, false, DT_F16), GA_RWD(UNA, false, DT_BF16)}, \
      {GA_RWD(UNA, true, DT_F32), GA_RWD(UNA, true, DT_F16), GA_RWD(UNA, true, DT_BF16)} }
// [unaligned rows][round trip][dtype][log2 G - 2][log2 VPL]
const void *const kGeluRows[2][2][3][4][3] = {GA_RWU(false), GA_RWU(true)};
#undef GA_RW
#undef GA_RWD
#undef GA_RWU

int group_index(int g) { return g == 4 ? 0 : g == 8 ? 1 : g == 16 ? 2 : g == 32 ? 3 : -1; }
int vpl_index(int v) { return v == 1 ? 0 : v == 2 ? 1 : v == 4 ? 2 : -1; }

}  // namespace

bool gelu_rows_available(int dtype, int lanes_per_row, int vpl) {
    return dtype >= 0 && dtype <= 2 && group_index(lanes_per_row) >= 0 && vpl_index(vpl) >= 0;
}

hipError_t launch_gelu_rows(int dtype, int lanes_per_row, int vpl, bool round_trip, bool unaligned, int64_t grid,
                            const void *in, void *out, int32_t T, int32_t d, int32_t nvec, float z,
                            const int32_t *live, hipStream_t stream) {
    if (!gelu_rows_available(dtype, lanes_per_row, vpl)) return hipErrorInvalidValue;
    const void *fn =
        kGeluRows[unaligned ? 1 : 0][round_trip ? 1 : 0][dtype][group_index(lanes_per_row)][vpl_index(vpl)];
    const void *a_in = in;
    void *a_out = out;
    void *args[] = {&a_in, &a_out, &T, &d, &nvec, &z, &live};
    return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(ROWS_BLOCK), args, 0, stream);
}

}  // namespace ga
