// Host-side interface between the C-ABI (api.hip) and the kernel translation
// units.  Each launcher enqueues one kernel on `stream` and returns the HIP
// status of the launch, or hipErrorInvalidValue when no kernel is
// instantiated for the requested geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

// Geometries with a compiled kernel.
bool gelu_vec_available(int dtype, int waves, int vec_per_lane, int up_late);
bool gelu_elem_available(int dtype, int waves, int elem_per_lane);
// Elementwise activation ops sharing one kernel family.
enum : int { OP_SILU_MUL = 0, OP_GELU_TANH_MUL = 1, OP_GELU_ERF_MUL = 2, OP_SQUARED_RELU = 3, OP_COUNT = 4 };
bool act_available(int op, int path, int dtype, int per_lane);

constexpr int SILU_BLOCK = 256;

// Split-row gelu workspace: one record per row, the same layout for every T
// and split count: SPLIT_MAX 16-byte slots of two 64-bit words,
// {uint32 tag, fp32 mean} and {uint32 tag, fp32 M2}.
constexpr int SPLIT_MAX = 16;
constexpr int SPLIT_SLOT_BYTES = 16;  // slot stride: the two words, packed (one slot per cache line measured slower)
constexpr size_t SPLIT_RECORD_BYTES = (size_t)SPLIT_MAX * SPLIT_SLOT_BYTES;
inline size_t split_workspace_bytes(int64_t T) { return (size_t)T * SPLIT_RECORD_BYTES; }
bool gelu_split_available(int dtype, int waves, int vec_per_lane, int splits);
hipError_t launch_gelu_split(int dtype, int waves, int vec_per_lane, int splits, const void *in, void *out,
                             int32_t T, int32_t d, int32_t nvec, float z, const int32_t *live, void *workspace,
                             uint32_t spin_limit, hipStream_t stream);

// Replicated-statistics path for few rows: REP (2, 4, 8) workgroups per row,
// each reducing the whole gate row itself and applying its REP-th share;
// grid = gelu_rep_grid(T, REP) (rows rounded up to groups of 8).
bool gelu_rep_available(int dtype, int waves, int vec_per_lane, int rep);
int64_t gelu_rep_grid(int64_t T, int rep);
hipError_t launch_gelu_rep(int dtype, int waves, int vec_per_lane, int rep, const void *in, void *out, int32_t T,
                           int32_t d, int32_t nvec, float z, const int32_t *live, hipStream_t stream);

// The activation fused with the down projection y = a . w^T (w: [H, d]).
// At most DOWN_MAX_SPLITS slices of d per row in the tiled form.
constexpr int DOWN_MAX_SPLITS = 64;

// Decode form of the fused op, for T <= tmax tokens (1 or 2): one launch, no
// workspace; workgroups of f output features (2, 4 or 8) over all of d,
// grid ceil(H / f).  Available where a kernel of that geometry reaches d.
bool gelu_down_decode_available(int dtype, int tmax, int f, int waves, int64_t d);
hipError_t launch_gelu_down_decode(int dtype, int tmax, int f, int waves, const void *gu, const void *w, void *y,
                                   int32_t T, int32_t d, int32_t H, float z, const int32_t *live,
                                   hipStream_t stream);

// Workspace of the staged and tiled forms: [0, 256) unused, the tiled
// product's output-tile counters at a fixed place (DOWN_MAX_TILES words,
// zero between calls: each tile's last workgroup resets its own), the stored
// activation ([T, d]) from DOWN_ACT_OFFSET, then the tiled product's fp32
// partial tiles.
constexpr int64_t DOWN_TILE_CNT_OFFSET = 256;
constexpr int64_t DOWN_MAX_TILES = 16384;
constexpr int64_t DOWN_ACT_OFFSET = DOWN_TILE_CNT_OFFSET + DOWN_MAX_TILES * 4;
__host__ __device__ inline int64_t down_tiled_part_offset(int64_t T, int64_t d) {
    return DOWN_ACT_OFFSET + (T * d * 2 + 255) / 256 * 256;
}

// Tiled form's product launch, for any T: y = a . w^T with a the stored
// activation at workspace + DOWN_ACT_OFFSET; workgroups of tm tokens x bh
// features x kc elements of d (grid ceil(T / tm) * ceil(H / bh) * ceil(d / kc));
// several slices of d add their partials through the workspace
// (gelu_down_tiled_workspace_bytes), at most DOWN_MAX_TILES output tiles.
bool gelu_down_tiled_available(int dtype, int tm, int bh, int waves, int kstep, int depth);
size_t gelu_down_tiled_workspace_bytes(int64_t T, int64_t d, int64_t H, int tm, int bh, int64_t kc);
hipError_t launch_gelu_down_tiled(int dtype, int tm, int bh, int waves, int kstep, int depth, int32_t kc, const void *a,
                                  const void *w, void *y, int32_t T, int32_t d, int32_t H, const int32_t *live,
                                  void *workspace, hipStream_t stream);

// Staged form's product launch, for T <= tmax tokens (2 or 4): y = a . w^T
// with a the stored activation ([T, d], rows past the live count not read);
// workgroups of f output features over all of d, grid ceil(H / f).
bool gelu_down_staged_available(int dtype, int tmax, int f, int waves, int64_t d);
hipError_t launch_gelu_down_staged(int dtype, int tmax, int f, int waves, const void *a, const void *w, void *y,
                                   int32_t T, int32_t d, int32_t H, const int32_t *live, hipStream_t stream);

// Packed-rows path for short rows: ROWS_BLOCK threads per workgroup,
// lanes_per_row in {4, 8, 16, 32} lanes per row, vec_per_lane in {1, 2, 4};
// grid = ceil(T / (ROWS_BLOCK / lanes_per_row)).  nvec: the row's 16-byte
// vectors (a partial last one included); unaligned: rows or bases off 16-byte
// alignment (unaligned 16-byte vectors).
constexpr int ROWS_BLOCK = 256;
bool gelu_rows_available(int dtype, int lanes_per_row, int vec_per_lane);
hipError_t launch_gelu_rows(int dtype, int lanes_per_row, int vec_per_lane, bool round_trip, bool unaligned,
                            int64_t grid, const void *in, void *out, int32_t T, int32_t d, int32_t nvec, float z,
                            const int32_t *live, hipStream_t stream);

// Unaligned path for rows that are not 16-byte aligned: waves 1, 2, 4, 8, 16;
// vectors per lane 1 .. 8 (vector j = elements [j * 16 / es, (j + 1) * 16 / es),
// one unaligned 16-byte access); up_late 0 (up loaded with the gate) or 1
// (one vector at a time after the statistics).
bool gelu_unaligned_available(int dtype, int waves, int vec_per_lane, int up_late);
hipError_t launch_gelu_unaligned(int dtype, int waves, int vec_per_lane, int up_late, bool round_trip,
                                 int64_t grid, const void *in, void *out, int32_t T, int32_t d, float z,
                                 const int32_t *live, hipStream_t stream);

// round_trip selects the form that rounds each intermediate (mean, std, z,
// z * std, cutoff, gate - cutoff, GELU output) to the element type.
hipError_t launch_gelu_vec(int dtype, int waves, int vec_per_lane, int up_late, bool round_trip, int64_t grid,
                           const void *in, void *out, int32_t T, int32_t d, int32_t nvec,
                           float z, const int32_t *live, hipStream_t stream);

hipError_t launch_gelu_elem(int dtype, int waves, int elem_per_lane, bool round_trip, int64_t grid,
                            const void *in, void *out, int32_t T, int32_t d,
                            float z, const int32_t *live, hipStream_t stream);

// path 0: 16-byte items (nitems_row = d / elements per 16 bytes),
// path 1: single elements (nitems_row = d), path 2: unaligned 16-byte vectors
// numbered flat over the live output region (nitems_row = d).  live may be
// null (all M rows).
hipError_t launch_act(int op, int path, int dtype, int per_lane, int64_t grid, const void *in, void *out,
                      int32_t M, uint32_t nitems_row, const int32_t *live, hipStream_t stream);

hipError_t launch_xor_rows(int64_t grid, const void *in, void *out, int32_t rows,
                           uint32_t nvec_row, hipStream_t stream);

}  // namespace ga
