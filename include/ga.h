/*
 * ga.h -- fused row-wise gated activations on AMD Instinct MI355X (gfx950).
 *
 * Two operations of a transformer FFN / MoE layer, on rows of an input laid
 * out as [rows, 2d] with the gate in columns [0, d) and up in [d, 2d):
 *
 *   ga_gelu_and_mul_sparse   Gemma3n-style sparse GELU-and-multiply (vLLM PR
 *       48498, "[Performance] Add Triton kernel for Gemma3n sparse GELU",
 *       section Purpose): per row, mean and population std of the gate,
 *       cutoff = mean + z * std, out = gelu_tanh(max(gate - cutoff, 0)) * up,
 *       where gelu_tanh(s) = 0.5 s (1 + tanh(sqrt(2/pi) (s + 0.044715 s^3)))
 *       and z = Phi^-1(target sparsity) (1.6448536 for 95%).
 *   ga_silu_and_mul_bounded  silu(gate) * up over only the live rows of a
 *       capture-sized MoE buffer (Megatron-LM PR 6328, "Size MoE activation
 *       kernel grid to the row count", section What changed and why): the
 *       launch shape depends on the buffer capacity only, and the live count
 *       is read on the device, so one launch can be replayed from a graph
 *       while the count changes.
 *
 * Arithmetic is fp32 inside the kernels; the result is rounded once, to
 * nearest even, to the element type.  Input and output share one element
 * type: fp32, fp16 or bf16.
 *
 * Conventions for every entry point:
 *   - Pointers named in/out/live_rows are DEVICE pointers on the current HIP
 *     device; the caller owns all memory.  Tensors are dense and row-major
 *     (row stride 2d elements for in, d for out).  The library allocates
 *     nothing on the device and keeps no state apart from a per-device cache
 *     of the compute-unit count.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Launches are
 *     asynchronous on that stream and never synchronise, so they may be
 *     recorded into a HIP graph by stream capture.
 *   - All argument checks happen on the host before any HIP call; a rejected
 *     call touches no memory.  ga_last_error() then returns a message.
 *   - Out-of-range device live counts are clamped to [0, rows]; they cannot
 *     be reported (no synchronisation).  A live_rows pointer must be 4-byte
 *     aligned (GA_EINVAL otherwise).
 *   - Any alignment natural to the element type is accepted; when in and out
 *     are 16-byte aligned and a row's bytes are a multiple of 16, 16-byte
 *     vector loads and stores are used.  Otherwise the data still moves as
 *     16-byte vectors of consecutive elements, each one unaligned 16-byte
 *     access (gfx950 runs global memory in unaligned-access mode):
 *     gelu_and_mul_sparse per row (rows up to 8192 vectors; rows of up to 32
 *     vectors packed several to a wavefront, as aligned ones are), the other
 *     ops flat over the output region.
 */
#ifndef GA_H
#define GA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GA_F32 = 0, GA_F16 = 1, GA_BF16 = 2 } ga_dtype;

typedef enum {
    GA_OK = 0,
    GA_EINVAL = 1,       /* malformed argument (null pointer, negative size, ...) */
    GA_EUNSUPPORTED = 2, /* well-formed but outside what the kernels handle;
                            callers fall back to another implementation */
    GA_EHIP = 3          /* the HIP runtime reported an error at launch */
} ga_status;

/* A hipStream_t, passed opaquely so this header needs no HIP include. */
typedef void *ga_stream;

/* Largest d (elements per half row) the kernels take. */
#define GA_MAX_D 65536

/* Launch geometry.  Filled by the planners, or by a caller that wants a
 * specific geometry (a tuning sweep); see ga_gelu_and_mul_sparse_with_plan. */
typedef struct {
    int32_t path;          /* 0: 16-byte vector path, 1: per-element path,
                              2: unaligned path (rows off 16-byte alignment; gelu: per
                                 row, the elementwise ops: flat over the output),
                              3: gelu packed-rows path (short rows of any alignment,
                              several rows per wavefront),
                              4: gelu replicated-statistics path (few rows: `splits`
                                 workgroups per row each reduce the whole gate row and
                                 apply their share; 16-byte rows, no workspace) */
    int32_t waves_per_row; /* gelu: 64-lane wavefronts per workgroup (1,2,4,8,16) */
    int32_t per_lane;      /* gelu vector path: 16-byte gate vectors per lane (1,2,4,8;
                              split rows 1,2,4); gelu element path: gate elements per
                              lane (4,16,64); gelu unaligned path: 16-byte vectors per
                              lane (1..8); gelu packed rows: vectors per lane (1,2,4);
                              silu: items per lane per step (1,2,4) */
    int32_t up_late;       /* gelu vector and unaligned paths: 0 = load the up row together
                              with the gate row (shortest latency), 1 = load it after the
                              statistics, a vector (a chunk) at a time (fewer registers, more
                              rows resident); split rows: 0 only */
    int32_t block;         /* threads per workgroup */
    int32_t splits;        /* gelu vector path: workgroups sharing one row; 1, or 2 .. 16
                              (needs a workspace, see ga_gelu_and_mul_sparse_ws); gelu
                              replicated-statistics path: 2, 4 or 8 */
    int64_t grid;          /* workgroups launched (silu: from the capacity M only) */
    uint32_t spin_limit;   /* split rows: rounds of polls of the row's partials before a
                              workgroup computes the whole row's statistics itself */
    int32_t flags;         /* gelu_and_mul_sparse: 0 or GA_ROUND_INTERMEDIATES (not
                              with split rows); silu: zero */
    int32_t lanes_per_row; /* gelu packed-rows path: lanes sharing one row (4, 8, 16, 32;
                              a 256-lane workgroup holds 256 / lanes_per_row rows);
                              other paths: zero */
    int32_t reserved;      /* zero */
} ga_plan;

/*
 * Round-trip form of gelu_and_mul_sparse (vLLM PR 48498, section
 * Cross-architecture warp and dtype validation and the review thread that
 * follows it: the Triton kernel rounds intermediates to the input dtype so
 * that it reproduces native PyTorch, whose every operation returns a tensor
 * of that dtype).  The pages do not list the rounding points; this library
 * rounds where an eager PyTorch composition of the op stores a tensor: the
 * row mean, the row std, z, z * std, the cutoff mean + z * std, gate -
 * cutoff, the GELU output, and the product.  Statistics are still computed
 * in fp32 from the input values.  For fp32 data the form differs from the
 * default only by the fp32 roundings of those intermediates.  The match with
 * the eager composition covers finite inputs: a NaN in a gate row makes that
 * composition's whole row NaN, while both forms here take max(NaN, 0) as 0.
 */
#define GA_ROUND_INTERMEDIATES 1

/*
 * Sparse GELU-and-multiply.
 *   in        [T, 2d] device array of `dtype`; gate = cols [0,d), up = cols [d,2d).
 *   out       [T, d] device array of `dtype`; must not overlap `in`.
 *   T         rows (tokens), 0 <= T <= INT32_MAX; T == 0 launches nothing.
 *   d         elements per half row, 1 <= d <= GA_MAX_D (larger: GA_EUNSUPPORTED).
 *   dtype     a ga_dtype.
 *   z         cutoff multiplier Phi^-1(target sparsity); must be finite.
 *   live_rows NULL: all T rows.  Else a device int32; rows r with
 *             r >= clamp(*live_rows, 0, T) are left untouched.
 * Returns GA_OK once the launch is enqueued.  A launch is one workgroup per
 * row (rows of up to 32 16-byte vectors: several rows per workgroup); where
 * its work-items would reach 2^32 (T >= 2^26 / waves per row, e.g. T = 2^26
 * rows of d = 512 bf16), the call returns GA_EUNSUPPORTED before any HIP call
 * (split the rows over several calls).
 */
ga_status ga_gelu_and_mul_sparse(const void *in, void *out, int64_t T, int64_t d,
                                 int32_t dtype, float z, const int32_t *live_rows,
                                 ga_stream stream);

/*
 * Bounded SiLU-and-multiply over the live rows of a capture-sized buffer.
 *   in        [M, 2d] device array; gate = cols [0,d), up = cols [d,2d).
 *   out       [M, d] device array; must not overlap `in`.
 *   M         buffer capacity in rows, 0 <= M <= INT32_MAX.
 *   d         1 <= d <= GA_MAX_D.
 *   live_rows required device int32; rows [0, clamp(*live_rows, 0, M)) are
 *             computed, every other row of `out` is left untouched.
 * The grid depends on (M, d, dtype, alignment, device) only, never on the
 * live count, so a captured launch stays valid when the count changes.
 */
ga_status ga_silu_and_mul_bounded(const void *in, void *out, int64_t M, int64_t d,
                                  int32_t dtype, const int32_t *live_rows,
                                  ga_stream stream);

/*
 * Sparse GELU-and-multiply with a workspace, for few rows: when the planner
 * splits each row over several workgroups (T small against the compute-unit
 * count), they exchange per-chunk (mean, M2) partials through `workspace`
 * and combine them (Chan's parallel-variance formula, in a fixed order) so
 * every workgroup of a row uses the same cutoff.  Otherwise this is
 * ga_gelu_and_mul_sparse and the workspace is not touched.
 *   workspace        device memory of at least
 *                    ga_gelu_and_mul_sparse_workspace_bytes(T) bytes, 256-byte
 *                    aligned, zero-filled before its first use; the kernels keep
 *                    it valid for every later call (each call tags its partials
 *                    with the previous call's tag plus 16), so it is zeroed
 *                    once, not per call, and survives graph replay.
 *   Calls that share a workspace must not run concurrently (the same stream
 *   serialises them).  A row's workgroups wait for each other for a bounded
 *   number of polls; past it a workgroup computes the row's statistics on
 *   its own, so a launch always completes with a correct result.
 */
size_t ga_gelu_and_mul_sparse_workspace_bytes(int64_t T);
/* The planner splits rows only in calls of at most this many rows, so a
 * workspace of ga_gelu_and_mul_sparse_workspace_bytes(GA_SPLIT_PLAN_ROWS)
 * bytes (64 KiB) lets every call that the planner would split do so. */
#define GA_SPLIT_PLAN_ROWS 256
ga_status ga_gelu_and_mul_sparse_ws(const void *in, void *out, int64_t T, int64_t d,
                                    int32_t dtype, float z, const int32_t *live_rows,
                                    void *workspace, size_t workspace_bytes, ga_stream stream);

/*
 * ga_gelu_and_mul_sparse_ws without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the split records live in the
 * library's own static device array (64 KiB per device, held until the
 * process ends).  It allocates nothing and calls no allocating routine.
 *   Same arguments and checks as ga_gelu_and_mul_sparse, and
 *   T <= GA_SPLIT_PLAN_ROWS (larger T: GA_EUNSUPPORTED; such calls never
 *   split rows, and ga_gelu_and_mul_sparse serves them with no memory).
 * The first call on a device also enqueues a zero fill of that device's
 * array on `stream` (recorded into the graph when `stream` is capturing,
 * and then repeated by the next call).  Every call on one device shares its
 * array: calls that overlap in time on one device (other streams, other
 * threads, concurrent graph replays) race and may compute wrong cutoffs;
 * serialise them, e.g. on one stream.
 */
ga_status ga_gelu_and_mul_sparse_noalloc(const void *in, void *out, int64_t T, int64_t d,
                                         int32_t dtype, float z, const int32_t *live_rows,
                                         ga_stream stream);

/*
 * ga_gelu_and_mul_sparse_ws with flags: 0 (the same as _ws) or
 * GA_ROUND_INTERMEDIATES (the round-trip form above; it never splits rows,
 * so the workspace may then be NULL).  Unknown flag bits: GA_EINVAL.
 */
ga_status ga_gelu_and_mul_sparse_ex(const void *in, void *out, int64_t T, int64_t d,
                                    int32_t dtype, float z, const int32_t *live_rows,
                                    int32_t flags, void *workspace, size_t workspace_bytes,
                                    ga_stream stream);

/*
 * GELU-and-multiply without the sparsity step (vLLM PR 48498, section
 * Purpose: the provider is chosen per "approximation mode"):
 * out = gelu(gate) * up, gelu in the tanh form (GA_GELU_TANH, the same
 * constants as above) or the exact form x * Phi(x) (GA_GELU_ERF).
 *   in [T, 2d], out [T, d]; live_rows NULL for all rows, else a device int32
 *   bounding the rows written (as for ga_silu_and_mul_bounded).
 */
typedef enum { GA_GELU_ERF = 0, GA_GELU_TANH = 1 } ga_gelu_approx;
ga_status ga_gelu_and_mul(const void *in, void *out, int64_t T, int64_t d, int32_t dtype,
                          int32_t approximate, const int32_t *live_rows, ga_stream stream);

/*
 * Bounded squared ReLU, not gated (Megatron-LM PR 6328, section Scope and
 * risks, names the squared-ReLU activation kernel as sharing the bounded
 * row pattern): out[r, i] = max(in[r, i], 0)^2 for rows below
 * clamp(*live_rows, 0, M) of in[M, d]; other rows of out[M, d] untouched.
 * live_rows is required; the grid depends on M only.
 */
ga_status ga_squared_relu_bounded(const void *in, void *out, int64_t M, int64_t d, int32_t dtype,
                                  const int32_t *live_rows, ga_stream stream);

/*
 * Sparse GELU-and-multiply fused with the down projection that consumes it
 * (the vLLM page, Test Result, Correctness: the activation's write feeds the
 * layer's downstream projection, and a fused build must keep the two in that
 * order).  For live rows r and output features h:
 *     a[r, k] = gelu_and_mul_sparse(gu)[r, k], rounded once to `dtype`
 *               (the value ga_gelu_and_mul_sparse would store);
 *     y[r, h] = sum over k of a[r, k] * w[h, k], summed in fp32, rounded
 *               once to `dtype`.
 * The plan's form decides how (results within one rounding of the sum of
 * each other; every form is deterministic: fixed summation orders):
 *   GA_DOWN_DECODE  one or two tokens, d up to 16384 (32768 for one token):
 *                   one launch; each workgroup forms its tokens' statistics
 *                   and activation in registers; no workspace.
 *   GA_DOWN_STAGED  two to four tokens, d up to 16384: the activation is
 *                   stored once into the workspace by the library's own
 *                   activation kernel, then a second launch streams the
 *                   weights against it (fp32 dot products).
 *   GA_DOWN_TILED   any T: the activation stored once as in the staged form,
 *                   then a matrix-core product over it; the sum runs over d
 *                   in slices of k_chunk whose fp32 partials are added in
 *                   slice order.  The planner's choice from three tokens.
 *   gu        [T, 2d] device array (gate | up), 16-byte aligned.
 *   w         [H, d] device array, 16-byte aligned: one row of d weights per
 *             output feature (a linear layer's weight layout).
 *   y         [T, H] device array, 16-byte aligned; must not overlap gu or w.
 *   T         0 <= T <= GA_DOWN_MAX_ROWS tokens (more: GA_EUNSUPPORTED; use
 *             ga_gelu_and_mul_sparse and a matrix product).
 *   d         8 <= d <= GA_MAX_D, a multiple of 8 (16-byte rows).
 *   H         16 <= H <= GA_DOWN_MAX_H, a multiple of 16.
 *   dtype     GA_BF16 or GA_F16 (GA_F32: GA_EUNSUPPORTED).
 *   z, live_rows  as for ga_gelu_and_mul_sparse; rows of y at or past the
 *             live count are left untouched.
 *   workspace device memory of ga_gelu_and_mul_sparse_down_workspace_bytes()
 *             bytes, 256-byte aligned, zero-filled before its first use (the
 *             decode form needs none: NULL is accepted).  Each call leaves it
 *             ready for the next (the tiled form's output-tile counters,
 *             kept in a region of their own, are back at zero), so it is
 *             zeroed once and then serves any later calls and shapes that
 *             fit it, and graph replays.  It must not overlap gu, w or y
 *             (GA_EINVAL).  Calls that share a workspace must not overlap in
 *             time (one stream serialises them).
 */
#define GA_DOWN_MAX_ROWS 256
#define GA_DOWN_MAX_H 65536
#define GA_DOWN_DECODE 1
#define GA_DOWN_STAGED 2
#define GA_DOWN_TILED 3
typedef struct {
    int32_t rows_per_block;     /* tokens per workgroup: 16, 32, 64 or 128 in the tiled form; decode
                                   form: 1 or 2; staged form: 2 or 4 (at least T) */
    int32_t features_per_block; /* output features per workgroup: 16 per wavefront feature group in
                                   the tiled form; decode and staged forms: 2, 4 or 8 */
    int32_t waves;              /* wavefronts per workgroup */
    int32_t k_step;             /* tiled form: elements of d per iteration of a workgroup's loop (64,
                                   128 or 256); 0 in the decode and staged forms (each workgroup
                                   covers all of d) */
    int32_t k_chunk;            /* elements of d per workgroup, a multiple of k_step; d in the decode
                                   and staged forms */
    int32_t splits;             /* ceil(d / k_chunk), at most 64: workgroups that share an output tile */
    int32_t form;               /* GA_DOWN_DECODE, GA_DOWN_STAGED or GA_DOWN_TILED */
    int32_t depth;              /* tiled form: steps of loads each wavefront keeps in flight (1-3);
                                   0 in the other forms */
    int64_t grid;               /* workgroups of the product launch */
} ga_down_plan;
ga_status ga_plan_gelu_and_mul_sparse_down(int64_t T, int64_t d, int64_t H, int32_t dtype, ga_down_plan *plan);
/* Workspace for this plan (NULL: the planner's plan for T, d, H). */
size_t ga_gelu_and_mul_sparse_down_workspace_bytes(int64_t T, int64_t d, int64_t H, const ga_down_plan *plan);
ga_status ga_gelu_and_mul_sparse_down(const void *gu, const void *w, void *y, int64_t T, int64_t d, int64_t H,
                                      int32_t dtype, float z, const int32_t *live_rows, void *workspace,
                                      size_t workspace_bytes, ga_stream stream);
ga_status ga_gelu_and_mul_sparse_down_with_plan(const void *gu, const void *w, void *y, int64_t T, int64_t d,
                                                int64_t H, int32_t dtype, float z, const int32_t *live_rows,
                                                const ga_down_plan *plan, void *workspace,
                                                size_t workspace_bytes, ga_stream stream);

/*
 * Host-only helper: z = Phi^-1(target_sparsity), the cutoff multiplier for
 * a target fraction of zeros (0.95 -> 1.6448536...).  NaN outside (0, 1).
 * Newton's method on the normal CDF, to full double precision.
 */
double ga_z_from_sparsity(double target_sparsity);

/*
 * Host-only planners (no HIP call, usable without a GPU): the geometry the
 * entry points above would launch for these sizes.  `aligned` says whether
 * the 16-byte vector path applies (both base pointers 16-byte aligned and
 * d * element size a multiple of 16); `num_cus` is the device's compute-unit
 * count (256 on MI355X); `with_workspace` allows split rows.
 */
ga_status ga_plan_gelu_and_mul_sparse(int64_t T, int64_t d, int32_t dtype, int32_t aligned,
                                      int32_t num_cus, int32_t with_workspace, ga_plan *plan);
/* The elementwise ops (silu_and_mul_bounded, gelu_and_mul, squared ReLU)
 * share one kernel family and this planner; M is the row capacity. */
ga_status ga_plan_silu_and_mul_bounded(int64_t M, int64_t d, int32_t dtype, int32_t aligned,
                                       int32_t num_cus, ga_plan *plan);

/*
 * The same operations with an explicit geometry (for tuning sweeps and the
 * geometry-independence tests).  The plan must name an instantiated kernel
 * (the values listed in ga_plan) and cover the row: vector path
 * splits * waves_per_row * 64 * per_lane * (16 / element size) >= d, with
 * every split owning at least one vector; element path
 * waves_per_row * 64 * per_lane >= d; unaligned path (any alignment)
 * waves_per_row * 64 * per_lane * e >= d with e = 16 / element size;
 * packed rows (any alignment) lanes_per_row * per_lane * e >= d;
 * else GA_EUNSUPPORTED.
 * `block` and
 * `grid` are derived for gelu; silu takes its grid from the plan.  A split
 * plan needs the workspace described above (else GA_EINVAL) and T <= 65535.
 * `flags` selects the round-trip form for gelu (no split rows with it) and
 * must be zero for silu.  The planners leave it zero.
 */
ga_status ga_gelu_and_mul_sparse_with_plan(const void *in, void *out, int64_t T, int64_t d,
                                           int32_t dtype, float z, const int32_t *live_rows,
                                           const ga_plan *plan, void *workspace,
                                           size_t workspace_bytes, ga_stream stream);
ga_status ga_silu_and_mul_bounded_with_plan(const void *in, void *out, int64_t M, int64_t d,
                                            int32_t dtype, const int32_t *live_rows,
                                            const ga_plan *plan, ga_stream stream);

/*
 * Measurement aid, not part of the activations: a streaming kernel with the
 * same access pattern (read the two halves of rows [0, rows) of in[rows, 2w]
 * 16 bytes at a time, write out[rows, w] = first half XOR second half).  Its
 * bandwidth is the ceiling a row-wise gated activation can reach on the
 * device.  `w_bytes` (bytes per half row) must be a positive multiple of 16
 * and both pointers 16-byte aligned.
 */
ga_status ga_stream_xor_rows(const void *in, void *out, int64_t rows, int64_t w_bytes,
                             ga_stream stream);

/* Static name of a status code. */
const char *ga_status_str(int32_t status);

/* Message describing the last non-OK status returned on this thread. */
const char *ga_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t ga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GA_H */
