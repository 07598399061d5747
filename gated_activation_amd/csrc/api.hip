// The C-ABI of libga.so: argument checks, launch planning, dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect and the checks can be exercised without a GPU.  The only HIP
// calls are the device / compute-unit query (cached per device) and the
// kernel launch itself; nothing allocates, copies or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/ga.h"
#include "ga_internal.h"

namespace {

// ---------------------------------------------------------------------------
// Errors, sizes, pointer checks
// ---------------------------------------------------------------------------
thread_local char g_last_error[256] = "";

ga_status fail(ga_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
ga_status fail(ga_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

ga_status launched(const char *op, hipError_t e) {
    if (e != hipSuccess) return fail(GA_EHIP, "%s: launch failed: %s", op, hipGetErrorString(e));
    return GA_OK;
}

size_t elem_size(int32_t dtype) {
    return dtype == GA_F32 ? 4 : (dtype == GA_F16 || dtype == GA_BF16) ? 2 : 0;
}

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// The 16-byte path: both bases 16-byte aligned and every row a whole number
// of 16-byte vectors.
bool vector_aligned(const void *in, const void *out, int64_t d, int32_t dtype) {
    return ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
           ((size_t)d * elem_size(dtype)) % 16 == 0;
}

int next_pow2(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Checks of [rows, cols_in * d] in and [rows, d] out: cols_in is 2 for the
// gated layout (gate | up) and 1 for the ungated one.
ga_status check_rows(const char *op, const void *in, const void *out, int64_t rows, int64_t d,
                     int32_t dtype, int cols_in = 2) {
    if (in == nullptr || out == nullptr) return fail(GA_EINVAL, "%s: null in/out pointer", op);
    if (rows < 0 || rows > INT32_MAX)
        return fail(GA_EINVAL, "%s: row count %lld out of [0, 2^31)", op, (long long)rows);
    if (d < 1) return fail(GA_EINVAL, "%s: d = %lld must be >= 1", op, (long long)d);
    const size_t es = elem_size(dtype);
    if (es == 0) return fail(GA_EINVAL, "%s: unknown dtype %d", op, (int)dtype);
    if (d > GA_MAX_D) return fail(GA_EUNSUPPORTED, "%s: d = %lld above %d", op, (long long)d, GA_MAX_D);
    if ((uintptr_t)in % es != 0 || (uintptr_t)out % es != 0)
        return fail(GA_EINVAL, "%s: pointer not aligned to the element size", op);
    const size_t in_bytes = (size_t)rows * (size_t)cols_in * (size_t)d * es;
    const size_t out_bytes = (size_t)rows * (size_t)d * es;
    if (rows > 0 && overlaps(in, in_bytes, out, out_bytes))
        return fail(GA_EINVAL, "%s: in and out overlap (in-place is not supported)", op);
    return GA_OK;
}

// Compute-unit count of the current device, cached per device.
std::atomic<int> g_cus[64];

ga_status current_cus(int *cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return GA_OK;
        }
    }
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || c <= 0)
        return fail(GA_EHIP, "hipDeviceGetAttribute(CU count): %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) g_cus[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return GA_OK;
}

// ---------------------------------------------------------------------------
// gelu_and_mul_sparse: planning, plan checks, launch
// ---------------------------------------------------------------------------
constexpr uint32_t kDefaultSpinLimit = 1u << 16;
constexpr int64_t kSplitMaxRows = 65535;  // the grid's y limit

// Waves for `nvec` vectors of one workgroup at `target` vectors per lane
// (at most 16 waves; the vectors per lane grow to cover the rest).
void waves_for(int64_t nvec, int target, int *w_out, int *v_out) {
    int w = next_pow2((nvec + 64 * target - 1) / (64 * target));
    if (w > 16) w = 16;
    *w_out = w;
    *v_out = next_pow2((nvec + 64 * w - 1) / (64 * w));
}

// The analytic row rule, from a first sweep of power-of-two shapes (T in
// 256..8192, 128..4096 vectors per row, bf16): loading up after the
// statistics frees registers for more resident rows; it pays once the gate
// alone is >= 2^20 vectors (16 MiB) and either there are >= 1024 rows or the
// gate is >= 2^21 vectors.  Two vectors per lane suit rows of 65..1024
// vectors (one for up to 256 when up comes early), four longer rows.  The
// vector path now takes its geometry from the measured table below; this rule
// remains for the unaligned path's choice of when to load up and as the
// fallback where the table has no data.
bool late_by_size(int64_t nvec, int64_t T) {
    const int64_t gate_vectors = T * nvec;
    return gate_vectors >= ((int64_t)1 << 20) && (T >= 1024 || gate_vectors >= ((int64_t)1 << 21));
}

void analytic_row_geometry(int64_t nvec, int64_t T, int *w_out, int *v_out, int *late_out) {
    const bool late = late_by_size(nvec, T);
    int target;
    if (nvec <= 64) target = 1;
    else if (nvec <= 128) target = 2;
    else if (nvec <= 256) target = late ? 2 : 1;
    else target = nvec <= 1024 ? 2 : 4;
    waves_for(nvec, target, w_out, v_out);
    *late_out = late ? 1 : 0;
}

// The measured geometry tables: Loss[t][n][g] is how much slower geometry g
// ran than the best geometry at T[t] rows of N[n] vectors (in 1/400 steps;
// 255 = not run), from sweeps of every compiled geometry on MI355X
// (gated_activation_amd/tune; bf16 rows: the choice depends on bytes per
// row, so it serves every type).  kPlan*: the vector kernel; kUna*: the
// unaligned kernel on rows one element off 16-byte alignment.
#include "planner_table.inc"
#include "planner_table_una.inc"
#include "planner_table_split.inc"
#include "planner_table_rep.inc"

constexpr int kPlanWaves[5] = {1, 2, 4, 8, 16};
constexpr int kPlanPerLane[4] = {1, 2, 4, 8};
static_assert(kPlanNG == 40 && kUnaNG == 40, "geometry tables: 5 wave counts x 4 per-lane counts x 2 up modes");

struct GeoTable {
    const int *T;
    int nT;
    const int *N;
    int nN;
    const unsigned char *loss;  // [nT][nN][40]
};
const GeoTable kVecTable{kPlanT, kPlanNT, kPlanN, kPlanNN, &kPlanLoss[0][0][0]};
const GeoTable kUnaTable{kUnaT, kUnaNT, kUnaN, kUnaNN, &kUnaLoss[0][0][0]};

// Grid interval around x: indices lo <= hi and the weight of lo, linear in
// log2 x; outside the grid both indices are the end point.
void plan_bracket(const int *grid, int n, double x, int *lo, int *hi, double *wlo) {
    *lo = *hi = x <= grid[0] ? 0 : n - 1;
    *wlo = 1.0;
    if (x <= grid[0] || x >= grid[n - 1]) return;
    for (int i = 0; i + 1 < n; ++i) {
        if (grid[i] <= x && x <= grid[i + 1]) {
            *lo = i;
            *hi = i + 1;
            const double l0 = std::log2((double)grid[i]), l1 = std::log2((double)grid[i + 1]);
            *wlo = (l1 - std::log2(x)) / (l1 - l0);
            return;
        }
    }
}

// The valid candidate with the least loss interpolated over the four grid
// points around (T, nvec) (weights linear in log2 T and log2 nvec), scored as
// half the weighted mean plus half the largest loss over the points where it
// was run (at least half of the weight); ties go to the first candidate in
// table order.  loss: [nT][nN][nc].  -1 if no candidate qualifies.
template <typename Valid>
int table_argmin(const int *Tg, int nT, const int *Ng, int nN, const unsigned char *loss, int nc, int64_t T,
                 int64_t nvec, Valid valid) {
    int t0, t1, n0, n1;
    double wt, wn;
    plan_bracket(Tg, nT, (double)T, &t0, &t1, &wt);
    plan_bracket(Ng, nN, (double)nvec, &n0, &n1, &wn);
    const int ti[4] = {t0, t0, t1, t1}, ni[4] = {n0, n1, n0, n1};
    const double pw[4] = {wt * wn, wt * (1.0 - wn), (1.0 - wt) * wn, (1.0 - wt) * (1.0 - wn)};
    int best = -1;
    double best_score = 0.0;
    for (int c = 0; c < nc; ++c) {
        if (!valid(c)) continue;
        double sum = 0.0, wsum = 0.0, mx = 0.0;
        for (int k = 0; k < 4; ++k) {
            if (pw[k] <= 0.0) continue;
            const int l = loss[((size_t)ti[k] * nN + ni[k]) * nc + c];
            if (l == 255) continue;
            sum += pw[k] * l;
            wsum += pw[k];
            mx = std::max(mx, (double)l);
        }
        if (wsum < 0.5) continue;
        const double score = 0.5 * sum / wsum + 0.5 * mx;
        if (best < 0 || score < best_score) {
            best = c;
            best_score = score;
        }
    }
    return best;
}

// The tabled row geometry (40 candidates: waves x vectors per lane x up mode)
// that covers nvec.  False if no geometry qualifies.
bool table_geometry(const GeoTable &tb, int64_t nvec, int64_t T, int *w_out, int *v_out, int *late_out) {
    const int best = table_argmin(tb.T, tb.nT, tb.N, tb.nN, tb.loss, 40, T, nvec, [&](int g) {
        return (int64_t)kPlanWaves[g / 8] * 64 * kPlanPerLane[(g / 2) % 4] >= nvec;
    });
    if (best < 0) return false;
    *w_out = kPlanWaves[best / 8];
    *v_out = kPlanPerLane[(best / 2) % 4];
    *late_out = best % 2;
    return true;
}

// One workgroup per row, vector path.  On 153 shapes off the grid the tabled
// choice ran at 1.007x the best geometry on average, 1.013x at the 90th
// percentile (the analytic rule: 1.027x and 1.080x, up to 1.28x).
void pick_row_geometry(int64_t nvec, int64_t T, int *w_out, int *v_out, int *late_out) {
    if (!table_geometry(kVecTable, nvec, T, w_out, v_out, late_out))
        analytic_row_geometry(nvec, T, w_out, v_out, late_out);
}

// Unaligned path (rows off 16-byte alignment).  On the same 153 shapes, one
// element off alignment, the tabled choice ran at 1.012x the best geometry on
// average, 1.037x at the 90th percentile; the earlier rule (below, the
// fallback) at 1.045x and 1.103x, up to 1.39x.  That rule: up early or late
// by the analytic rule; one vector per lane for 129..256-vector rows, else the
// analytic rule's vectors per lane.
void pick_unaligned_geometry(int64_t nvec, int64_t T, int *w_out, int *v_out, int *late_out) {
    if (table_geometry(kUnaTable, nvec, T, w_out, v_out, late_out)) return;
    *late_out = late_by_size(nvec, T) ? 1 : 0;
    const int target = nvec <= 64 ? 1 : nvec <= 128 ? 2 : nvec <= 256 ? 1 : nvec <= 1024 ? 2 : 4;
    waves_for(nvec, target, w_out, v_out);
}

// Few long rows, with a workspace: whether to split each row over several
// workgroups, and into which chunks, from the measured split table
// (kSplitLoss: 15 chunk geometries of the split kernel, waves 1..16 times
// vectors per lane 1, 2, 4, each row taking ceil(nvec / chunk) splits in
// 2..16, and not splitting as the last candidate; 1 <= T <= 256, 2048 ..
// 8192 vectors per row).  On 36 shapes off the grid the tabled choice ran at
// 1.0085x the best plan on average (the earlier rule, about 512-vector chunks
// for about 256 workgroups: 1.04x, up to 1.26x).  False: do not split.
bool pick_split(int64_t nvec, int64_t T, int *w_out, int *v_out, int *splits_out) {
    static_assert(kSplitNG == 16, "split table: 15 chunk geometries and the row path");
    static_assert(kSplitT[kSplitNT - 1] <= GA_SPLIT_PLAN_ROWS, "the planner splits calls of <= GA_SPLIT_PLAN_ROWS rows");
    if (T < 1 || T > kSplitT[kSplitNT - 1] || T > GA_SPLIT_PLAN_ROWS || nvec < kSplitN[0] || nvec > kSplitN[kSplitNN - 1]) return false;
    auto chunk_of = [](int c) { return (int64_t)kPlanWaves[c / 3] * 64 * (1 << (c % 3)); };
    const int best = table_argmin(kSplitT, kSplitNT, kSplitN, kSplitNN, &kSplitLoss[0][0][0], kSplitNG, T, nvec,
                                  [&](int c) {
                                      if (c == 15) return true;
                                      const int64_t splits = (nvec + chunk_of(c) - 1) / chunk_of(c);
                                      return splits >= 2 && splits <= ga::SPLIT_MAX;
                                  });
    if (best < 0 || best == 15) return false;
    *w_out = kPlanWaves[best / 3];
    *v_out = 1 << (best % 3);
    *splits_out = (int)((nvec + chunk_of(best) - 1) / chunk_of(best));
    return true;
}

// Few rows: whether the replicated-statistics path (each of REP workgroups
// per row reduces the whole gate row and applies its share; no workspace)
// beats the row path and, with a workspace, the split path, and with which
// geometry, from the measured table kRepLoss (60 replicated geometries,
// waves 1..16 times vectors per lane 1, 2, 4, 8 times REP 2, 4, 8; then the
// fastest row geometry and the fastest split plan; 1 <= T <= 256 rows of
// 256 .. 8192 vectors).  False: not replicated (the row and split tables
// decide).
bool pick_rep(int64_t nvec, int64_t T, bool with_workspace, int *w_out, int *v_out, int *rep_out) {
    static_assert(kRepNG == 62, "replicated table: 60 geometries, the row path and the split path");
    if (T < 1 || T > kRepT[kRepNT - 1] || nvec < kRepN[0] || nvec > kRepN[kRepNN - 1]) return false;
    const int best = table_argmin(kRepT, kRepNT, kRepN, kRepNN, &kRepLoss[0][0][0], kRepNG, T, nvec, [&](int c) {
        if (c == 60) return true;
        if (c == 61) return with_workspace;
        return (int64_t)kPlanWaves[c / 12] * 64 * kPlanPerLane[(c / 3) % 4] >= nvec;
    });
    if (best < 0 || best >= 60) return false;
    *w_out = kPlanWaves[best / 12];
    *v_out = kPlanPerLane[(best / 3) % 4];
    *rep_out = 2 << (best % 3);
    return true;
}

ga_status check_gelu_plan(const ga_plan *p, int64_t T, int64_t d, int32_t dtype) {
    if ((p->flags & ~GA_ROUND_INTERMEDIATES) != 0)
        return fail(GA_EINVAL, "gelu plan: unknown flag bits 0x%x", (unsigned)p->flags);
    if ((p->flags & GA_ROUND_INTERMEDIATES) && p->splits != 1)
        return fail(GA_EUNSUPPORTED, "gelu plan: the round-trip form does not split rows");
    if ((p->path != 3 && p->lanes_per_row != 0) || p->reserved != 0)
        return fail(GA_EINVAL, "gelu plan: lanes_per_row is for the packed-rows path; reserved must be zero");
    if (p->path == 0) {
        const int64_t per16 = 16 / (int64_t)elem_size(dtype);
        const int64_t nvec = (d + per16 - 1) / per16;
        if (p->splits == 1) {
            if (!ga::gelu_vec_available(dtype, p->waves_per_row, p->per_lane, p->up_late))
                return fail(GA_EUNSUPPORTED, "gelu plan: no vector kernel for waves=%d per_lane=%d up_late=%d",
                            p->waves_per_row, p->per_lane, p->up_late);
            if ((int64_t)p->waves_per_row * 64 * p->per_lane < nvec)
                return fail(GA_EUNSUPPORTED, "gelu plan: geometry covers fewer than d elements");
        } else {
            if (!ga::gelu_split_available(dtype, p->waves_per_row, p->per_lane, p->splits) || p->up_late != 0)
                return fail(GA_EUNSUPPORTED, "gelu plan: no split kernel for waves=%d per_lane=%d splits=%d",
                            p->waves_per_row, p->per_lane, p->splits);
            const int64_t chunk = (int64_t)p->waves_per_row * 64 * p->per_lane;
            if (chunk * p->splits < nvec || chunk * (p->splits - 1) >= nvec)
                return fail(GA_EUNSUPPORTED, "gelu plan: %d splits of %lld vectors do not tile a %lld-vector row",
                            p->splits, (long long)chunk, (long long)nvec);
            if (T > kSplitMaxRows)
                return fail(GA_EUNSUPPORTED, "gelu plan: split rows need T <= %lld", (long long)kSplitMaxRows);
        }
    } else if (p->path == 4) {
        if ((p->flags & GA_ROUND_INTERMEDIATES) != 0)
            return fail(GA_EUNSUPPORTED, "gelu plan: the round-trip form has no replicated-statistics kernel");
        if (p->up_late != 0 || !ga::gelu_rep_available(dtype, p->waves_per_row, p->per_lane, p->splits))
            return fail(GA_EUNSUPPORTED,
                        "gelu plan: no replicated-statistics kernel for waves=%d per_lane=%d splits=%d up_late=%d",
                        p->waves_per_row, p->per_lane, p->splits, p->up_late);
        const int64_t per16 = 16 / (int64_t)elem_size(dtype);
        if ((int64_t)p->waves_per_row * 64 * p->per_lane < (d + per16 - 1) / per16)
            return fail(GA_EUNSUPPORTED, "gelu plan: geometry covers fewer than d elements");
    } else if (p->path == 3) {
        if (p->splits != 1 || p->up_late != 0)
            return fail(GA_EUNSUPPORTED, "gelu plan: the packed-rows path takes splits=1, up_late=0");
        if (!ga::gelu_rows_available(dtype, p->lanes_per_row, p->per_lane))
            return fail(GA_EUNSUPPORTED, "gelu plan: no packed-rows kernel for lanes_per_row=%d per_lane=%d",
                        p->lanes_per_row, p->per_lane);
        const int64_t per16 = 16 / (int64_t)elem_size(dtype);
        if ((int64_t)p->lanes_per_row * p->per_lane * per16 < d)
            return fail(GA_EUNSUPPORTED, "gelu plan: geometry covers fewer than d elements");
    } else if (p->path == 2) {
        if (p->splits != 1) return fail(GA_EUNSUPPORTED, "gelu plan: the unaligned path does not split rows");
        if (!ga::gelu_unaligned_available(dtype, p->waves_per_row, p->per_lane, p->up_late))
            return fail(GA_EUNSUPPORTED, "gelu plan: no unaligned-path kernel for waves=%d per_lane=%d up_late=%d",
                        p->waves_per_row, p->per_lane, p->up_late);
        const int64_t per16 = 16 / (int64_t)elem_size(dtype);
        if ((int64_t)p->waves_per_row * 64 * p->per_lane < (d + per16 - 1) / per16)
            return fail(GA_EUNSUPPORTED, "gelu plan: geometry covers fewer than the row's 16-byte vectors");
    } else if (p->path == 1) {
        if (p->splits != 1) return fail(GA_EUNSUPPORTED, "gelu plan: the element path does not split rows");
        if (!ga::gelu_elem_available(dtype, p->waves_per_row, p->per_lane))
            return fail(GA_EUNSUPPORTED, "gelu plan: no element kernel for waves=%d per_lane=%d",
                        p->waves_per_row, p->per_lane);
        if ((int64_t)p->waves_per_row * 64 * p->per_lane < d)
            return fail(GA_EUNSUPPORTED, "gelu plan: geometry covers fewer than d elements");
    } else {
        return fail(GA_EINVAL, "gelu plan: path %d", p->path);
    }
    return GA_OK;
}

// One launch dimension holds fewer than 2^32 work-items (grid * block): the
// dispatch packet's grid size is a 32-bit count of work-items.
constexpr int64_t kMaxWorkItems = (int64_t)1 << 32;

// Work-items of a gelu launch with this plan over T rows.
int64_t gelu_work_items(const ga_plan &p, int64_t T) {
    if (p.path == 4) return ga::gelu_rep_grid(T, p.splits) * (int64_t)p.waves_per_row * 64;
    if (p.path == 3) {
        const int64_t rows_per_block = ga::ROWS_BLOCK / p.lanes_per_row;
        return (T + rows_per_block - 1) / rows_per_block * ga::ROWS_BLOCK;
    }
    return T * (int64_t)p.splits * (int64_t)p.waves_per_row * 64;
}

ga_status check_work_items(const ga_plan &p, int64_t T) {
    if (gelu_work_items(p, T) >= kMaxWorkItems)
        return fail(GA_EUNSUPPORTED,
                    "ga_gelu_and_mul_sparse: %lld rows need %lld work-items in one launch (limit 2^32); "
                    "split the rows over several calls",
                    (long long)T, (long long)gelu_work_items(p, T));
    return GA_OK;
}

ga_status check_workspace(const ga_plan &p, int64_t T, const void *workspace, size_t workspace_bytes) {
    if (p.path != 0 || p.splits <= 1) return GA_OK;
    if (workspace == nullptr) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: a split plan needs a workspace");
    if ((uintptr_t)workspace % 256 != 0)
        return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: workspace not 256-byte aligned");
    if (workspace_bytes < ga::split_workspace_bytes(T))
        return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: workspace of %zu bytes, %zu needed", workspace_bytes,
                    ga::split_workspace_bytes(T));
    return GA_OK;
}

ga_status launch_gelu(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, float z,
                      const int32_t *live, const ga_plan &p, void *workspace, ga_stream stream) {
    const char *name = "ga_gelu_and_mul_sparse";
    if ((uintptr_t)live % 4 != 0) return fail(GA_EINVAL, "%s: live_rows is not 4-byte aligned", name);
    ga_status st = check_work_items(p, T);
    if (st != GA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool rt = (p.flags & GA_ROUND_INTERMEDIATES) != 0;
    if (p.path == 0) {
        const int32_t nvec = (int32_t)(d * (int64_t)elem_size(dtype) / 16);
        if (p.splits > 1)
            return launched(name, ga::launch_gelu_split(dtype, p.waves_per_row, p.per_lane, p.splits, in, out,
                                                        (int32_t)T, (int32_t)d, nvec, z, live, workspace,
                                                        p.spin_limit, s));
        return launched(name, ga::launch_gelu_vec(dtype, p.waves_per_row, p.per_lane, p.up_late, rt, T, in, out,
                                                  (int32_t)T, (int32_t)d, nvec, z, live, s));
    }
    if (p.path == 4) {
        if (rt) return fail(GA_EUNSUPPORTED, "%s: the round-trip form has no replicated-statistics kernel", name);
        const int32_t nvec = (int32_t)(d * (int64_t)elem_size(dtype) / 16);
        return launched(name, ga::launch_gelu_rep(dtype, p.waves_per_row, p.per_lane, p.splits, in, out, (int32_t)T,
                                                  (int32_t)d, nvec, z, live, s));
    }
    if (p.path == 3) {
        // Rows' 16-byte vectors, a partial last one included; rows or bases
        // off 16-byte alignment take the unaligned-vector kernel.
        const int32_t nvec = (int32_t)((d * (int64_t)elem_size(dtype) + 15) / 16);
        const int64_t rows_per_block = ga::ROWS_BLOCK / p.lanes_per_row;
        return launched(name, ga::launch_gelu_rows(dtype, p.lanes_per_row, p.per_lane, rt,
                                                   !vector_aligned(in, out, d, dtype),
                                                   (T + rows_per_block - 1) / rows_per_block, in, out, (int32_t)T,
                                                   (int32_t)d, nvec, z, live, s));
    }
    if (p.path == 2)
        return launched(name, ga::launch_gelu_unaligned(dtype, p.waves_per_row, p.per_lane, p.up_late, rt, T, in,
                                                        out, (int32_t)T, (int32_t)d, z, live, s));
    return launched(name, ga::launch_gelu_elem(dtype, p.waves_per_row, p.per_lane, rt, T, in, out, (int32_t)T,
                                               (int32_t)d, z, live, s));
}

// ---------------------------------------------------------------------------
// Elementwise family (silu_and_mul_bounded, gelu_and_mul, squared ReLU)
// ---------------------------------------------------------------------------
// Flat item count of the live region must fit the kernels' 32-bit indices.
constexpr int64_t kMaxItems = (int64_t)1 << 31;

// Items (16 bytes, or one element) per lane per step and workgroups, as
// measured best on MI355X: one item per lane and up to sixteen workgroups per
// compute unit up to 2M items (the MoE decode buffer), two items per lane
// beyond, and up to 32 workgroups per compute unit beyond 4M items.  The
// grid-stride loop covers the rest.  The grid depends on the capacity, never
// on a live count.
// 16-byte items of a plan: whole-row vectors (path 0), elements (path 1), or
// vectors numbered flat over the output region (path 2, the last one partial).
int64_t act_items(int path, int64_t rows, int64_t d, size_t es) {
    const int64_t per = 16 / (int64_t)es;
    return path == 0 ? rows * (d / per) : path == 1 ? rows * d : (rows * d + per - 1) / per;
}

ga_plan plan_act(int64_t rows, int64_t d, size_t es, bool aligned, int num_cus) {
    ga_plan p{};
    // Rows off 16-byte alignment take unaligned 16-byte vectors (measured on
    // MI355X: 1.3-2x the per-element path, which stays for explicit plans).
    p.path = (aligned && ((size_t)d * es) % 16 == 0) ? 0 : 2;
    const int64_t items = act_items(p.path, rows, d, es);
    p.per_lane = items > ((int64_t)2 << 20) ? 2 : 1;
    p.waves_per_row = 0;
    p.splits = 1;
    p.block = ga::SILU_BLOCK;
    const int64_t per_wg = (int64_t)ga::SILU_BLOCK * p.per_lane;
    int64_t g = (items + per_wg - 1) / per_wg;
    const int64_t cap = (int64_t)num_cus * (items > ((int64_t)4 << 20) ? 32 : 16);
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    p.grid = g;
    return p;
}

ga_status check_act_plan(const ga_plan *p, int op, int64_t rows, int64_t d, int32_t dtype) {
    if (p->flags != 0) return fail(GA_EINVAL, "plan: flags must be zero for this op");
    if (!ga::act_available(op, p->path, dtype, p->per_lane))
        return fail(GA_EUNSUPPORTED, "plan: no kernel for path=%d per_lane=%d", p->path, p->per_lane);
    if (p->grid < 1 || p->grid > INT32_MAX) return fail(GA_EINVAL, "plan: grid %lld", (long long)p->grid);
    // The kernels step through items with 32-bit counters: both the region
    // and one grid-wide step must stay below 2^31 so their sum cannot wrap;
    // paths 1 and 2 also index elements of the region with 32 bits.
    if (p->grid * ga::SILU_BLOCK * p->per_lane > kMaxItems)
        return fail(GA_EUNSUPPORTED, "plan: grid too large for 32-bit item indices");
    if (act_items(p->path, rows, d, elem_size(dtype)) >= kMaxItems || (p->path != 0 && rows * d >= kMaxItems))
        return fail(GA_EUNSUPPORTED, "plan: rows * d too large for 32-bit item indices");
    return GA_OK;
}

ga_status launch_act(const char *name, int op, const void *in, void *out, int64_t rows, int64_t d,
                     int32_t dtype, const int32_t *live, const ga_plan &p, ga_stream stream) {
    if ((uintptr_t)live % 4 != 0) return fail(GA_EINVAL, "%s: live_rows is not 4-byte aligned", name);
    const int64_t items_row = p.path == 0 ? d * (int64_t)elem_size(dtype) / 16 : d;
    return launched(name, ga::launch_act(op, p.path, dtype, p.per_lane, p.grid, in, out, (int32_t)rows,
                                         (uint32_t)items_row, live, static_cast<hipStream_t>(stream)));
}

// Shared body of the elementwise entry points.  live may be null (all rows)
// unless the op requires it.
ga_status run_act(const char *name, int op, const void *in, void *out, int64_t rows, int64_t d,
                  int32_t dtype, const int32_t *live, bool live_required, ga_stream stream) {
    const int cols_in = op == ga::OP_SQUARED_RELU ? 1 : 2;
    ga_status st = check_rows(name, in, out, rows, d, dtype, cols_in);
    if (st != GA_OK) return st;
    if (live_required && live == nullptr) return fail(GA_EINVAL, "%s: live_rows is required", name);
    if ((uintptr_t)live % 4 != 0) return fail(GA_EINVAL, "%s: live_rows is not 4-byte aligned", name);
    if (rows * d >= kMaxItems) return fail(GA_EUNSUPPORTED, "%s: rows * d >= 2^31", name);
    if (rows == 0) return GA_OK;
    int cus = 0;
    if ((st = current_cus(&cus)) != GA_OK) return st;
    const ga_plan p = plan_act(rows, d, elem_size(dtype), vector_aligned(in, out, d, dtype), cus);
    return launch_act(name, op, in, out, rows, d, dtype, live, p, stream);
}

// ---------------------------------------------------------------------------
// Inverse normal CDF, for z = Phi^-1(target sparsity).  Newton's method on
// Phi(z) = p (p <= 1/2), with Phi(z) = erfc(-z / sqrt 2) / 2 from the C
// library, started from Abramowitz & Stegun 26.2.23 (a rational
// approximation with absolute error below 4.5e-4).
// ---------------------------------------------------------------------------
double normal_quantile_lower(double p) {
    const double t = std::sqrt(-2.0 * std::log(p));
    double z = -(t - (2.515517 + 0.802853 * t + 0.010328 * t * t) /
                         (1.0 + 1.432788 * t + 0.189269 * t * t + 0.001308 * t * t * t));
    const double inv_sqrt_2pi = 0.39894228040143267794;
    for (int it = 0; it < 60; ++it) {
        const double cdf = 0.5 * std::erfc(-z * 0.70710678118654752440);
        const double pdf = inv_sqrt_2pi * std::exp(-0.5 * z * z);
        if (pdf == 0.0) break;
        const double step = (cdf - p) / pdf;
        z -= step;
        if (std::fabs(step) <= 1e-16 * (1.0 + std::fabs(z))) break;
    }
    return z;
}

// ---------------------------------------------------------------------------
// The library's own split-row workspace, for ga_gelu_and_mul_sparse_noalloc:
// callers that cannot allocate device memory (stream capture, serving loops).
// One copy per device, holding the records of GA_SPLIT_PLAN_ROWS rows (64 KiB),
// kept until the process ends.  Host code never uses the array's name as an
// address: its per-device address comes from hipGetSymbolAddress.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)GA_SPLIT_PLAN_ROWS * ga::SPLIT_RECORD_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero fill by a kernel (a memset node recorded into a graph is avoided).
__global__ __launch_bounds__(256) void zero_scratch_kernel(uint4 *p, int32_t n) {
    const int32_t i = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = uint4{0u, 0u, 0u, 0u};
}

struct DeviceScratch {
    void *ptr = nullptr;   // device address of `scratch` on this device
    bool zeroed = false;   // a zero fill has been enqueued outside stream capture
};
std::mutex g_scratch_mu;
DeviceScratch g_scratch[64];

// The current device's scratch: its address is resolved once per device; the
// first call on a device also enqueues a zero fill on the caller's stream
// (the split kernels need every record zeroed before first use).  A fill made
// while the stream is being captured lands in the graph, and the next call
// fills again, so the memory is zeroed before any launch that runs eagerly.
ga_status device_scratch(ga_stream stream, void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(GA_EUNSUPPORTED, "device %d: at most 64 devices", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    DeviceScratch &ds = g_scratch[dev];
    if (ds.ptr == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(GA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        ds.ptr = p;
    }
    if (!ds.zeroed) {
        const hipStream_t s = static_cast<hipStream_t>(stream);
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(s, &cap);
        if (e != hipSuccess) return fail(GA_EHIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
        const int32_t n = (int32_t)(kScratchBytes / 16);
        uint4 *a = static_cast<uint4 *>(ds.ptr);
        void *args[] = {&a, (void *)&n};
        e = hipLaunchKernel((const void *)&zero_scratch_kernel, dim3((n + 255) / 256), dim3(256), args, 0, s);
        if (e != hipSuccess) return fail(GA_EHIP, "scratch zero fill: %s", hipGetErrorString(e));
        if (cap == hipStreamCaptureStatusNone) ds.zeroed = true;
    }
    *ptr = ds.ptr;
    return GA_OK;
}

// ---------------------------------------------------------------------------
// gelu_and_mul_sparse fused with the down projection
// ---------------------------------------------------------------------------
// The tiled form's plan from a measured table (planner_table_down.inc,
// written by tests/planner_rule.py --down from profiles/
// planner_sweep_down_bf16.csv): every instantiated geometry and slice count
// timed at (d, H) = (4096, 1024), (8192, 2048), (8192, 8192), (12288, 3072),
// (16384, 2048), (16384, 8192), (32768, 2048) and 13 token counts from 3 to
// 256.  A call takes the measured token count nearest to T in log2, then the
// nearest measured (d, H) in log2 distance, and that point's geometry with as
// many slices of d as bring its launch to that point's workgroup count.
#include "planner_table_down.inc"

struct TiledPick {
    bool staged;  // the staged form measured faster there (three or four tokens)
    int tm, bh, waves, kstep, depth;
    int64_t kc;
};

TiledPick pick_down_tiled(int64_t T, int64_t d, int64_t H) {
    int lo = -1, hi = -1;  // the measured token counts around T
    for (int i = 0; i < kDownTableN; ++i) {
        const int t = kDownTable[i].T;
        if (t <= T && (lo < 0 || t > lo)) lo = t;
        if (t >= T && (hi < 0 || t < hi)) hi = t;
    }
    const int64_t Tn = lo < 0 ? hi : hi < 0 ? lo : (T * T < (int64_t)lo * hi ? lo : hi);
    const DownTableEntry *best = nullptr;
    double best_dist = 0.0;
    for (int i = 0; i < kDownTableN; ++i) {
        const DownTableEntry &e = kDownTable[i];
        if (e.T != Tn) continue;
        const double a = std::log2((double)d / e.d), b = std::log2((double)H / e.H);
        const double dist = a * a + b * b;
        if (best == nullptr || dist < best_dist) {
            best = &e;
            best_dist = dist;
        }
    }
    TiledPick p{};
    p.staged = best->staged != 0 && T <= 4;
    p.tm = best->tm;
    p.bh = best->bh;
    p.waves = best->waves;
    p.kstep = best->kstep;
    p.depth = best->depth;
    const int64_t tiles = std::max<int64_t>((T + p.tm - 1) / p.tm * ((H + p.bh - 1) / p.bh), 1);
    int64_t slices = (best->grid + tiles / 2) / tiles;
    slices = std::min<int64_t>({std::max<int64_t>(slices, 1), ga::DOWN_MAX_SPLITS, (d + p.kstep - 1) / p.kstep});
    const int64_t kc = (d + slices - 1) / slices;
    p.kc = (kc + p.kstep - 1) / p.kstep * p.kstep;
    return p;
}

// The tiled form: workgroups of tm tokens x bh features x kc elements of d.
void fill_down_tiled_plan(int tm, int bh, int waves, int kstep, int depth, int64_t kc, int64_t T, int64_t d,
                          int64_t H, ga_down_plan *p) {
    std::memset(p, 0, sizeof *p);
    p->rows_per_block = tm;
    p->features_per_block = bh;
    p->waves = waves;
    p->k_step = kstep;
    p->k_chunk = (int32_t)kc;
    p->splits = (int32_t)((d + kc - 1) / kc);
    p->form = GA_DOWN_TILED;
    p->depth = depth;
    p->grid = (T + tm - 1) / tm * ((H + bh - 1) / bh) * p->splits;
}

ga_status check_down_sizes(const char *op, int64_t T, int64_t d, int64_t H, int32_t dtype) {
    if (T < 0 || d < 1 || H < 1)
        return fail(GA_EINVAL, "%s: negative or zero size (T %lld, d %lld, H %lld)", op, (long long)T,
                    (long long)d, (long long)H);
    if (elem_size(dtype) == 0) return fail(GA_EINVAL, "%s: unknown dtype %d", op, (int)dtype);
    if (dtype == GA_F32) return fail(GA_EUNSUPPORTED, "%s: fp32 has no fused form (bf16 and fp16 only)", op);
    if (T > GA_DOWN_MAX_ROWS)
        return fail(GA_EUNSUPPORTED, "%s: %lld tokens above %d", op, (long long)T, GA_DOWN_MAX_ROWS);
    if (d % 8 != 0 || d > GA_MAX_D)
        return fail(GA_EUNSUPPORTED, "%s: d = %lld is not a multiple of 8 up to %d", op, (long long)d, GA_MAX_D);
    if (H % 16 != 0 || H > GA_DOWN_MAX_H)
        return fail(GA_EUNSUPPORTED, "%s: H = %lld is not a multiple of 16 up to %d", op, (long long)H,
                    GA_DOWN_MAX_H);
    return GA_OK;
}

static_assert(sizeof(ga_down_plan) == 40 && offsetof(ga_down_plan, grid) == 32, "ga_down_plan layout");

// Field by field: the struct has padding before `grid`, which a caller need
// not have cleared.
bool same_down_plan(const ga_down_plan &a, const ga_down_plan &b) {
    return a.rows_per_block == b.rows_per_block && a.features_per_block == b.features_per_block &&
           a.waves == b.waves && a.k_step == b.k_step && a.k_chunk == b.k_chunk && a.splits == b.splits &&
           a.form == b.form && a.depth == b.depth && a.grid == b.grid;
}

// The decode and staged forms: every workgroup covers all of d for
// features_per_block output features and at most rows_per_block tokens.
void fill_down_whole_plan(int form, int tmax, int f, int waves, int64_t d, int64_t H, ga_down_plan *p) {
    std::memset(p, 0, sizeof *p);
    p->rows_per_block = tmax;
    p->features_per_block = f;
    p->waves = waves;
    p->k_step = 0;
    p->k_chunk = (int32_t)d;
    p->splits = 1;
    p->form = form;
    p->grid = (H + f - 1) / f;
}

bool down_whole_available(int form, int32_t dtype, int tmax, int f, int waves, int64_t d) {
    return form == GA_DOWN_DECODE ? ga::gelu_down_decode_available(dtype, tmax, f, waves, d)
                                  : ga::gelu_down_staged_available(dtype, tmax, f, waves, d);
}

// The decode and staged kernels the planner takes, by the longest row each
// serves (measured on MI355X at H = 2048): the first entry whose token
// capacity is the call's (rounded up to 1, 2 or 4) and whose reach covers d.
struct WholeChoice {
    int form, tmax;
    int64_t max_d;
    int f, waves;
};
const WholeChoice kWholeChoice[] = {
    {GA_DOWN_DECODE, 1, 16384, 4, 8},
    {GA_DOWN_DECODE, 1, 32768, 4, 16},
    {GA_DOWN_STAGED, 2, 16384, 4, 16},
    {GA_DOWN_STAGED, 4, 16384, 4, 16},
};

ga_status check_down_plan(const char *op, const ga_down_plan *p, int64_t T, int64_t d, int64_t H, int32_t dtype) {
    if (p->form == GA_DOWN_DECODE || p->form == GA_DOWN_STAGED) {
        const char *what = p->form == GA_DOWN_DECODE ? "decode" : "staged";
        if (!down_whole_available(p->form, dtype, p->rows_per_block, p->features_per_block, p->waves, d))
            return fail(GA_EINVAL,
                        "%s: no %s kernel for rows_per_block %d, features_per_block %d, waves %d at d = %lld", op,
                        what, (int)p->rows_per_block, (int)p->features_per_block, (int)p->waves, (long long)d);
        if (T > p->rows_per_block)
            return fail(GA_EINVAL, "%s: %lld tokens above the %s plan's %d", op, (long long)T, what,
                        (int)p->rows_per_block);
        ga_down_plan want;
        fill_down_whole_plan(p->form, p->rows_per_block, p->features_per_block, p->waves, d, H, &want);
        if (!same_down_plan(want, *p))
            return fail(GA_EINVAL,
                        "%s: a %s plan has k_step 0, k_chunk d, splits 1 and grid ceil(H / features_per_block)",
                        op, what);
        return GA_OK;
    }
    if (p->form == GA_DOWN_TILED) {
        if (!ga::gelu_down_tiled_available(dtype, p->rows_per_block, p->features_per_block, p->waves, p->k_step,
                                           p->depth))
            return fail(GA_EINVAL,
                        "%s: no tiled kernel for rows_per_block %d, features_per_block %d, waves %d, k_step %d, "
                        "depth %d", op, (int)p->rows_per_block, (int)p->features_per_block, (int)p->waves,
                        (int)p->k_step, (int)p->depth);
        if (p->k_chunk < p->k_step || p->k_chunk % p->k_step != 0)
            return fail(GA_EINVAL, "%s: k_chunk %d is not a positive multiple of k_step %d", op, (int)p->k_chunk,
                        (int)p->k_step);
        ga_down_plan want;
        fill_down_tiled_plan(p->rows_per_block, p->features_per_block, p->waves, p->k_step, p->depth, p->k_chunk, T,
                             d, H, &want);
        if (!same_down_plan(want, *p))
            return fail(GA_EINVAL, "%s: splits %d / grid %lld do not match the geometry (%d / %lld)", op,
                        (int)p->splits, (long long)p->grid, (int)want.splits, (long long)want.grid);
        if (p->splits > ga::DOWN_MAX_SPLITS)
            return fail(GA_EUNSUPPORTED, "%s: %d slices of d above %d", op, (int)p->splits, ga::DOWN_MAX_SPLITS);
        if (p->splits > 1 && p->grid / p->splits > ga::DOWN_MAX_TILES)
            return fail(GA_EUNSUPPORTED, "%s: %lld output tiles above %lld", op, (long long)(p->grid / p->splits),
                        (long long)ga::DOWN_MAX_TILES);
        if (p->grid * p->waves * 64 >= kMaxWorkItems)
            return fail(GA_EUNSUPPORTED, "%s: %lld work-items reach 2^32", op, (long long)(p->grid * p->waves * 64));
        return GA_OK;
    }
    return fail(GA_EINVAL, "%s: unknown plan form %d", op, (int)p->form);
}

size_t down_workspace_bytes(const ga_down_plan &p, int64_t T, int64_t d, int64_t H) {
    if (p.form == GA_DOWN_DECODE) return 0;  // everything stays on chip
    if (p.form == GA_DOWN_STAGED) return (size_t)ga::down_tiled_part_offset(T, d);  // the stored activation
    return ga::gelu_down_tiled_workspace_bytes(T, d, H, p.rows_per_block, p.features_per_block, p.k_chunk);
}

}  // namespace

// The planner.  allow_rep: the replicated-statistics path may be chosen (it
// has no round-trip form, so calls in that form pass false).
static ga_status plan_gelu(int64_t T, int64_t d, int32_t dtype, int32_t aligned, int32_t num_cus,
                           int32_t with_workspace, bool allow_rep, ga_plan *plan) {
    if (plan == nullptr) return fail(GA_EINVAL, "plan: null output");
    if (T < 0 || T > INT32_MAX || d < 1) return fail(GA_EINVAL, "plan: bad sizes");
    const size_t es = elem_size(dtype);
    if (es == 0) return fail(GA_EINVAL, "plan: unknown dtype %d", (int)dtype);
    if (d > GA_MAX_D) return fail(GA_EUNSUPPORTED, "plan: d above %d", GA_MAX_D);
    if (num_cus < 1) num_cus = 256;
    ga_plan p{};
    p.splits = 1;
    p.spin_limit = kDefaultSpinLimit;
    const int64_t nvec = (int64_t)d * (int64_t)es / 16;
    const int64_t nvec_ceil = (d * (int64_t)es + 15) / 16;
    if (nvec_ceil <= 32) {
        // Short rows, aligned or not: several rows per wavefront, a group of
        // G lanes per row with one vector each (measured on MI355X at
        // T = 65536: d = 64 bf16 14 % -> 52 % of peak, d = 128 29 % -> 62 %,
        // d = 256 57 % -> 71 %).
        int g = next_pow2((int)nvec_ceil);
        g = g < 4 ? 4 : g > 32 ? 32 : g;
        p.path = 3;
        p.lanes_per_row = g;
        p.per_lane = next_pow2((int)((nvec_ceil + g - 1) / g));
    } else if (aligned && ((size_t)d * es) % 16 == 0 && nvec <= 16 * 64 * 8) {
        int w, v, late;
        pick_row_geometry(nvec, T, &w, &v, &late);
        p.path = 0;
        p.waves_per_row = w;
        p.per_lane = v;
        p.up_late = late;
        // Few rows: share each row among several workgroups, either each
        // reducing the whole gate row itself (replicated statistics) or
        // exchanging partial statistics through the workspace (split rows;
        // about a microsecond), where the measured tables say it pays.
        int sw, sv, ss;
        if (allow_rep && pick_rep(nvec, T, with_workspace != 0, &sw, &sv, &ss)) {
            p.path = 4;
            p.waves_per_row = sw;
            p.per_lane = sv;
            p.up_late = 0;
            p.splits = ss;
        } else if (with_workspace && pick_split(nvec, T, &sw, &sv, &ss)) {
            p.waves_per_row = sw;
            p.per_lane = sv;
            p.up_late = 0;
            p.splits = ss;
        }
    } else if (nvec_ceil <= 16 * 64 * 8) {
        // Rows that are not 16-byte aligned: the same vectors, each one
        // unaligned 16-byte access.
        int w, v, late;
        pick_unaligned_geometry(nvec_ceil, T, &w, &v, &late);
        p.path = 2;
        p.waves_per_row = w;
        p.per_lane = v;
        p.up_late = late;
    } else {
        // Element path: up to 16 elements per lane, 1, 4 or 16 waves.
        const int64_t lanes = (d + 15) / 16;
        const int w = lanes <= 64 ? 1 : lanes <= 256 ? 4 : 16;
        const int64_t per = (d + 64 * w - 1) / (64 * w);
        p.path = 1;
        p.waves_per_row = w;
        p.per_lane = per <= 4 ? 4 : per <= 16 ? 16 : 64;
    }
    if (p.path == 3) {
        const int64_t rows_per_block = ga::ROWS_BLOCK / p.lanes_per_row;
        p.block = ga::ROWS_BLOCK;
        p.grid = (T + rows_per_block - 1) / rows_per_block;
    } else if (p.path == 4) {
        p.block = p.waves_per_row * 64;
        p.grid = ga::gelu_rep_grid(T, p.splits);
    } else {
        p.block = p.waves_per_row * 64;
        p.grid = T * p.splits;
    }
    const ga_status st = check_work_items(p, T);
    if (st != GA_OK) return st;
    *plan = p;
    return GA_OK;
}

extern "C" {

// ---------------------------------------------------------------------------
// gelu_and_mul_sparse
// ---------------------------------------------------------------------------
ga_status ga_plan_gelu_and_mul_sparse(int64_t T, int64_t d, int32_t dtype, int32_t aligned,
                                      int32_t num_cus, int32_t with_workspace, ga_plan *plan) {
    return plan_gelu(T, d, dtype, aligned, num_cus, with_workspace, true, plan);
}

size_t ga_gelu_and_mul_sparse_workspace_bytes(int64_t T) {
    return T < 1 ? 0 : ga::split_workspace_bytes(std::min<int64_t>(T, kSplitMaxRows));
}

ga_status ga_gelu_and_mul_sparse_with_plan(const void *in, void *out, int64_t T, int64_t d, int32_t dtype,
                                           float z, const int32_t *live_rows, const ga_plan *plan,
                                           void *workspace, size_t workspace_bytes, ga_stream stream) {
    ga_status st = check_rows("ga_gelu_and_mul_sparse", in, out, T, d, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: z is not finite");
    if (plan == nullptr) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: null plan");
    if ((st = check_gelu_plan(plan, T, d, dtype)) != GA_OK) return st;
    if ((plan->path == 0 || plan->path == 4) && !vector_aligned(in, out, d, dtype))
        return fail(GA_EUNSUPPORTED, "ga_gelu_and_mul_sparse: vector path needs 16-byte rows and bases");
    if ((st = check_workspace(*plan, T, workspace, workspace_bytes)) != GA_OK) return st;
    if (T == 0) return GA_OK;
    return launch_gelu(in, out, T, d, dtype, z, live_rows, *plan, workspace, stream);
}

ga_status ga_gelu_and_mul_sparse_ex(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, float z,
                                    const int32_t *live_rows, int32_t flags, void *workspace,
                                    size_t workspace_bytes, ga_stream stream) {
    ga_status st = check_rows("ga_gelu_and_mul_sparse", in, out, T, d, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: z is not finite");
    if ((flags & ~GA_ROUND_INTERMEDIATES) != 0)
        return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: unknown flag bits 0x%x", (unsigned)flags);
    if ((uintptr_t)live_rows % 4 != 0)
        return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: live_rows is not 4-byte aligned");
    if (T == 0) return GA_OK;
    // The round-trip form has no split-row kernel.
    const bool have_ws = !(flags & GA_ROUND_INTERMEDIATES) && workspace != nullptr &&
                         (uintptr_t)workspace % 256 == 0 && T <= kSplitMaxRows &&
                         workspace_bytes >= ga::split_workspace_bytes(T);
    int cus = 256;
    if (have_ws && (st = current_cus(&cus)) != GA_OK) return st;
    ga_plan p;
    if ((st = plan_gelu(T, d, dtype, vector_aligned(in, out, d, dtype), cus, have_ws,
                        !(flags & GA_ROUND_INTERMEDIATES), &p)) != GA_OK)
        return st;
    p.flags = flags;
    return launch_gelu(in, out, T, d, dtype, z, live_rows, p, workspace, stream);
}

ga_status ga_gelu_and_mul_sparse_ws(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, float z,
                                    const int32_t *live_rows, void *workspace, size_t workspace_bytes,
                                    ga_stream stream) {
    return ga_gelu_and_mul_sparse_ex(in, out, T, d, dtype, z, live_rows, 0, workspace, workspace_bytes, stream);
}

ga_status ga_gelu_and_mul_sparse(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, float z,
                                 const int32_t *live_rows, ga_stream stream) {
    ga_status st = check_rows("ga_gelu_and_mul_sparse", in, out, T, d, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: z is not finite");
    if (T == 0) return GA_OK;
    ga_plan p;
    if ((st = ga_plan_gelu_and_mul_sparse(T, d, dtype, vector_aligned(in, out, d, dtype), 256, 0, &p)) != GA_OK)
        return st;
    return launch_gelu(in, out, T, d, dtype, z, live_rows, p, nullptr, stream);
}

ga_status ga_gelu_and_mul_sparse_noalloc(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, float z,
                                         const int32_t *live_rows, ga_stream stream) {
    const char *name = "ga_gelu_and_mul_sparse_noalloc";
    ga_status st = check_rows(name, in, out, T, d, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "%s: z is not finite", name);
    if ((uintptr_t)live_rows % 4 != 0) return fail(GA_EINVAL, "%s: live_rows is not 4-byte aligned", name);
    if (T > GA_SPLIT_PLAN_ROWS)
        return fail(GA_EUNSUPPORTED,
                    "%s: %lld rows; its scratch holds the split records of at most %d rows (calls of more "
                    "rows never split: ga_gelu_and_mul_sparse serves them and needs no memory either)",
                    name, (long long)T, GA_SPLIT_PLAN_ROWS);
    if (T == 0) return GA_OK;
    void *ws = nullptr;
    if ((st = device_scratch(stream, &ws)) != GA_OK) return st;
    return ga_gelu_and_mul_sparse_ex(in, out, T, d, dtype, z, live_rows, 0, ws, kScratchBytes, stream);
}

double ga_z_from_sparsity(double target_sparsity) {
    const double p = target_sparsity;
    if (!(p > 0.0 && p < 1.0)) return std::nan("");
    if (p == 0.5) return 0.0;
    return p < 0.5 ? normal_quantile_lower(p) : -normal_quantile_lower(1.0 - p);
}

// ---------------------------------------------------------------------------
// Elementwise family
// ---------------------------------------------------------------------------
ga_status ga_plan_silu_and_mul_bounded(int64_t M, int64_t d, int32_t dtype, int32_t aligned, int32_t num_cus,
                                       ga_plan *plan) {
    if (plan == nullptr) return fail(GA_EINVAL, "plan: null output");
    if (M < 0 || M > INT32_MAX || d < 1) return fail(GA_EINVAL, "plan: bad sizes");
    const size_t es = elem_size(dtype);
    if (es == 0) return fail(GA_EINVAL, "plan: unknown dtype %d", (int)dtype);
    if (d > GA_MAX_D) return fail(GA_EUNSUPPORTED, "plan: d above %d", GA_MAX_D);
    if (num_cus < 1) return fail(GA_EINVAL, "plan: num_cus %d", (int)num_cus);
    *plan = plan_act(M, d, es, aligned != 0, num_cus);
    return GA_OK;
}

ga_status ga_silu_and_mul_bounded_with_plan(const void *in, void *out, int64_t M, int64_t d, int32_t dtype,
                                            const int32_t *live_rows, const ga_plan *plan, ga_stream stream) {
    const char *name = "ga_silu_and_mul_bounded";
    ga_status st = check_rows(name, in, out, M, d, dtype);
    if (st != GA_OK) return st;
    if (live_rows == nullptr) return fail(GA_EINVAL, "%s: live_rows is required", name);
    if ((uintptr_t)live_rows % 4 != 0) return fail(GA_EINVAL, "%s: live_rows is not 4-byte aligned", name);
    if (plan == nullptr) return fail(GA_EINVAL, "%s: null plan", name);
    if ((st = check_act_plan(plan, ga::OP_SILU_MUL, M, d, dtype)) != GA_OK) return st;
    if (plan->path == 0 && !vector_aligned(in, out, d, dtype))
        return fail(GA_EUNSUPPORTED, "%s: vector path needs 16-byte rows and bases", name);
    if (M == 0) return GA_OK;
    return launch_act(name, ga::OP_SILU_MUL, in, out, M, d, dtype, live_rows, *plan, stream);
}

ga_status ga_silu_and_mul_bounded(const void *in, void *out, int64_t M, int64_t d, int32_t dtype,
                                  const int32_t *live_rows, ga_stream stream) {
    return run_act("ga_silu_and_mul_bounded", ga::OP_SILU_MUL, in, out, M, d, dtype, live_rows, true, stream);
}

ga_status ga_gelu_and_mul(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, int32_t approximate,
                          const int32_t *live_rows, ga_stream stream) {
    if (approximate != GA_GELU_ERF && approximate != GA_GELU_TANH)
        return fail(GA_EINVAL, "ga_gelu_and_mul: approximate must be GA_GELU_ERF or GA_GELU_TANH");
    const int op = approximate == GA_GELU_TANH ? ga::OP_GELU_TANH_MUL : ga::OP_GELU_ERF_MUL;
    return run_act("ga_gelu_and_mul", op, in, out, T, d, dtype, live_rows, false, stream);
}

ga_status ga_squared_relu_bounded(const void *in, void *out, int64_t M, int64_t d, int32_t dtype,
                                  const int32_t *live_rows, ga_stream stream) {
    return run_act("ga_squared_relu_bounded", ga::OP_SQUARED_RELU, in, out, M, d, dtype, live_rows, true, stream);
}

// ---------------------------------------------------------------------------
// Measurement aid and diagnostics
// ---------------------------------------------------------------------------
ga_status ga_stream_xor_rows(const void *in, void *out, int64_t rows, int64_t w_bytes, ga_stream stream) {
    if (in == nullptr || out == nullptr) return fail(GA_EINVAL, "ga_stream_xor_rows: null pointer");
    if (rows < 0 || rows > INT32_MAX || w_bytes < 16 || w_bytes % 16 != 0)
        return fail(GA_EINVAL, "ga_stream_xor_rows: bad sizes");
    if ((uintptr_t)in % 16 != 0 || (uintptr_t)out % 16 != 0)
        return fail(GA_EINVAL, "ga_stream_xor_rows: pointers must be 16-byte aligned");
    const int64_t nvec = w_bytes / 16;
    if (rows * nvec >= kMaxItems) return fail(GA_EUNSUPPORTED, "ga_stream_xor_rows: too large");
    if (overlaps(in, (size_t)rows * 2 * (size_t)w_bytes, out, (size_t)rows * (size_t)w_bytes))
        return fail(GA_EINVAL, "ga_stream_xor_rows: in and out overlap");
    if (rows == 0) return GA_OK;
    int cus = 0;
    ga_status st = current_cus(&cus);
    if (st != GA_OK) return st;
    // Two vectors per lane, one pass over the rows (measured fastest).
    int64_t g = (rows * nvec + ga::SILU_BLOCK * 2 - 1) / (ga::SILU_BLOCK * 2);
    if (g > (int64_t)cus * 64) g = (int64_t)cus * 64;
    return launched("ga_stream_xor_rows", ga::launch_xor_rows(g, in, out, (int32_t)rows, (uint32_t)nvec,
                                                              static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// gelu_and_mul_sparse fused with the down projection
// ---------------------------------------------------------------------------
ga_status ga_plan_gelu_and_mul_sparse_down(int64_t T, int64_t d, int64_t H, int32_t dtype, ga_down_plan *plan) {
    const char *name = "ga_plan_gelu_and_mul_sparse_down";
    if (plan == nullptr) return fail(GA_EINVAL, "%s: null plan", name);
    ga_status st = check_down_sizes(name, T, d, H, dtype);
    if (st != GA_OK) return st;
    // One token: the decode form (one launch, no workspace); two: the staged
    // form; where their rows fit.  Three or more: the measured table's
    // tiled plan, or the staged form where the table found it faster (three
    // or four tokens) and its row fits.
    const TiledPick t = pick_down_tiled(T < 1 ? 1 : T, d, H);
    if (T <= 4) {
        const int tmax = T <= 1 ? 1 : T <= 2 ? 2 : 4;
        if (T <= 2 || t.staged)
            for (const WholeChoice &c : kWholeChoice)
                if (c.tmax == tmax && d <= c.max_d && down_whole_available(c.form, dtype, tmax, c.f, c.waves, d)) {
                    fill_down_whole_plan(c.form, tmax, c.f, c.waves, d, H, plan);
                    return GA_OK;
                }
    }
    fill_down_tiled_plan(t.tm, t.bh, t.waves, t.kstep, t.depth, t.kc, T, d, H, plan);
    return GA_OK;
}

size_t ga_gelu_and_mul_sparse_down_workspace_bytes(int64_t T, int64_t d, int64_t H, const ga_down_plan *plan) {
    ga_down_plan p;
    if (plan == nullptr) {
        if (ga_plan_gelu_and_mul_sparse_down(T, d, H, GA_BF16, &p) != GA_OK) return 0;
        plan = &p;
    }
    if (T < 1 || d < 1 || H < 1) return 0;
    return down_workspace_bytes(*plan, T, d, H);
}

ga_status ga_gelu_and_mul_sparse_down_with_plan(const void *gu, const void *w, void *y, int64_t T, int64_t d,
                                                int64_t H, int32_t dtype, float z, const int32_t *live_rows,
                                                const ga_down_plan *plan, void *workspace,
                                                size_t workspace_bytes, ga_stream stream) {
    const char *name = "ga_gelu_and_mul_sparse_down";
    if (gu == nullptr || w == nullptr || y == nullptr) return fail(GA_EINVAL, "%s: null gu/w/y pointer", name);
    if (plan == nullptr) return fail(GA_EINVAL, "%s: null plan", name);
    ga_status st = check_down_sizes(name, T, d, H, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "%s: z is not finite", name);
    if ((uintptr_t)live_rows % 4 != 0) return fail(GA_EINVAL, "%s: live_rows is not 4-byte aligned", name);
    if ((uintptr_t)gu % 16 != 0 || (uintptr_t)w % 16 != 0 || (uintptr_t)y % 16 != 0)
        return fail(GA_EUNSUPPORTED, "%s: gu, w and y must be 16-byte aligned", name);
    const size_t es = elem_size(dtype);
    const size_t y_bytes = (size_t)T * (size_t)H * es;
    if (T > 0 && (overlaps(gu, (size_t)T * 2 * (size_t)d * es, y, y_bytes) ||
                  overlaps(w, (size_t)H * (size_t)d * es, y, y_bytes)))
        return fail(GA_EINVAL, "%s: y overlaps gu or w", name);
    if ((st = check_down_plan(name, plan, T, d, H, dtype)) != GA_OK) return st;
    if (T == 0) return GA_OK;
    if (plan->form == GA_DOWN_DECODE)
        return launched(name, ga::launch_gelu_down_decode(dtype, plan->rows_per_block, plan->features_per_block,
                                                          plan->waves, gu, w, y,
                                                          (int32_t)T, (int32_t)d, (int32_t)H, z, live_rows,
                                                          static_cast<hipStream_t>(stream)));
    const size_t need = down_workspace_bytes(*plan, T, d, H);
    if (workspace == nullptr || (uintptr_t)workspace % 256 != 0)
        return fail(GA_EINVAL, "%s: a 256-byte aligned workspace is required", name);
    if (workspace_bytes < need)
        return fail(GA_EINVAL, "%s: workspace of %zu bytes, the plan needs %zu", name, workspace_bytes, need);
    if (overlaps(workspace, need, gu, (size_t)T * 2 * (size_t)d * es) ||
        overlaps(workspace, need, w, (size_t)H * (size_t)d * es) || overlaps(workspace, need, y, y_bytes))
        return fail(GA_EINVAL, "%s: the workspace overlaps gu, w or y", name);
    if (plan->form == GA_DOWN_STAGED || plan->form == GA_DOWN_TILED) {
        // The activation of the call's rows into the workspace, by the row
        // kernel ga_gelu_and_mul_sparse would run (no workspace of its own),
        // then the product against it.
        void *a = static_cast<unsigned char *>(workspace) + ga::DOWN_ACT_OFFSET;
        ga_plan act;
        if ((st = ga_plan_gelu_and_mul_sparse(T, d, dtype, vector_aligned(gu, a, d, dtype), 256, 0, &act)) != GA_OK)
            return st;
        if ((st = launch_gelu(gu, a, T, d, dtype, z, live_rows, act, nullptr, stream)) != GA_OK) return st;
        if (plan->form == GA_DOWN_STAGED)
            return launched(name, ga::launch_gelu_down_staged(dtype, plan->rows_per_block, plan->features_per_block,
                                                              plan->waves, a, w, y, (int32_t)T, (int32_t)d,
                                                              (int32_t)H, live_rows,
                                                              static_cast<hipStream_t>(stream)));
        return launched(name, ga::launch_gelu_down_tiled(dtype, plan->rows_per_block, plan->features_per_block,
                                                         plan->waves, plan->k_step, plan->depth, plan->k_chunk, a, w, y,
                                                         (int32_t)T, (int32_t)d, (int32_t)H, live_rows, workspace,
                                                         static_cast<hipStream_t>(stream)));
    }
    return fail(GA_EINVAL, "%s: unknown plan form %d", name, (int)plan->form);  // unreachable: checked above
}

ga_status ga_gelu_and_mul_sparse_down(const void *gu, const void *w, void *y, int64_t T, int64_t d, int64_t H,
                                      int32_t dtype, float z, const int32_t *live_rows, void *workspace,
                                      size_t workspace_bytes, ga_stream stream) {
    if (gu == nullptr || w == nullptr || y == nullptr)
        return fail(GA_EINVAL, "ga_gelu_and_mul_sparse_down: null gu/w/y pointer");
    ga_down_plan p;
    ga_status st = ga_plan_gelu_and_mul_sparse_down(T, d, H, dtype, &p);
    if (st != GA_OK) return st;
    return ga_gelu_and_mul_sparse_down_with_plan(gu, w, y, T, d, H, dtype, z, live_rows, &p, workspace,
                                                 workspace_bytes, stream);
}

const char *ga_status_str(int32_t status) {
    switch (status) {
    case GA_OK: return "GA_OK";
    case GA_EINVAL: return "GA_EINVAL";
    case GA_EUNSUPPORTED: return "GA_EUNSUPPORTED";
    case GA_EHIP: return "GA_EHIP";
    default: return "GA_UNKNOWN_STATUS";
    }
}

const char *ga_last_error(void) { return g_last_error; }

int32_t ga_version(void) { return 100; }

}  // extern "C"
