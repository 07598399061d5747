// The C-ABI of libga.so: argument checks, the launch heuristic, dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect and the checks can be exercised without a GPU.  The only HIP
// calls are the device / compute-unit query (cached per device) and the
// kernel launch itself; nothing allocates, copies or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/ga.h"
#include "ga_internal.h"

namespace {

thread_local char g_last_error[256] = "";

ga_status fail(ga_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
ga_status fail(ga_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

size_t elem_size(int32_t dtype) {
    return dtype == GA_F32 ? 4 : (dtype == GA_F16 || dtype == GA_BF16) ? 2 : 0;
}

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool vector_aligned(const void *in, const void *out, int64_t d, int32_t dtype) {
    return ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
           ((size_t)d * elem_size(dtype)) % 16 == 0;
}

int next_pow2(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Shared checks of the two operations: [rows, 2d] in, [rows, d] out.
ga_status check_rows(const char *op, const void *in, const void *out, int64_t rows, int64_t d,
                     int32_t dtype) {
    if (in == nullptr || out == nullptr) return fail(GA_EINVAL, "%s: null in/out pointer", op);
    if (rows < 0 || rows > INT32_MAX) return fail(GA_EINVAL, "%s: row count %lld out of [0, 2^31)", op, (long long)rows);
    if (d < 1) return fail(GA_EINVAL, "%s: d = %lld must be >= 1", op, (long long)d);
    const size_t es = elem_size(dtype);
    if (es == 0) return fail(GA_EINVAL, "%s: unknown dtype %d", op, (int)dtype);
    if (d > GA_MAX_D) return fail(GA_EUNSUPPORTED, "%s: d = %lld above %d", op, (long long)d, GA_MAX_D);
    if ((uintptr_t)in % es != 0 || (uintptr_t)out % es != 0)
        return fail(GA_EINVAL, "%s: pointer not aligned to the element size", op);
    const size_t in_bytes = (size_t)rows * 2 * (size_t)d * es;
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
    if (e != hipSuccess || c <= 0) return fail(GA_EHIP, "hipDeviceGetAttribute(CU count): %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) g_cus[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return GA_OK;
}

ga_status launched(const char *op, hipError_t e) {
    if (e != hipSuccess) return fail(GA_EHIP, "%s: launch failed: %s", op, hipGetErrorString(e));
    return GA_OK;
}

// ---------------------------------------------------------------------------
// Geometry checks shared by the planners and the *_with_plan entry points.
// ---------------------------------------------------------------------------
constexpr uint32_t kDefaultSpinLimit = 1u << 16;
constexpr int64_t kSplitMaxRows = 65535;  // grid y limit

ga_status check_gelu_plan(const ga_plan *p, int64_t T, int64_t d, int32_t dtype) {
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
            if (T > kSplitMaxRows) return fail(GA_EUNSUPPORTED, "gelu plan: split rows need T <= %lld",
                                               (long long)kSplitMaxRows);
        }
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

ga_status launch_gelu(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, float z,
                      const int32_t *live, const ga_plan &p, void *workspace, ga_stream stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.path == 0) {
        const int32_t nvec = (int32_t)(d * (int64_t)elem_size(dtype) / 16);
        if (p.splits > 1)
            return launched("ga_gelu_and_mul_sparse",
                            ga::launch_gelu_split(dtype, p.waves_per_row, p.per_lane, p.splits, in, out, (int32_t)T,
                                                  (int32_t)d, nvec, z, live, workspace, p.spin_limit, s));
        return launched("ga_gelu_and_mul_sparse",
                        ga::launch_gelu_vec(dtype, p.waves_per_row, p.per_lane, p.up_late, T, in, out, (int32_t)T,
                                            (int32_t)d, nvec, z, live, s));
    }
    return launched("ga_gelu_and_mul_sparse",
                    ga::launch_gelu_elem(dtype, p.waves_per_row, p.per_lane, T, in, out, (int32_t)T,
                                         (int32_t)d, z, live, s));
}

// Vectors per lane and waves for `nvec` vectors of one workgroup: 1 vector
// per lane up to 512 vectors, 2 up to 1024, else 4 (at most max_v); enough
// waves (at most 16) to cover them.  Measured on MI355X: wide workgroups with
// a few vectors per lane keep the most bytes in flight per compute unit.
void pick_waves(int64_t nvec, int max_v, int *w_out, int *v_out) {
    int target = nvec <= 512 ? 1 : nvec <= 1024 ? 2 : 4;
    if (target > max_v) target = max_v;
    int w = next_pow2((nvec + 64 * target - 1) / (64 * target));
    if (w > 16) w = 16;
    *w_out = w;
    *v_out = next_pow2((nvec + 64 * w - 1) / (64 * w));
}

// Flat item count of the live region must fit the kernels' 32-bit indices.
constexpr int64_t kSiluMaxItems = (int64_t)1 << 31;

ga_status launch_silu(const void *in, void *out, int64_t M, int64_t d, int32_t dtype,
                      const int32_t *live, const ga_plan &p, ga_stream stream) {
    const int64_t items_row = p.path == 0 ? d * (int64_t)elem_size(dtype) / 16 : d;
    return launched("ga_silu_and_mul_bounded",
                    ga::launch_silu(p.path, dtype, p.per_lane, p.grid, in, out, (int32_t)M,
                                    (uint32_t)items_row, live, static_cast<hipStream_t>(stream)));
}

ga_status check_silu_plan(const ga_plan *p, int64_t M, int64_t d, int32_t dtype) {
    if (!ga::silu_available(p->path, dtype, p->per_lane))
        return fail(GA_EUNSUPPORTED, "silu plan: no kernel for path=%d per_lane=%d", p->path, p->per_lane);
    if (p->grid < 1 || p->grid > INT32_MAX) return fail(GA_EINVAL, "silu plan: grid %lld", (long long)p->grid);
    const int64_t items_row = p->path == 0 ? d * (int64_t)elem_size(dtype) / 16 : d;
    // The kernels step through items with 32-bit counters: both the region
    // and one grid-wide step must stay below 2^31 so their sum cannot wrap.
    if (p->grid * ga::SILU_BLOCK * p->per_lane > kSiluMaxItems)
        return fail(GA_EUNSUPPORTED, "silu plan: grid too large for 32-bit item indices");
    if (M * items_row >= kSiluMaxItems)
        return fail(GA_EUNSUPPORTED, "silu: M * d too large for 32-bit item indices");
    return GA_OK;
}

}  // namespace

extern "C" {

ga_status ga_plan_gelu_and_mul_sparse(int64_t T, int64_t d, int32_t dtype, int32_t aligned,
                                      int32_t num_cus, int32_t with_workspace, ga_plan *plan) {
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
    if (aligned && ((size_t)d * es) % 16 == 0 && nvec <= 16 * 64 * 8) {
        int w, v;
        pick_waves(nvec, 8, &w, &v);
        p.path = 0;
        p.waves_per_row = w;
        p.per_lane = v;
        // With at least ~4 rows per compute unit, loading up after the
        // statistics frees registers for more resident rows; with fewer rows
        // the shorter dependency chain of loading it early wins.
        p.up_late = T >= 1024 ? 1 : 0;
        // Few long rows: split each over several workgroups that exchange
        // partial statistics.  Measured on MI355X, the exchange costs about
        // a microsecond, which pays off once a row has >= 2048 vectors
        // (32 KB of bf16 gate) and there are at most 64 rows per 2048
        // vectors; splits aim at ~512-vector chunks and ~256 workgroups.
        if (with_workspace && T >= 1 && T <= kSplitMaxRows && nvec >= 2048 && T * 2048 <= 64 * nvec) {
            int64_t splits = std::min<int64_t>(nvec / 512, std::max<int64_t>(2, 256 / T));
            if (splits > ga::SPLIT_MAX) splits = ga::SPLIT_MAX;
            int sw, sv;
            pick_waves((nvec + splits - 1) / splits, 4, &sw, &sv);
            const int64_t chunk = (int64_t)sw * 64 * sv;
            splits = (nvec + chunk - 1) / chunk;   // every split owns >= 1 vector
            if (splits >= 2 && splits <= ga::SPLIT_MAX) {
                p.waves_per_row = sw;
                p.per_lane = sv;
                p.up_late = 0;
                p.splits = (int32_t)splits;
            }
        }
    } else {
        // Element path: up to 16 elements per lane, 1, 4 or 16 waves.
        const int64_t lanes = (d + 15) / 16;
        const int w = lanes <= 64 ? 1 : lanes <= 256 ? 4 : 16;
        const int64_t per = (d + 64 * w - 1) / (64 * w);
        p.path = 1;
        p.waves_per_row = w;
        p.per_lane = per <= 4 ? 4 : per <= 16 ? 16 : 64;
    }
    p.block = p.waves_per_row * 64;
    p.grid = T * p.splits;
    *plan = p;
    return GA_OK;
}

size_t ga_gelu_and_mul_sparse_workspace_bytes(int64_t T) {
    return T < 1 ? 0 : ga::split_workspace_bytes(T > kSplitMaxRows ? kSplitMaxRows : T);
}

ga_status ga_plan_silu_and_mul_bounded(int64_t M, int64_t d, int32_t dtype, int32_t aligned,
                                       int32_t num_cus, ga_plan *plan) {
    if (plan == nullptr) return fail(GA_EINVAL, "plan: null output");
    if (M < 0 || M > INT32_MAX || d < 1) return fail(GA_EINVAL, "plan: bad sizes");
    const size_t es = elem_size(dtype);
    if (es == 0) return fail(GA_EINVAL, "plan: unknown dtype %d", (int)dtype);
    if (d > GA_MAX_D) return fail(GA_EUNSUPPORTED, "plan: d above %d", GA_MAX_D);
    if (num_cus < 1) return fail(GA_EINVAL, "plan: num_cus %d", (int)num_cus);
    ga_plan p{};
    p.path = (aligned && ((size_t)d * es) % 16 == 0) ? 0 : 1;
    p.per_lane = 1;
    p.waves_per_row = 0;
    p.block = ga::SILU_BLOCK;
    // One item per lane per step and up to sixteen workgroups per compute
    // unit (measured best on MI355X for the decode buffer); the grid-stride
    // loop covers larger buffers.  The live count plays no part.
    const int64_t items = M * (p.path == 0 ? d * (int64_t)es / 16 : d);
    const int64_t per_wg = (int64_t)ga::SILU_BLOCK * p.per_lane;
    int64_t g = (items + per_wg - 1) / per_wg;
    const int64_t cap = (int64_t)num_cus * 16;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    p.grid = g;
    *plan = p;
    return GA_OK;
}

ga_status check_workspace(const ga_plan &p, int64_t T, const void *workspace, size_t workspace_bytes) {
    if (p.path != 0 || p.splits <= 1) return GA_OK;
    if (workspace == nullptr) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: a split plan needs a workspace");
    if ((uintptr_t)workspace % 256 != 0) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: workspace not 256-byte aligned");
    if (workspace_bytes < ga::split_workspace_bytes(T))
        return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: workspace of %zu bytes, %zu needed", workspace_bytes,
                    ga::split_workspace_bytes(T));
    return GA_OK;
}

ga_status ga_gelu_and_mul_sparse_with_plan(const void *in, void *out, int64_t T, int64_t d,
                                           int32_t dtype, float z, const int32_t *live_rows,
                                           const ga_plan *plan, void *workspace, size_t workspace_bytes,
                                           ga_stream stream) {
    ga_status st = check_rows("ga_gelu_and_mul_sparse", in, out, T, d, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: z is not finite");
    if (plan == nullptr) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: null plan");
    if ((st = check_gelu_plan(plan, T, d, dtype)) != GA_OK) return st;
    if (plan->path == 0 && !vector_aligned(in, out, d, dtype))
        return fail(GA_EUNSUPPORTED, "ga_gelu_and_mul_sparse: vector path needs 16-byte rows and bases");
    if ((st = check_workspace(*plan, T, workspace, workspace_bytes)) != GA_OK) return st;
    if (T == 0) return GA_OK;
    return launch_gelu(in, out, T, d, dtype, z, live_rows, *plan, workspace, stream);
}

ga_status ga_gelu_and_mul_sparse_ws(const void *in, void *out, int64_t T, int64_t d, int32_t dtype, float z,
                                    const int32_t *live_rows, void *workspace, size_t workspace_bytes,
                                    ga_stream stream) {
    ga_status st = check_rows("ga_gelu_and_mul_sparse", in, out, T, d, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: z is not finite");
    if (T == 0) return GA_OK;
    const bool have_ws = workspace != nullptr && (uintptr_t)workspace % 256 == 0 &&
                         workspace_bytes >= ga::split_workspace_bytes(T > kSplitMaxRows ? 1 : T);
    int cus = 256;
    if (have_ws && (st = current_cus(&cus)) != GA_OK) return st;
    ga_plan p;
    if ((st = ga_plan_gelu_and_mul_sparse(T, d, dtype, vector_aligned(in, out, d, dtype), cus, have_ws, &p)) != GA_OK)
        return st;
    if ((st = check_workspace(p, T, workspace, workspace_bytes)) != GA_OK) return st;
    return launch_gelu(in, out, T, d, dtype, z, live_rows, p, workspace, stream);
}

ga_status ga_gelu_and_mul_sparse(const void *in, void *out, int64_t T, int64_t d, int32_t dtype,
                                 float z, const int32_t *live_rows, ga_stream stream) {
    ga_status st = check_rows("ga_gelu_and_mul_sparse", in, out, T, d, dtype);
    if (st != GA_OK) return st;
    if (!std::isfinite(z)) return fail(GA_EINVAL, "ga_gelu_and_mul_sparse: z is not finite");
    if (T == 0) return GA_OK;
    ga_plan p;
    if ((st = ga_plan_gelu_and_mul_sparse(T, d, dtype, vector_aligned(in, out, d, dtype), 256, 0, &p)) != GA_OK)
        return st;
    return launch_gelu(in, out, T, d, dtype, z, live_rows, p, nullptr, stream);
}

ga_status ga_silu_and_mul_bounded_with_plan(const void *in, void *out, int64_t M, int64_t d,
                                            int32_t dtype, const int32_t *live_rows,
                                            const ga_plan *plan, ga_stream stream) {
    ga_status st = check_rows("ga_silu_and_mul_bounded", in, out, M, d, dtype);
    if (st != GA_OK) return st;
    if (live_rows == nullptr) return fail(GA_EINVAL, "ga_silu_and_mul_bounded: live_rows is required");
    if (plan == nullptr) return fail(GA_EINVAL, "ga_silu_and_mul_bounded: null plan");
    if ((st = check_silu_plan(plan, M, d, dtype)) != GA_OK) return st;
    if (plan->path == 0 && !vector_aligned(in, out, d, dtype))
        return fail(GA_EUNSUPPORTED, "ga_silu_and_mul_bounded: vector path needs 16-byte rows and bases");
    if (M == 0) return GA_OK;
    return launch_silu(in, out, M, d, dtype, live_rows, *plan, stream);
}

ga_status ga_silu_and_mul_bounded(const void *in, void *out, int64_t M, int64_t d, int32_t dtype,
                                  const int32_t *live_rows, ga_stream stream) {
    ga_status st = check_rows("ga_silu_and_mul_bounded", in, out, M, d, dtype);
    if (st != GA_OK) return st;
    if (live_rows == nullptr) return fail(GA_EINVAL, "ga_silu_and_mul_bounded: live_rows is required");
    const int64_t items = M * d;  // upper bound on items of either path
    if (items >= kSiluMaxItems) return fail(GA_EUNSUPPORTED, "ga_silu_and_mul_bounded: M * d >= 2^31");
    if (M == 0) return GA_OK;
    int cus = 0;
    if ((st = current_cus(&cus)) != GA_OK) return st;
    ga_plan p;
    if ((st = ga_plan_silu_and_mul_bounded(M, d, dtype, vector_aligned(in, out, d, dtype), cus, &p)) != GA_OK)
        return st;
    return launch_silu(in, out, M, d, dtype, live_rows, p, stream);
}

ga_status ga_stream_xor_rows(const void *in, void *out, int64_t rows, int64_t w_bytes, ga_stream stream) {
    if (in == nullptr || out == nullptr) return fail(GA_EINVAL, "ga_stream_xor_rows: null pointer");
    if (rows < 0 || rows > INT32_MAX || w_bytes < 16 || w_bytes % 16 != 0)
        return fail(GA_EINVAL, "ga_stream_xor_rows: bad sizes");
    if ((uintptr_t)in % 16 != 0 || (uintptr_t)out % 16 != 0)
        return fail(GA_EINVAL, "ga_stream_xor_rows: pointers must be 16-byte aligned");
    const int64_t nvec = w_bytes / 16;
    if (rows * nvec >= kSiluMaxItems) return fail(GA_EUNSUPPORTED, "ga_stream_xor_rows: too large");
    if (overlaps(in, (size_t)rows * 2 * (size_t)w_bytes, out, (size_t)rows * (size_t)w_bytes))
        return fail(GA_EINVAL, "ga_stream_xor_rows: in and out overlap");
    if (rows == 0) return GA_OK;
    int cus = 0;
    ga_status st = current_cus(&cus);
    if (st != GA_OK) return st;
    int64_t g = (rows * nvec + ga::SILU_BLOCK * 4 - 1) / (ga::SILU_BLOCK * 4);
    if (g > (int64_t)cus * 8) g = (int64_t)cus * 8;
    return launched("ga_stream_xor_rows",
                    ga::launch_xor_rows(g, in, out, (int32_t)rows, (uint32_t)nvec, static_cast<hipStream_t>(stream)));
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
