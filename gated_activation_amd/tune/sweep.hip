// Geometry sweep for the gelu_and_mul_sparse planner (a tuning tool, not part
// of the library).  For each (rows T, 16-byte vectors per row nvec) of a grid,
// every compiled one-row-per-workgroup geometry of the vector kernel (waves
// 1..16, vectors per lane 1, 2, 4, 8, the up row loaded with the gate or after
// the statistics) is launched through the public entry point
// ga_gelu_and_mul_sparse_with_plan on bf16 rows (d = 8 nvec), back to back on
// the null stream over buffer sets rotated past the 256 MB Infinity Cache, and
// timed with HIP events; each geometry's time is the best of 3 interleaved
// passes.  Output, one CSV line per geometry: T,d,nvec,waves,per_lane,up_late,us
//
//   sweep <T values> -- <nvec values>      (pool size from GA_SWEEP_POOL_GB, default 16)
//
// GA_SWEEP_PATH=2 sweeps the unaligned path instead (vectors per lane 1..8):
// the input view starts one element past a 16-byte boundary.
// GA_SWEEP_PATH=split sweeps few-row shapes for the split path: every row
// geometry as above (splits = 1) and every split plan (chunks of waves 1..16
// times vectors per lane 1, 2, 4; splits = the chunks a row needs, 2..16),
// with a zero-filled workspace, each timed by replaying a graph of 64 launches
// (the calls are a few microseconds); an eighth column holds the splits.
// GA_SWEEP_PATH=packed sweeps short rows (nvec <= 32): every packed-rows
// geometry (lanes per row 4..32 times vectors per lane 1, 2, 4, covering the
// row without a spare half) and the one-wave row geometry, timed by graph
// replay; an eighth column holds the lanes per row (0 for the row geometry).
//
// gated_activation_amd/tune/make_table.py turns one or more such files into
// the planner's table (csrc/planner_table.inc).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <vector>

#include "ga.h"

#define CK(x)                                                                              \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);    \
            std::exit(1);                                                                  \
        }                                                                                  \
    } while (0)

// Finite bf16 values in [-2, 2) from a hash of the index (the kernels' speed
// does not depend on the values).
__global__ void fill_bf16(uint16_t *p, size_t n, uint32_t seed) {
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) {
        uint32_t h = (uint32_t)i * 2654435761u ^ seed;
        h ^= h >> 13;
        h *= 0x5bd1e995u;
        h ^= h >> 15;
        const float f = ((h & 0xFFFFu) / 65536.0f - 0.5f) * 4.0f;
        p[i] = (uint16_t)(__builtin_bit_cast(uint32_t, f) >> 16);
    }
}

// Per-call time from a graph of 64 launches replayed 8 times.
static float time_graph(hipGraphExec_t exec) {
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    CK(hipGraphLaunch(exec, nullptr));
    CK(hipEventRecord(a, nullptr));
    for (int i = 0; i < 8; ++i) CK(hipGraphLaunch(exec, nullptr));
    CK(hipEventRecord(b, nullptr));
    CK(hipEventSynchronize(b));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, a, b));
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return ms * 1000.0f / (8.0f * 64.0f);
}

static float time_pass(int sets, int iters, const std::function<void(int)> &launch) {
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    CK(hipEventRecord(a, nullptr));
    for (int i = 0; i < iters; ++i) launch(i % sets);
    CK(hipEventRecord(b, nullptr));
    CK(hipEventSynchronize(b));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, a, b));
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return ms * 1000.0f / (float)iters;
}

int main(int argc, char **argv) {
    std::vector<int> Ts, NVs;
    int a = 1;
    for (; a < argc && std::strcmp(argv[a], "--") != 0; ++a) Ts.push_back(std::atoi(argv[a]));
    for (++a; a < argc; ++a) NVs.push_back(std::atoi(argv[a]));
    if (Ts.empty() || NVs.empty()) {
        std::fprintf(stderr, "usage: sweep <T values> -- <nvec values>\n");
        return 2;
    }
    const char *path_env = std::getenv("GA_SWEEP_PATH");
    const bool split_mode = path_env && std::strcmp(path_env, "split") == 0;
    const bool packed_mode = path_env && std::strcmp(path_env, "packed") == 0;
    const int path = path_env && std::strcmp(path_env, "2") == 0 ? 2 : 0;
    const size_t shift = path == 2 ? 2 : 0;  // bytes: one bf16 element
    const char *gb = std::getenv("GA_SWEEP_POOL_GB");
    const size_t pool_bytes = (size_t)(gb ? std::atof(gb) : 16.0) * ((size_t)1 << 30);
    uint16_t *pool = nullptr;
    CK(hipMalloc(&pool, pool_bytes));
    // Split plans: one zero-filled workspace for the largest T (the kernels
    // keep it consistent across calls).
    int tmax = 1;
    for (int T : Ts) tmax = std::max(tmax, T);
    const size_t ws_bytes = split_mode ? ga_gelu_and_mul_sparse_workspace_bytes(tmax) : 0;
    void *ws = nullptr;
    if (split_mode) {
        CK(hipMalloc(&ws, ws_bytes));
        CK(hipMemset(ws, 0, ws_bytes));
    }
    fill_bf16<<<8192, 256>>>(pool, pool_bytes / 2, 99u);
    CK(hipDeviceSynchronize());
    // Clocks up before the first measurement.
    for (int i = 0; i < 6000; ++i)
        ga_stream_xor_rows(pool, (char *)pool + ((size_t)512 << 20), 2048, 32768, nullptr);
    CK(hipDeviceSynchronize());

    for (int T : Ts) {
        for (int nvec : NVs) {
            const int d = nvec * 8;
            const size_t in_b = (size_t)T * 2 * d * 2, out_b = (size_t)T * d * 2;
            // the output starts 256 bytes past the input's end (room for the shift)
            const size_t per = (in_b + 256 + out_b + 4095) / 4096 * 4096;
            // At least two sets, and sets enough to span 1 GiB.
            if (2 * per > pool_bytes) continue;
            int sets = (int)std::min<size_t>(64, std::max<size_t>(2, ((size_t)1 << 30) / per + 1));
            if ((size_t)sets * per > pool_bytes) sets = (int)(pool_bytes / per);
            std::vector<void *> vin(sets), vout(sets);
            for (int s = 0; s < sets; ++s) {
                vin[s] = (char *)pool + (size_t)s * per + shift;
                vout[s] = (char *)pool + (size_t)s * per + in_b + 256;
            }
            const double bytes = (double)(in_b + out_b);
            const int iters = std::max(30, std::min(800, (int)(1.5e5 / (bytes / 5e3 + 3.0))));
            std::vector<ga_plan> plans;
            if (packed_mode) {
                for (int g : {4, 8, 16, 32})
                    for (int v : {1, 2, 4}) {
                        if (g * v < nvec || (v > 1 && g * (v / 2) >= nvec)) continue;
                        ga_plan p;
                        std::memset(&p, 0, sizeof p);
                        p.path = 3;
                        p.lanes_per_row = g;
                        p.per_lane = v;
                        p.splits = 1;
                        if (ga_gelu_and_mul_sparse_with_plan(vin[0], vout[0], 0, d, GA_BF16, 1.6448536f, nullptr, &p,
                                                             nullptr, 0, nullptr) == GA_OK)
                            plans.push_back(p);
                    }
            }
            for (int w : {1, 2, 4, 8, 16})
                for (int v = 1; v <= 8; ++v) {
                    if (path == 0 && (v & (v - 1)) != 0) continue;
                    const long slots = (long)w * 64 * v;
                    // Packed mode: the one-wave geometry only (the library rejects it
                    // if it does not cover the row).
                    if (packed_mode ? (w != 1 || v != 1) : (slots < nvec || slots >= 8L * nvec)) continue;
                    for (int late : {0, 1}) {
                        ga_plan p;
                        std::memset(&p, 0, sizeof p);
                        p.path = path;
                        p.waves_per_row = w;
                        p.per_lane = v;
                        p.up_late = late;
                        p.splits = 1;
                        p.block = w * 64;
                        p.grid = T;
                        // Zero rows: the library validates the plan and launches nothing.
                        if (ga_gelu_and_mul_sparse_with_plan(vin[0], vout[0], 0, d, GA_BF16, 1.6448536f, nullptr, &p,
                                                             nullptr, 0, nullptr) == GA_OK)
                            plans.push_back(p);
                    }
                }
            if (split_mode) {
                for (int w : {1, 2, 4, 8, 16})
                    for (int v : {1, 2, 4}) {
                        const int chunk = w * 64 * v;
                        const int splits = (nvec + chunk - 1) / chunk;
                        if (splits < 2 || splits > 16) continue;
                        ga_plan p;
                        std::memset(&p, 0, sizeof p);
                        p.path = 0;
                        p.waves_per_row = w;
                        p.per_lane = v;
                        p.splits = splits;
                        p.spin_limit = 1u << 16;
                        p.block = w * 64;
                        p.grid = (int64_t)T * splits;
                        if (ga_gelu_and_mul_sparse_with_plan(vin[0], vout[0], 0, d, GA_BF16, 1.6448536f, nullptr, &p,
                                                             ws, ws_bytes, nullptr) == GA_OK)
                            plans.push_back(p);
                    }
            }
            auto call = [&](const ga_plan &p, int s, hipStream_t st) {
                ga_gelu_and_mul_sparse_with_plan(vin[s], vout[s], T, d, GA_BF16, 1.6448536f, nullptr, &p, ws,
                                                 ws_bytes, st);
            };
            std::vector<float> best(plans.size(), 1e30f);
            for (size_t i = 0; i < plans.size(); ++i)
                for (int k = 0; k < 3; ++k) call(plans[i], k % sets, nullptr);
            CK(hipDeviceSynchronize());
            if (split_mode || packed_mode) {
                // one graph of 64 launches per plan, replayed in 3 interleaved passes
                std::vector<hipGraphExec_t> execs(plans.size());
                hipStream_t st;
                CK(hipStreamCreate(&st));
                for (size_t i = 0; i < plans.size(); ++i) {
                    hipGraph_t g;
                    CK(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
                    for (int k = 0; k < 64; ++k) call(plans[i], k % sets, st);
                    CK(hipStreamEndCapture(st, &g));
                    CK(hipGraphInstantiate(&execs[i], g, nullptr, nullptr, 0));
                    CK(hipGraphDestroy(g));
                }
                CK(hipStreamDestroy(st));
                for (int pass = 0; pass < 3; ++pass)
                    for (size_t i = 0; i < plans.size(); ++i) best[i] = std::min(best[i], time_graph(execs[i]));
                for (hipGraphExec_t e : execs) CK(hipGraphExecDestroy(e));
            } else {
                for (int pass = 0; pass < 3; ++pass)
                    for (size_t i = 0; i < plans.size(); ++i)
                        best[i] = std::min(best[i], time_pass(sets, iters, [&](int s) { call(plans[i], s, nullptr); }));
            }
            CK(hipGetLastError());
            for (size_t i = 0; i < plans.size(); ++i) {
                std::printf("%d,%d,%d,%d,%d,%d,%.3f", T, d, nvec, plans[i].waves_per_row, plans[i].per_lane,
                            plans[i].up_late, best[i]);
                if (split_mode) std::printf(",%d", plans[i].splits);
                if (packed_mode) std::printf(",%d", plans[i].lanes_per_row);
                std::printf("\n");
            }
            std::fflush(stdout);
        }
    }
    if (ws) CK(hipFree(ws));
    CK(hipFree(pool));
    std::printf("done\n");
    return 0;
}
