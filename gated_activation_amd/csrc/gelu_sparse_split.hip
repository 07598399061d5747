// gelu_and_mul_sparse with each row split over several workgroups, for few
// rows (a row per workgroup would leave most of the 256 compute units idle).
//
// Same op as gelu_sparse.hip (vLLM PR 48498, "[Performance] Add Triton kernel
// for Gemma3n sparse GELU", section Purpose).  Workgroup (s, r) of the grid
// (splits, T) owns vectors [s*CHUNK, (s+1)*CHUNK) of row r:
//   1. load its gate chunk (and, early mode, its up chunk) into registers;
//   2. reduce the chunk's mean m_s and M2_s = sum (g - m_s)^2 (two passes over
//      the registers);
//   3. publish (m_s, M2_s) in the workspace and add this workgroup's share of
//      16 to the row's arrival counter;
//   4. poll the counter until this call's 16 have arrived, then combine the
//      partials of s = 0..splits-1 in that order with Chan's parallel-variance
//      formula, so every workgroup of the row derives the same mean, M2 and
//      cutoff;
//   5. apply to its chunk and store.
// The partials and the counter are only ever touched by device-scope atomic
// operations, which are coherent across the XCDs without cache maintenance;
// the partial's store is waited for (vmcnt) before the counter add that
// announces it.  Release/acquire fences would instead write back and
// invalidate the whole L2 of every participating workgroup, which measured
// several microseconds per call.
// The counter only ever grows by 16 per row per call, so a call finds it at
// a multiple of 16 and waits for the next one: the workspace is zero-filled
// once and then serves any sequence of calls and graph replays.  The poll is
// bounded (spin_limit polls); a workgroup that gives up computes the whole
// row's statistics from global memory itself, so the kernel always finishes
// and stays correct even if the row's workgroups are not co-resident.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

// Chan et al.: combine (n_a, mean_a, M2_a) with (n_b, mean_b, M2_b).
__device__ __forceinline__ void chan_combine(float &n_a, float &mean_a, float &m2_a, float n_b,
                                             float mean_b, float m2_b) {
    const float n = n_a + n_b;
    const float delta = mean_b - mean_a;
    const float w = n_b / n;
    mean_a = __builtin_fmaf(delta, w, mean_a);
    m2_a = m2_a + m2_b + delta * delta * n_a * w;
    n_a = n;
}

}  // namespace

template <int DT, int WAVES, int VPL, int UP, bool NONTEMP = true>
__global__ __launch_bounds__(WAVES * 64) void gelu_sparse_split_kernel(
    const uint4 *__restrict__ in, uint4 *__restrict__ out, int32_t T, int32_t d, int32_t nvec,
    float z, const int32_t *__restrict__ live, unsigned char *__restrict__ workspace,
    uint32_t spin_limit) {
    using E = Elem<DT>;
    constexpr int NT = WAVES * 64;
    constexpr int CHUNK = NT * VPL;
    constexpr int PER = E::PER16;
    __shared__ float red[4][WAVES];
    __shared__ int flag;

    const int32_t s = (int32_t)blockIdx.x;
    const int32_t splits = (int32_t)gridDim.x;
    const int32_t r = (int32_t)blockIdx.y;
    if (live != nullptr && r >= clamp_live(live, T)) return;  // the whole row exits

    const uint4 *grow = in + (size_t)r * 2 * (size_t)nvec;
    const uint4 *urow = grow + nvec;
    uint4 *orow = out + (size_t)r * (size_t)nvec;
    const int t = (int)threadIdx.x;
    const int v0 = s * CHUNK;
    const int nhere = nvec - v0 < CHUNK ? nvec - v0 : CHUNK;  // >= 1 (host guarantees)

    uint4 gv[VPL], uv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int i = k * NT + t;
        gv[k] = i < nhere ? ld16<NONTEMP>(grow + v0 + i) : uint4{0u, 0u, 0u, 0u};
    }
    if constexpr (UP == 0) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int i = k * NT + t;
            uv[k] = i < nhere ? ld16<NONTEMP>(urow + v0 + i) : uint4{0u, 0u, 0u, 0u};
        }
    }

    // Chunk statistics.
    const float n_here = (float)(nhere * PER);
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float f[PER];
        E::unpack(gv[k], f);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc += f[e];
    }
    const float m_here = block_sum<WAVES>(acc, red[0]) / n_here;
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        if (k * NT + t < nhere) {
            float f[PER];
            E::unpack(gv[k], f);
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float dv = f[e] - m_here;
                q = __builtin_fmaf(dv, dv, q);
            }
        }
    }
    const float m2_here = block_sum<WAVES>(q, red[1]);

    // Publish, then wait for the other workgroups of the row.  Row r's
    // record: a 16-byte header holding the counter, then SPLIT_MAX partials.
    uint32_t *counter = reinterpret_cast<uint32_t *>(workspace + (size_t)r * SPLIT_RECORD_BYTES);
    uint64_t *partials = reinterpret_cast<uint64_t *>(workspace + (size_t)r * SPLIT_RECORD_BYTES + 16);
    if (t == 0) {
        const uint64_t packed = (uint64_t)__builtin_bit_cast(uint32_t, m_here) |
                                ((uint64_t)__builtin_bit_cast(uint32_t, m2_here) << 32);
        __hip_atomic_store(partials + s, packed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partial has landed
        // The row's workgroups add exactly 16 in total (16 / splits each, one
        // more for the first 16 % splits of them), whatever the split count.
        const uint32_t inc = 16u / (uint32_t)splits + ((uint32_t)s < 16u % (uint32_t)splits ? 1u : 0u);
        const uint32_t old = __hip_atomic_fetch_add(counter, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t base = old - (old % 16u);
        uint32_t polls = 0;
        int ok = 0;
        while (true) {
            const uint32_t now = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (now - base >= 16u) {
                ok = 1;
                break;
            }
            if (++polls > spin_limit) break;
            __builtin_amdgcn_s_sleep(1);
        }
        flag = ok;
    }
    __syncthreads();
    const bool ok = flag != 0;

    float mean, m2;
    if (ok) {
        float n_acc = 0.0f;
        mean = 0.0f;
        m2 = 0.0f;
        for (int i = 0; i < splits; ++i) {
            const uint64_t raw = __hip_atomic_load(partials + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float pm = __builtin_bit_cast(float, (uint32_t)raw);
            const float pq = __builtin_bit_cast(float, (uint32_t)(raw >> 32));
            const int pv0 = i * CHUNK;
            const float pn = (float)((nvec - pv0 < CHUNK ? nvec - pv0 : CHUNK) * PER);
            if (i == 0) {
                n_acc = pn;
                mean = pm;
                m2 = pq;
            } else {
                chan_combine(n_acc, mean, m2, pn, pm, pq);
            }
        }
    } else {
        // Bounded wait expired: the whole row's statistics from global
        // memory, two passes, by this workgroup alone.
        float a = 0.0f;
        for (int j = t; j < nvec; j += NT) {
            float f[PER];
            E::unpack(ld16<false>(grow + j), f);
#pragma unroll
            for (int e = 0; e < PER; ++e) a += f[e];
        }
        mean = block_sum<WAVES>(a, red[2]) / (float)d;
        float b = 0.0f;
        for (int j = t; j < nvec; j += NT) {
            float f[PER];
            E::unpack(ld16<false>(grow + j), f);
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const float dv = f[e] - mean;
                b = __builtin_fmaf(dv, dv, b);
            }
        }
        m2 = block_sum<WAVES>(b, red[3]);
    }
    const float cut = __builtin_fmaf(z, __builtin_sqrtf(m2 / (float)d), mean);

    if constexpr (UP == 1) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int i = k * NT + t;
            uv[k] = i < nhere ? ld16<NONTEMP>(urow + v0 + i) : uint4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int i = k * NT + t;
        if (i < nhere) {
            float g[PER], u[PER], y[PER];
            E::unpack(gv[k], g);
            E::unpack(uv[k], u);
#pragma unroll
            for (int e = 0; e < PER; ++e) y[e] = gelu_tanh(__builtin_fmaxf(g[e] - cut, 0.0f)) * u[e];
            st16<NONTEMP>(orow + v0 + i, E::pack(y));
        }
    }
}

namespace {

using SplitFn = void (*)(const uint4 *, uint4 *, int32_t, int32_t, int32_t, float, const int32_t *,
                         unsigned char *, uint32_t);

// Index [dtype][log2 waves][log2 vectors per lane]; up loaded with the gate.
#define GA_SP(DT, W) \
    { &gelu_sparse_split_kernel<DT, W, 1, 0>, &gelu_sparse_split_kernel<DT, W, 2, 0>, \
      &gelu_sparse_split_kernel<DT, W, 4, 0> }
#define GA_SPD(DT) { GA_SP(DT, 1), GA_SP(DT, 2), GA_SP(DT, 4), GA_SP(DT, 8), GA_SP(DT, 16) }
const SplitFn kGeluSplit[3][5][3] = {GA_SPD(DT_F32), GA_SPD(DT_F16), GA_SPD(DT_BF16)};
#undef GA_SP
#undef GA_SPD

int ilog2(int v) {
    if (v <= 0 || v > 1024) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return (1 << l) == v ? l : -1;
}

}  // namespace

bool gelu_split_available(int dtype, int waves, int vec_per_lane, int splits) {
    const int wi = ilog2(waves), vi = ilog2(vec_per_lane);
    return dtype >= 0 && dtype <= 2 && wi >= 0 && wi <= 4 && vi >= 0 && vi <= 2 && splits >= 2 &&
           splits <= SPLIT_MAX;
}

hipError_t launch_gelu_split(int dtype, int waves, int vpl, int splits, const void *in, void *out, int32_t T,
                             int32_t d, int32_t nvec, float z, const int32_t *live, void *workspace,
                             uint32_t spin_limit, hipStream_t stream) {
    if (!gelu_split_available(dtype, waves, vpl, splits)) return hipErrorInvalidValue;
    const SplitFn fn = kGeluSplit[dtype][ilog2(waves)][ilog2(vpl)];
    const uint4 *a_in = static_cast<const uint4 *>(in);
    uint4 *a_out = static_cast<uint4 *>(out);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    void *args[] = {&a_in, &a_out, &T, &d, &nvec, &z, &live, &ws, &spin_limit};
    return hipLaunchKernel((const void *)fn, dim3((uint32_t)splits, (uint32_t)T), dim3(waves * 64), args, 0, stream);
}

}  // namespace ga
