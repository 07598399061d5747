// gelu_and_mul_sparse with each row split over several workgroups, for few
// rows (a row per workgroup would leave most of the 256 compute units idle).
//
// Same op as gelu_sparse.hip (vLLM PR 48498, "[Performance] Add Triton kernel
// for Gemma3n sparse GELU", section Purpose).  Workgroup (s, r) of the grid
// (splits, T) owns vectors [s*CHUNK, (s+1)*CHUNK) of row r:
//   1. read the tag in its own slot of the row's record (the previous call's)
//      while loading its gate chunk (and, early mode, its up chunk) into
//      registers; this call's tag is 16 more;
//   2. reduce the chunk's mean m_s and M2_s = sum (g - m_s)^2 (two passes over
//      the registers);
//   3. publish (m_s, M2_s) as two tagged 64-bit words, {tag, m_s} and
//      {tag, M2_s}, in its slot;
//   4. read the row's other slots, one lane per slot, all at once, until each
//      holds this call's tag, then combine the partials of s = 0..splits-1 in
//      that order with Chan's parallel-variance formula, so every workgroup
//      of the row derives the same mean, M2 and cutoff;
//   5. apply to its chunk and store.
// A tagged word carries its own proof of arrival, so a poll that succeeds
// has also read the data: once the row's workgroups have all published, the
// exchange costs one round of parallel loads, with no wait on a store, no
// read-modify-write and no second read.  The words are only ever touched by
// device-scope atomic loads and stores, which are coherent across the XCDs
// without cache maintenance (release/acquire fences would instead write back
// and invalidate the whole L2 of every participating workgroup, which
// measured several microseconds per call).
// Tags: a call writes its tag into all SPLIT_MAX slots of each row it
// processes (slots no workgroup owns at this split count get a zero
// payload), and within a call only workgroup s writes the slots
// l = s mod splits.  So when a call starts, every slot of the row holds the
// previous call's tag, each workgroup derives the same new tag from its own
// slot, and no slot holds the new tag before its owner writes it (tags step
// by 16 mod 2^32, so a slot never repeats the tag of the call before).  The
// workspace is zero-filled once and then serves any sequence of calls, split
// counts and graph replays.  The poll is bounded (spin_limit rounds); a
// workgroup that gives up computes the whole row's statistics from global
// memory itself, so the kernel always finishes and stays correct even if the
// row's workgroups are not co-resident.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

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
    __shared__ float row_stats[2];
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

    // Row r's record: SPLIT_MAX slots of two words, {tag, mean} and
    // {tag, M2}.  Every call writes all of them with one tag, so the tag in
    // this workgroup's own slot (which no other workgroup writes) is the
    // previous call's, and this call's is 16 more.  Lane 0 reads it, at an
    // address kept per lane by the empty asm so that it stays a vector load.
    uint64_t *slots = reinterpret_cast<uint64_t *>(workspace + (size_t)r * SPLIT_RECORD_BYTES);
    constexpr int SW = SPLIT_SLOT_BYTES / 8;  // 64-bit words from one slot to the next
    uint32_t prev = 0;
    if (t == 0) {
        int32_t lane_off = SW * s;
        asm volatile("" : "+v"(lane_off));
        prev = (uint32_t)__hip_atomic_load(slots + lane_off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

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
    const float m_here = row_mean<false>(block_sum<WAVES>(acc, red[0]), n_here);
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

    // Publish and gather, in the first wavefront: lane l < SPLIT_MAX writes
    // slot l when l % splits == s (its own partial at l == s, a zero payload
    // elsewhere), and lane l < splits gathers slot l.
    if (t < 64) {
        const uint32_t tag = (uint32_t)__builtin_amdgcn_readlane(prev, 0) + 16u;
        if (t < SPLIT_MAX && t % splits == s) {
            const bool own = t == s;
            const uint64_t w0 = (uint64_t)tag | ((uint64_t)__builtin_bit_cast(uint32_t, own ? m_here : 0.0f) << 32);
            const uint64_t w1 = (uint64_t)tag | ((uint64_t)__builtin_bit_cast(uint32_t, own ? m2_here : 0.0f) << 32);
            __hip_atomic_store(slots + SW * t, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(slots + SW * t + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // Lanes that gather nothing count as arrived; lane s has its own.
        bool have = t >= splits || t == s;
        float pm = t == s ? m_here : 0.0f, pq = t == s ? m2_here : 0.0f;
        uint32_t polls = 0;
        bool ok;
        while (true) {
            if (!have) {
                const uint64_t a = __hip_atomic_load(slots + SW * t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t b = __hip_atomic_load(slots + SW * t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((uint32_t)a == tag && (uint32_t)b == tag) {
                    have = true;
                    pm = __builtin_bit_cast(float, (uint32_t)(a >> 32));
                    pq = __builtin_bit_cast(float, (uint32_t)(b >> 32));
                }
            }
            if (__builtin_amdgcn_ballot_w64(!have) == 0) {
                ok = true;
                break;
            }
            if (++polls > spin_limit) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (ok) {
            // Every lane combines the same scalars in slot order.
            float n_acc = 0.0f, mean = 0.0f, m2 = 0.0f;
            for (int i = 0; i < splits; ++i) {
                const float im = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pm), i));
                const float iq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pq), i));
                const int pv0 = i * CHUNK;
                const float pn = (float)((nvec - pv0 < CHUNK ? nvec - pv0 : CHUNK) * PER);
                if (i == 0) {
                    n_acc = pn;
                    mean = im;
                    m2 = iq;
                } else {
                    chan_combine(n_acc, mean, m2, pn, im, iq);
                }
            }
            if (t == 0) {
                row_stats[0] = mean;
                row_stats[1] = m2;
            }
        }
        if (t == 0) flag = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = flag != 0;

    float mean, m2;
    if (ok) {
        mean = row_stats[0];
        m2 = row_stats[1];
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
        mean = row_mean<false>(block_sum<WAVES>(a, red[2]), (float)d);
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
    const float cut = sparse_cutoff<E, false>(mean, row_var<false>(m2, (float)d), z);

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
