// gelu_and_mul_sparse fused with the down projection, staged form: two to
// four tokens.
//   y[r, h] = sum_k a[r, k] * w[h, k],   a = gelu_and_mul_sparse(gu) as stored
// gu is [T, 2d] (gate | up), w is [H, d] with one row of weights per output
// feature, y is [T, H]; fp32 sums, rounded once.
//
// Two launches.  The first is the library's own activation kernel for the
// call's rows (the planner's row kernel, no workspace of its own) writing a
// into the caller's workspace: T * d elements, formed once.  The second,
// down_staged_kernel, streams the weights: a few tokens per weight is a
// matrix-vector product, bound by the H * d weight bytes.  Workgroup b owns
// output features [b*F, +F) over all of d (no two workgroups share an
// output; nothing is exchanged between them); lane i of its W wavefronts
// owns the 8-element vectors j = v * 64W + i (v < NV) of a's rows and of
// each of its F weight rows, so it loads only the activation it multiplies.
// Its activation loads go first (they come from the cache), then the
// weights of the first WA vectors; the weights of vector v + WA are issued
// once vector v's products are done, into the registers vector v held.
// fp32 FMA dot products, a DPP sum per wavefront and a fixed-order sum over
// the wavefronts.  Rows past the live count and vectors past d read zero
// through buffer descriptors without touching memory.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

// An offset at or past a buffer descriptor's range reads zero and touches no
// memory; kOob is past every range the kernel builds.
constexpr int kOob = (int)0x80000000;

}  // namespace

template <int DT, int TMAX, int F, int WAVES, int NV, int WA>
__global__ __launch_bounds__(WAVES * 64) void down_staged_kernel(const uint16_t *a, const uint16_t *w, uint16_t *y,
                                                                 int32_t T, int32_t d, int32_t H,
                                                                 const int32_t *live) {
    static_assert(1 <= WA && WA <= NV, "weight vectors in flight");
    using E = Elem<DT>;
    constexpr int NTH = WAVES * 64;
    __shared__ float part[TMAX * F][WAVES];

    const int tid = threadIdx.x, wv = tid >> 6;
    const int n_live = live ? clamp_live(live, T) : T;
    const int nrows = n_live < TMAX ? n_live : TMAX;
    if (nrows <= 0) return;
    const int nvec = d / 8;
    const int h_first = blockIdx.x * F;
    const int hrows = H - h_first < F ? H - h_first : F;
    const __amdgpu_buffer_rsrc_t asrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a), (short)0, nrows * d * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w + (int64_t)h_first * d), (short)0, hrows * d * 2, 0x00020000);

    uint4 av[TMAX][NV], wr[NV][F];
    auto issue_w = [&](int v) {
        const int j = v * NTH + tid;
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int off = j < nvec ? (f * d + j * 8) * 2 : kOob;
            wr[v][f] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, 0));
        }
    };
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int j = v * NTH + tid;
            const int off = j < nvec ? (t * d + j * 8) * 2 : kOob;
            av[t][v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(asrc, off, 0, 0));
        }
#pragma unroll
    for (int v = 0; v < WA; ++v) issue_w(v);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    float acc[TMAX][F];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int f = 0; f < F; ++f) acc[t][f] = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float a8[TMAX][8];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) E::unpack(av[t][v], a8[t]);
#pragma unroll
        for (int f = 0; f < F; ++f) {
            float w8[8];
            E::unpack(wr[v][f], w8);
#pragma unroll
            for (int t = 0; t < TMAX; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[t][f] = __builtin_fmaf(a8[t][e], w8[e], acc[t][f]);
        }
        if (v + WA < NV) {
            issue_w(v + WA);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Lanes, then wavefronts in order.
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const float s = wave_sum(acc[t][f]);
            if ((tid & 63) == 0) part[t * F + f][wv] = s;
        }
    __syncthreads();
    if (tid < TMAX * F) {
        const int t = tid / F, f = tid % F;
        if (t < nrows && f < hrows) {
            float s = part[tid][0];
#pragma unroll
            for (int i = 1; i < WAVES; ++i) s += part[tid][i];
            y[(int64_t)t * H + h_first + f] = E::from_f32(s);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

typedef void (*StagedKernel)(const uint16_t *, const uint16_t *, uint16_t *, int32_t, int32_t, int32_t,
                             const int32_t *);

struct StagedEntry {
    int tmax, f, waves, nv;
    StagedKernel bf16, f16;
};

#define GA_STAGED(TMAX, F, W, NV, WA) \
    {TMAX, F, W, NV, down_staged_kernel<DT_BF16, TMAX, F, W, NV, WA>, down_staged_kernel<DT_F16, TMAX, F, W, NV, WA>}

// (most tokens, features per workgroup, wavefronts, 16-byte vectors of a row
// per lane, weight vectors in flight); entries of one (tokens, features,
// wavefronts) by rising reach.  The fastest measured on MI355X at H = 2048,
// d = 8192 and 16384.
const StagedEntry kStaged[] = {
    GA_STAGED(2, 4, 16, 1, 1),
    GA_STAGED(2, 4, 16, 2, 1),
    GA_STAGED(4, 4, 16, 1, 1),
    GA_STAGED(4, 4, 16, 2, 1),
};

#undef GA_STAGED

const StagedEntry *find_staged(int tmax, int f, int waves, int64_t d) {
    for (const StagedEntry &e : kStaged)
        if (e.tmax == tmax && e.f == f && e.waves == waves && d <= (int64_t)8 * e.nv * waves * 64) return &e;
    return nullptr;
}

}  // namespace

bool gelu_down_staged_available(int dtype, int tmax, int f, int waves, int64_t d) {
    return (dtype == DT_BF16 || dtype == DT_F16) && find_staged(tmax, f, waves, d) != nullptr;
}

hipError_t launch_gelu_down_staged(int dtype, int tmax, int f, int waves, const void *a, const void *w, void *y,
                                   int32_t T, int32_t d, int32_t H, const int32_t *live, hipStream_t stream) {
    const StagedEntry *e = find_staged(tmax, f, waves, d);
    if (!e || (dtype != DT_BF16 && dtype != DT_F16) || T > tmax) return hipErrorInvalidValue;
    const uint16_t *a_a = static_cast<const uint16_t *>(a);
    const uint16_t *a_w = static_cast<const uint16_t *>(w);
    uint16_t *a_y = static_cast<uint16_t *>(y);
    void *args[] = {&a_a, &a_w, &a_y, &T, &d, &H, &live};
    return hipLaunchKernel(reinterpret_cast<const void *>(dtype == DT_BF16 ? e->bf16 : e->f16),
                           dim3((uint32_t)((H + f - 1) / f)), dim3(waves * 64), args, 0, stream);
}

}  // namespace ga
