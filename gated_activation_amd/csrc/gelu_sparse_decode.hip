// gelu_and_mul_sparse fused with the down projection, decode form: one or
// two tokens.
//   y[r, h] = sum_k a[r, k] * w[h, k],   a = gelu_and_mul_sparse(gu) as stored
// (the activation rounded once to the element type), summed in fp32,
// rounded once.  gu is [T, 2d] (gate | up), w is [H, d] with one row of
// weights per output feature, y is [T, H].  The vLLM page (PR 48498, Test
// Result, Correctness) has the activation's write feed the layer's
// downstream projection; here the activation never leaves registers.
//
// At one or two tokens the product is a matrix-vector product: every weight
// is used once or twice, so the call is bound by the weight stream (H * d *
// 2 bytes) and nothing about it is a tile for the matrix cores.  One launch
// does everything: no workspace, no second launch, no exchange between
// workgroups.  Each workgroup owns a few output features over all of d and
// recomputes the tokens' statistics and activation itself (the gate and up
// rows are read from L2 by every workgroup; the weights from HBM once).
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

// An offset at or past a buffer descriptor's range reads zero and touches no
// memory; kOob is past every range the kernels build.
constexpr int kOob = (int)0x80000000;

}  // namespace

// Decode form, for T <= TMAX tokens and d <= 8 * NV * (WAVES * 64): one
// launch, no workspace, no matrix cores (a token or two per weight is a dot
// product, not a tile).  Workgroup hb owns output features [hb*F, +F) over
// all of d, so no other workgroup shares its output.  Lane i of the workgroup
// owns the 8-element vectors j = v * NTH + i (v < NV) of every row, the same
// k positions in gate, up and each of its F weight rows, so the activation
// never leaves the registers of the lane that multiplies it:
//   a. the loads, all issued before any result is used: the weights of
//      vectors v < WPRE, the tokens' gate rows, their up rows, the weights of
//      vectors WPRE <= v < WA.  Loads complete in issue order, so the
//      statistics wait for the gate (and the first WPRE weight vectors) only,
//      while the rest of the weights stream;
//   b. each row's mean and M2 (fixed-order workgroup sums, the same value on
//      every thread), the cutoff, and the activation in fp32 rounded to the
//      element type; vectors past d and tokens past the live count are zero.
//      The weights of vectors v >= WA are issued only now, into the
//      registers the gate and up rows held;
//   c. fp32 dot products a . w as the weights arrive;
//   d. each (token, feature) sum over the wavefront's lanes, then over the
//      wavefronts in order, and the store.
template <int DT, int TMAX, int F, int WAVES, int NV, int WPRE, int WA, int MINW = 1>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(MINW))) void down_decode_kernel(const uint16_t *gu, const uint16_t *w, uint16_t *y,
                                                                 int32_t T, int32_t d, int32_t H, float z,
                                                                 const int32_t *live) {
    static_assert(0 <= WPRE && WPRE <= WA && WA <= NV, "weight issue points out of order");
    using E = Elem<DT>;
    constexpr int NTH = WAVES * 64;
    __shared__ float red[2 * TMAX][WAVES];
    __shared__ float part[TMAX * F][WAVES];

    const int tid = threadIdx.x, wv = tid >> 6;
    const int n_live = live ? clamp_live(live, T) : T;
    const int nrows = n_live < TMAX ? n_live : TMAX;
    if (nrows <= 0) return;
    const int nvec = d / 8;
    const int h_first = blockIdx.x * F;
    const int hrows = H - h_first < F ? H - h_first : F;
    // Offsets at or past a descriptor's range read zero without touching
    // memory: tokens past the live count, weight rows past H, vectors past d
    // (given kOob).
    const __amdgpu_buffer_rsrc_t gsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(gu), (short)0, nrows * 4 * d, 0x00020000);
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w + (int64_t)h_first * d), (short)0, hrows * 2 * d, 0x00020000);

    // a. the loads.
    uint4 gv[TMAX][NV], uv[TMAX][NV], wr[NV][F];
    auto issue_w = [&](int v) {
        const int j = v * NTH + tid;
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int off = j < nvec ? (f * d + j * 8) * 2 : kOob;
            wr[v][f] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, 0));
        }
    };
#pragma unroll
    for (int v = 0; v < WPRE; ++v) issue_w(v);
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int j = v * NTH + tid;
            const int off = j < nvec ? (t * 2 * d + j * 8) * 2 : kOob;
            gv[t][v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(gsrc, off, 0, 0));
        }
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int j = v * NTH + tid;
            const int off = j < nvec ? (t * 2 * d + d + j * 8) * 2 : kOob;
            uv[t][v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(gsrc, off, 0, 0));
        }
#pragma unroll
    for (int v = WPRE; v < WA; ++v) issue_w(v);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // b. statistics and the activation.  Vectors past d read zero, so they
    // drop out of the sum; the squared deviations skip them.
    float cut[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float f8[8];
            E::unpack(gv[t][v], f8);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += f8[e];
        }
        const float mean = row_mean<false>(block_sum<WAVES>(s, red[2 * t]), (float)d);
        float q = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float f8[8];
            E::unpack(gv[t][v], f8);
            const bool in = v * NTH + tid < nvec;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dv = in ? f8[e] - mean : 0.0f;
                q = __builtin_fmaf(dv, dv, q);
            }
        }
        cut[t] = sparse_cutoff<E, false>(mean, row_var<false>(block_sum<WAVES>(q, red[2 * t + 1]), (float)d), z);
    }
    uint4 act[TMAX][NV];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float g8[8], u8[8];
            E::unpack(gv[t][v], g8);
            E::unpack(uv[t][v], u8);
#pragma unroll
            for (int e = 0; e < 8; ++e) g8[e] = sparse_apply<E, false>(g8[e], cut[t], u8[e]);
            act[t][v] = t < nrows && v * NTH + tid < nvec ? E::pack(g8) : uint4{0, 0, 0, 0};
        }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = WA; v < NV; ++v) issue_w(v);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // c. the dot products, vector by vector as the weights arrive.
    float acc[TMAX][F];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int f = 0; f < F; ++f) acc[t][f] = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float a8[TMAX][8];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) E::unpack(act[t][v], a8[t]);
#pragma unroll
        for (int f = 0; f < F; ++f) {
            float w8[8];
            E::unpack(wr[v][f], w8);
#pragma unroll
            for (int t = 0; t < TMAX; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[t][f] = __builtin_fmaf(a8[t][e], w8[e], acc[t][f]);
        }
    }

    // d. lanes, then wavefronts in order.
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

typedef void (*DecodeKernel)(const uint16_t *, const uint16_t *, uint16_t *, int32_t, int32_t, int32_t, float,
                             const int32_t *);

struct DecodeEntry {
    int tmax, f, waves, nv;
    DecodeKernel bf16, f16;
};

#define GA_DECODE(TMAX, F, W, NV, WPRE, WA)                                            \
    {TMAX, F, W, NV, down_decode_kernel<DT_BF16, TMAX, F, W, NV, WPRE, WA>, \
     down_decode_kernel<DT_F16, TMAX, F, W, NV, WPRE, WA>}

// (most tokens, features per workgroup, wavefronts, 16-byte vectors of a row
// per lane, weight vectors issued before the gate, before the activation);
// entries of one (tokens, features, wavefronts) by rising reach.  The issue
// points are the fastest measured on MI355X at H = 2048 and d = 8192..32768.
const DecodeEntry kDecode[] = {
    GA_DECODE(1, 4, 8, 4, 0, 1),  GA_DECODE(1, 4, 16, 2, 0, 0), GA_DECODE(1, 4, 16, 4, 0, 1),
    GA_DECODE(1, 4, 4, 8, 0, 2),  GA_DECODE(1, 2, 8, 4, 0, 2),  GA_DECODE(1, 2, 16, 4, 0, 1),
    GA_DECODE(1, 8, 16, 2, 0, 1), GA_DECODE(2, 4, 16, 2, 0, 0), GA_DECODE(2, 4, 8, 4, 0, 1),
    GA_DECODE(2, 2, 16, 2, 0, 0),
};

#undef GA_DECODE

// The entry of this geometry with the fewest vectors per lane that still
// reach d.
const DecodeEntry *find_decode(int tmax, int f, int waves, int64_t d) {
    for (const DecodeEntry &e : kDecode)
        if (e.tmax == tmax && e.f == f && e.waves == waves && d <= (int64_t)8 * e.nv * waves * 64) return &e;
    return nullptr;
}

}  // namespace


bool gelu_down_decode_available(int dtype, int tmax, int f, int waves, int64_t d) {
    return (dtype == DT_BF16 || dtype == DT_F16) && find_decode(tmax, f, waves, d) != nullptr;
}

hipError_t launch_gelu_down_decode(int dtype, int tmax, int f, int waves, const void *gu, const void *w, void *y,
                                   int32_t T, int32_t d, int32_t H, float z, const int32_t *live,
                                   hipStream_t stream) {
    const DecodeEntry *e = find_decode(tmax, f, waves, d);
    if (!e || (dtype != DT_BF16 && dtype != DT_F16) || T > tmax) return hipErrorInvalidValue;
    const uint16_t *a_gu = static_cast<const uint16_t *>(gu);
    const uint16_t *a_w = static_cast<const uint16_t *>(w);
    uint16_t *a_y = static_cast<uint16_t *>(y);
    void *args[] = {&a_gu, &a_w, &a_y, &T, &d, &H, &z, &live};
    return hipLaunchKernel(reinterpret_cast<const void *>(dtype == DT_BF16 ? e->bf16 : e->f16),
                           dim3((uint32_t)((H + f - 1) / f)), dim3(waves * 64), args, 0, stream);
}

}  // namespace ga
