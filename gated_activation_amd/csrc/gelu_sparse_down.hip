// gelu_and_mul_sparse fused with the down projection that consumes it:
//   y[r, h] = sum_k a[r, k] * w[h, k],   a = gelu_and_mul_sparse(gu) as stored
// (the activation rounded once to the element type), summed in fp32 on the
// matrix cores, rounded once.  gu is [T, 2d] (gate | up), w is [H, d] with one
// row of weights per output feature (a linear layer's layout), y is [T, H].
// The vLLM page (PR 48498, Test Result, Correctness) has the activation's
// write feed the layer's downstream projection; here the activation never
// reaches memory: it is formed while the product's operand is staged.
//
// This file holds the k-loop form, for five or more tokens (one token: the
// one-launch decode form, gelu_sparse_decode.hip; two to four: the staged
// form, gelu_sparse_staged.hip).  Two launches on the caller's stream.
//
// 1. down_cutoff_kernel, one workgroup per row: the row's mean and
//    population variance (two passes over the gate, fp32) and the cutoff
//    mean + z * std into the workspace (live rows only).  It also zeroes the
//    call's output-tile counters and advances the workspace's call counter
//    (the tag of the partial tiles below).
//
// 2. down_product_kernel.  Workgroup (rb, hb, ks) owns tokens [rb*TM, +TM),
//    output features [hb*BH, +BH) and the slice [ks*BK, +BK) of d.  Its
//    wavefronts form WH feature groups of 16 x WK slice parts of BK / WK.
//    Each workgroup
//      a. loads its tokens' cutoffs and the gate and up slices of its first
//         two steps of k, then (after a barrier, so every one of those loads
//         is queued first) those steps' w blocks straight into registers:
//         the bulk of the bytes;
//      b. applies relu, tanh-GELU and the product with up in fp32, rounds to
//         the element type and writes the result to LDS in the matrix
//         cores' operand order (while w is still arriving);
//      c. runs the 16x16x32 MFMAs as w arrives: w as the A operand (16
//         features x 32 k per instruction, from registers), the activation
//         as B (32 k x 16 tokens, from LDS), fp32 accumulators;
//      d. adds the WK slice parts' accumulators through LDS in part order;
//      e. with one slice (nK == 1) stores y; otherwise publishes its fp32
//         partial tile as tagged words and bumps the output tile's counter.
//         The last of the tile's nK workgroups to arrive sums the nK
//         partials in slice order (a deterministic split-k reduction) and
//         stores y.
//    Nothing waits on another workgroup until every MFMA is done: the
//    statistics dependency is met by the first launch, so the weight stream
//    (which fills each compute unit's memory queue) never delays it.
//
// Operand order.  The MFMA pairs lane l's eight A elements with its eight B
// elements at the same k positions.  In k block kb (128 elements),
// instruction jj covers elements [kb*128 + jj*32, +32); lane l (g = l / 16)
// supplies [kb*128 + jj*32 + g*8, +8) of feature row l % 16 (A) and of token
// l % 16 (B): each load instruction reads 64 contiguous bytes of each of 16
// rows, and the B fragments are written to and read from LDS as 1 KB runs.
//
// Tags.  The partial words of a call carry 2 * counter + 1, the call counter
// as advanced by the first launch; a word from an earlier call, of any shape,
// carries an older tag (a reuse needs 2^31 calls with the workspace), and the
// tile counters are zeroed by each call's first launch, so the zero-filled
// workspace serves any later sequence of calls and shapes, and graph
// replays.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4 &a, const uint4 &b, f32x4_t c) {
    if constexpr (DT == DT_BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                       __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

__device__ __forceinline__ uint64_t tagged(uint32_t tag, float v) {
    return (uint64_t)tag | ((uint64_t)__builtin_bit_cast(uint32_t, v) << 32);
}

__device__ __forceinline__ float tag_value(uint64_t w) { return __builtin_bit_cast(float, (uint32_t)(w >> 32)); }

__device__ __forceinline__ uint64_t load_word(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_word(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int CUT_WAVES = 16;
// 16-byte vectors per lane for the longest row the library takes (65536
// elements: 8192 vectors over 1024 lanes).
constexpr int CUT_MAXV = 8;

}  // namespace

template <int DT>
__global__ __launch_bounds__(CUT_WAVES * 64) void down_cutoff_kernel(const uint16_t *gu, int32_t T, int32_t d,
                                                                     float z, const int32_t *live,
                                                                     unsigned char *ws, int32_t ngroups) {
    using E = Elem<DT>;
    constexpr int NTH = CUT_WAVES * 64;
    __shared__ float red[2][CUT_WAVES];
    // This call's output-tile counters start at zero whatever an earlier
    // call of another shape left in these bytes; the call counter advances.
    uint32_t *cnt = reinterpret_cast<uint32_t *>(ws + down_cnt_offset(T));
    for (int i = blockIdx.x * NTH + threadIdx.x; i < ngroups; i += T * NTH)
        __hip_atomic_store(cnt + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        uint32_t *epoch = reinterpret_cast<uint32_t *>(ws);
        const uint32_t e = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(epoch, e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int n_live = live ? clamp_live(live, T) : T;
    const int r = blockIdx.x;
    if (r >= n_live) return;
    // The whole gate row in registers (at most CUT_MAXV vectors per lane),
    // all loads issued at once; then two passes over the registers.
    const uint4 *row = reinterpret_cast<const uint4 *>(gu + (int64_t)r * 2 * d);
    const int nvec = d / 8;
    uint4 v[CUT_MAXV];
#pragma unroll
    for (int k = 0; k < CUT_MAXV; ++k) {
        const int j = threadIdx.x + k * NTH;
        v[k] = row[j < nvec ? j : 0];
    }
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < CUT_MAXV; ++k) {
        if (threadIdx.x + k * NTH < nvec) {
            float f[8];
            E::unpack(v[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) a += f[e];
        }
    }
    const float mean = row_mean<false>(block_sum<CUT_WAVES>(a, red[0]), (float)d);
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < CUT_MAXV; ++k) {
        if (threadIdx.x + k * NTH < nvec) {
            float f[8];
            E::unpack(v[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dv = f[e] - mean;
                q = __builtin_fmaf(dv, dv, q);
            }
        }
    }
    const float m2 = block_sum<CUT_WAVES>(q, red[1]);
    if (threadIdx.x == 0)
        reinterpret_cast<float *>(ws + down_cut_offset())[r] =
            sparse_cutoff<E, false>(mean, row_var<false>(m2, (float)d), z);
}

// The product kernel walks its k range in steps of STEP elements.  Step s
// + 1's gate, up and weight loads are issued before step s's activation and
// MFMAs, so one step of loads is always in flight behind the arithmetic.
// All global reads are raw buffer loads: an offset past the descriptor's
// range (rows past the live count, features past H) or set to kOob (elements
// past d, steps past the range) returns zero and touches no memory, so every
// load is issued unconditionally (a load under a branch would make the
// compiler wait for all earlier loads at the join).
constexpr int kOob = (int)0x80000000;

template <int DT, int TM, int WH, int WK, int NKBW>
__global__ __launch_bounds__(WH * WK * 64) void down_product_kernel(const uint16_t *gu, const uint16_t *w,
                                                                    uint16_t *y, int32_t T, int32_t d, int32_t H,
                                                                    int32_t nK, int32_t nH, int32_t KS,
                                                                    const int32_t *live, unsigned char *ws) {
    using E = Elem<DT>;
    constexpr int WAVES = WH * WK;
    constexpr int NTH = WAVES * 64;
    constexpr int NT = TM / 16;                    // 16-token tiles
    constexpr int NKB = WK * NKBW;                 // 128-element k blocks per step
    constexpr int STEP = NKB * 128;
    constexpr int BH = WH * 16;
    constexpr int NUNITS = NT * NKB;               // (token tile, k block) units of the activation
    constexpr int UPW = (NUNITS + WAVES - 1) / WAVES;

    __shared__ uint4 act[2][NUNITS * 4 * 64];      // B operands: [step parity][tile][k block][instr][lane]
    __shared__ f32x4_t part_acc[WK > 1 ? (WK - 1) * WH * NT * 64 : 1];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int hg = wv % WH, kg = wv / WH;          // feature group, part of each step
    const int64_t b = blockIdx.x;
    const int ks = (int)(b % nK);
    const int64_t grp = b / nK;
    const int hb = (int)(grp % nH);
    const int rb = (int)(grp / nH);
    const int n_live = live ? clamp_live(live, T) : T;
    const int r0 = rb * TM;
    if (r0 >= n_live) return;  // no live token in this block (uniform)
    const int nrows = n_live - r0 < TM ? n_live - r0 : TM;
    const int k0 = ks * KS;
    const int k_end = d - k0 < KS ? d : k0 + KS;   // this workgroup's range [k0, k_end)
    const int nsteps = (k_end - k0 + STEP - 1) / STEP;
    const int h_first = hb * BH;
    const int h0 = h_first + hg * 16;              // this wavefront's 16 features
    const bool h_ok = h0 < H;                      // H is a multiple of 16: whole wavefronts in or out

    // Descriptors: the block's live token rows of gu, the block's feature rows of w.
    const __amdgpu_buffer_rsrc_t gsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(gu + (int64_t)r0 * 2 * d), (short)0, nrows * 4 * d, 0x00020000);
    const int hrows = H - h_first < BH ? H - h_first : BH;
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w + (int64_t)h_first * d), (short)0, hrows * 2 * d, 0x00020000);
    const float *cuts = reinterpret_cast<const float *>(ws + down_cut_offset());

    float cut[UPW];
#pragma unroll
    for (int q = 0; q < UPW; ++q) {
        const int u = wv + WAVES * q < NUNITS ? wv + WAVES * q : NUNITS - 1;
        const int i = (u / NKB) * 16 + l16;
        cut[q] = cuts[r0 + (i < nrows ? i : 0)];
    }
    uint32_t epoch = 0;
    if (nK > 1 && tid == 0) epoch = __hip_atomic_load(reinterpret_cast<const uint32_t *>(ws), __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);

    // Loads of step s: gate and up of this wavefront's activation units ...
    auto issue_small = [&](int s, uint4 (&G)[UPW][4], uint4 (&U)[UPW][4]) {
#pragma unroll
        for (int q = 0; q < UPW; ++q) {
            const int u = wv + WAVES * q < NUNITS ? wv + WAVES * q : NUNITS - 1;
            const int i = (u / NKB) * 16 + l16;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int k = k0 + s * STEP + (u % NKB) * 128 + jj * 32 + g * 8;
                const int off = s < nsteps && k < k_end ? (i * 2 * d + k) * 2 : kOob;
                G[q][jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(gsrc, off, 0, 0));
                U[q][jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(gsrc, off + 2 * d, 0, 0));
            }
        }
    };
    // ... and this wavefront's 16 weight rows over its part of the step.
    auto issue_w = [&](int s, uint4 (&Wr)[NKBW][4]) {
#pragma unroll
        for (int kb = 0; kb < NKBW; ++kb) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int k = k0 + s * STEP + (kg * NKBW + kb) * 128 + jj * 32 + g * 8;
                const int off = s < nsteps && k < k_end ? ((hg * 16 + l16) * d + k) * 2 : kOob;
                Wr[kb][jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, 0));
            }
        }
    };
    // The activation of step s, rounded to the element type, into the
    // operand layout of LDS buffer P.  Computed for every lane (zeroed loads
    // give zero) and masked for tokens past the live count.
    auto activate = [&](uint4 (&G)[UPW][4], uint4 (&U)[UPW][4], uint4 *buf) {
#pragma unroll
        for (int q = 0; q < UPW; ++q) {
            const int u = wv + WAVES * q;
            if (u < NUNITS) {
                const int i = (u / NKB) * 16 + l16;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float f[8], v[8];
                    E::unpack(G[q][jj], f);
                    E::unpack(U[q][jj], v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = sparse_apply<E, false>(f[e], cut[q], v[e]);
                    const uint4 o = E::pack(f);
                    buf[(u * 4 + jj) * 64 + lane] = i < nrows ? o : uint4{0, 0, 0, 0};
                }
            }
        }
    };
    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto product = [&](uint4 (&Wr)[NKBW][4], const uint4 *buf) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt * 16 < nrows && h_ok) {
#pragma unroll
                for (int kb = 0; kb < NKBW; ++kb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        acc[nt] = mfma_16x16x32<DT>(Wr[kb][jj], buf[((nt * NKB + kg * NKBW + kb) * 4 + jj) * 64 + lane],
                                                    acc[nt]);
            }
        }
    };

    uint4 ga[UPW][4], ua[UPW][4], wa[NKBW][4];
    uint4 gb[UPW][4], ub[UPW][4], wb[NKBW][4];
    // Steps 0 and 1: every wavefront's gate and up loads of both enter the
    // compute unit's memory queue before any weight load (loads complete in
    // issue order, so the activations of both steps then wait for no weight
    // data; the barrier waits for no load).
    issue_small(0, ga, ua);
    issue_small(1, gb, ub);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_w(0, wa);
    issue_w(1, wb);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    activate(ga, ua, act[0]);
    activate(gb, ub, act[1]);
    __syncthreads();
    // Later pairs of steps (rows of many tokens; decode-sized calls have one
    // or two steps): the next pair's loads are issued once this pair's MFMAs
    // have consumed their registers, small loads first again.
    for (int s = 0; s < nsteps; s += 2) {
        product(wa, act[0]);
        if (s + 1 >= nsteps) break;
        product(wb, act[1]);
        if (s + 2 >= nsteps) break;
        issue_small(s + 2, ga, ua);
        issue_small(s + 3, gb, ub);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        issue_w(s + 2, wa);
        issue_w(s + 3, wb);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // every wavefront is done with both buffers
        activate(ga, ua, act[0]);
        activate(gb, ub, act[1]);
        __syncthreads();
    }

    // The parts' sums, in part order, into the kg == 0 wavefronts.
    if constexpr (WK > 1) {
        if (kg > 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) part_acc[(((kg - 1) * WH + hg) * NT + nt) * 64 + lane] = acc[nt];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int p = 1; p < WK; ++p)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] += part_acc[(((p - 1) * WH + hg) * NT + nt) * 64 + lane];
        }
    }

    // Store, or exchange the split-k partials.  In the kg == 0 wavefronts,
    // lane l holds features h0 + g*4 + 0..3 of token nt*16 + l16.
    if (nK == 1) {
        if (kg == 0 && h_ok) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int i = nt * 16 + l16;
                if (i < nrows) {
                    const uint32_t lo = E::pack2(acc[nt][0], acc[nt][1]), hi = E::pack2(acc[nt][2], acc[nt][3]);
                    *reinterpret_cast<uint2 *>(y + (int64_t)(r0 + i) * H + h0 + g * 4) = uint2{lo, hi};
                }
            }
        }
        return;
    }
    const int64_t ngroups = (int64_t)((T + TM - 1) / TM) * nH;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(ws + down_cnt_offset(T));
    uint64_t *part = reinterpret_cast<uint64_t *>(ws + down_part_offset(T, ngroups));
    if (tid == 0) s_last = (int)epoch;
    __syncthreads();
    const uint32_t tag = 2u * (uint32_t)s_last + 1u;
    __syncthreads();
    if (kg == 0 && h_ok) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int i = nt * 16 + l16;
            if (i < nrows) {
                uint64_t *p = part + ((grp * nK + ks) * TM + i) * BH + hg * 16 + g * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) store_word(p + j, tagged(tag, acc[nt][j]));
            }
        }
    }
    // The tile counter is bumped by the last wavefront, which stores no
    // partials when WK > 1 (its wait for the counter's reply does not wait
    // for partial stores); the words carry their own proof of arrival, so the
    // counter need not follow their completion.
    __builtin_amdgcn_s_barrier();
    if (tid == NTH - 64) {
        const uint32_t prev = __hip_atomic_fetch_add(cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(nK - 1);
    }
    __syncthreads();
    if (!s_last) return;
    // The tile's last arrival: every partial it reads was stored before its
    // writer's counter update, so each poll below ends within a few memory
    // round trips; the bound (one budget of rounds per thread for all its
    // words) only guarantees termination.
    uint32_t budget = 1u << 20;
    for (int p = tid; p < nrows * (BH / 4); p += NTH) {
        const int i = p / (BH / 4), h4 = p % (BH / 4);
        const int h = h_first + h4 * 4;
        if (h >= H) continue;
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        constexpr int BATCH = 8;
        for (int s0 = 0; s0 < nK; s0 += BATCH) {
            uint64_t v[BATCH][4];
#pragma unroll
            for (int t = 0; t < BATCH; ++t) {
                if (s0 + t < nK) {
                    const uint64_t *q = part + ((grp * nK + s0 + t) * TM + i) * BH + h4 * 4;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[t][j] = load_word(q + j);
                }
            }
#pragma unroll
            for (int t = 0; t < BATCH; ++t) {
                if (s0 + t < nK) {
                    const uint64_t *q = part + ((grp * nK + s0 + t) * TM + i) * BH + h4 * 4;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        while ((uint32_t)v[t][j] != tag && budget > 0) {
                            --budget;
                            __builtin_amdgcn_s_sleep(1);
                            v[t][j] = load_word(q + j);
                        }
                        s4[j] += tag_value(v[t][j]);
                    }
                }
            }
        }
        const uint32_t lo = E::pack2(s4[0], s4[1]), hi = E::pack2(s4[2], s4[3]);
        *reinterpret_cast<uint2 *>(y + (int64_t)(r0 + i) * H + h) = uint2{lo, hi};
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

typedef void (*ProductKernel)(const uint16_t *, const uint16_t *, uint16_t *, int32_t, int32_t, int32_t, int32_t,
                              int32_t, int32_t, const int32_t *, unsigned char *);

struct DownEntry {
    int tm, wh, wk, nkbw;
    ProductKernel bf16, f16;
};

#define GA_DOWN(TM, WH, WK, NKBW)                                      \
    {TM, WH, WK, NKBW, down_product_kernel<DT_BF16, TM, WH, WK, NKBW>, \
     down_product_kernel<DT_F16, TM, WH, WK, NKBW>}

// (tokens, feature groups of 16, parts per step, 128-element blocks per part)
const DownEntry kDown[] = {
    GA_DOWN(16, 4, 2, 2), GA_DOWN(16, 8, 1, 2), GA_DOWN(16, 4, 1, 4), GA_DOWN(16, 4, 2, 1),
    GA_DOWN(16, 4, 1, 2), GA_DOWN(16, 2, 2, 2), GA_DOWN(16, 2, 1, 4), GA_DOWN(16, 4, 1, 1),
    GA_DOWN(32, 4, 2, 2), GA_DOWN(32, 4, 2, 1), GA_DOWN(32, 4, 1, 2), GA_DOWN(64, 4, 2, 1),
    GA_DOWN(64, 8, 1, 2), GA_DOWN(64, 4, 1, 2),
};

#undef GA_DOWN

const DownEntry *find_down(int tm, int waves, int bh, int step) {
    for (const DownEntry &e : kDown)
        if (e.tm == tm && e.wh * e.wk == waves && e.wh * 16 == bh && e.wk * e.nkbw * 128 == step) return &e;
    return nullptr;
}

}  // namespace

bool gelu_down_available(int dtype, int tm, int waves, int bh, int step) {
    return (dtype == DT_BF16 || dtype == DT_F16) && find_down(tm, waves, bh, step) != nullptr;
}

size_t gelu_down_workspace_bytes(int64_t T, int64_t d, int64_t H, int tm, int bh, int64_t ks) {
    const int64_t nK = (d + ks - 1) / ks;
    const int64_t ngroups = (T + tm - 1) / tm * ((H + bh - 1) / bh);
    if (nK <= 1) return (size_t)down_cnt_offset(T);
    return (size_t)(down_part_offset(T, ngroups) + ngroups * nK * tm * (int64_t)bh * 8);
}

hipError_t launch_gelu_down(int dtype, int tm, int waves, int bh, int step, int32_t ks, const void *gu,
                            const void *w, void *y, int32_t T, int32_t d, int32_t H, float z, const int32_t *live,
                            void *workspace, hipStream_t stream) {
    const DownEntry *e = find_down(tm, waves, bh, step);
    if (!e || (dtype != DT_BF16 && dtype != DT_F16) || ks % step != 0) return hipErrorInvalidValue;
    int32_t nK = (d + ks - 1) / ks;
    int32_t nH = (H + bh - 1) / bh;
    const int64_t grid = (int64_t)((T + tm - 1) / tm) * nH * nK;
    const uint16_t *a_gu = static_cast<const uint16_t *>(gu);
    const uint16_t *a_w = static_cast<const uint16_t *>(w);
    uint16_t *a_y = static_cast<uint16_t *>(y);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    int32_t ngroups = nK > 1 ? (int32_t)(grid / nK) : 0;
    void *cut_args[] = {&a_gu, &T, &d, &z, &live, &ws, &ngroups};
    const void *cut_k = dtype == DT_BF16 ? reinterpret_cast<const void *>(down_cutoff_kernel<DT_BF16>)
                                         : reinterpret_cast<const void *>(down_cutoff_kernel<DT_F16>);
    hipError_t err = hipLaunchKernel(cut_k, dim3((uint32_t)T), dim3(CUT_WAVES * 64), cut_args, 0, stream);
    if (err != hipSuccess) return err;
    ProductKernel k = dtype == DT_BF16 ? e->bf16 : e->f16;
    void *args[] = {&a_gu, &a_w, &a_y, &T, &d, &H, &nK, &nH, &ks, &live, &ws};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), dim3((uint32_t)grid), dim3(waves * 64), args, 0,
                           stream);
}

}  // namespace ga
