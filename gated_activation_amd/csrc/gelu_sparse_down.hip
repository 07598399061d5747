// gelu_and_mul_sparse fused with the down projection that consumes it:
//   y[r, h] = sum_k a[r, k] * w[h, k],   a = gelu_and_mul_sparse(gu) as stored
// (the activation rounded once to the element type), summed in fp32 on the
// matrix cores, rounded once.  gu is [T, 2d] (gate | up), w is [H, d] with one
// row of weights per output feature (a linear layer's layout), y is [T, H].
// The vLLM page (PR 48498, Test Result, Correctness) has the activation's
// write feed the layer's downstream projection; here the activation never
// leaves the compute unit: it is formed in the staging of the product's
// operand.
//
// Work decomposition.  Workgroup (rb, hb, ks) owns tokens [rb*TM, rb*TM+TM),
// output features [hb*BH, hb*BH+BH) (BH = 16 per wavefront) and the k-slice
// [ks*BK, ks*BK+BK) of d.  The nK = ceil(d / BK) workgroups of one (rb, hb)
// form a group; they are consecutive in launch order.  Each workgroup:
//   1. issues the loads of its gate and up slices (TM x BK each), then of its
//      BH x BK block of w straight into registers (the bulk of the bytes at
//      decode sizes, in flight during steps 2-4);
//   2. reduces each token row's slice to (mean, M2) (two passes over the
//      registers);
//   3. publishes them as tagged words and polls the group's other slices
//      (bounded; past the bound it computes the rows' statistics itself), then
//      combines the nK partials in slice order with Chan's update, so every
//      workgroup of the row derives the same cutoff;
//   4. applies relu, tanh-GELU and the product with up in fp32, rounds to the
//      element type and writes the result to LDS in the matrix cores' operand
//      order;
//   5. runs the 16x16x32 MFMAs: w as the A operand (16 features x 32 k per
//      instruction, from registers), the activation as B (32 k x 16 tokens,
//      from LDS), fp32 accumulators;
//   6. with nK > 1, publishes its fp32 partial tile as tagged words and bumps
//      the group's counter; the last of the group to arrive sums the nK
//      partials in slice order (a deterministic split-k reduction) and stores
//      y.  With nK == 1 it stores y directly.
//
// Operand order.  The MFMA pairs lane l's A elements with lane l's B elements
// at the same eight k positions, so any permutation of k shared by A and B
// leaves the product unchanged.  Lane l (g = l / 16) takes, in k block kb
// (128 elements), the 32 consecutive elements [kb*128 + g*32, +32) as the
// four instructions' eight-element operands: one 64-byte run of w per lane
// and per k block, and of gate and up when the activation is formed, so
// both sides load whole runs and the LDS operand layout is conflict-free.
//
// Tags.  Each call tags its words with 2 * epoch + 1, where epoch is a word
// of the workspace that the last group to finish advances by one; every
// workgroup reads it before it can take part in the group counts, so all of
// a call's workgroups use the same tag, and a word written in an earlier call
// carries an older tag (a reuse needs 2^31 calls with the workspace).
// Counters return to zero at the end of each call, so the zero-filled
// workspace serves any sequence of calls and shapes, and graph replays.
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

}  // namespace

template <int TM, int NUNITS>
struct DownShared {
    uint4 act[NUNITS * 4 * 64];  // B operands: [tile][k block][instruction][lane]
    float red[NUNITS * 64];      // per-lane partial sums
    float pm[TM][DOWN_MAX_SPLITS], pq[TM][DOWN_MAX_SPLITS];
    float mean[TM], m2[TM], cut[TM];
    int flag;
};

// The kernel body, instantiated twice: POLLER for wavefront 0, which runs the
// statistics exchange and only then loads its share of w, and !POLLER for the
// others, which load w first.  Loads complete in issue order, so a
// wavefront with w in flight could not see a polled word before its w had
// arrived; and one body with a branch around the w loads would make the
// compiler wait, in every wavefront, as if none had been issued.  The
// dispatch is uniform per wavefront, and both copies pass the same barriers.
template <int DT, int TM, int WAVES, int BK, bool POLLER>
__device__ __forceinline__ void down_body(DownShared<TM, (TM / 16) * (BK / 128)> &sh, const uint16_t *__restrict__ gu,
                                          const uint16_t *__restrict__ w, uint16_t *__restrict__ y, int32_t T,
                                          int32_t d, int32_t H, int32_t nK, int32_t nH, float z,
                                          const int32_t *__restrict__ live, unsigned char *__restrict__ ws,
                                          uint32_t spin_limit) {
    using E = Elem<DT>;
    constexpr int NT = TM / 16;                               // 16-token tiles
    constexpr int NKB = BK / 128;                             // 128-element k blocks
    constexpr int NUNITS = NT * NKB;                          // (token tile, k block) units
    constexpr int UPW = (NUNITS + WAVES - 1) / WAVES;         // units per wavefront
    constexpr int NTH = WAVES * 64;
    constexpr int BH = WAVES * 16;

    uint4 *act = sh.act;
    float *red = sh.red;
    float(&pm)[TM][DOWN_MAX_SPLITS] = sh.pm;
    float(&pq)[TM][DOWN_MAX_SPLITS] = sh.pq;
    float *s_mean = sh.mean, *s_m2 = sh.m2, *s_cut = sh.cut;
    int &s_flag = sh.flag;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t b = blockIdx.x;
    const int ks = (int)(b % nK);
    const int64_t grp = b / nK;
    const int hb = (int)(grp % nH);
    const int rb = (int)(grp / nH);
    const int n_live = live ? clamp_live(live, T) : T;
    const int r0 = rb * TM;
    if (r0 >= n_live) return;  // no live token in this block (uniform)
    const int nrows = n_live - r0 < TM ? n_live - r0 : TM;
    const int k0 = ks * BK;
    const int nk_here = d - k0 < BK ? d - k0 : BK;  // a multiple of 8
    const int64_t two_d = 2 * (int64_t)d;

    // Workspace: [0] epoch, [128] groups done, [256 ..) group counters, then
    // the statistics words and the partial tiles.
    uint32_t *epoch_p = reinterpret_cast<uint32_t *>(ws);
    uint32_t *done_p = reinterpret_cast<uint32_t *>(ws + 128);
    const int64_t ngroups = (int64_t)((T + TM - 1) / TM) * nH;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(ws + 256);
    const int64_t cnt_bytes = (ngroups * 4 + 255) / 256 * 256;
    uint64_t *stat = reinterpret_cast<uint64_t *>(ws + 256 + cnt_bytes);
    uint64_t *part = stat + ngroups * nK * TM * 2;
    uint32_t tag = 0;
    if (nK > 1) {
        const uint32_t e = __hip_atomic_load(epoch_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tag = 2u * (uint32_t)__builtin_amdgcn_readfirstlane((int)e) + 1u;
    }

    // 1. gate and up slices for this wavefront's units, then the w block.
    // Every load is issued unconditionally, from a clamped in-bounds address
    // where the element lies outside the data (tokens past the live count:
    // the block's first row; k past d: the slice's first run; features past
    // H: the last 16 rows of w), and such values are replaced by zero where
    // they are used.  Conditional loads would make the compiler wait for
    // each one before the next, serialising the stream of w.
    uint4 gv[UPW][4], uv[UPW][4];
#pragma unroll
    for (int q = 0; q < UPW; ++q) {
        const int u = wv + WAVES * q < NUNITS ? wv + WAVES * q : NUNITS - 1;
        const int i = (u / NKB) * 16 + l16;            // token in the block
        const int kl = (u % NKB) * 128 + g * 32;       // first element of the lane's run
        const uint16_t *grow = gu + (int64_t)(r0 + (i < nrows ? i : 0)) * two_d + k0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int kj = kl + jj * 8 < nk_here ? kl + jj * 8 : 0;
            gv[q][jj] = *reinterpret_cast<const uint4 *>(grow + kj);
            uv[q][jj] = *reinterpret_cast<const uint4 *>(grow + d + kj);
        }
    }
    const int h0 = hb * BH + wv * 16;  // this wavefront's 16 features
    const bool h_ok = h0 < H;          // H is a multiple of 16: whole wavefronts in or out
    const uint16_t *wrow = w + (int64_t)((h_ok ? h0 : H - 16) + l16) * d + k0;
    uint4 wr[NKB][4];
    auto load_w = [&]() {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int kj = kb * 128 + g * 32 + jj * 8;
                wr[kb][jj] = ld16<true>(reinterpret_cast<const uint4 *>(wrow + (kj < nk_here ? kj : 0)));
            }
        }
    };
    if constexpr (!POLLER) load_w();

    // 2. per-row (mean, M2) of this slice: lane partials, then a fixed-order
    // sum over lanes g = 0..3 and k blocks.
    {
#pragma unroll
        for (int q = 0; q < UPW; ++q) {
            const int u = wv + WAVES * q;
            const int i = (u / NKB) * 16 + l16;
            const int kl = (u % NKB) * 128 + g * 32;
            float acc = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if (i < nrows && kl + jj * 8 < nk_here) {
                    float f[8];
                    E::unpack(gv[q][jj], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += f[e];
                }
            }
            if (u < NUNITS) red[u * 64 + lane] = acc;
        }
    }
    __syncthreads();
    const float n_here = (float)nk_here;
    if (tid < nrows) {
        const int nt = tid / 16, i16 = tid & 15;
        float s = 0.0f;
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) s += red[(nt * NKB + kb) * 64 + gg * 16 + i16];
        s_mean[tid] = row_mean<false>(s, n_here);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < UPW; ++q) {
        const int u = wv + WAVES * q;
        const int i = (u / NKB) * 16 + l16;
        const int kl = (u % NKB) * 128 + g * 32;
        float acc = 0.0f;
        if (u < NUNITS && i < nrows) {
            const float m = s_mean[i];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if (kl + jj * 8 < nk_here) {
                    float f[8];
                    E::unpack(gv[q][jj], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float dv = f[e] - m;
                        acc = __builtin_fmaf(dv, dv, acc);
                    }
                }
            }
        }
        if (u < NUNITS) red[u * 64 + lane] = acc;
    }
    __syncthreads();
    if (tid < nrows) {
        const int nt = tid / 16, i16 = tid & 15;
        float s = 0.0f;
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) s += red[(nt * NKB + kb) * 64 + gg * 16 + i16];
        s_m2[tid] = s;
        if (nK > 1) {
            uint64_t *slot = stat + ((grp * nK + ks) * TM + tid) * 2;
            store_word(slot, tagged(tag, s_mean[tid]));
            store_word(slot + 1, tagged(tag, s));
        }
    }
    __syncthreads();

    // 3. the other slices' partials of the group, then the cutoffs, in
    // wavefront 0: rounds of up to 256 (row, slice) pairs, four per lane,
    // each round's loads issued together.
    if constexpr (POLLER) {
        bool ok = true;
        if (nK > 1) {
            const int npairs = nrows * nK;
            for (int p0 = 0; p0 < npairs && ok; p0 += 256) {
                uint32_t pending = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int p = p0 + q * 64 + lane;
                    if (p < npairs) {
                        const int i = p / nK, s = p % nK;
                        if (s == ks) {
                            pm[i][s] = s_mean[i];
                            pq[i][s] = s_m2[i];
                        } else {
                            pending |= 1u << q;
                        }
                    }
                }
                uint32_t polls = 0;
                while (true) {
                    uint64_t a[4], c[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (pending & (1u << q)) {
                            const int p = p0 + q * 64 + lane;
                            const uint64_t *slot = stat + ((grp * nK + p % nK) * TM + p / nK) * 2;
                            a[q] = load_word(slot);
                            c[q] = load_word(slot + 1);
                        }
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if ((pending & (1u << q)) && (uint32_t)a[q] == tag && (uint32_t)c[q] == tag) {
                            const int p = p0 + q * 64 + lane;
                            pm[p / nK][p % nK] = tag_value(a[q]);
                            pq[p / nK][p % nK] = tag_value(c[q]);
                            pending &= ~(1u << q);
                        }
                    }
                    if (__builtin_amdgcn_ballot_w64(pending != 0) == 0) break;
                    if (++polls > spin_limit) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
        }
        if (ok) {
            if (lane < nrows) {
                float n_acc = 0.0f, mean = 0.0f, m2 = 0.0f;
                for (int s = 0; s < nK; ++s) {
                    const int ns = d - s * BK < BK ? d - s * BK : BK;
                    const float im = nK > 1 ? pm[lane][s] : s_mean[lane];
                    const float iq = nK > 1 ? pq[lane][s] : s_m2[lane];
                    if (s == 0) {
                        n_acc = (float)ns;
                        mean = im;
                        m2 = iq;
                    } else {
                        chan_combine(n_acc, mean, m2, (float)ns, im, iq);
                    }
                }
                s_cut[lane] = sparse_cutoff<E, false>(mean, row_var<false>(m2, (float)d), z);
            }
        } else {
            // Bounded wait expired: the rows' statistics from global memory,
            // a row at a time, two passes.
            const int nvec = d / 8;
            for (int i = 0; i < nrows; ++i) {
                const uint4 *grow = reinterpret_cast<const uint4 *>(gu + (int64_t)(r0 + i) * two_d);
                float a = 0.0f;
                for (int j = lane; j < nvec; j += 64) {
                    float f[8];
                    E::unpack(grow[j], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) a += f[e];
                }
                const float mean = row_mean<false>(wave_sum(a), (float)d);
                float c = 0.0f;
                for (int j = lane; j < nvec; j += 64) {
                    float f[8];
                    E::unpack(grow[j], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float dv = f[e] - mean;
                        c = __builtin_fmaf(dv, dv, c);
                    }
                }
                const float m2 = wave_sum(c);
                if (lane == 0) s_cut[i] = sparse_cutoff<E, false>(mean, row_var<false>(m2, (float)d), z);
            }
        }
        load_w();
    }
    __syncthreads();

    // 4. the activation, rounded to the element type, into the operand layout.
#pragma unroll
    for (int q = 0; q < UPW; ++q) {
        const int u = wv + WAVES * q;
        if (u < NUNITS) {
            const int i = (u / NKB) * 16 + l16;
            const int kl = (u % NKB) * 128 + g * 32;
            const float cut = i < nrows ? s_cut[i] : 0.0f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint4 o = {0, 0, 0, 0};
                if (i < nrows && kl + jj * 8 < nk_here) {
                    float f[8], v[8];
                    E::unpack(gv[q][jj], f);
                    E::unpack(uv[q][jj], v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = sparse_apply<E, false>(f[e], cut, v[e]);
                    o = E::pack(f);
                }
                act[(u * 4 + jj) * 64 + lane] = o;
            }
        }
    }
    __syncthreads();

    // 5. the product on the matrix cores.
    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (h_ok) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt * 16 < nrows) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        acc[nt] = mfma_16x16x32<DT>(kb * 128 + g * 32 + jj * 8 < nk_here ? wr[kb][jj] : uint4{0, 0, 0, 0},
                                                    act[((nt * NKB + kb) * 4 + jj) * 64 + lane], acc[nt]);
            }
        }
    }

    // 6. store, or exchange the split-k partials.  Lane l holds features
    // h0 + g*4 + 0..3 of token nt*16 + l16.
    if (nK == 1) {
        if (h_ok) {
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
    if (h_ok) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int i = nt * 16 + l16;
            if (i < nrows) {
                uint64_t *p = part + ((grp * nK + ks) * TM + i) * BH + wv * 16 + g * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) store_word(p + j, tagged(tag, acc[nt][j]));
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = prev == (uint32_t)(nK - 1) ? 2 : 3;
    }
    __syncthreads();
    if (s_flag != 2) return;
    if (tid == 0) __hip_atomic_store(cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The group's last arrival: every partial it reads was stored before its
    // writer's counter update, so each poll below ends within a few memory
    // round trips; the bound (one budget of rounds per thread for all its
    // words, independent of spin_limit) only guarantees termination.
    uint32_t budget = 1u << 20;
    for (int p = tid; p < nrows * (BH / 4); p += NTH) {
        const int i = p / (BH / 4), h4 = p % (BH / 4);
        const int h = hb * BH + h4 * 4;
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
    __syncthreads();
    if (tid == 0) {
        const int64_t live_groups = (int64_t)((n_live + TM - 1) / TM) * nH;
        const uint32_t prev = __hip_atomic_fetch_add(done_p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int64_t)prev == live_groups - 1) {
            __hip_atomic_store(done_p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t e = __hip_atomic_load(epoch_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(epoch_p, e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int DT, int TM, int WAVES, int BK>
__global__ __launch_bounds__(WAVES * 64) void gelu_sparse_down_kernel(
    const uint16_t *__restrict__ gu, const uint16_t *__restrict__ w, uint16_t *__restrict__ y, int32_t T,
    int32_t d, int32_t H, int32_t nK, int32_t nH, float z, const int32_t *__restrict__ live,
    unsigned char *__restrict__ ws, uint32_t spin_limit) {
    __shared__ DownShared<TM, (TM / 16) * (BK / 128)> sh;
    if (__builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) == 0) {
        down_body<DT, TM, WAVES, BK, true>(sh, gu, w, y, T, d, H, nK, nH, z, live, ws, spin_limit);
    } else {
        down_body<DT, TM, WAVES, BK, false>(sh, gu, w, y, T, d, H, nK, nH, z, live, ws, spin_limit);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

typedef void (*DownKernel)(const uint16_t *, const uint16_t *, uint16_t *, int32_t, int32_t, int32_t, int32_t,
                           int32_t, float, const int32_t *, unsigned char *, uint32_t);

struct DownEntry {
    int tm, waves, bk;
    DownKernel bf16, f16;
};

#define GA_DOWN(TM, W, BK) \
    {TM, W, BK, gelu_sparse_down_kernel<DT_BF16, TM, W, BK>, gelu_sparse_down_kernel<DT_F16, TM, W, BK>}

const DownEntry kDown[] = {
    GA_DOWN(16, 4, 256), GA_DOWN(16, 4, 512), GA_DOWN(16, 4, 1024), GA_DOWN(16, 8, 256),
    GA_DOWN(16, 8, 512), GA_DOWN(16, 8, 1024), GA_DOWN(32, 4, 512), GA_DOWN(32, 8, 512),
    GA_DOWN(64, 4, 256), GA_DOWN(64, 4, 512), GA_DOWN(64, 8, 512),
};

#undef GA_DOWN

const DownEntry *find_down(int tm, int waves, int bk) {
    for (const DownEntry &e : kDown)
        if (e.tm == tm && e.waves == waves && e.bk == bk) return &e;
    return nullptr;
}

}  // namespace

bool gelu_down_available(int dtype, int tm, int waves, int bk) {
    return (dtype == DT_BF16 || dtype == DT_F16) && find_down(tm, waves, bk) != nullptr;
}

size_t gelu_down_workspace_bytes(int64_t T, int64_t d, int64_t H, int tm, int waves, int bk) {
    const int64_t nK = (d + bk - 1) / bk;
    if (nK <= 1) return 0;
    const int64_t ngroups = (T + tm - 1) / tm * ((H + waves * 16 - 1) / (waves * 16));
    const int64_t cnt_bytes = (ngroups * 4 + 255) / 256 * 256;
    return (size_t)(256 + cnt_bytes + ngroups * nK * tm * 16 + ngroups * nK * tm * (int64_t)(waves * 16) * 8);
}

hipError_t launch_gelu_down(int dtype, int tm, int waves, int bk, const void *gu, const void *w, void *y,
                            int32_t T, int32_t d, int32_t H, float z, const int32_t *live, void *workspace,
                            uint32_t spin_limit, hipStream_t stream) {
    const DownEntry *e = find_down(tm, waves, bk);
    if (!e || (dtype != DT_BF16 && dtype != DT_F16)) return hipErrorInvalidValue;
    int32_t nK = (d + bk - 1) / bk;
    int32_t nH = (H + waves * 16 - 1) / (waves * 16);
    const int64_t grid = (int64_t)((T + tm - 1) / tm) * nH * nK;
    DownKernel k = dtype == DT_BF16 ? e->bf16 : e->f16;
    const uint16_t *a_gu = static_cast<const uint16_t *>(gu);
    const uint16_t *a_w = static_cast<const uint16_t *>(w);
    uint16_t *a_y = static_cast<uint16_t *>(y);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    void *args[] = {&a_gu, &a_w, &a_y, &T, &d, &H, &nK, &nH, &z, &live, &ws, &spin_limit};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), dim3((uint32_t)grid), dim3(waves * 64), args, 0,
                           stream);
}

}  // namespace ga
