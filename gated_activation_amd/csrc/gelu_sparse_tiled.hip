// gelu_and_mul_sparse fused with the down projection, tiled form: three to
// 256 tokens.
//   y[r, h] = sum_k a[r, k] * w[h, k],   a = gelu_and_mul_sparse(gu) as stored
// gu is [T, 2d] (gate | up), w is [H, d] with one row of weights per output
// feature, y is [T, H]; fp32 sums on the matrix cores, rounded once.
//
// Two launches.  The first is the library's own activation kernel for the
// call's rows writing a into the caller's workspace ([T, d], formed once).
// The second, down_tiled_kernel, is a matrix product over that stored
// activation.  Workgroup (tb, hb, ks) owns tokens [tb*TM, +TM), output
// features [hb*BH, +BH) and the slice [ks*KC, +KC) of d; each of its WAVES
// wavefronts owns FW groups of 16 features.  Per step of KSTEP elements of d
//   - the workgroup loads the step's activation tile (TM tokens x KSTEP) once,
//     each lane 16-byte vectors already in the matrix cores' operand order,
//     and parks it in LDS, where every wavefront reads it: the activation
//     comes from the cache once per workgroup, not once per wavefront;
//   - each wavefront loads its own weights straight into registers (the
//     A operand, 16 features x 32 k per instruction), the bulk of the bytes;
//   - v_mfma_f32_16x16x32 with the weights as A and the activation as B
//     (32 k x 16 tokens, read from LDS once per instruction column and used
//     for all FW feature groups), fp32 accumulators.
// The loads of step s + PD (activation tile, then weights) are issued before
// step s's products, into the registers step s - 1 used; one barrier per step
// guards the LDS tiles.  The weight stream is the cost: the matrix cores and
// LDS take a small share of the time at these token counts.
//
// Operand order.  The MFMA pairs lane l's eight A elements with its eight B
// elements at the same k positions: in a step, instruction kk covers elements
// [kk*32, +32) and lane l (g = l / 16) supplies [kk*32 + g*8, +8) of feature
// row l % 16 (A) and of token l % 16 (B).  Each load instruction reads 64
// contiguous bytes of each of 16 rows (measured as fast, for the weights, as
// whole contiguous rows per instruction).  The accumulator of lane l holds
// features 4g .. 4g+3 of token l % 16.
//
// Slices of d.  Workgroup ks = blockIdx % nK: the dispatcher deals workgroups
// to the eight XCDs in turn, so with nK a multiple of 8 every workgroup on an
// XCD works on the same slices of d and that XCD's L2 holds their activation.
// With one slice the workgroup stores y.  With several, each stores its fp32
// partial tile into the workspace with device-scope stores, waits for their
// acknowledgement and bumps the output tile's counter; the last of the nK to
// arrive reads the nK partials with device-scope loads, adds them in
// slice order (so the result does not depend on which workgroup came last),
// stores y and sets the counter back to zero.  The counters live in a fixed
// region of the workspace that nothing else writes, so a zero-filled
// workspace serves any sequence of calls and shapes, and graph replays.
//
// Rows past the live count, features past H and elements past the slice read
// zero through buffer descriptors without touching memory.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4_t mfma16(const uint4 &a, const uint4 &b, f32x4_t c) {
    if constexpr (DT == DT_BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                       __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// An offset at or past a buffer descriptor's range reads zero and touches no
// memory; kOob is past every range the kernel builds.
constexpr int kOob = (int)0x80000000;

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t src, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, 0));
}

// Cache-policy bits of the buffer instructions on gfx950: SC1 makes a store
// write through to the device's coherence point and a load read from it (the
// bits a device-scope atomic store or load carries), for all 16 bytes at once.
constexpr int kSc1 = 16;

__device__ __forceinline__ f32x4_t coherent_load4(__amdgpu_buffer_rsrc_t src, int off) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, kSc1));
}

__device__ __forceinline__ void coherent_store4(__amdgpu_buffer_rsrc_t dst, int off, f32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), dst, off, 0, kSc1);
}

}  // namespace

template <int DT, int TM, int FW, int WAVES, int KSTEP, int PD>
__global__ __launch_bounds__(WAVES * 64) void down_tiled_kernel(const uint16_t *a, const uint16_t *w, uint16_t *y,
                                                                int32_t T, int32_t d, int32_t H, int32_t nK,
                                                                int32_t nH, int32_t KC, const int32_t *live,
                                                                unsigned char *ws) {
    using E = Elem<DT>;
    constexpr int NTH = WAVES * 64;
    constexpr int NT = TM / 16;             // 16-token tiles
    constexpr int KK = KSTEP / 32;          // MFMA instructions per tile and step
    constexpr int BH = WAVES * FW * 16;
    constexpr int AVEC = NT * KK * 64;      // 16-byte vectors of one step's activation tile
    constexpr int APL = (AVEC + NTH - 1) / NTH;
    constexpr int NB = PD + 1;              // steps per loop body: register sets and LDS tiles
    static_assert(TM % 16 == 0 && KSTEP % 32 == 0 && PD >= 1, "whole operand tiles");
    static_assert(NB * AVEC * 16 <= 65536, "at most 64 KB of LDS per workgroup");
    __shared__ uint4 lds[NB * AVEC];        // activation tiles: [step % NB][(tile * KK + kk) * 64 + lane]
    int &s_last = *reinterpret_cast<int *>(lds);  // after the loop: whether this workgroup sums the tile

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront: scalar branches
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t b = blockIdx.x;
    const int ks = (int)(b % nK);
    const int64_t tile = b / nK;
    const int hb = (int)(tile % nH);
    const int tb = (int)(tile / nH);
    const int n_live = live ? clamp_live(live, T) : T;
    const int r0 = tb * TM;
    if (r0 >= n_live) return;  // no live token in this block (uniform over the tile's nK workgroups)
    const int nrows = n_live - r0 < TM ? n_live - r0 : TM;
    const int k0 = ks * KC;
    const int k_end = d - k0 < KC ? d : k0 + KC;
    const int nsteps = (k_end - k0 + KSTEP - 1) / KSTEP;
    const int h_first = hb * BH;
    const int hrows = H - h_first < BH ? H - h_first : BH;
    const int hw = wv * FW * 16;            // the wavefront's first feature in the block
    const bool w_live = hw < hrows;         // H is a multiple of 16: whole feature groups in or out
                                            // (with FW > 1 the later groups are tested again)

    const __amdgpu_buffer_rsrc_t asrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a + (int64_t)r0 * d), (short)0, nrows * d * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w + (int64_t)h_first * d), (short)0, hrows * d * 2, 0x00020000);

    // The activation tile of step s: vector q = (tile * KK + kk) * 64 + l
    // holds token tile*16 + l % 16, elements kk*32 + (l / 16)*8 .. +8 of the
    // step.  A step at or past nsteps starts at or past k_end, so all its
    // loads read zero: no separate test of s.
    auto issue_act = [&](int s, uint4 (&ar)[APL]) {
#pragma unroll
        for (int i = 0; i < APL; ++i) {
            const int q = tid + NTH * i;
            const int fi = q >> 6, ln = q & 63;
            const int tok = (fi / KK) * 16 + (ln & 15);
            const int k = k0 + s * KSTEP + (fi % KK) * 32 + (ln >> 4) * 8;
            const int off = (AVEC % NTH == 0 || q < AVEC) && k < k_end ? (tok * d + k) * 2 : kOob;
            ar[i] = bload(asrc, off);
        }
    };
    auto park_act = [&](const uint4 (&ar)[APL], uint4 *buf) {
#pragma unroll
        for (int i = 0; i < APL; ++i) {
            const int q = tid + NTH * i;
            if (AVEC % NTH == 0 || q < AVEC) buf[q] = ar[i];
        }
    };
    auto issue_w = [&](int s, uint4 (&Wr)[FW][KK]) {
#pragma unroll
        for (int f = 0; f < FW; ++f)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int k = k0 + s * KSTEP + kk * 32 + g * 8;
                const int off = k < k_end ? ((hw + f * 16 + l16) * d + k) * 2 : kOob;
                Wr[f][kk] = bload(wsrc, off);
            }
    };
    f32x4_t acc[FW][NT];
#pragma unroll
    for (int f = 0; f < FW; ++f)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[f][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // Every token tile, live or not (tiles past the live rows multiply zeros
    // and are never stored): a test per tile would put a branch between the
    // LDS reads and the MFMAs and serialise them.
    auto product = [&](const uint4 (&Wr)[FW][KK], const uint4 *buf) {
        if (!w_live) return;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 bv[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bv[nt] = buf[(nt * KK + kk) * 64 + lane];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int f = 0; f < FW; ++f) acc[f][nt] = mfma16<DT>(Wr[f][kk], bv[nt], acc[f][nt]);
        }
    };

    // Loads PD steps ahead: at step j those of step j + PD are issued (the
    // activation tile into registers, then the weights), into the register
    // sets step j - 1 used, and the activation of step j + 1 moves from its
    // registers into LDS.  The loop body covers NB steps so every index is
    // fixed at compile time (a count that is not a multiple of NB ends with
    // steps of zeros: their loads read nothing).
    uint4 aset[NB][APL];
    uint4 wset[NB][FW][KK];
#pragma unroll
    for (int p = 0; p < PD; ++p) {
        issue_act(p, aset[p]);
        issue_w(p, wset[p]);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    park_act(aset[0], lds);
    __syncthreads();
    for (int s = 0; s < nsteps; s += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            issue_act(s + j + PD, aset[(j + PD) % NB]);
            issue_w(s + j + PD, wset[(j + PD) % NB]);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            product(wset[j], lds + j * AVEC);
            park_act(aset[(j + 1) % NB], lds + ((j + 1) % NB) * AVEC);
            __syncthreads();
        }
    }

    // Lane l holds features hw + f*16 + 4g .. +3 of token nt*16 + l16.
    if (nK == 1) {
        if (w_live) {
#pragma unroll
            for (int f = 0; f < FW; ++f)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int i = nt * 16 + l16;
                    if (i < nrows && hw + f * 16 < hrows) {
                        const uint32_t lo = E::pack2(acc[f][nt][0], acc[f][nt][1]);
                        const uint32_t hi = E::pack2(acc[f][nt][2], acc[f][nt][3]);
                        *reinterpret_cast<uint2 *>(y + (int64_t)(r0 + i) * H + h_first + hw + f * 16 + g * 4) =
                            uint2{lo, hi};
                    }
                }
        }
        return;
    }
    // This tile's nK partial tiles, [slice][token][feature] fp32, through a
    // descriptor of their own (offsets in bytes from the tile's first).
    const __amdgpu_buffer_rsrc_t psrc = __builtin_amdgcn_make_buffer_rsrc(
        ws + down_tiled_part_offset(T, d) + tile * nK * TM * BH * 4, (short)0, nK * TM * BH * 4, 0x00020000);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(ws + DOWN_TILE_CNT_OFFSET);
    // Partials are written with the device-scope cache policy (SC1), which
    // acknowledges a store once it has reached the device's point of
    // coherence, and every wavefront waits for those acknowledgements before
    // the workgroup's counter update; whoever sees the count reach nK - 1
    // reads them with device-scope loads, served from that point.  (A release
    // fence here would write the whole L2 back: measured 1.7x slower.)
    if (w_live) {
#pragma unroll
        for (int f = 0; f < FW; ++f)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int i = nt * 16 + l16;
                if (i < nrows && hw + f * 16 < hrows)
                    coherent_store4(psrc, ((ks * TM + i) * BH + hw + f * 16 + g * 4) * 4, acc[f][nt]);
            }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(nK - 1);
    }
    __syncthreads();
    if (!s_last) return;
    // The tile's last arrival: the nK partials in slice order.  Each thread
    // sums U of the tile's 4-feature outputs at a time with the loads of QB
    // slices of all U in flight together (16 loads), so a thread's outputs
    // take a few memory round trips, not one each.
    constexpr int C4 = BH / 4;
    constexpr int PER = (TM * C4 + NTH - 1) / NTH;  // outputs per thread in a full tile
    constexpr int U = PER < 1 ? 1 : PER > 4 ? 4 : PER;
    constexpr int QB = 16 / U;
    const int n4 = nrows * C4;
    for (int p0 = tid; p0 < n4; p0 += NTH * U) {
        f32x4_t s4[U];
#pragma unroll
        for (int u = 0; u < U; ++u) s4[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int q0 = 0; q0 < nK; q0 += QB) {
            f32x4_t v[U][QB];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = p0 + u * NTH;
                const int i = p / C4, c = p % C4;
                const bool ok = p < n4 && c * 4 < hrows;
#pragma unroll
                for (int q = 0; q < QB; ++q)
                    v[u][q] = coherent_load4(psrc, ok && q0 + q < nK ? (((q0 + q) * TM + i) * BH + c * 4) * 4 : kOob);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < QB; ++q)
                    if (q0 + q < nK) s4[u] += v[u][q];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * NTH;
            const int i = p / C4, c = p % C4;
            if (p < n4 && c * 4 < hrows) {
                const uint32_t lo = E::pack2(s4[u][0], s4[u][1]), hi = E::pack2(s4[u][2], s4[u][3]);
                *reinterpret_cast<uint2 *>(y + (int64_t)(r0 + i) * H + h_first + c * 4) = uint2{lo, hi};
            }
        }
    }
    if (tid == 0) __hip_atomic_store(cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

typedef void (*TiledKernel)(const uint16_t *, const uint16_t *, uint16_t *, int32_t, int32_t, int32_t, int32_t,
                            int32_t, int32_t, const int32_t *, unsigned char *);

struct TiledEntry {
    int tm, fw, waves, kstep, pd;
    TiledKernel bf16, f16;
};

#define GA_TILED(TM, FW, W, KS, PD)                                                     \
    {TM, FW, W, KS, PD, down_tiled_kernel<DT_BF16, TM, FW, W, KS, PD>, \
     down_tiled_kernel<DT_F16, TM, FW, W, KS, PD>}

// (tokens, 16-feature groups per wavefront, wavefronts, elements of d per
// step, steps of loads in flight): the planner's choices (measured fastest at
// d = 16384, H = 2048) and their neighbours in the sweep.
const TiledEntry kTiled[] = {
    GA_TILED(16, 1, 4, 128, 1), GA_TILED(16, 1, 4, 256, 1), GA_TILED(16, 1, 4, 64, 3), GA_TILED(16, 1, 8, 128, 2),
    GA_TILED(16, 1, 4, 256, 2), GA_TILED(16, 1, 4, 128, 3), GA_TILED(16, 1, 2, 256, 2),
    GA_TILED(32, 1, 4, 128, 1), GA_TILED(32, 1, 4, 64, 3), GA_TILED(32, 1, 4, 128, 2), GA_TILED(32, 1, 4, 128, 3),
    GA_TILED(64, 1, 8, 128, 1), GA_TILED(64, 1, 8, 64, 3), GA_TILED(64, 2, 4, 64, 2), GA_TILED(64, 1, 8, 128, 2),
    GA_TILED(64, 1, 4, 128, 2), GA_TILED(64, 1, 4, 128, 3), GA_TILED(64, 2, 4, 128, 3),
    GA_TILED(128, 1, 8, 64, 1), GA_TILED(128, 1, 8, 64, 2), GA_TILED(128, 2, 8, 64, 2), GA_TILED(128, 1, 8, 128, 1),
    GA_TILED(128, 1, 8, 64, 3), GA_TILED(128, 2, 8, 64, 3), GA_TILED(128, 2, 4, 64, 3),
};

#undef GA_TILED

const TiledEntry *find_tiled(int tm, int bh, int waves, int kstep, int depth) {
    for (const TiledEntry &e : kTiled)
        if (e.tm == tm && e.waves == waves && e.fw * 16 * e.waves == bh && e.kstep == kstep && e.pd == depth)
            return &e;
    return nullptr;
}

}  // namespace

bool gelu_down_tiled_available(int dtype, int tm, int bh, int waves, int kstep, int depth) {
    return (dtype == DT_BF16 || dtype == DT_F16) && find_tiled(tm, bh, waves, kstep, depth) != nullptr;
}

size_t gelu_down_tiled_workspace_bytes(int64_t T, int64_t d, int64_t H, int tm, int bh, int64_t kc) {
    const int64_t nK = (d + kc - 1) / kc;
    const int64_t tiles = (T + tm - 1) / tm * ((H + bh - 1) / bh);
    return (size_t)(down_tiled_part_offset(T, d) + (nK > 1 ? tiles * nK * tm * (int64_t)bh * 4 : 0));
}

hipError_t launch_gelu_down_tiled(int dtype, int tm, int bh, int waves, int kstep, int depth, int32_t kc, const void *a,
                                  const void *w, void *y, int32_t T, int32_t d, int32_t H, const int32_t *live,
                                  void *workspace, hipStream_t stream) {
    const TiledEntry *e = find_tiled(tm, bh, waves, kstep, depth);
    if (!e || (dtype != DT_BF16 && dtype != DT_F16) || kc % kstep != 0) return hipErrorInvalidValue;
    int32_t nK = (d + kc - 1) / kc;
    int32_t nH = (H + bh - 1) / bh;
    const int64_t grid = (int64_t)((T + tm - 1) / tm) * nH * nK;
    const uint16_t *a_a = static_cast<const uint16_t *>(a);
    const uint16_t *a_w = static_cast<const uint16_t *>(w);
    uint16_t *a_y = static_cast<uint16_t *>(y);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    void *args[] = {&a_a, &a_w, &a_y, &T, &d, &H, &nK, &nH, &kc, &live, &ws};
    return hipLaunchKernel(reinterpret_cast<const void *>(dtype == DT_BF16 ? e->bf16 : e->f16), dim3((uint32_t)grid),
                           dim3(waves * 64), args, 0, stream);
}

}  // namespace ga
