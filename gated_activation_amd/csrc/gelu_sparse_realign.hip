// gelu_and_mul_sparse for rows that are not 16-byte aligned (gfx950).
//
// The op is the one of gelu_sparse.hip (vLLM PR 48498, "[Performance] Add
// Triton kernel for Gemma3n sparse GELU", section Purpose).  This path takes
// rows whose gate, up or output start is not on a 16-byte boundary: a base
// pointer offset by a few elements, or d * element size not a multiple of 16
// (then the phase changes from row to row).  One-element accesses would run
// at a third of the vector path's bandwidth, so each stream is still moved in
// its own 16-byte blocks:
//   - the gate row is loaded block by block into registers (the blocks at
//     the two ends, which reach past the row, element by element) and the
//     statistics skip the positions outside the row;
//   - the output is produced one output-aligned block per lane, in chunks of
//     NT blocks; for each chunk the gate blocks (from registers) and the up
//     blocks (loaded for the chunk) go through an LDS window of NT + 1 slots,
//     from which each lane reads the 16 bytes that line up with its output
//     block (a 2-byte funnel shift for 16-bit types when needed).
// Writes never leave the row: end blocks that reach past it are written
// per element.  Reads of end blocks are whole aligned 16-byte blocks whose
// bytes outside the row are never used (see load_block).  Block geometry:
// ga_realign.h.
#include "ga_device.h"
#include "ga_internal.h"
#include "ga_realign.h"

namespace ga {

namespace {

template <typename E>
__device__ __forceinline__ typename E::storage elem_of(const uint4 &v, int e) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (E::PER16 == 4) {
        return w[e];
    } else {
        return (typename E::storage)(w[e >> 1] >> ((e & 1) * 16));
    }
}

// Block i of a stream that starts `phase` elements into its first block:
// one aligned 16-byte load (zero for blocks outside [0, blocks)).  An end
// block reaches past the row: an aligned 16-byte block never crosses a page
// and holds at least one of the row's bytes, so the access stays inside
// mapped memory; its bytes beyond the row are never used (the statistics
// skip them and no output element reads them).  Every lane loads a
// different block, so these stay vector-memory loads (a load whose address
// the compiler can prove uniform may become a scalar load, which would drop
// the low address bits of a 2-byte-aligned row base).
template <typename E>
__device__ __forceinline__ uint4 load_block(const typename E::storage *row, int32_t i, const RealignStream &s) {
    if (i < 0 || i >= s.blocks) return uint4{0u, 0u, 0u, 0u};
    return ld16<true>(reinterpret_cast<const uint4 *>(row + realign_first(i, s.phase, E::PER16)));
}

template <typename E>
__device__ __forceinline__ void store_block(typename E::storage *row, int32_t i, const RealignStream &s, int32_t d,
                                            const uint4 &v) {
    constexpr int PER = E::PER16;
    if (realign_full(i, s.phase, d, PER)) {
        st16<true>(reinterpret_cast<uint4 *>(row + realign_first(i, s.phase, PER)), v);
        return;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int32_t idx = realign_first(i, s.phase, PER) + e;
        if (idx >= 0 && idx < d) row[idx] = elem_of<E>(v, e);
    }
}

template <int SLOTS>
__device__ __forceinline__ void write_slot(uint32_t *w, int32_t slot, const uint4 &v) {
    w[0 * SLOTS + slot] = v.x;
    w[1 * SLOTS + slot] = v.y;
    w[2 * SLOTS + slot] = v.z;
    w[3 * SLOTS + slot] = v.w;
}

// The 16 bytes that start `shift` elements into slot t.
template <typename E, int SLOTS>
__device__ __forceinline__ uint4 read_shifted(const uint32_t *w, int32_t t, int32_t shift) {
    constexpr int ES = 16 / E::PER16;
    const int32_t b = shift * ES;
    const int32_t q = b >> 2;
    uint32_t dw[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) dw[i] = w[realign_dword_index(t, q + i, SLOTS)];
    if ((b & 3) == 0) return uint4{dw[0], dw[1], dw[2], dw[3]};
    // 2-byte offset (16-bit types only): each word takes the high half of
    // one dword and the low half of the next.
    return uint4{(dw[0] >> 16) | (dw[1] << 16), (dw[1] >> 16) | (dw[2] << 16), (dw[2] >> 16) | (dw[3] << 16),
                 (dw[3] >> 16) | (dw[4] << 16)};
}

// Window of output chunk c from registers holding blocks k * NT + t: each
// lane writes its block c to slot t - lead, and the one slot left over takes
// lane 0's block c + 1 (lead 0) or lane NT - 1's block c - 1 (lead -1), zero
// past either end of the registers.
template <int VPL, int SLOTS>
__device__ __forceinline__ void fill_window(uint32_t *w, const uint4 (&regs)[VPL], int c, int32_t t, int32_t lead) {
    constexpr int NT = SLOTS - 1;
    write_slot<SLOTS>(w, realign_slot_of_own(t, lead), regs[c]);
    if (t == realign_extra_lane(lead, NT)) {
        uint4 v{0u, 0u, 0u, 0u};
        if (lead == 0) {
            if (c + 1 < VPL) v = regs[c + 1 < VPL ? c + 1 : 0];
        } else if (c >= 1) {
            v = regs[c >= 1 ? c - 1 : 0];
        }
        write_slot<SLOTS>(w, realign_extra_slot(lead, NT), v);
    }
}

}  // namespace

// Lane t holds gate blocks t, t + NT, ... (VPL of them, VPL * NT >= the
// blocks any phase can touch).  RT: round-trip form.  UPLATE: load the up
// blocks chunk by chunk after the statistics (fewer registers, more rows
// resident) instead of all of them with the gate.
template <int DT, int WAVES, int VPL, bool RT = false, bool UPLATE = false>
__global__ __launch_bounds__(WAVES * 64) void gelu_sparse_realign_kernel(
    const typename Elem<DT>::storage *__restrict__ in, typename Elem<DT>::storage *__restrict__ out, int32_t T,
    int32_t d, float z, const int32_t *__restrict__ live) {
    using E = Elem<DT>;
    using S = typename E::storage;
    constexpr int NT = WAVES * 64;
    constexpr int PER = E::PER16;
    constexpr int ES = 16 / PER;
    constexpr int SLOTS = NT + 1;
    // Two sets of windows (one barrier per chunk) while they fit in 64 KB.
    constexpr int NBUF = 2 * 2 * 4 * SLOTS * 4 <= 65536 ? 2 : 1;
    __shared__ float red[2][WAVES];
    __shared__ uint32_t win[NBUF][2][4 * SLOTS];  // [set][gate, up][dword-major slots]

    const int32_t r = (int32_t)blockIdx.x;
    if (live != nullptr && r >= clamp_live(live, T)) return;  // uniform per workgroup

    const S *grow = in + (size_t)r * 2 * (size_t)d;
    const S *urow = grow + d;
    S *orow = out + (size_t)r * (size_t)d;
    const int32_t t = (int32_t)threadIdx.x;
    const RealignStream sg = realign_stream((uintptr_t)grow, d, ES);
    const RealignStream su = realign_stream((uintptr_t)urow, d, ES);
    const RealignStream so = realign_stream((uintptr_t)orow, d, ES);

    // Gate blocks (and, unless UPLATE, up blocks) into registers: register
    // k of lane t holds block k * NT + t.
    constexpr int NUV = UPLATE ? 1 : VPL;
    uint4 gv[VPL], uv[NUV];
#pragma unroll
    for (int k = 0; k < VPL; ++k) gv[k] = load_block<E>(grow, k * NT + t, sg);
    if constexpr (!UPLATE) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) uv[k] = load_block<E>(urow, k * NT + t, su);
    }

    // Statistics over the row's elements only (end blocks hold others).
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t i = k * NT + t;
        if (i < sg.blocks) {
            float g[PER];
            E::unpack(gv[k], g);
            const bool full = realign_full(i, sg.phase, d, PER);
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int32_t idx = realign_first(i, sg.phase, PER) + e;
                s += (full || (idx >= 0 && idx < d)) ? g[e] : 0.0f;
            }
        }
    }
    const float mean = block_sum<WAVES>(s, red[0]) / (float)d;

    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int32_t i = k * NT + t;
        if (i < sg.blocks) {
            float g[PER];
            E::unpack(gv[k], g);
            const bool full = realign_full(i, sg.phase, d, PER);
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int32_t idx = realign_first(i, sg.phase, PER) + e;
                const float dv = (full || (idx >= 0 && idx < d)) ? g[e] - mean : 0.0f;
                q = __builtin_fmaf(dv, dv, q);
            }
        }
    }
    const float var = block_sum<WAVES>(q, red[1]) / (float)d;
    const float cut = sparse_cutoff<E, RT>(mean, var, z);

    // Apply, one chunk of NT output blocks at a time.
    const RealignMap mg = realign_map(sg.phase, so.phase, PER);
    const RealignMap mu = realign_map(su.phase, so.phase, PER);
    uint4 uprev{0u, 0u, 0u, 0u};  // UPLATE: this lane's up block of the previous chunk
#pragma unroll
    for (int c = 0; c < VPL; ++c) {
        if (c * NT >= so.blocks) break;  // uniform per workgroup
        uint32_t *wg = win[c % NBUF][0];
        uint32_t *wu = win[c % NBUF][1];
        fill_window<VPL, SLOTS>(wg, gv, c, t, mg.lead);
        if constexpr (UPLATE) {
            // The same window from blocks loaded now: own block c * NT + t;
            // the left-over slot takes lane 0's block (c + 1) * NT (loaded
            // here by lane 0 as well; the asm makes the index look per-lane
            // so the load stays a vector-memory load) or lane NT - 1's block
            // of the previous chunk.
            const uint4 ucur = load_block<E>(urow, c * NT + t, su);
            uint4 uext = uprev;
            if (mu.lead == 0 && t == 0) {
                int32_t i = (c + 1) * NT;
                asm volatile("" : "+v"(i));
                uext = load_block<E>(urow, i, su);
            }
            write_slot<SLOTS>(wu, realign_slot_of_own(t, mu.lead), ucur);
            if (t == realign_extra_lane(mu.lead, NT)) write_slot<SLOTS>(wu, realign_extra_slot(mu.lead, NT), uext);
            uprev = ucur;
        } else {
            fill_window<VPL, SLOTS>(wu, uv, c, t, mu.lead);
        }
        __syncthreads();

        const int32_t j = c * NT + t;
        if (j < so.blocks) {
            float g[PER], u[PER], y[PER];
            E::unpack(read_shifted<E, SLOTS>(wg, t, mg.shift), g);
            E::unpack(read_shifted<E, SLOTS>(wu, t, mu.shift), u);
#pragma unroll
            for (int e = 0; e < PER; ++e) y[e] = sparse_apply<E, RT>(g[e], cut, u[e]);
            store_block<E>(orow, j, so, d, E::pack(y));
        }
        // With two sets, chunk c + 2 rewrites this set only after every lane
        // has passed chunk c + 1's barrier, i.e. after its reads here.
        if constexpr (NBUF == 1) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Launch table: [round trip][up late][dtype][log2 waves][vectors per lane - 1].
// ---------------------------------------------------------------------------
namespace {

#define GA_RK(RT, UL, DT, W, V) (const void *)&gelu_sparse_realign_kernel<DT, W, V, RT, UL>
#define GA_RA(RT, UL, DT, W)                                                                                 \
    { GA_RK(RT, UL, DT, W, 1), GA_RK(RT, UL, DT, W, 2), GA_RK(RT, UL, DT, W, 3), GA_RK(RT, UL, DT, W, 4), \
      GA_RK(RT, UL, DT, W, 5), GA_RK(RT, UL, DT, W, 6), GA_RK(RT, UL, DT, W, 7), GA_RK(RT, UL, DT, W, 8) }
#define GA_RAD(RT, UL, DT) \
    { GA_RA(RT, UL, DT, 1), GA_RA(RT, UL, DT, 2), GA_RA(RT, UL, DT, 4), GA_RA(RT, UL, DT, 8), GA_RA(RT, UL, DT, 16) }
#define GA_RAU(RT, UL) { GA_RAD(RT, UL, DT_F32), GA_RAD(RT, UL, DT_F16), GA_RAD(RT, UL, DT_BF16) }
const void *const kGeluRealign[2][2][3][5][8] = {{GA_RAU(false, false), GA_RAU(false, true)},
                                                  {GA_RAU(true, false), GA_RAU(true, true)}};
#undef GA_RK
#undef GA_RA
#undef GA_RAD
#undef GA_RAU

int waves_index(int waves) {
    return waves == 1 ? 0 : waves == 2 ? 1 : waves == 4 ? 2 : waves == 8 ? 3 : waves == 16 ? 4 : -1;
}

}  // namespace

bool gelu_realign_available(int dtype, int waves, int vpl, int up_late) {
    return dtype >= 0 && dtype <= 2 && waves_index(waves) >= 0 && vpl >= 1 && vpl <= 8 &&
           (up_late == 0 || up_late == 1);
}

hipError_t launch_gelu_realign(int dtype, int waves, int vpl, int up_late, bool round_trip, int64_t grid,
                               const void *in, void *out, int32_t T, int32_t d, float z, const int32_t *live,
                               hipStream_t stream) {
    if (!gelu_realign_available(dtype, waves, vpl, up_late)) return hipErrorInvalidValue;
    const void *fn = kGeluRealign[round_trip ? 1 : 0][up_late][dtype][waves_index(waves)][vpl - 1];
    const void *a_in = in;
    void *a_out = out;
    void *args[] = {&a_in, &a_out, &T, &d, &z, &live};
    return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(waves * 64), args, 0, stream);
}

}  // namespace ga
