// Rows of gelu_and_mul_sparse that are not 16-byte aligned, seen as 16-byte
// vectors of consecutive elements: vector j of a stream of d elements is its
// elements [PER j, PER j + PER), PER = 16 bytes / element size, each moved as
// one unaligned 16-byte access (ldu16 / stu16 in ga_device.h).  Only the
// last vector can be partial (d % PER elements).
#pragma once

#include "ga_device.h"

namespace ga {

// The first n elements of a 16-byte vector, the rest zero.
template <typename E>
__device__ __forceinline__ uint4 keep_first(const uint4 &v, int32_t n) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (E::PER16 == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e >= n) w[e] = 0u;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e >= n) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    }
    return uint4{w[0], w[1], w[2], w[3]};
}

template <typename E>
__device__ __forceinline__ typename E::storage elem_of(const uint4 &v, int e) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (E::PER16 == 4) {
        return w[e];
    } else {
        return (typename E::storage)(w[e >> 1] >> ((e & 1) * 16));
    }
}

// Vector j of a stream of a row (zero past the row).  `spill`: the 16 bytes
// of the partial last vector lie inside the input buffer.
template <typename E>
__device__ __forceinline__ uint4 load_vec(const typename E::storage *row, int32_t j, int32_t nfull, int32_t tail,
                                         bool spill) {
    constexpr int PER = E::PER16;
    if (j < nfull) return ldu16(row + (size_t)PER * j);
    uint4 v{0u, 0u, 0u, 0u};
    if (j == nfull && tail > 0) {
        // Few lanes get here (one per row), at an address the compiler could
        // prove uniform and turn into a scalar load, which would drop the low
        // bits of a 2-byte-aligned address; the empty asm keeps j per lane.
        int32_t jv = j;
        asm volatile("" : "+v"(jv));
        if (spill) {
            v = keep_first<E>(ldu16(row + (size_t)PER * jv), tail);
        } else {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                if (e < tail) {
                    const uint32_t x = (uint32_t)row[(size_t)PER * jv + e];
                    if constexpr (PER == 4) w[e] = x;
                    else w[e >> 1] |= x << ((e & 1) * 16);
                }
            }
            v = uint4{w[0], w[1], w[2], w[3]};
        }
    }
    return v;
}

template <typename E>
__device__ __forceinline__ void store_vec(typename E::storage *row, int32_t j, int32_t nfull, int32_t tail,
                                          const uint4 &v) {
    constexpr int PER = E::PER16;
    if (j < nfull) {
        stu16(row + (size_t)PER * j, v);
        return;
    }
    if (j != nfull) return;  // past the row
#pragma unroll
    for (int e = 0; e < PER; ++e)
        if (e < tail) row[(size_t)PER * j + e] = elem_of<E>(v, e);
}

}  // namespace ga
