// Block geometry of the realigning gelu_and_mul_sparse path: rows whose gate,
// up or output start is not 16-byte aligned (a misaligned base pointer, or
// d * element size not a multiple of 16).  Each of the three streams of a row
// is read or written in its own 16-byte blocks; blocks of the two input
// streams are shifted onto the output's blocks through a window in LDS.
//
// Everything here is plain integer arithmetic shared by the kernel and the
// host (the planner, and a CPU emulation of the kernel's accesses), so that
// the index math is checked without a GPU.
#pragma once

#include <stdint.h>

namespace ga {

// Most 16-byte blocks a stream of d elements (per elements to a block) can
// touch, over every starting phase.
__host__ __device__ inline int32_t realign_blocks_max(int32_t d, int32_t per) {
    return (d + 2 * per - 2) / per;
}

// A stream of a row relative to 16-byte blocks: element e lies in block
// (e + phase) / per at position (e + phase) % per.
struct RealignStream {
    int32_t phase;   // elements of the first block before the stream starts, 0 .. per - 1
    int32_t blocks;  // blocks the stream touches
};

__host__ __device__ inline RealignStream realign_stream(uintptr_t addr, int32_t d, int32_t es) {
    const int32_t per = 16 / es;
    RealignStream s;
    s.phase = (int32_t)((addr & 15u) / (uintptr_t)es);
    s.blocks = (d + s.phase + per - 1) / per;
    return s;
}

// First element index of block i (negative for the part before the stream).
__host__ __device__ inline int32_t realign_first(int32_t i, int32_t phase, int32_t per) {
    return i * per - phase;
}

// Whether block i lies wholly inside the stream's elements [0, d).
__host__ __device__ inline bool realign_full(int32_t i, int32_t phase, int32_t d, int32_t per) {
    const int32_t first = realign_first(i, phase, per);
    return first >= 0 && first + per <= d;
}

// How an input stream maps onto the output's blocks.  Output block j starts
// at element j * per - out_phase, which lies in input block j + lead at
// position shift: lead = -1 when the input's phase is the smaller one, else 0.
struct RealignMap {
    int32_t lead;
    int32_t shift;  // elements, 0 .. per - 1
};

__host__ __device__ inline RealignMap realign_map(int32_t in_phase, int32_t out_phase, int32_t per) {
    RealignMap m;
    m.lead = in_phase < out_phase ? -1 : 0;
    m.shift = in_phase - out_phase + (in_phase < out_phase ? per : 0);
    return m;
}

// The window for output chunk c (output blocks c * nt .. c * nt + nt - 1)
// has nt + 1 slots; slot s holds input block c * nt + lead + s, so the
// lane of output block c * nt + t reads slots t and t + 1.  A lane that holds
// input block k * nt + t in register k writes, for chunk c, its block k = c
// to slot t - lead; the one slot left over is written by lane 0 from its
// block c + 1 (lead 0) or by lane nt - 1 from its block c - 1 (lead -1).
__host__ __device__ inline int32_t realign_slot_of_own(int32_t t, int32_t lead) {
    return t - lead;
}

// The lane that fills the left-over slot, and that slot.
__host__ __device__ inline int32_t realign_extra_lane(int32_t lead, int32_t nt) {
    return lead == 0 ? 0 : nt - 1;
}
__host__ __device__ inline int32_t realign_extra_slot(int32_t lead, int32_t nt) {
    return lead == 0 ? nt : 0;
}

// A window slot is four dwords kept dword-major (dword m of slot s at
// m * slots + s) so that consecutive lanes touch consecutive LDS words.
// Reading `per` elements that start `shift` elements into slot t takes the
// dwords q .. q + 4 of slots t, t + 1 (q = byte offset / 4) and, for a 2-byte
// offset, a 16-bit funnel shift.
__host__ __device__ inline int32_t realign_dword_index(int32_t t, int32_t x, int32_t slots) {
    return (x & 3) * slots + t + (x >> 2);
}

}  // namespace ga
