// CPU emulation of the realigning gelu_and_mul_sparse kernel's data movement
// (gated_activation_amd/csrc/gelu_sparse_realign.hip), built on the same
// geometry helpers (ga_realign.h).  For each case read from stdin,
//   es d waves vpl gate_phase up_phase out_phase
// (optionally followed by up_late, 0 or 1), it runs every lane of one workgroup through the kernel's loads, window
// writes, shifted window reads and stores, and checks that
//   - every 16-byte access is aligned and lies inside its row, every
//     element access inside [0, d);
//   - no two lanes write one window slot in a chunk, and every slot a lane
//     reads was written in that chunk;
//   - every LDS word index is inside the window array;
//   - each output element gets exactly the gate and up elements of its own
//     index, and every output element is written exactly once.
// Prints "ok <cases>" or the first failure; exits non-zero on failure.
#define __host__
#define __device__
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../gated_activation_amd/csrc/ga_realign.h"

using namespace ga;

namespace {

struct Fail {
    char msg[256];
};

// A stream of d elements whose value at index e is a tag (e + 1 + base);
// memory is a byte image with the row starting at byte phase * es of a
// 16-byte aligned buffer.
struct Stream {
    int es, d, phase;
    uint32_t base;
    std::vector<uint8_t> mem;  // aligned image, whole blocks
    Stream(int es_, int d_, int phase_, uint32_t base_) : es(es_), d(d_), phase(phase_), base(base_) {
        const int per = 16 / es;
        const int blocks = (d + phase + per - 1) / per;
        mem.assign((size_t)blocks * 16 + 16, 0xEE);
        for (int e = 0; e < d; ++e) put(e, tag(e));
    }
    uint32_t tag(int e) const {
        const uint32_t v = (uint32_t)e + 1u + base;
        return es == 2 ? (v & 0xFFFFu) : v;
    }
    size_t off(int e) const { return (size_t)(phase + e) * es; }
    void put(int e, uint32_t v) { std::memcpy(&mem[off(e)], &v, es); }
    uint32_t get(int e) const {
        uint32_t v = 0;
        std::memcpy(&v, &mem[off(e)], es);
        return v;
    }
};

typedef uint32_t Block[4];

bool check(bool ok, Fail &f, const char *what, int a, int b, int c) {
    if (!ok && f.msg[0] == 0) std::snprintf(f.msg, sizeof f.msg, "%s (%d, %d, %d)", what, a, b, c);
    return ok;
}

// load_block of the kernel: one aligned 16-byte read of block i, which must
// hold at least one byte of the row.
void load_block(const Stream &s, const RealignStream &rs, int i, Block out, Fail &f) {
    const int per = 16 / s.es;
    std::memset(out, 0, 16);
    if (i < 0 || i >= rs.blocks) return;
    const int first = realign_first(i, rs.phase, per);
    const long byte0 = (long)(s.phase + first) * s.es;   // offset in the aligned image
    check(byte0 % 16 == 0, f, "misaligned 16-byte load", i, first, (int)byte0);
    const long row0 = (long)s.phase * s.es, row1 = row0 + (long)s.d * s.es;
    check(byte0 < row1 && byte0 + 16 > row0, f, "16-byte load holds no byte of the row", i, first, s.d);
    check(byte0 >= 0 && byte0 + 16 <= (long)s.mem.size(), f, "load outside the image", i, first, (int)byte0);
    std::memcpy(out, &s.mem[byte0], 16);   // bytes outside the row come along unused
}

uint32_t elem_of(const Block b, int e, int es) {
    if (es == 4) return b[e];
    return (b[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
}

bool run_case(int es, int d, int waves, int vpl, int pg, int pu, int po, int up_late, Fail &f) {
    const int per = 16 / es;
    const int nt = waves * 64;
    const int slots = nt + 1;
    Stream g(es, d, pg, 0), u(es, d, pu, 1000000), o(es, d, po, 0);
    for (int e = 0; e < d; ++e) o.put(e, 0);
    std::vector<int> written(d, 0);
    const RealignStream sg = realign_stream((uintptr_t)pg * es, d, es);
    const RealignStream su = realign_stream((uintptr_t)pu * es, d, es);
    const RealignStream so = realign_stream((uintptr_t)po * es, d, es);
    if (!check(sg.phase == pg && su.phase == pu && so.phase == po, f, "phase", pg, pu, po)) return false;
    if (!check((int64_t)vpl * nt >= realign_blocks_max(d, per), f, "geometry does not cover the row", d, waves, vpl))
        return false;
    check(sg.blocks <= realign_blocks_max(d, per) && so.blocks <= realign_blocks_max(d, per), f,
          "blocks above the maximum", sg.blocks, so.blocks, d);

    // Gate registers of every lane.
    std::vector<Block> gv((size_t)nt * vpl);
    for (int t = 0; t < nt; ++t)
        for (int k = 0; k < vpl; ++k) load_block(g, sg, k * nt + t, gv[(size_t)t * vpl + k], f);
    // Every gate element appears once in the registers (statistics input).
    {
        std::vector<int> seen(d, 0);
        for (int t = 0; t < nt; ++t)
            for (int k = 0; k < vpl; ++k) {
                const int i = k * nt + t;
                if (i >= sg.blocks) continue;
                for (int e = 0; e < per; ++e) {
                    const int idx = realign_first(i, sg.phase, per) + e;
                    if (idx >= 0 && idx < d) {
                        seen[idx]++;
                        check(elem_of(gv[(size_t)t * vpl + k], e, es) == g.tag(idx), f, "gate register", t, k, e);
                    }
                }
            }
        for (int e = 0; e < d; ++e) check(seen[e] == 1, f, "gate element not held once", e, seen[e], 0);
    }

    const RealignMap mg = realign_map(sg.phase, so.phase, per);
    const RealignMap mu = realign_map(su.phase, so.phase, per);
    // Up registers: lane t, register k holds block k * nt + t.
    std::vector<Block> uv((size_t)nt * vpl);
    for (int t = 0; t < nt; ++t)
        for (int k = 0; k < vpl; ++k) load_block(u, su, k * nt + t, uv[(size_t)t * vpl + k], f);
    std::vector<uint32_t> win[2];
    std::vector<int> owner[2];
    for (int c = 0; c < vpl; ++c) {
        if (c * nt >= so.blocks) break;
        for (int w = 0; w < 2; ++w) {
            win[w].assign((size_t)4 * slots, 0xDEADBEEFu);
            owner[w].assign(slots, -1);
        }
        auto write_slot = [&](int w, int slot, int lane, const Block v) {
            if (!check(slot >= 0 && slot < slots, f, "slot outside the window", w, slot, lane)) return;
            check(owner[w][slot] == -1, f, "two lanes write one slot", w, slot, lane);
            owner[w][slot] = lane;
            for (int m = 0; m < 4; ++m) win[w][(size_t)m * slots + slot] = v[m];
        };
        // fill_window of the kernel, for both streams.
        auto fill = [&](int w, const std::vector<Block> &regs, int lead) {
            for (int t = 0; t < nt; ++t) {
                write_slot(w, realign_slot_of_own(t, lead), t, regs[(size_t)t * vpl + c]);
                if (t == realign_extra_lane(lead, nt)) {
                    Block v = {0, 0, 0, 0};
                    if (lead == 0) {
                        if (c + 1 < vpl) std::memcpy(v, regs[(size_t)t * vpl + c + 1], 16);
                    } else if (c >= 1) {
                        std::memcpy(v, regs[(size_t)t * vpl + c - 1], 16);
                    }
                    write_slot(w, realign_extra_slot(lead, nt), t, v);
                }
            }
        };
        fill(0, gv, mg.lead);
        if (!up_late) {
            fill(1, uv, mu.lead);
        } else {
            // Up blocks loaded for this chunk: own block c * nt + t; the
            // left-over slot from lane 0's load of block (c + 1) * nt (lead
            // 0) or lane nt - 1's block of the previous chunk (lead -1).
            for (int t = 0; t < nt; ++t) {
                Block cur;
                load_block(u, su, c * nt + t, cur, f);
                write_slot(1, realign_slot_of_own(t, mu.lead), t, cur);
                if (t == realign_extra_lane(mu.lead, nt)) {
                    Block ext = {0, 0, 0, 0};
                    if (mu.lead == 0)
                        load_block(u, su, (c + 1) * nt, ext, f);
                    else if (c >= 1)
                        load_block(u, su, (c - 1) * nt + t, ext, f);
                    write_slot(1, realign_extra_slot(mu.lead, nt), t, ext);
                }
            }
        }
        for (int w = 0; w < 2; ++w)
            for (int sl = 0; sl < slots; ++sl) check(owner[w][sl] != -1, f, "slot not written", w, sl, c);
        // The window holds the expected input blocks.
        for (int sl = 0; sl < slots; ++sl) {
            Block ge, ue;
            load_block(g, sg, c * nt + mg.lead + sl, ge, f);
            load_block(u, su, c * nt + mu.lead + sl, ue, f);
            for (int m = 0; m < 4; ++m) {
                check(win[0][(size_t)m * slots + sl] == ge[m], f, "gate window content", c, sl, m);
                check(win[1][(size_t)m * slots + sl] == ue[m], f, "up window content", c, sl, m);
            }
        }
        for (int t = 0; t < nt; ++t) {
            const int j = c * nt + t;
            if (j >= so.blocks) continue;
            Block gb, ub;
            for (int w = 0; w < 2; ++w) {
                const int shift = w == 0 ? mg.shift : mu.shift;
                const int b = shift * es, q = b >> 2;
                uint32_t dw[5];
                for (int i = 0; i < 5; ++i) {
                    const int x = realign_dword_index(t, q + i, slots);
                    if (!check(x >= 0 && x < 4 * slots, f, "LDS word outside the window", t, q, i)) return false;
                    dw[i] = win[w][x];
                }
                uint32_t *dst = w == 0 ? gb : ub;
                for (int i = 0; i < 4; ++i)
                    dst[i] = (b & 3) == 0 ? dw[i] : ((dw[i] >> 16) | (dw[i + 1] << 16));
            }
            // Output block j: element e has index j * per - po + e.
            const bool full = realign_full(j, so.phase, d, per);
            for (int e = 0; e < per; ++e) {
                const int idx = realign_first(j, so.phase, per) + e;
                if (idx < 0 || idx >= d) continue;
                check(elem_of(gb, e, es) == g.tag(idx), f, "realigned gate element", j, e, idx);
                check(elem_of(ub, e, es) == u.tag(idx), f, "realigned up element", j, e, idx);
                written[idx]++;
            }
            if (full) {
                const int first = realign_first(j, so.phase, per);
                check(o.off(first) % 16 == 0, f, "misaligned 16-byte store", j, first, (int)o.off(first));
            }
        }
    }
    for (int e = 0; e < d; ++e) check(written[e] == 1, f, "output element not written once", e, written[e], 0);
    return f.msg[0] == 0;
}

}  // namespace

int main() {
    int es, d, waves, vpl, pg, pu, po, up_late, n = 0;
    char line[256];
    while (std::fgets(line, sizeof line, stdin)) {
        up_late = 0;
        const int got = std::sscanf(line, "%d %d %d %d %d %d %d %d", &es, &d, &waves, &vpl, &pg, &pu, &po, &up_late);
        if (got < 7) continue;
        Fail f;
        f.msg[0] = 0;
        if (!run_case(es, d, waves, vpl, pg, pu, po, up_late, f)) {
            std::printf("FAIL es=%d d=%d waves=%d vpl=%d phases=%d,%d,%d up_late=%d: %s\n", es, d, waves, vpl, pg,
                        pu, po, up_late, f.msg);
            return 1;
        }
        ++n;
    }
    std::printf("ok %d\n", n);
    return 0;
}
