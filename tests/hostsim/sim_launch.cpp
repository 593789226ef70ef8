// sim_launch.cpp -- TEST INFRASTRUCTURE: a host-memory stand-in for the two
// kernel launch functions of rr_kernels.hip, linked with the product's
// rr_api.cpp into tests/hostsim/libhostsim.so.  It replays, workgroup by
// workgroup and lane by lane, the tile and index arithmetic the kernels use,
// checks every access against the buffers the test registered, and performs
// the access on host memory.  It exercises the C ABI's validation, geometry,
// segment tables, head/body/tail splits and launch batching on the CPU, so an
// addressing mistake shows up here as a recorded violation rather than as a
// fault on the GPU.  It is never part of the product library.
//
// In check-only mode (sim_set_check_only) the registered ranges need hold no
// memory -- they may be made-up device addresses for buffers of any size --
// and no access is performed: every access is checked as above, except that
// the aligned body of a tile is checked as one range per input and output
// after every lane's vector has been shown to land in it exactly once, which
// keeps full-size launches (tens of GB of accesses) to seconds.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "rr_internal.h"

namespace {

using rr::TileBody;

struct Buf {
    uintptr_t lo, hi;
    bool writable;
};
std::vector<Buf> g_bufs;
long g_violations = 0;
char g_msg[256];
long g_launches = 0;
bool g_check_only = false;  // accesses are checked, never performed

bool inside(uintptr_t a, int64_t n, bool write)
{
    for (const Buf &b : g_bufs)
        if (a >= b.lo && a + uintptr_t(n) <= b.hi && (!write || b.writable))
            return true;
    return false;
}

// The realigned copy reads whole aligned 16-byte words; one that holds at
// least one byte of a registered buffer stays inside that buffer's page.
bool touches(uintptr_t a, int64_t n)
{
    for (const Buf &b : g_bufs)
        if (a < b.hi && b.lo < a + uintptr_t(n))
            return true;
    return false;
}

long g_forms[2][3];  // launches per (copy?, launch form)
long g_long_copies[2];  // copy launches per tiling (0 default, 1 long-call)
long g_shifted_copies;  // copy launches in the mixed-mode (realigning) kernels
long g_nt_copies[2];    // copy launches per store policy (0 agent scope, 1 non-temporal)

void violation(const char *what, uintptr_t a, int64_t n)
{
    if (g_violations++ == 0)
        snprintf(g_msg, sizeof g_msg, "%s at %#lx (+%lld)", what, (unsigned long)a, (long long)n);
}

float ld(const void *p, int64_t i, bool bf16)
{
    const uintptr_t a = uintptr_t(p) + uintptr_t(i * (bf16 ? 2 : 4));
    if (!inside(a, bf16 ? 2 : 4, false)) {
        violation("read", a, bf16 ? 2 : 4);
        return 0.0f;
    }
    if (g_check_only)
        return 0.0f;
    if (bf16) {
        uint32_t u = uint32_t(*reinterpret_cast<const uint16_t *>(a)) << 16;
        float f;
        memcpy(&f, &u, 4);
        return f;
    }
    return *reinterpret_cast<const float *>(a);
}

void st(void *p, int64_t i, float v, bool bf16)
{
    const uintptr_t a = uintptr_t(p) + uintptr_t(i * (bf16 ? 2 : 4));
    if (!inside(a, bf16 ? 2 : 4, true)) {
        violation("write", a, bf16 ? 2 : 4);
        return;
    }
    if (g_check_only)
        return;
    if (bf16) {
        uint32_t u;
        memcpy(&u, &v, 4);
        if ((u & 0x7fffffffu) > 0x7f800000u)
            u = (u | 0x00400000u);
        else
            u += 0x7fffu + ((u >> 16) & 1u);
        *reinterpret_cast<uint16_t *>(a) = uint16_t(u >> 16);
    } else {
        *reinterpret_cast<float *>(a) = v;
    }
}

void fold(const rr::RedSeg &s, int64_t i, bool bf16)
{
    float acc = ld(s.in[0], i, bf16);
    for (int k = 1; k < s.k; ++k)
        acc = acc + ld(s.in[k], i, bf16);
    st(s.out, i, acc * s.scale, bf16);
}

void copy_byte(const unsigned char *src, unsigned char *dst, int64_t i)
{
    if (!inside(uintptr_t(src + i), 1, false))
        violation("copy read", uintptr_t(src + i), 1);
    else if (!inside(uintptr_t(dst + i), 1, true))
        violation("copy write", uintptr_t(dst + i), 1);
    else if (!g_check_only)
        dst[i] = src[i];
}

// The (segment, tile) pairs that the workgroups of a launch process, in the
// launch form the library chose: the table form walks the batch's tiles, the
// uniform form its (tile, segment) grid, the single-segment form segment 0.
// Flags a form whose grid would not cover every tile of the batch exactly once.
template <typename Batch>
std::vector<std::pair<int, int64_t>> tiles_of(const Batch &b, int64_t total, const rr::LaunchShape &sh)
{
    std::vector<std::pair<int, int64_t>> out;
    auto tiles = [&](int s) { return (s + 1 < b.nseg ? int64_t(b.tile0[s + 1]) : total) - b.tile0[s]; };
    if (sh.form == rr::kFormUniform) {
        if (sh.gy != b.nseg)
            violation("uniform grid height differs from the segment count", 0, sh.gy);
        for (int y = 0; y < sh.gy && y < b.nseg; ++y) {
            if (tiles(y) != sh.gx)
                violation("uniform grid width differs from a segment's tile count", 0, tiles(y));
            for (int64_t x = 0; x < sh.gx; ++x)
                out.emplace_back(y, x);
        }
    } else if (sh.form == rr::kFormOne) {
        if (b.nseg != 1 || sh.gx != total || sh.gy != 1)
            violation("single-segment grid for a batch it does not cover", 0, b.nseg);
        for (int64_t x = 0; x < sh.gx; ++x)
            out.emplace_back(0, x);
    } else {
        if (sh.gx != total || sh.gy != 1)
            violation("table grid differs from the tile count", 0, sh.gx);
        for (int64_t t = 0; t < total; ++t) {
            const int s = rr::find_seg(b.tile0, b.nseg, int32_t(t));
            out.emplace_back(s, t - b.tile0[s]);
        }
    }
    return out;
}

// Check-only mode: the body vectors the lanes of tile lt store (vec_index for
// every lane and step with v < nv), each exactly once, and exactly the
// tile's body range.  Returns that range.
template <int U>
TileBody stored_body(int64_t lt, int64_t nv, uintptr_t where)
{
    using namespace rr;
    constexpr int64_t tv = tile_vecs<U>();
    const TileBody tb = tile_body(lt, tv, nv);
    static std::vector<unsigned char> seen;
    seen.assign(size_t(tv), 0);
    int64_t stored = 0;
    for (int x = 0; x < kBlock; ++x)
        for (int u = 0; u < U; ++u) {
            const int64_t v = vec_index<U>(lt, x, u);
            if (v >= nv)
                continue;
            const int64_t i = v - tb.first;
            if (i < 0 || i >= tb.count || seen[size_t(i)]) {
                violation("lane vector outside its tile's body or stored twice", where, v);
                continue;
            }
            seen[size_t(i)] = 1;
            ++stored;
        }
    if (stored != tb.count)
        violation("tile leaves part of its body unstored", where, stored);
    return tb;
}

// Tiles of segment s of a launch of `total` tiles.
template <typename Batch>
int64_t seg_tiles(const Batch &b, int s, int64_t total)
{
    return (s + 1 < b.nseg ? int64_t(b.tile0[s + 1]) : total) - b.tile0[s];
}

// Replay of tile lt of a reduction segment, lane by lane, with the kernels'
// own index functions (rr_internal.h): which body vectors each lane folds,
// which aligned input words it loads, and which edge elements tile 0's lanes
// compute.  U is the segment mode's vectors per lane.
template <int U>
void replay_red_tile(const rr::RedBatch &b, int s, int64_t total, int64_t lt, const rr::RedSeg &sg, int64_t head,
                     int64_t nv, int64_t tail, bool bf16)
{
    using namespace rr;
    const int64_t es = bf16 ? 2 : 4, ve = 16 / es;
    constexpr int64_t tv = tile_vecs<U>();
    if (seg_tiles(b, s, total) != body_tiles(nv, tv))
        violation("reduction segment tile count differs from its body", uintptr_t(sg.out), seg_tiles(b, s, total));
    const bool shift_mode = sg.mode == kRedShifted;
    const unsigned char *base[kMaxIn];
    bool shifted[kMaxIn];
    for (int k = 0; k < sg.k; ++k) {
        const WordAt w = word_at(static_cast<const unsigned char *>(sg.in[k]) + head * es);
        shifted[k] = shift_mode && w.shift != 0;
        base[k] = shift_mode ? w.base : static_cast<const unsigned char *>(sg.in[k]) + head * es;
    }
    const bool full = full_tile(lt, tv, nv);
    if (g_check_only && !shift_mode) {
        if (nv > 0) {
            const TileBody tb = stored_body<U>(lt, nv, uintptr_t(sg.out));
            const int64_t off = (head + tb.first * ve) * es, len = tb.count * 16;
            for (int k = 0; k < sg.k; ++k)
                if (!inside(uintptr_t(sg.in[k]) + uintptr_t(off), len, false))
                    violation("read", uintptr_t(sg.in[k]) + uintptr_t(off), len);
            if (!inside(uintptr_t(sg.out) + uintptr_t(off), len, true))
                violation("write", uintptr_t(sg.out) + uintptr_t(off), len);
        }
    } else if (full || nv > 0)
        for (int x = 0; x < kBlock; ++x)
            for (int u = 0; u < U; ++u) {
                const int64_t v = vec_index<U>(lt, x, u);
                for (int k = 0; k < sg.k; ++k) {
                    if (!shift_mode)
                        continue;  // aligned inputs: the fold below checks every element read
                    if (loads_own_word(full, v, nv, shifted[k]) && !touches(uintptr_t(base[k] + v * 16), 16))
                        violation("realigned input word outside every buffer", uintptr_t(base[k] + v * 16), 16);
                    if (loads_next_word(full, v, nv, shifted[k], wave_end(x)) &&
                        !touches(uintptr_t(base[k] + (v + 1) * 16), 16))
                        violation("realigned input word outside every buffer", uintptr_t(base[k] + (v + 1) * 16), 16);
                }
                if (full || v < nv)  // the lanes that store
                    for (int64_t e = 0; e < ve; ++e)
                        fold(sg, head + v * ve + e, bf16);
            }
    if (lt == 0)
        for (int x = 0; x < kBlock; ++x) {
            if (head_lane(x, head))
                fold(sg, x, bf16);
            else if (tail_lane(x, tail))
                fold(sg, tail_elem(x, head + nv * ve), bf16);
        }
}

// Replay of tile lt of a copy segment, lane by lane, with the kernels' own
// index functions.
template <int U>
void replay_copy_tile(const rr::CopyBatch &b, int s, int64_t total, int64_t lt, const rr::CopySeg &sg,
                      const rr::CopySplit &sp, bool shift_mode)
{
    using namespace rr;
    constexpr int64_t tv = tile_vecs<U>();
    const int64_t nv = sp.nv;
    if (seg_tiles(b, s, total) != body_tiles(nv, tv))
        violation("copy segment tile count differs from its body", uintptr_t(sg.dst), seg_tiles(b, s, total));
    const unsigned char *base = sg.src + sp.head - (shift_mode ? sg.shift : 0);  // aligned words read
    const bool full = full_tile(lt, tv, nv);
    if (g_check_only && !shift_mode) {
        if (nv > 0) {
            // every lane stores vector i of its tile's body range (as below)
            const TileBody tb = stored_body<U>(lt, nv, uintptr_t(sg.dst));
            for (int x = 0; x < kBlock; ++x)
                for (int u = 0; u < U; ++u) {
                    const int64_t v = vec_index<U>(lt, x, u), i = vec_index<U>(0, x, u);
                    if (v < nv && (tb.first + i != v || i >= tb.count))
                        violation("copy store outside its tile's buffer range", uintptr_t(sg.dst), i);
                }
            const int64_t off = sp.head + tb.first * 16, len = tb.count * 16;
            if (!inside(uintptr_t(sg.src) + uintptr_t(off), len, false))
                violation("copy read", uintptr_t(sg.src) + uintptr_t(off), len);
            if (!inside(uintptr_t(sg.dst) + uintptr_t(off), len, true))
                violation("copy write", uintptr_t(sg.dst) + uintptr_t(off), len);
        }
    } else if (full || nv > 0)
        for (int x = 0; x < kBlock; ++x)
            for (int u = 0; u < U; ++u) {
                const int64_t v = vec_index<U>(lt, x, u);
                if (shift_mode) {
                    if (loads_own_word(full, v, nv, true) && !touches(uintptr_t(base + v * 16), 16))
                        violation("realigned word outside every buffer", uintptr_t(base + v * 16), 16);
                    if (loads_next_word(full, v, nv, true, wave_end(x)) && !touches(uintptr_t(base + (v + 1) * 16), 16))
                        violation("realigned word outside every buffer", uintptr_t(base + (v + 1) * 16), 16);
                }
                if (full || v < nv) {
                    // the kernel stores vector i of the tile's body range
                    const TileBody tb = tile_body(lt, tv, nv);
                    const int64_t i = vec_index<U>(0, x, u);
                    if (tb.first + i != v || i < 0 || i >= tb.count)
                        violation("copy store outside its tile's buffer range", uintptr_t(sg.dst), i);
                    for (int e = 0; e < 16; ++e)
                        copy_byte(sg.src, sg.dst, sp.head + (tb.first + i) * 16 + e);
                }
            }
    if (lt == 0)
        for (int x = 0; x < kBlock; ++x) {
            if (head_lane(x, sp.head))
                copy_byte(sg.src, sg.dst, x);
            else if (tail_lane(x, sp.tail))
                copy_byte(sg.src, sg.dst, tail_elem(x, sp.head + 16 * sp.nv));
        }
}

}  // namespace

namespace rr {

hipError_t launch_reduce(const RedBatch &b, int64_t total_tiles, bool shifted, hipStream_t)
{
    ++g_launches;
    const bool bf16 = b.bf16;
    const int64_t es = bf16 ? 2 : 4, ve = 16 / es;
    const LaunchShape sh = reduce_shape(b, total_tiles);
    ++g_forms[0][sh.form];
    if (sh.form == kFormOne && (b.nseg != 1 || b.seg[0].mode != (shifted ? kRedShifted : kRedAligned) ||
                                b.seg[0].k < 1 || b.seg[0].k > kMaxIn))
        violation("single-segment form for a segment it cannot run", uintptr_t(b.seg[0].out), b.seg[0].k);
    for (const auto &st : tiles_of(b, total_tiles, sh)) {
        const RedSeg &sg = b.seg[st.first];
        const int64_t lt = st.second;
        const bool shift_mode = sg.mode == kRedShifted;
        if (shift_mode != shifted)
            violation("reduction mode in the wrong kernel", uintptr_t(sg.out), sg.mode);
        if (sg.mode != kRedAligned && sg.mode != kRedShifted)
            violation("unknown reduction mode", uintptr_t(sg.out), sg.mode);
        if (sg.k < 1 || sg.k > kMaxIn) {
            violation("reduction with no kernel for its input count", uintptr_t(sg.out), sg.k);
            continue;
        }
        const uintptr_t o = uintptr_t(sg.out);
        if (!shift_mode) {
            bool aligned = o % 16 == 0;
            for (int k = 0; k < sg.k; ++k)
                aligned = aligned && uintptr_t(sg.in[k]) % 16 == 0;
            if (!aligned)
                violation("unaligned pointer in an aligned reduction", o, sg.n);
        }
        const RedSplit sp = red_split(sg.out, sg.n, es);
        const int64_t head = sp.head, nv = sp.nv, tail = sp.tail;
        // the split against its definition: head elements up to the output's
        // 16-byte boundary, whole output vectors, the remaining tail elements
        if (head != std::min<int64_t>(sg.n, int64_t((16 - o % 16) % 16) / es) || head + nv * ve + tail != sg.n ||
            tail < 0 || tail >= ve)
            violation("reduction split differs from its definition", o, sg.n);
        if (shift_mode)
            replay_red_tile<kShiftRedUnroll>(b, st.first, total_tiles, lt, sg, head, nv, tail, bf16);
        else
            replay_red_tile<kUnroll>(b, st.first, total_tiles, lt, sg, head, nv, tail, bf16);
    }
    return hipSuccess;
}

hipError_t launch_copy(const CopyBatch &b, int64_t total_tiles, bool shifted, hipStream_t)
{
    ++g_launches;
    const LaunchShape sh = copy_shape(b, total_tiles);
    ++g_forms[1][sh.form];
    if (sh.form == kFormOne)
        violation("single-segment form for a copy", 0, 0);
    if (b.long_tiles != 0 && b.long_tiles != 1)
        violation("copy batch with an unknown tiling", 0, b.long_tiles);
    if (b.nt_stores != 0 && b.nt_stores != 1)
        violation("copy batch with an unknown store policy", 0, b.nt_stores);
    if (b.long_tiles && !b.nt_stores)
        violation("long-call tiles without the long call's store policy", 0, 0);
    ++g_nt_copies[b.nt_stores != 0];
    ++g_long_copies[b.long_tiles != 0];
    g_shifted_copies += shifted ? 1 : 0;
    if (b.long_tiles && shifted)
        violation("long-call tiling in a launch with a realigned move", 0, 0);
    for (const auto &st : tiles_of(b, total_tiles, sh)) {
        const CopySeg &sg = b.seg[st.first];
        const int64_t lt = st.second;
        if (sg.mode == kCopyShifted && !shifted)
            violation("realigned copy segment in the aligned-only kernel", uintptr_t(sg.dst), sg.mode);
        if (sg.mode != kCopyAligned && sg.mode != kCopyShifted)
            violation("unknown copy mode", uintptr_t(sg.dst), sg.mode);
        const uintptr_t d = uintptr_t(sg.dst);
        const CopySplit sp = copy_split(sg.dst, sg.nbytes);
        // the split against its definition: head bytes up to the destination's
        // 16-byte boundary, whole 16-byte body vectors, the remaining tail
        if (sp.head != std::min<int64_t>(sg.nbytes, int64_t((16 - d % 16) % 16)) ||
            sp.head + 16 * sp.nv + sp.tail != sg.nbytes || sp.tail < 0 || sp.tail > 15)
            violation("copy split differs from its definition", d, sg.nbytes);
        const unsigned char *bsrc = sg.src + sp.head;
        const bool shift_mode = sg.mode == kCopyShifted;
        if ((d + uintptr_t(sp.head)) % 16 && sp.nv > 0)
            violation("copy body destination not 16-byte aligned", d, sp.head);
        if (!shift_mode && uintptr_t(bsrc) % 16 && sp.nv > 0)
            violation("aligned copy body with an unaligned source", uintptr_t(bsrc), 16);
        if (shift_mode && (sg.shift < 1 || sg.shift > 15 || int64_t(uintptr_t(bsrc) % 16) != sg.shift))
            violation("realigned copy with a wrong source shift", uintptr_t(bsrc), sg.shift);
        if (shift_mode)
            replay_copy_tile<kShiftUnroll>(b, st.first, total_tiles, lt, sg, sp, true);
        else if (b.long_tiles)
            replay_copy_tile<kCopyUnrollLong>(b, st.first, total_tiles, lt, sg, sp, false);
        else
            replay_copy_tile<kCopyUnroll>(b, st.first, total_tiles, lt, sg, sp, false);
    }
    return hipSuccess;
}

}  // namespace rr

extern "C" {
// 1: registered ranges hold no memory; accesses are checked, never performed
void sim_set_check_only(int on) { g_check_only = on != 0; }
void sim_reset(void)
{
    g_bufs.clear();
    g_violations = 0;
    g_launches = 0;
    memset(g_forms, 0, sizeof g_forms);
    memset(g_long_copies, 0, sizeof g_long_copies);
    g_shifted_copies = 0;
    memset(g_nt_copies, 0, sizeof g_nt_copies);
    g_msg[0] = '\0';
}
void sim_register(const void *p, int64_t bytes, int writable)
{
    g_bufs.push_back(Buf{uintptr_t(p), uintptr_t(p) + uintptr_t(bytes), writable != 0});
}
long sim_violations(void) { return g_violations; }
long sim_launches(void) { return g_launches; }
// launches since the last reset in launch form `form` (0 table, 1 uniform,
// 2 single segment) of the reduction (copy == 0) or copy (copy == 1) kernels
long sim_form_launches(int copy, int form) { return g_forms[copy != 0][form]; }
const char *sim_message(void) { return g_msg; }
// copy launches since the last reset with the default (0) or long-call (1) tiling
long sim_copy_launches(int long_tiles) { return g_long_copies[long_tiles != 0]; }
// copy launches since the last reset in the mixed-mode (realigning) kernels
long sim_shifted_copy_launches(void) { return g_shifted_copies; }
// copy launches since the last reset with agent-scope (0) or non-temporal (1) stores
long sim_nt_copy_launches(int nt) { return g_nt_copies[nt != 0]; }
}
