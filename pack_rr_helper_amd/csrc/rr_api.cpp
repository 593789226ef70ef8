// rr_api.cpp -- the C ABI declared in include/rr.h: argument validation,
// relay geometry, and the translation of each relay step into the segment
// tables the gfx950 kernels execute (rr_kernels.hip).
//
// Everything here runs on the host and returns before any HIP call when the
// arguments are rejected.  Nothing is allocated: segment tables travel in the
// kernel arguments.
#include "rr.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "rr_internal.h"

namespace {

thread_local char g_err[512];

rr_status fail(rr_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

rr_status ok()
{
    g_err[0] = '\0';
    return RR_OK;
}

int64_t elem_size(int dtype) { return dtype == RR_F32 ? 4 : 2; }

int64_t align_down_128(int64_t x) { return (x / 128) * 128; }

uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }

// ---------------------------------------------------------------------------
// Plans: between rr_plan_begin and rr_plan_end the launchers of this thread
// append their batches to the caller's plan buffer instead of launching them.
// ---------------------------------------------------------------------------

thread_local rr::PlanHeader *g_plan = nullptr;

rr::PlanRec *plan_records(rr::PlanHeader *h)
{
    return reinterpret_cast<rr::PlanRec *>(reinterpret_cast<char *>(h) + sizeof(rr::PlanHeader));
}

// A batch goes to the plan being recorded, or to the GPU.  A full plan is
// marked broken and the call reports it (hipErrorOutOfMemory stands for "no
// record left" inside this file).
hipError_t emit_reduce(const rr::RedBatch &b, int64_t tiles, bool shifted, hipStream_t st)
{
    if (!g_plan)
        return rr::launch_reduce(b, tiles, shifted, st);
    if (g_plan->count >= g_plan->capacity) {
        g_plan->broken = 1;
        return hipErrorOutOfMemory;
    }
    rr::PlanRec &r = plan_records(g_plan)[g_plan->count++];
    r.kind = rr::kPlanReduce;
    r.shifted = shifted ? 1 : 0;
    r.tiles = tiles;
    r.red.nseg = b.nseg;
    r.red.bf16 = b.bf16;
    for (int i = 0; i < b.nseg; ++i) {
        r.red.tile0[i] = b.tile0[i];
        r.red.seg[i] = b.seg[i];
    }
    return hipSuccess;
}

hipError_t emit_copy(const rr::CopyBatch &b, int64_t tiles, bool shifted, hipStream_t st)
{
    if (!g_plan)
        return rr::launch_copy(b, tiles, shifted, st);
    if (g_plan->count >= g_plan->capacity) {
        g_plan->broken = 1;
        return hipErrorOutOfMemory;
    }
    rr::PlanRec &r = plan_records(g_plan)[g_plan->count++];
    r.kind = rr::kPlanCopy;
    r.shifted = shifted ? 1 : 0;
    r.tiles = tiles;
    r.copy.nseg = b.nseg;
    r.copy.long_tiles = b.long_tiles;
    r.copy.nt_stores = b.nt_stores;
    for (int i = 0; i < b.nseg; ++i) {
        r.copy.tile0[i] = b.tile0[i];
        r.copy.seg[i] = b.seg[i];
    }
    return hipSuccess;
}

rr_status launch_failed(hipError_t e)
{
    if (e == hipErrorOutOfMemory && g_plan)
        return fail(RR_EINVAL, "the plan buffer holds %d launches and this call needs more; the plan is "
                    "unusable (record it again into a larger buffer)", g_plan->capacity);
    return fail(RR_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Geometry (pull request summary sections 1, 4 and 6; zero-chunk fallback)
// ---------------------------------------------------------------------------

rr_status compute_geometry(const rr_relay *r, int coll, int dtype, rr_geom *g)
{
    if (!r)
        return fail(RR_EINVAL, "relay descriptor is null");
    memset(g, 0, sizeof *g);
    const int A = r->A, H = r->H;
    if (A != 2 && A != 4)
        return fail(RR_EINVAL, "A=%d: the relay supports 2 or 4 active ranks per group", A);
    if (H < 1)
        return fail(RR_EINVAL, "H=%d: a relay group needs at least one helper", H);
    if (r->count < 0)
        return fail(RR_EINVAL, "count=%lld is negative", (long long)r->count);
    if (r->count > RR_MAX_COUNT)
        return fail(RR_EINVAL, "count=%lld exceeds RR_MAX_COUNT (2^48 elements)", (long long)r->count);
    if (coll < RR_ALLREDUCE || coll > RR_ALLTOALL)
        return fail(RR_EINVAL, "unknown collective %d", coll);
    if (dtype != RR_F32 && dtype != RR_BF16)
        return fail(RR_EINVAL, "unknown dtype %d", dtype);

    const int64_t es = elem_size(dtype);
    int64_t chunk = 0;
    if (A == 2) {
        if (r->numChunks < H + 2)
            return fail(RR_EINVAL,
                        "numChunks=%d: the two-group A=2 schedule needs at least H+2=%d chunks",
                        r->numChunks, H + 2);
        chunk = align_down_128(r->count / r->numChunks);
    } else if (coll == RR_ALLTOALL) {
        if (r->numChunks < H + 1)
            return fail(RR_EINVAL, "numChunks=%d: all-to-all needs at least H+1=%d chunks",
                        r->numChunks, H + 1);
        chunk = align_down_128(r->count / r->numChunks);
    } else {
        if (r->permille <= 0 || r->permille > 1000)
            return fail(RR_EINVAL, "permille=%d must be in (0, 1000]", r->permille);
        const bool under_floor = coll == RR_ALLREDUCE && r->count * es < (int64_t(2) << 20);
        chunk = under_floor ? 0 : align_down_128(r->count * r->permille / (int64_t(1000) * H));
        if (coll == RR_REDUCE_SCATTER && int64_t(A) * A * chunk > 2 * r->count)
            return fail(RR_EINVAL,
                        "permille=%d: A*(A-1) input chunks plus A reduced chunks exceed the "
                        "2*recvCount helper contract",
                        r->permille);
    }

    g->chunk = chunk;
    g->pure_direct = chunk == 0;
    g->relay_total = int64_t(H) * chunk;
    g->direct_off = g->relay_total;
    g->direct_len = r->count - g->relay_total;
    if (A == 2) {
        if (chunk > 0) {
            g->dirA_off = int64_t(H) * chunk;
            g->dirA_len = chunk;
            g->dirB_off = int64_t(H + 1) * chunk;
            g->dirB_len = r->count - g->dirB_off;
        } else {
            g->dirA_off = 0;
            g->dirA_len = r->count / 2;
            g->dirB_off = g->dirA_len;
            g->dirB_len = r->count - g->dirA_len;
        }
        g->helper_elems = int64_t(A) * chunk;
    } else if (coll == RR_ALLTOALL) {
        g->helper_elems = int64_t(A) * (A - 1) * chunk;
    } else {
        g->dslice = g->direct_len / A;
        g->helper_elems = 2 * r->count;
    }
    return RR_OK;
}

// ---------------------------------------------------------------------------
// Byte ranges and aliasing
// ---------------------------------------------------------------------------

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range range_of(const void *p, int64_t off_elems, int64_t n_elems, int64_t es)
{
    const uintptr_t lo = addr(p) + uintptr_t(off_elems * es);
    return Range{lo, lo + uintptr_t(n_elems * es)};
}

bool overlap(Range a, Range b)
{
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool same(Range a, Range b) { return a.lo == b.lo && a.hi == b.hi; }

rr_status check_ptr(const void *p, int64_t es, const char *what, int idx)
{
    if (!p)
        return fail(RR_EINVAL, "%s[%d] is null", what, idx);
    if (addr(p) % uintptr_t(es))
        return fail(RR_EINVAL, "%s[%d]=%p is not aligned to the %lld-byte element", what, idx,
                    p, (long long)es);
    return RR_OK;
}

// ---------------------------------------------------------------------------
// Reduction items: one element-wise K-input sum with its own scale
// ---------------------------------------------------------------------------

struct RedItem {
    const void *in[rr::kMaxIn];
    int k;
    void *out;
    int64_t n;
    float scale;
    int job;  // the job of a batched call the item belongs to
};

// Output ranges sorted by start, after checking that no two overlap (one
// sort, then neighbours).  Empty ranges are left out: they overlap nothing.
struct OutRange {
    Range r;
    int item;
};

// Sorts `outs` by start; returns a position i whose range overlaps the one
// before it, or 0 when all are disjoint.
size_t sort_outputs(std::vector<OutRange> &outs)
{
    std::sort(outs.begin(), outs.end(), [](const OutRange &a, const OutRange &b) { return a.r.lo < b.r.lo; });
    for (size_t i = 1; i < outs.size(); ++i)
        if (outs[i].r.lo < outs[i - 1].r.hi)
            return i;
    return 0;
}

// Calls f(output) for every output in the sorted, disjoint list that overlaps x.
template <typename F>
bool each_overlapping(const std::vector<OutRange> &outs, Range x, F f)
{
    // disjoint and sorted by start, so also sorted by end: the first output
    // ending after x.lo is the first that can overlap x
    auto it = std::upper_bound(outs.begin(), outs.end(), x.lo,
                               [](uintptr_t lo, const OutRange &o) { return lo < o.r.hi; });
    for (; it != outs.end() && it->r.lo < x.hi; ++it)
        if (!f(*it))
            return false;
    return true;
}

// An element-wise output is safe when its range equals an input's range
// exactly (each lane reads its inputs before writing the same elements) or is
// disjoint from it; everything else is a forbidden alias.  Outputs must also
// be disjoint from every other item's inputs and outputs, since all items of
// one call run concurrently.  On RR_EALIAS, culprit[] holds the indices of
// the two items in conflict (the same index twice for an item whose output
// overlaps its own input).
rr_status check_items(const std::vector<RedItem> &items, int64_t es, size_t culprit[2])
{
    std::vector<OutRange> outs;
    outs.reserve(items.size());
    for (size_t i = 0; i < items.size(); ++i) {
        const Range o = range_of(items[i].out, 0, items[i].n, es);
        if (!o.empty())
            outs.push_back(OutRange{o, int(i)});
    }
    if (const size_t i = sort_outputs(outs)) {
        culprit[0] = size_t(outs[i - 1].item);
        culprit[1] = size_t(outs[i].item);
        return fail(RR_EALIAS, "two output ranges overlap");
    }
    for (size_t j = 0; j < items.size(); ++j)
        for (int k = 0; k < items[j].k; ++k) {
            const Range x = range_of(items[j].in[k], 0, items[j].n, es);
            if (x.empty())
                continue;
            const bool ok = each_overlapping(outs, x, [&](const OutRange &o) {
                culprit[0] = j;
                culprit[1] = size_t(o.item);
                return o.item == int(j) && same(o.r, x);
            });
            if (!ok)
                return fail(RR_EALIAS,
                            "an output range overlaps an input range other than an exact in-place alias");
        }
    return RR_OK;
}

// Prefixes the current message with the job (or the two jobs) at fault.
rr_status jobs_error(int a, int b, rr_status st)
{
    char tmp[sizeof g_err];
    if (a == b)
        snprintf(tmp, sizeof tmp, "job %d: %.480s", a, g_err);
    else
        snprintf(tmp, sizeof tmp, "jobs %d and %d: %.470s", std::min(a, b), std::max(a, b), g_err);
    memcpy(g_err, tmp, sizeof g_err);
    return st;
}

class RedLauncher {
public:
    // Only the counts are reset: table entries are written before they are
    // read, and clearing the full-capacity tables costs host time per call.
    RedLauncher(bool bf16, hipStream_t st) : bf16_(bf16), st_(st)
    {
        for (int i = 0; i < 2; ++i) {
            q_[i].b.nseg = 0;
            q_[i].b.bf16 = bf16;
            q_[i].tiles = 0;
            q_[i].shifted = i == 1;
        }
    }

    // One segment per item (tile 0 also computes its element-wise head and
    // tail): in the aligned kernels' queue when every pointer is 16-byte
    // aligned, in the realigning kernels' queue otherwise.
    void add(const RedItem &it, int64_t es)
    {
        if (it.n <= 0)
            return;
        bool aligned = addr(it.out) % 16 == 0;
        for (int k = 0; k < it.k; ++k)
            aligned = aligned && addr(it.in[k]) % 16 == 0;
        piece(it, aligned ? rr::kRedAligned : rr::kRedShifted, es);
    }

    hipError_t finish()
    {
        flush(q_[0]);
        flush(q_[1]);
        return err_;
    }

private:
    struct Queue {
        rr::RedBatch b;
        int64_t tiles;
        bool shifted;
    };

    void piece(const RedItem &it, int32_t mode, int64_t es)
    {
        Queue &q = q_[mode == rr::kRedShifted ? 1 : 0];
        const int64_t tv = rr::red_tile_vecs(mode), ve = 16 / es;
        int64_t off = 0, n = it.n;
        while (n > 0) {
            if (q.b.nseg == rr::kMaxRedSegs || q.tiles >= rr::kMaxTilesPerLaunch)
                flush(q);
            rr::RedSeg s{};
            for (int k = 0; k < it.k; ++k)
                s.in[k] = static_cast<const char *>(it.in[k]) + off * es;
            s.out = static_cast<char *>(it.out) + off * es;
            const rr::RedSplit sp = rr::red_split(s.out, n, es);
            int64_t tiles = rr::body_tiles(sp.nv, tv);
            int64_t take = n;
            const int64_t room = rr::kMaxTilesPerLaunch - q.tiles;
            if (tiles > room) {
                // whole tiles of the body only: the rest starts on a 16-byte
                // output boundary with every input's shift unchanged
                tiles = room;
                take = sp.head + room * tv * ve;
            }
            s.k = it.k;
            s.mode = mode;
            s.scale = it.scale;
            s.n = take;
            q.b.tile0[q.b.nseg] = int32_t(q.tiles);
            q.b.seg[q.b.nseg++] = s;
            q.tiles += tiles;
            off += take;
            n -= take;
        }
    }

    void flush(Queue &q)
    {
        if (q.b.nseg == 0)
            return;
        const hipError_t e = emit_reduce(q.b, q.tiles, q.shifted, st_);
        if (e != hipSuccess && err_ == hipSuccess)
            err_ = e;
        q.b.nseg = 0;
        q.tiles = 0;
    }

    Queue q_[2];
    bool bf16_;
    hipStream_t st_;
    hipError_t err_ = hipSuccess;
};

// Checks and launches the items of one call.  In a batched call (`batch`)
// the message of an alias names the job, or the two jobs, it involves.
rr_status run_reduce(const std::vector<RedItem> &items, int dtype, void *stream, bool batch)
{
    const int64_t es = elem_size(dtype);
    size_t culprit[2];
    rr_status st = check_items(items, es, culprit);
    if (st != RR_OK)
        return batch ? jobs_error(items[culprit[0]].job, items[culprit[1]].job, st) : st;
    RedLauncher L(dtype == RR_BF16, static_cast<hipStream_t>(stream));
    for (const RedItem &it : items)
        L.add(it, es);
    const hipError_t e = L.finish();
    if (e != hipSuccess)
        return launch_failed(e);
    return ok();
}

float op_scale(int op, int A) { return op == RR_AVG ? 1.0f / float(A) : 1.0f; }

rr_status check_common(const rr_relay *r, int coll, int dtype, int op, rr_geom *g)
{
    rr_status st = compute_geometry(r, coll, dtype, g);
    if (st != RR_OK)
        return st;
    if (op != RR_SUM && op != RR_AVG)
        return fail(RR_EINVAL, "op=%d: the relay supports SUM and AVG only", op);
    return RR_OK;
}

rr_status check_array(const void *const *arr, int n, int64_t es, const char *what)
{
    if (!arr)
        return fail(RR_EINVAL, "%s pointer array is null", what);
    for (int i = 0; i < n; ++i) {
        rr_status st = check_ptr(arr[i], es, what, i);
        if (st != RR_OK)
            return st;
    }
    return RR_OK;
}

// ---------------------------------------------------------------------------
// Per-job collectors: validate one job and append its reduction items
// ---------------------------------------------------------------------------

rr_status collect_helper(const rr_relay *relay, int coll, int dtype, int op, int helper,
                         const void *const *slots, int nSlots, void *out, std::vector<RedItem> &items)
{
    rr_geom g;
    rr_status st = check_common(relay, coll, dtype, op, &g);
    if (st != RR_OK)
        return st;
    if (coll == RR_REDUCE_SCATTER)
        return fail(RR_EINVAL,
                    relay->A == 2
                        ? "A=2 reduce-scatter helpers are passthrough: slot 0 and slot 1 feed "
                          "different outputs and are not summable"
                        : "the A=4 reduce-scatter helper reduces with rr_rs_multi_reduce pass 1");
    if (coll == RR_ALLTOALL)
        return fail(RR_EINVAL, "all-to-all performs no reduction");
    const int A = relay->A;
    if (nSlots != A)
        return fail(RR_EINVAL, "nSlots=%d: the allreduce helper sums exactly A=%d slots", nSlots, A);
    if (helper < 0 || helper >= relay->H)
        return fail(RR_EINVAL, "helper=%d outside [0, H=%d)", helper, relay->H);
    if (g.chunk == 0)
        return RR_OK;  // pure direct: the helper has nothing to reduce
    const int64_t es = elem_size(dtype);
    if ((st = check_array(slots, nSlots, es, "slots")) != RR_OK)
        return st;
    if ((st = check_ptr(out, es, "out", 0)) != RR_OK)
        return st;
    RedItem it{};
    for (int a = 0; a < A; ++a)
        it.in[a] = slots[a];
    it.k = A;
    it.out = out;
    it.n = g.chunk;
    it.scale = op_scale(op, A);
    items.push_back(it);
    return RR_OK;
}

rr_status collect_active(const rr_relay *relay, int coll, int dtype, int op, int activeIdx,
                         const void *const *in, int nIn, void *out, std::vector<RedItem> &items)
{
    rr_geom g;
    rr_status st = check_common(relay, coll, dtype, op, &g);
    if (st != RR_OK)
        return st;
    const int A = relay->A;
    if (coll == RR_ALLTOALL)
        return fail(RR_EINVAL, "all-to-all performs no reduction");
    if (coll == RR_REDUCE_SCATTER && A != 2)
        return fail(RR_EINVAL, "the A=4 reduce-scatter owner reduces with rr_rs_multi_reduce pass 2");
    if (nIn != A)
        return fail(RR_EINVAL, "nIn=%d: the active epilogue sums one input per active (A=%d)", nIn, A);
    if (activeIdx < 0 || activeIdx >= A)
        return fail(RR_EINVAL, "activeIdx=%d outside [0, A=%d)", activeIdx, A);
    const int64_t es = elem_size(dtype);
    if ((st = check_array(in, nIn, es, "in")) != RR_OK)
        return st;
    if ((st = check_ptr(out, es, "out", 0)) != RR_OK)
        return st;

    int64_t lo = 0, n = relay->count;  // reduce-scatter: the whole block
    if (coll == RR_ALLREDUCE) {
        lo = g.direct_off;
        n = g.direct_len;
        if (A > 2) {
            lo = g.direct_off + int64_t(activeIdx) * g.dslice;
            n = activeIdx == A - 1 ? g.direct_off + g.direct_len - lo : g.dslice;
        }
    }
    if (n == 0)
        return RR_OK;
    RedItem it{};
    for (int s = 0; s < A; ++s)
        it.in[s] = static_cast<const char *>(in[s]) + lo * es;
    it.k = A;
    it.out = static_cast<char *>(out) + lo * es;
    it.n = n;
    it.scale = op_scale(op, A);
    items.push_back(it);
    return RR_OK;
}

rr_status collect_rs(const rr_relay *relay, int dtype, int op, int pass, int idx,
                     const void *const *in, int nIn, void *out, std::vector<RedItem> &items)
{
    rr_geom g;
    rr_status st = check_common(relay, RR_REDUCE_SCATTER, dtype, op, &g);
    if (st != RR_OK)
        return st;
    const int A = relay->A, H = relay->H;
    if (A != 4)
        return fail(RR_EINVAL,
                    "the two multi-input passes belong to the A=4 reduce-scatter; A=2 helpers "
                    "are passthrough and the owner uses rr_active_add_scale");
    const int64_t es = elem_size(dtype);
    const int64_t c = g.chunk;
    if (pass == 1) {
        if (idx < 0 || idx >= H)
            return fail(RR_EINVAL, "pass 1: helper idx=%d outside [0, H=%d)", idx, H);
        if (nIn != 1)
            return fail(RR_EINVAL, "pass 1 takes the helper scratch as its single input (nIn=%d)", nIn);
        if (c == 0)
            return RR_OK;
        if ((st = check_array(in, 1, es, "in")) != RR_OK)
            return st;
        if ((st = check_ptr(out, es, "out", 0)) != RR_OK)
            return st;
        if (overlap(range_of(out, 0, A * c, es), range_of(in[0], 0, int64_t(A) * (A - 1) * c, es)))
            return fail(RR_EALIAS, "pass 1 output overlaps the A*(A-1) input chunks of the scratch");
        for (int o = 0; o < A; ++o) {
            RedItem it{};
            for (int j = 0; j < A - 1; ++j)
                it.in[j] = static_cast<const char *>(in[0]) + (int64_t(o) * (A - 1) + j) * c * es;
            it.k = A - 1;
            it.out = static_cast<char *>(out) + int64_t(o) * c * es;
            it.n = c;
            it.scale = 1.0f;  // a partial sum: the owner applies the op scale once
            items.push_back(it);
        }
        return RR_OK;
    }
    if (pass != 2)
        return fail(RR_EINVAL, "pass=%d: the reduction has two passes (1 helper, 2 owner)", pass);
    if (idx < 0 || idx >= A)
        return fail(RR_EINVAL, "pass 2: owner idx=%d outside [0, A=%d)", idx, A);
    if (nIn != A + H)
        return fail(RR_EINVAL, "pass 2 takes A blocks and H reduced chunks (nIn=%d, expected %d)",
                    nIn, A + H);
    if ((st = check_array(in, A, es, "in")) != RR_OK)
        return st;
    if (c > 0 && (st = check_array(in + A, H, es, "in[A+h]")) != RR_OK)
        return st;
    if ((st = check_ptr(out, es, "out", 0)) != RR_OK)
        return st;
    // The direct region goes out in pieces of one offload chunk, so that with
    // the offload slices every segment of the owner's pass spans the same
    // tiles and the pass launches on the uniform grid (500 permille: the
    // direct region is exactly H chunks).  Its A-input pieces come first:
    // workgroups are dispatched in segment order, and the heavier tiles
    // started first leave the lighter ones to fill the launch's tail.
    const int64_t piece = c > 0 ? c : g.direct_len;
    for (int64_t lo = 0; lo < g.direct_len; lo += piece) {
        RedItem it{};
        for (int s = 0; s < A; ++s)
            it.in[s] = static_cast<const char *>(in[s]) + (g.direct_off + lo) * es;
        it.k = A;
        it.out = static_cast<char *>(out) + (g.direct_off + lo) * es;
        it.n = std::min(piece, g.direct_len - lo);
        it.scale = op_scale(op, A);
        items.push_back(it);
    }
    for (int h = 0; h < H && c > 0; ++h) {
        RedItem it{};
        it.in[0] = static_cast<const char *>(in[idx]) + int64_t(h) * c * es;
        it.in[1] = in[A + h];
        it.k = 2;
        it.out = static_cast<char *>(out) + int64_t(h) * c * es;
        it.n = c;
        it.scale = op_scale(op, A);
        items.push_back(it);
    }
    return RR_OK;
}

// ---------------------------------------------------------------------------
// Copy moves (all-to-all pack / unpack)
// ---------------------------------------------------------------------------

struct Move {
    const void *src;
    void *dst;
    int64_t nbytes;
    int job;  // the job of a batched call the move belongs to
};

// Every destination range is written by one move only and is read by none.
// On RR_EALIAS, culprit[] holds the two moves in conflict.
rr_status check_moves(const std::vector<Move> &mv, size_t culprit[2])
{
    std::vector<OutRange> dsts;
    dsts.reserve(mv.size());
    for (size_t i = 0; i < mv.size(); ++i) {
        const Range d{addr(mv[i].dst), addr(mv[i].dst) + uintptr_t(mv[i].nbytes)};
        if (!d.empty())
            dsts.push_back(OutRange{d, int(i)});
    }
    if (const size_t i = sort_outputs(dsts)) {
        culprit[0] = size_t(dsts[i - 1].item);
        culprit[1] = size_t(dsts[i].item);
        return fail(RR_EALIAS, "two destination chunks overlap");
    }
    for (size_t i = 0; i < mv.size(); ++i) {
        const Range src{addr(mv[i].src), addr(mv[i].src) + uintptr_t(mv[i].nbytes)};
        if (!src.empty() && !each_overlapping(dsts, src, [&](const OutRange &o) {
                culprit[0] = i;
                culprit[1] = size_t(o.item);
                return false;
            }))
            return fail(RR_EALIAS, "a destination chunk overlaps a source chunk");
    }
    return RR_OK;
}

class CopyLauncher {
public:
    // total: the bytes the call moves; aligned: all of them in aligned moves.
    // A call of at least kCopyLongBytes takes the long-call tiles if it is
    // aligned; one of at least kCopyAgentMaxBytes (or a long one) stores
    // non-temporally.
    CopyLauncher(hipStream_t st, int64_t total, bool aligned) : st_(st)
    {
        const bool long_call = total >= rr::kCopyLongBytes;
        b_.nseg = 0;
        b_.long_tiles = long_call && aligned ? 1 : 0;
        b_.nt_stores = long_call || total >= rr::kCopyAgentMaxBytes ? 1 : 0;
        b_.pad = 0;
    }

    // One segment per move (tile 0 also copies its head and tail bytes), all
    // in one batch: aligned when source and destination agree modulo 16
    // bytes, realigned otherwise.  A batch with a realigned move runs in the
    // mixed-mode kernels, one without in the aligned-only kernels.
    void add(const void *src, void *dst, int64_t nbytes)
    {
        if (nbytes <= 0)
            return;
        const unsigned char *s = static_cast<const unsigned char *>(src);
        unsigned char *d = static_cast<unsigned char *>(dst);
        if (addr(s) % 16 == addr(d) % 16) {
            piece(s, d, nbytes, rr::kCopyAligned, 0);
        } else {
            const int64_t head = rr::copy_split(d, nbytes).head;
            piece(s, d, nbytes, rr::kCopyShifted, int32_t(addr(s + head) % 16));
        }
    }

    hipError_t finish()
    {
        flush();
        return err_;
    }

private:
    void piece(const unsigned char *src, unsigned char *dst, int64_t nbytes, int32_t mode,
               int32_t shift)
    {
        const int64_t tv = rr::copy_tile_vecs(mode, b_.long_tiles != 0);
        while (nbytes > 0) {
            if (b_.nseg == rr::kMaxCopySegs || tiles_ >= rr::kMaxTilesPerLaunch)
                flush();
            const rr::CopySplit sp = rr::copy_split(dst, nbytes);
            int64_t tiles = rr::body_tiles(sp.nv, tv);
            int64_t take = nbytes;
            const int64_t room = rr::kMaxTilesPerLaunch - tiles_;
            if (tiles > room) {
                // whole tiles of the body only: the rest starts on a 16-byte
                // destination boundary with the same source shift
                tiles = room;
                take = sp.head + room * tv * 16;
            }
            rr::CopySeg s{};
            s.src = src;
            s.dst = dst;
            s.nbytes = take;
            s.mode = mode;
            s.shift = shift;
            b_.tile0[b_.nseg] = int32_t(tiles_);
            b_.seg[b_.nseg++] = s;
            tiles_ += tiles;
            shifted_ = shifted_ || mode == rr::kCopyShifted;
            src += take;
            dst += take;
            nbytes -= take;
        }
    }

    void flush()
    {
        if (b_.nseg == 0)
            return;
        const hipError_t e = emit_copy(b_, tiles_, shifted_, st_);
        if (e != hipSuccess && err_ == hipSuccess)
            err_ = e;
        b_.nseg = 0;
        tiles_ = 0;
        shifted_ = false;
    }

    rr::CopyBatch b_;
    int64_t tiles_ = 0;
    bool shifted_ = false;
    hipStream_t st_;
    hipError_t err_ = hipSuccess;
};

// Checks and launches the moves of one call (aliases in a batched call are
// named as in run_reduce).
rr_status run_copy(const std::vector<Move> &mv, void *stream, bool batch)
{
    size_t culprit[2];
    rr_status st = check_moves(mv, culprit);
    if (st != RR_OK)
        return batch ? jobs_error(mv[culprit[0]].job, mv[culprit[1]].job, st) : st;
    // Long-call tiles only when every move is aligned: a realigned move keeps
    // its own tile size, and moves of one size with unequal tiles would leave
    // the uniform launch form for the table form.
    int64_t total = 0;
    bool aligned = true;
    for (const Move &m : mv) {
        total += m.nbytes;
        aligned = aligned && (m.nbytes <= 0 || addr(m.src) % 16 == addr(m.dst) % 16);
    }
    CopyLauncher L(static_cast<hipStream_t>(stream), total, aligned);
    for (const Move &m : mv)
        L.add(m.src, m.dst, m.nbytes);
    const hipError_t e = L.finish();
    if (e != hipSuccess)
        return launch_failed(e);
    return ok();
}

// Validates one pack (unpack == false) or unpack job of helper slice `helper`
// and appends its A*(A-1) chunk moves: for destination d and the j-th source
// s_j != d, (segment d of source s_j at slice helper) <-> (chunk j of the
// per-destination buffer of d).  `ins` are the job's read buffers (sources or
// per-destination receive buffers), `outs` its written buffers.
rr_status collect_a2a(const rr_relay *relay, int dtype, int helper, const void *const *ins,
                      void *const *outs, bool unpack, std::vector<Move> &mv)
{
    rr_geom g;
    rr_status st = compute_geometry(relay, RR_ALLTOALL, dtype, &g);
    if (st != RR_OK)
        return st;
    if (helper < 0 || helper >= relay->H)
        return fail(RR_EINVAL, "helper=%d outside [0, H=%d)", helper, relay->H);
    if (g.chunk == 0)
        return RR_OK;
    const int A = relay->A;
    const int64_t es = elem_size(dtype), seg = relay->count, c = g.chunk;
    const int64_t full = int64_t(A) * seg, packed = int64_t(A - 1) * c;
    const char *in_name = unpack ? "recv" : "src";
    const char *out_name = unpack ? "out" : "dst";
    if ((st = check_array(ins, A, es, in_name)) != RR_OK)
        return st;
    if ((st = check_array(const_cast<const void *const *>(outs), A, es, out_name)) != RR_OK)
        return st;
    const int64_t in_len = unpack ? packed : full, out_len = unpack ? full : packed;
    // no written buffer may overlap a read buffer (nor another written one)
    for (int d = 0; d < A; ++d) {
        const Range ro = range_of(outs[d], 0, out_len, es);
        for (int s = 0; s < A; ++s)
            if (overlap(ro, range_of(ins[s], 0, in_len, es)))
                return fail(RR_EALIAS, "all-to-all output overlaps an input: %s[%d] overlaps %s[%d]", out_name,
                            d, in_name, s);
        for (int e = 0; e < d; ++e)
            if (overlap(ro, range_of(outs[e], 0, out_len, es)))
                return fail(RR_EALIAS, "%s[%d] overlaps %s[%d]", out_name, d, out_name, e);
    }
    for (int d = 0; d < A; ++d) {
        int j = 0;
        for (int s = 0; s < A; ++s) {
            if (s == d)
                continue;
            const int64_t strided = (int64_t(d) * seg + int64_t(helper) * c) * es;
            const int64_t strided_out = (int64_t(s) * seg + int64_t(helper) * c) * es;
            const int64_t contiguous = int64_t(j) * c * es;
            if (!unpack)
                mv.push_back(Move{static_cast<const char *>(ins[s]) + strided,
                                  static_cast<char *>(outs[d]) + contiguous, c * es, 0});
            else
                mv.push_back(Move{static_cast<const char *>(ins[d]) + contiguous,
                                  static_cast<char *>(outs[d]) + strided_out, c * es, 0});
            ++j;
        }
    }
    return RR_OK;
}

// Job j of a batched call: `collect` validates the job's arguments and
// appends its items (or moves), which are tagged with j so that an alias
// found later over the whole call can name the job(s) at fault.
template <typename Collect>
rr_status add_reduce_job(int j, std::vector<RedItem> &items, Collect collect)
{
    const size_t first = items.size();
    const rr_status st = collect();
    if (st != RR_OK)
        return jobs_error(j, j, st);
    for (size_t i = first; i < items.size(); ++i)
        items[i].job = j;
    return RR_OK;
}

template <typename Collect>
rr_status add_copy_job(int j, std::vector<Move> &mv, Collect collect)
{
    const size_t first = mv.size();
    const rr_status st = collect();
    if (st != RR_OK)
        return jobs_error(j, j, st);
    for (size_t i = first; i < mv.size(); ++i)
        mv[i].job = j;
    return RR_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Launch forms (declared in rr_internal.h)
// ---------------------------------------------------------------------------

namespace rr {

namespace {

// Uniform when every segment of the batch spans the same number of tiles.
template <typename Batch>
LaunchShape uniform_or_table(const Batch &b, int64_t total_tiles)
{
    const int n = b.nseg;
    const int64_t first = n > 1 ? int64_t(b.tile0[1]) - b.tile0[0] : total_tiles;
    for (int s = 1; s < n; ++s) {
        const int64_t end = s + 1 < n ? int64_t(b.tile0[s + 1]) : total_tiles;
        if (end - b.tile0[s] != first)
            return LaunchShape{kFormTable, total_tiles, 1};
    }
    return LaunchShape{kFormUniform, first, n};
}

}  // namespace

LaunchShape reduce_shape(const RedBatch &b, int64_t total_tiles)
{
    if (b.nseg == 1 && (b.seg[0].mode == kRedAligned || b.seg[0].mode == kRedShifted) && b.seg[0].k >= 1 &&
        b.seg[0].k <= kMaxIn)
        return LaunchShape{kFormOne, total_tiles, 1};
    return uniform_or_table(b, total_tiles);
}

LaunchShape copy_shape(const CopyBatch &b, int64_t total_tiles)
{
    return uniform_or_table(b, total_tiles);
}

}  // namespace rr

// ===========================================================================
// Exported entry points
// ===========================================================================

extern "C" {

int rr_abi_version(void) { return RR_ABI_VERSION; }

const char *rr_last_error(void) { return g_err; }

rr_status rr_geometry(const rr_relay *relay, int coll, int dtype, rr_geom *out)
{
    if (!out)
        return fail(RR_EINVAL, "output geometry pointer is null");
    rr_status st = compute_geometry(relay, coll, dtype, out);
    return st == RR_OK ? ok() : st;
}

int64_t rr_passthrough_helper_size(int64_t count_g, int32_t A, int32_t num_chunks)
{
    if (count_g < 0 || A < 1 || num_chunks < 1)
        return -1;
    // min(count_g, A * per_slot) without forming a product that can overflow:
    // A * per_slot > count_g exactly when per_slot > floor(count_g / A)
    const int64_t per_slot = align_down_128(count_g / num_chunks);
    return per_slot > count_g / A ? count_g : int64_t(A) * per_slot;
}

rr_status rr_helper_reduce(const rr_relay *relay, int coll, int dtype, int op, int helper,
                           const void *const *slots, int nSlots, void *out, void *stream)
{
    std::vector<RedItem> items;
    rr_status st = collect_helper(relay, coll, dtype, op, helper, slots, nSlots, out, items);
    return st != RR_OK ? st : run_reduce(items, dtype, stream, false);
}

rr_status rr_active_add_scale(const rr_relay *relay, int coll, int dtype, int op, int activeIdx,
                              const void *const *in, int nIn, void *out, void *stream)
{
    std::vector<RedItem> items;
    rr_status st = collect_active(relay, coll, dtype, op, activeIdx, in, nIn, out, items);
    return st != RR_OK ? st : run_reduce(items, dtype, stream, false);
}

rr_status rr_rs_multi_reduce(const rr_relay *relay, int dtype, int op, int pass, int idx,
                             const void *const *in, int nIn, void *out, void *stream)
{
    std::vector<RedItem> items;
    rr_status st = collect_rs(relay, dtype, op, pass, idx, in, nIn, out, items);
    return st != RR_OK ? st : run_reduce(items, dtype, stream, false);
}

rr_status rr_a2a_pack(const rr_relay *relay, int dtype, int helper, const void *const *src,
                      void *const *dst, void *stream)
{
    std::vector<Move> mv;
    rr_status st = collect_a2a(relay, dtype, helper, src, dst, false, mv);
    return st != RR_OK ? st : run_copy(mv, stream, false);
}

rr_status rr_a2a_unpack(const rr_relay *relay, int dtype, int helper, const void *const *recv,
                        void *const *out, void *stream)
{
    std::vector<Move> mv;
    rr_status st = collect_a2a(relay, dtype, helper, recv, out, true, mv);
    return st != RR_OK ? st : run_copy(mv, stream, false);
}

rr_status rr_helper_reduce_many(int coll, int dtype, int op, const rr_helper_job *jobs, int nJobs,
                                void *stream)
{
    if (nJobs < 0 || (nJobs > 0 && !jobs))
        return fail(RR_EINVAL, "job array is null or nJobs=%d is negative", nJobs);
    std::vector<RedItem> items;
    for (int j = 0; j < nJobs; ++j) {
        const rr_helper_job &b = jobs[j];
        rr_status st = add_reduce_job(j, items, [&] {
            return collect_helper(&b.relay, coll, dtype, op, b.helper, b.slots, b.nSlots, b.out, items);
        });
        if (st != RR_OK)
            return st;
    }
    return run_reduce(items, dtype, stream, true);
}

rr_status rr_active_add_scale_many(int coll, int dtype, int op, const rr_active_job *jobs, int nJobs,
                                   void *stream)
{
    if (nJobs < 0 || (nJobs > 0 && !jobs))
        return fail(RR_EINVAL, "job array is null or nJobs=%d is negative", nJobs);
    std::vector<RedItem> items;
    for (int j = 0; j < nJobs; ++j) {
        const rr_active_job &b = jobs[j];
        rr_status st = add_reduce_job(j, items, [&] {
            return collect_active(&b.relay, coll, dtype, op, b.activeIdx, b.in, b.nIn, b.out, items);
        });
        if (st != RR_OK)
            return st;
    }
    return run_reduce(items, dtype, stream, true);
}

rr_status rr_rs_multi_reduce_many(int dtype, int op, const rr_rs_job *jobs, int nJobs, void *stream)
{
    if (nJobs < 0 || (nJobs > 0 && !jobs))
        return fail(RR_EINVAL, "job array is null or nJobs=%d is negative", nJobs);
    std::vector<RedItem> items;
    for (int j = 0; j < nJobs; ++j) {
        const rr_rs_job &b = jobs[j];
        rr_status st = add_reduce_job(j, items, [&] {
            return collect_rs(&b.relay, dtype, op, b.pass, b.idx, b.in, b.nIn, b.out, items);
        });
        if (st != RR_OK)
            return st;
    }
    return run_reduce(items, dtype, stream, true);
}

rr_status rr_phase_reduce_many(int coll, int dtype, int op, const rr_helper_job *helperJobs, int nHelper,
                               const rr_active_job *activeJobs, int nActive, void *stream)
{
    if (nHelper < 0 || (nHelper > 0 && !helperJobs))
        return fail(RR_EINVAL, "helper job array is null or nHelper=%d is negative", nHelper);
    if (nActive < 0 || (nActive > 0 && !activeJobs))
        return fail(RR_EINVAL, "active job array is null or nActive=%d is negative", nActive);
    std::vector<RedItem> items;
    for (int j = 0; j < nHelper; ++j) {
        const rr_helper_job &b = helperJobs[j];
        rr_status st = add_reduce_job(j, items, [&] {
            return collect_helper(&b.relay, coll, dtype, op, b.helper, b.slots, b.nSlots, b.out, items);
        });
        if (st != RR_OK)
            return st;
    }
    for (int j = 0; j < nActive; ++j) {
        const rr_active_job &b = activeJobs[j];
        rr_status st = add_reduce_job(nHelper + j, items, [&] {
            return collect_active(&b.relay, coll, dtype, op, b.activeIdx, b.in, b.nIn, b.out, items);
        });
        if (st != RR_OK)
            return st;
    }
    return run_reduce(items, dtype, stream, true);
}

static rr_status a2a_many(int dtype, const rr_a2a_job *jobs, int nJobs, bool unpack, void *stream)
{
    if (nJobs < 0 || (nJobs > 0 && !jobs))
        return fail(RR_EINVAL, "job array is null or nJobs=%d is negative", nJobs);
    std::vector<Move> mv;
    for (int j = 0; j < nJobs; ++j) {
        const rr_a2a_job &b = jobs[j];
        rr_status st = add_copy_job(j, mv, [&] {
            return collect_a2a(&b.relay, dtype, b.helper, b.in, b.out, unpack, mv);
        });
        if (st != RR_OK)
            return st;
    }
    return run_copy(mv, stream, true);
}

rr_status rr_a2a_pack_many(int dtype, const rr_a2a_job *jobs, int nJobs, void *stream)
{
    return a2a_many(dtype, jobs, nJobs, false, stream);
}

rr_status rr_a2a_unpack_many(int dtype, const rr_a2a_job *jobs, int nJobs, void *stream)
{
    return a2a_many(dtype, jobs, nJobs, true, stream);
}

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------

size_t rr_plan_bytes(int32_t max_launches)
{
    if (max_launches < 1 || max_launches > RR_PLAN_MAX_LAUNCHES)
        return 0;
    return sizeof(rr::PlanHeader) + size_t(max_launches) * sizeof(rr::PlanRec);
}

rr_status rr_plan_begin(void *plan, size_t bytes)
{
    if (g_plan)
        return fail(RR_EINVAL, "this thread is already recording a plan");
    if (!plan)
        return fail(RR_EINVAL, "plan buffer is null");
    if (addr(plan) % alignof(rr::PlanRec) != 0)
        return fail(RR_EINVAL, "plan buffer is not %zu-byte aligned", alignof(rr::PlanRec));
    if (bytes < rr_plan_bytes(1))
        return fail(RR_EINVAL, "plan buffer of %zu bytes holds no launch (rr_plan_bytes(1) = %zu)", bytes,
                    rr_plan_bytes(1));
    auto *h = static_cast<rr::PlanHeader *>(plan);
    const size_t cap = (bytes - sizeof(rr::PlanHeader)) / sizeof(rr::PlanRec);
    h->magic = rr::kPlanMagic;
    h->capacity = int32_t(std::min<size_t>(cap, RR_PLAN_MAX_LAUNCHES));
    h->count = 0;
    h->recording = 1;
    h->broken = 0;
    g_plan = h;
    return ok();
}

rr_status rr_plan_end(int32_t *launches)
{
    if (!g_plan)
        return fail(RR_EINVAL, "this thread is not recording a plan");
    rr::PlanHeader *h = g_plan;
    g_plan = nullptr;
    h->recording = 0;
    if (launches)
        *launches = h->count;
    if (h->broken)
        return fail(RR_EINVAL, "a call ran out of plan records; the plan is unusable");
    return ok();
}

namespace {

// A finished, unbroken plan (RR_OK) or the reason it is not one.
rr_status check_plan(const void *plan, const char *what)
{
    if (!plan)
        return fail(RR_EINVAL, "%s is null", what);
    if (addr(plan) % alignof(rr::PlanRec) != 0)
        return fail(RR_EINVAL, "%s buffer is not %zu-byte aligned", what, alignof(rr::PlanRec));
    const auto *h = static_cast<const rr::PlanHeader *>(plan);
    if (h->magic != rr::kPlanMagic)
        return fail(RR_EINVAL, "%s is not a plan (record one with rr_plan_begin/rr_plan_end)", what);
    if (h->recording)
        return fail(RR_EINVAL, "%s is still being recorded", what);
    if (h->broken)
        return fail(RR_EINVAL, "%s ran out of records while it was recorded and is unusable", what);
    return RR_OK;
}

}  // namespace

rr_status rr_plan_append(void *plan, size_t bytes, const void *other)
{
    rr_status st = check_plan(plan, "plan");
    if (st == RR_OK)
        st = check_plan(other, "appended plan");
    if (st != RR_OK)
        return st;
    auto *h = static_cast<rr::PlanHeader *>(plan);
    const auto *o = static_cast<const rr::PlanHeader *>(other);
    const size_t room = bytes >= sizeof(rr::PlanHeader) ? (bytes - sizeof(rr::PlanHeader)) / sizeof(rr::PlanRec) : 0;
    const int64_t cap = std::min<int64_t>(std::min<int64_t>(h->capacity, int64_t(room)), RR_PLAN_MAX_LAUNCHES);
    if (int64_t(h->count) + o->count > cap)
        return fail(RR_EINVAL, "the plan holds %lld launches; it has %d and the appended plan %d",
                    (long long)cap, h->count, o->count);
    if (plan == other)
        return fail(RR_EINVAL, "a plan cannot be appended to itself");
    const auto *src = reinterpret_cast<const rr::PlanRec *>(reinterpret_cast<const char *>(o) +
                                                            sizeof(rr::PlanHeader));
    memcpy(plan_records(h) + h->count, src, size_t(o->count) * sizeof(rr::PlanRec));
    h->count += o->count;
    return ok();
}

rr_status rr_plan_launch(const void *plan, void *stream)
{
    const rr_status chk = check_plan(plan, "plan");
    if (chk != RR_OK)
        return chk;
    const auto *h = static_cast<const rr::PlanHeader *>(plan);
    const auto *rec = reinterpret_cast<const rr::PlanRec *>(reinterpret_cast<const char *>(h) +
                                                            sizeof(rr::PlanHeader));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < h->count; ++i) {
        const rr::PlanRec &r = rec[i];
        const hipError_t e = r.kind == rr::kPlanReduce ? rr::launch_reduce(r.red, r.tiles, r.shifted != 0, st)
                                                       : rr::launch_copy(r.copy, r.tiles, r.shifted != 0, st);
        if (e != hipSuccess)
            return fail(RR_EHIP, "kernel launch %d of the plan failed: %s", i, hipGetErrorString(e));
    }
    return ok();
}

}  // extern "C"
