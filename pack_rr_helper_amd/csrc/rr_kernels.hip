// rr_kernels.hip -- gfx950 (MI355X) streaming kernels for the sharded relay
// hot path: the K-input reduction (helper reduce-at-helper, active add+scale
// epilogue, the reduce-scatter multi-input passes) and the chunk copy engine
// (all-to-all strided gather/scatter).
//
// Both are HBM-bound element-wise operations (at most 0.4 flop per byte), so
// the design is about moving bytes: 16-byte global loads per lane, several of
// them in flight per input before any arithmetic, non-temporal hints on data
// that is touched exactly once, fp32 accumulation in registers, and one
// packed bf16 conversion (v_cvt_pk_bf16_f32, round-to-nearest-even) per pair
// of outputs.  No LDS allocation: nothing is reused, and where a source and
// its destination disagree modulo 16 bytes (strided all-to-all chunks, views
// at other element offsets) the data is realigned in registers
// (v_alignbyte), each lane taking its neighbouring source word from the next
// lane (a DPP wave shift) instead of loading it a second time or staging the
// tile.
//
// Tiling: one workgroup of 256 threads processes one tile of one segment.  A
// launch's segments live in the kernel arguments; how a workgroup finds its
// segment depends on the launch form the host chose (rr_internal.h): a single
// reduction segment arrives as plain arguments preloaded into scalar
// registers, equal segments are the rows of a 2-D grid, and otherwise a
// branch-free count over the table's tile offsets finds it.
#include "rr_internal.h"

namespace rr {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));


__device__ __forceinline__ u32x4 ld16(const u32x4 *p)
{
#if RR_LOAD_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

__device__ __forceinline__ void st16(u32x4 *p, u32x4 v)
{
#if RR_STORE_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// bf16 is the upper half of a binary32: widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values to a packed bf16 pair, round-to-nearest-even, lo in bits 0..15.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void *p, int64_t i)
{
    if constexpr (BF16)
        return __uint_as_float((unsigned)static_cast<const unsigned short *>(p)[i] << 16);
    else
        return static_cast<const float *>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void *p, int64_t i, float v)
{
    if constexpr (BF16)
        static_cast<__bf16 *>(p)[i] = (__bf16)v;
    else
        static_cast<float *>(p)[i] = v;
}

// A segment descriptor read as one vector, so it arrives in a single scalar
// load (s_load_dwordx16 / x8) before the workgroup branches on its fields;
// read field by field, the loads are issued one dependent round at a time.
template <typename Seg>
__device__ __forceinline__ Seg load_seg(const Seg &p)
{
    constexpr int kWords = (int)(sizeof(Seg) / 4);
    typedef int32_t words __attribute__((ext_vector_type(kWords), aligned(4)));
    return __builtin_bit_cast(Seg, *reinterpret_cast<const words *>(&p));
}

// This lane's index in its workgroup.
__device__ __forceinline__ int lane() { return (int)threadIdx.x; }

// ---------------------------------------------------------------------------
// Cross-lane realignment (the realigning reduction and copy)
// ---------------------------------------------------------------------------

// The 16-byte vector held by the next lane of this wave: a DPP move with the
// whole-wave left shift by one lane (wave_shl:1, lane i reads lane i + 1), a
// plain VALU operation with no LDS access and no wait counter.  Call it outside
// any lane-dependent branch: a lane reading from a lane that is switched off
// gets no data.  The last lane, which has no next lane, receives 0.
constexpr int kDppWaveShl1 = 0x130;

__device__ __forceinline__ u32x4 next_lane(u32x4 x)
{
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)x[j], kDppWaveShl1, 0xf, 0xf, false);
    return o;
}

// Bytes [4Q + r, 4Q + r + 16) of the 32 bytes a (low) and b (high).
template <int Q>
__device__ __forceinline__ u32x4 realign(u32x4 a, u32x4 b, unsigned r)
{
    const unsigned w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = __builtin_amdgcn_alignbyte(w[j + Q + 1], w[j + Q], r);
    return o;
}

// ---------------------------------------------------------------------------
// Reduction
// ---------------------------------------------------------------------------

// One 16-byte output vector from the K inputs' vectors at the same index.
template <bool BF16, int K>
__device__ __forceinline__ u32x4 fold_vec(const u32x4 (&x)[K], float scale)
{
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if constexpr (BF16) {
            float lo = bf16_lo(x[0][w]);
            float hi = bf16_hi(x[0][w]);
#pragma unroll
            for (int k = 1; k < K; ++k) {
                lo = lo + bf16_lo(x[k][w]);
                hi = hi + bf16_hi(x[k][w]);
            }
            r[w] = pack_bf16x2(lo * scale, hi * scale);
        } else {
            float a = __uint_as_float(x[0][w]);
#pragma unroll
            for (int k = 1; k < K; ++k)
                a = a + __uint_as_float(x[k][w]);
            r[w] = __float_as_uint(a * scale);
        }
    }
    return r;
}

// Element i of a segment through the same fp32 fold, one element at a time
// (heads and tails).
template <bool BF16, int K>
__device__ __forceinline__ void reduce_elem(const RedSeg &sg, int64_t i)
{
    float acc = load_elem<BF16>(sg.in[0], i);
#pragma unroll
    for (int k = 1; k < K; ++k)
        acc = acc + load_elem<BF16>(sg.in[k], i);
    store_elem<BF16>(sg.out, i, acc * sg.scale);
}

// Tile 0 of a segment also computes its element-wise edges: the first
// wave's lanes the head (elements [0, head)), the second wave's the tail
// (elements [tail0, tail0 + tail)); each is shorter than one 16-byte vector.
template <bool BF16, int K>
__device__ __forceinline__ void reduce_edges(const RedSeg &sg, int64_t head, int64_t tail0, int64_t tail)
{
    const int x = lane();
    if (head_lane(x, head))
        reduce_elem<BF16, K>(sg, x);
    else if (tail_lane(x, tail))
        reduce_elem<BF16, K>(sg, tail_elem(x, tail0));
}

// kRedAligned segment: every pointer 16-byte aligned.
template <bool BF16, int K>
__device__ __forceinline__ void reduce_vec(const RedSeg &sg, int64_t lt)
{
    constexpr int kVecElems = BF16 ? 8 : 4;
    const int64_t nv = sg.n / kVecElems;
    const float scale = sg.scale;

    const u32x4 *in[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        in[k] = static_cast<const u32x4 *>(sg.in[k]);
    u32x4 *out = static_cast<u32x4 *>(sg.out);

    if (full_tile(lt, tile_vecs<kUnroll>(), nv)) {
        // Full tile: issue every load before any arithmetic.
        u32x4 x[kUnroll][K];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int k = 0; k < K; ++k)
                x[u][k] = ld16(in[k] + vec_index<kUnroll>(lt, lane(), u));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            st16(out + vec_index<kUnroll>(lt, lane(), u), fold_vec<BF16, K>(x[u], scale));
    } else {
        // The segment's last, partial tile (indices grow with u).
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t v = vec_index<kUnroll>(lt, lane(), u);
            if (v >= nv)
                break;
            u32x4 x[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                x[k] = ld16(in[k] + v);
            st16(out + v, fold_vec<BF16, K>(x, scale));
        }
    }
    if (lt == 0)
        reduce_edges<BF16, K>(sg, 0, nv * kVecElems, sg.n - nv * kVecElems);
}

// Body vector v of an input whose body starts s bytes (uniform across the
// workgroup) past aligned word v: bytes [s, 16) of word v (a) and [0, s) of
// word v+1, which the next lane holds; the wave's last lane loaded word v+1
// itself (c).
__device__ __forceinline__ u32x4 shifted_word(u32x4 a, u32x4 c, unsigned s, bool last)
{
    if (s == 0)
        return a;
    const u32x4 nb = next_lane(a);  // every lane is active here: s is uniform
    const u32x4 b = last ? c : nb;
    switch (s >> 2) {
    case 0: return realign<0>(a, b, s & 3);
    case 1: return realign<1>(a, b, s & 3);
    case 2: return realign<2>(a, b, s & 3);
    default: return realign<3>(a, b, s & 3);
    }
}

// One tile of a realigning body.  Every lane loads aligned word v of each
// input once; for an input with s > 0 the wave's last lane also loads word
// v+1, and in a partial tile a lane loads word nv, which its left neighbour
// needs, and stores nothing.  Word nv of such an input holds at least one
// byte of its body, and an aligned 16-byte word never straddles a page.
template <bool BF16, int K, bool kFull>
__device__ __forceinline__ void shifted_tile(const u32x4 *const (&base)[K], const unsigned (&sh)[K],
                                             u32x4 *out, int64_t lt, int64_t nv, float scale)
{
    constexpr int U = kShiftRedUnroll;
    const bool last = wave_end(lane());
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 a[U][K], c[U][K];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t v = vec_index<U>(lt, lane(), u);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            a[u][k] = loads_own_word(kFull, v, nv, sh[k] != 0) ? ld16(base[k] + v) : zero;
            c[u][k] = loads_next_word(kFull, v, nv, sh[k] != 0, last) ? ld16(base[k] + v + 1) : zero;
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t v = vec_index<U>(lt, lane(), u);
        u32x4 x[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            x[k] = shifted_word(a[u][k], c[u][k], sh[k], last);
        if (kFull || v < nv)
            st16(out + v, fold_vec<BF16, K>(x, scale));
    }
}

// kRedShifted segment: pointers at any element alignment.  The body covers
// the output's whole 16-byte vectors; each input's body is read as aligned
// words and realigned in registers (v_alignbyte).
template <bool BF16, int K>
__device__ __forceinline__ void reduce_shifted(const RedSeg &sg, int64_t lt)
{
    constexpr int64_t es = BF16 ? 2 : 4;
    const RedSplit sp = red_split(sg.out, sg.n, es);
    const u32x4 *base[K];
    unsigned sh[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const WordAt w = word_at(static_cast<const unsigned char *>(sg.in[k]) + sp.head * es);
        sh[k] = w.shift;
        base[k] = reinterpret_cast<const u32x4 *>(w.base);
    }
    u32x4 *out = reinterpret_cast<u32x4 *>(static_cast<unsigned char *>(sg.out) + sp.head * es);
    if (full_tile(lt, tile_vecs<kShiftRedUnroll>(), sp.nv))
        shifted_tile<BF16, K, true>(base, sh, out, lt, sp.nv, sg.scale);
    else if (sp.nv > 0)  // uniform across the workgroup
        shifted_tile<BF16, K, false>(base, sh, out, lt, sp.nv, sg.scale);
    if (lt == 0)
        reduce_edges<BF16, K>(sg, sp.head, sp.head + sp.nv * (16 / es), sp.tail);
}

// Tile lt of one segment.
template <bool BF16>
__device__ __forceinline__ void reduce_seg(const RedSeg &sg, int64_t lt)
{
    switch (sg.k) {
    case 1: reduce_vec<BF16, 1>(sg, lt); break;
    case 2: reduce_vec<BF16, 2>(sg, lt); break;
    case 3: reduce_vec<BF16, 3>(sg, lt); break;
    case 4: reduce_vec<BF16, 4>(sg, lt); break;
    default: break;
    }
}

template <bool BF16>
__device__ __forceinline__ void reduce_shifted_seg(const RedSeg &sg, int64_t lt)
{
    switch (sg.k) {
    case 1: reduce_shifted<BF16, 1>(sg, lt); break;
    case 2: reduce_shifted<BF16, 2>(sg, lt); break;
    case 3: reduce_shifted<BF16, 3>(sg, lt); break;
    case 4: reduce_shifted<BF16, 4>(sg, lt); break;
    default: break;
    }
}

// One workgroup per tile in every launch form.  Workgroups reach the eight
// XCDs round-robin, so neighbouring tiles stream through different XCDs; this
// interleave measured faster than giving each XCD a contiguous range of tiles.

// Table form: tile t of the whole batch.
template <bool BF16, int CAP>
__global__ __launch_bounds__(kBlock) void reduce_kernel(RedBatchT<CAP> b)
{
    const int32_t t = (int32_t)blockIdx.x;
    const int s = find_seg(b.tile0, b.nseg, t);
    reduce_seg<BF16>(load_seg(b.seg[s]), (int64_t)(t - b.tile0[s]));
}

// Uniform form: segment blockIdx.y, tile blockIdx.x (every segment has
// gridDim.x tiles), so no table is searched.
template <bool BF16, int CAP>
__global__ __launch_bounds__(kBlock) void reduce_uniform_kernel(RedBatchT<CAP> b)
{
    reduce_seg<BF16>(load_seg(b.seg[blockIdx.y]), (int64_t)blockIdx.x);
}

// The realigning reduction, in the table and uniform forms.
template <bool BF16, int CAP>
__global__ __launch_bounds__(kBlock) void reduce_shifted_kernel(RedBatchT<CAP> b)
{
    const int32_t t = (int32_t)blockIdx.x;
    const int s = find_seg(b.tile0, b.nseg, t);
    reduce_shifted_seg<BF16>(load_seg(b.seg[s]), (int64_t)(t - b.tile0[s]));
}

template <bool BF16, int CAP>
__global__ __launch_bounds__(kBlock) void reduce_shifted_uniform_kernel(RedBatchT<CAP> b)
{
    reduce_shifted_seg<BF16>(load_seg(b.seg[blockIdx.y]), (int64_t)blockIdx.x);
}

// Single-segment form: the aligned segment's pointers, length and scale are
// plain arguments, preloaded into scalar registers at wave launch, and K is
// a template parameter, so the first vector load issues at once.
template <bool BF16, int K>
__global__ __launch_bounds__(kBlock) void reduce_one_kernel(const void *in0, const void *in1,
                                                            const void *in2, const void *in3,
                                                            void *out, int64_t n, float scale)
{
    RedSeg sg;
    sg.in[0] = in0;
    sg.in[1] = in1;
    sg.in[2] = in2;
    sg.in[3] = in3;
    sg.out = out;
    sg.n = n;
    sg.k = K;
    sg.mode = kRedAligned;
    sg.scale = scale;
    sg.pad = 0;
    reduce_vec<BF16, K>(sg, (int64_t)blockIdx.x);
}

// The same for one realigning (kRedShifted) segment.
template <bool BF16, int K>
__global__ __launch_bounds__(kBlock) void reduce_shifted_one_kernel(const void *in0, const void *in1,
                                                                    const void *in2, const void *in3,
                                                                    void *out, int64_t n, float scale)
{
    RedSeg sg;
    sg.in[0] = in0;
    sg.in[1] = in1;
    sg.in[2] = in2;
    sg.in[3] = in3;
    sg.out = out;
    sg.n = n;
    sg.k = K;
    sg.mode = kRedShifted;
    sg.scale = scale;
    sg.pad = 0;
    reduce_shifted<BF16, K>(sg, (int64_t)blockIdx.x);
}

// ---------------------------------------------------------------------------
// Copy
// ---------------------------------------------------------------------------

// The destination of one copy tile.  Copies of calls under kCopyAgentMaxBytes
// store with agent scope (WT: the sc1 cache-policy bit, no non-temporal
// hint): the L2 writes each line through to memory at once instead of holding
// it dirty until the end-of-kernel release, so less is left to drain between
// this launch and the next.  A buffer store carries that policy; its resource
// starts at the tile's first destination vector (uniform across the
// workgroup) and spans the tile's body vectors.  Larger calls keep
// non-temporal stores, which measured faster there.
constexpr int kBufferFormat = 0x00020000;  // raw buffer: 32-bit data format, no swizzle
constexpr int kStoreAgentScope = 16;       // cache-policy operand: sc1

template <bool WT>
struct TileOut {
    u32x4 *first;
    __amdgpu_buffer_rsrc_t r;
    __device__ TileOut(u32x4 *first_, int64_t nvec)
        : first(first_), r(__builtin_amdgcn_make_buffer_rsrc(first_, (short)0, (int)(nvec * 16), kBufferFormat))
    {
    }
    // Vector i of the tile (0 <= i < nvec).
    __device__ void put(int64_t i, u32x4 v) const
    {
        if constexpr (WT)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)(i * 16), 0, kStoreAgentScope);
        else
            st16(first + i, v);
    }
};

// Tile lt of a body of nv vectors in tiles of tv vectors.
template <bool WT>
__device__ __forceinline__ TileOut<WT> tile_out(u32x4 *dst, int64_t lt, int64_t tv, int64_t nv)
{
    const TileBody tb = tile_body(lt, tv, nv);
    return TileOut<WT>(dst + tb.first, tb.count);
}

// Tile 0 of a copy segment also moves its head and tail bytes (at most 15
// each): the first wave's lanes the head, the second wave's the tail.
__device__ __forceinline__ void copy_edges(const CopySeg &sg, const CopySplit &sp)
{
    const int x = lane();
    if (head_lane(x, sp.head)) {
        sg.dst[x] = sg.src[x];
    } else if (tail_lane(x, sp.tail)) {
        const int64_t i = tail_elem(x, sp.head + 16 * sp.nv);
        sg.dst[i] = sg.src[i];
    }
}

// U: 16-byte vectors per lane in a tile (kCopyUnroll, or kCopyUnrollLong
// for the batches of a long call); WT: agent-scope stores (TileOut).
template <int U, bool WT>
__device__ __forceinline__ void copy_aligned(const CopySeg &sg, int64_t lt)
{
    const CopySplit sp = copy_split(sg.dst, sg.nbytes);
    const int64_t nv = sp.nv;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(sg.src + sp.head);
    u32x4 *dst = reinterpret_cast<u32x4 *>(sg.dst + sp.head);
    if (full_tile(lt, tile_vecs<U>(), nv)) {
        const TileOut<WT> out = tile_out<WT>(dst, lt, tile_vecs<U>(), nv);
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            x[u] = ld16(src + vec_index<U>(lt, lane(), u));
#pragma unroll
        for (int u = 0; u < U; ++u)
            out.put(vec_index<U>(0, lane(), u), x[u]);
    } else if (nv > 0) {  // uniform across the workgroup
        const TileOut<WT> out = tile_out<WT>(dst, lt, tile_vecs<U>(), nv);
        for (int u = 0; u < U; ++u) {
            const int64_t v = vec_index<U>(lt, lane(), u);
            if (v >= nv)
                break;
            out.put(vec_index<U>(0, lane(), u), ld16(src + v));
        }
    }
    if (lt == 0)
        copy_edges(sg, sp);
}

// Body vector v is bytes [shift + 16v, shift + 16v + 16) of the aligned
// source base (the body's first source byte less `shift`): the tail of
// source word v and the head of word v+1.  Each lane loads its own word once
// (non-temporal) and takes word v+1 from the next lane of its wave; the
// wave's last lane, whose neighbour word belongs to another wave or tile,
// loads word v+1 itself, issued with the other loads.  In a partial tile a
// lane also loads word nv, which its left neighbour needs, and stores
// nothing.  Word nv always holds at least one byte of the body (shift > 0),
// and an aligned 16-byte word never straddles a page, so that read stays in
// mapped memory even where the source buffer ends inside the word.
template <int Q, bool WT>
__device__ __forceinline__ void copy_shifted(const CopySeg &sg, int64_t lt)
{
    const CopySplit sp = copy_split(sg.dst, sg.nbytes);
    const int64_t nv = sp.nv;
    const unsigned r = (unsigned)(sg.shift & 3);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(sg.src + sp.head - sg.shift);
    u32x4 *dst = reinterpret_cast<u32x4 *>(sg.dst + sp.head);
    const bool last = wave_end(lane());
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 a[kShiftUnroll], c[kShiftUnroll];
    if (full_tile(lt, tile_vecs<kShiftUnroll>(), nv)) {
#pragma unroll
        for (int u = 0; u < kShiftUnroll; ++u) {
            const int64_t v = vec_index<kShiftUnroll>(lt, lane(), u);
            a[u] = loads_own_word(true, v, nv, true) ? ld16(src + v) : zero;
            c[u] = loads_next_word(true, v, nv, true, last) ? ld16(src + v + 1) : zero;
        }
        const TileOut<WT> out = tile_out<WT>(dst, lt, tile_vecs<kShiftUnroll>(), nv);
#pragma unroll
        for (int u = 0; u < kShiftUnroll; ++u) {
            const u32x4 nb = next_lane(a[u]);  // on every lane: the source lane must be active
            const u32x4 b = last ? c[u] : nb;
            out.put(vec_index<kShiftUnroll>(0, lane(), u), realign<Q>(a[u], b, r));
        }
    } else if (nv > 0) {  // uniform across the workgroup
#pragma unroll
        for (int u = 0; u < kShiftUnroll; ++u) {
            const int64_t v = vec_index<kShiftUnroll>(lt, lane(), u);
            a[u] = loads_own_word(false, v, nv, true) ? ld16(src + v) : zero;
            c[u] = loads_next_word(false, v, nv, true, last) ? ld16(src + v + 1) : zero;
        }
        const TileOut<WT> out = tile_out<WT>(dst, lt, tile_vecs<kShiftUnroll>(), nv);
#pragma unroll
        for (int u = 0; u < kShiftUnroll; ++u) {
            const int64_t v = vec_index<kShiftUnroll>(lt, lane(), u);
            const u32x4 nb = next_lane(a[u]);
            const u32x4 b = last ? c[u] : nb;
            if (v < nv)
                out.put(vec_index<kShiftUnroll>(0, lane(), u), realign<Q>(a[u], b, r));
        }
    }
    if (lt == 0)
        copy_edges(sg, sp);
}

// Segments whose source and destination agree modulo 16 bytes.  U and WT
// as in copy_aligned.
template <int CAP, int U, bool WT>
__global__ __launch_bounds__(kBlock) void copy_kernel(CopyBatchT<CAP> b)
{
    const int32_t t = (int32_t)blockIdx.x;
    const int s = find_seg(b.tile0, b.nseg, t);
    copy_aligned<U, WT>(load_seg(b.seg[s]), (int64_t)(t - b.tile0[s]));
}

template <int CAP, int U, bool WT>
__global__ __launch_bounds__(kBlock) void copy_uniform_kernel(CopyBatchT<CAP> b)
{
    copy_aligned<U, WT>(load_seg(b.seg[blockIdx.y]), (int64_t)blockIdx.x);
}

// Any segment: realigned (source and destination disagree modulo 16 bytes)
// or aligned, by the segment's mode, so that a call whose chunk moves mix
// both (a segmentCount that is not a multiple of 8) takes one launch.  The
// aligned-only kernels above keep the smaller register budget for calls
// without realigned moves.
template <int U, bool WT>
__device__ __forceinline__ void copy_mixed_seg(const CopySeg &sg, int64_t lt)
{
    if (sg.mode != kCopyShifted) {  // uniform across the workgroup
        copy_aligned<U, WT>(sg, lt);
        return;
    }
    switch (sg.shift >> 2) {
    case 0: copy_shifted<0, WT>(sg, lt); break;
    case 1: copy_shifted<1, WT>(sg, lt); break;
    case 2: copy_shifted<2, WT>(sg, lt); break;
    default: copy_shifted<3, WT>(sg, lt); break;
    }
}

template <int CAP, int U, bool WT>
__global__ __launch_bounds__(kBlock) void copy_mixed_kernel(CopyBatchT<CAP> b)
{
    const int32_t t = (int32_t)blockIdx.x;
    const int s = find_seg(b.tile0, b.nseg, t);
    copy_mixed_seg<U, WT>(load_seg(b.seg[s]), (int64_t)(t - b.tile0[s]));
}

template <int CAP, int U, bool WT>
__global__ __launch_bounds__(kBlock) void copy_mixed_uniform_kernel(CopyBatchT<CAP> b)
{
    copy_mixed_seg<U, WT>(load_seg(b.seg[blockIdx.y]), (int64_t)blockIdx.x);
}

}  // namespace

namespace {

template <bool BF16, int K>
void launch_one_k(const RedSeg &sg, const dim3 &grid, bool shifted, hipStream_t stream)
{
    const dim3 block(kBlock);
    const unsigned lds = grid.x >= kThrottleTiles ? kThrottleLds : 0u;
    if (shifted)
        reduce_shifted_one_kernel<BF16, K><<<grid, block, lds, stream>>>(sg.in[0], sg.in[1], sg.in[2], sg.in[3],
                                                                         sg.out, sg.n, sg.scale);
    else
        reduce_one_kernel<BF16, K><<<grid, block, 0, stream>>>(sg.in[0], sg.in[1], sg.in[2], sg.in[3], sg.out,
                                                               sg.n, sg.scale);
}

template <bool BF16>
void launch_one(const RedSeg &sg, int64_t tiles, bool shifted, hipStream_t stream)
{
    const dim3 grid((unsigned)tiles);
    switch (sg.k) {
    case 1: launch_one_k<BF16, 1>(sg, grid, shifted, stream); break;
    case 2: launch_one_k<BF16, 2>(sg, grid, shifted, stream); break;
    case 3: launch_one_k<BF16, 3>(sg, grid, shifted, stream); break;
    default: launch_one_k<BF16, 4>(sg, grid, shifted, stream); break;
    }
}

}  // namespace

namespace {

// The first n entries of a full-capacity table in a table of capacity CAP.
template <typename Small, typename Full>
Small shrink(const Full &b)
{
    Small t{};
    t.nseg = b.nseg;
    for (int i = 0; i < b.nseg; ++i) {
        t.tile0[i] = b.tile0[i];
        t.seg[i] = b.seg[i];
    }
    return t;
}

template <bool BF16, int CAP>
void launch_reduce_table(const RedBatchT<CAP> &b, const LaunchShape &sh, int64_t total_tiles, bool shifted,
                         hipStream_t stream)
{
    const dim3 block(kBlock);
    if (sh.form == kFormUniform) {
        const dim3 grid((unsigned)sh.gx, (unsigned)sh.gy);
        if (shifted)
            reduce_shifted_uniform_kernel<BF16, CAP><<<grid, block, 0, stream>>>(b);
        else
            reduce_uniform_kernel<BF16, CAP><<<grid, block, 0, stream>>>(b);
    } else {
        const dim3 grid((unsigned)total_tiles);
        if (shifted)
            reduce_shifted_kernel<BF16, CAP><<<grid, block, 0, stream>>>(b);
        else
            reduce_kernel<BF16, CAP><<<grid, block, 0, stream>>>(b);
    }
}

template <bool BF16>
void launch_reduce_sized(const RedBatch &b, const LaunchShape &sh, int64_t total_tiles, bool shifted,
                         hipStream_t stream)
{
    if (b.nseg <= kSmallRedSegs) {
        RedBatchT<kSmallRedSegs> t = shrink<RedBatchT<kSmallRedSegs>>(b);
        t.bf16 = b.bf16;
        launch_reduce_table<BF16>(t, sh, total_tiles, shifted, stream);
    } else {
        launch_reduce_table<BF16>(b, sh, total_tiles, shifted, stream);
    }
}

template <int CAP, int U, bool WT>
void launch_copy_table(const CopyBatchT<CAP> &b, const LaunchShape &sh, int64_t total_tiles, bool shifted,
                       hipStream_t stream)
{
    const dim3 block(kBlock);
    if (sh.form == kFormUniform) {
        const dim3 grid((unsigned)sh.gx, (unsigned)sh.gy);
        const unsigned lds = total_tiles >= kThrottleTiles ? kThrottleLds : 0u;
        if (shifted)
            copy_mixed_uniform_kernel<CAP, U, WT><<<grid, block, lds, stream>>>(b);
        else
            copy_uniform_kernel<CAP, U, WT><<<grid, block, lds, stream>>>(b);
    } else {
        const dim3 grid((unsigned)total_tiles);
        if (shifted)
            copy_mixed_kernel<CAP, U, WT><<<grid, block, 0, stream>>>(b);
        else
            copy_kernel<CAP, U, WT><<<grid, block, 0, stream>>>(b);
    }
}

// Large calls (the batch's nt_stores) keep non-temporal stores, long aligned
// ones in the long-call tiles; every other copy stores with agent scope.
template <int CAP>
void launch_copy_sized(const CopyBatchT<CAP> &b, const LaunchShape &sh, int64_t total_tiles, bool shifted,
                       hipStream_t stream)
{
    if (b.long_tiles)
        launch_copy_table<CAP, kCopyUnrollLong, false>(b, sh, total_tiles, shifted, stream);
    else if (b.nt_stores || !kCopyAgentStores)
        launch_copy_table<CAP, kCopyUnroll, false>(b, sh, total_tiles, shifted, stream);
    else
        launch_copy_table<CAP, kCopyUnroll, true>(b, sh, total_tiles, shifted, stream);
}

}  // namespace

hipError_t launch_reduce(const RedBatch &b, int64_t total_tiles, bool shifted, hipStream_t stream)
{
    if (total_tiles <= 0)
        return hipSuccess;
    (void)hipGetLastError();  // report this launch's status only
    const LaunchShape sh = reduce_shape(b, total_tiles);
    if (sh.form == kFormOne) {
        if (b.bf16)
            launch_one<true>(b.seg[0], sh.gx, shifted, stream);
        else
            launch_one<false>(b.seg[0], sh.gx, shifted, stream);
    } else if (b.bf16) {
        launch_reduce_sized<true>(b, sh, total_tiles, shifted, stream);
    } else {
        launch_reduce_sized<false>(b, sh, total_tiles, shifted, stream);
    }
    return hipGetLastError();
}

hipError_t launch_copy(const CopyBatch &b, int64_t total_tiles, bool shifted, hipStream_t stream)
{
    if (total_tiles <= 0)
        return hipSuccess;
    (void)hipGetLastError();  // report this launch's status only
    const LaunchShape sh = copy_shape(b, total_tiles);
    if (b.nseg <= kSmallCopySegs) {
        CopyBatchT<kSmallCopySegs> t = shrink<CopyBatchT<kSmallCopySegs>>(b);
        t.long_tiles = b.long_tiles;
        t.nt_stores = b.nt_stores;
        launch_copy_sized(t, sh, total_tiles, shifted, stream);
    } else {
        launch_copy_sized(b, sh, total_tiles, shifted, stream);
    }
    return hipGetLastError();
}

}  // namespace rr
