// rr_internal.h -- launch descriptors shared by the C-ABI layer (rr_api.cpp)
// and the gfx950 kernels (rr_kernels.hip).  Not part of the public ABI.
//
// Every relay step is a streaming element-wise operation: a K-input
// fp32-accumulated sum with one scale and one rounding, or a raw copy of
// chunks between strided and contiguous layouts.  A launch therefore carries a
// small table of independent "segments" in its kernel arguments; each
// workgroup processes one fixed-size tile of one segment.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace rr {

#ifndef RR_BLOCK
#define RR_BLOCK 256                 // threads per workgroup (4 wave64)
#endif
constexpr int kBlock = RR_BLOCK;
constexpr int kMaxIn = 4;            // inputs per reduction segment (A <= 4)
constexpr int kMaxRedSegs = 40;      // segments per reduction launch
constexpr int kMaxCopySegs = 64;     // segments per copy launch
#ifndef RR_MAX_TILES_PER_LAUNCH
#define RR_MAX_TILES_PER_LAUNCH (int64_t(1) << 22)  // longer batches continue in further launches
#endif
constexpr int64_t kMaxTilesPerLaunch = RR_MAX_TILES_PER_LAUNCH;

#ifndef RR_UNROLL
#define RR_UNROLL 4                  // 16-byte vectors per thread per input
#endif
#ifndef RR_LOAD_NT
#define RR_LOAD_NT 1                 // inputs are read exactly once
#endif
#ifndef RR_STORE_NT
#define RR_STORE_NT 1                // outputs are written exactly once
#endif

#ifndef RR_COPY_UNROLL
#define RR_COPY_UNROLL 2             // 16-byte vectors per thread in a copy tile:
                                     // 8 KiB tiles measured faster than 16 and 32 KiB
                                     // from 16 MiB to 1 GiB
#endif
#ifndef RR_COPY_UNROLL_LONG
#define RR_COPY_UNROLL_LONG 1        // the same for calls that move at least
                                     // RR_COPY_LONG_BYTES: 4 KiB tiles moved a 1 GiB
                                     // message's all-to-all 5% faster than 8 KiB tiles,
                                     // equal at 256 MiB, 5% slower at 64 MiB
#endif
#ifndef RR_COPY_LONG_BYTES
#define RR_COPY_LONG_BYTES (int64_t(1) << 29)
#endif
#ifndef RR_COPY_AGENT_STORES
#define RR_COPY_AGENT_STORES 1       // copies of calls under RR_COPY_AGENT_MAX_BYTES store with
                                     // agent scope (write-through L2); 0: non-temporal throughout
#endif
#ifndef RR_COPY_AGENT_MAX_BYTES
#define RR_COPY_AGENT_MAX_BYTES (int64_t(1) << 28)  // calls moving this much or more store
                                                    // non-temporally: the step gained with agent-
                                                    // scope stores up to 161 MB per call, lost a
                                                    // point at 322 MB
#endif

#ifndef RR_SHIFT_RED_UNROLL
#define RR_SHIFT_RED_UNROLL 2        // 16-byte vectors per thread per input in a realigning
                                     // reduction tile (8 KiB per input)
#endif

constexpr int kUnroll = RR_UNROLL;
constexpr int kShiftRedUnroll = RR_SHIFT_RED_UNROLL;
constexpr int kCopyUnroll = RR_COPY_UNROLL;
constexpr int kCopyUnrollLong = RR_COPY_UNROLL_LONG;
constexpr int64_t kCopyLongBytes = RR_COPY_LONG_BYTES;
constexpr bool kCopyAgentStores = RR_COPY_AGENT_STORES != 0;
constexpr int64_t kCopyAgentMaxBytes = RR_COPY_AGENT_MAX_BYTES;
#ifndef RR_SHIFT_UNROLL
#define RR_SHIFT_UNROLL 2            // 16-byte vectors per thread in a realigning copy tile
                                     // (8 KiB tiles; measured faster than 16 and 32 KiB)
#endif
constexpr int kShiftUnroll = RR_SHIFT_UNROLL;

// Launches of at least kThrottleTiles tiles in the uniform copy kernels
// (aligned and mixed) and in the realigning single-segment reduction reserve
// kThrottleLds bytes of (unused) LDS per workgroup, which lets 6 of them
// share a CU's 160 KiB instead of 8: with fewer loads and stores in flight,
// HBM serves a long stream 1-4% faster.  Aligned reductions and short
// launches measured best at full occupancy; the other realigning reductions
// already run 6 per CU (their register count).
#ifndef RR_THROTTLE_TILES
#define RR_THROTTLE_TILES 4096
#endif
#ifndef RR_THROTTLE_LDS
#define RR_THROTTLE_LDS (26 * 1024)
#endif
constexpr int64_t kThrottleTiles = RR_THROTTLE_TILES;
constexpr unsigned kThrottleLds = RR_THROTTLE_LDS;

enum RedMode : int32_t { kRedAligned = 1, kRedShifted = 2 };

// One reduction segment: out[i] = RND(scale * fold_k in[k][i]) for i < n,
// every pointer aligned to the element.  The elements before out's first
// 16-byte boundary (the head) and those after the last whole 16-byte output
// vector (the tail) are computed element by element by tile 0; the vectors
// between them (the body) are spread over the segment's tiles.
// kRedAligned: every pointer is 16-byte aligned (no head).  kRedShifted: any
// alignment; each input's body is realigned to the output's vectors.
struct RedSeg {
    const void *in[kMaxIn];
    void *out;
    int64_t n;
    int32_t k;
    int32_t mode;
    float scale;
    int32_t pad;
};

static_assert(sizeof(RedSeg) == 64, "a reduction descriptor is one 64-byte scalar load");

// A launch's segment table, passed by value in the kernel arguments.  The
// launcher fills a table of the full capacity; a launch of few segments is
// passed in a small one, since every byte of kernel arguments costs host time
// at each launch (a 2.8 KB table added about 0.75 us per call against a 0.6 KB
// one).
template <int CAP>
struct RedBatchT {
    int32_t tile0[CAP];  // first tile of each segment within this launch
    int32_t nseg;
    int32_t bf16;        // element type: 1 bf16, 0 fp32
    RedSeg seg[CAP];
};
constexpr int kSmallRedSegs = 8;
using RedBatch = RedBatchT<kMaxRedSegs>;

enum CopyMode : int32_t { kCopyAligned = 1, kCopyShifted = 2 };

// One copy segment: nbytes from src to dst, both at any byte address.  The
// bytes before dst's first 16-byte boundary (the head) and those after the
// last whole 16-byte vector (the tail) are copied byte by byte by tile 0;
// the vectors between them (the body) are spread over the segment's tiles.
// kCopyAligned: src and dst agree modulo 16 bytes, so the body's source is
// 16-byte aligned too.  kCopyShifted: they disagree; the body's first source
// byte lies `shift` bytes (1..15) past a 16-byte boundary.
struct CopySeg {
    const unsigned char *src;
    unsigned char *dst;
    int64_t nbytes;
    int32_t mode;
    int32_t shift;
};

static_assert(sizeof(CopySeg) == 32, "a copy descriptor is one 32-byte scalar load");

// Head elements, 16-byte body vectors and tail elements of a reduction of n
// elements of es bytes into out (out aligned to es).
struct RedSplit {
    int64_t head, nv, tail;
};

__host__ __device__ inline RedSplit red_split(const void *out, int64_t n, int64_t es)
{
    const int64_t to_line = int64_t((16u - unsigned(reinterpret_cast<uintptr_t>(out) & 15u)) & 15u) / es;
    const int64_t head = to_line < n ? to_line : n;
    const int64_t nv = (n - head) / (16 / es);
    return RedSplit{head, nv, n - head - (16 / es) * nv};
}

// Head bytes (at most 15), 16-byte body vectors and tail bytes (at most 15)
// of a copy of nbytes to dst.
struct CopySplit {
    int64_t head, nv, tail;
};

__host__ __device__ inline CopySplit copy_split(const unsigned char *dst, int64_t nbytes)
{
    const int64_t to_line = int64_t((16u - unsigned(reinterpret_cast<uintptr_t>(dst) & 15u)) & 15u);
    const int64_t head = to_line < nbytes ? to_line : nbytes;
    const int64_t nv = (nbytes - head) / 16;
    return CopySplit{head, nv, nbytes - head - 16 * nv};
}

// ---------------------------------------------------------------------------
// Index arithmetic of a tile.  The kernels (rr_kernels.hip) and the host
// replay of their accesses (the bounds checks of the test suite) both call
// these functions, so the replay follows the shipped indexing by
// construction.  `x` is the lane's index in the workgroup (threadIdx.x).
// ---------------------------------------------------------------------------

constexpr int kWave = 64;  // gfx950 runs wave64

// 16-byte vectors in one tile of a body processed U vectors per lane.
template <int U>
__host__ __device__ constexpr int64_t tile_vecs()
{
    return int64_t(kBlock) * U;
}

// Vector index of unroll step u of lane x within tile lt: step u of lane x is
// x + u*kBlock, so each wave instruction covers 1 KiB and the workgroup's four
// waves fill each 4 KiB.
template <int U>
__host__ __device__ inline int64_t vec_index(int64_t lt, int x, int u)
{
    return lt * tile_vecs<U>() + int64_t(x) + int64_t(u) * kBlock;
}

// The body vectors of tile lt (tiles of tv vectors, body of nv vectors, the
// tile holding at least one): the first one and how many.  A copy tile's
// stores address its vectors relative to `first` (vec_index with lt = 0), in
// a buffer range of `count` vectors.
struct TileBody {
    int64_t first, count;
};

__host__ __device__ inline TileBody tile_body(int64_t lt, int64_t tv, int64_t nv)
{
    const int64_t first = lt * tv;
    return TileBody{first, nv - first < tv ? nv - first : tv};
}

// Tile lt of a body of nv vectors is full (every lane's every step in range).
__host__ __device__ inline bool full_tile(int64_t lt, int64_t tv, int64_t nv)
{
    return (lt + 1) * tv <= nv;
}

// Tiles of a body of nv vectors: at least one, which also handles the edges.
__host__ __device__ inline int64_t body_tiles(int64_t nv, int64_t tv)
{
    return nv > tv ? (nv + tv - 1) / tv : 1;
}

// The last lane of its wave, which has no next lane to take a word from.
__host__ __device__ inline bool wave_end(int x)
{
    return (x & (kWave - 1)) == kWave - 1;
}

// Which aligned 16-byte words a lane loads for body vector v of a realigning
// tile (full: the whole tile is in range).  Every lane in range loads its own
// word v; for an input whose body is not 16-byte aligned (`shifted`) the
// wave's last lane also loads word v+1, which the other lanes take from their
// next lane, and in a partial tile a lane whose v == nv still loads word nv
// (its left neighbour needs it) and stores nothing.
__host__ __device__ inline bool loads_own_word(bool full, int64_t v, int64_t nv, bool shifted)
{
    return full || v < nv || (v == nv && shifted);
}

__host__ __device__ inline bool loads_next_word(bool full, int64_t v, int64_t nv, bool shifted, bool last_lane)
{
    return last_lane && shifted && (full || v < nv);
}

// The lanes of a segment's tile 0 that compute its edges, element by element
// (or byte by byte): lane x < head computes head element x; a lane of the
// second wave with tail_lane(x, tail) computes element tail_elem(x, tail0) of
// the tail [tail0, tail0 + tail).  Each edge is shorter than one 16-byte
// vector.
__host__ __device__ inline bool head_lane(int x, int64_t head)
{
    return x < head;
}

__host__ __device__ inline bool tail_lane(int x, int64_t tail)
{
    return x >= kWave && x - kWave < tail;
}

__host__ __device__ inline int64_t tail_elem(int x, int64_t tail0)
{
    return tail0 + (x - kWave);
}

// Index of the segment that owns tile t in a table form launch: the number of
// later segment starts at or before t.  Unrolled over the table, one bit per
// start in a 64-bit mask, then a population count: on the GPU every step stays
// on the scalar unit (a running sum of the compares was compiled to a chain of
// 64-bit vector adds, several hundred cycles before a workgroup's first load).
template <int MAXS>
__host__ __device__ inline int find_seg(const int32_t (&tile0)[MAXS], int nseg, int32_t t)
{
    static_assert(MAXS >= 1 && MAXS <= 64, "one mask bit per segment");
    uint64_t m = 0;
#pragma unroll
    for (int i = 1; i < MAXS; ++i)
        m |= uint64_t(t >= tile0[i]) << i;
    const uint64_t valid = nseg >= 64 ? ~uint64_t(0) : (uint64_t(1) << nseg) - 1;
    return __builtin_popcountll(m & valid);
}

// The aligned 16-byte word holding byte p, and p's offset in it (0..15).
// The base stays a pointer derived from p (not an integer), so device code
// keeps p's address space and loads through it as global memory.
struct WordAt {
    const unsigned char *base;
    unsigned shift;
};

__host__ __device__ inline WordAt word_at(const unsigned char *p)
{
    const unsigned s = unsigned(reinterpret_cast<uintptr_t>(p) & 15u);
    return WordAt{p - s, s};
}

// Work per tile (one workgroup) of each segment mode: a segment spans
// body_tiles(nv, tile vectors) tiles.
__host__ __device__ constexpr int64_t red_tile_vecs(int32_t mode)
{
    return mode == kRedShifted ? tile_vecs<kShiftRedUnroll>() : tile_vecs<kUnroll>();
}

// long_tiles: the batch belongs to a call that moves at least kCopyLongBytes
// in aligned moves only; they use tiles of kCopyUnrollLong vectors per lane.
// nt_stores: the batch belongs to a call that moves at least
// kCopyAgentMaxBytes (aligned or not); its stores are non-temporal, those of
// every other call agent-scope write-through stores.
template <int CAP>
struct CopyBatchT {
    int32_t tile0[CAP];
    int32_t nseg;
    int32_t long_tiles;
    int32_t nt_stores;
    int32_t pad;
    CopySeg seg[CAP];
};
constexpr int kSmallCopySegs = 16;
using CopyBatch = CopyBatchT<kMaxCopySegs>;

__host__ __device__ constexpr int64_t copy_tile_vecs(int32_t mode, bool long_tiles)
{
    return mode == kCopyShifted ? tile_vecs<kShiftUnroll>()
                                : long_tiles ? tile_vecs<kCopyUnrollLong>() : tile_vecs<kCopyUnroll>();
}

// How a batch is launched.  Every form runs the same work per tile; they
// differ in how a workgroup learns its segment before its first load:
//   kFormTable:   1-D grid of all tiles; a count over tile0 finds the
//                 segment, then its descriptor is loaded (dependent scalar
//                 loads from the kernel arguments);
//   kFormUniform: every segment has gx tiles: 2-D grid (gx, nseg), the
//                 segment is blockIdx.y and the tile blockIdx.x;
//   kFormOne:     one reduction segment (either mode): 1-D grid of gx
//                 tiles, the descriptor passed as scalar kernel arguments
//                 that the hardware preloads into registers.
enum LaunchForm : int32_t { kFormTable = 0, kFormUniform = 1, kFormOne = 2 };
struct LaunchShape {
    int32_t form;
    int64_t gx, gy;
};
// One recorded launch of a plan (rr_plan_begin .. rr_plan_launch): the batch
// as the launcher built it, and how it is launched.
enum PlanKind : int32_t { kPlanReduce = 1, kPlanCopy = 2 };
struct PlanRec {
    int32_t kind;
    int32_t shifted;
    int64_t tiles;
    union {
        RedBatch red;
        CopyBatch copy;
    };
};

// Header of a plan buffer, followed by `capacity` PlanRec records.
constexpr uint64_t kPlanMagic = 0x3150524c4559414cull;  // a tag for caller-owned plan memory
struct PlanHeader {
    uint64_t magic;
    int32_t capacity;   // records the buffer holds
    int32_t count;      // records written
    int32_t recording;  // 1 between rr_plan_begin and rr_plan_end
    int32_t broken;     // a call ran out of records; the plan cannot be launched
};

// Host-side choice of the form for a filled batch (rr_api.cpp).
LaunchShape reduce_shape(const RedBatch &b, int64_t total_tiles);
LaunchShape copy_shape(const CopyBatch &b, int64_t total_tiles);

// Enqueue one launch; the batch's tile0/nseg must be filled and the total
// tile count must not exceed kMaxTilesPerLaunch.  Returns the HIP status.
// A reduction batch holds either only kRedShifted segments (shifted = true)
// or none of them.
hipError_t launch_reduce(const RedBatch &b, int64_t total_tiles, bool shifted, hipStream_t stream);
// A copy batch with any kCopyShifted segment runs in the mixed-mode kernels
// (shifted = true), one without in the aligned-only kernels.
hipError_t launch_copy(const CopyBatch &b, int64_t total_tiles, bool shifted, hipStream_t stream);

}  // namespace rr
