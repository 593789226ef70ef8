// bench_calib.hip -- calibration streams for bench.py (not part of the relay
// library): R input streams read and W output streams written, 16-byte
// vectors per lane, 256-thread workgroups.  Timing each (R, W) mix at a size
// past the caches gives the HBM rate that streaming kernels of that mix reach
// on this GPU, beside the spec peak.
//
// Several access patterns are measured, so that the ceiling does not rest on
// the relay kernels' own pattern alone:
//   0 relay       16 KiB per stream per workgroup (4 vectors per lane), one
//                 tile per workgroup, every load of the tile before its
//                 stores, non-temporal loads and stores (the relay kernels'
//                 pattern);
//   1 tile8k      the same with 8 KiB tiles (2 vectors per lane);
//   2 tile4k      4 KiB tiles (1 vector per lane);
//   3 multi2      two 16 KiB tiles per workgroup, the second tile's loads
//                 issued before the first tile's stores;
//   4 multi4      four 8 KiB tiles per workgroup, each next tile's loads
//                 issued before the current tile's stores (register double
//                 buffer);
//   5 persistent  one workgroup per resident slot (occupancy x CUs), looping
//                 over 8 KiB tiles with a stride of the grid, register double
//                 buffered as multi4;
//   6 persist_wb  persistent with write-back (cached) stores;
//   7 relay_wb    the relay pattern with write-back stores;
//   8 relay_wt    the relay pattern with agent-scope stores (the sc1
//                 cache-policy bit: the L2 writes each line through at once);
//   9 tile8k_wt   8 KiB tiles with agent-scope stores (the relay copies'
//                 pattern for calls moving under 256 MiB).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kMaxStreams = 4;

struct Streams {
    const u32x4 *in[kMaxStreams];
    u32x4 *out[kMaxStreams];
    u32x4 *sink;  // written only if a (practically impossible) value appears
};

template <int R>
struct Tile {
    u32x4 x[4][R > 0 ? R : 1];
};

template <int R, int U>
__device__ __forceinline__ void load_tile(const Streams &s, int64_t t, Tile<R> &d)
{
    const int64_t base = t * (kBlock * U) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r)
            d.x[u][r] = __builtin_nontemporal_load(s.in[r] + base + u * kBlock);
}

// Store policies: non-temporal, write-back (cached), agent scope (a buffer
// store with the sc1 cache-policy bit, resource on the tile).
enum StorePolicy { kNT = 0, kWB = 1, kWT = 2 };

template <int R, int W, int U, int SP>
__device__ __forceinline__ void store_tile(const Streams &s, int64_t t, const Tile<R> &d)
{
    const int64_t base = t * (kBlock * U) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x4 v = {(unsigned)base, (unsigned)u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < R; ++r)
            v ^= d.x[u][r];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (SP == kNT) {
                __builtin_nontemporal_store(v, s.out[w] + base + u * kBlock);
            } else if (SP == kWB) {
                s.out[w][base + u * kBlock] = v;
            } else {
                __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(s.out[w] + t * (kBlock * U), (short)0,
                                                                              kBlock * U * 16, 0x00020000);
                __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)((threadIdx.x + u * kBlock) * 16), 0, 16);
            }
        }
        if (W == 0 && v.x == 0x9E3779B9u && v.y == 0x7F4A7C15u && v.z == 0xF39CC060u)
            s.sink[0] = v;  // keeps the loads of a read-only stream alive
    }
}

// Tiles first, first + step, first + 2*step, ... below ntiles, each tile's
// successor loaded before the tile is stored.  Every tile index is checked
// against ntiles before it is touched.
template <int R, int W, int U, int SP>
__device__ __forceinline__ void run_tiles(const Streams &s, int64_t first, int64_t step, int64_t last,
                                          int64_t ntiles)
{
    const int64_t end = last < ntiles ? last : ntiles;
    if (first >= end)
        return;
    Tile<R> a, b;
    load_tile<R, U>(s, first, a);
    for (int64_t t = first; t < end; t += 2 * step) {
        const int64_t t1 = t + step;
        if (t1 < end)
            load_tile<R, U>(s, t1, b);
        store_tile<R, W, U, SP>(s, t, a);
        if (t1 >= end)
            break;
        const int64_t t2 = t1 + step;
        if (t2 < end)
            load_tile<R, U>(s, t2, a);
        store_tile<R, W, U, SP>(s, t1, b);
    }
}

// One tile per workgroup (patterns 0, 1, 2, 7, 8, 9).
template <int R, int W, int U, int SP>
__global__ __launch_bounds__(kBlock) void one_tile_kernel(Streams s, int64_t ntiles)
{
    const int64_t t = blockIdx.x;
    if (t >= ntiles)
        return;
    Tile<R> a;
    load_tile<R, U>(s, t, a);
    store_tile<R, W, U, SP>(s, t, a);
}

// TPW consecutive tiles per workgroup (patterns 3, 4).
template <int R, int W, int U, int TPW>
__global__ __launch_bounds__(kBlock) void multi_tile_kernel(Streams s, int64_t ntiles)
{
    const int64_t first = (int64_t)blockIdx.x * TPW;
    run_tiles<R, W, U, kNT>(s, first, 1, first + TPW, ntiles);
}

// A grid of resident workgroups striding over the tiles (patterns 5, 6).
template <int R, int W, int U, int SP>
__global__ __launch_bounds__(kBlock) void persistent_kernel(Streams s, int64_t ntiles)
{
    run_tiles<R, W, U, SP>(s, blockIdx.x, gridDim.x, ntiles, ntiles);
}

// The fixed cost of a launch, apart: a kernel that touches no memory, and
// kernels that only load or only store one 16-byte vector per lane.
__global__ __launch_bounds__(kBlock) void empty_kernel(int *never)
{
    if (never != nullptr && threadIdx.x == kBlock)  // threadIdx.x < kBlock: never taken
        never[0] = 1;
}

__global__ __launch_bounds__(kBlock) void touch_kernel(const u32x4 *in, u32x4 *out, u32x4 *sink)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (in != nullptr) {
        const u32x4 v = __builtin_nontemporal_load(in + i);
        if (v.x == 0x9E3779B9u && v.y == 0x7F4A7C15u && v.z == 0xF39CC060u)
            sink[0] = v;  // keeps the load alive
    } else {
        const u32x4 v = {(unsigned)i, 1u, 2u, 3u};
        __builtin_nontemporal_store(v, out + i);
    }
}

constexpr int kPatterns = 10;

template <int R, int W>
hipError_t launch(int pattern, const Streams &s, int64_t vectors, hipStream_t st)
{
    const dim3 block(kBlock);
    auto one = [&](auto kern, int U) -> hipError_t {
        const int64_t ntiles = vectors / (kBlock * U);
        kern<<<dim3((unsigned)ntiles), block, 0, st>>>(s, ntiles);
        return hipGetLastError();
    };
    auto multi = [&](auto kern, int U, int tpw) -> hipError_t {
        const int64_t ntiles = vectors / (kBlock * U);
        kern<<<dim3((unsigned)((ntiles + tpw - 1) / tpw)), block, 0, st>>>(s, ntiles);
        return hipGetLastError();
    };
    auto persist = [&](auto kern, int U) -> hipError_t {
        const int64_t ntiles = vectors / (kBlock * U);
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, 0);
        if (e != hipSuccess)
            return e;
        int64_t grid = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
        if (grid > ntiles)
            grid = ntiles;
        kern<<<dim3((unsigned)grid), block, 0, st>>>(s, ntiles);
        return hipGetLastError();
    };
    switch (pattern) {
    case 0: return one(one_tile_kernel<R, W, 4, kNT>, 4);
    case 1: return one(one_tile_kernel<R, W, 2, kNT>, 2);
    case 2: return one(one_tile_kernel<R, W, 1, kNT>, 1);
    case 3: return multi(multi_tile_kernel<R, W, 4, 2>, 4, 2);
    case 4: return multi(multi_tile_kernel<R, W, 2, 4>, 2, 4);
    case 5: return persist(persistent_kernel<R, W, 2, kNT>, 2);
    case 6: return persist(persistent_kernel<R, W, 2, kWB>, 2);
    case 7: return one(one_tile_kernel<R, W, 4, kWB>, 4);
    case 8: return one(one_tile_kernel<R, W, 4, kWT>, 4);
    case 9: return one(one_tile_kernel<R, W, 2, kWT>, 2);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" {

int calib_patterns(void) { return kPatterns; }

// Streams `vectors` 16-byte vectors (a positive multiple of 1024) through R
// inputs and W outputs in access pattern `pattern` (0..9, listed above), all
// device buffers owned by the caller.  Returns a hipError_t.
int calib_stream_pattern(int pattern, int R, int W, const void *const *in, void *const *out, void *sink,
                         int64_t vectors, void *stream)
{
    if (pattern < 0 || pattern >= kPatterns || R < 0 || R > kMaxStreams || W < 0 || W > kMaxStreams ||
        R + W == 0 || vectors <= 0 || vectors % (kBlock * 4) != 0 || vectors / kBlock > INT32_MAX)
        return (int)hipErrorInvalidValue;
    Streams s{};
    for (int r = 0; r < R; ++r)
        s.in[r] = static_cast<const u32x4 *>(in[r]);
    for (int w = 0; w < W; ++w)
        s.out[w] = static_cast<u32x4 *>(out[w]);
    s.sink = static_cast<u32x4 *>(sink);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
#define RR_CALIB(r, w)                                                   \
    if (R == r && W == w)                                                \
        return (int)launch<r, w>(pattern, s, vectors, st);
    RR_CALIB(1, 0) RR_CALIB(2, 0) RR_CALIB(4, 0)
    RR_CALIB(0, 1)
    RR_CALIB(1, 1) RR_CALIB(2, 1) RR_CALIB(3, 1) RR_CALIB(4, 1)
    RR_CALIB(2, 2)
#undef RR_CALIB
    return (int)hipErrorInvalidValue;
}

// kind 0: `blocks` workgroups that touch no memory; kind 1: each lane loads
// one 16-byte vector of `buf` (blocks * 4 KiB); kind 2: each lane stores one.
int calib_fixed(int kind, int64_t blocks, void *buf, void *sink, void *stream)
{
    if (kind < 0 || kind > 2 || blocks < 1 || blocks > INT32_MAX || (kind > 0 && (buf == nullptr || sink == nullptr)))
        return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const dim3 grid((unsigned)blocks), block(kBlock);
    if (kind == 0)
        empty_kernel<<<grid, block, 0, st>>>(nullptr);
    else if (kind == 1)
        touch_kernel<<<grid, block, 0, st>>>(static_cast<const u32x4 *>(buf), nullptr, static_cast<u32x4 *>(sink));
    else
        touch_kernel<<<grid, block, 0, st>>>(nullptr, static_cast<u32x4 *>(buf), static_cast<u32x4 *>(sink));
    return (int)hipGetLastError();
}

// The relay kernels' pattern (pattern 0).
int calib_stream(int R, int W, const void *const *in, void *const *out, void *sink, int64_t vectors,
                 void *stream)
{
    return calib_stream_pattern(0, R, W, in, out, sink, vectors, stream);
}

}  // extern "C"
