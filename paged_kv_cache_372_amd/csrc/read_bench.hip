// Read-only HBM microbenchmark: the plain-read ceiling that the decode's
// KV-read rate is reported beside.
//
// Decode reads every cached key and value of a sequence once per step and is
// bound by memory bandwidth (runbyai section 1); the cache sits in
// fixed-size blocks scattered through one pool (architvora "Paged
// Attention").  This kernel reads bytes and does nothing else with them:
// either a contiguous buffer front to back, or a list of equal tiles at
// arbitrary tile-aligned places in it (one tile per physical block of the
// decode's pool, say).  The rate it reaches is what plain 16-byte loads
// give for that access pattern on the device, with the same choice of
// streaming (non-temporal) or ordinary loads the decode makes.
//
// Work split: the whole read is one list of 16-byte units (unit u of a tile
// list is unit u mod (tile / 16) of tile u / (tile / 16)).  Thread t takes
// units t, t + S, t + 2S, ... with S the number of threads in the grid,
// kInFlight of them per iteration, all loads issued before any is used, so
// neighbouring lanes read neighbouring 16 bytes of one tile.
#include "kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;       // 16-byte loads each thread keeps in flight
constexpr int kGroupsPerCu = 8;    // 8 x 256 threads: 32 waves per compute unit
constexpr int kSinkWords = 1024;   // size of the sink buffer

template <bool kStreaming>
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4_t* __restrict__ src, int64_t units,
                                                            const int32_t* __restrict__ tiles, int tile_shift,
                                                            int64_t num_src_tiles, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t tile_mask = ((int64_t)1 << tile_shift) - 1;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += kInFlight * stride) {
        u32x4_t r[kInFlight];
#pragma unroll
        for (int i = 0; i < kInFlight; ++i) {
            const int64_t v = u + i * stride;
            r[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (v < units) {
                int64_t a = v;
                if (tiles) {
                    const int64_t t = tiles[v >> tile_shift];
                    if (t < 0 || t >= num_src_tiles) continue;  // outside the buffer: not read
                    a = (t << tile_shift) + (v & tile_mask);
                }
                r[i] = kStreaming ? __builtin_nontemporal_load(src + a) : src[a];
            }
        }
#pragma unroll
        for (int i = 0; i < kInFlight; ++i) acc ^= r[i];
    }
    // keeps the loads: a store that (almost) never happens, at a per-lane
    // address
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u)
        sink[(blockIdx.x * kThreads + threadIdx.x) & (kSinkWords - 1)] = 1u;
}

}  // namespace

hipError_t launch_hbm_read(const void* src, int64_t bytes, const int32_t* tiles, int64_t num_tiles,
                           int32_t tile_bytes, bool streaming, uint32_t* sink, hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int shift = 0;
    while ((16 << shift) < tile_bytes) ++shift;
    const int64_t units = tiles ? num_tiles << shift : bytes / 16;
    const int64_t src_tiles = tiles ? bytes / tile_bytes : 0;
    if (units == 0) return hipSuccess;
    const dim3 grid((unsigned)(cus * kGroupsPerCu)), block(kThreads);
    const u32x4_t* s = static_cast<const u32x4_t*>(src);
    if (streaming)
        hipLaunchKernelGGL(hbm_read_kernel<true>, grid, block, 0, stream, s, units, tiles, shift, src_tiles, sink);
    else
        hipLaunchKernelGGL(hbm_read_kernel<false>, grid, block, 0, stream, s, units, tiles, shift, src_tiles, sink);
    return hipGetLastError();
}

}  // namespace pkv
