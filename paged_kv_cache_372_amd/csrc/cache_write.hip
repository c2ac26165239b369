// reshape_and_cache: store each new token's K and V rows into its pool slot.
//
// Caching the key/value of every processed token is what lets decode skip
// recomputing them (runbyai sections 1-2); with paging, the slot names a
// physical block and an offset inside it (runbyai section 3).  The copy is
// bit for bit: the kernel moves 16-byte words (K) and raw elements (V) and
// never converts a value.
//
// One wave64 per (token, KV head); four waves per workgroup.
//   K: the D values of the token are D/x 16-byte chunks; chunk c goes to
//      tile + (c * 16 + offset) * x  (one lane per chunk).
//   V: dim d goes to tile + d * 16 + offset (one element per lane and pass).
#include "kernels.h"

namespace pkv {
namespace {

template <typename E, int D>
__global__ __launch_bounds__(256) void cache_write_kernel(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                                          const int64_t* __restrict__ slot_mapping,
                                                          E* __restrict__ k_cache, E* __restrict__ v_cache,
                                                          int64_t num_tokens, int num_kv_heads, int64_t num_slots) {
    constexpr int X = 16 / (int)sizeof(E);
    constexpr int NCH = D / X;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= num_tokens * num_kv_heads) return;
    const int64_t t = w / num_kv_heads;
    const int h = (int)(w % num_kv_heads);
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const int64_t tile = (blk * num_kv_heads + h) * (int64_t)(D * kBlockSize);
    const int64_t row = (t * num_kv_heads + h) * (int64_t)D;

    if (lane < NCH) {
        const uint4 c = reinterpret_cast<const uint4*>(k_new + row)[lane];
        reinterpret_cast<uint4*>(k_cache + tile)[lane * kBlockSize + off] = c;
    }
#pragma unroll
    for (int d = lane; d < D; d += 64) v_cache[tile + (int64_t)d * kBlockSize + off] = v_new[row + d];
}

template <typename E>
hipError_t launch_typed(const void* k_new, const void* v_new, const int64_t* slots, void* k_cache, void* v_cache,
                        int64_t num_tokens, int num_kv_heads, int head_dim, int64_t num_blocks, hipStream_t stream) {
    const int64_t waves = num_tokens * num_kv_heads;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    const int64_t num_slots = num_blocks * kBlockSize;
    const E* kn = static_cast<const E*>(k_new);
    const E* vn = static_cast<const E*>(v_new);
    E* kc = static_cast<E*>(k_cache);
    E* vc = static_cast<E*>(v_cache);
    if (head_dim == 128)
        hipLaunchKernelGGL((cache_write_kernel<E, 128>), grid, block, 0, stream, kn, vn, slots, kc, vc, num_tokens,
                           num_kv_heads, num_slots);
    else
        hipLaunchKernelGGL((cache_write_kernel<E, 64>), grid, block, 0, stream, kn, vn, slots, kc, vc, num_tokens,
                           num_kv_heads, num_slots);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_write(const void* k_new, const void* v_new, const int64_t* slot_mapping, void* k_cache,
                              void* v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int64_t num_blocks, bool bf16, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    if (bf16)
        return launch_typed<uint16_t>(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, head_dim,
                                      num_blocks, stream);
    return launch_typed<uint32_t>(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, head_dim,
                                  num_blocks, stream);
}

}  // namespace pkv
