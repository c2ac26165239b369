// reshape_and_cache: store each new token's K and V rows into its pool slot.
//
// Caching the key/value of every processed token is what lets decode skip
// recomputing them (runbyai sections 1-2); with paging, the slot names a
// physical block and an offset inside it (runbyai section 3).  The copy is
// bit for bit: the kernel moves 16-byte words (K) and raw 16-bit or 32-bit
// elements (V) and never converts a value.
//
// One workgroup (256 threads) per (group of 16 consecutive tokens, KV head).
// Tokens are independent -- any slot mapping works -- but the lanes are laid
// out so that when consecutive tokens fill consecutive slots of a block (a
// prompt being written) the stores of a wave land in contiguous runs:
//   K: tile [D/x][16][x]; thread (c, t) copies 16-byte chunk c of token t to
//      tile(t) + (c * 16 + offset(t)) * 16 B -- 16 consecutive offsets form
//      one contiguous run of 16 * 16 B.
//   V: tile [D][16]; the 16 rows go through LDS and thread (t, d) writes
//      element d of token t to tile(t) + d * 16 + offset(t), lanes running
//      over t first -- consecutive offsets of one dim are contiguous.
// A single appended token per sequence (the decode step) gets scattered
// writes whatever the layout; there the launch, not the stores, dominates.
// The stores are non-temporal: the rows are read next by attention, which
// streams the pool from HBM anyway, and dirty lines left in L2 and the
// Infinity Cache were measured to slow the following decode (a step with
// 17k prompt tokens written: decode 241 -> 205 us, step 280 -> 258 us;
// Llama-shaped decode step 108 -> 104 us).
#include "kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTokens = 16;   // tokens per workgroup
constexpr int kThreads = 256;

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                                               const int64_t* __restrict__ slot_mapping,
                                                               E* __restrict__ k_cache, E* __restrict__ v_cache,
                                                               int64_t num_tokens, int num_kv_heads, int64_t num_slots) {
    constexpr int X = 16 / (int)sizeof(E);  // elements per 16-byte chunk
    constexpr int NCH = D / X;              // chunks per row
    constexpr int kRowPad = 16 / (int)sizeof(E);
    __shared__ __align__(16) E vrow[kTokens][D + kRowPad];
    __shared__ int64_t tile_of[kTokens];    // element offset of the token's (block, head) tile, -1 = skip
    __shared__ int off_of[kTokens];

    const int h = blockIdx.x % num_kv_heads;
    const int64_t t0 = (int64_t)(blockIdx.x / num_kv_heads) * kTokens;
    const int tid = threadIdx.x;

    if (tid < kTokens) {
        const int64_t t = t0 + tid;
        int64_t tile = -1;
        int off = 0;
        if (t < num_tokens) {
            const int64_t slot = slot_mapping[t];
            if (slot >= 0 && slot < num_slots) {
                tile = (slot / kBlockSize * num_kv_heads + h) * (int64_t)(D * kBlockSize);
                off = (int)(slot % kBlockSize);
            }
        }
        tile_of[tid] = tile;
        off_of[tid] = off;
    }
    // K chunks of this thread (thread (c, t), t fastest), loaded now: their
    // address does not depend on the slot, so the loads overlap the slot
    // and V loads instead of following the barrier
    constexpr int K_IT = (kTokens * NCH + kThreads - 1) / kThreads;
    uint4 kw[K_IT];
#pragma unroll
    for (int it = 0; it < K_IT; ++it) {
        const int i = tid + it * kThreads;
        const int t = i % kTokens;
        const int c = i / kTokens;
        kw[it] = make_uint4(0, 0, 0, 0);
        if (i < kTokens * NCH && t0 + t < num_tokens)
            kw[it] = reinterpret_cast<const uint4*>(k_new + ((t0 + t) * num_kv_heads + h) * (int64_t)D)[c];
    }
    // V rows into LDS: thread (t, c) reads 16-byte chunk c of token t
    for (int i = tid; i < kTokens * NCH; i += kThreads) {
        const int t = i / NCH;
        const int c = i % NCH;
        if (t0 + t < num_tokens) {
            const uint4 w = reinterpret_cast<const uint4*>(v_new + ((t0 + t) * num_kv_heads + h) * (int64_t)D)[c];
            *reinterpret_cast<uint4*>(&vrow[t][c * X]) = w;
        }
    }
    __syncthreads();

    // K stores
#pragma unroll
    for (int it = 0; it < K_IT; ++it) {
        const int i = tid + it * kThreads;
        if (i >= kTokens * NCH) continue;
        const int t = i % kTokens;
        const int c = i / kTokens;
        const int64_t tile = tile_of[t];
        if (tile < 0) continue;
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, kw[it]),
                                    reinterpret_cast<u32x4_t*>(k_cache + tile) + c * kBlockSize + off_of[t]);
    }
    // V: thread (d, t), t fastest
    for (int i = tid; i < kTokens * D; i += kThreads) {
        const int t = i % kTokens;
        const int d = i / kTokens;
        const int64_t tile = tile_of[t];
        if (tile < 0) continue;
        __builtin_nontemporal_store(vrow[t][d], v_cache + tile + (int64_t)d * kBlockSize + off_of[t]);
    }
}

// fp32 -> OCP E4M3 code: round to nearest (ties to even mantissa), saturate
// at +-448; the sign of zero is kept.  Written out from the format (1 sign,
// 4 exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9) with
// integer operations, so the result is fixed bit for bit.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.f);
    if (a < 0.015625f)                                   // below 2^-6: multiples of 2^-9
        return sign | (uint32_t)__builtin_rintf(a * 512.f);  // exact scaling, rint rounds to even
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = (ab >> 20) & 7u;                  // top 3 mantissa bits
    const uint32_t rem = ab & 0xFFFFFu;                  // the 20 dropped bits
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ? 1u : 0u;
    const uint32_t code = ((((ab >> 23) - 120u) << 3) | r) + up;  // exponent bias 127 -> 7; a carry bumps it
    return sign | (code < 0x7Eu ? code : 0x7Eu);
}

// Quantising cache write: fp8 pools, bf16 or fp32 inputs, one scale per KV
// head for K and for V.  Same thread layout as the copy kernel above; a K
// output chunk now holds 16 dims (16 one-byte codes).
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void cache_write_fp8_kernel(const E* __restrict__ k_new,
                                                                   const E* __restrict__ v_new,
                                                                   const int64_t* __restrict__ slot_mapping,
                                                                   uint8_t* __restrict__ k_cache,
                                                                   uint8_t* __restrict__ v_cache,
                                                                   const float* __restrict__ k_scale,
                                                                   const float* __restrict__ v_scale,
                                                                   int64_t num_tokens, int num_kv_heads,
                                                                   int64_t num_slots) {
    constexpr int NCH = D / 16;                       // 16-dim output chunks per row
    constexpr int kRowPad = 16 / (int)sizeof(E);
    __shared__ __align__(16) E vrow[kTokens][D + kRowPad];
    __shared__ int64_t tile_of[kTokens];
    __shared__ int off_of[kTokens];

    const int h = blockIdx.x % num_kv_heads;
    const int64_t t0 = (int64_t)(blockIdx.x / num_kv_heads) * kTokens;
    const int tid = threadIdx.x;
    const float ks = k_scale[h];
    const float vs = v_scale[h];

    if (tid < kTokens) {
        const int64_t t = t0 + tid;
        int64_t tile = -1;
        int off = 0;
        if (t < num_tokens) {
            const int64_t slot = slot_mapping[t];
            if (slot >= 0 && slot < num_slots) {
                tile = (slot / kBlockSize * num_kv_heads + h) * (int64_t)(D * kBlockSize);
                off = (int)(slot % kBlockSize);
            }
        }
        tile_of[tid] = tile;
        off_of[tid] = off;
    }
    constexpr int X = 16 / (int)sizeof(E);            // input elements per 16-byte load
    // K inputs of this thread (thread (c, t), t fastest: the 16 elements of
    // output chunk c of token t), loaded before the barrier as for bf16
    constexpr int K_IT = (kTokens * NCH + kThreads - 1) / kThreads;
    constexpr int KW = 16 / X;                        // 16-byte loads per output chunk
    uint4 kraw[K_IT][KW];
#pragma unroll
    for (int it = 0; it < K_IT; ++it) {
        const int i = tid + it * kThreads;
        const int t = i % kTokens;
        const int c = i / kTokens;
#pragma unroll
        for (int u = 0; u < KW; ++u) kraw[it][u] = make_uint4(0, 0, 0, 0);
        if (i < kTokens * NCH && t0 + t < num_tokens) {
            const uint4* src = reinterpret_cast<const uint4*>(k_new + ((t0 + t) * num_kv_heads + h) * (int64_t)D + 16 * c);
#pragma unroll
            for (int u = 0; u < KW; ++u) kraw[it][u] = src[u];
        }
    }
    for (int i = tid; i < kTokens * (D / X); i += kThreads) {
        const int t = i / (D / X);
        const int c = i % (D / X);
        if (t0 + t < num_tokens) {
            const uint4 w = reinterpret_cast<const uint4*>(v_new + ((t0 + t) * num_kv_heads + h) * (int64_t)D)[c];
            *reinterpret_cast<uint4*>(&vrow[t][c * X]) = w;
        }
    }
    __syncthreads();

    auto to_f32 = [](E e) -> float {
        if constexpr (sizeof(E) == 2) return __uint_as_float((uint32_t)e << 16);
        else return __uint_as_float((uint32_t)e);
    };
    // K: 16 codes of chunk c of token t
#pragma unroll
    for (int it = 0; it < K_IT; ++it) {
        const int i = tid + it * kThreads;
        if (i >= kTokens * NCH) continue;
        const int t = i % kTokens;
        const int c = i / kTokens;
        const int64_t tile = tile_of[t];
        if (tile < 0) continue;
        const E* src = reinterpret_cast<const E*>(kraw[it]);
        uint32_t w[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t b = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) b |= e4m3_rne_sat(to_f32(src[4 * q4 + e]) / ks) << (8 * e);
            w[q4] = b;
        }
        __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]},
                                    reinterpret_cast<u32x4_t*>(k_cache + tile) + c * kBlockSize + off_of[t]);
    }
    // V: thread (d, t), t fastest: one code per (token, dim)
    for (int i = tid; i < kTokens * D; i += kThreads) {
        const int t = i % kTokens;
        const int d = i / kTokens;
        const int64_t tile = tile_of[t];
        if (tile < 0) continue;
        __builtin_nontemporal_store((uint8_t)e4m3_rne_sat(to_f32(vrow[t][d]) / vs),
                                    v_cache + tile + (int64_t)d * kBlockSize + off_of[t]);
    }
}

template <typename E>
hipError_t launch_fp8(const void* k_new, const void* v_new, const int64_t* slots, void* k_cache, void* v_cache,
                      const float* k_scale, const float* v_scale, int64_t num_tokens, int num_kv_heads,
                      int head_dim, int64_t num_blocks, hipStream_t stream) {
    const int64_t groups = (num_tokens + kTokens - 1) / kTokens * num_kv_heads;
    const dim3 grid((unsigned)groups), block(kThreads);
    const int64_t num_slots = num_blocks * kBlockSize;
    const E* kn = static_cast<const E*>(k_new);
    const E* vn = static_cast<const E*>(v_new);
    uint8_t* kc = static_cast<uint8_t*>(k_cache);
    uint8_t* vc = static_cast<uint8_t*>(v_cache);
    if (head_dim == 128)
        hipLaunchKernelGGL((cache_write_fp8_kernel<E, 128>), grid, block, 0, stream, kn, vn, slots, kc, vc, k_scale,
                           v_scale, num_tokens, num_kv_heads, num_slots);
    else
        hipLaunchKernelGGL((cache_write_fp8_kernel<E, 64>), grid, block, 0, stream, kn, vn, slots, kc, vc, k_scale,
                           v_scale, num_tokens, num_kv_heads, num_slots);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_typed(const void* k_new, const void* v_new, const int64_t* slots, void* k_cache, void* v_cache,
                        int64_t num_tokens, int num_kv_heads, int head_dim, int64_t num_blocks, hipStream_t stream) {
    const int64_t groups = (num_tokens + kTokens - 1) / kTokens * num_kv_heads;
    const dim3 grid((unsigned)groups), block(kThreads);
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

hipError_t launch_cache_write_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping, void* k_cache,
                                  void* v_cache, const float* k_scale, const float* v_scale, int64_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, bool src_bf16,
                                  hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    if (src_bf16)
        return launch_fp8<uint16_t>(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, num_tokens,
                                    num_kv_heads, head_dim, num_blocks, stream);
    return launch_fp8<uint32_t>(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, num_tokens,
                                num_kv_heads, head_dim, num_blocks, stream);
}

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
