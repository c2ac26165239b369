// reshape_and_cache: store each new token's K and V rows into its pool slot.
//
// Caching the key/value of every processed token is what lets decode skip
// recomputing them (runbyai sections 1-2); with paging, the slot names a
// physical block and an offset inside it (runbyai section 3).  Into bf16 or
// fp32 pools the copy is bit for bit (16-byte words and raw elements, never
// converted); into fp8 pools each value is encoded to E4M3 with its KV head's
// scale.
//
// Copying kernel (bf16 and fp32 pools).  A run is a stretch of consecutive
// tokens that go to consecutive slots of one block (a prompt being written is
// a chain of runs, one per block; a decode step's single token per sequence
// is a run of one); it holds at most 16 tokens.  The workgroup of (16
// consecutive tokens, KV head) writes every run that starts among its 16
// tokens, so it reads a window of 32; any slot mapping works, and no token is
// written twice.  A run then lands as whole pieces of its block's tile:
//   K: tile [D/x][16][x] (x elements per 16 bytes); thread (c, t) copies
//      16-byte chunk c of token t to tile + (c * 16 + offset(t)) * 16 B, lanes
//      over t first -- a full run writes 16 * 16 B in one piece per chunk.
//   V: tile [D][16]; the rows go through LDS, and a V unit -- the tokens of a
//      run inside one 16-byte piece of a dim's 16-token row (8 bf16 or 4 fp32
//      elements) -- is one store when it fills the piece, element stores
//      otherwise.  Thread (d, unit), units first: a full bf16 run writes its
//      tile's V as one contiguous 4 KiB.
// Against one workgroup per 16 tokens writing each V element on its own:
// 38 against 46 us for a continuous-batching step's 17k prompt tokens, 18
// against 20 us for 8,192 chunked-prefill tokens.
// The stores are non-temporal: the rows are read next by attention, which
// streams the pool from HBM anyway, and dirty lines left in L2 and the
// Infinity Cache were measured to slow the following decode (a step with
// 17k prompt tokens written: decode 241 -> 205 us, step 280 -> 258 us;
// Llama-shaped decode step 108 -> 104 us).
#include "e4m3.h"
#include "kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTokens = 16;            // run starts per workgroup
constexpr int kWindow = 2 * kTokens;   // tokens a workgroup may write
constexpr int kThreads = 256;

// Copying cache write (bf16 or fp32 pools): one workgroup per (16
// consecutive tokens, KV head), writing the runs that start among them.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                                               const int64_t* __restrict__ slot_mapping,
                                                               E* __restrict__ k_cache, E* __restrict__ v_cache,
                                                               int64_t num_tokens, int num_kv_heads, int64_t num_slots) {
    constexpr int X = 16 / (int)sizeof(E);  // elements per 16 bytes: K chunk width, V unit length
    constexpr int NCH = D / X;              // K chunks per token
    __shared__ __align__(16) E vrow[kWindow][D + X];
    __shared__ int64_t tile_of[kWindow];    // element offset of the token's (block, head) tile; -1: not ours
    __shared__ int off_of[kWindow];
    __shared__ int unit_of[kWindow];        // V units: first window position | length << 8
    __shared__ int n_units;                 // unit count | log2 of its power-of-two round-up << 8

    const int h = blockIdx.x % num_kv_heads;
    const int64_t t0 = (int64_t)(blockIdx.x / num_kv_heads) * kTokens;
    const int tid = threadIdx.x;

    // ---- loads of the whole window go out before the slots are read (their
    // addresses need none).  A token of the window that belongs to a
    // neighbour's run is loaded too and not stored.  K: thread (c, j) keeps
    // chunk c of token j (j fastest); V rows into LDS.
    constexpr int K_IT = (kWindow * NCH + kThreads - 1) / kThreads;
    uint4 kraw[K_IT] = {};
#pragma unroll
    for (int it = 0; it < K_IT; ++it) {
        const int i = tid + it * kThreads;
        const int j = i % kWindow;
        const int c = i / kWindow;
        if (i < kWindow * NCH && t0 + j < num_tokens)
            kraw[it] = reinterpret_cast<const uint4*>(k_new + ((t0 + j) * num_kv_heads + h) * (int64_t)D)[c];
    }
    for (int i = tid; i < kWindow * NCH; i += kThreads) {
        const int j = i / NCH;
        const int c = i % NCH;
        if (t0 + j < num_tokens)
            *reinterpret_cast<uint4*>(&vrow[j][c * X]) =
                reinterpret_cast<const uint4*>(v_new + ((t0 + j) * num_kv_heads + h) * (int64_t)D)[c];
    }

    // ---- which tokens of the window [t0, t0 + 32) are this workgroup's, and
    // its V units (wave 0; lane i looks at token t0 - 1 + i, position i - 1)
    if (tid < 64) {
        const int64_t t = t0 - 1 + tid;
        int64_t slot = -1;
        if (tid <= kWindow && t >= 0 && t < num_tokens) {
            const int64_t sl = slot_mapping[t];
            if (sl >= 0 && sl < num_slots) slot = sl;
        }
        const int lo = __shfl_up((int)(uint32_t)slot, 1), hi = __shfl_up((int)(slot >> 32), 1);
        const int64_t prev = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);  // lane i - 1's slot
        const bool valid = slot >= 0;
        // token continues the run of the token before it
        const bool cont = tid > 0 && valid && prev >= 0 && slot == prev + 1 && slot % kBlockSize != 0;
        const uint64_t V = __ballot(valid), C = __ballot(cont);
        const uint64_t A = __ballot(valid && slot % X == 0);  // first slot of a 16-byte piece
        // positions 0 .. p - 1 continue a run that began before t0 (the
        // previous workgroup's; a run holds at most 16 tokens, so p <= 15)
        const int p = __builtin_ctzll(~(C >> 1));
        uint64_t O = V & (((1ull << 17) - 1) & ~((1ull << (p + 1)) - 1));  // lanes p + 1 .. 16: positions p .. 15
        // a run that is ours at position 15 may go on to position 30
        if ((O >> 16) & 1ull) {
            const int q = __builtin_ctzll(~(C >> 17));  // continuations at positions 16 .. 15 + q
            O |= ((1ull << q) - 1) << 17;
        }
        // V units start at a run start or at the first slot of a piece
        const uint64_t S = O & (~C | A);
        const bool mine = (O >> tid) & 1ull;
        if (tid >= 1 && tid <= kWindow) {
            const int j = tid - 1;
            tile_of[j] = mine ? (slot / kBlockSize * num_kv_heads + h) * (int64_t)(D * kBlockSize) : -1;
            off_of[j] = mine ? (int)(slot % kBlockSize) : 0;
        }
        if ((S >> tid) & 1ull) {
            const uint64_t ends = (S | ~O) >> (tid + 1);  // the next unit start, or the end of our tokens
            const int len = ends ? __builtin_ctzll(ends) + 1 : 64 - tid;
            unit_of[__builtin_popcountll(S & ((1ull << tid) - 1))] = (tid - 1) | (len << 8);
        }
        if (tid == 0) {
            // unit count and the log2 of its round-up to a power of two (V
            // items split into (dim, unit) with shifts)
            const int nu = __builtin_popcountll(S);
            n_units = nu | ((nu > 1 ? 32 - __builtin_clz(nu - 1) : 0) << 8);
        }
    }
    __syncthreads();

    // ---- K: chunk c of token j
#pragma unroll
    for (int it = 0; it < K_IT; ++it) {
        const int i = tid + it * kThreads;
        if (i >= kWindow * NCH) continue;
        const int j = i % kWindow;
        const int c = i / kWindow;
        const int64_t tile = tile_of[j];
        if (tile < 0) continue;
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, kraw[it]),
                                    reinterpret_cast<u32x4_t*>(k_cache + tile) + c * kBlockSize + off_of[j]);
    }
    // ---- V: unit u of dim d (units first)
    const int nu = n_units & 0xff, lg = n_units >> 8;
    for (int i = tid; i < (D << lg); i += kThreads) {
        const int u = i & ((1 << lg) - 1);
        const int d = i >> lg;
        if (u >= nu) continue;
        const int j = unit_of[u] & 0xff;
        const int len = unit_of[u] >> 8;
        E* const dst = v_cache + tile_of[j] + (int64_t)d * kBlockSize + off_of[j];
        if (len == X) {
            // a whole 16-byte piece (it then starts on a piece boundary)
            E e[X];
#pragma unroll
            for (int k = 0; k < X; ++k) e[k] = vrow[j + k][d];
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, e), reinterpret_cast<u32x4_t*>(dst));
        } else {
            for (int k = 0; k < len; ++k) __builtin_nontemporal_store(vrow[j + k][d], dst + k);
        }
    }
}

// Quantising cache write: fp8 pools, bf16 or fp32 inputs, one scale per KV
// head for K and for V.  One workgroup per (16 consecutive tokens, KV head)
// writes every token of its group: thread (c, t), t fastest, encodes the 16
// codes of K chunk c of token t, thread (d, t) one V code.  Here the encoding
// (a correctly rounded division and the E4M3 rounding per value) is the
// costly part, and this layout keeps whole waves busy with it; the run
// layout of the copy kernel, with its extra reads and idle lanes, measured
// slower for fp8 pools.
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

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t_last = num_tokens - 1;  // launched for num_tokens >= 1
    // ---- every load goes out before any is waited for: the slots (wave 0,
    // lane t: token t0 + t), then the K and V rows.  Tokens past the last one
    // read the last one again and are not stored; so are the clamped chunks of
    // threads with no K chunk of their own.
    int64_t slot_in = -1;
    if (wave == 0) slot_in = slot_mapping[t0 + tid < t_last ? t0 + tid : t_last];
    constexpr int X = 16 / (int)sizeof(E);            // input elements per 16-byte load
    // K inputs of this thread (thread (c, t), t fastest: the 16 elements of
    // output chunk c of token t)
    constexpr int K_IT = (kTokens * NCH + kThreads - 1) / kThreads;
    constexpr int KW = 16 / X;                        // 16-byte loads per output chunk
    uint4 kraw[K_IT][KW];
#pragma unroll
    for (int it = 0; it < K_IT; ++it) {
        const int i = tid + it * kThreads;
        const int64_t t = t0 + i % kTokens < t_last ? t0 + i % kTokens : t_last;
        const int c = i / kTokens < NCH ? i / kTokens : NCH - 1;
        const uint4* src = reinterpret_cast<const uint4*>(k_new + (t * num_kv_heads + h) * (int64_t)D + 16 * c);
#pragma unroll
        for (int u = 0; u < KW; ++u) kraw[it][u] = src[u];
    }
    // V rows: 16-byte pieces, thread i takes piece i % (D / X) of token i / (D / X)
    constexpr int V_PIECES = kTokens * (D / X);
    constexpr int V_IT = (V_PIECES + kThreads - 1) / kThreads;
    uint4 vraw[V_IT];
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
        const int i = (tid + it * kThreads) < V_PIECES ? tid + it * kThreads : V_PIECES - 1;
        const int64_t t = t0 + i / (D / X) < t_last ? t0 + i / (D / X) : t_last;
        vraw[it] = reinterpret_cast<const uint4*>(v_new + (t * num_kv_heads + h) * (int64_t)D)[i % (D / X)];
    }
    if (wave == 0 && tid < kTokens) {
        int64_t tile = -1;
        int off = 0;
        if (t0 + tid < num_tokens && slot_in >= 0 && slot_in < num_slots) {
            tile = (slot_in / kBlockSize * num_kv_heads + h) * (int64_t)(D * kBlockSize);
            off = (int)(slot_in % kBlockSize);
        }
        tile_of[tid] = tile;
        off_of[tid] = off;
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
        const int i = tid + it * kThreads;
        if (i < V_PIECES) *reinterpret_cast<uint4*>(&vrow[i / (D / X)][(i % (D / X)) * X]) = vraw[it];
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
            for (int e = 0; e < 4; ++e) b |= e4m3_encode(to_f32(src[4 * q4 + e]), ks) << (8 * e);
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
        __builtin_nontemporal_store((uint8_t)e4m3_encode(to_f32(vrow[t][d]), vs),
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
