// Internal interface between the C-ABI layer (pagedkv_abi.hip) and the
// kernel translation units.  Not installed; the public surface is
// include/pagedkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockSize = 16;           // tokens per KV block
constexpr int kMfmaHeadsPerUnit = 16;    // query heads one MFMA decode wave serves (tile width)
constexpr int kValuHeadsPerUnit = 8;     // query heads one VALU decode wave serves (register budget)
constexpr int kMaxWavesPerGroup = 8;     // KV-head waves in one balanced-decode workgroup
constexpr int kMaxSeqsPerLaunch = 4096;  // sequences one balanced-decode launch takes (LDS tables)
constexpr int kMinRangeBlocks = 4;       // shortest range of blocks one workgroup walks


// Everything one decode launch needs.  Passed by value as the kernel argument.
struct DecodeParams {
    const void* q;               // [B][Hq][D]
    const void* k_cache;         // [NB][Hkv][D/x][16][x]
    const void* v_cache;         // [NB][Hkv][D][16]
    const int32_t* block_tables; // [B][max_blocks_per_seq]
    const int32_t* context_lens; // [B]
    void* out;                   // [B][Hq][D]
    float* o_part;               // partial outputs (layout depends on the path, see below)
    float* m_part;               // partial reference max, log2 units
    float* l_part;               // partial sum of 2^(s - m)
    int32_t* seq_off;            // balanced path: [B + 1] first flattened block of each sequence
    float scale_log2;            // scale * log2(e)
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;               // Hq / Hkv
    int32_t n_head_groups;       // ceil(group / heads per wave)
    int32_t head_dim;
    int64_t num_blocks;          // pool size; table entries outside it are skipped
    int32_t max_blocks_per_seq;
    int32_t ctx_cap;             // context lengths are clamped to [0, ctx_cap]
    int32_t out_bf16;            // 1: bf16 output, 0: f32 output
    int32_t cached_kv;           // 1: read K/V with cache-resident loads (blocks shared between sequences)
    int32_t kv_fp8;              // 1: pools hold E4M3 codes (balanced path only)
    const float* k_scale;        // fp8: [Hkv] K dequantisation scale
    const float* v_scale;        // fp8: [Hkv] V dequantisation scale
    // partitioned path (fp32 KV): fixed partitions of part_blocks blocks,
    // partials laid out [B][P][Hq](×D), merged by the reduce kernel
    int32_t part_blocks;
    int32_t num_parts;
    // balanced path (bf16 KV): `walkers` workgroup columns split the
    // flattened block list of all sequences into ranges; partials laid out
    // [2 * ranges][Hq](×D), merged by the reduce kernel
    int32_t walkers;             // workgroups per head-unit group
    int32_t range_cap;           // longest range in blocks (0 = no cap)
    int32_t waves_per_group;     // KV-head waves per workgroup
    int32_t head_units;          // Hkv * n_head_groups
    int32_t head_unit_groups;    // ceil(head_units / waves_per_group)
    int64_t part_bytes;          // bytes of the o_part region (buffer-resource extent)
    // fused append (balanced bf16 path, one head group per KV head): the
    // token each sequence gains this step, [B][Hkv][D], which the wave that
    // walks the sequence's last block writes into position L - 1 of it;
    // null = no append
    const void* k_new;
    const void* v_new;
};

// Split of T flattened blocks into ranges for `walkers` workgroups: each
// range holds `cs` blocks (the last one possibly fewer), `nr` ranges in all.
// Shared by the decode and the reduce so that both see the same ranges.
__host__ __device__ inline void range_geometry(int32_t T, int32_t walkers, int32_t cap, int32_t& cs, int32_t& nr) {
    int32_t c = T > 0 ? (T + walkers - 1) / walkers : 1;
    if (c < kMinRangeBlocks) c = kMinRangeBlocks;
    if (cap > 0 && c > cap) c = cap;
    cs = c;
    nr = T > 0 ? (T + c - 1) / c : 0;
}

// Partial-result row of range r for a sequence whose blocks start at flattened
// offset `first`: slot 0 if the sequence began before the range (the range's
// first piece), slot 1 otherwise (its last piece).
__host__ __device__ inline int32_t range_slot(int32_t r, int32_t cs, int32_t first) {
    return 2 * r + (first < r * cs ? 0 : 1);
}

// Number of decode work units (one wave each) the partitioned kernel launches.
inline int64_t decode_units(const DecodeParams& p) {
    return (int64_t)p.num_parts * p.num_seqs * p.n_head_groups * p.num_kv_heads;
}

// Balanced bf16 decode: dynamic LDS bytes and launch shape.
size_t balanced_lds_bytes(int32_t num_seqs);
const void* balanced_kernel(int32_t head_dim);

hipError_t launch_decode_bf16_balanced(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, bool bf16, hipStream_t stream);
hipError_t launch_splitk_reduce(const DecodeParams& p, bool balanced, hipStream_t stream);
hipError_t launch_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int64_t* pairs,
                              int64_t num_pairs, int64_t num_src_blocks, int64_t num_dst_blocks,
                              int64_t block_bytes, hipStream_t stream);
hipError_t launch_cache_write_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping, void* k_cache,
                                  void* v_cache, const float* k_scale, const float* v_scale, int64_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, bool src_bf16,
                                  hipStream_t stream);
// Issue-rate microbenchmark (issue_rates.hip): pattern 0..6 as
// pkv_issue_rate_bench; one workgroup of 256 x waves_per_simd threads per CU.
hipError_t launch_issue_rate(int32_t pattern, int32_t waves_per_simd, int32_t iters, uint32_t* sink,
                             hipStream_t stream);

hipError_t launch_hbm_read(const void* src, int64_t bytes, const int32_t* tiles, int64_t num_tiles,
                           int32_t tile_bytes, bool streaming, uint32_t* sink, hipStream_t stream);
hipError_t launch_cache_write(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                              void* k_cache, void* v_cache, int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int64_t num_blocks, bool bf16, hipStream_t stream);

// ---------------------------------------------------------------------------
// device helpers shared by the kernels
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f);
}

__device__ __forceinline__ float exp2_fast(float x) {
    // v_exp_f32: 2^x, exp2(-inf) = 0
    return __builtin_amdgcn_exp2f(x);
}

// Reductions over the four lane groups of an MFMA column (lanes l, l^16,
// l^32, l^48) with the gfx950 lane-swap instructions: plain VALU work, no
// LDS traffic, so nothing in the block loop waits on the LDS counter.
__device__ __forceinline__ float max_over_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ int clamp_ctx(int L, int cap) {
    return L < 0 ? 0 : (L > cap ? cap : L);
}

}  // namespace pkv
