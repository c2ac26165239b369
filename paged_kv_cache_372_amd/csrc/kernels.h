// Internal interface between the C-ABI layer (pagedkv_abi.hip) and the
// kernel translation units.  Not installed; the public surface is
// include/pagedkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockSize = 16;       // tokens per KV block
constexpr int kMaxPartBlocks = 64;   // blocks per split-K partition (1024 tokens)
constexpr int kMfmaHeadsPerUnit = 16;  // query heads one MFMA decode wave serves (tile width)
constexpr int kValuHeadsPerUnit = 8;   // query heads one VALU decode wave serves (register budget)

// Everything one decode launch needs.  Passed by value as the kernel argument.
struct DecodeParams {
    const void* q;               // [B][Hq][D]
    const void* k_cache;         // [NB][Hkv][D/x][16][x]
    const void* v_cache;         // [NB][Hkv][D][16]
    const int32_t* block_tables; // [B][max_blocks_per_seq]
    const int32_t* context_lens; // [B]
    void* out;                   // [B][Hq][D]
    float* o_part;               // [B][P][Hq][D]   (split only)
    float* m_part;               // [B][P][Hq]      reference max, log2 units
    float* l_part;               // [B][P][Hq]      sum of 2^(s - m)
    float scale_log2;            // scale * log2(e)
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;               // Hq / Hkv
    int32_t heads_per_unit;      // query heads per decode wave
    int32_t n_head_groups;       // ceil(group / heads_per_unit)
    int32_t head_dim;
    int64_t num_blocks;          // pool size; table entries outside it are skipped
    int32_t max_blocks_per_seq;
    int32_t ctx_cap;             // context lengths are clamped to [0, ctx_cap]
    int32_t part_blocks;         // blocks per partition
    int32_t num_parts;           // P = partitions covering ctx_cap
    int32_t out_bf16;            // 1: bf16 output, 0: f32 output
};

// Number of decode work units (one wave each) the partition kernels launch.
inline int64_t decode_units(const DecodeParams& p) {
    return (int64_t)p.num_parts * p.num_seqs * p.n_head_groups * p.num_kv_heads;
}

hipError_t launch_decode_bf16_mfma(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, bool bf16, hipStream_t stream);
hipError_t launch_splitk_reduce(const DecodeParams& p, hipStream_t stream);
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

__device__ __forceinline__ int clamp_ctx(int L, int cap) {
    return L < 0 ? 0 : (L > cap ? cap : L);
}

}  // namespace pkv
