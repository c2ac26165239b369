// Internal interface of the chunked-prefill kernel (prefill_wide.hip) for the
// C-ABI layer.  Kept apart from kernels.h so that the decode and copy code
// does not see it.
#pragma once

#include "kernels.h"

namespace pkv {

// Everything one multi-token-query (chunked prefill) launch needs.
struct PrefillParams {
    const void* q;                  // [T][Hq][D] bf16, requests' rows packed
    const void* k_cache;            // bf16 [NB][Hkv][D/8][16][8]; fp8 [NB][Hkv][D/16][16][16]
    const void* v_cache;            // [NB][Hkv][D][16]
    const int32_t* block_tables;    // [B][max_blocks_per_seq] (this launch's requests)
    const int32_t* context_lens;    // [B]
    const int32_t* query_start_loc; // [B + 1] absolute rows of q / out
    void* out;                      // [T][Hq][D]
    float scale_log2;
    int32_t num_seqs;               // B of this launch
    int32_t num_tokens;             // T of the whole call: rows are clamped to it
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;                  // Hq / Hkv
    int32_t head_dim;
    int64_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t ctx_cap;
    int32_t out_bf16;
    int32_t tile_bound;             // workgroup tiles launched per KV head (>= the tiles needed)
    int32_t kv_fp8;                 // 1: pools hold E4M3 codes
    const float* k_scale;           // fp8: [Hkv] K dequantisation scale
    const float* v_scale;           // fp8: [Hkv] V dequantisation scale
    int32_t lpt_buckets;            // tile weight classes (tiles are taken heaviest first)
    int32_t lpt_shift;              // a weight class is 2^lpt_shift keys
};

// Rows (query token x head of a KV group) one prefill workgroup covers.
constexpr int kPrefillRowsPerGroup = 256;
// LDS for a prefill workgroup's tile order: num_seqs + 3 + lpt_buckets ints.
// With the fp8 kernel's 112 KiB of staging this fills the 160 KiB a
// workgroup may take.
constexpr int kPrefillPlanLdsBytes = 48 * 1024;

size_t prefill_lds_bytes(int32_t num_seqs, int32_t lpt_buckets);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

}  // namespace pkv
