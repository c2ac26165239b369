// C-ABI layer of libpagedkv.so: argument checks, workspace carving, launch
// selection.  Declarations and the contract of every entry point are in
// include/pagedkv.h.  Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/pagedkv.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

pkv_status fail(pkv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

pkv_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return PKV_OK;
    return fail(PKV_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool dtype_ok(pkv_dtype d) { return d == PKV_F32 || d == PKV_BF16; }

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Effective context cap: lengths are clamped to what the tables can address.
int32_t context_cap(int32_t max_context_len, int32_t max_blocks_per_seq, int32_t block_size) {
    const int64_t by_table = (int64_t)max_blocks_per_seq * block_size;
    return (int32_t)(max_context_len < by_table ? max_context_len : by_table);
}

int32_t auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
    (void)num_seqs;
    (void)num_kv_heads;
    const int32_t bs = pkv::kBlockSize;
    const int32_t cap = pkv::kMaxPartBlocks * bs;
    if (max_context_len <= 0) return bs;
    if (max_context_len <= cap) return ceil_div(max_context_len, bs) * bs;  // one partition, no reduce
    // the waves of a decode workgroup split a partition's blocks among
    // themselves, so long partitions keep every wave busy with few partials
    return cap;
}

struct Resolved {
    int32_t part_tokens;
    int32_t num_parts;
    int32_t ctx_cap;
    size_t workspace;
};

pkv_status resolve(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, Resolved* r) {
    if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (num_q_heads <= 0 || num_kv_heads <= 0)
        return fail(PKV_ERR_INVALID_ARG, "head counts must be positive (q %d, kv %d)", num_q_heads, num_kv_heads);
    if (num_q_heads % num_kv_heads)
        return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", num_q_heads,
                    num_kv_heads);
    if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size != pkv::kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
    if (max_blocks_per_seq < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and max_context_len must be >= 0");
    if (partition_size != 0 &&
        (partition_size < block_size || partition_size > pkv::kMaxPartBlocks * block_size || partition_size % block_size))
        return fail(PKV_ERR_UNSUPPORTED, "partition_size %d: 0 or a multiple of %d in [%d, %d]", partition_size,
                    block_size, block_size, pkv::kMaxPartBlocks * block_size);
    // partition count and workspace depend on max_context_len only, so the
    // workspace query agrees with every decode call of the same sizes
    const int32_t pt = partition_size ? partition_size : auto_partition(num_seqs, num_kv_heads, max_context_len);
    r->part_tokens = pt;
    r->ctx_cap = context_cap(max_context_len, max_blocks_per_seq, block_size);
    r->num_parts = max_context_len > 0 ? ceil_div(max_context_len, pt) : 1;
    r->workspace = r->num_parts > 1 ? (size_t)num_seqs * num_q_heads * r->num_parts * (head_dim + 2) * sizeof(float) : 0;
    return PKV_OK;
}

pkv_status build_params(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
                        size_t workspace_bytes, pkv_dtype kv_dtype, pkv_dtype out_dtype, pkv::DecodeParams* p,
                        Resolved* r) {
    pkv_status st = resolve(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            max_context_len, partition_size, r);
    if (st != PKV_OK) return st;
    if (!dtype_ok(kv_dtype) || !dtype_ok(out_dtype)) return fail(PKV_ERR_UNSUPPORTED, "unknown dtype");
    if (num_seqs > 0 && (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out))
        return fail(PKV_ERR_INVALID_ARG, "null tensor pointer");
    if (num_blocks <= 0 && num_seqs > 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive");
    if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) % 16)
        return fail(PKV_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (!isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
    if (r->workspace > 0) {
        if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", r->workspace);
        if (workspace_bytes < r->workspace)
            return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", r->workspace, workspace_bytes);
        if (((uintptr_t)workspace) % 256) return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    const int32_t group = num_q_heads / num_kv_heads;
    p->q = q;
    p->k_cache = k_cache;
    p->v_cache = v_cache;
    p->block_tables = block_tables;
    p->context_lens = context_lens;
    p->out = out;
    const size_t rows = (size_t)num_seqs * num_q_heads * r->num_parts;
    float* ws = static_cast<float*>(workspace);
    p->o_part = r->workspace ? ws : nullptr;
    p->m_part = r->workspace ? ws + rows * head_dim : nullptr;
    p->l_part = r->workspace ? ws + rows * (head_dim + 1) : nullptr;
    p->scale_log2 = (float)((double)scale * 1.4426950408889634);
    p->num_seqs = num_seqs;
    p->num_q_heads = num_q_heads;
    p->num_kv_heads = num_kv_heads;
    p->group = group;
    p->heads_per_unit = kv_dtype == PKV_BF16 ? pkv::kMfmaHeadsPerUnit : pkv::kValuHeadsPerUnit;
    p->n_head_groups = (group + p->heads_per_unit - 1) / p->heads_per_unit;
    p->head_dim = head_dim;
    p->num_blocks = num_blocks;
    p->max_blocks_per_seq = max_blocks_per_seq;
    p->ctx_cap = r->ctx_cap;
    p->part_blocks = r->part_tokens / block_size;
    p->num_parts = r->num_parts;
    p->out_bf16 = out_dtype == PKV_BF16;
    return PKV_OK;
}

pkv_status run_partitions(const pkv::DecodeParams& p, pkv_dtype kv_dtype, hipStream_t stream) {
    if (p.num_seqs == 0) return PKV_OK;
    hipError_t e = kv_dtype == PKV_BF16 ? pkv::launch_decode_bf16_mfma(p, stream)
                                        : pkv::launch_decode_valu(p, false, stream);
    return from_hip(e, "decode partition kernel launch");
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return 1; }

const char* pkv_status_string(pkv_status status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_INVALID_ARG: return "invalid argument";
        case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case PKV_ERR_WORKSPACE: return "workspace missing or too small";
        case PKV_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error; }

pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, const int64_t* slot_mapping, void* k_cache,
                                 void* v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, pkv_dtype dtype, void* stream) {
    g_last_error[0] = 0;
    if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
    if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size != pkv::kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
    if (!dtype_ok(dtype)) return fail(PKV_ERR_UNSUPPORTED, "unknown dtype");
    if (num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive");
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return fail(PKV_ERR_INVALID_ARG, "null pointer");
    if ((uintptr_t)k_new % 16 || (uintptr_t)k_cache % 16)
        return fail(PKV_ERR_INVALID_ARG, "k_new and k_cache must be 16-byte aligned");
    return from_hip(pkv::launch_cache_write(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads,
                                            head_dim, num_blocks, dtype == PKV_BF16, static_cast<hipStream_t>(stream)),
                    "reshape_and_cache launch");
}

int32_t pkv_decode_auto_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_context_len) {
    (void)num_q_heads;
    (void)head_dim;
    return auto_partition(num_seqs, num_kv_heads > 0 ? num_kv_heads : 1, max_context_len);
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size) {
    Resolved r;
    const int32_t blocks = ceil_div(max_context_len > 0 ? max_context_len : 0, pkv::kBlockSize);
    if (resolve(num_seqs, num_q_heads, num_kv_heads, head_dim, pkv::kBlockSize, blocks, max_context_len,
                partition_size, &r) != PKV_OK)
        return 0;
    return r.workspace;
}

pkv_status pkv_paged_attention_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                                 void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                                 pkv_dtype kv_dtype, pkv_dtype out_dtype, void* stream) {
    g_last_error[0] = 0;
    pkv::DecodeParams p;
    Resolved r;
    pkv_status st = build_params(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                                 num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                                 partition_size, workspace, workspace_bytes, kv_dtype, out_dtype, &p, &r);
    if (st != PKV_OK) return st;
    return run_partitions(p, kv_dtype, static_cast<hipStream_t>(stream));
}

pkv_status pkv_paged_attention_decode_reduce(const int32_t* context_lens, void* out, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                                             int32_t partition_size, void* workspace, size_t workspace_bytes,
                                             pkv_dtype out_dtype, void* stream) {
    g_last_error[0] = 0;
    pkv::DecodeParams p;
    Resolved r;
    // the reduce reads only lengths, partials and out; the K/V/q/table
    // pointers are not used, so stand-ins keep the shared checks happy
    const void* unused = context_lens;
    pkv_status st = build_params(unused, unused, unused, context_lens, context_lens, 1.0f, out, num_seqs, num_q_heads,
                                 num_kv_heads, head_dim, block_size, 1, max_blocks_per_seq, max_context_len,
                                 partition_size, workspace, workspace_bytes, PKV_BF16, out_dtype, &p, &r);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return PKV_OK;
    return from_hip(pkv::launch_splitk_reduce(p, static_cast<hipStream_t>(stream)), "split-K reduce launch");
}

pkv_status pkv_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                                      int32_t max_context_len, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_dtype kv_dtype, pkv_dtype out_dtype, void* stream) {
    g_last_error[0] = 0;
    pkv::DecodeParams p;
    Resolved r;
    pkv_status st = build_params(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                                 num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                                 partition_size, workspace, workspace_bytes, kv_dtype, out_dtype, &p, &r);
    if (st != PKV_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_partitions(p, kv_dtype, s);
    if (st != PKV_OK || p.num_parts <= 1 || num_seqs == 0) return st;
    return from_hip(pkv::launch_splitk_reduce(p, s), "split-K reduce launch");
}

}  // extern "C"
