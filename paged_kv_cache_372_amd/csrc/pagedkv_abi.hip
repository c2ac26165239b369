// C-ABI layer of libpagedkv.so: argument checks, launch planning, workspace
// carving.  Declarations and the contract of every entry point are in
// include/pagedkv.h.  Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/pagedkv.h"
#include "kernels.h"
#include "prefill.h"

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
bool kv_dtype_ok(pkv_dtype d) { return d == PKV_F32 || d == PKV_BF16 || d == PKV_FP8_E4M3; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int32_t kMaxPartitionTokens = 1 << 24;
constexpr int32_t kValuAutoPartition = 1024;  // fp32 path: automatic partition length (tokens)

// Workgroups of the balanced decode that fit on the current device at once.
int64_t resident_groups(int32_t head_dim, int32_t waves_per_group, int32_t seqs_per_launch) {
    int dev = 0, cus = 0, per_cu = 0;
    const size_t lds = pkv::balanced_lds_bytes(seqs_per_launch);
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pkv::balanced_kernel(head_dim), 64 * waves_per_group,
                                                     lds) != hipSuccess ||
        per_cu <= 0) {
        (void)hipGetLastError();  // no usable device: plan for a 256-CU part, two waves per SIMD
        cus = 256;
        per_cu = waves_per_group >= pkv::kMaxWavesPerGroup ? 1 : pkv::kMaxWavesPerGroup / waves_per_group;  // 8 waves per CU
    }
    return (int64_t)cus * per_cu;
}

// How one decode call is carried out.
struct Plan {
    bool balanced;       // bf16 KV: balanced ranges; fp32 KV: fixed partitions
    int32_t ctx_cap;     // context lengths are clamped to this
    int32_t group;
    int32_t n_head_groups;
    // partitioned path
    int32_t part_tokens;
    int32_t num_parts;
    // balanced path
    int32_t chunk_seqs;  // sequences per launch
    int32_t num_chunks;
    int32_t walkers;
    int32_t waves_per_group;
    int32_t head_units;
    int32_t head_unit_groups;
    int32_t range_cap;   // blocks
    int64_t max_ranges;  // per launch
    size_t off_bytes;    // per-launch offset table
    size_t chunk_bytes;  // per-launch workspace
    size_t workspace;    // whole call
};

pkv_status make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size,
                     pkv_dtype kv_dtype, Plan* pl) {
    if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (num_q_heads <= 0 || num_kv_heads <= 0)
        return fail(PKV_ERR_INVALID_ARG, "head counts must be positive (q %d, kv %d)", num_q_heads, num_kv_heads);
    if (num_q_heads % num_kv_heads)
        return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", num_q_heads,
                    num_kv_heads);
    if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size != pkv::kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
    if (!kv_dtype_ok(kv_dtype)) return fail(PKV_ERR_UNSUPPORTED, "unknown KV dtype");
    if (max_blocks_per_seq < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and max_context_len must be >= 0");
    if (partition_size != 0 &&
        (partition_size < block_size || partition_size > kMaxPartitionTokens || partition_size % block_size))
        return fail(PKV_ERR_UNSUPPORTED, "partition_size %d: 0 or a multiple of %d in [%d, %d]", partition_size,
                    block_size, block_size, kMaxPartitionTokens);
    memset(pl, 0, sizeof(*pl));
    const int64_t by_table = (int64_t)max_blocks_per_seq * block_size;
    pl->ctx_cap = (int32_t)(max_context_len < by_table ? max_context_len : by_table);
    pl->group = num_q_heads / num_kv_heads;
    pl->balanced = kv_dtype != PKV_F32;  // bf16 and fp8 caches
    const int32_t heads_per_wave = pl->balanced ? pkv::kMfmaHeadsPerUnit : pkv::kValuHeadsPerUnit;
    pl->n_head_groups = (int32_t)ceil_div(pl->group, heads_per_wave);
    if (!pl->balanced) {
        // partition count and workspace depend on max_context_len only, so the
        // workspace query agrees with every decode call of the same sizes
        int32_t pt = partition_size;
        if (!pt) pt = max_context_len <= kValuAutoPartition ? (int32_t)(ceil_div(max_context_len, block_size) * block_size)
                                                            : kValuAutoPartition;
        if (pt <= 0) pt = block_size;
        pl->part_tokens = pt;
        pl->num_parts = max_context_len > 0 ? (int32_t)ceil_div(max_context_len, pt) : 1;
        pl->workspace =
            pl->num_parts > 1 ? (size_t)num_seqs * num_q_heads * pl->num_parts * (head_dim + 2) * sizeof(float) : 0;
        return PKV_OK;
    }
    pl->chunk_seqs = num_seqs < pkv::kMaxSeqsPerLaunch ? num_seqs : pkv::kMaxSeqsPerLaunch;
    pl->num_chunks = num_seqs > 0 ? (int32_t)ceil_div(num_seqs, pl->chunk_seqs) : 0;
    pl->head_units = num_kv_heads * pl->n_head_groups;

    // Up to eight KV-head waves per workgroup, one workgroup per compute
    // unit, kept in lockstep by the kernel (a barrier per round of blocks).
    pl->waves_per_group = pl->head_units < pkv::kMaxWavesPerGroup ? pl->head_units : pkv::kMaxWavesPerGroup;
    pl->head_unit_groups = (int32_t)ceil_div(pl->head_units, pl->waves_per_group);
    const int64_t slots = resident_groups(head_dim, pl->waves_per_group, pl->chunk_seqs > 0 ? pl->chunk_seqs : 1);
    const int64_t w = slots / pl->head_unit_groups;
    pl->walkers = (int32_t)(w < 1 ? 1 : (w > (1 << 20) ? (1 << 20) : w));
    pl->range_cap = partition_size / block_size;
    const int64_t t_max = (int64_t)pl->chunk_seqs * ceil_div(pl->ctx_cap, block_size);
    if (t_max >= (int64_t)1 << 30)
        return fail(PKV_ERR_UNSUPPORTED, "%d sequences of up to %d tokens: too many blocks for one launch",
                    pl->chunk_seqs, pl->ctx_cap);
    int64_t nr = pl->walkers;
    if (pl->range_cap > 0 && ceil_div(t_max, pl->range_cap) > nr) nr = ceil_div(t_max, pl->range_cap);
    pl->max_ranges = nr;
    if ((int64_t)(2 * nr) * num_q_heads * head_dim * (int64_t)sizeof(float) >= ((int64_t)1 << 31))
        return fail(PKV_ERR_UNSUPPORTED, "partial results of %lld ranges x %d heads exceed 2 GiB", (long long)nr,
                    num_q_heads);
    pl->off_bytes = align_up((size_t)(pl->chunk_seqs + 1) * sizeof(int32_t), 256);
    pl->chunk_bytes =
        align_up(pl->off_bytes + (size_t)(2 * nr) * num_q_heads * (head_dim + 2) * sizeof(float), 256);
    pl->workspace = num_seqs > 0 ? pl->chunk_bytes * pl->num_chunks : 0;
    return PKV_OK;
}

// The arguments of one decode call, checked.
struct Call {
    Plan plan;
    pkv::DecodeParams base;
    pkv_dtype kv_dtype;
    size_t q_row_bytes;    // bytes of q per sequence
    size_t out_row_bytes;  // bytes of out per sequence
    size_t new_row_bytes;  // fused append: bytes of k_new / v_new per sequence
    char* workspace;
};

// Point a checked call at its workspace (the balanced path carves it per
// launch in chunk_params; the partitioned path keeps its partials here).
void bind_workspace(Call* c, void* workspace) {
    const Plan& pl = c->plan;
    pkv::DecodeParams& p = c->base;
    c->workspace = static_cast<char*>(workspace);
    if (!pl.balanced) {
        float* ws = static_cast<float*>(workspace);
        const size_t rows = (size_t)p.num_seqs * p.num_q_heads * pl.num_parts;
        p.o_part = pl.workspace ? ws : nullptr;
        p.m_part = pl.workspace ? ws + rows * p.head_dim : nullptr;
        p.l_part = pl.workspace ? ws + rows * (p.head_dim + 1) : nullptr;
    }
}

pkv_status prepare(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                   const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
                   size_t workspace_bytes, pkv_dtype kv_dtype, pkv_dtype out_dtype, uint32_t flags,
                   const float* k_scale, const float* v_scale, Call* c) {
    pkv_status st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              max_context_len, partition_size, kv_dtype, &c->plan);
    if (st != PKV_OK) return st;
    const Plan& pl = c->plan;
    if (!dtype_ok(out_dtype)) return fail(PKV_ERR_UNSUPPORTED, "unknown output dtype");
    if (flags & ~(uint32_t)PKV_DECODE_SHARED_BLOCKS) return fail(PKV_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
    if (num_seqs > 0 && (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out))
        return fail(PKV_ERR_INVALID_ARG, "null tensor pointer");
    if (num_blocks <= 0 && num_seqs > 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive");
    if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) % 16)
        return fail(PKV_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (!isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
    if (pl.workspace > 0) {
        if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", pl.workspace);
        if (workspace_bytes < pl.workspace)
            return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", pl.workspace, workspace_bytes);
        if (((uintptr_t)workspace) % 256) return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    pkv::DecodeParams& p = c->base;
    memset(&p, 0, sizeof(p));
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.out = out;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = pl.group;
    p.n_head_groups = pl.n_head_groups;
    p.head_dim = head_dim;
    p.num_blocks = num_blocks;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.ctx_cap = pl.ctx_cap;
    p.out_bf16 = out_dtype == PKV_BF16;
    p.cached_kv = (flags & PKV_DECODE_SHARED_BLOCKS) ? 1 : 0;
    p.kv_fp8 = kv_dtype == PKV_FP8_E4M3;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    if (pl.balanced) {
        p.walkers = pl.walkers;
        p.range_cap = pl.range_cap;
        p.waves_per_group = pl.waves_per_group;
        p.head_units = pl.head_units;
        p.head_unit_groups = pl.head_unit_groups;
        if (p.cached_kv) {
            // Blocks shared by several sequences: one wave per workgroup, so
            // that workgroup i serves head unit i mod head_units.  Workgroups
            // go to the 8 XCDs in turn (i mod 8), so with 8 KV heads each
            // XCD reads one head's tiles and its L2 keeps that head's shared
            // blocks (a 2048-token prefix: 1 MiB of K and V per head) for
            // every sequence that reads them.  The ranges, and so the
            // partials and the reduce, stay those of the plan.
            p.waves_per_group = 1;
            p.head_unit_groups = pl.head_units;
        }
        p.part_bytes = (int64_t)(2 * pl.max_ranges) * num_q_heads * head_dim * (int64_t)sizeof(float);
    } else {
        p.part_blocks = pl.part_tokens / block_size;
        p.num_parts = pl.num_parts;
    }
    c->kv_dtype = kv_dtype;
    c->q_row_bytes = (size_t)num_q_heads * head_dim * (kv_dtype == PKV_F32 ? 4 : 2);  // q is bf16 for fp8 caches
    c->out_row_bytes = (size_t)num_q_heads * head_dim * (out_dtype == PKV_BF16 ? 2 : 4);
    c->new_row_bytes = 0;
    bind_workspace(c, workspace);
    return PKV_OK;
}

// Parameters of launch chunk i of a balanced call (a slice of the batch with
// its own region of the workspace).
pkv::DecodeParams chunk_params(const Call& c, int32_t i) {
    const Plan& pl = c.plan;
    pkv::DecodeParams p = c.base;
    const int32_t s0 = i * pl.chunk_seqs;
    const int32_t n = c.base.num_seqs - s0 < pl.chunk_seqs ? c.base.num_seqs - s0 : pl.chunk_seqs;
    p.num_seqs = n;
    p.q = static_cast<const char*>(c.base.q) + (size_t)s0 * c.q_row_bytes;
    p.out = static_cast<char*>(c.base.out) + (size_t)s0 * c.out_row_bytes;
    p.block_tables = c.base.block_tables + (int64_t)s0 * c.base.max_blocks_per_seq;
    p.context_lens = c.base.context_lens + s0;
    if (c.base.k_new) {
        p.k_new = static_cast<const char*>(c.base.k_new) + (size_t)s0 * c.new_row_bytes;
        p.v_new = static_cast<const char*>(c.base.v_new) + (size_t)s0 * c.new_row_bytes;
    }
    char* w = c.workspace + (size_t)i * pl.chunk_bytes;
    p.seq_off = reinterpret_cast<int32_t*>(w);
    const size_t rows = (size_t)(2 * pl.max_ranges) * c.base.num_q_heads;
    float* f = reinterpret_cast<float*>(w + pl.off_bytes);
    p.o_part = f;
    p.m_part = f + rows * c.base.head_dim;
    p.l_part = f + rows * (c.base.head_dim + 1);
    return p;
}

pkv_status run_decode_kernels(const Call& c, hipStream_t stream) {
    if (c.base.num_seqs == 0) return PKV_OK;
    if (!c.plan.balanced)
        return from_hip(pkv::launch_decode_valu(c.base, false, stream), "decode partition kernel launch");
    for (int32_t i = 0; i < c.plan.num_chunks; ++i) {
        pkv_status st = from_hip(pkv::launch_decode_bf16_balanced(chunk_params(c, i), stream), "decode kernel launch");
        if (st != PKV_OK) return st;
    }
    return PKV_OK;
}

pkv_status run_reduce_kernels(const Call& c, hipStream_t stream) {
    if (c.base.num_seqs == 0) return PKV_OK;
    if (!c.plan.balanced) return from_hip(pkv::launch_splitk_reduce(c.base, false, stream), "split-K reduce launch");
    for (int32_t i = 0; i < c.plan.num_chunks; ++i) {
        pkv_status st = from_hip(pkv::launch_splitk_reduce(chunk_params(c, i), true, stream), "split-K reduce launch");
        if (st != PKV_OK) return st;
    }
    return PKV_OK;
}

// A decode call with the new tokens' append fused into its decode launch.
pkv_status prepare_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                          int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype kv_dtype,
                          pkv_dtype out_dtype, uint32_t flags, const float* k_scale, const float* v_scale, Call* c) {
    if (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "the fused append takes bf16 or fp8 pools (use pkv_reshape_and_cache and the decode)");
    if (kv_dtype == PKV_FP8_E4M3 && num_seqs > 0 && (!k_scale || !v_scale))
        return fail(PKV_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
    pkv_status st = prepare(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                            partition_size, workspace, workspace_bytes, kv_dtype, out_dtype, flags, k_scale, v_scale,
                            c);
    if (st != PKV_OK) return st;
    if (c->plan.n_head_groups != 1)
        return fail(PKV_ERR_UNSUPPORTED, "the fused append takes at most %d query heads per KV head (got %d)",
                    pkv::kMfmaHeadsPerUnit, c->plan.group);
    if (num_seqs > 0 && (!k_new || !v_new)) return fail(PKV_ERR_INVALID_ARG, "null k_new or v_new");
    if ((uintptr_t)k_new % 16) return fail(PKV_ERR_INVALID_ARG, "k_new must be 16-byte aligned");
    c->base.k_new = k_new;
    c->base.v_new = v_new;
    c->new_row_bytes = (size_t)num_kv_heads * head_dim * sizeof(uint16_t);
    return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return 7; }

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
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16)
        return fail(PKV_ERR_INVALID_ARG, "k_new, v_new, k_cache and v_cache must be 16-byte aligned");
    return from_hip(pkv::launch_cache_write(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads,
                                            head_dim, num_blocks, dtype == PKV_BF16, static_cast<hipStream_t>(stream)),
                    "reshape_and_cache launch");
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size, pkv_dtype kv_dtype) {
    Plan pl;
    const int32_t blocks = (int32_t)ceil_div(max_context_len > 0 ? max_context_len : 0, pkv::kBlockSize);
    const char saved = g_last_error[0];
    pkv_status st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, pkv::kBlockSize, blocks,
                              max_context_len, partition_size, kv_dtype, &pl);
    g_last_error[0] = saved;
    return st == PKV_OK ? pl.workspace : 0;
}

pkv_status pkv_paged_attention_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                                 void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                                 pkv_dtype kv_dtype, pkv_dtype out_dtype, uint32_t flags,
                                                 void* stream) {
    g_last_error[0] = 0;
    if (kv_dtype == PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "an fp8 cache needs its scales: use pkv_paged_attention_decode_fp8");
    Call c;
    pkv_status st = prepare(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                            partition_size, workspace, workspace_bytes, kv_dtype, out_dtype, flags, nullptr, nullptr,
                            &c);
    if (st != PKV_OK) return st;
    return run_decode_kernels(c, static_cast<hipStream_t>(stream));
}

pkv_status pkv_paged_attention_decode_reduce(const int32_t* context_lens, void* out, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                                             int32_t partition_size, void* workspace, size_t workspace_bytes,
                                             pkv_dtype kv_dtype, pkv_dtype out_dtype, void* stream) {
    g_last_error[0] = 0;
    Call c;
    // the reduce reads only lengths, partials and out; the K/V/q/table
    // pointers are not used, so stand-ins keep the shared checks happy
    const void* unused = context_lens;
    pkv_status st = prepare(unused, unused, unused, context_lens, context_lens, 1.0f, out, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, block_size, 1, max_blocks_per_seq, max_context_len,
                            partition_size, workspace, workspace_bytes, kv_dtype, out_dtype, 0, nullptr, nullptr, &c);
    if (st != PKV_OK) return st;
    return run_reduce_kernels(c, static_cast<hipStream_t>(stream));
}

pkv_status pkv_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                                      int32_t max_context_len, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_dtype kv_dtype, pkv_dtype out_dtype, uint32_t flags,
                                      void* stream) {
    g_last_error[0] = 0;
    if (kv_dtype == PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "an fp8 cache needs its scales: use pkv_paged_attention_decode_fp8");
    Call c;
    pkv_status st = prepare(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                            partition_size, workspace, workspace_bytes, kv_dtype, out_dtype, flags, nullptr, nullptr,
                            &c);
    if (st != PKV_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_decode_kernels(c, s);
    if (st != PKV_OK) return st;
    return run_reduce_kernels(c, s);
}

pkv_status pkv_paged_attention_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                             void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                             float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                             int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                             int32_t partition_size, void* workspace, size_t workspace_bytes,
                                             pkv_dtype kv_dtype, pkv_dtype out_dtype, uint32_t flags, void* stream) {
    g_last_error[0] = 0;
    if (kv_dtype == PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "an fp8 cache needs its scales: use pkv_paged_attention_decode_append_fp8");
    Call c;
    pkv_status st = prepare_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                   max_context_len, partition_size, workspace, workspace_bytes, kv_dtype, out_dtype,
                                   flags, nullptr, nullptr, &c);
    if (st != PKV_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_decode_kernels(c, s);
    if (st != PKV_OK) return st;
    return run_reduce_kernels(c, s);
}

pkv_status pkv_paged_attention_decode_append_partitions(const void* q, const void* k_new, const void* v_new,
                                                        void* k_cache, void* v_cache, const int32_t* block_tables,
                                                        const int32_t* context_lens, float scale, void* out,
                                                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                        int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                                        int32_t max_blocks_per_seq, int32_t max_context_len,
                                                        int32_t partition_size, void* workspace,
                                                        size_t workspace_bytes, pkv_dtype kv_dtype,
                                                        pkv_dtype out_dtype, uint32_t flags, void* stream) {
    g_last_error[0] = 0;
    if (kv_dtype == PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "an fp8 cache needs its scales: use pkv_paged_attention_decode_append_fp8");
    Call c;
    pkv_status st = prepare_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                   max_context_len, partition_size, workspace, workspace_bytes, kv_dtype, out_dtype,
                                   flags, nullptr, nullptr, &c);
    if (st != PKV_OK) return st;
    return run_decode_kernels(c, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Scratch of pkv_paged_attention_decode_noalloc: a fixed device array that
// takes the place of the caller's workspace (the flattened block offsets
// and the split-K partials).  Every device the library runs on holds its
// own copy, from the first use of this code object until the process ends.
// In host code `scratch` is only a host-side stand-in for the symbol; its
// device address is looked up once per device (scratch_address) and only
// that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Address of `scratch` on the current device (looked up on the first call
// on that device, with that device current).
pkv_status scratch_address(void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKV_ERR_UNSUPPORTED, "device %d: the fixed scratch serves devices 0..%d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r != hipSuccess || !p) return from_hip(r != hipSuccess ? r : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* context_lens, float scale,
                                              void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                              int32_t max_blocks_per_seq, int32_t max_context_len,
                                              int32_t partition_size, pkv_dtype kv_dtype, pkv_dtype out_dtype,
                                              uint32_t flags, void* stream) {
    g_last_error[0] = 0;
    if (kv_dtype == PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "an fp8 cache needs its scales: use pkv_paged_attention_decode_fp8");
    Plan pl;
    pkv_status st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              max_context_len, partition_size, kv_dtype, &pl);
    if (st != PKV_OK) return st;
    if (pl.workspace > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
        return fail(PKV_ERR_WORKSPACE,
                    "these sizes need %zu bytes of scratch; the fixed scratch holds %zu (pass a workspace to "
                    "pkv_paged_attention_decode instead)",
                    pl.workspace, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
    // every host-side check first, against a stand-in address (256-byte
    // aligned, never dereferenced), then the scratch's device address
    void* const stand_in = reinterpret_cast<void*>((uintptr_t)256);
    Call c;
    st = prepare(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads, num_kv_heads,
                 head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, partition_size,
                 pl.workspace ? stand_in : nullptr, pl.workspace ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0, kv_dtype,
                 out_dtype, flags, nullptr, nullptr, &c);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return PKV_OK;
    void* ws = nullptr;
    if (pl.workspace > 0) {
        st = scratch_address(&ws);
        if (st != PKV_OK) return st;
    }
    bind_workspace(&c, ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_decode_kernels(c, s);
    if (st != PKV_OK) return st;
    return run_reduce_kernels(c, s);
}

pkv_status pkv_reshape_and_cache_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                     void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                                     int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, pkv_dtype src_dtype, void* stream) {
    g_last_error[0] = 0;
    if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
    if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
    if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size != pkv::kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
    if (!dtype_ok(src_dtype)) return fail(PKV_ERR_UNSUPPORTED, "input rows must be f32 or bf16");
    if (num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive");
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
        return fail(PKV_ERR_INVALID_ARG, "null pointer");
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_cache) % 16)
        return fail(PKV_ERR_INVALID_ARG, "k_new, v_new and k_cache must be 16-byte aligned");
    return from_hip(pkv::launch_cache_write_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                                                num_tokens, num_kv_heads, head_dim, num_blocks, src_dtype == PKV_BF16,
                                                static_cast<hipStream_t>(stream)),
                    "reshape_and_cache_fp8 launch");
}

pkv_status pkv_paged_attention_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                          const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                                          int32_t max_context_len, int32_t partition_size, void* workspace,
                                          size_t workspace_bytes, pkv_dtype out_dtype, uint32_t flags, void* stream) {
    g_last_error[0] = 0;
    if (num_seqs > 0 && (!k_scale || !v_scale))
        return fail(PKV_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
    Call c;
    pkv_status st = prepare(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                            partition_size, workspace, workspace_bytes, PKV_FP8_E4M3, out_dtype, flags, k_scale,
                            v_scale, &c);
    if (st != PKV_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_decode_kernels(c, s);
    if (st != PKV_OK) return st;
    return run_reduce_kernels(c, s);
}

pkv_status pkv_paged_attention_decode_partitions_fp8(const void* q, const void* k_cache, const void* v_cache,
                                                     const float* k_scale, const float* v_scale,
                                                     const int32_t* block_tables, const int32_t* context_lens,
                                                     float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                     int64_t num_blocks, int32_t max_blocks_per_seq,
                                                     int32_t max_context_len, int32_t partition_size,
                                                     void* workspace, size_t workspace_bytes, pkv_dtype out_dtype,
                                                     uint32_t flags, void* stream) {
    g_last_error[0] = 0;
    if (num_seqs > 0 && (!k_scale || !v_scale))
        return fail(PKV_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
    Call c;
    pkv_status st = prepare(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                            partition_size, workspace, workspace_bytes, PKV_FP8_E4M3, out_dtype, flags, k_scale,
                            v_scale, &c);
    if (st != PKV_OK) return st;
    return run_decode_kernels(c, static_cast<hipStream_t>(stream));
}

pkv_status pkv_paged_attention_decode_append_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                                 void* v_cache, const float* k_scale, const float* v_scale,
                                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                                 void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                                 pkv_dtype out_dtype, uint32_t flags, void* stream) {
    g_last_error[0] = 0;
    Call c;
    pkv_status st = prepare_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                   max_context_len, partition_size, workspace, workspace_bytes, PKV_FP8_E4M3,
                                   out_dtype, flags, k_scale, v_scale, &c);
    if (st != PKV_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_decode_kernels(c, s);
    if (st != PKV_OK) return st;
    return run_reduce_kernels(c, s);
}

pkv_status pkv_paged_attention_decode_append_partitions_fp8(
    const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pkv_dtype out_dtype, uint32_t flags, void* stream) {
    g_last_error[0] = 0;
    Call c;
    pkv_status st = prepare_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                   max_context_len, partition_size, workspace, workspace_bytes, PKV_FP8_E4M3,
                                   out_dtype, flags, k_scale, v_scale, &c);
    if (st != PKV_OK) return st;
    return run_decode_kernels(c, static_cast<hipStream_t>(stream));
}

// The address a kernel uses for `p`: device memory as it is; pinned host
// memory through its device mapping.  Anything else (pageable host memory,
// an unknown pointer) is refused before launch, because a kernel touching
// it would fault.
pkv_status device_view(const void* p, const char* what, const void** out) {
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof(a));
    const hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", what);
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
        *out = p;
        return PKV_OK;
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer) {
        // the attributes may describe the allocation's start: keep p's offset
        const ptrdiff_t off = a.hostPointer ? static_cast<const char*>(p) - static_cast<const char*>(a.hostPointer) : 0;
        *out = static_cast<const char*>(a.devicePointer) + off;
        return PKV_OK;
    }
    return fail(PKV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", what);
}

pkv_status pkv_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int64_t* pairs,
                           int64_t num_pairs, int64_t num_src_blocks, int64_t num_dst_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, pkv_dtype dtype, void* stream) {
    g_last_error[0] = 0;
    if (num_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "num_pairs must be >= 0");
    if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
    if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size != pkv::kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
    if (!kv_dtype_ok(dtype)) return fail(PKV_ERR_UNSUPPORTED, "unknown dtype");
    if (num_src_blocks <= 0 || num_dst_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "pool sizes must be positive");
    if (num_pairs == 0) return PKV_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return fail(PKV_ERR_INVALID_ARG, "null pointer");
    if (((uintptr_t)src_k | (uintptr_t)src_v | (uintptr_t)dst_k | (uintptr_t)dst_v) % 16)
        return fail(PKV_ERR_INVALID_ARG, "pools must be 16-byte aligned");
    const void* views[5];
    const void* ptrs[5] = {src_k, src_v, dst_k, dst_v, pairs};
    const char* names[5] = {"src_k", "src_v", "dst_k", "dst_v", "pairs"};
    for (int i = 0; i < 5; ++i) {
        pkv_status st = device_view(ptrs[i], names[i], &views[i]);
        if (st != PKV_OK) return st;
    }
    const int64_t es = dtype == PKV_F32 ? 4 : (dtype == PKV_BF16 ? 2 : 1);
    const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * es;
    const int64_t chunks = ceil_div(block_bytes / 16, 2048);
    if (num_pairs * 2 * chunks >= ((int64_t)1 << 31))
        return fail(PKV_ERR_UNSUPPORTED, "%lld block pairs: too many for one launch", (long long)num_pairs);
    return from_hip(pkv::launch_copy_blocks(views[0], views[1], const_cast<void*>(views[2]),
                                            const_cast<void*>(views[3]), static_cast<const int64_t*>(views[4]),
                                            num_pairs, num_src_blocks, num_dst_blocks, block_bytes,
                                            static_cast<hipStream_t>(stream)),
                    "copy_blocks launch");
}

namespace {

// Shared body of the bf16 and fp8 prefill entry points (kv_fp8: E4M3 pools
// with per-KV-head scales k_scale / v_scale).
pkv_status prefill_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        const int32_t* context_lens, const int32_t* query_start_loc, float scale, void* out,
                        int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                        int32_t max_context_len, bool kv_fp8, const float* k_scale, const float* v_scale,
                        pkv_dtype out_dtype, void* stream) {
    if (num_seqs < 0 || num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs and num_tokens must be >= 0");
    if (num_q_heads <= 0 || num_kv_heads <= 0)
        return fail(PKV_ERR_INVALID_ARG, "head counts must be positive (q %d, kv %d)", num_q_heads, num_kv_heads);
    if (num_q_heads % num_kv_heads)
        return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", num_q_heads,
                    num_kv_heads);
    if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size != pkv::kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 16)", block_size);
    if (!dtype_ok(out_dtype)) return fail(PKV_ERR_UNSUPPORTED, "unknown output dtype");
    if (max_blocks_per_seq < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and max_context_len must be >= 0");
    if (!isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
    if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc || !out)
        return fail(PKV_ERR_INVALID_ARG, "null tensor pointer");
    if (kv_fp8 && (!k_scale || !v_scale)) return fail(PKV_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
    if (num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive");
    if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) % 16)
        return fail(PKV_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
    const int32_t group = num_q_heads / num_kv_heads;
    const int64_t rows = (int64_t)num_tokens * group;
    const int64_t by_table = (int64_t)max_blocks_per_seq * block_size;
    pkv::PrefillParams p;
    memset(&p, 0, sizeof(p));
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.out = out;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    p.num_tokens = num_tokens;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = group;
    p.head_dim = head_dim;
    p.num_blocks = num_blocks;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.ctx_cap = (int32_t)(max_context_len < by_table ? max_context_len : by_table);
    p.out_bf16 = out_dtype == PKV_BF16;
    p.kv_fp8 = kv_fp8 ? 1 : 0;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int32_t s0 = 0; s0 < num_seqs; s0 += pkv::kMaxSeqsPerLaunch) {
        const int32_t n = num_seqs - s0 < pkv::kMaxSeqsPerLaunch ? num_seqs - s0 : pkv::kMaxSeqsPerLaunch;
        p.num_seqs = n;
        p.block_tables = block_tables + (int64_t)s0 * max_blocks_per_seq;
        p.context_lens = context_lens + s0;
        p.query_start_loc = query_start_loc + s0;
        const int64_t bound = ceil_div(rows, pkv::kPrefillRowsPerGroup) + n;
        if (bound * num_kv_heads >= ((int64_t)1 << 31))
            return fail(PKV_ERR_UNSUPPORTED, "%d tokens x %d query heads: too many workgroups for one launch",
                        num_tokens, num_q_heads);
        p.tile_bound = (int32_t)bound;
        // weight classes for the heaviest-first tile order: 64-key classes,
        // coarser when the LDS for them would not fit
        p.lpt_shift = 6;
        while ((int64_t)(n + 3 + (p.ctx_cap >> p.lpt_shift) + 2) * 4 > pkv::kPrefillPlanLdsBytes) ++p.lpt_shift;
        p.lpt_buckets = (p.ctx_cap >> p.lpt_shift) + 2;
        pkv_status rc = from_hip(pkv::launch_prefill(p, st), "prefill kernel launch");
        if (rc != PKV_OK) return rc;
    }
    return PKV_OK;
}

}  // namespace

pkv_status pkv_paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       const int32_t* query_start_loc, float scale, void* out, int32_t num_seqs,
                                       int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len, pkv_dtype kv_dtype,
                                       pkv_dtype out_dtype, void* stream) {
    g_last_error[0] = 0;
    if (kv_dtype != PKV_BF16)
        return fail(PKV_ERR_UNSUPPORTED, "prefill takes bf16 KV (fp8 pools: pkv_paged_attention_prefill_fp8)");
    return prefill_impl(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, num_seqs,
                        num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                        max_context_len, false, nullptr, nullptr, out_dtype, stream);
}

pkv_status pkv_paged_attention_prefill_fp8(const void* q, const void* k_cache, const void* v_cache,
                                           const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                           const int32_t* context_lens, const int32_t* query_start_loc, float scale,
                                           void* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                           pkv_dtype out_dtype, void* stream) {
    g_last_error[0] = 0;
    return prefill_impl(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, num_seqs,
                        num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                        max_context_len, true, k_scale, v_scale, out_dtype, stream);
}

pkv_status pkv_hbm_read_bench(const void* src, int64_t bytes, const int32_t* tiles, int64_t num_tiles,
                              int32_t tile_bytes, int32_t streaming, uint32_t* sink, void* stream) {
    g_last_error[0] = 0;
    if (bytes <= 0 || bytes % 16) return fail(PKV_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if (num_tiles < 0) return fail(PKV_ERR_INVALID_ARG, "num_tiles must be >= 0");
    if (!src || !sink) return fail(PKV_ERR_INVALID_ARG, "null pointer");
    if ((uintptr_t)src % 16) return fail(PKV_ERR_INVALID_ARG, "src must be 16-byte aligned");
    if (tiles) {
        if (tile_bytes < 16 || tile_bytes > (1 << 24) || (tile_bytes & (tile_bytes - 1)))
            return fail(PKV_ERR_INVALID_ARG, "tile_bytes must be a power of two in [16, 2^24]");
        if (num_tiles > ((int64_t)1 << 40) / tile_bytes) return fail(PKV_ERR_INVALID_ARG, "too many tiles");
    }
    return from_hip(pkv::launch_hbm_read(src, bytes, tiles, num_tiles, tile_bytes, streaming != 0, sink,
                                         static_cast<hipStream_t>(stream)),
                    "hbm_read launch");
}

pkv_status pkv_issue_rate_bench(int32_t pattern, int32_t waves_per_simd, int32_t iters, uint32_t* sink,
                                void* stream) {
    g_last_error[0] = 0;
    if (pattern < 0 || pattern > 6) return fail(PKV_ERR_INVALID_ARG, "pattern must be 0 .. 6");
    if (waves_per_simd < 1 || waves_per_simd > 2) return fail(PKV_ERR_INVALID_ARG, "waves_per_simd must be 1 or 2");
    if (iters < 1 || iters > 10000000) return fail(PKV_ERR_INVALID_ARG, "iters must be 1 .. 10^7");
    if (!sink) return fail(PKV_ERR_INVALID_ARG, "null sink");
    return from_hip(pkv::launch_issue_rate(pattern, waves_per_simd, iters, sink, static_cast<hipStream_t>(stream)),
                    "issue_rate launch");
}

pkv_status pkv_paged_attention_decode_vector_alu(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_tables, const int32_t* context_lens,
                                                 float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int64_t num_blocks, int32_t max_blocks_per_seq,
                                                 int32_t max_context_len, int32_t partition_size, void* workspace,
                                                 size_t workspace_bytes, pkv_dtype out_dtype, void* stream) {
    g_last_error[0] = 0;
    // the fp32 path's plan (fixed partitions, its workspace rule); the
    // kernel reads bf16 elements
    Call c;
    pkv_status st = prepare(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                            partition_size, workspace, workspace_bytes, PKV_F32, out_dtype, 0, nullptr, nullptr, &c);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return PKV_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = from_hip(pkv::launch_decode_valu(c.base, true, s), "vector-ALU decode launch");
    if (st != PKV_OK) return st;
    return from_hip(pkv::launch_splitk_reduce(c.base, false, s), "split-K reduce launch");
}

}  // extern "C"

