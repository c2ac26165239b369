/*
 * pagedkv.h -- C ABI of libpagedkv.so: paged-KV cache write and decode
 * attention on AMD MI355X (gfx950).
 *
 * The problem statement comes from the pages on PagedAttention:
 *   - the KV cache of a sequence is cut into fixed-size blocks that live in
 *     one large pool allocated once at start-up (architvora, "Just a python
 *     process"; runbyai, section 3 "The core idea of PagedAttention");
 *   - a per-sequence block table maps logical blocks to physical ones
 *     (ai-hpc, "2.1 Algorithm Principle");
 *   - each decode step the engine packs the tables into tensors and sends
 *     them to the GPU, where the kernel follows that map to gather the blocks
 *     (architvora, "Just a python process" and "Paged Attention");
 *   - decode: the one new token of each sequence attends over the keys and
 *     values of all its earlier tokens (runbyai, section 1).
 *
 * Conventions for every call:
 *   - Pointers marked [device] are device addresses (e.g. from a torch CUDA
 *     tensor); the caller owns all memory.  The library never allocates,
 *     frees or synchronises, and keeps no state between calls (it reads
 *     the current device's compute-unit count to plan a launch).  The one
 *     exception is the fixed device scratch of
 *     pkv_paged_attention_decode_noalloc (see there).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  A returned PKV_OK means the work was enqueued.
 *   - Problems visible on the host (null pointer, bad size, unsupported
 *     shape or dtype, workspace too small) return an error status before any
 *     GPU work is enqueued; the message is in pkv_last_error().  A failed
 *     launch returns PKV_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Values that live on the device are never validated on the host (that
 *     would need a synchronisation).  Kernels guard every address instead:
 *     a slot or physical block id outside the pool is skipped, and context
 *     lengths are clamped to [0, min(max_context_len,
 *     max_blocks_per_seq * block_size)].
 *   - Thread-safe: calls may come from several host threads at once.
 *
 * Element types: PKV_F32 (IEEE binary32) or PKV_BF16 (bfloat16, 16-bit); a KV
 * pool may also hold PKV_FP8_E4M3 codes (one byte per element, see below).
 * Tensors are dense, row-major, with the shapes given below.
 *
 * KV pool layout (one K pool and one V pool, shape fixed at allocation):
 *   k_cache [num_blocks][num_kv_heads][head_dim/x][block_size][x],
 *           x = 16 / element_size (4 for f32, 8 for bf16, 16 for fp8): the head_dim
 *           values of a token are split into 16-byte chunks, and the chunks
 *           of the 16 tokens of a block are stored chunk-major;
 *   v_cache [num_blocks][num_kv_heads][head_dim][block_size]: for each dim,
 *           the block's tokens are contiguous.
 * A flat slot index is  physical_block * block_size + offset_in_block.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = 1,  /* null pointer, negative or inconsistent size */
    PKV_ERR_UNSUPPORTED = 2,  /* shape or dtype this build does not handle   */
    PKV_ERR_WORKSPACE = 3,    /* workspace missing or too small              */
    PKV_ERR_HIP = 4           /* the HIP runtime reported an error           */
} pkv_status;

typedef enum pkv_dtype {
    PKV_F32 = 0,
    PKV_BF16 = 1,
    PKV_FP8_E4M3 = 2  /* KV pools only: OCP E4M3 codes, see the fp8 calls */
} pkv_dtype;

/* Decode flags (a performance choice only: results are bit-identical with
 * and without).
 * PKV_DECODE_SHARED_BLOCKS: several sequences of the batch point at the same
 *   physical blocks (a common prompt prefix, forked samples: runbyai
 *   section 3 "Shared prefix"; ai-hpc 2.2 "Flexible Sharing").  With bf16 KV
 *   the decode then reads K and V with ordinary loads, which keep a shared
 *   block in the caches for its next reader.  Without it, K and V are read
 *   with streaming (non-temporal) loads, the faster choice when every block
 *   is read once.  fp32 KV ignores the flag. */
#define PKV_DECODE_SHARED_BLOCKS 1u

/* Version of this ABI (bumped on any incompatible change). */
int32_t pkv_abi_version(void);

/*
 * Cache write: for every token t in [0, num_tokens) with slot_mapping[t] >= 0,
 * copy k_new[t][h][:] and v_new[t][h][:] for every KV head h into the pool
 * slot slot_mapping[t] (block = slot / block_size, offset = slot % block_size),
 * bit for bit.  This is the "cache the key/value of every token" step of
 * runbyai section 1 / section 2, addressed through the paged layout.
 *
 *   k_new, v_new   [device] [num_tokens][num_kv_heads][head_dim], dtype
 *   slot_mapping   [device] int64 [num_tokens]; negative = skip (padding);
 *                  slots >= num_blocks * block_size are skipped as well
 *   k_cache, v_cache [device] pools in the layout above, num_blocks blocks
 *   head_dim       64 or 128;  block_size 16;  dtype PKV_F32 or PKV_BF16
 *   k_new, v_new, k_cache and v_cache 16-byte aligned (else
 *   PKV_ERR_INVALID_ARG)
 * Two tokens must not name the same slot (the write order between them is
 * unspecified).  num_tokens == 0 is a no-op.
 */
pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                 void* k_cache, void* v_cache, int64_t num_tokens, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks, pkv_dtype dtype,
                                 void* stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for these sizes
 * on the current HIP device (the bf16 plan depends on its compute-unit
 * count; with no usable device a 256-CU part is assumed).  Returns 0 for
 * invalid sizes, and 0 when none is needed (fp32 KV whose contexts fit in one
 * partition).  bf16 KV always needs some: the flattened block offsets of
 * the batch and the partial results of sequences split across ranges.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                                  pkv_dtype kv_dtype);

/*
 * Decode attention over the paged cache (runbyai sections 1 and 3;
 * ai-hpc 2.1; architvora "Paged Attention": the kernel follows each
 * sequence's block table to gather its blocks).  For sequence s and query
 * head h, with L = context_lens[s] and g = h / (num_q_heads / num_kv_heads):
 *     out[s][h][:] = sum_i softmax_i(scale * <q[s][h], K_i>) * V_i,
 * over the tokens i < L of sequence s, K_i / V_i the KV-head-g rows of token
 * i read through block_tables[s][i / block_size] at offset i % block_size.
 * L == 0 gives zeros.  Accumulation is fp32; with bf16 KV the products of
 * the softmax weights with V use the weights split into two bf16 terms.
 *
 *   q              [device] [num_seqs][num_q_heads][head_dim], kv_dtype
 *   k_cache, v_cache [device] pools (layout above), kv_dtype
 *   block_tables   [device] int32 [num_seqs][max_blocks_per_seq]; entries
 *                  past a sequence's last block are never read
 *   context_lens   [device] int32 [num_seqs], counting the token written
 *                  this step
 *   out            [device] [num_seqs][num_q_heads][head_dim], out_dtype
 *                  (PKV_F32 or PKV_BF16, rounded to nearest even)
 *   num_q_heads    a multiple of num_kv_heads
 *   head_dim 64 or 128; block_size 16; num_blocks = pool size in blocks
 *   max_context_len  host-known upper bound of context_lens (sizes the
 *                  workspace; larger lengths are clamped to it)
 *   partition_size   0 or a multiple of block_size in [16, 2^24]: the
 *                  longest piece of a context reduced before the split-K
 *                  merge (see below); 0 = let the library choose
 *   workspace      [device] >= pkv_decode_workspace_bytes(...) bytes,
 *                  256-byte aligned; may be NULL when that is 0.  Its
 *                  contents need no initialisation; one workspace serves one
 *                  call at a time.
 *   flags          0 or PKV_DECODE_SHARED_BLOCKS; other bits are rejected
 *                  (PKV_ERR_INVALID_ARG)
 * Work split.  bf16 KV: the blocks of all sequences, taken in order, form
 * one flattened list that is cut into equal ranges, one per workgroup the
 * device holds at once (or shorter, at most partition_size tokens each), so
 * every workgroup streams the same number of KV bytes whatever the mix of
 * context lengths.  A sequence inside one range is finished where it is
 * read; the pieces of a sequence spread over several ranges leave partial
 * softmax statistics that a second kernel merges (log-sum-exp rescaling).
 * fp32 KV: each sequence is cut into partitions of partition_size tokens
 * (1024 when 0 is passed and the longest context exceeds that), merged the
 * same way.  Batches of more than 4096 sequences are run as consecutive
 * launches of up to 4096.  Results are deterministic: the order of every
 * sum depends only on logical token positions and on the sizes of the
 * call, never on where blocks sit in the pool or on timing.
 */
pkv_status pkv_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                                      void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                                      pkv_dtype kv_dtype, pkv_dtype out_dtype, uint32_t flags, void* stream);

/*
 * The two launches of pkv_paged_attention_decode, callable one at a time
 * (same arguments and meaning; the reduce takes the subset it reads and
 * no flags).
 * _partitions runs the block-table walk and writes `out` for the sequences
 * it finishes and fp32 partials for the others; _reduce merges those
 * partials into `out` (and, with bf16 KV, writes the zeros of empty
 * contexts).  _reduce must follow _partitions on the same stream with the
 * same arguments and workspace.  With fp32 KV it is a no-op when no split
 * is needed.
 */
pkv_status pkv_paged_attention_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_tables, const int32_t* context_lens,
                                                 float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int64_t num_blocks, int32_t max_blocks_per_seq,
                                                 int32_t max_context_len, int32_t partition_size, void* workspace,
                                                 size_t workspace_bytes, pkv_dtype kv_dtype, pkv_dtype out_dtype,
                                                 uint32_t flags, void* stream);

pkv_status pkv_paged_attention_decode_reduce(const int32_t* context_lens, void* out, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq,
                                             int32_t max_context_len, int32_t partition_size, void* workspace,
                                             size_t workspace_bytes, pkv_dtype kv_dtype, pkv_dtype out_dtype,
                                             void* stream);

/*
 * One decode step with the cache write fused into the decode launch: for
 * every sequence s with L = context_lens[s] >= 1, store the token it gains
 * this step, k_new[s][h][:] and v_new[s][h][:] for every KV head h, at
 * position L - 1 of s (block_tables[s][(L - 1) / block_size], offset
 * (L - 1) % block_size), then attend as pkv_paged_attention_decode.  The
 * result, pool and out, is bit for bit that of pkv_reshape_and_cache with
 * slot_mapping[s] = block_tables[s][(L - 1) / 16] * 16 + (L - 1) % 16
 * followed by pkv_paged_attention_decode with the same sizes.  The decode
 * step appends one token per sequence and then attends over the whole
 * cache, the new token included (runbyai sections 1-2; architvora "Paged
 * Attention": a new block is taken when the last one is full); the two
 * steps share one launch here because, for each KV head, the workgroup
 * that reads a sequence's last block is the one that stores its token.
 *
 *   k_new, v_new   [device] [num_seqs][num_kv_heads][head_dim], kv_dtype;
 *                  k_new 16-byte aligned
 *   k_cache, v_cache [device] pools, written at the appended slots
 *   kv_dtype       PKV_BF16 only (others: PKV_ERR_UNSUPPORTED; fp8 pools:
 *                  pkv_paged_attention_decode_append_fp8)
 *   num_q_heads    at most 16 query heads per KV head (else
 *                  PKV_ERR_UNSUPPORTED)
 * All other arguments, the workspace and the flags as for
 * pkv_paged_attention_decode.  The caller must have made the block that
 * holds position L - 1 private to s (copy-on-write), as for any cache
 * write; a table entry outside the pool is skipped, as the decode skips it.
 * A context length above max_context_len (undefined for the decode) places
 * the token at the clamped length.
 */
pkv_status pkv_paged_attention_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                             void* v_cache, const int32_t* block_tables,
                                             const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                                             int32_t max_context_len, int32_t partition_size, void* workspace,
                                             size_t workspace_bytes, pkv_dtype kv_dtype, pkv_dtype out_dtype,
                                             uint32_t flags, void* stream);

/* The decode launch of pkv_paged_attention_decode_append on its own (the
 * append included); follow it with pkv_paged_attention_decode_reduce on the
 * same stream with the same sizes and workspace. */
pkv_status pkv_paged_attention_decode_append_partitions(const void* q, const void* k_new, const void* v_new,
                                                        void* k_cache, void* v_cache, const int32_t* block_tables,
                                                        const int32_t* context_lens, float scale, void* out,
                                                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                        int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                                        int32_t max_blocks_per_seq, int32_t max_context_len,
                                                        int32_t partition_size, void* workspace,
                                                        size_t workspace_bytes, pkv_dtype kv_dtype,
                                                        pkv_dtype out_dtype, uint32_t flags, void* stream);

/*
 * Decode with no allocation and no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, result and
 * launches as pkv_paged_attention_decode (bit-identical output), with the
 * workspace taken from a fixed device array of PKV_NOALLOC_SCRATCH_BYTES
 * inside the library instead of from the caller.
 *   - Each device holds its own copy of that array from the first use of
 *     the library on it until the process ends; its address is looked up on
 *     the first call on each device.  The call allocates and frees nothing.
 *   - Sizes whose workspace (pkv_decode_workspace_bytes) exceeds
 *     PKV_NOALLOC_SCRATCH_BYTES return PKV_ERR_WORKSPACE before any launch
 *     (e.g. 64 query heads of 8 x 128k-token contexts fit with
 *     partition_size 0, not with partition_size 512).
 *   - All calls on one device share the array, which keeps the last call's
 *     contents (the kernels need no initialised contents).  Calls that
 *     overlap on one device -- on different streams, or from several host
 *     threads without ordering -- race on it: order them on one stream.
 *   - fp8 pools are refused (PKV_ERR_UNSUPPORTED), as for the plain call.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)

pkv_status pkv_paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* context_lens, float scale,
                                              void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                              int32_t max_blocks_per_seq, int32_t max_context_len,
                                              int32_t partition_size, pkv_dtype kv_dtype, pkv_dtype out_dtype,
                                              uint32_t flags, void* stream);

/*
 * fp8 KV cache.  The pages name quantisation of the KV cache as the lever for
 * long contexts (runbyai section 5); they fix no format.  Here a pool element
 * is an OCP E4M3 code (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, largest finite 448, 0x7F / 0xFF NaN) and each KV head has
 * one positive fp32 scale for K and one for V, chosen by the caller:
 *   stored code = E4M3(fp32(x / scale[h]))  (a correctly rounded fp32
 *                 division, then round to nearest even, saturating at +-448);
 *   value read  = decode(code) * scale[h].
 * Pools use the layout at the top with one-byte elements: a (block, head) tile
 * is 2 KiB at head_dim 128, half the bytes of bf16.
 *
 * Quantising cache write: like pkv_reshape_and_cache, from f32 or bf16 rows
 * (src_dtype) into fp8 pools.
 *   k_scale, v_scale  [device] fp32 [num_kv_heads]
 */
pkv_status pkv_reshape_and_cache_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                     void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                                     int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, pkv_dtype src_dtype, void* stream);

/*
 * Decode over an fp8 cache: pkv_paged_attention_decode with K = decode(code) *
 * k_scale[g] and V = decode(code) * v_scale[g] for KV head g.  q is bf16; out
 * is out_dtype.  The codes are converted exactly: K to bf16 for the products
 * with q, V to fp16 for the products with the softmax weights, which enter
 * them rounded to fp16 (the scales enter the score scale and the output).
 * Workspace: pkv_decode_workspace_bytes(..., PKV_FP8_E4M3).  The other decode
 * entry points reject PKV_FP8_E4M3.
 */
pkv_status pkv_paged_attention_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                          const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                                          int32_t max_context_len, int32_t partition_size, void* workspace,
                                          size_t workspace_bytes, pkv_dtype out_dtype, uint32_t flags, void* stream);

/* The decode launch of pkv_paged_attention_decode_fp8 on its own; follow it
 * with pkv_paged_attention_decode_reduce(..., kv_dtype = PKV_FP8_E4M3, ...)
 * on the same stream with the same arguments and workspace. */
pkv_status pkv_paged_attention_decode_partitions_fp8(const void* q, const void* k_cache, const void* v_cache,
                                                     const float* k_scale, const float* v_scale,
                                                     const int32_t* block_tables, const int32_t* context_lens,
                                                     float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                     int64_t num_blocks, int32_t max_blocks_per_seq,
                                                     int32_t max_context_len, int32_t partition_size,
                                                     void* workspace, size_t workspace_bytes, pkv_dtype out_dtype,
                                                     uint32_t flags, void* stream);

/*
 * The fused decode step over an fp8 cache: pkv_paged_attention_decode_append
 * with E4M3 pools.  The new tokens arrive as bf16 rows and are stored as the
 * codes pkv_reshape_and_cache_fp8(..., src_dtype = PKV_BF16) would store
 * (E4M3 of fp32(x / scale) with the KV head's k_scale or v_scale); the
 * attention is that of pkv_paged_attention_decode_fp8.  Pools and out are
 * bit for bit those of those two calls in a row with slot_mapping as for
 * pkv_paged_attention_decode_append.  The decode step appends the token and
 * attends over the whole cache (runbyai sections 1-2); the codes are the
 * reading of KV quantisation for long contexts (runbyai section 5) that
 * pkv_reshape_and_cache_fp8 states.
 *   k_new, v_new      [device] bf16 [num_seqs][num_kv_heads][head_dim];
 *                     k_new 16-byte aligned
 *   k_cache, v_cache  [device] fp8 pools (layout as for
 *                     pkv_reshape_and_cache_fp8), written at the appended
 *                     slots
 *   k_scale, v_scale  [device] fp32 [num_kv_heads], positive
 * Null scales return PKV_ERR_INVALID_ARG; everything else as for
 * pkv_paged_attention_decode_append (at most 16 query heads per KV head).
 * Workspace: pkv_decode_workspace_bytes(..., PKV_FP8_E4M3).
 */
pkv_status pkv_paged_attention_decode_append_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                                 void* v_cache, const float* k_scale, const float* v_scale,
                                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                                 void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                                 pkv_dtype out_dtype, uint32_t flags, void* stream);

/* The decode launch of pkv_paged_attention_decode_append_fp8 on its own (the
 * append included); follow it with pkv_paged_attention_decode_reduce(...,
 * kv_dtype = PKV_FP8_E4M3, ...) on the same stream with the same sizes and
 * workspace. */
pkv_status pkv_paged_attention_decode_append_partitions_fp8(
    const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pkv_dtype out_dtype, uint32_t flags, void* stream);

/*
 * Whole-block copies between KV pools: copy-on-write and swapping.
 * Sequences forked from one prompt (parallel sampling, beam search) share its
 * physical blocks copy-on-write ("Deep Dive into vLLM", 2.2 "Advantages"): a
 * shared block is copied to a fresh one when an owner writes into it.  A
 * preempted sequence's blocks can be moved to CPU memory and back (architvora,
 * "Paged Attention").  Both copy, for each pair (src, dst) in `pairs`, the
 * whole block src of the source pools into block dst of the destination
 * pools: every KV head and token slot of K and of V, bit for bit.
 *
 *   src_k, src_v   source pools (layout above, num_src_blocks blocks)
 *   dst_k, dst_v   destination pools (num_dst_blocks blocks); the same
 *                  pointers as src_* for copy-on-write inside one pool
 *   pairs          int64 [num_pairs][2] (src block, dst block)
 * Pools and `pairs` may live in device memory or in pinned host memory that
 * the device can access (hipHostMalloc / torch pin_memory): the kernel reads
 * and writes them directly, one launch for all pairs.  Each pointer is looked
 * up first; anything else (pageable host memory) returns PKV_ERR_INVALID_ARG
 * before any launch.  A pair with an id
 * outside its pool is skipped.  Destinations must be distinct, and inside
 * one pool no destination may also be a source (the order of copies is
 * unspecified).  dtype: PKV_F32, PKV_BF16 or PKV_FP8_E4M3 (the element size).
 */
pkv_status pkv_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int64_t* pairs,
                           int64_t num_pairs, int64_t num_src_blocks, int64_t num_dst_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, pkv_dtype dtype, void* stream);

/*
 * Multi-token-query paged attention (chunked prefill).  Prefill processes a
 * whole prompt at once and is compute-bound (runbyai section 1); long
 * prompts are cut into chunks that share each step with decode requests,
 * and a request may process any number of tokens in a step (architvora
 * "Continuous Batching").
 *
 * Request s owns rows r0 = query_start_loc[s] .. r1 = query_start_loc[s+1]-1
 * of q and out: n = r1 - r0 query tokens, the last n of its L =
 * context_lens[s] cached tokens (the cache write of their keys and values
 * comes first, as for decode).  Query i sits at position p = L - n + i and
 * attends causally to positions 0..p of its own sequence, read through
 * block_tables[s]:
 *     out[r0+i][h][:] = sum_{j<=p} softmax_j(scale * <q[r0+i][h], K_j>) * V_j,
 * with K_j / V_j the KV-head h / (num_q_heads / num_kv_heads) rows of token
 * j.  n = 1 is decode.  A query with p < 0 (n > L) gets zeros.  Matrix
 * products take bf16 operands with fp32 accumulation; the softmax weights
 * enter the product with V rounded to bf16 once.
 *
 *   q              [device] bf16 [num_tokens][num_q_heads][head_dim]
 *   k_cache, v_cache [device] pools (layout above), bf16 only
 *   block_tables   [device] int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   [device] int32 [num_seqs]
 *   query_start_loc [device] int32 [num_seqs + 1], non-decreasing, first 0,
 *                  last num_tokens (rows outside [0, num_tokens) are
 *                  clamped away, never read or written)
 *   out            [device] [num_tokens][num_q_heads][head_dim], out_dtype
 *   max_context_len  host-known bound of context_lens (larger are clamped)
 * No workspace.  Requests are processed 4096 per launch.  Results do not
 * depend on where blocks sit in the pool.  fp32 KV returns
 * PKV_ERR_UNSUPPORTED; fp8 pools take pkv_paged_attention_prefill_fp8.
 */
pkv_status pkv_paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       const int32_t* query_start_loc, float scale, void* out, int32_t num_seqs,
                                       int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len, pkv_dtype kv_dtype,
                                       pkv_dtype out_dtype, void* stream);

/*
 * Chunked prefill over an fp8 cache: pkv_paged_attention_prefill with K =
 * decode(code) * k_scale[g] and V = decode(code) * v_scale[g] for KV head g
 * (fp8 format and pool layout as for pkv_reshape_and_cache_fp8).  The pages
 * name KV quantisation for long contexts (runbyai section 5) and chunked
 * prefill as the step that shares the batch with decode (architvora
 * "Continuous Batching"); this is the two together.  q is bf16; out is
 * out_dtype.  The codes are converted to bf16 exactly, so the products are
 * those of a bf16 cache holding the dequantised values.
 *   k_scale, v_scale  [device] fp32 [num_kv_heads], positive
 * Null scales return PKV_ERR_INVALID_ARG; otherwise as the bf16 entry point
 * (no workspace, requests 4096 per launch).
 */
pkv_status pkv_paged_attention_prefill_fp8(const void* q, const void* k_cache, const void* v_cache,
                                           const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                           const int32_t* context_lens, const int32_t* query_start_loc, float scale,
                                           void* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                           pkv_dtype out_dtype, void* stream);

/*
 * Measurement aid: the plain-read ceiling.  Decode is bound by memory
 * bandwidth (runbyai section 1) and reads its KV as fixed-size blocks
 * scattered through one pool (architvora "Paged Attention"); this call reads
 * bytes with 16-byte loads and nothing else, so its rate is the ceiling of
 * that access pattern on the device, reported beside the decode's.
 *   src        [device] buffer of `bytes` bytes (a positive multiple of 16),
 *              16-byte aligned
 *   tiles      NULL: read src front to back once.  Otherwise [device] int32
 *              [num_tiles]: read tile_bytes bytes at byte offset
 *              tiles[i] * tile_bytes for each i (entries outside the buffer
 *              are skipped)
 *   tile_bytes a power of two in [16, 2^24] (ignored when tiles is NULL)
 *   streaming  nonzero: non-temporal loads (as the decode's default);
 *              zero: ordinary loads
 *   sink       [device] uint32 [1024]; the kernel may write to it (it keeps
 *              the loads from being dropped); its contents mean nothing
 * One launch; asynchronous on `stream`.
 */
pkv_status pkv_hbm_read_bench(const void* src, int64_t bytes, const int32_t* tiles, int64_t num_tiles,
                              int32_t tile_bytes, int32_t streaming, uint32_t* sink, void* stream);

/*
 * Measurement aid: issue rates of the instructions the chunked-prefill
 * kernels are built from (prefill is the compute-heavy stage, runbyai
 * section 1).  One launch, one workgroup per compute unit of
 * 256 x waves_per_simd threads (one or two waves per SIMD); each wave runs
 * `iters` iterations of 16 instructions of one pattern:
 *   0, 1  mfma_f32_16x16x32_bf16 into 1 accumulator (one dependent chain) or 4
 *   2, 3  mfma_f32_32x32x16_bf16, likewise
 *   4     v_fma_f32, 16 independent chains
 *   5     v_exp_f32 each followed by a v_add_f32, 16 chains
 *   6     16-byte LDS reads, consecutive lanes on consecutive 16 bytes of a
 *         64 KiB array, one XOR each
 * Time it with events around the call on `stream`; the instruction counts
 * follow from the pattern, the number of compute units and the arguments.
 *   pattern          0 .. 6
 *   waves_per_simd   1 or 2
 *   iters            1 .. 10^7
 *   sink             device memory, at least 512 uint32 (written only in a
 *                    branch that is never taken)
 * Errors: PKV_ERR_INVALID_ARG for any argument out of range or a null sink.
 * Asynchronous on `stream`.
 */
pkv_status pkv_issue_rate_bench(int32_t pattern, int32_t waves_per_simd, int32_t iters, uint32_t* sink,
                                void* stream);

/*
 * Measurement aid: decode over a bf16 cache with every product on the vector
 * ALU instead of the matrix cores, to weigh the two for this bandwidth-bound
 * step (runbyai section 1).  Same result as pkv_paged_attention_decode within
 * the bf16 bar, not bit for bit: every product is an fp32 FMA of the widened
 * bf16 values.  It runs the fp32 path's kernel on bf16 elements (one wave
 * per partition x sequence x up to 8 query heads x KV head, query rows and
 * weights through LDS) and its split-K reduce; the work split differs from
 * the balanced matrix-core decode, so a comparison weighs the two designs.
 *   Arguments as pkv_paged_attention_decode with bf16 q and pools; the
 *   workspace is pkv_decode_workspace_bytes(..., PKV_F32) bytes (the fp32
 *   path's partials; 0 when every context fits in one partition).
 */
pkv_status pkv_paged_attention_decode_vector_alu(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_tables, const int32_t* context_lens,
                                                 float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int64_t num_blocks, int32_t max_blocks_per_seq,
                                                 int32_t max_context_len, int32_t partition_size, void* workspace,
                                                 size_t workspace_bytes, pkv_dtype out_dtype, void* stream);

/* Static description of a status code.  Never NULL. */
const char* pkv_status_string(pkv_status status);

/* Message of the last failed call on this host thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
