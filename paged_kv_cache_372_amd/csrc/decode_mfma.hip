// Paged decode attention, bf16 KV, on the gfx950 matrix cores, with the
// work balanced over the whole batch.
//
// What is computed: for every sequence and query head, softmax(scale q K^T) V
// over the sequence's cached tokens, which the kernel reaches by following
// the sequence's block table (runbyai section 1: decode attends over the
// cached KV of all earlier tokens; architvora "Paged Attention": the kernel
// follows the block table to gather the blocks).
//
// Work decomposition.  Take the blocks of all sequences in order, sequence
// after sequence: a flattened list of T blocks (the same list for every KV
// head).  It is cut into ranges of equal length and range r goes to
// workgroup column r mod W, so every workgroup walks the same number of
// blocks whatever the mix of context lengths -- no tail of long sequences.
// A range may start or end inside a sequence.  A sequence that lies wholly
// inside one range is finished in place (out = o / l); the pieces of a
// sequence that straddles ranges leave their (max, sum, unnormalised
// output) and a second kernel (splitk_reduce.hip) merges them with
// log-sum-exp weights.  (Merging in this kernel, by whichever wave brings
// the last piece of a sequence, was measured slower: the merge becomes a
// chain of dependent loads at the very end of the walk.)
//
// A workgroup holds one wave per KV head (up to 8); all its waves walk the
// same blocks, so at any moment they read the neighbouring 4 KiB tiles of
// the same physical block.  Each wave is persistent over its walk: the
// block-table window, the query rows and the next KV blocks are fetched
// ahead of use, across sequence and range boundaries, so a wave stalls on
// memory only once, at its start.
//
// With the fused append (a decode step's cache write in this launch, bf16
// or fp8 pools), the wave that walks a sequence's last block also stores
// the token the sequence gains this step; see the comment at its prologue.
//
// Per 16-token block, per wave:
//   S[16 tok x 16 heads] = K[16 x D] . Q^T[D x 16]  D/32 x mfma_f32_16x16x32_bf16
//   online softmax on S (exp2 domain, scale*log2e folded in)
//   O^T[D x 16 heads]  += V^T[D x 16] . P^T[16 x 16]   D/16 x mfma_f32_16x16x16_bf16
// P is fed as two bf16 terms (hi + lo), so the PV product carries about 16
// mantissa bits of the fp32 weights.  With bf16 pools and at most 8 heads in
// the group, the lo terms ride in the otherwise unused head columns 8..15 and
// one MFMA per 16 dims carries both; otherwise a second MFMA takes them.
// Over an fp8 cache the V codes are widened to fp16 (exactly) and P is
// rounded to fp16 once (11 significant bits): one fp16 MFMA per 16 dims.
//
// Why the pool layout is what it is: the MFMA A operand wants, in lane l,
// 8 consecutive K values of token (l % 16); with K stored as 16-byte chunks
// chunk-major inside a block ([D/8][16][8]), load kk of a wave reads one
// contiguous 1 KiB run.  The PV A operand wants 4 consecutive tokens of one
// dim; with V stored dim-major ([D][16]) each load reads a contiguous 512 B
// run.  The QK result layout (lane: head l%16, tokens 4(l/16)..+3) is
// exactly the PV B-operand layout, so no data moves between the two.
//
// Results depend only on logical token positions and the range split (a
// function of the context lengths and the launch width), never on where
// blocks sit in the pool.
#include <type_traits>

#include "e4m3.h"
#include "kernels.h"

namespace pkv {
namespace {

#ifndef PKV_PREFETCH_BLOCKS
#define PKV_PREFETCH_BLOCKS 3
#endif
constexpr int kPrefetchBlocks = PKV_PREFETCH_BLOCKS;  // KV blocks each wave keeps in flight
// An fp8 ring slot takes 3/4 of the registers of a bf16 one; a 4-deep fp8
// ring measured no faster, so fp8 keeps the same depth.
constexpr int kPrefetchBlocksFp8 = kPrefetchBlocks;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// One ring slot: a block's K and V tiles of this wave's KV head and the
// query rows of the block's sequence.
template <int D>
struct SlotRegs {
    uint4 k[D / 32];       // K chunks: load kk holds chunk 4kk + lane/16 of token lane%16
    uint2 v[D / 16];       // V^T: load c holds dim 16c + lane%16, tokens 4(lane/16)..+3
    bf16x8_t q[D / 32];    // Q^T as the B operand: column = head, k-group lane/16 holds chunk 4kk + lane/16
};

// The same for an fp8 (E4M3) cache: the raw codes, converted to bf16 operands
// when the block is used (the conversion is exact).  K: load i holds the
// 16-dim chunk 4i + lane/16 of token lane%16; the QK contraction takes dims in
// the order that makes step kk read half (kk & 1) of load kk/2, and q is
// loaded in that order.  V: load i holds the whole 16-token row of dim
// 64i + lane (16 bytes, a contiguous 1 KiB per wave); fp8_v_words regroups
// the rows across lanes into the PV operand layout.
template <int D>
struct SlotRegs8 {
    uint4 k[D / 64];
    uint4 v[D / 64];
    bf16x8_t q[D / 32];    // q step kk, k-group g: dims 64(kk/2) + 16g + 8(kk&1) .. +7
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    // codes of bytes 2*kHigh, 2*kHigh + 1; scale 1.0: the exact value of each code
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    // the same codes as fp16, also exact (E4M3: at most 448, 4 significant
    // bits, nothing below 2^-9 but zero)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHigh));
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed fp16, round to nearest even (one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, f16x2_t));
}

template <int D>
__device__ __forceinline__ bf16x8_t k_operand(const SlotRegs<D>& r, int kk) {
    return __builtin_bit_cast(bf16x8_t, r.k[kk]);
}
template <int D>
__device__ __forceinline__ bf16x8_t k_operand(const SlotRegs8<D>& r, int kk) {
    const uint4 w = r.k[kk >> 1];
    const uint32_t a = (kk & 1) ? w.z : w.x;
    const uint32_t b = (kk & 1) ? w.w : w.y;
    return __builtin_bit_cast(bf16x8_t, make_uint4(e4m3x2_to_bf16x2<false>(a), e4m3x2_to_bf16x2<true>(a),
                                                   e4m3x2_to_bf16x2<false>(b), e4m3x2_to_bf16x2<true>(b)));
}
// The V words of an fp8 slot in the PV operand layout: word c of lane
// (d = lane % 16, g = lane / 16) holds the codes of tokens 4g..4g+3 of dim
// 16c + d.  Lane (d, r) loaded dims 64i + 16r + d, word t = tokens 4t..4t+3:
// a 4 x 4 transpose of words between the four 16-lane rows, done with two
// rounds of row swaps (rows 2,3 <-> 0,1 of a register pair, then odd <->
// even rows).
template <int D>
__device__ __forceinline__ void fp8_v_words(const SlotRegs8<D>& r, uint32_t* w) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
        uint32_t x0 = r.v[i].x, x1 = r.v[i].y, x2 = r.v[i].z, x3 = r.v[i].w;
        const auto a = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
        x0 = a[0];
        x2 = a[1];
        x1 = b[0];
        x3 = b[1];
        const auto c = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);
        const auto e = __builtin_amdgcn_permlane16_swap(x2, x3, false, false);
        w[4 * i + 0] = c[0];
        w[4 * i + 1] = c[1];
        w[4 * i + 2] = e[0];
        w[4 * i + 3] = e[1];
    }
}

// Uniform facts about the block a ring slot holds.
struct SlotInfo {
    int seq;    // sequence
    int meta;   // valid tokens (0..16) | kSegLast | kSeqEnd
    int slot;   // partial row pair index, or -1 when the sequence completes here
    int pb;     // physical block loaded into the slot
};

constexpr int kSegLast = 1 << 5;  // this block ends a segment (sequence or range)
constexpr int kSeqEnd = 1 << 6;   // fused append: the sequence's last block, which holds its new token
constexpr int kAppendSlots = 4;   // fused append: new-token rows a wave keeps in LDS
constexpr int kCoherent = 16;     // buffer cache policy: sc1 (device scope, write-through)
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit raw data

struct SoftmaxState {
    float m;   // reference max (log2 units), same in all lanes of a head column
    float l;   // this lane's share of sum 2^(s - m)
};

// The reference max is raised only when a block's max exceeds it by more
// than 2^kRescaleSlack: until then the weights 2^(s - m) stay below 2^8,
// which fp32 holds exactly as well as weights below 1, and the accumulator
// rescale (a full pass over the output registers) is skipped.  The result is
// the same softmax; only the common reference of numerator and denominator
// moves less often.
constexpr float kRescaleSlack = 8.f;

// An fp8 V word (fp8_v_words) as an fp16 operand with the tokens past
// valid_n zeroed: one byte per token (tokens 4g..4g+3), so one mask serves
// all words.
__device__ __forceinline__ uint2 v_operand_fp8(uint32_t w, uint32_t vm) {
    w &= vm;
    return make_uint2(e4m3x2_to_f16x2<false>(w), e4m3x2_to_f16x2<true>(w));
}
template <int D>
__device__ __forceinline__ uint2 v_operand_masked(const SlotRegs<D>& r, int c, uint2 vm) {
    return make_uint2(r.v[c].x & vm.x, r.v[c].y & vm.y);
}

// Per-lane masks that zero V tokens 4g + j >= valid_n (valid_n < 16).
__device__ __forceinline__ uint32_t v_mask_fp8(int valid_n, int g) {
    const int nv = valid_n - 4 * g;
    return nv >= 4 ? 0xFFFFFFFFu : (nv <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * nv)));
}
__device__ __forceinline__ uint2 v_mask_bf16(int valid_n, int g) {
    const int nv = valid_n - 4 * g;
    return make_uint2(nv >= 2 ? 0xFFFFFFFFu : (nv == 1 ? 0x0000FFFFu : 0u),
                      nv >= 4 ? 0xFFFFFFFFu : (nv == 3 ? 0x0000FFFFu : 0u));
}

// kPackLo (group <= 8): head column c and column c + 8 hold the same query
// row, so both compute the same scores, softmax state and weights.  Column c
// feeds the weights truncated to bf16 to the PV product and column c + 8 the
// remainder, itself truncated to bf16 (together about 16 mantissa bits);
// finish_segment adds the two output columns.  One MFMA per 16 dims then
// carries both terms.  lo_mask is 0 in columns 0..7 and 0xFFFF0000 in
// columns 8..15.  Without kPackLo (group > 8) the two terms take two MFMAs.
template <int D, bool kPackLo, typename Slot>
__device__ __forceinline__ void compute_block(const Slot& r, float4_t* acc, SoftmaxState& st, int valid_n,
                                              float scale_log2, int g, uint32_t lo_mask) {
    // S = K . Q^T: lane holds S[token 4g + i][head lane%16], i = 0..3
    float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<D>(r, kk), r.q[kk], sacc, 0, 0, 0);

    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (4 * g + i < valid_n) ? sacc[i] * scale_log2 : -INFINITY;
    const float mx = max_over_groups(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const bool raise = mx > st.m + kRescaleSlack;
    if (__any(raise)) {
        const float alpha = raise ? exp2_fast(st.m - mx) : 1.f;   // st.m = -inf -> 0
        st.l *= alpha;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) acc[c] *= alpha;
        st.m = raise ? mx : st.m;
    }
    const float m_use = (st.m == -INFINITY) ? 0.f : st.m;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(sv[i] - m_use);
    st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    if constexpr (std::is_same_v<Slot, SlotRegs<D>>) {
        // P^T as the B operand: x = p - (p & lo_mask) is p itself in the hi
        // columns and p minus its bf16 truncation in the lo columns; the upper
        // 16 bits of x are the term the column feeds.
        uint32_t xw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t pb = __float_as_uint(pr[i]);
            xw[i] = kPackLo ? __float_as_uint(pr[i] - __uint_as_float(pb & lo_mask)) : pb;
        }
        const short4_t p_hi = __builtin_bit_cast(short4_t, make_uint2(__builtin_amdgcn_perm(xw[1], xw[0], 0x07060302u),
                                                                      __builtin_amdgcn_perm(xw[3], xw[2], 0x07060302u)));
        short4_t p_lo;
        if constexpr (!kPackLo) {
            uint32_t lw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) lw[i] = __float_as_uint(pr[i] - __uint_as_float(xw[i] & 0xFFFF0000u));
            p_lo = __builtin_bit_cast(short4_t, make_uint2(__builtin_amdgcn_perm(lw[1], lw[0], 0x07060302u),
                                                           __builtin_amdgcn_perm(lw[3], lw[2], 0x07060302u)));
        }
        // tokens past the end hold stale or NaN data: zero them (0 * NaN =
        // NaN); only the last block of a sequence has such tokens
        const uint2 vm = valid_n < 16 ? v_mask_bf16(valid_n, g) : make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            const short4_t a = __builtin_bit_cast(short4_t, v_operand_masked<D>(r, c, vm));
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, p_hi, acc[c], 0, 0, 0);
            if constexpr (!kPackLo) acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, p_lo, acc[c], 0, 0, 0);
        }
    } else {
        // fp8 pools: V widened to fp16 (exact) and the weights rounded to
        // fp16 once (11 significant bits), one fp16 MFMA per 16 dims.
        const f16x4_t p16 = __builtin_bit_cast(f16x4_t, make_uint2(pack_f16x2(pr[0], pr[1]), pack_f16x2(pr[2], pr[3])));
        const uint32_t vm = valid_n < 16 ? v_mask_fp8(valid_n, g) : 0xFFFFFFFFu;
        uint32_t w[D / 16];
        fp8_v_words<D>(r, w);
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, v_operand_fp8(w[c], vm)), p16,
                                                           acc[c], 0, 0, 0);
    }
}

// Walk-position window: lane i describes position base + i of the wave's
// walk.  Built from the LDS tables only; the block-table entry itself is
// read later through the scalar cache.
struct Window {
    int seq;    // sequence
    int blk;    // logical block within the sequence
    int meta;   // valid tokens (1..16) | kSegLast | kSeqEnd
    int slot;   // partial row pair index, -1 = the sequence completes in this range
};

// A block-table entry fetched ahead of its ring refill, with the facts
// about its block.
struct Pending {
    int raw;    // physical block id as read from the table (validated at use)
    SlotInfo info;
};

typedef const int32_t __attribute__((address_space(4)))* scalar_i32_ptr;

// Dynamic LDS of the balanced kernel: the flattened offsets and lengths of
// the batch ([B + 1] and [B] int32), then, with the fused append, each
// wave's kAppendSlots new-token rows (K and V, D pool elements each: bf16,
// or E4M3 codes) from a 16-byte boundary.
__host__ __device__ inline int append_rows_offset(int num_seqs) { return (2 * num_seqs + 1 + 3) & ~3; }

template <int D, int kDepth, bool kCached, bool kFp8, bool kPackLo>
__global__ __launch_bounds__(64 * kMaxWavesPerGroup) void decode_bf16_balanced_kernel(DecodeParams p) {
    using Elem = std::conditional_t<kFp8, uint8_t, uint16_t>;  // one K/V pool element
    using Slot = std::conditional_t<kFp8, SlotRegs8<D>, SlotRegs<D>>;
    extern __shared__ __align__(16) int32_t tables[];
    __shared__ int32_t wave_total[kMaxWavesPerGroup];
    const int B = p.num_seqs;
    int32_t* s_off = tables;          // [B + 1] first flattened block of each sequence
    int32_t* s_len = tables + B + 1;  // [B] clamped context length
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nthr = blockDim.x;
    const int walker = blockIdx.x / p.head_unit_groups;
    const int hug = blockIdx.x - walker * p.head_unit_groups;

    // ---- flattened block offsets of the batch (exclusive prefix sums)
    {
        const int per = (B + nthr - 1) / nthr;
        const int i0 = min(B, tid * per);
        const int i1 = min(B, i0 + per);
        int sum = 0;
        for (int i = i0; i < i1; ++i) {
            const int L = clamp_ctx(p.context_lens[i], p.ctx_cap);
            s_len[i] = L;
            sum += (L + kBlockSize - 1) / kBlockSize;
        }
        int x = sum;  // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (lane == 63) wave_total[wave] = x;
        __syncthreads();
        int run = x - sum;
        for (int w = 0; w < wave; ++w) run += wave_total[w];
        for (int i = i0; i < i1; ++i) {
            s_off[i] = run;
            run += (s_len[i] + kBlockSize - 1) / kBlockSize;
        }
        if (tid == nthr - 1) s_off[B] = run;
        __syncthreads();
    }
    if (walker == 0 && hug == 0)
        for (int i = tid; i <= B; i += nthr) p.seq_off[i] = s_off[i];

    const int hu = hug * p.waves_per_group + wave;
    if (hu >= p.head_units) return;  // no barrier follows
    const int kvh = hu % p.num_kv_heads;
    const int hg = hu / p.num_kv_heads;
    const int col = lane & 15;  // head column of the MFMA tiles
    const int g = lane >> 4;    // lane group
    const int Hq = p.num_q_heads;
    const int h0 = kvh * p.group + hg * kMfmaHeadsPerUnit;
    const int nh = min(kMfmaHeadsPerUnit, p.group - hg * kMfmaHeadsPerUnit);

    // Store one output row group: lane (col, g) holds dims 16c + 4g .. +3 of
    // head h0 + col; only the group's nh heads are written.
    auto store_out = [&](int seq, const float4_t* v, float scale) {
        if (col >= nh) return;
        const int64_t o = ((int64_t)seq * Hq + h0 + col) * D + 4 * g;
        if (p.out_bf16) {
            uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + o;
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                *reinterpret_cast<uint2*>(ob + 16 * c) =
                    make_uint2(f32_to_bf16_bits(v[c][0] * scale) | (f32_to_bf16_bits(v[c][1] * scale) << 16),
                               f32_to_bf16_bits(v[c][2] * scale) | (f32_to_bf16_bits(v[c][3] * scale) << 16));
        } else {
            float* of = reinterpret_cast<float*>(p.out) + o;
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                *reinterpret_cast<float4*>(of + 16 * c) =
                    make_float4(v[c][0] * scale, v[c][1] * scale, v[c][2] * scale, v[c][3] * scale);
        }
    };

    const int T = s_off[B];
    const int NG = p.walkers;
    int CS, NR;
    range_geometry(T, NG, p.range_cap, CS, NR);
    if (walker >= NR) return;
    const int n_ranges = (NR - 1 - walker) / NG + 1;
    const int r_final = walker + NG * (n_ranges - 1);
    const int K = (n_ranges - 1) * CS + min(CS, T - r_final * CS);  // blocks this workgroup walks
    const bool appending = p.k_new != nullptr;  // fused append of the new tokens

    // last sequence starting at or before flattened block f (it holds block f)
    auto seq_of_block = [&](int f) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= f) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    // columns past the group repeat the group's last head: finite values,
    // never stored, and the softmax never mixes head columns.  With kPackLo
    // column c + 8 repeats column c.
    const int qcol = min(kPackLo ? (col & 7) : col, nh - 1);
    const uint32_t lo_mask = (kPackLo && col >= 8) ? 0xFFFF0000u : 0u;

    const int64_t block_stride = (int64_t)p.num_kv_heads * D * kBlockSize;
    const Elem* k_head = reinterpret_cast<const Elem*>(p.k_cache) + (int64_t)kvh * D * kBlockSize;
    const Elem* v_head = reinterpret_cast<const Elem*>(p.v_cache) + (int64_t)kvh * D * kBlockSize;
    // an fp8 cache: K's scale folds into the score scale, V's into the output
    const float score_scale = kFp8 ? p.scale_log2 * p.k_scale[kvh] : p.scale_log2;
    const float out_scale = kFp8 ? p.v_scale[kvh] : 1.f;
    const uint16_t* q_base = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)(h0 + qcol) * D;

    // Describe walk positions [base, base + 64).
    auto build_window = [&](int base, Window& w) {
        const int k = base + lane;
        w.seq = 0;
        w.blk = 0;
        w.meta = 0;
        w.slot = -1;
        if (k < K) {
            const int ri = k / CS;
            const int r = walker + NG * ri;
            const int rs = r * CS;
            const int re = min(rs + CS, T);
            const int f = rs + (k - ri * CS);
            const int lo = seq_of_block(f);
            const int o0 = s_off[lo];
            const int o1 = s_off[lo + 1];
            const int j = f - o0;
            w.seq = lo;
            w.blk = j;
            w.meta = min(kBlockSize, s_len[lo] - j * kBlockSize) | ((f == re - 1 || f == o1 - 1) ? kSegLast : 0) |
                     (appending && f == o1 - 1 ? kSeqEnd : 0);
            w.slot = (o0 >= rs && o1 <= re) ? -1 : range_slot(r, CS, o0);
        }
    };

    Window cur, nxt;
    int win_base = 0;
    build_window(0, cur);
    build_window(64, nxt);
    const scalar_i32_ptr bt = (scalar_i32_ptr)p.block_tables;

    // Table entry and facts of walk position k (clamped to the last one).
    // Positions are asked for in increasing order, one at a time.
    auto fetch = [&](int k, Pending& e) {
        const int kc = min(k, K - 1);
        if (kc >= win_base + 64) {
            win_base += 64;
            cur = nxt;
            build_window(win_base + 64, nxt);
        }
        const int li = kc - win_base;
        const int seq = __builtin_amdgcn_readlane(cur.seq, li);
        const int blk = __builtin_amdgcn_readlane(cur.blk, li);
        e.raw = bt[(int64_t)seq * p.max_blocks_per_seq + blk];
        e.info.seq = seq;
        e.info.meta = __builtin_amdgcn_readlane(cur.meta, li);
        e.info.slot = __builtin_amdgcn_readlane(cur.slot, li);
    };

    // Fused append (p.k_new set): the token each sequence gains this step
    // goes to position L - 1, in the sequence's last block.  For each KV
    // head that block is walked by exactly one wave (the launch has one
    // head group per KV head), the one whose range holds it, so that wave
    // does the whole append: it keeps the token's K/V rows in its LDS rows
    // (the first kAppendSlots tokens of its walk), writes them into the
    // block's registers once the block's loads have arrived, and stores
    // them into the pool when its walk is done.  The wave never reads pool
    // lines it has written, and no other wave reads the slot.  Tokens past the
    // first kAppendSlots of a walk (short sequences) are stored into the
    // pool before the walk instead, and read back from it.  A table entry
    // outside the pool is skipped, as the walk skips it.  The new rows are
    // bf16; into an fp8 pool they go as the codes the quantising cache write
    // stores (e4m3_encode with the KV head's scales), encoded once, when they
    // enter LDS or the pool, each lane encoding its own dims.
    // LDS rows: K then V, D pool elements each
    Elem* const ap_rows = reinterpret_cast<Elem*>(tables + append_rows_offset(B)) + wave * (kAppendSlots * 2 * D);
    constexpr int kRowChunks = D * (int)sizeof(Elem) / 16;  // 16-byte chunks of a row as the pool holds it
    // next sequence, from cursor (ri, s) on, whose last block lies in range
    // ri of this walk; -1 when none is left
    auto next_append = [&](int& ri, int& s) -> int {
        for (; ri < n_ranges; ++ri) {
            const int rs = (walker + NG * ri) * CS;
            const int re = min(rs + CS, T);
            if (s < 0) s = __builtin_amdgcn_readfirstlane(seq_of_block(rs));
            for (; s < B; ++s) {
                const int o0 = __builtin_amdgcn_readfirstlane(s_off[s]);
                if (o0 >= re) break;
                const int o1 = __builtin_amdgcn_readfirstlane(s_off[s + 1]);
                if (o1 > o0 && o1 > rs && o1 <= re) return s++;
            }
            s = -1;
        }
        return -1;
    };
    // A new token's rows as loaded (bf16 bits).  bf16 pools: lanes <
    // kRowChunks hold the 8 dims of K chunk `lane`.  fp8 pools: every lane
    // holds K dims lane + 64i (an fp8 K row as the pool holds it is its codes
    // in dim order, chunk c being dims 16c..16c+15, so each lane encodes its
    // own dims).  V: dims lane + 64i.
    struct NewRow {
        uint4 k;
        uint32_t kd[(D + 63) / 64];
        uint32_t v[(D + 63) / 64];
    };
    auto load_new_row = [&](int s, NewRow& a) {
        const int64_t src = ((int64_t)s * p.num_kv_heads + kvh) * D;
        const uint16_t* kn = reinterpret_cast<const uint16_t*>(p.k_new) + src;
        if constexpr (kFp8) {
#pragma unroll
            for (int i = 0; i < (D + 63) / 64; ++i) a.kd[i] = lane + 64 * i < D ? kn[lane + 64 * i] : 0u;
        } else {
            a.k = lane < kRowChunks ? reinterpret_cast<const uint4*>(kn)[lane] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < (D + 63) / 64; ++i)
            a.v[i] = lane + 64 * i < D ? reinterpret_cast<const uint16_t*>(p.v_new)[src + lane + 64 * i] : 0u;
    };
    // fp8 pools: the code of a bf16 value, with the KV head's K or V scale
    const float ks_new = kFp8 ? p.k_scale[kvh] : 1.f;
    const float vs_new = kFp8 ? p.v_scale[kvh] : 1.f;
    auto encode = [&](uint32_t bits, float scale) -> Elem {
        return (Elem)e4m3_encode(__uint_as_float(bits << 16), scale);
    };
    Elem* const kc_base = reinterpret_cast<Elem*>(const_cast<void*>(p.k_cache)) + (int64_t)kvh * D * kBlockSize;
    Elem* const vc_base = reinterpret_cast<Elem*>(const_cast<void*>(p.v_cache)) + (int64_t)kvh * D * kBlockSize;
    int ap_ri = 0, ap_s = -1;
    int ap_count = 0;  // rows kept in LDS
    int ap_used = 0;   // sequence ends the walk has reached
    NewRow ap_row[kAppendSlots];
    if (appending) {
        // rows of the first kAppendSlots ends, requested before the walk's
        // first table fetches and written to LDS once its first KV loads are
        // issued
#pragma unroll
        for (int j = 0; j < kAppendSlots; ++j) {
            const int s = ap_count == j ? next_append(ap_ri, ap_s) : -1;
            if (s >= 0) {
                load_new_row(s, ap_row[j]);
                ++ap_count;
            }
        }
    }
    // The kept rows into this wave's LDS rows.  Called once the walk's
    // first KV loads are issued, so the wait for the rows is not on the
    // walk's start-up chain (the rows are read when their block is
    // computed).  Llama-shaped batch, fused decode launch, same session:
    // 99.3-100.0 us against 99.6-100.7 us with the rows written before the
    // first loads.
    auto append_rows_to_lds = [&]() {
#pragma unroll
        for (int j = 0; j < kAppendSlots; ++j) {
            if (j < ap_count) {
                Elem* r = ap_rows + j * 2 * D;
                if constexpr (kFp8) {
#pragma unroll
                    for (int i = 0; i < (D + 63) / 64; ++i)
                        if (lane + 64 * i < D) {
                            r[lane + 64 * i] = encode(ap_row[j].kd[i], ks_new);
                            r[D + lane + 64 * i] = encode(ap_row[j].v[i], vs_new);
                        }
                } else {
                    if (lane < kRowChunks) reinterpret_cast<uint4*>(r)[lane] = ap_row[j].k;
#pragma unroll
                    for (int i = 0; i < (D + 63) / 64; ++i)
                        if (lane + 64 * i < D) r[D + lane + 64 * i] = (Elem)ap_row[j].v[i];
                }
            }
        }
    };
    // The ends past the first kAppendSlots of the walk, stored into the pool
    // before the walk's first loads (which then read them back).
    auto append_overflow = [&]() {
        if (ap_count < kAppendSlots) return;
        for (int s = next_append(ap_ri, ap_s); s >= 0; s = next_append(ap_ri, ap_s)) {
            const int pos = __builtin_amdgcn_readfirstlane(s_len[s]) - 1;
            const int e = bt[(int64_t)s * p.max_blocks_per_seq + pos / kBlockSize];
            NewRow a;
            load_new_row(s, a);
            if (e < 0 || (int64_t)e >= p.num_blocks) continue;
            const int o = pos % kBlockSize;
            Elem* kc = kc_base + (int64_t)e * block_stride;
            Elem* vc = vc_base + (int64_t)e * block_stride;
            // K tile [D*sizeof(Elem)/16][16][16 bytes]: chunk c of token o at
            // 16-byte unit 16c + o (fp8: dim d is byte d % 16 of chunk d / 16);
            // V tile [D][16]: dim d of token o at 16d + o
            if constexpr (kFp8) {
#pragma unroll
                for (int i = 0; i < (D + 63) / 64; ++i) {
                    const int d = lane + 64 * i;
                    if (d < D) {
                        kc[((d >> 4) * kBlockSize + o) * 16 + (d & 15)] = encode(a.kd[i], ks_new);
                        vc[d * kBlockSize + o] = encode(a.v[i], vs_new);
                    }
                }
            } else {
                if (lane < kRowChunks) reinterpret_cast<uint4*>(kc)[lane * kBlockSize + o] = a.k;
#pragma unroll
                for (int i = 0; i < (D + 63) / 64; ++i)
                    if (lane + 64 * i < D) vc[(lane + 64 * i) * kBlockSize + o] = (Elem)a.v[i];
            }
        }
    };
    // The new token (position o of the block in ring slot r, LDS row j) in
    // the slot's operand registers.  bf16: K chunk 4kk + g of token
    // lane % 16, and V dims 16c + lane % 16 of tokens 4g..4g+3 (two per
    // 32-bit word).  fp8: K code chunk 4i + g of token lane % 16, and byte o
    // of the 16 codes of dim 64i + lane.
    auto patch_slot = [&](Slot& r, int j, int o) {
        const Elem* row = ap_rows + j * 2 * D;
        const bool kt = (lane & 15) == o;
        if constexpr (kFp8) {
#pragma unroll
            for (int i = 0; i < D / 64; ++i) {
                const uint4 w = reinterpret_cast<const uint4*>(row)[4 * i + g];
                if (kt) r.k[i] = w;
            }
            const uint32_t sh = (o & 3) * 8;
            const uint32_t keep = ~(0xFFu << sh);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) {
                const uint32_t x = (uint32_t)row[D + 64 * i + lane] << sh;
                switch (o >> 2) {  // the same in every lane
                    case 0: r.v[i].x = (r.v[i].x & keep) | x; break;
                    case 1: r.v[i].y = (r.v[i].y & keep) | x; break;
                    case 2: r.v[i].z = (r.v[i].z & keep) | x; break;
                    default: r.v[i].w = (r.v[i].w & keep) | x; break;
                }
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const uint4 w = reinterpret_cast<const uint4*>(row)[4 * kk + g];
                if (kt) r.k[kk] = w;
            }
            const bool vt = g == (o >> 2);
            const uint32_t sh = (o & 1) * 16;
            const uint32_t keep = ~(0xFFFFu << sh);
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const uint32_t x = (uint32_t)row[D + 16 * c + (lane & 15)] << sh;
                if (vt) {
                    if (o & 2) r.v[c].y = (r.v[c].y & keep) | x;
                    else r.v[c].x = (r.v[c].x & keep) | x;
                }
            }
        }
    };
    // The new token of LDS row j into position o of pool block pb, after
    // the walk's last wait.  On this chip stores share the in-order counter
    // of the loads, so a store issued inside the walk makes the next waits
    // for KV blocks wait on it too.  Measured on the Llama-shaped batch
    // (decode launch): stores after the walk 100.6 us; the token stored
    // when its block is reached 103.9 us; the whole patched tile written
    // back there 105.5 us; the token stored into the pool before the walk
    // and read back 102.6 us (streaming stores) or 108.5 us (ordinary);
    // later, with the token still patched into the registers, stored right
    // after the walk's first KV loads were issued: 103.9-104.4 us against
    // 99.7-100.1 us stored after the walk (same session) -- the
    // acknowledgement of a store under the full read stream stalls the
    // wait that first covers it.
    auto store_token = [&](int j, int pb, int o) {
        const Elem* row = ap_rows + j * 2 * D;
        Elem* kc = kc_base + (int64_t)pb * block_stride;
        Elem* vc = vc_base + (int64_t)pb * block_stride;
        if (lane < kRowChunks)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, reinterpret_cast<const uint4*>(row)[lane]),
                                        reinterpret_cast<u32x4_t*>(kc) + lane * kBlockSize + o);
#pragma unroll
        for (int i = 0; i < (D + 63) / 64; ++i)
            if (lane + 64 * i < D) __builtin_nontemporal_store(row[D + lane + 64 * i], vc + (lane + 64 * i) * kBlockSize + o);
    };
    int ap_pb[kAppendSlots], ap_o[kAppendSlots];
#pragma unroll
    for (int j = 0; j < kAppendSlots; ++j) ap_pb[j] = ap_o[j] = -1;

    Slot ring[kDepth];
    SlotInfo info[kDepth];
    Pending pend[kDepth];

    // A fetched table entry, checked: the physical block to load (an id
    // outside the pool loads block 0 with no valid token).  The empty asm
    // pins the check here, so the wait for the scalar load happens now and
    // not where the block is loaded.
    auto accept = [&](const Pending& e, int& pb, SlotInfo& inf) {
        const bool ok = e.raw >= 0 && (int64_t)e.raw < p.num_blocks;
        pb = ok ? e.raw : 0;
        inf = e.info;
        if (!ok) inf.meta &= kSegLast | kSeqEnd;
        asm volatile("" : "+s"(pb));
    };

    // Fill ring slot d with physical block pb.  Every refill issues the same
    // vector loads, so the wait before a block covers only that block's loads.
    auto load_slot = [&](int d, int pb, const SlotInfo& inf) {
        info[d] = inf;
        info[d].pb = pb;
        const uint4* qr = reinterpret_cast<const uint4*>(q_base + (int64_t)info[d].seq * Hq * D);
        if constexpr (kFp8) {
            const u32x4_t* kt = reinterpret_cast<const u32x4_t*>(k_head + (int64_t)pb * block_stride);
            const u32x4_t* vt = reinterpret_cast<const u32x4_t*>(v_head + (int64_t)pb * block_stride);
#pragma unroll
            for (int i = 0; i < D / 64; ++i)
                ring[d].k[i] = __builtin_bit_cast(uint4, kCached ? kt[i * 64 + lane]
                                                                 : __builtin_nontemporal_load(kt + i * 64 + lane));
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                ring[d].q[kk] = __builtin_bit_cast(bf16x8_t, qr[8 * (kk >> 1) + 2 * g + (kk & 1)]);
#pragma unroll
            for (int i = 0; i < D / 64; ++i)
                ring[d].v[i] = __builtin_bit_cast(uint4, kCached ? vt[i * 64 + lane]
                                                                 : __builtin_nontemporal_load(vt + i * 64 + lane));
        } else {
            const u32x4_t* kt = reinterpret_cast<const u32x4_t*>(k_head + (int64_t)pb * block_stride);
            const u32x2_t* vt = reinterpret_cast<const u32x2_t*>(v_head + (int64_t)pb * block_stride);
            // Streaming (the default): each KV tile is read once, so non-temporal
            // loads keep it from displacing reusable lines (q, tables) and
            // measurably raise the rate.  kCached: sequences share blocks, so
            // ordinary loads leave them in the caches for the next reader.
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                ring[d].k[kk] = __builtin_bit_cast(uint4, kCached ? kt[kk * 64 + lane]
                                                                  : __builtin_nontemporal_load(kt + kk * 64 + lane));
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) ring[d].q[kk] = __builtin_bit_cast(bf16x8_t, qr[4 * kk + g]);
            // (bf16 V in 16-byte loads, regrouped across lanes as for fp8,
            // measured slightly slower: 8-byte loads are kept here)
            const int vo = (lane & 15) * 4 + (lane >> 4);
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                ring[d].v[c] = __builtin_bit_cast(uint2, kCached ? vt[c * 64 + vo]
                                                                 : __builtin_nontemporal_load(vt + c * 64 + vo));
        }
    };

    float4_t acc[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) acc[c] = {0.f, 0.f, 0.f, 0.f};
    SoftmaxState st{-INFINITY, 0.f};

    // the partial rows, addressed as one buffer
    const __amdgpu_buffer_rsrc_t part_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(p.o_part, (short)0, (int)p.part_bytes, kBufferWord3);

    // End of a segment: finish the sequence (out = o / l) or leave the
    // piece's statistics for the merge, then start afresh.
    auto finish_segment = [&](int seq, int slot) {
        const float l_tot = sum_over_groups(st.l);
        if constexpr (kPackLo) {
            // output column c = hi term (column c) + lo term (column c + 8);
            // row_ror:8 gives every lane the other half of its pair
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[c][j] += __int_as_float(
                        __builtin_amdgcn_update_dpp(0, __float_as_int(acc[c][j]), 0x128, 0xF, 0xF, false));
        }
        if (col < nh) {
            if (slot < 0) {
                store_out(seq, acc, l_tot > 0.f ? out_scale / l_tot : 0.f);
            } else {
                if constexpr (kFp8) {
#pragma unroll
                    for (int c = 0; c < D / 16; ++c) acc[c] *= out_scale;
                }
                // write-through stores (sc1): the rows are read once, by the
                // reduce kernel, so they need not sit dirty in this XCD's L2
                // (measured faster than plain stores when pieces are many)
                const int64_t row = (int64_t)slot * Hq + h0 + col;
                const int ob = (int)((row * D + 4 * g) * sizeof(float));
#pragma unroll
                for (int c = 0; c < D / 16; ++c)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[c]), part_rsrc,
                                                           ob + 64 * c, 0, kCoherent);
                if (g == 0) {
                    __hip_atomic_store(p.m_part + row, st.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(p.l_part + row, l_tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < D / 16; ++c) acc[c] = {0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.f;
    };

    // Table entries travel through the scalar cache, whose loads complete
    // out of order: any wait for one waits for all in flight.  So the
    // entries are fetched in one burst at the top of an iteration and used
    // at the top of the next, with no scalar load issued in between --
    // the wait then finds them long arrived.  The scheduling barriers keep
    // each refill's vector loads together and in slot order, in the prologue
    // as in the loop, so the count of loads issued after a slot's loads is
    // the same on every path into the loop and the compiler waits for
    // exactly that slot.
    int next_pb[kDepth];
    SlotInfo next_info[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) fetch(d, pend[d]);
    if (appending) append_overflow();
#pragma unroll
    for (int d = 0; d < kDepth; ++d) accept(pend[d], next_pb[d], next_info[d]);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) fetch(kDepth + d, pend[d]);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        load_slot(d, next_pb[d], next_info[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (appending) append_rows_to_lds();
    __builtin_amdgcn_sched_barrier(0);
    // One round: compute the kDepth blocks in the ring, refilling each slot
    // with the block kDepth positions further on.  In the last rounds the
    // refills past the walk's end are skipped (kFinal); before that every
    // refill is issued, which keeps the loop's waits exact.
    //
    // The waves of a workgroup run in lockstep: a barrier at the top of
    // every round (no memory wait; every wave of the workgroup walks the
    // same ranges, so all run the same rounds).  Two waves share each SIMD,
    // and left alone one of them ran ahead: wave timestamps (s_memrealtime)
    // on 8 x 128k tokens showed the waves of one compute unit finishing up
    // to ~240 us apart around a 700 us launch, every compute unit alike,
    // and the unit slowing once its fast waves were done (the last 10 % of
    // the blocks took a fifth of the launch).  Whatever the cause (wave
    // priorities, KV-head order and four-wave workgroups were tried), in
    // lockstep the unit keeps all eight waves' loads in flight to the end.
    // Measured (rocprof, same session): 8 x 128k decode 672 us against 693
    // (eight waves, no barrier) and 691-695 (two four-wave workgroups per
    // unit); the Llama-shaped batch 94.1-94.7 us against 94.6.
    auto round = [&](int i, auto final_tag) {
        constexpr bool kFinal = decltype(final_tag)::value;
        __builtin_amdgcn_s_barrier();
        // entries of positions i + kDepth + d, fetched one round ago
#pragma unroll
        for (int d = 0; d < kDepth; ++d) accept(pend[d], next_pb[d], next_info[d]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < kDepth; ++d) fetch(i + 2 * kDepth + d, pend[d]);
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (!kFinal || i + d < K) {
                // fused append: the block that holds a sequence's new token
                bool patched = false;
                if (info[d].meta & kSeqEnd) {
                    const int nv = info[d].meta & 31;
                    patched = ap_used < ap_count && nv > 0;
                    if (patched) patch_slot(ring[d], ap_used, nv - 1);
                    ++ap_used;
                }
                compute_block<D, kPackLo>(ring[d], acc, st, info[d].meta & 31, score_scale, g, lo_mask);
                if (info[d].meta & kSegLast) {
                    finish_segment(info[d].seq, info[d].slot);
                    if (patched) {  // stored after the walk
#pragma unroll
                        for (int j = 0; j < kAppendSlots; ++j)
                            if (j == ap_used - 1) {
                                ap_pb[j] = info[d].pb;
                                ap_o[j] = (info[d].meta & 31) - 1;
                            }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (!kFinal || i + d + kDepth < K) load_slot(d, next_pb[d], next_info[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int i = 0;
    for (; i + 2 * kDepth <= K; i += kDepth) round(i, std::false_type{});
    for (; i < K; i += kDepth) round(i, std::true_type{});
    // fused append: the new tokens patched in above, into the pool
#pragma unroll
    for (int j = 0; j < kAppendSlots; ++j)
        if (ap_pb[j] >= 0) store_token(j, ap_pb[j], ap_o[j]);

}

}  // namespace

size_t balanced_lds_bytes(int32_t num_seqs) { return (size_t)(2 * num_seqs + 1) * sizeof(int32_t); }

size_t balanced_lds_bytes(const DecodeParams& p) {
    if (p.k_new == nullptr) return balanced_lds_bytes(p.num_seqs);
    return (size_t)append_rows_offset(p.num_seqs) * sizeof(int32_t) +
           (size_t)p.waves_per_group * kAppendSlots * 2 * p.head_dim * (p.kv_fp8 ? 1 : sizeof(uint16_t));
}

const void* balanced_kernel(int32_t head_dim) {
    // the plan sizes the grid from the occupancy of the streaming bf16
    // variant with packed lo terms (the one bf16 groups of up to 8 heads
    // run); the other variants need no more registers or LDS
    return head_dim == 128
               ? reinterpret_cast<const void*>(&decode_bf16_balanced_kernel<128, kPrefetchBlocks, false, false, true>)
               : reinterpret_cast<const void*>(&decode_bf16_balanced_kernel<64, kPrefetchBlocks, false, false, true>);
}

template <int D, bool kFp8, bool kPackLo>
void launch_balanced(const DecodeParams& p, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
    constexpr int kDepth = kFp8 ? kPrefetchBlocksFp8 : kPrefetchBlocks;
    if (p.cached_kv)
        hipLaunchKernelGGL((decode_bf16_balanced_kernel<D, kDepth, true, kFp8, kPackLo>), grid, block, lds, stream, p);
    else
        hipLaunchKernelGGL((decode_bf16_balanced_kernel<D, kDepth, false, kFp8, kPackLo>), grid, block, lds, stream, p);
}

// The packed lo terms are used for bf16 pools only; fp8 pools take fp16
// weights, one MFMA per 16 dims (compute_block).
template <int D, bool kFp8>
void launch_balanced(const DecodeParams& p, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
    if (!kFp8 && p.group <= kMfmaHeadsPerUnit / 2) launch_balanced<D, false, true>(p, grid, block, lds, stream);
    else launch_balanced<D, kFp8, false>(p, grid, block, lds, stream);
}

hipError_t launch_decode_bf16_balanced(const DecodeParams& p, hipStream_t stream) {
    if (p.num_seqs == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.walkers * p.head_unit_groups)), block(64 * p.waves_per_group);
    const size_t lds = balanced_lds_bytes(p);
    if (p.kv_fp8) {
        if (p.head_dim == 128) launch_balanced<128, true>(p, grid, block, lds, stream);
        else launch_balanced<64, true>(p, grid, block, lds, stream);
    } else {
        if (p.head_dim == 128) launch_balanced<128, false>(p, grid, block, lds, stream);
        else launch_balanced<64, false>(p, grid, block, lds, stream);
    }
    return hipGetLastError();
}

}  // namespace pkv
