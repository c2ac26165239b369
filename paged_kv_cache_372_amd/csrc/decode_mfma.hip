// Paged decode attention, bf16 KV, on the gfx950 matrix cores.
//
// What is computed: for one sequence, one KV head and the query heads that
// share it (grouped-query attention), walk the sequence's block table over
// one partition of its context, and produce softmax(scale q K^T) V for that
// partition (runbyai section 1: decode attends over the cached KV of all
// earlier tokens; architvora "Paged Attention": the kernel follows the block
// table to gather the blocks).  Long contexts are split into partitions
// whose (max, sum, unnormalised output) statistics are merged by
// splitk_reduce.hip.
//
// Work decomposition: one wave64 per unit (partition, sequence, head group,
// KV head).  The unit id puts the KV head in the lowest digit, so with 8 KV
// heads consecutive workgroups -- dealt round-robin to the 8 XCDs -- keep
// each KV head on one XCD and its L2 (shared-prefix blocks stay resident).
//
// Per 16-token block, per wave:
//   S[16 tok x 16 heads] = K[16 x D] . Q^T[D x 16]  D/32 x mfma_f32_16x16x32_bf16
//   online softmax on S (exp2 domain, scale*log2e folded in)
//   O^T[D x 16 heads]  += V^T[D x 16] . P^T[16 x 16]   D/16 x 2 x mfma_f32_16x16x16_bf16
// P is fed as two bf16 terms (hi + lo), so the PV product carries about 16
// mantissa bits of the fp32 weights.  Unused head columns (group < 16) cost
// matrix-core cycles only; the kernel is bound by HBM, not by the MFMA pipe.
//
// Why the pool layout is what it is: the MFMA A operand wants, in lane l,
// 8 consecutive K values of token (l % 16); with K stored as 16-byte chunks
// chunk-major inside a block ([D/8][16][8]), load kk of a wave reads one
// contiguous 1 KiB run.  The PV A operand wants 4 consecutive tokens of one
// dim; with V stored dim-major ([D][16]) each load reads a contiguous 512 B
// run.  The QK result layout (lane: head l%16, tokens 4(l/16)..+3) is
// exactly the PV B-operand layout, so no data moves between the two.
#include "kernels.h"

namespace pkv {
namespace {

#ifndef PKV_PREFETCH_BLOCKS
#define PKV_PREFETCH_BLOCKS 3
#endif
constexpr int kPrefetchBlocks = PKV_PREFETCH_BLOCKS;  // KV blocks each wave keeps in flight
#ifndef PKV_WAVES_PER_UNIT
#define PKV_WAVES_PER_UNIT 4
#endif
constexpr int kWavesPerUnit = PKV_WAVES_PER_UNIT;  // waves sharing one unit's blocks

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int D>
struct BlockRegs {
    uint4 k[D / 32];   // K chunks: load kk holds chunk 4kk + lane/16 of token lane%16
    uint2 v[D / 16];   // V^T: load c holds dim 16c + lane%16, tokens 4(lane/16)..+3
};

template <int D>
__device__ __forceinline__ void load_block(BlockRegs<D>& r, const uint16_t* __restrict__ k_head,
                                           const uint16_t* __restrict__ v_head, int64_t block_stride,
                                           int pb, int lane) {
    const uint4* kt = reinterpret_cast<const uint4*>(k_head + (int64_t)pb * block_stride);
    const uint2* vt = reinterpret_cast<const uint2*>(v_head + (int64_t)pb * block_stride);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) r.k[kk] = kt[kk * 64 + lane];
    const int vo = (lane & 15) * 4 + (lane >> 4);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) r.v[c] = vt[c * 64 + vo];
}

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

template <int D>
__device__ __forceinline__ void compute_block(const BlockRegs<D>& r, const bf16x8_t* qop, float4_t* acc,
                                              SoftmaxState& st, int valid_n, float scale_log2, int g) {
    // S = K . Q^T: lane holds S[token 4g + i][head lane%16], i = 0..3
    float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[kk]), qop[kk], sacc, 0, 0, 0);

    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (4 * g + i < valid_n) ? sacc[i] * scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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

    // P^T as B operand, split into bf16 hi + lo terms
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = f32_to_bf16_bits(pr[i]);
        lo[i] = f32_to_bf16_bits(pr[i] - bf16_bits_to_f32(hi[i]));
    }
    const short4_t p_hi = __builtin_bit_cast(short4_t, make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)));
    const short4_t p_lo = __builtin_bit_cast(short4_t, make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)));

    // tokens past the end hold stale or NaN data: zero them (0 * NaN = NaN)
    uint32_t vm0 = 0xFFFFFFFFu, vm1 = 0xFFFFFFFFu;
    if (valid_n < 16) {
        const int nv = valid_n - 4 * g;
        vm0 = nv >= 2 ? 0xFFFFFFFFu : (nv == 1 ? 0x0000FFFFu : 0u);
        vm1 = nv >= 4 ? 0xFFFFFFFFu : (nv == 3 ? 0x0000FFFFu : 0u);
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const short4_t a = __builtin_bit_cast(short4_t, make_uint2(r.v[c].x & vm0, r.v[c].y & vm1));
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, p_hi, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, p_lo, acc[c], 0, 0, 0);
    }
}

template <int D, int kDepth, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void decode_bf16_mfma_kernel(DecodeParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;  // head column of the MFMA tiles
    const int g = lane >> 4;    // lane group

    int64_t u = blockIdx.x;
    const int kvh = (int)(u % p.num_kv_heads);
    u /= p.num_kv_heads;
    const int hg = (int)(u % p.n_head_groups);
    u /= p.n_head_groups;
    const int s = (int)(u % p.num_seqs);
    const int part = (int)(u / p.num_seqs);

    const int L = clamp_ctx(p.context_lens[s], p.ctx_cap);
    const int n_blk = (L + kBlockSize - 1) / kBlockSize;
    const int n_parts = (n_blk + p.part_blocks - 1) / p.part_blocks;
    const int h0 = kvh * p.group + hg * kMfmaHeadsPerUnit;
    const int nh = min(kMfmaHeadsPerUnit, p.group - hg * kMfmaHeadsPerUnit);
    const int Hq = p.num_q_heads;

    if (n_parts == 0) {  // empty context: zeros
        if (part != 0) return;
        for (int idx = threadIdx.x; idx < nh * D; idx += 64 * kWaves) {
            const int64_t o = ((int64_t)s * Hq + h0) * D + idx;
            if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = 0;
            else reinterpret_cast<float*>(p.out)[o] = 0.f;
        }
        return;
    }
    if (part >= n_parts) return;

    const int blk0 = part * p.part_blocks;
    const int nb = min(p.part_blocks, n_blk - blk0);
    // the waves of the workgroup take the partition's blocks in turn:
    // wave w handles blocks w, w + kWaves, w + 2 kWaves, ...
    const int nbw = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0;

    // Q^T as the B operand: column = head, k-group g holds chunk 4kk + g
    bf16x8_t qop[D / 32];
    {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)s * Hq + h0 + col) * D;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (col < nh) v = reinterpret_cast<const uint4*>(qrow)[4 * kk + g];
            qop[kk] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // this partition's slice of the block table, one entry per lane
    const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq + blk0;
    const int bt_lane = lane < nb ? bt[lane] : 0;

    const int64_t block_stride = (int64_t)p.num_kv_heads * D * kBlockSize;
    const uint16_t* k_head = reinterpret_cast<const uint16_t*>(p.k_cache) + (int64_t)kvh * D * kBlockSize;
    const uint16_t* v_head = reinterpret_cast<const uint16_t*>(p.v_cache) + (int64_t)kvh * D * kBlockSize;

    float4_t acc[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) acc[c] = {0.f, 0.f, 0.f, 0.f};
    SoftmaxState st{-INFINITY, 0.f};

    // i-th block of this wave -> physical block and number of valid tokens
    auto block_of = [&](int i, int& valid_n) {
        const int j = wave + kWaves * i;
        const int pb = __builtin_amdgcn_readlane(bt_lane, j);
        const bool ok = pb >= 0 && (int64_t)pb < p.num_blocks;
        valid_n = ok ? L - (blk0 + j) * kBlockSize : 0;
        return ok ? pb : 0;
    };

    if (nbw > 0) {
        // Ring of kDepth blocks in flight.  The refill of a slot is issued
        // unconditionally (past the end it re-reads the wave's last block,
        // an L2 hit), so the number of loads in flight is the same on every
        // path and the wait before a block covers only that block's loads.
        BlockRegs<D> ring[kDepth];
        int vn[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            load_block<D>(ring[d], k_head, v_head, block_stride, block_of(min(d, nbw - 1), vn[d]), lane);
        for (int i = 0; i < nbw; i += kDepth) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                if (i + d < nbw) compute_block<D>(ring[d], qop, acc, st, vn[d], p.scale_log2, g);
                load_block<D>(ring[d], k_head, v_head, block_stride, block_of(min(i + d + kDepth, nbw - 1), vn[d]),
                              lane);
            }
        }
    }

    float l_tot = st.l + __shfl_xor(st.l, 16);
    l_tot = l_tot + __shfl_xor(l_tot, 32);

    // Epilogue.  Each wave parks its unnormalised accumulator tiles (lane:
    // head col, dims 16c+4g..) and its (m, l) per head in LDS; the
    // workgroup then merges the waves with the log-sum-exp weights
    // 2^(m_w - M) in wave order and writes the unit's nh rows of D values
    // -- contiguous in either destination (out[s][h0..][:], or the partial
    // block of (s, part) laid out [part][head][dim]) -- as 16-byte pieces.
    __shared__ float tile[kWaves][kMfmaHeadsPerUnit][D + 4];
    __shared__ float m_w[kWaves][kMfmaHeadsPerUnit];
    __shared__ float l_w[kWaves][kMfmaHeadsPerUnit];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        *reinterpret_cast<float4*>(&tile[wave][col][16 * c + 4 * g]) = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
    if (g == 0) {
        m_w[wave][col] = st.m;
        l_w[wave][col] = l_tot;
    }
    __syncthreads();
    constexpr int kQuads = D / 4;  // 16-byte pieces per fp32 row
    const int n4 = nh * kQuads;
    const bool single = n_parts == 1;
    for (int f = threadIdx.x; f < n4; f += 64 * kWaves) {
        const int row = f / kQuads;
        const int c4 = f % kQuads;
        float M = m_w[0][row];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, m_w[w][row]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float a = kWaves == 1 ? 1.f : exp2_fast(m_w[w][row] - M_use);
            const float4 v = *reinterpret_cast<const float4*>(&tile[w][row][4 * c4]);
            num.x = fmaf(a, v.x, num.x);
            num.y = fmaf(a, v.y, num.y);
            num.z = fmaf(a, v.z, num.z);
            num.w = fmaf(a, v.w, num.w);
            den = fmaf(a, l_w[w][row], den);
        }
        if (single) {
            const float inv = den > 0.f ? 1.f / den : 0.f;
            const int64_t o = ((int64_t)s * Hq + h0) * D + 4 * f;
            if (p.out_bf16) {
                const uint2 w2 = make_uint2(f32_to_bf16_bits(num.x * inv) | (f32_to_bf16_bits(num.y * inv) << 16),
                                            f32_to_bf16_bits(num.z * inv) | (f32_to_bf16_bits(num.w * inv) << 16));
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o) = w2;
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) =
                    make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
            }
        } else {
            const int64_t row0 = ((int64_t)s * p.num_parts + part) * Hq + h0;
            *reinterpret_cast<float4*>(p.o_part + row0 * D + 4 * f) = num;
            if (c4 == 0) {
                p.m_part[row0 + row] = M;
                p.l_part[row0 + row] = den;
            }
        }
    }
}

}  // namespace

hipError_t launch_decode_bf16_mfma(const DecodeParams& p, hipStream_t stream) {
    const int64_t units = decode_units(p);
    if (units == 0) return hipSuccess;
    const dim3 grid((unsigned)units), block(64 * kWavesPerUnit);
    if (p.head_dim == 128)
        hipLaunchKernelGGL((decode_bf16_mfma_kernel<128, kPrefetchBlocks, kWavesPerUnit>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((decode_bf16_mfma_kernel<64, kPrefetchBlocks, kWavesPerUnit>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
