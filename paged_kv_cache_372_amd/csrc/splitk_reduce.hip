// Split-K merge of partial results into the decode output.
//
// A piece p of a sequence's context left, per query head, its reference max
// m_p (log2 units), its sum l_p = sum 2^(s_i - m_p) and its unnormalised
// output o_p = sum 2^(s_i - m_p) v_i.  Softmax over the whole context is then
//     out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// an identity of the exponential (nothing here is an approximation beyond
// fp32 rounding).  Pieces with no valid token (m = -inf, l = 0) weigh 0.
// One 256-thread workgroup per (sequence, query head); its 256 / (D / 4)
// slots each merge every SLOTS-th piece with a running maximum (the same
// identity applied one piece at a time), then slot 0 merges the slots.  All
// sums run in a fixed order, so the result does not depend on scheduling.
//
// Where the pieces are depends on the decode path:
//   partitioned (fp32 KV): partition i of sequence s at row (s * P + i) * Hq + h;
//     sequences that fit in one partition were finished by the decode.
//   balanced (bf16 KV): the sequence's blocks [o0, o1) of the flattened list
//     fall in ranges r0 = o0 / cs .. r1 = (o1 - 1) / cs; range r's piece is
//     at row range_slot(r, cs, o0) * Hq + h.  A sequence inside one range was
//     finished by the decode; an empty sequence gets zeros here.
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// Weight 2^(m - M) of a piece with reference max m against a running max M;
// an empty piece (m = -inf) weighs 0 whatever M is.
__device__ __forceinline__ float piece_weight(float m, float M) { return m == -INFINITY ? 0.f : exp2_fast(m - M); }

template <int D>
__device__ __forceinline__ void write_row(const DecodeParams& p, int64_t row, int c4, float4 v) {
    const int64_t ob = row * D + 4 * c4;
    if (p.out_bf16) {
        const uint2 w = make_uint2(f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16),
                                   f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + ob) = w;
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + ob) = v;
    }
}

template <int D, bool kBalanced>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(DecodeParams p) {
    constexpr int LPR = D / 4;             // threads per output row (float4 each)
    constexpr int SLOTS = kThreads / LPR;  // pieces in flight per step
    __shared__ float4 part_acc[SLOTS][LPR];
    __shared__ float part_m[SLOTS], part_l[SLOTS];

    const int Hq = p.num_q_heads;
    const int s = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    const int tid = threadIdx.x;
    const int slot = tid / LPR;
    const int c4 = tid % LPR;
    const int64_t out_row = (int64_t)s * Hq + h;

    // piece i of this (sequence, head) is at partial row row0 + i * stride,
    // except (balanced) the first, whose row is first_row
    int n_pieces;
    int64_t row0, stride, first_row;
    if (kBalanced) {
        const int o0 = p.seq_off[s];
        const int o1 = p.seq_off[s + 1];
        if (o1 <= o0) {  // empty context: zeros
            if (slot == 0) write_row<D>(p, out_row, c4, make_float4(0.f, 0.f, 0.f, 0.f));
            return;
        }
        int cs, nr;
        range_geometry(p.seq_off[p.num_seqs], p.walkers, p.range_cap, cs, nr);
        const int r0 = o0 / cs;
        const int r1 = (o1 - 1) / cs;
        if (r0 == r1) return;
        n_pieces = r1 - r0 + 1;
        // ranges after the first hold the sequence from their start: slot 0
        row0 = (int64_t)range_slot(r0 + 1, cs, o0) * Hq + h - 2 * Hq;
        stride = 2 * Hq;
        first_row = (int64_t)range_slot(r0, cs, o0) * Hq + h;
    } else {
        const int L = clamp_ctx(p.context_lens[s], p.ctx_cap);
        const int n_blk = (L + kBlockSize - 1) / kBlockSize;
        n_pieces = (n_blk + p.part_blocks - 1) / p.part_blocks;
        if (n_pieces > p.num_parts) n_pieces = p.num_parts;
        if (n_pieces <= 1) return;
        row0 = (int64_t)s * p.num_parts * Hq + h;
        stride = Hq;
        first_row = row0;
    }
    auto row_of = [&](int i) -> int64_t { return i == 0 ? first_row : row0 + (int64_t)i * stride; };

    // Each slot merges its pieces i = slot, slot + SLOTS, ... in order with a
    // running (max, sum, output): the loads of a piece need nothing from the
    // previous one, so they are all in flight at once.
    float M = -INFINITY, den = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int i = slot; i < n_pieces; i += SLOTS) {
        const int64_t r = row_of(i);
        const float m = p.m_part[r];
        const float l = p.l_part[r];
        const float4 v = reinterpret_cast<const float4*>(p.o_part + r * D)[c4];
        const float Mn = fmaxf(M, m);
        const float wa = piece_weight(M, Mn);  // rescale of what is merged so far
        const float wb = piece_weight(m, Mn);
        den = den * wa + l * wb;
        a.x = a.x * wa + v.x * wb;
        a.y = a.y * wa + v.y * wb;
        a.z = a.z * wa + v.z * wb;
        a.w = a.w * wa + v.w * wb;
        M = Mn;
    }
    part_acc[slot][c4] = a;
    if (c4 == 0) {
        part_m[slot] = M;
        part_l[slot] = den;
    }
    __syncthreads();
    if (slot != 0) return;
    // slots in order: a fixed summation order, independent of scheduling
    float Mt = part_m[0];
    for (int k = 1; k < SLOTS; ++k) Mt = fmaxf(Mt, part_m[k]);
    den = 0.f;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < SLOTS; ++k) {
        const float w = piece_weight(part_m[k], Mt);
        const float4 v = part_acc[k][c4];
        den = fmaf(w, part_l[k], den);
        sum.x = fmaf(w, v.x, sum.x);
        sum.y = fmaf(w, v.y, sum.y);
        sum.z = fmaf(w, v.z, sum.z);
        sum.w = fmaf(w, v.w, sum.w);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    write_row<D>(p, out_row, c4, make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv));
}

template <bool kBalanced>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.num_seqs * p.num_q_heads)), block(kThreads);
    if (p.head_dim == 128) hipLaunchKernelGGL((splitk_reduce_kernel<128, kBalanced>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((splitk_reduce_kernel<64, kBalanced>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_splitk_reduce(const DecodeParams& p, bool balanced, hipStream_t stream) {
    if (p.num_seqs == 0) return hipSuccess;
    if (balanced) return launch<true>(p, stream);
    if (p.num_parts <= 1) return hipSuccess;
    return launch<false>(p, stream);
}

}  // namespace pkv
