// Split-K merge of partition partials into the decode output.
//
// A partition p of a sequence's context left, per query head, its running
// max m_p (log2 units), its sum l_p = sum 2^(s_i - m_p) and its unnormalised
// output o_p = sum 2^(s_i - m_p) v_i.  Softmax over the whole context is then
//     out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// an identity of the exponential (nothing here is an approximation beyond
// fp32 rounding).  One 256-thread workgroup per (sequence, query head);
// sequences that fit in one partition were finished by the partition kernel
// and are skipped.  All sums run in a fixed order, so the result does not
// depend on scheduling.
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off) red[tid] = red[tid] + red[tid + off];
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

template <int D>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(DecodeParams p) {
    constexpr int LPR = D / 4;             // threads per output row (float4 each)
    constexpr int SLOTS = kThreads / LPR;  // partitions in flight per step
    __shared__ float red[kThreads];
    __shared__ float4 part_acc[SLOTS][LPR];

    const int Hq = p.num_q_heads;
    const int s = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    const int L = clamp_ctx(p.context_lens[s], p.ctx_cap);
    const int n_blk = (L + kBlockSize - 1) / kBlockSize;
    int n_parts = (n_blk + p.part_blocks - 1) / p.part_blocks;
    if (n_parts > p.num_parts) n_parts = p.num_parts;
    if (n_parts <= 1) return;

    // partials of (s, partition i, head h) sit at row (s * P + i) * Hq + h
    const int64_t base = (int64_t)s * p.num_parts * Hq + h;
    const float* m = p.m_part + base;
    const float* l = p.l_part + base;
    const int tid = threadIdx.x;

    float mx = -INFINITY;
    for (int i = tid; i < n_parts; i += kThreads) mx = fmaxf(mx, m[(int64_t)i * Hq]);
    const float M = block_max(mx, red);
    const float M_use = (M == -INFINITY) ? 0.f : M;

    float den = 0.f;
    for (int i = tid; i < n_parts; i += kThreads) den += exp2_fast(m[(int64_t)i * Hq] - M_use) * l[(int64_t)i * Hq];
    den = block_sum(den, red);

    const int slot = tid / LPR;
    const int c4 = tid % LPR;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4* o = reinterpret_cast<const float4*>(p.o_part + base * D);
#pragma unroll 4
    for (int i = slot; i < n_parts; i += SLOTS) {
        const float w = exp2_fast(m[(int64_t)i * Hq] - M_use);
        const float4 v = o[(int64_t)i * Hq * LPR + c4];
        a.x = fmaf(w, v.x, a.x);
        a.y = fmaf(w, v.y, a.y);
        a.z = fmaf(w, v.z, a.z);
        a.w = fmaf(w, v.w, a.w);
    }
    part_acc[slot][c4] = a;
    __syncthreads();
    if (slot != 0) return;
    float4 sum = part_acc[0][c4];
    for (int k = 1; k < SLOTS; ++k) {
        const float4 v = part_acc[k][c4];
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const float r0 = sum.x * inv, r1 = sum.y * inv, r2 = sum.z * inv, r3 = sum.w * inv;
    const int64_t ob = ((int64_t)s * Hq + h) * D + 4 * c4;
    if (p.out_bf16) {
        const uint2 w = make_uint2(f32_to_bf16_bits(r0) | (f32_to_bf16_bits(r1) << 16),
                                   f32_to_bf16_bits(r2) | (f32_to_bf16_bits(r3) << 16));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + ob) = w;
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + ob) = make_float4(r0, r1, r2, r3);
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const DecodeParams& p, hipStream_t stream) {
    if (p.num_parts <= 1 || p.num_seqs == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.num_seqs * p.num_q_heads)), block(kThreads);
    if (p.head_dim == 128) hipLaunchKernelGGL(splitk_reduce_kernel<128>, grid, block, 0, stream, p);
    else hipLaunchKernelGGL(splitk_reduce_kernel<64>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
