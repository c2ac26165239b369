// Paged decode attention on the vector ALUs: the fp32-KV path, and, on bf16
// elements, the measurement aid pkv_paged_attention_decode_vector_alu that
// weighs vector-ALU products against the matrix-core decode.
//
// Same problem, unit decomposition and split-K partials as decode_mfma.hip
// (one wave64 per partition x sequence x head group x KV head), but every
// product is an fp32 FMA, so fp32 KV keeps fp32 accuracy end to end.
//
// Per 16-token block:
//   QK   lane (t = lane%16, group g = lane/16) reads the K chunks 4i+g of
//        token t (each load of the wave is one contiguous 1 KiB run), dots
//        them with the query rows kept in LDS, and the four lane groups are
//        summed with two cross-group shuffles.
//   softmax  per head over the 16 lanes of a group (xor 1, 2, 4, 8).
//   PV   lane owns dims lane + 64k of every head; it reads the V^T row of
//        each dim (the block's 16 tokens are contiguous) and the weights
//        from LDS.
#include "kernels.h"

namespace pkv {
namespace {

template <typename E>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kX = 4;  // elements per 16-byte chunk
    __device__ static inline void unpack(const uint4& w, float* f) {
        f[0] = __uint_as_float(w.x);
        f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z);
        f[3] = __uint_as_float(w.w);
    }
};
template <>
struct Elem<uint16_t> {
    static constexpr int kX = 8;
    __device__ static inline void unpack(const uint4& w, float* f) {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(a[i] << 16);
            f[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
        }
    }
    __device__ static inline float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
};

__device__ inline float load_q(const float* q, int64_t i) { return q[i]; }
__device__ inline float load_q(const uint16_t* q, int64_t i) { return __uint_as_float((uint32_t)q[i] << 16); }

template <typename E, int D, int HMAX>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
    constexpr int X = Elem<E>::kX;
    constexpr int NCH = D / X;       // chunks per token row
    constexpr int CPL = NCH / 4;     // chunks per lane group
    constexpr int DPL = D / 64;      // PV dims per lane
    constexpr int VW = 16 / X;       // 16-byte words per V^T row (16 tokens)
    __shared__ float qs[HMAX][D];
    __shared__ float ps[HMAX][16];

    const int lane = threadIdx.x;
    const int t = lane & 15;
    const int g = lane >> 4;

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
    const int h0 = kvh * p.group + hg * kValuHeadsPerUnit;
    const int nh = min(HMAX, p.group - hg * kValuHeadsPerUnit);
    const int Hq = p.num_q_heads;

    if (n_parts == 0) {
        if (part != 0) return;
        for (int idx = lane; idx < nh * D; idx += 64) {
            const int64_t o = ((int64_t)s * Hq + h0) * D + idx;
            if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = 0;
            else reinterpret_cast<float*>(p.out)[o] = 0.f;
        }
        return;
    }
    if (part >= n_parts) return;
    const int blk0 = part * p.part_blocks;
    const int nb = min(p.part_blocks, n_blk - blk0);

    const E* q = reinterpret_cast<const E*>(p.q) + ((int64_t)s * Hq + h0) * D;
    for (int idx = lane; idx < HMAX * D; idx += 64)
        qs[idx / D][idx % D] = (idx / D) < nh ? load_q(q, idx) : 0.f;
    __syncthreads();

    const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq + blk0;
    const int64_t block_stride = (int64_t)p.num_kv_heads * D * kBlockSize;
    const E* k_head = reinterpret_cast<const E*>(p.k_cache) + (int64_t)kvh * D * kBlockSize;
    const E* v_head = reinterpret_cast<const E*>(p.v_cache) + (int64_t)kvh * D * kBlockSize;

    float m_run[HMAX], l_run[HMAX], acc[HMAX][DPL];
#pragma unroll
    for (int h = 0; h < HMAX; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[h][k] = 0.f;
    }

    for (int j = 0; j < nb; ++j) {
        const int pb_raw = bt[j];
        const bool ok = pb_raw >= 0 && (int64_t)pb_raw < p.num_blocks;
        const int pb = ok ? pb_raw : 0;
        const int valid_n = ok ? L - (blk0 + j) * kBlockSize : 0;
        const uint4* kt = reinterpret_cast<const uint4*>(k_head + (int64_t)pb * block_stride);
        const E* vt = v_head + (int64_t)pb * block_stride;

        // ---- QK: partial dots over this lane group's chunks
        float sp[HMAX];
#pragma unroll
        for (int h = 0; h < HMAX; ++h) sp[h] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = 4 * i + g;
            float kv[X];
            Elem<E>::unpack(kt[i * 64 + lane], kv);
#pragma unroll
            for (int h = 0; h < HMAX; ++h) {
                float a = sp[h];
#pragma unroll
                for (int e = 0; e < X; ++e) a = fmaf(kv[e], qs[h][c * X + e], a);
                sp[h] = a;
            }
        }
        const bool tok_ok = t < valid_n;
        float alpha[HMAX];
#pragma unroll
        for (int h = 0; h < HMAX; ++h) {
            float v = sp[h];
            v = v + __shfl_xor(v, 16);
            v = v + __shfl_xor(v, 32);
            const float sv = tok_ok ? v * p.scale_log2 : -INFINITY;
            float mx = sv;
            mx = fmaxf(mx, __shfl_xor(mx, 1));
            mx = fmaxf(mx, __shfl_xor(mx, 2));
            mx = fmaxf(mx, __shfl_xor(mx, 4));
            mx = fmaxf(mx, __shfl_xor(mx, 8));
            const float m_new = fmaxf(m_run[h], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            alpha[h] = exp2_fast(m_run[h] - m_use);
            m_run[h] = m_new;
            if (g == 0) ps[h][t] = exp2_fast(sv - m_use);
        }
        __syncthreads();

        // ---- PV
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            const int d = lane + 64 * k;
            float vv[16];
#pragma unroll
            for (int w = 0; w < VW; ++w) Elem<E>::unpack(reinterpret_cast<const uint4*>(vt + d * kBlockSize)[w], vv + w * X);
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) vv[tt] = tt < valid_n ? vv[tt] : 0.f;
#pragma unroll
            for (int h = 0; h < HMAX; ++h) {
                float a = 0.f;
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) a = fmaf(ps[h][tt], vv[tt], a);
                acc[h][k] = acc[h][k] * alpha[h] + a;
            }
        }
#pragma unroll
        for (int h = 0; h < HMAX; ++h) {
            float sum = 0.f;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) sum += ps[h][tt];
            l_run[h] = l_run[h] * alpha[h] + sum;
        }
        __syncthreads();
    }

#pragma unroll
    for (int h = 0; h < HMAX; ++h) {
        if (h >= nh) continue;
        const int qh = h0 + h;
        if (n_parts == 1) {
            const float inv = l_run[h] > 0.f ? 1.f / l_run[h] : 0.f;
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
                const int64_t o = ((int64_t)s * Hq + qh) * D + lane + 64 * k;
                const float val = acc[h][k] * inv;
                if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16_bits(val);
                else reinterpret_cast<float*>(p.out)[o] = val;
            }
        } else {
            const int64_t row = ((int64_t)s * p.num_parts + part) * Hq + qh;
#pragma unroll
            for (int k = 0; k < DPL; ++k) p.o_part[row * D + lane + 64 * k] = acc[h][k];
            if (lane == 0) {
                p.m_part[row] = m_run[h];
                p.l_part[row] = l_run[h];
            }
        }
    }
}

template <typename E, int D>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)decode_units(p)), block(64);
    const int hm = min(p.group, kValuHeadsPerUnit);
    if (hm <= 1) hipLaunchKernelGGL((decode_valu_kernel<E, D, 1>), grid, block, 0, stream, p);
    else if (hm <= 2) hipLaunchKernelGGL((decode_valu_kernel<E, D, 2>), grid, block, 0, stream, p);
    else if (hm <= 4) hipLaunchKernelGGL((decode_valu_kernel<E, D, 4>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_valu_kernel<E, D, 8>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, bool bf16, hipStream_t stream) {
    if (decode_units(p) == 0) return hipSuccess;
    if (bf16) return p.head_dim == 128 ? launch_typed<uint16_t, 128>(p, stream) : launch_typed<uint16_t, 64>(p, stream);
    return p.head_dim == 128 ? launch_typed<float, 128>(p, stream) : launch_typed<float, 64>(p, stream);
}

}  // namespace pkv
