// Pieces shared by the two chunked-prefill kernels (prefill_mfma.hip: 16 x 16
// tiles, fp8 pools; prefill_wide.hip: 32 x 32 tiles staged in LDS, bf16
// pools): how a workgroup finds its rows, and small numeric helpers.
#pragma once

#include "kernels.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef const int32_t __attribute__((address_space(4)))* scalar_i32_ptr;

constexpr float kSlack = 8.f;  // lazy-rescale margin (log2 units): weights stay below 2^8

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 (round to nearest even), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ uint32_t tail_mask(int nv, int first) {
    // 16-bit lanes [first, first + 1] of a token run, kept when inside nv
    return nv >= first + 2 ? 0xFFFFFFFFu : (nv == first + 1 ? 0x0000FFFFu : 0u);
}

// The rows a wave takes: request s (rows [r0, r0 + n) of q/out, context
// length L), KV head kvh, and the wave's first (token, head) row R0 of the
// request's n * G rows.
struct WaveRows {
    int s, r0, n, rows, R0, L, kvh;
};

// Fills t_off[0..B] (first workgroup tile of each request; exclusive prefix
// sums over the requests) and finds the workgroup's tile and the wave's rows
// (none when R0 >= rows).  False when the workgroup has no tile.
template <int kWaves, int kRowsPerWave>
__device__ __forceinline__ bool locate_rows(const PrefillParams& p, int32_t* t_off, int32_t* wave_total,
                                            WaveRows& w) {
    const int B = p.num_seqs;
    const int T = p.num_tokens;
    const int G = p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // rows [r0, r1) of q/out belong to request i (clamped to the call's T)
    auto rows_of = [&](int i, int& r0, int& r1) {
        r0 = min(max(p.query_start_loc[i], 0), T);
        r1 = min(max(p.query_start_loc[i + 1], r0), T);
    };
    {
        const int nthr = 64 * kWaves;
        const int per = (B + nthr - 1) / nthr;
        const int i0 = min(B, tid * per);
        const int i1 = min(B, i0 + per);
        int sum = 0;
        for (int i = i0; i < i1; ++i) {
            int a, b;
            rows_of(i, a, b);
            sum += ((b - a) * G + kPrefillRowsPerGroup - 1) / kPrefillRowsPerGroup;
        }
        int x = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (lane == 63) wave_total[wave] = x;
        __syncthreads();
        int run = x - sum;
        for (int v = 0; v < wave; ++v) run += wave_total[v];
        for (int i = i0; i < i1; ++i) {
            t_off[i] = run;
            int a, b;
            rows_of(i, a, b);
            run += ((b - a) * G + kPrefillRowsPerGroup - 1) / kPrefillRowsPerGroup;
        }
        if (tid == nthr - 1) t_off[B] = run;
        __syncthreads();
    }
    // values read from LDS or memory below are the same in every lane; say
    // so, so that table entries are fetched through the scalar cache
    const int total = __builtin_amdgcn_readfirstlane(t_off[B]);
    const int idx = blockIdx.x / p.num_kv_heads;
    w.kvh = blockIdx.x - idx * p.num_kv_heads;
    if (idx >= total) return false;
    const int tile = total - 1 - idx;  // heaviest tiles first
    int lo = 0, hi = B - 1;            // last request whose first tile is <= tile
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t_off[mid] <= tile) lo = mid;
        else hi = mid - 1;
    }
    w.s = __builtin_amdgcn_readfirstlane(lo);
    int r0, r1;
    rows_of(w.s, r0, r1);
    w.r0 = __builtin_amdgcn_readfirstlane(r0);
    w.n = __builtin_amdgcn_readfirstlane(r1) - w.r0;
    w.rows = w.n * G;
    w.R0 = (tile - __builtin_amdgcn_readfirstlane(t_off[w.s])) * kPrefillRowsPerGroup + wave * kRowsPerWave;
    w.L = __builtin_amdgcn_readfirstlane(clamp_ctx(p.context_lens[w.s], p.ctx_cap));
    return true;
}

}  // namespace

// The bf16-pool kernel (prefill_wide.hip); same grid and LDS table as
// launch_prefill_bf16, which calls it.
hipError_t launch_prefill_wide(const PrefillParams& p, hipStream_t stream);

}  // namespace pkv
