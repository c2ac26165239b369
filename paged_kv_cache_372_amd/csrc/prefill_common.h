// Pieces of the chunked-prefill kernel (prefill_wide.hip) kept apart: how a
// workgroup finds its tile and each wave its rows (heaviest tiles first), and
// small numeric helpers.
#pragma once

#include "prefill.h"

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
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
// two fp32 -> packed fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, f16x2_t));
}
// E4M3 codes (bytes 2 kHigh and 2 kHigh + 1 of w) -> their exact values,
// packed as two bf16 or two fp16: every E4M3 value (at most 448, at least
// 2^-9 apart from zero, 4 significant bits) is exact in both
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHigh));
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

// Block-wide exclusive prefix sum of one value per thread (wave_total:
// kWaves ints of LDS).  Returns this thread's prefix; *total gets the sum.
// Two barriers: every thread of the workgroup must call it.
template <int kWaves>
__device__ __forceinline__ int block_exclusive_scan(int x, int32_t* wave_total, int* total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const int wt = wave_total[v];
        before += v < wave ? wt : 0;
        all += wt;
    }
    __syncthreads();  // wave_total may be reused right after
    *total = all;
    return before + incl - x;
}

// Finds the workgroup's tile and the wave's rows (none when R0 >= rows);
// false when the workgroup has no tile.  A request's n * G rows are cut into
// tiles of kPrefillRowsPerGroup; the weight of a tile is the number of keys
// its last row sees, in units of 2^p.lpt_shift keys.  Workgroup idx =
// blockIdx / Hkv takes the tile of rank idx in the order of decreasing
// weight, ties by request and tile (longest processing time first: the
// workgroups of one KV head share one XCD, which then hands each free CU the
// heaviest tile left).  Every workgroup works the order out on its own, in
// LDS (p.lpt_buckets + num_seqs + 3 ints of it): the first tile of each
// request, a histogram of the weights and its suffix sums, the weight class
// of rank idx, then the tile of that class.
template <int kWaves, int kRowsPerWave>
__device__ __forceinline__ bool locate_rows(const PrefillParams& p, int32_t* lds, int32_t* wave_total, WaveRows& w) {
    constexpr int nthr = 64 * kWaves;
    const int B = p.num_seqs;
    const int T = p.num_tokens;
    const int G = p.group;
    const int K = p.lpt_buckets;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int32_t* t_off = lds;          // [B + 1] first tile of each request
    int32_t* ge = lds + B + 1;     // [K] tiles of weight >= w (first a histogram)
    int32_t* pick = ge + K;        // [2] the workgroup's request and tile

    // rows [r0, r1) of q/out belong to request i (clamped to the call's T)
    auto rows_of = [&](int i, int& r0, int& r1) {
        r0 = min(max(p.query_start_loc[i], 0), T);
        r1 = min(max(p.query_start_loc[i + 1], r0), T);
    };
    // weight of tile t of request s
    auto weight = [&](int s, int t) {
        int r0, r1;
        rows_of(s, r0, r1);
        const int n = r1 - r0;
        const int L = clamp_ctx(p.context_lens[s], p.ctx_cap);
        const int Rg = min(t * kPrefillRowsPerGroup + kPrefillRowsPerGroup - 1, n * G - 1);
        const int kend = min(L, L - n + Rg / G + 1);
        return kend > 0 ? min(((kend - 1) >> p.lpt_shift) + 1, K - 1) : 0;
    };
    // the request of tile g: the last s with t_off[s] <= g
    auto request_of = [&](int g) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (t_off[mid] <= g) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };

    // ---- first tile of each request (contiguous runs of requests per thread)
    int total;
    {
        const int per = (B + nthr - 1) / nthr;
        const int i0 = min(B, tid * per);
        const int i1 = min(B, i0 + per);
        int sum = 0;
        for (int i = i0; i < i1; ++i) {
            int a, b;
            rows_of(i, a, b);
            sum += ((b - a) * G + kPrefillRowsPerGroup - 1) / kPrefillRowsPerGroup;
        }
        int run = block_exclusive_scan<kWaves>(sum, wave_total, &total);
        for (int i = i0; i < i1; ++i) {
            t_off[i] = run;
            int a, b;
            rows_of(i, a, b);
            run += ((b - a) * G + kPrefillRowsPerGroup - 1) / kPrefillRowsPerGroup;
        }
        if (tid == 0) t_off[B] = total;
        for (int i = tid; i < K; i += nthr) ge[i] = 0;
        __syncthreads();
    }
    total = __builtin_amdgcn_readfirstlane(total);
    const int idx = blockIdx.x / p.num_kv_heads;
    w.kvh = blockIdx.x - idx * p.num_kv_heads;
    if (idx >= total) return false;  // the whole workgroup

    // ---- histogram of the weights, then suffix sums: ge[w] = tiles of weight >= w
    for (int g = tid; g < total; g += nthr) {
        const int s = request_of(g);
        atomicAdd(&ge[weight(s, g - t_off[s])], 1);
    }
    __syncthreads();
    {
        const int per = (K + nthr - 1) / nthr;  // thread tid takes weights [K - (tid+1) per, K - tid per)
        const int w1 = max(K - tid * per, 0), w0 = max(K - (tid + 1) * per, 0);
        int sum = 0;
        for (int v = w1 - 1; v >= w0; --v) sum += ge[v];
        int unused;
        int run = block_exclusive_scan<kWaves>(sum, wave_total, &unused);
        for (int v = w1 - 1; v >= w0; --v) {
            run += ge[v];
            ge[v] = run;
        }
        __syncthreads();
    }
    // ---- weight class of rank idx: the largest c with ge[c] > idx, and the
    // rank within it (ge is non-increasing; ge[0] = total > idx)
    int c = 0;
    {
        int lo = 0, hi = K - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ge[mid] > idx) lo = mid;
            else hi = mid - 1;
        }
        c = __builtin_amdgcn_readfirstlane(lo);
    }
    const int k = idx - (c + 1 < K ? ge[c + 1] : 0);
    // ---- the k-th tile of weight c, in tile order (contiguous runs of tiles per thread)
    {
        const int per = (total + nthr - 1) / nthr;
        const int g0 = min(total, tid * per), g1 = min(total, g0 + per);
        int cnt = 0;
        int s = g0 < g1 ? request_of(g0) : 0;
        for (int g = g0; g < g1; ++g) {
            while (s + 1 < B && t_off[s + 1] <= g) ++s;
            cnt += weight(s, g - t_off[s]) == c;
        }
        int unused;
        int before = block_exclusive_scan<kWaves>(cnt, wave_total, &unused);
        if (before <= k && k < before + cnt) {
            s = g0 < g1 ? request_of(g0) : 0;
            for (int g = g0; g < g1; ++g) {
                while (s + 1 < B && t_off[s + 1] <= g) ++s;
                if (weight(s, g - t_off[s]) == c) {
                    if (before == k) {
                        pick[0] = s;
                        pick[1] = g - t_off[s];
                    }
                    ++before;
                }
            }
        }
        __syncthreads();
    }
    // values read from LDS or memory below are the same in every lane; say
    // so, so that table entries are fetched through the scalar cache
    w.s = __builtin_amdgcn_readfirstlane(pick[0]);
    const int tile = __builtin_amdgcn_readfirstlane(pick[1]);
    int r0, r1;
    rows_of(w.s, r0, r1);
    w.r0 = __builtin_amdgcn_readfirstlane(r0);
    w.n = __builtin_amdgcn_readfirstlane(r1) - w.r0;
    w.rows = w.n * G;
    w.R0 = tile * kPrefillRowsPerGroup + wave * kRowsPerWave;
    w.L = __builtin_amdgcn_readfirstlane(clamp_ctx(p.context_lens[w.s], p.ctx_cap));
    return true;
}

}  // namespace

}  // namespace pkv
