// Chunked-prefill attention over bf16 pools on 32 x 32 matrix tiles, with K
// and V staged in LDS.  What is computed, and how the rows of a request are
// cut into workgroup tiles, is the same as in prefill_mfma.hip: causal
// attention of each request's n_s new query tokens over its L_s cached
// tokens, aligned at the end of the context, the keys reached through the
// request's block table (architvora "Paged Attention"; runbyai section 1).
// Workgroups take their tiles heaviest first (locate_rows).
//
// Matrix shape.  A wave owns one 32-row tile and uses mfma_f32_32x32x16_bf16,
// whose operands carry twice the products per byte of the 16 x 16 shape (both
// shapes issue at close to the matrix cores' peak: pkv_issue_rate_bench).
// Per pair of blocks (A, B) = 32 keys:
//   S^T[32 keys x 32 rows] = K . Q^T            D/16 x mfma_f32_32x32x16_bf16
//   O^T[32 dims x 32 rows] += V^T . P^T          per 32-dim tile: 2 (blocks)
// Operands of mfma_f32_32x32x16_bf16, lane l = 32h + n: A holds row n,
// k = 8h..8h+7; B holds k = 8h..8h+7 of column n; result register r holds
// row 8(r/4) + 4h + r%4 of column n.  The QK product takes key row m as
// token (m mod 16, bits 2 and 3 swapped) of block m/16: result registers
// 0..7 of lane (n, h) then hold row n's scores against tokens 8h..8h+7 of
// block A and registers 8..15 those of block B -- the PV product's B operand
// for block b as it stands.  Its A operand (dim 32t + n, tokens 8h..8h+7)
// is one 16-byte run of the pool's [dim][16 tokens] V block.
//
// Two waves per SIMD.  Eight waves of 32 rows (256 per workgroup) fit the
// register file twice over.  One wave alone issues a VALU instruction about
// every seventh cycle, two waves every fourth (pkv_issue_rate_bench), and
// the softmax is some 140 VALU instructions per wave and step: the second
// wave of a SIMD keeps its VALU and matrix cores fed while the first waits.
// A step takes two pairs (64 keys): the wave runs their QK products as two
// independent chains, the mask, maxima and weights over 64 keys, then their
// PV products.
//
// Staging.  The workgroup loads each block once, with direct-to-LDS buffer
// loads: wave w copies block w mod 4 of the step, K for w < 4 and V for the
// others, from one descriptor (the block).  A K block is copied as it lies
// in the pool ([D/8][16 tokens][8 dims]): a QK operand then reads, per 16
// lanes, 256 consecutive bytes, in the token order the product wants.  V is
// loaded in operand order (lane l of load t fetches dim 32t + l % 32, tokens
// 8(l / 32) .. +7): a PV operand is 1 KiB of consecutive LDS.  Both are read
// without bank conflicts.  (The buffer form, unlike the flat one, leaves the
// compiler counting LDS reads precisely: a flat load into LDS makes it wait
// for all of them.)  K and V share a ring of three slots of two pairs each,
// one LDS array per slot (distinct objects, so the compiler knows which slot
// a read touches and adds no waits of its own).  Step u, one barrier: every
// load but those of step u - 1 has landed; the loads of step u + 2 go into
// the slot step u - 1 read, issued between step u's QK products.  The waits
// are explicit vmcnt counts: loads return in issue order, and every thread
// issues the same number of loads in every step.
#include <type_traits>

#include "prefill_common.h"

namespace pkv {
namespace {

typedef float float16v_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) const void* global_cvoid_ptr;

__device__ __forceinline__ int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// max and sum over lanes n and n + 32 (the two halves of a 32 x 32 result)
__device__ __forceinline__ float max_halves(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt in bits 3:0 and 15:14), with
// lgkmcnt(0) too when kLgkm0; expcnt untouched
template <int N, bool kLgkm0 = false>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((kLgkm0 ? 0 : 15) << 8));
}

// One 16-byte-per-lane buffer load into LDS: lane l's 16 bytes at rs +
// voffset land at dst + 16 l.  (A plain device function: inside the kernel
// template the size argument is also checked against the host target, and
// the kernel's host stub is silently dropped.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, lds_void_ptr dst, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voffset, 0, 0, 0);
}

template <int D>
struct WideShape {
    static constexpr int kThreads = 512;             // eight waves
    static constexpr int kPairs = 2;                 // pairs of blocks per step
    static constexpr int kKC = D / 16;               // QK steps per pair
    static constexpr int kDT = D / 32;               // 32-dim output tiles
    static constexpr int kKChunks = kKC * 64;        // 16-byte K operand chunks per pair
    static constexpr int kVChunks = 2 * kDT * 64;    // 16-byte V operand chunks per pair
    static constexpr int kBlockChunks = D * kBlockSize * 2 / 16;        // 16-byte chunks of one K or V block
    static constexpr int kSlotChunks = kPairs * (kKChunks + kVChunks);  // one ring slot: K of both pairs, then V
    static constexpr int kStepLoads = kBlockChunks / 64;                 // direct-to-LDS loads per thread per step
    // each wave loads one block of K or of V per step
    static_assert(kThreads / 64 == 2 * 2 * kPairs && kKChunks == 2 * kBlockChunks && kVChunks == 2 * kBlockChunks,
                  "one wave per block and kind");
};

template <int D>
__global__ __launch_bounds__(512) void prefill_wide_kernel(PrefillParams p) {
    using WS = WideShape<D>;
    constexpr int kWaves = WS::kThreads / 64;
    constexpr int kRowsPerWave = kPrefillRowsPerGroup / kWaves;  // 32
    static_assert(kRowsPerWave == 32, "one 32-row tile per wave");
    constexpr int kP = WS::kPairs;
    constexpr int kKC = WS::kKC, kDT = WS::kDT, kStepLoads = WS::kStepLoads;
    constexpr int kKeysPerStep = 2 * kP * kBlockSize;  // 64
    extern __shared__ int32_t plan[];  // tile order (see locate_rows)
    __shared__ int32_t wave_total[kWaves];
    // slot layout: K chunks of pair 0, of pair 1, then V chunks of pair 0, of pair 1
    __shared__ uint4 slot0[WS::kSlotChunks], slot1[WS::kSlotChunks], slot2[WS::kSlotChunks];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    WaveRows wr;
    if (!locate_rows<kWaves, kRowsPerWave>(p, plan, wave_total, wr)) return;  // the whole workgroup
    const int s = wr.s, r0 = wr.r0, nq = wr.n, rows = wr.rows, R0 = wr.R0, L = wr.L, kvh = wr.kvh;
    const int G = p.group;
    const bool has_rows = R0 < rows;
    // every wave walks the keys visible to some row of the workgroup (the
    // loads are shared); a wave's own masks hide what its rows cannot see
    const int Rg = min(R0 - wave * kRowsPerWave + kPrefillRowsPerGroup - 1, rows - 1);
    const int kend = min(L, L - nq + Rg / G + 1);
    const int nblk = kend > 0 ? (kend + kBlockSize - 1) / kBlockSize : 0;
    const int NU = (nblk + 2 * kP - 1) / (2 * kP);  // steps
    const int n = lane & 31;
    const int h = lane >> 5;
    const int Hq = p.num_q_heads;

    int qpos = -1;
    int64_t orow = -1;
    {
        const int R = R0 + n;
        if (R < rows) {
            const int t = R / G;
            qpos = L - nq + t;  // < 0: no key is visible
            orow = ((int64_t)(r0 + t) * Hq + kvh * G + (R - t * G)) * D;
        }
    }
    // Q^T operands, step c: dims 16c + 8h .. +7 of row n.  A negative scale
    // rides on q (negating bf16 is exact); the softmax uses c = |scale log2 e|.
    const float c_scale = fabsf(p.scale_log2);
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    bf16x8_t qv[kKC];
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int c = 0; c < kKC; ++c) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (orow >= 0) w = *reinterpret_cast<const uint4*>(qb + orow + 16 * c + 8 * h);
        w.x ^= qsign;
        w.y ^= qsign;
        w.z ^= qsign;
        w.w ^= qsign;
        qv[c] = __builtin_bit_cast(bf16x8_t, w);
    }

    float16v_t acc[kDT];
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    float m_ref = -INFINITY;  // reference max (log2 units, same in both halves)
    float l_sum = 0.f;        // this lane's share of the sum of weights

    if (NU > 0) {
        const int64_t block_stride = (int64_t)p.num_kv_heads * D * kBlockSize;
        const uint16_t* k_head = reinterpret_cast<const uint16_t*>(p.k_cache) + (int64_t)kvh * D * kBlockSize;
        const uint16_t* v_head = reinterpret_cast<const uint16_t*>(p.v_cache) + (int64_t)kvh * D * kBlockSize;
        const scalar_i32_ptr bt = (scalar_i32_ptr)(p.block_tables + (int64_t)s * p.max_blocks_per_seq);
        // This wave's loads: wave w copies block (w mod 4) of the step (pair
        // (w mod 4) / 2, block A or B of it), K for w < 4, V otherwise, in
        // kStepLoads loads of 64 chunks.  K is copied as the pool lays it
        // out; V chunk 64t + lane' (lane' = 32h' + n') is dim 32t + n',
        // tokens 8h' .. +7.
        const bool ld_v = wave >= 4;
        const int ld_blk = wave & 3;
        const uint16_t* const ld_head = ld_v ? v_head : k_head;
        const int ld_at = (ld_v ? kP * WS::kKChunks : 0) + ld_blk * WS::kBlockChunks;  // its chunks in a slot
        int ld_off[kStepLoads];  // this lane's byte offset within the block, per load
#pragma unroll
        for (int j = 0; j < kStepLoads; ++j)
            ld_off[j] = 16 * (ld_v ? (32 * j + (lane & 31)) * 2 + (lane >> 5) : 64 * j + lane);
        // the step's blocks -> the descriptor of this wave's block (scalar
        // work), then its loads into one ring slot
        auto dma_prepare = [&](const int (&pb)[2 * kP]) __attribute__((always_inline)) {
            static_assert(kP == 2, "four blocks per step");
            // this wave's block by a uniform two-level choice (an indexed
            // array, which a chain of selects becomes, would go to scratch)
            const int lo = (ld_blk & 1) ? pb[1] : pb[0];
            const int hi = (ld_blk & 1) ? pb[3] : pb[2];
            const int blk = (ld_blk & 2) ? hi : lo;
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ld_head + (int64_t)blk * block_stride),
                                                     (short)0, WS::kBlockChunks * 16, 0x00020000);
        };
        // slot q is a constant: each slot is an LDS array of its own
        auto dma_issue = [&](auto q_tag, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
            constexpr int q = decltype(q_tag)::value;
            uint4* const dst = (q == 0 ? slot0 : q == 1 ? slot1 : slot2) + ld_at;
#pragma unroll
            for (int j = 0; j < kStepLoads; ++j) buffer_load_lds16(rs, (lds_void_ptr)(dst + 64 * j), ld_off[j]);
        };

        const uint32_t nb_u32 = (uint32_t)min(p.num_blocks, (int64_t)0x7fffffff);  // entries are int32
        uint32_t okm = 0;  // bit 4(u mod 4) + b: block b of step u lies inside the pool (and the walk)
        struct Pending {
            int e[2 * kP];  // table entries as read (checked when accepted)
            int u;          // their step
        };
        auto fetch = [&](Pending& pd, int u) __attribute__((always_inline)) {
            pd.u = min(u, NU - 1);  // past the end: the last step's blocks again (loaded, never used)
#pragma unroll
            for (int b = 0; b < 2 * kP; ++b) pd.e[b] = bt[min(2 * kP * pd.u + b, nblk - 1)];
        };
        // checked entries -> physical blocks (an id outside the pool loads
        // block 0); the empty asm pins the wait for the scalar loads here
        auto accept = [&](const Pending& pd, int (&pb)[2 * kP]) __attribute__((always_inline)) {
            uint32_t bits = 0;
#pragma unroll
            for (int b = 0; b < 2 * kP; ++b) {
                // 0 <= entry < pool size, as one unsigned compare
                const bool ok = ((uint32_t)pd.e[b] < nb_u32) & (2 * kP * pd.u + b < nblk);
                pb[b] = ok ? pd.e[b] : 0;
                bits |= (uint32_t)ok << b;
                asm volatile("" : "+s"(pb[b]));
            }
            const int sh = 2 * kP * (pd.u & 3);
            okm = (okm & ~(((1u << (2 * kP)) - 1) << sh)) | (bits << sh);
        };
        // valid tokens of block b (0 .. 2 kP - 1) of step u
        auto nv_of = [&](int u, int b) __attribute__((always_inline)) {
            return ((okm >> (2 * kP * (u & 3) + b)) & 1u) ? min(kBlockSize, L - (2 * kP * u + b) * kBlockSize) : 0;
        };

        // prologue: the entries of steps 0, 1 and 2 read together, the
        // loads of steps 0 and 1.  Later steps read the entries of step
        // u + 3 after their last LDS read, so the scalar reads land during
        // the next barrier (see below).
        Pending pend;
        {
            Pending p0, p1;
            fetch(p0, 0);
            fetch(p1, 1);
            fetch(pend, 2);
            int pb[2 * kP];
            accept(p0, pb);
            __builtin_amdgcn_sched_barrier(0);
            dma_issue(std::integral_constant<int, 0>{}, dma_prepare(pb));
            __builtin_amdgcn_sched_barrier(0);
            accept(p1, pb);
            __builtin_amdgcn_sched_barrier(0);
            dma_issue(std::integral_constant<int, 1>{}, dma_prepare(pb));
            __builtin_amdgcn_sched_barrier(0);
        }

        if (has_rows) {
            const int qmin = L - nq + R0 / G;  // first query position of the wave
            // QK operand of step c: key row n = token swap_bits23(n % 16) of
            // block n / 16, dims 16c + 8h .. +7 = chunk (2c + h, token) of the
            // block as the pool lays it out
            const int k_lane = (n >> 4) * WS::kBlockChunks + h * kBlockSize + swap_bits23(n & 15);

            // Step u (pairs 2u, 2u + 1).  kMasked: some block holds tokens
            // past the context end or past some row's position (the causal
            // diagonal), or lies outside the pool.
            auto step = [&](int u, auto masked_tag, auto q_tag) __attribute__((always_inline)) {
                constexpr bool kMasked = decltype(masked_tag)::value;
                constexpr int kQ = decltype(q_tag)::value;  // u mod 3
                const uint4* const src = kQ == 0 ? slot0 : kQ == 1 ? slot1 : slot2;  // step u
                // every load but those of step u - 1 has landed, in every wave
                wait_vmcnt<kStepLoads>();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                // the loads of step u + 2 (into the slot step u - 1 read) go out
                // under the QK products below
                __amdgpu_buffer_rsrc_t rs;
                {
                    int pb[2 * kP];
                    accept(pend, pb);  // step u + 2
                    rs = dma_prepare(pb);
                }
                // No scalar read may be out during the operand reads: scalar
                // and LDS reads share one counter, and while a scalar read is
                // out (they may return out of order) every LDS wait is a wait
                // for all of them.  (The entries of step u + 3 are read after
                // this step's last LDS read.)
                __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
                __builtin_amdgcn_sched_barrier(0);

                // ---- QK: one chain of D/16 products per pair, interleaved
                dma_issue(std::integral_constant<int, (kQ + 2) % 3>{}, rs);
                float16v_t x[kP];
#pragma unroll
                for (int a = 0; a < kP; ++a)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[a][r] = 0.f;
#pragma unroll
                for (int c = 0; c < kKC; ++c)
#pragma unroll
                    for (int a = 0; a < kP; ++a)
                        x[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, src[a * WS::kKChunks + 32 * c + k_lane]), qv[c], x[a], 0, 0, 0);
                // K reads run two products ahead (LDS latency is some 100
                // cycles); the step's loads go out one per product pair
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * kP, 0);
#pragma unroll
                for (int c = 0; c < kKC; ++c) {
                    __builtin_amdgcn_sched_group_barrier(0x8, kP, 0);
                    if (c + 2 < kKC) __builtin_amdgcn_sched_group_barrier(0x100, kP, 0);
                    if (c < kStepLoads) __builtin_amdgcn_sched_group_barrier(0x20, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                // V operands of the first block: read now, used after the softmax
                uint4 v_first[kDT];
#pragma unroll
                for (int t = 0; t < kDT; ++t) v_first[t] = src[kP * WS::kKChunks + 64 * t + lane];
                __builtin_amdgcn_sched_barrier(0);
                // ---- mask, maxima, new reference, weights
                if constexpr (kMasked) {
#pragma unroll
                    for (int b = 0; b < 2 * kP; ++b) {
                        const int nv = nv_of(u, b);
                        const int kp0 = (2 * kP * u + b) * kBlockSize + 8 * h;  // key position of its register 0
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            const float e = x[b >> 1][8 * (b & 1) + r];
                            x[b >> 1][8 * (b & 1) + r] = (8 * h + r < nv) && (kp0 + r <= qpos) ? e * c_scale : -INFINITY;
                        }
                    }
                }
                float m16 = x[0][0];
#pragma unroll
                for (int a = 0; a < kP; ++a)
#pragma unroll
                    for (int r = (a == 0 ? 1 : 0); r < 16; ++r) m16 = fmaxf(m16, x[a][r]);
                // unmasked: every score is live and c >= 0, so scale the max only
                const float mx = kMasked ? max_halves(m16) : max_halves(m16) * c_scale;
                const bool raise = mx > m_ref + kSlack;
                const float alpha = raise ? exp2_fast(m_ref - mx) : 1.f;  // m_ref = -inf -> 0
                m_ref = raise ? mx : m_ref;
                const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
                uint4 pw[kP][2];  // bf16 weights: B operands of the PV products, pair a, block b
                float lp = 0.f;
#pragma unroll
                for (int a = 0; a < kP; ++a) {
                    float pr[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        pr[r] = kMasked ? exp2_fast(x[a][r] - m_use) : exp2_fast(fmaf(x[a][r], c_scale, -m_use));
                    lp += (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]))) +
                          (((pr[8] + pr[9]) + (pr[10] + pr[11])) + ((pr[12] + pr[13]) + (pr[14] + pr[15])));
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        pw[a][b] = make_uint4(pack_bf16x2(pr[8 * b + 0], pr[8 * b + 1]), pack_bf16x2(pr[8 * b + 2], pr[8 * b + 3]),
                                              pack_bf16x2(pr[8 * b + 4], pr[8 * b + 5]), pack_bf16x2(pr[8 * b + 6], pr[8 * b + 7]));
                }
                // rarely taken (see kSlack): the output so far moves to the new reference
                if (__any(raise)) {
#pragma unroll
                    for (int t = 0; t < kDT; ++t) acc[t] *= alpha;
                }
                l_sum = fmaf(l_sum, alpha, lp);
                __builtin_amdgcn_sched_barrier(0);

                // ---- PV; tokens past a block's valid count are zeroed in
                // masked steps (they may hold NaN, and 0 * NaN = NaN)
#pragma unroll
                for (int a = 0; a < kP; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        uint4 vop[kDT];
#pragma unroll
                        for (int t = 0; t < kDT; ++t)
                            vop[t] = (a == 0 && b == 0) ? v_first[t]
                                                        : src[kP * WS::kKChunks + a * WS::kVChunks + 64 * (b * kDT + t) + lane];
                        if constexpr (kMasked) {
                            const int nv = nv_of(u, 2 * a + b) - 8 * h;
                            const uint32_t m0 = tail_mask(nv, 0), m1 = tail_mask(nv, 2), m2 = tail_mask(nv, 4),
                                           m3 = tail_mask(nv, 6);
#pragma unroll
                            for (int t = 0; t < kDT; ++t) {
                                vop[t].x &= m0;
                                vop[t].y &= m1;
                                vop[t].z &= m2;
                                vop[t].w &= m3;
                            }
                        }
#pragma unroll
                        for (int t = 0; t < kDT; ++t)
                            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8_t, vop[t]), __builtin_bit_cast(bf16x8_t, pw[a][b]), acc[t], 0, 0, 0);
                    }
                if constexpr (!kMasked) {
                    // each block's V reads go out under the previous block's products
#pragma unroll
                    for (int g = 0; g < 2 * kP; ++g) {
                        if (g + 1 < 2 * kP) __builtin_amdgcn_sched_group_barrier(0x100, kDT, 0);
                        __builtin_amdgcn_sched_group_barrier(0x8, kDT, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                fetch(pend, u + 3);
            };

            // Steps [0, NUf) see only keys visible to every row of the wave,
            // all cached: they skip the mask.  (A table entry outside the pool
            // there is read as block 0 -- never out of bounds, but the result
            // is then unspecified; masked steps skip such a block.)
            const int NUf = min(NU, (qmin + 1) / kKeysPerStep);
            using F = std::false_type;
            using T = std::true_type;
            int u = 0;
            for (; u + 3 <= NUf; u += 3) {
                step(u, F{}, std::integral_constant<int, 0>{});
                step(u + 1, F{}, std::integral_constant<int, 1>{});
                step(u + 2, F{}, std::integral_constant<int, 2>{});
            }
            for (; u < NU; u += 3) {
                step(u, T{}, std::integral_constant<int, 0>{});
                if (u + 1 < NU) step(u + 1, T{}, std::integral_constant<int, 1>{});
                if (u + 2 < NU) step(u + 2, T{}, std::integral_constant<int, 2>{});
            }
        } else {
            // no rows here: this wave's share of the loads, and the barriers
            for (int u = 0; u < NU; ++u) {
                wait_vmcnt<kStepLoads>();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                int pb[2 * kP];
                accept(pend, pb);  // step u + 2
                const __amdgpu_buffer_rsrc_t rs = dma_prepare(pb);
                const int q = (u + 2) % 3;
                if (q == 0) dma_issue(std::integral_constant<int, 0>{}, rs);
                else if (q == 1) dma_issue(std::integral_constant<int, 1>{}, rs);
                else dma_issue(std::integral_constant<int, 2>{}, rs);
                __builtin_amdgcn_sched_barrier(0);
                fetch(pend, u + 3);
            }
        }
        wait_vmcnt<0>();  // no load into LDS outlives the workgroup
    }
    if (!has_rows) return;

    // ---- epilogue: out = O / l (zeros for rows that see no key); lane
    // (n, h), register 4q + e of tile t holds dim 32t + 8q + 4h + e
    const float lt = sum_halves(l_sum);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (orow < 0) return;
    const bool obf = p.out_bf16 != 0;
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int64_t o = orow + 32 * t + 8 * q4 + 4 * h;
            const float a0 = acc[t][4 * q4 + 0] * inv, a1 = acc[t][4 * q4 + 1] * inv;
            const float a2 = acc[t][4 * q4 + 2] * inv, a3 = acc[t][4 * q4 + 3] * inv;
            if (obf)
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o) =
                    make_uint2(f32_to_bf16_bits(a0) | (f32_to_bf16_bits(a1) << 16),
                               f32_to_bf16_bits(a2) | (f32_to_bf16_bits(a3) << 16));
            else
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) = make_float4(a0, a1, a2, a3);
        }
}

}  // namespace

hipError_t launch_prefill_wide(const PrefillParams& p, hipStream_t stream) {
    if (p.num_seqs == 0 || p.tile_bound == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.tile_bound * p.num_kv_heads));
    const size_t lds = prefill_lds_bytes(p.num_seqs, p.lpt_buckets);
    if (p.head_dim == 128) hipLaunchKernelGGL((prefill_wide_kernel<128>), grid, dim3(512), lds, stream, p);
    else hipLaunchKernelGGL((prefill_wide_kernel<64>), grid, dim3(512), lds, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
