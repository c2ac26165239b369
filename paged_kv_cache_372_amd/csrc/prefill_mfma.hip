// Multi-token-query paged attention (chunked prefill) over an fp8 (E4M3)
// cache, on the gfx950 matrix cores.  (bf16 pools take prefill_wide.hip.)
//
// What is computed.  A request s brings n_s >= 1 new query tokens whose keys
// and values are already in the paged cache, which then holds L_s tokens, the
// new ones last.  Query i (position p = L_s - n_s + i) attends over positions
// 0..p: causal attention aligned at the end of the context.  n_s = 1 is
// decode.  Prefill is the parallel, compute-heavy stage (runbyai section 1);
// long prompts are cut into chunks that share each step with decode requests
// (architvora "Continuous Batching"), so a chunk attends over everything
// cached before it plus itself.  The keys are reached through the request's
// block table (architvora "Paged Attention").  K and V are stored as E4M3
// codes with one scale per KV head: K's scale joins the score scale, V's
// the output.
//
// Work decomposition.  The rows of a request are its (query token, head of
// the KV group) pairs, token-major: n_s * G rows per KV head.  A workgroup
// takes 256 consecutive rows of one (request, KV head); each of its 8 waves
// takes 32 rows and walks, on its own, the key blocks those rows can see.
// The waves read the same K/V blocks at about the same time, so the
// workgroup's loads hit in L1/L2 after the first; the KV head is the
// workgroup index modulo Hkv, which keeps each head on one XCD (with 8 KV
// heads) and its blocks in that XCD's L2.  Heaviest tiles (the last rows of
// a request see the most keys) are launched first.
//
// Per pair of 16-token blocks (A, B), per wave, for each of its two 16-row
// column tiles j:
//   S^T[32 keys x 16 rows] = K . Q_j^T        2 x D/32 x mfma_f32_16x16x32_bf16
//   online softmax on S (exp2 domain, scale*log2e folded in, causal mask)
//   O_j^T[D x 16 rows] += V^T . P_j^T         D/16 x mfma_f32_16x16x32_f16
// The K-dimension of the PV product runs over the 32 keys of the pair in the
// order (A 4g..4g+3, B 4g..4g+3) for lane group g: that is exactly what the
// QK result leaves in each lane, so P needs no data movement, and the V^T
// operand is the two 8-byte V rows of A and B side by side (see widen_pair).
// P is rounded once, to fp16, against V's codes as fp16.
//
// Memory: K/V codes are loaded straight from the pool into a register ring
// two pairs deep (each load a contiguous 1 KiB run per wave); table entries
// come through the scalar cache one round ahead, as in the decode kernel.
#include <type_traits>

#include "prefill_common.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Shape of a workgroup: 8 waves of 32 rows.  The ring of raw codes is half
// the registers bf16 operands would take, so two waves fit per SIMD and one
// wave's softmax runs under the other's products.  Measured on the
// chunked-prefill workload over an fp8 cache: 662 against 583 TFLOP/s for 4
// waves of 64 rows (one pair in flight: 637).
struct Fp8Shape {
    static constexpr int kWaves = 8;
    static constexpr int kRowsPerWave = kPrefillRowsPerGroup / kWaves;
    static constexpr int kNQ = kRowsPerWave / 16;  // 16-row column tiles per wave
    static constexpr int kPairDepth = 2;           // block pairs in flight per wave
};
constexpr int kExpValu = 28;                     // VALU instructions for one column tile's weights

template <int D>
struct PairRegs {
    uint4 k[2][D / 32];  // block A, B: load kk holds chunk 4kk + l/16 of token l%16
    u32x4_t v[D / 16];   // dim 16c + l%16: A's tokens 4(l/16)..+3 in .xy, B's in .zw
};

// The same pair from an fp8 (E4M3) cache, as loaded: K load i holds the
// 16-dim chunk 4i + l/16 of token l%16; V load i holds the 16-token row of
// dim 64i + l.  widen_pair turns it into the bf16 operands above (every
// E4M3 value is exact in bf16).
template <int D>
struct PairRegs8 {
    uint4 k[2][D / 64];
    uint4 v[2][D / 64];
};

template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    // codes of bytes 2*kHigh, 2*kHigh + 1; scale 1.0: the exact value of each code
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    // the same codes as fp16: every E4M3 value (at most 448, at least 2^-9
    // apart from zero, 4 significant bits) is exact in fp16 too
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHigh));
}

// K becomes bf16 operands (q is bf16); V becomes fp16 operands, for a PV
// product in fp16: the weights then enter it with 11 significant bits
// instead of bf16's 8 (weights lie in [0, 2^8], inside fp16's range; those
// below 2^-24 flush to zero, next to a largest weight of at least 1).
// K: the QK contraction takes dims in the order that makes step kk read half
// (kk & 1) of chunk load kk / 2 (q is loaded in the same order).  V: word c
// of lane (d, g) must hold tokens 4g..4g+3 of dim 16c + d, while lane
// (d, r) loaded dims 64i + 16r + d: a 4 x 4 transpose of words between the
// four 16-lane rows, in two rounds of row swaps.
template <int D>
__device__ __forceinline__ PairRegs<D> widen_pair(const PairRegs8<D>& r) {
    PairRegs<D> o;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const uint4 w = r.k[b][kk >> 1];
            const uint32_t x = (kk & 1) ? w.z : w.x;
            const uint32_t y = (kk & 1) ? w.w : w.y;
            o.k[b][kk] = make_uint4(e4m3x2_to_bf16x2<false>(x), e4m3x2_to_bf16x2<true>(x),
                                    e4m3x2_to_bf16x2<false>(y), e4m3x2_to_bf16x2<true>(y));
        }
    uint32_t w[2][D / 16];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const auto a = __builtin_amdgcn_permlane32_swap(r.v[b][i].x, r.v[b][i].z, false, false);
            const auto c = __builtin_amdgcn_permlane32_swap(r.v[b][i].y, r.v[b][i].w, false, false);
            const auto e = __builtin_amdgcn_permlane16_swap(a[0], c[0], false, false);
            const auto f = __builtin_amdgcn_permlane16_swap(a[1], c[1], false, false);
            w[b][4 * i + 0] = e[0];
            w[b][4 * i + 1] = e[1];
            w[b][4 * i + 2] = f[0];
            w[b][4 * i + 3] = f[1];
        }
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        o.v[c] = u32x4_t{e4m3x2_to_f16x2<false>(w[0][c]), e4m3x2_to_f16x2<true>(w[0][c]),
                         e4m3x2_to_f16x2<false>(w[1][c]), e4m3x2_to_f16x2<true>(w[1][c])};
    return o;
}

// Uniform facts about a pair: first logical block and valid tokens of A, B.
struct PairInfo {
    int blk;
    int nv_a;
    int nv_b;
};

struct PairPending {
    int ea, eb;  // table entries as read (validated at use)
    int k;       // pair index (clamped)
};

struct ColState {
    float m;  // reference max, log2 units (same in the four lane groups of a column)
    float l;  // this lane's share of the sum of weights
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
// two fp32 -> packed fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, f16x2_t));
}

template <int D>
__global__ __launch_bounds__(64 * Fp8Shape::kWaves) void prefill_fp8_kernel(PrefillParams p) {
    constexpr int kPrefillWaves = Fp8Shape::kWaves;
    constexpr int kPrefillRowsPerWave = Fp8Shape::kRowsPerWave;
    constexpr int kNQ = Fp8Shape::kNQ;
    constexpr int kPairDepth = Fp8Shape::kPairDepth;
    using Ring = PairRegs8<D>;
    extern __shared__ int32_t plan[];  // tile order (see locate_rows)
    __shared__ int32_t wave_total[kPrefillWaves];
    const int G = p.group;
    const int lane = threadIdx.x & 63;
    WaveRows wr;
    if (!locate_rows<kPrefillWaves, kPrefillRowsPerWave>(p, plan, wave_total, wr)) return;
    const int s = wr.s, r0 = wr.r0, n = wr.n, rows = wr.rows, R0 = wr.R0, L = wr.L, kvh = wr.kvh;
    if (R0 >= rows) return;  // no barrier follows
    const int Rl = min(R0 + kPrefillRowsPerWave - 1, rows - 1);
    const int kend = min(L, L - n + Rl / G + 1);  // keys [0, kend) are visible to some row

    const int col = lane & 15;
    const int g = lane >> 4;
    const int Hq = p.num_q_heads;

    // per column tile: query position of this lane's row and its row offset
    int qpos[kNQ];
    int64_t orow[kNQ];
#pragma unroll
    for (int j = 0; j < kNQ; ++j) {
        const int R = R0 + 16 * j + col;
        if (R < rows) {
            const int t = R / G;
            qpos[j] = L - n + t;  // < 0: no key is visible
            orow[j] = ((int64_t)(r0 + t) * Hq + kvh * G + (R - t * G)) * D;
        } else {
            qpos[j] = -1;
            orow[j] = -1;
        }
    }

    // Q^T operands: step kk, k-group g holds dims 64(kk/2) + 16g + 8(kk&1)
    // .. +7, the order widen_pair gives K.  A negative scale is carried by q
    // (negating bf16 is exact), so the softmax below works with
    // c = |scale * log2 e * k_scale| >= 0.
    const float eff_scale = p.scale_log2 * p.k_scale[kvh];
    const float c_scale = fabsf(eff_scale);
    const uint32_t qsign = eff_scale < 0.f ? 0x80008000u : 0u;
    bf16x8_t qv[kNQ][D / 32];
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int j = 0; j < kNQ; ++j)
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            uint4 w = make_uint4(0, 0, 0, 0);
            const int dq = 64 * (kk >> 1) + 16 * g + 8 * (kk & 1);
            if (orow[j] >= 0) w = *reinterpret_cast<const uint4*>(qb + orow[j] + dq);
            w.x ^= qsign;
            w.y ^= qsign;
            w.z ^= qsign;
            w.w ^= qsign;
            qv[j][kk] = __builtin_bit_cast(bf16x8_t, w);
        }
    // first query position of the wave: a pair ending at or before it is
    // visible to every row
    const int qmin = L - n + R0 / G;

    float4_t acc[kNQ][D / 16];
#pragma unroll
    for (int j = 0; j < kNQ; ++j)
#pragma unroll
        for (int c = 0; c < D / 16; ++c) acc[j][c] = {0.f, 0.f, 0.f, 0.f};
    ColState st[kNQ];
#pragma unroll
    for (int j = 0; j < kNQ; ++j) st[j] = {-INFINITY, 0.f};

    const int nblk = kend > 0 ? (kend + kBlockSize - 1) / kBlockSize : 0;
    const int NP = (nblk + 1) / 2;

    if (NP > 0) {
        const int64_t block_stride = (int64_t)p.num_kv_heads * D * kBlockSize;
        const uint8_t* k_head = reinterpret_cast<const uint8_t*>(p.k_cache) + (int64_t)kvh * D * kBlockSize;
        const uint8_t* v_head = reinterpret_cast<const uint8_t*>(p.v_cache) + (int64_t)kvh * D * kBlockSize;
        const scalar_i32_ptr bt = (scalar_i32_ptr)(p.block_tables + (int64_t)s * p.max_blocks_per_seq);

        Ring ring[kPairDepth];
        PairInfo info[kPairDepth];
        PairPending pend[kPairDepth];

        auto fetch = [&](int k, PairPending& e) __attribute__((always_inline)) {
            const int kc = min(k, NP - 1);
            e.k = kc;
            e.ea = bt[2 * kc];
            e.eb = bt[min(2 * kc + 1, nblk - 1)];
        };
        // checked entries -> physical blocks to load (an id outside the pool
        // loads block 0 with no valid token); the empty asm pins the wait
        // for the scalar loads here
        auto accept = [&](const PairPending& e, int& pa, int& pb, PairInfo& inf) __attribute__((always_inline)) {
            const bool oka = e.ea >= 0 && (int64_t)e.ea < p.num_blocks;
            const bool okb = e.eb >= 0 && (int64_t)e.eb < p.num_blocks && 2 * e.k + 1 < nblk;
            pa = oka ? e.ea : 0;
            pb = okb ? e.eb : 0;
            inf.blk = 2 * e.k;
            inf.nv_a = oka ? min(kBlockSize, L - 2 * e.k * kBlockSize) : 0;
            inf.nv_b = okb ? min(kBlockSize, L - (2 * e.k + 1) * kBlockSize) : 0;
            asm volatile("" : "+s"(pa), "+s"(pb));
        };
        auto load_pair = [&](int d, int pa, int pb, const PairInfo& inf) __attribute__((always_inline)) {
            info[d] = inf;
            // ordinary loads: the other waves and workgroups of this request
            // read the same blocks
            const u32x4_t* ka = reinterpret_cast<const u32x4_t*>(k_head + (int64_t)pa * block_stride);
            const u32x4_t* kb = reinterpret_cast<const u32x4_t*>(k_head + (int64_t)pb * block_stride);
            const u32x4_t* va = reinterpret_cast<const u32x4_t*>(v_head + (int64_t)pa * block_stride);
            const u32x4_t* vb = reinterpret_cast<const u32x4_t*>(v_head + (int64_t)pb * block_stride);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) ring[d].k[0][i] = __builtin_bit_cast(uint4, ka[i * 64 + lane]);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) ring[d].k[1][i] = __builtin_bit_cast(uint4, kb[i * 64 + lane]);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) ring[d].v[0][i] = __builtin_bit_cast(uint4, va[i * 64 + lane]);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) ring[d].v[1][i] = __builtin_bit_cast(uint4, vb[i * 64 + lane]);
        };

        // One pair.  kMasked: the pair holds tokens past the context end or
        // past some row's position (the causal diagonal); otherwise every
        // score is live and the mask work is skipped.
        auto compute_pair = [&](Ring& rr, const PairInfo& inf, auto masked_tag) __attribute__((always_inline)) {
            constexpr bool kMasked = decltype(masked_tag)::value;
            PairRegs<D> r = widen_pair<D>(rr);
            if constexpr (kMasked) {
                // tokens past a block's valid count are zeroed in place (they
                // may hold NaN, and 0 * NaN = NaN)
                const uint32_t ma0 = tail_mask(inf.nv_a - 4 * g, 0), ma1 = tail_mask(inf.nv_a - 4 * g, 2);
                const uint32_t mb0 = tail_mask(inf.nv_b - 4 * g, 0), mb1 = tail_mask(inf.nv_b - 4 * g, 2);
#pragma unroll
                for (int c = 0; c < D / 16; ++c) r.v[c] &= u32x4_t{ma0, ma1, mb0, mb1};
            }
            const int kpa = inf.blk * kBlockSize + 4 * g;  // key position of this lane's first A token
            const int kpb = kpa + kBlockSize;
            // S^T of both blocks for every column tile, then the new maxima
            float sv[kNQ][8];
            float mx[kNQ];
#pragma unroll
            for (int j = 0; j < kNQ; ++j) {
                float4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk) {
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[0][kk]), qv[j][kk],
                                                                 sa, 0, 0, 0);
                    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[1][kk]), qv[j][kk],
                                                                 sb, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sv[j][i] = sa[i];
                    sv[j][4 + i] = sb[i];
                }
                if constexpr (kMasked) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool oa = (4 * g + i < inf.nv_a) && (kpa + i <= qpos[j]);
                        const bool ob = (4 * g + i < inf.nv_b) && (kpb + i <= qpos[j]);
                        sv[j][i] = oa ? sv[j][i] * c_scale : -INFINITY;
                        sv[j][4 + i] = ob ? sv[j][4 + i] * c_scale : -INFINITY;
                    }
                }
                float m8 = fmaxf(fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3])),
                                 fmaxf(fmaxf(sv[j][4], sv[j][5]), fmaxf(sv[j][6], sv[j][7])));
                // unmasked: all scores live and c >= 0, so scale the max only
                mx[j] = kMasked ? max_over_groups(m8) : max_over_groups(m8) * c_scale;
            }
            // one rescale check for the pair (rarely taken: see kSlack)
            bool raise[kNQ];
            bool any = false;
#pragma unroll
            for (int j = 0; j < kNQ; ++j) {
                raise[j] = mx[j] > st[j].m + kSlack;
                any = any || raise[j];
            }
            if (__any(any)) {
#pragma unroll
                for (int j = 0; j < kNQ; ++j) {
                    const float alpha = raise[j] ? exp2_fast(st[j].m - mx[j]) : 1.f;  // m = -inf -> 0
                    st[j].l *= alpha;
#pragma unroll
                    for (int c = 0; c < D / 16; ++c) acc[j][c] *= alpha;
                    st[j].m = raise[j] ? mx[j] : st[j].m;
                }
            }
            // weights and the PV products
#pragma unroll
            for (int j = 0; j < kNQ; ++j) {
                const float m_use = st[j].m == -INFINITY ? 0.f : st[j].m;
                float pr[8];
                if constexpr (kMasked) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) pr[i] = exp2_fast(sv[j][i] - m_use);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) pr[i] = exp2_fast(fmaf(sv[j][i], c_scale, -m_use));
                }
                st[j].l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
                // fp16 weights against the fp16 V operands (see widen_pair)
                const f16x8_t pj = __builtin_bit_cast(
                    f16x8_t, make_uint4(pack_f16x2(pr[0], pr[1]), pack_f16x2(pr[2], pr[3]),
                                        pack_f16x2(pr[4], pr[5]), pack_f16x2(pr[6], pr[7])));
#pragma unroll
                for (int c = 0; c < D / 16; ++c)
                    acc[j][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, r.v[c]), pj,
                                                                       acc[j][c], 0, 0, 0);
            }
            if constexpr (!kMasked) {
                // Interleave: the weights of tile j + 1 (VALU) are computed
                // while the matrix core runs the PV products of tile j, so
                // neither unit waits for the other.  (Masks: 0x2 VALU,
                // 0x8 MFMA.)
                __builtin_amdgcn_sched_group_barrier(0x2, kExpValu, 0);
#pragma unroll
                for (int t = 0; t < (kNQ - 1) * (D / 16); ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x2, kExpValu / (D / 16), 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x8, D / 16, 0);
            }
        };

        // prologue: entries of the first kPairDepth pairs, then those of the
        // next round, then the first loads
        int next_pa[kPairDepth], next_pb[kPairDepth];
        PairInfo next_info[kPairDepth];
#pragma unroll
        for (int d = 0; d < kPairDepth; ++d) fetch(d, pend[d]);
#pragma unroll
        for (int d = 0; d < kPairDepth; ++d) accept(pend[d], next_pa[d], next_pb[d], next_info[d]);
#pragma unroll
        for (int d = 0; d < kPairDepth; ++d) fetch(kPairDepth + d, pend[d]);
#pragma unroll
        for (int d = 0; d < kPairDepth; ++d) {
            load_pair(d, next_pa[d], next_pb[d], next_info[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
        auto round = [&](int i, auto final_tag, auto masked_tag) __attribute__((always_inline)) {
            constexpr bool kFinal = decltype(final_tag)::value;
#pragma unroll
            for (int d = 0; d < kPairDepth; ++d) accept(pend[d], next_pa[d], next_pb[d], next_info[d]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < kPairDepth; ++d) fetch(i + 2 * kPairDepth + d, pend[d]);
#pragma unroll
            for (int d = 0; d < kPairDepth; ++d) {
                if (!kFinal || i + d < NP) compute_pair(ring[d], info[d], masked_tag);
                __builtin_amdgcn_sched_barrier(0);
                if (!kFinal || i + d + kPairDepth < NP) load_pair(d, next_pa[d], next_pb[d], next_info[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // Pairs [0, NPf) are visible to every row of the wave and hold 32
        // cached tokens: their rounds skip the mask.  (A table entry outside
        // the pool there is read as block 0 -- never out of bounds, but the
        // result is then unspecified; in masked rounds such a block is
        // skipped.)  The rest, the causal diagonal and the context end
        // included, take the masked form.
        const int NPf = min(NP, (qmin + 1) / (2 * kBlockSize));
        int i = 0;
        for (; i + 2 * kPairDepth <= NP && i + kPairDepth <= NPf; i += kPairDepth)
            round(i, std::false_type{}, std::false_type{});
        for (; i + 2 * kPairDepth <= NP; i += kPairDepth) round(i, std::false_type{}, std::true_type{});
        for (; i < NP; i += kPairDepth) round(i, std::true_type{}, std::true_type{});
    }

    // ---- epilogue: out = O / l (zeros for rows that see no key)
    const bool obf = p.out_bf16 != 0;
#pragma unroll
    for (int j = 0; j < kNQ; ++j) {
        const float lt = sum_over_groups(st[j].l);
        const float inv = lt > 0.f ? p.v_scale[kvh] / lt : 0.f;
        if (orow[j] < 0) continue;
        if (obf) {
            uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + orow[j] + 4 * g;
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                *reinterpret_cast<uint2*>(ob + 16 * c) =
                    make_uint2(f32_to_bf16_bits(acc[j][c][0] * inv) | (f32_to_bf16_bits(acc[j][c][1] * inv) << 16),
                               f32_to_bf16_bits(acc[j][c][2] * inv) | (f32_to_bf16_bits(acc[j][c][3] * inv) << 16));
        } else {
            float* of = reinterpret_cast<float*>(p.out) + orow[j] + 4 * g;
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                *reinterpret_cast<float4*>(of + 16 * c) = make_float4(acc[j][c][0] * inv, acc[j][c][1] * inv,
                                                                      acc[j][c][2] * inv, acc[j][c][3] * inv);
        }
    }
}

}  // namespace

size_t prefill_lds_bytes(int32_t num_seqs, int32_t lpt_buckets) {
    return (size_t)(num_seqs + 3 + lpt_buckets) * sizeof(int32_t);
}

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
    if (p.num_seqs == 0 || p.tile_bound == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.tile_bound * p.num_kv_heads));
    if (!p.kv_fp8) return launch_prefill_wide(p, stream);
    const dim3 block(64 * Fp8Shape::kWaves);
    const size_t lds = prefill_lds_bytes(p.num_seqs, p.lpt_buckets);
    if (p.head_dim == 128) hipLaunchKernelGGL((prefill_fp8_kernel<128>), grid, block, lds, stream, p);
    else hipLaunchKernelGGL((prefill_fp8_kernel<64>), grid, block, lds, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
