// Multi-token-query paged attention (chunked prefill) over bf16 or fp8 (E4M3)
// pools on the gfx950 matrix cores: 32 x 32 tiles, K and V staged in LDS.
//
// What is computed.  A request s brings n_s >= 1 new query tokens whose keys
// and values are already in the paged cache, which then holds L_s tokens, the
// new ones last.  Query i (position p = L_s - n_s + i) attends over positions
// 0..p: causal attention aligned at the end of the context.  n_s = 1 is
// decode.  Prefill is the parallel, compute-heavy stage (runbyai section 1);
// long prompts are cut into chunks that share each step with decode requests
// (architvora "Continuous Batching"), so a chunk attends over everything
// cached before it plus itself.  The keys are reached through the request's
// block table (architvora "Paged Attention").  With E4M3 pools, K and V carry
// one scale per KV head: K's joins the score scale, V's the output.
//
// Work decomposition.  The rows of a request are its (query token, head of
// the KV group) pairs, token-major: n_s * G rows per KV head.  A workgroup
// takes a tile of 256 consecutive rows of one (request, KV head), eight waves
// of 32 rows; the KV head is the workgroup index modulo Hkv, which keeps each
// head on one XCD (with 8 KV heads) and its blocks in that XCD's L2.
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
//
// fp8 pools.  The codes are half the bytes, and are converted once per
// workgroup, not once per consuming wave.  Each wave copies its block's codes
// as stored into its own share of a three-slot ring, three steps ahead; at
// the end of step u it converts its block of step u + 1 into a two-slot ring
// of operands laid out as above (K exactly to bf16, V exactly to fp16), and
// the next barrier publishes them.  The rest of the step is the bf16 one,
// except that the PV product runs in fp16: the weights enter it with 11
// significant bits instead of bf16's 8.  K's scale joins the score scale, V's
// the output.  LDS: 48 + 64 KiB at D = 128.
#include <type_traits>

#include "prefill_common.h"

namespace pkv {
namespace {

typedef float float16v_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
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

template <int D, bool kFp8>
struct WideShape {
    static constexpr int kThreads = 512;             // eight waves
    static constexpr int kPairs = 2;                 // pairs of blocks per step
    static constexpr int kKC = D / 16;               // QK steps per pair
    static constexpr int kDT = D / 32;               // 32-dim output tiles
    static constexpr int kKChunks = kKC * 64;        // 16-byte K operand chunks per pair
    static constexpr int kVChunks = 2 * kDT * 64;    // 16-byte V operand chunks per pair
    static constexpr int kBlockChunks = D * kBlockSize * 2 / 16;        // 16-byte operand chunks of one K or V block
    static constexpr int kSlotChunks = kPairs * (kKChunks + kVChunks);  // operands of a step: K of both pairs, then V
    static constexpr int kCodeBytes = kFp8 ? 1 : 2;                     // bytes per cached value
    static constexpr int kRawChunks = D * kBlockSize * kCodeBytes / 16;  // 16-byte chunks of one block as stored
    static constexpr int kStepLoads = kRawChunks / 64;                   // direct-to-LDS loads per thread per step
    // ring slot of the loads: bf16, the step's operands; fp8, its eight
    // blocks as stored (wave w's block at chunk w kRawChunks)
    static constexpr int kRingChunks = kFp8 ? 4 * kPairs * kRawChunks : kSlotChunks;
    // each wave loads one block of K or of V per step
    static_assert(kThreads / 64 == 2 * 2 * kPairs && kKChunks == 2 * kBlockChunks && kVChunks == 2 * kBlockChunks,
                  "one wave per block and kind");
};

template <int D, bool kFp8>
__global__ __launch_bounds__(512) void prefill_wide_kernel(PrefillParams p) {
    using WS = WideShape<D, kFp8>;
    constexpr int kWaves = WS::kThreads / 64;
    constexpr int kRowsPerWave = kPrefillRowsPerGroup / kWaves;  // 32
    static_assert(kRowsPerWave == 32, "one 32-row tile per wave");
    constexpr int kP = WS::kPairs;
    constexpr int kKC = WS::kKC, kDT = WS::kDT, kStepLoads = WS::kStepLoads;
    constexpr int kKeysPerStep = 2 * kP * kBlockSize;  // 64
    // fp8: the loads of step u + 3 go out in step u (bf16: u + 2)
    constexpr int kAhead = kFp8 ? 3 : 2;
    extern __shared__ int32_t plan[];  // tile order (see locate_rows)
    // the load ring; operand slot layout: K chunks of pair 0, of pair 1,
    // then V chunks of pair 0, of pair 1
    __shared__ uint4 slot0[WS::kRingChunks], slot1[WS::kRingChunks], slot2[WS::kRingChunks];
    // fp8: the operand ring, two slots, written by the conversion
    __shared__ uint4 cbuf[kFp8 ? 2 * WS::kSlotChunks : 1];
    // the tile search runs before any load: its scratch shares the ring
    int32_t* const wave_total = reinterpret_cast<int32_t*>(slot0);

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
    // rides on q (negating bf16 is exact); the softmax uses c = |scale log2 e|
    // (fp8: times K's scale), kept at least 2^-126 so that c times a masked
    // score (-inf) stays -inf: a zero scale then still gives weights of
    // exactly 1 to every visible key.
    const float eff_scale = kFp8 ? p.scale_log2 * p.k_scale[kvh] : p.scale_log2;
    const float c_scale = fmaxf(fabsf(eff_scale), 0x1p-126f);
    const uint32_t qsign = eff_scale < 0.f ? 0x80008000u : 0u;
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
        const int64_t block_stride = (int64_t)p.num_kv_heads * D * kBlockSize * WS::kCodeBytes;  // bytes
        const uint8_t* k_head = reinterpret_cast<const uint8_t*>(p.k_cache) + (int64_t)kvh * D * kBlockSize * WS::kCodeBytes;
        const uint8_t* v_head = reinterpret_cast<const uint8_t*>(p.v_cache) + (int64_t)kvh * D * kBlockSize * WS::kCodeBytes;
        const scalar_i32_ptr bt = (scalar_i32_ptr)(p.block_tables + (int64_t)s * p.max_blocks_per_seq);
        // This wave's loads: wave w copies block (w mod 4) of the step (pair
        // (w mod 4) / 2, block A or B of it), K for w < 4, V otherwise, in
        // kStepLoads loads of 64 chunks.  bf16: K is copied as the pool lays
        // it out; V chunk 64t + lane' (lane' = 32h' + n') is dim 32t + n',
        // tokens 8h' .. +7.  fp8: both as stored, converted below.
        const bool ld_v = wave >= 4;
        const int ld_blk = wave & 3;
        const uint8_t* const ld_head = ld_v ? v_head : k_head;
        // this wave's block in an operand slot
        const int op_at = (ld_v ? kP * WS::kKChunks : 0) + ld_blk * WS::kBlockChunks;
        // ... and in a ring slot
        const int ld_at = kFp8 ? wave * WS::kRawChunks : op_at;
        int ld_off[kStepLoads];  // this lane's byte offset within the block, per load
#pragma unroll
        for (int j = 0; j < kStepLoads; ++j)
            ld_off[j] = 16 * (ld_v && !kFp8 ? (32 * j + (lane & 31)) * 2 + (lane >> 5) : 64 * j + lane);
        // the step's blocks -> the descriptor of this wave's block (scalar
        // work), then its loads into one ring slot
        auto dma_prepare = [&](const int (&pb)[2 * kP]) __attribute__((always_inline)) {
            static_assert(kP == 2, "four blocks per step");
            // this wave's block by a uniform two-level choice (an indexed
            // array, which a chain of selects becomes, would go to scratch)
            const int lo = (ld_blk & 1) ? pb[1] : pb[0];
            const int hi = (ld_blk & 1) ? pb[3] : pb[2];
            const int blk = (ld_blk & 2) ? hi : lo;
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ld_head + (int64_t)blk * block_stride),
                                                     (short)0, WS::kRawChunks * 16, 0x00020000);
        };
        // slot q is a constant: each slot is an LDS array of its own
        auto dma_issue = [&](auto q_tag, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
            constexpr int q = decltype(q_tag)::value;
            uint4* const dst = (q == 0 ? slot0 : q == 1 ? slot1 : slot2) + ld_at;
#pragma unroll
            for (int j = 0; j < kStepLoads; ++j) buffer_load_lds16(rs, (lds_void_ptr)(dst + 64 * j), ld_off[j]);
        };
        // fp8: this wave's block of a landed ring slot -> operands in
        // operand slot v mod 2: K (stored [D/16][16 tokens][16 dims]) as bf16
        // in the bf16 pool's order ([D/8][16][8]); V (stored [D][16 tokens])
        // as fp16 in operand order.  Nobody else reads a wave's ring share,
        // so only the operand slot needs the next barrier.  Each store is one
        // 16-byte vector store at an index the optimizer may not take apart
        // (the empty asm): the compiler then still tells it apart from the
        // loads in flight, while a store whose address it has built in more
        // steps would wait for every load.
        auto convert = [&](auto q_tag, int v) __attribute__((always_inline)) {
            constexpr int q = decltype(q_tag)::value;
            const uint4* const raw = (q == 0 ? slot0 : q == 1 ? slot1 : slot2) + ld_at;
            const int base = ((v & 1) ? WS::kSlotChunks : 0) + op_at;
            auto put = [&](int idx, uint32_t a, uint32_t b, uint32_t c, uint32_t d) __attribute__((always_inline)) {
                *reinterpret_cast<u32x4v_t*>(cbuf + idx) = u32x4v_t{a, b, c, d};
            };
            uint4 w[kStepLoads];
#pragma unroll
            for (int j = 0; j < kStepLoads; ++j) w[j] = raw[64 * j + lane];
            if (!ld_v) {
#pragma unroll
                for (int j = 0; j < kStepLoads; ++j) {
                    const int i = 64 * j + lane;                // 16-dim chunk i / 16 of token i % 16
                    int o = base + i + 16 * (i >> 4);  // 8-dim chunk 2 (i / 16) of the token
                    asm("" : "+v"(o));
                    put(o, e4m3x2_to_bf16x2<false>(w[j].x), e4m3x2_to_bf16x2<true>(w[j].x),
                        e4m3x2_to_bf16x2<false>(w[j].y), e4m3x2_to_bf16x2<true>(w[j].y));
                    put(o + kBlockSize, e4m3x2_to_bf16x2<false>(w[j].z), e4m3x2_to_bf16x2<true>(w[j].z),
                        e4m3x2_to_bf16x2<false>(w[j].w), e4m3x2_to_bf16x2<true>(w[j].w));
                }
            } else {
#pragma unroll
                for (int j = 0; j < kStepLoads; ++j) {
                    const int d = 64 * j + lane;                     // dim d, 16 tokens
                    int o = base + 64 * (d >> 5) + (d & 31);  // tokens 0..7; 8..15 at +32
                    asm("" : "+v"(o));
                    put(o, e4m3x2_to_f16x2<false>(w[j].x), e4m3x2_to_f16x2<true>(w[j].x),
                        e4m3x2_to_f16x2<false>(w[j].y), e4m3x2_to_f16x2<true>(w[j].y));
                    put(o + 32, e4m3x2_to_f16x2<false>(w[j].z), e4m3x2_to_f16x2<true>(w[j].z),
                        e4m3x2_to_f16x2<false>(w[j].w), e4m3x2_to_f16x2<true>(w[j].w));
                }
            }
        };
        auto cslot = [&](int u) __attribute__((always_inline)) { return cbuf + (u & 1) * WS::kSlotChunks; };

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
            const int sh = 2 * kP * (pd.u & 3);  // steps u .. u + kAhead are live: four places
            okm = (okm & ~(((1u << (2 * kP)) - 1) << sh)) | (bits << sh);
        };
        // valid tokens of block b (0 .. 2 kP - 1) of step u
        auto nv_of = [&](int u, int b) __attribute__((always_inline)) {
            return ((okm >> (2 * kP * (u & 3) + b)) & 1u) ? min(kBlockSize, L - (2 * kP * u + b) * kBlockSize) : 0;
        };
        // step start: bf16, every load of step u has landed (those of step
        // u + 1 may be out); fp8, this wave's conversion writes have.  Then
        // the barrier makes them everybody's.
        auto step_wait = [&]() __attribute__((always_inline)) {
            if constexpr (kFp8) __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            else wait_vmcnt<kStepLoads>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        };
        // fp8, end of step u: this wave's block of step u + 1 (its loads
        // went out in step u - 2; those of steps u + 2 and u + 3 may be out)
        auto step_convert = [&](int u, auto q_tag) __attribute__((always_inline)) {
            if constexpr (kFp8) {
                if (u + 1 < NU) {
                    wait_vmcnt<2 * kStepLoads>();
                    convert(q_tag, u + 1);
                }
            }
        };

        // prologue: the entries of steps 0 .. kAhead read together, the
        // loads of steps 0 .. kAhead - 1 (fp8: and the conversion of step
        // 0).  Later steps read the entries of step u + kAhead + 1 after
        // their last LDS read, so the scalar reads land during the next
        // barrier (see below).
        Pending pend;
        {
            Pending p0, p1, p2;
            fetch(p0, 0);
            fetch(p1, 1);
            if constexpr (kFp8) fetch(p2, 2);
            fetch(pend, kAhead);
            int pb[2 * kP];
            accept(p0, pb);
            __builtin_amdgcn_sched_barrier(0);
            dma_issue(std::integral_constant<int, 0>{}, dma_prepare(pb));
            __builtin_amdgcn_sched_barrier(0);
            accept(p1, pb);
            __builtin_amdgcn_sched_barrier(0);
            dma_issue(std::integral_constant<int, 1>{}, dma_prepare(pb));
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kFp8) {
                accept(p2, pb);
                __builtin_amdgcn_sched_barrier(0);
                dma_issue(std::integral_constant<int, 2>{}, dma_prepare(pb));
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<2 * kStepLoads>();
                convert(std::integral_constant<int, 0>{}, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (has_rows) {
            const int qmin = L - nq + R0 / G;  // first query position of the wave
            // QK operand of step c: key row n = token swap_bits23(n % 16) of
            // block n / 16, dims 16c + 8h .. +7 = chunk (2c + h, token) of the
            // block as the bf16 pool lays it out
            const int k_lane = (n >> 4) * WS::kBlockChunks + h * kBlockSize + swap_bits23(n & 15);

            // Step u (pairs 2u, 2u + 1).  kMasked: some block holds tokens
            // past the context end or past some row's position (the causal
            // diagonal), or lies outside the pool.
            auto step = [&](int u, auto masked_tag, auto q_tag) __attribute__((always_inline)) {
                constexpr bool kMasked = decltype(masked_tag)::value;
                constexpr int kQ = decltype(q_tag)::value;  // u mod 3
                // bf16: the ring slot of step u; fp8: operand slot u mod 2
                const uint4* const src = kFp8 ? cslot(u) : (kQ == 0 ? slot0 : kQ == 1 ? slot1 : slot2);
                step_wait();
                // the loads of step u + kAhead (into the ring slot step u - 1
                // used) go out under the QK products below
                __amdgpu_buffer_rsrc_t rs;
                {
                    int pb[2 * kP];
                    accept(pend, pb);
                    rs = dma_prepare(pb);
                }
                // No scalar read may be out during the operand reads: scalar
                // and LDS reads share one counter, and while a scalar read is
                // out (they may return out of order) every LDS wait is a wait
                // for all of them.  (The entries of the next loads are read
                // after this step's last LDS read.)
                __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
                __builtin_amdgcn_sched_barrier(0);

                // ---- QK: one chain of D/16 products per pair, interleaved
                dma_issue(std::integral_constant<int, (kQ + kAhead) % 3>{}, rs);
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
                    // block b's keys visible to this lane's row lie below
                    // min(end of its valid tokens, qpos + 1); the others'
                    // scores become -inf (unscaled: c > 0 keeps them -inf)
#pragma unroll
                    for (int b = 0; b < 2 * kP; ++b) {
                        const int kb = (2 * kP * u + b) * kBlockSize;  // the block's first key position
                        const int vis = min(kb + nv_of(u, b), qpos + 1) - kb - 8 * h;  // registers r < vis
#pragma unroll
                        for (int r = 0; r < 8; ++r)
                            x[b >> 1][8 * (b & 1) + r] = r < vis ? x[b >> 1][8 * (b & 1) + r] : -INFINITY;
                    }
                }
                float m16 = x[0][0];
#pragma unroll
                for (int a = 0; a < kP; ++a)
#pragma unroll
                    for (int r = (a == 0 ? 1 : 0); r < 16; ++r) m16 = fmaxf(m16, x[a][r]);
                // c > 0: scale the max only
                const float mx = max_halves(m16) * c_scale;
                const bool raise = mx > m_ref + kSlack;
                const float alpha = raise ? exp2_fast(m_ref - mx) : 1.f;  // m_ref = -inf -> 0
                m_ref = raise ? mx : m_ref;
                const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
                // weights, the PV products' B operands (pair a, block b):
                // bf16 against bf16 V; fp8, fp16 against V's codes as fp16
                // (11 significant bits; weights lie in [0, 2^8], and those
                // below 2^-24 flush to zero next to a largest one of at least 1)
                uint4 pw[kP][2];
                float lp = 0.f;
#pragma unroll
                for (int a = 0; a < kP; ++a) {
                    float pr[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        pr[r] = exp2_fast(fmaf(x[a][r], c_scale, -m_use));
                    lp += (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]))) +
                          (((pr[8] + pr[9]) + (pr[10] + pr[11])) + ((pr[12] + pr[13]) + (pr[14] + pr[15])));
                    auto pack = [](float lo, float hi) __attribute__((always_inline)) {
                        return kFp8 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
                    };
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        pw[a][b] = make_uint4(pack(pr[8 * b + 0], pr[8 * b + 1]), pack(pr[8 * b + 2], pr[8 * b + 3]),
                                              pack(pr[8 * b + 4], pr[8 * b + 5]), pack(pr[8 * b + 6], pr[8 * b + 7]));
                }
                // rarely taken (see kSlack): the output so far moves to the new reference
                if (__any(raise)) {
#pragma unroll
                    for (int t = 0; t < kDT; ++t) acc[t] *= alpha;
                }
                l_sum = fmaf(l_sum, alpha, lp);
                __builtin_amdgcn_sched_barrier(0);

                // ---- PV; tokens past a block's valid count (the context end,
                // a block outside the pool) are zeroed: they may hold NaN, and
                // 0 * NaN = NaN.  The causal diagonal needs no zeroing.
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
                            const int nvb = nv_of(u, 2 * a + b);
                            if (nvb < kBlockSize) {
                                const int nv = nvb - 8 * h;
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
                        }
#pragma unroll
                        for (int t = 0; t < kDT; ++t) {
                            if constexpr (kFp8)
                                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    __builtin_bit_cast(f16x8_t, vop[t]), __builtin_bit_cast(f16x8_t, pw[a][b]), acc[t], 0, 0, 0);
                            else
                                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    __builtin_bit_cast(bf16x8_t, vop[t]), __builtin_bit_cast(bf16x8_t, pw[a][b]), acc[t], 0, 0, 0);
                        }
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
                step_convert(u, std::integral_constant<int, (kQ + 1) % 3>{});
                __builtin_amdgcn_sched_barrier(0);
                fetch(pend, u + kAhead + 1);
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
            // no rows here: this wave's share of the loads (fp8: and of the
            // conversion), and the barriers
            for (int u = 0; u < NU; ++u) {
                step_wait();
                int pb[2 * kP];
                accept(pend, pb);
                const __amdgpu_buffer_rsrc_t rs = dma_prepare(pb);
                const int q = (u + kAhead) % 3;
                if (q == 0) dma_issue(std::integral_constant<int, 0>{}, rs);
                else if (q == 1) dma_issue(std::integral_constant<int, 1>{}, rs);
                else dma_issue(std::integral_constant<int, 2>{}, rs);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (kFp8) {
                    const int qc = (u + 1) % 3;
                    if (qc == 0) step_convert(u, std::integral_constant<int, 0>{});
                    else if (qc == 1) step_convert(u, std::integral_constant<int, 1>{});
                    else step_convert(u, std::integral_constant<int, 2>{});
                    __builtin_amdgcn_sched_barrier(0);
                }
                fetch(pend, u + kAhead + 1);
            }
        }
        wait_vmcnt<0>();  // no load into LDS outlives the workgroup
    }
    if (!has_rows) return;

    // ---- epilogue: out = O / l (fp8: times V's scale; zeros for rows that
    // see no key); lane (n, h), register 4q + e of tile t holds dim 32t + 8q
    // + 4h + e
    const float lt = sum_halves(l_sum);
    const float inv = lt > 0.f ? (kFp8 ? p.v_scale[kvh] : 1.f) / lt : 0.f;
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

size_t prefill_lds_bytes(int32_t num_seqs, int32_t lpt_buckets) {
    return (size_t)(num_seqs + 3 + lpt_buckets) * sizeof(int32_t);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    if (p.num_seqs == 0 || p.tile_bound == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.tile_bound * p.num_kv_heads));
    const size_t lds = prefill_lds_bytes(p.num_seqs, p.lpt_buckets);
    if (p.kv_fp8) {
        if (p.head_dim == 128) hipLaunchKernelGGL((prefill_wide_kernel<128, true>), grid, dim3(512), lds, stream, p);
        else hipLaunchKernelGGL((prefill_wide_kernel<64, true>), grid, dim3(512), lds, stream, p);
    } else {
        if (p.head_dim == 128) hipLaunchKernelGGL((prefill_wide_kernel<128, false>), grid, dim3(512), lds, stream, p);
        else hipLaunchKernelGGL((prefill_wide_kernel<64, false>), grid, dim3(512), lds, stream, p);
    }
    return hipGetLastError();
}

}  // namespace pkv
