// Split-K merge of partial results into the decode output.
//
// A piece p of a sequence's context left, per query head, its reference max
// m_p (log2 units), its sum l_p = sum 2^(s_i - m_p) and its unnormalised
// output o_p = sum 2^(s_i - m_p) v_i.  Softmax over the whole context is then
//     out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// an identity of the exponential (nothing here is an approximation beyond
// fp32 rounding).  Pieces with no valid token (m = -inf, l = 0) weigh 0.
// Merging two partial states (M1, l1, o1) and (M2, l2, o2) is the same
// identity: weights 2^(Mi - max(M1, M2)).  All sums run in a fixed order, so
// the result does not depend on scheduling.
//
// Two kernels, picked by the launch from a bound on the pieces per row
// (a row = one sequence and query head):
//   rows kernel (few pieces per row on average): a 256-thread workgroup
//     takes four rows, one per wave.  A wave's D/4-lane slots load its
//     row's pieces in rounds of 4 per slot (8 pieces a round at D = 128, 16
//     at D = 64), each slot merging its share with a running maximum, then
//     the slots merge across lanes.  A row with more than two rounds of
//     pieces is left to the whole workgroup afterwards.
//     Many rows in flight per compute unit: the merge is two dependent
//     memory round trips (where the pieces are, then the pieces), so at a
//     few pieces per row its time is the number of occupancy rounds.
//   wide kernel (many pieces per row, as at long context): one workgroup per
//     row; its 256 / (D / 4) slots each merge every SLOTS-th piece, then slot
//     0 merges the slots through LDS.
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
constexpr int kWaveLoads = 4;                      // pieces per slot one wave loads at once
constexpr int kWaveRounds = 2;                     // longer rows: the whole workgroup
constexpr int kRowsAvgPieces = 16;                 // rows kernel up to this many pieces per row on average

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

// A running merge state: reference max, sum and unnormalised output (the
// lane's four dims of it).
struct MergeState {
    float M = -INFINITY, den = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);

    __device__ __forceinline__ void add(float m, float l, float4 v) {
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
    __device__ __forceinline__ float4 normalised() const {
        const float inv = den > 0.f ? 1.f / den : 0.f;
        return make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    }
};

// The pieces of one row: n of them, piece i at partial row row0 + i * stride
// except (balanced) the first, at first_row.  n = 0: nothing to do here (the
// decode wrote the row); zero: the row is all zeros (empty context).
struct RowPieces {
    int n = 0;
    bool zero = false;
    int64_t row0 = 0, stride = 0, first_row = 0;

    __device__ __forceinline__ int64_t row_of(int i) const { return i == 0 ? first_row : row0 + (int64_t)i * stride; }
};

template <bool kBalanced>
__device__ __forceinline__ RowPieces locate_pieces(const DecodeParams& p, int s, int h) {
    const int Hq = p.num_q_heads;
    RowPieces rp;
    if (kBalanced) {
        // the three offsets are read together, before anything depends on
        // one of them: one memory round trip
        const int o0 = p.seq_off[s];
        const int o1 = p.seq_off[s + 1];
        int cs, nr;
        range_geometry(p.seq_off[p.num_seqs], p.walkers, p.range_cap, cs, nr);
        if (o1 <= o0) {
            rp.zero = true;
            return rp;
        }
        const int r0 = o0 / cs;
        const int r1 = (o1 - 1) / cs;
        if (r0 == r1) return rp;
        rp.n = r1 - r0 + 1;
        // ranges after the first hold the sequence from their start: slot 0
        rp.row0 = (int64_t)range_slot(r0 + 1, cs, o0) * Hq + h - 2 * Hq;
        rp.stride = 2 * Hq;
        rp.first_row = (int64_t)range_slot(r0, cs, o0) * Hq + h;
    } else {
        const int L = clamp_ctx(p.context_lens[s], p.ctx_cap);
        const int n_blk = (L + kBlockSize - 1) / kBlockSize;
        int n = (n_blk + p.part_blocks - 1) / p.part_blocks;
        if (n > p.num_parts) n = p.num_parts;
        if (n <= 1) return rp;
        rp.n = n;
        rp.row0 = (int64_t)s * p.num_parts * Hq + h;
        rp.stride = Hq;
        rp.first_row = rp.row0;
    }
    return rp;
}

template <int D>
struct WideLds {
    static constexpr int LPR = D / 4;
    static constexpr int SLOTS = kThreads / LPR;
    float4 acc[SLOTS][LPR];
    float m[SLOTS], l[SLOTS];
};

// One row merged by the whole workgroup (every thread calls it; rp is the
// same in all of them).  Slot k takes pieces k, k + SLOTS, ... in order with
// a running maximum: the loads of a piece need nothing from the previous
// one, so they are all in flight at once.  Slot 0 then merges the slots in
// order and writes the row.  Ends with the slots' LDS still being read by
// slot 0: a caller that reuses `lds` puts a barrier first.
template <int D>
__device__ __forceinline__ void merge_wide(const DecodeParams& p, const RowPieces& rp, int64_t out_row,
                                           WideLds<D>& lds) {
    constexpr int LPR = WideLds<D>::LPR;
    constexpr int SLOTS = WideLds<D>::SLOTS;
    const int tid = threadIdx.x;
    const int slot = tid / LPR;
    const int c4 = tid % LPR;
    MergeState st;
#pragma unroll 4
    for (int i = slot; i < rp.n; i += SLOTS) {
        const int64_t r = rp.row_of(i);
        st.add(p.m_part[r], p.l_part[r], reinterpret_cast<const float4*>(p.o_part + r * D)[c4]);
    }
    lds.acc[slot][c4] = st.a;
    if (c4 == 0) {
        lds.m[slot] = st.M;
        lds.l[slot] = st.den;
    }
    __syncthreads();
    if (slot != 0) return;
    float Mt = lds.m[0];
    for (int k = 1; k < SLOTS; ++k) Mt = fmaxf(Mt, lds.m[k]);
    float den = 0.f;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < SLOTS; ++k) {
        const float w = piece_weight(lds.m[k], Mt);
        const float4 v = lds.acc[k][c4];
        den = fmaf(w, lds.l[k], den);
        sum.x = fmaf(w, v.x, sum.x);
        sum.y = fmaf(w, v.y, sum.y);
        sum.z = fmaf(w, v.z, sum.z);
        sum.w = fmaf(w, v.w, sum.w);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    write_row<D>(p, out_row, c4, make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv));
}

// One workgroup per row.
template <int D, bool kBalanced>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(DecodeParams p) {
    __shared__ WideLds<D> lds;
    const int Hq = p.num_q_heads;
    const int s = blockIdx.x / Hq;
    const int h = blockIdx.x % Hq;
    const int64_t out_row = (int64_t)s * Hq + h;
    const RowPieces rp = locate_pieces<kBalanced>(p, s, h);
    if (rp.zero) {
        if (threadIdx.x < D / 4) write_row<D>(p, out_row, threadIdx.x, make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    if (rp.n <= 1) return;
    merge_wide<D>(p, rp, out_row, lds);
}

// One wave per row, four rows per workgroup; rows of more than kWaveRounds
// rounds of pieces are merged by the whole workgroup afterwards.
template <int D, bool kBalanced>
__global__ __launch_bounds__(kThreads) void splitk_reduce_rows_kernel(DecodeParams p) {
    constexpr int LPR = D / 4;         // lanes per row (float4 each)
    constexpr int SL = 64 / LPR;       // slots per wave
    constexpr int U = kWaveLoads;      // pieces per slot per round
    constexpr int kRound = SL * U;     // pieces per round: 8 (D = 128) or 16 (D = 64)
    __shared__ WideLds<D> lds;
    __shared__ int wide_row[kThreads / 64];

    const int Hq = p.num_q_heads;
    // the wave's row is the same in all its lanes: say so, so that where its
    // pieces are is read through the scalar cache
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int slot = lane / LPR;
    const int c4 = lane % LPR;
    // rows fit in 32 bits: each has a D-element row of q and of out
    const uint32_t rows = (uint32_t)p.num_seqs * (uint32_t)Hq;
    const uint32_t row = blockIdx.x * (kThreads / 64) + wave;

    bool wide = false;
    if (row < rows) {
        const int s = (int)(row / (uint32_t)Hq);
        const int h = (int)(row - (uint32_t)s * Hq);
        const RowPieces rp = locate_pieces<kBalanced>(p, s, h);
        if (rp.zero) {
            if (slot == 0) write_row<D>(p, row, c4, make_float4(0.f, 0.f, 0.f, 0.f));
        } else if (rp.n > kWaveRounds * kRound) {
            wide = true;
        } else if (rp.n > 1) {
            // rounds of kRound pieces, all loads of a round issued
            // together; indexes past the row read its last piece again and
            // weigh 0
            MergeState st;
            for (int base = 0; base < rp.n; base += kRound) {
                float m[U], l[U];
                float4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = base + u * SL + slot;
                    const int64_t r = rp.row_of(i < rp.n ? i : rp.n - 1);
                    m[u] = p.m_part[r];
                    l[u] = p.l_part[r];
                    v[u] = reinterpret_cast<const float4*>(p.o_part + r * D)[c4];
                    if (i >= rp.n) m[u] = -INFINITY;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) st.add(m[u], l[u], v[u]);
            }
            // slots merge across lanes: lane groups LPR apart, then 2 LPR
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) {
                const float m_o = __shfl_xor(st.M, off);
                const float l_o = __shfl_xor(st.den, off);
                float4 v_o;
                v_o.x = __shfl_xor(st.a.x, off);
                v_o.y = __shfl_xor(st.a.y, off);
                v_o.z = __shfl_xor(st.a.z, off);
                v_o.w = __shfl_xor(st.a.w, off);
                st.add(m_o, l_o, v_o);
            }
            if (slot == 0) write_row<D>(p, row, c4, st.normalised());
        }
    }
    if (lane == 0) wide_row[wave] = wide;
    __syncthreads();
#pragma unroll 1
    for (int w = 0; w < kThreads / 64; ++w) {
        if (!wide_row[w]) continue;  // the same in every thread
        const uint32_t r = blockIdx.x * (kThreads / 64) + w;
        const int s = (int)(r / (uint32_t)Hq);
        const int h = (int)(r - (uint32_t)s * Hq);
        merge_wide<D>(p, locate_pieces<kBalanced>(p, s, h), r, lds);
        __syncthreads();  // slot 0 has read lds before the next row writes it
    }
}

// Average pieces per row, at most, of a launch: the partitioned path has at
// most num_parts; in the balanced path the sequences' pieces number at most
// (ranges - 1) + num_seqs, and ranges <= max(walkers, blocks / range_cap).
bool few_pieces(const DecodeParams& p, bool balanced) {
    if (!balanced) return p.num_parts <= kRowsAvgPieces;
    const int64_t t_max = (int64_t)p.num_seqs * ((p.ctx_cap + kBlockSize - 1) / kBlockSize);
    int64_t nr = p.walkers;
    if (p.range_cap > 0 && (t_max + p.range_cap - 1) / p.range_cap > nr) nr = (t_max + p.range_cap - 1) / p.range_cap;
    return nr <= (int64_t)kRowsAvgPieces * p.num_seqs;
}

template <bool kBalanced>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads;
    const dim3 block(kThreads);
    if (few_pieces(p, kBalanced)) {
        const dim3 grid((unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64)));
        if (p.head_dim == 128)
            hipLaunchKernelGGL((splitk_reduce_rows_kernel<128, kBalanced>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((splitk_reduce_rows_kernel<64, kBalanced>), grid, block, 0, stream, p);
    } else {
        const dim3 grid((unsigned)rows);
        if (p.head_dim == 128) hipLaunchKernelGGL((splitk_reduce_kernel<128, kBalanced>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((splitk_reduce_kernel<64, kBalanced>), grid, block, 0, stream, p);
    }
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
