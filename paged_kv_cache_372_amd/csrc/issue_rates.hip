// Instruction issue-rate microbenchmarks: the rates the chunked-prefill
// kernels are shaped around (prefill is the compute-heavy stage of serving,
// runbyai section 1).  Timing only: each kernel repeats one instruction
// pattern and keeps its result alive with a store that never happens.
//
// One workgroup per compute unit, 4 x waves_per_simd waves (one or two per
// SIMD).  Per iteration every wave issues 16 instructions of its pattern:
//   matrix products: mfma_f32_16x16x32_bf16 or mfma_f32_32x32x16_bf16, into
//     1 accumulator (one dependent chain) or 4 (four chains);
//   v_fma_f32 over 16 independent chains;
//   v_exp_f32, each followed by a v_add_f32 (16 chains);
//   16-byte LDS reads (ds_read_b128), consecutive lanes on consecutive
//     16 bytes of a 64 KiB array (no bank conflicts), one XOR each to keep
//     the value.
#include "kernels.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16v_t __attribute__((ext_vector_type(16)));

constexpr int kPerIter = 16;  // instructions of the pattern per wave and iteration

template <int kNacc>
__global__ __launch_bounds__(512) void rate_mfma16(uint32_t* sink, int iters) {
    static_assert(kPerIter % kNacc == 0, "whole rounds");
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(threadIdx.x * 1e-3f + i);
        b[i] = (__bf16)(i * 0.5f);
    }
    float4_t acc[kNacc];
#pragma unroll
    for (int j = 0; j < kNacc; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kPerIter / kNacc; ++r)
#pragma unroll
            for (int j = 0; j < kNacc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kNacc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (s == 1234.5f) sink[threadIdx.x] = __float_as_uint(s);
}

template <int kNacc>
__global__ __launch_bounds__(512) void rate_mfma32(uint32_t* sink, int iters) {
    static_assert(kPerIter % kNacc == 0, "whole rounds");
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(threadIdx.x * 1e-3f + i);
        b[i] = (__bf16)(i * 0.5f);
    }
    float16v_t acc[kNacc];
#pragma unroll
    for (int j = 0; j < kNacc; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kPerIter / kNacc; ++r)
#pragma unroll
            for (int j = 0; j < kNacc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kNacc; ++j) s += acc[j][0] + acc[j][5];
    if (s == 1234.5f) sink[threadIdx.x] = __float_as_uint(s);
}

__global__ __launch_bounds__(512) void rate_fma(uint32_t* sink, int iters) {
    float x[kPerIter];
#pragma unroll
    for (int k = 0; k < kPerIter; ++k) x[k] = 1e-3f * (threadIdx.x + k);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kPerIter; ++k) x[k] = fmaf(x[k], 0.999f, 1e-4f);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kPerIter; ++k) s += x[k];
    if (s == 1234.5f) sink[threadIdx.x] = __float_as_uint(s);
}

__global__ __launch_bounds__(512) void rate_exp(uint32_t* sink, int iters) {
    float x[kPerIter];
#pragma unroll
    for (int k = 0; k < kPerIter; ++k) x[k] = -1e-3f * (threadIdx.x + k);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kPerIter; ++k) x[k] = __builtin_amdgcn_exp2f(x[k]) - 1.f;
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kPerIter; ++k) s += x[k];
    if (s == 1234.5f) sink[threadIdx.x] = __float_as_uint(s);
}

__global__ __launch_bounds__(512) void rate_lds(uint32_t* sink, int iters) {
    __shared__ uint4 buf[4096];  // 64 KiB
    const int t = threadIdx.x;
    for (int i = t; i < 4096; i += blockDim.x) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
    __syncthreads();
    const int lane = t & 63, w = t >> 6;
    uint32_t a = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kPerIter; ++k) {
            const uint4 v = buf[((k + it + w) & 63) * 64 + lane];
            a ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (a == 0x12345u) sink[t] = a;
}

}  // namespace

hipError_t launch_issue_rate(int32_t pattern, int32_t waves_per_simd, int32_t iters, uint32_t* sink,
                             hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)cus), block((unsigned)(256 * waves_per_simd));
    switch (pattern) {
        case 0: hipLaunchKernelGGL(rate_mfma16<1>, grid, block, 0, stream, sink, iters); break;
        case 1: hipLaunchKernelGGL(rate_mfma16<4>, grid, block, 0, stream, sink, iters); break;
        case 2: hipLaunchKernelGGL(rate_mfma32<1>, grid, block, 0, stream, sink, iters); break;
        case 3: hipLaunchKernelGGL(rate_mfma32<4>, grid, block, 0, stream, sink, iters); break;
        case 4: hipLaunchKernelGGL(rate_fma, grid, block, 0, stream, sink, iters); break;
        case 5: hipLaunchKernelGGL(rate_exp, grid, block, 0, stream, sink, iters); break;
        default: hipLaunchKernelGGL(rate_lds, grid, block, 0, stream, sink, iters); break;
    }
    return hipGetLastError();
}

}  // namespace pkv
