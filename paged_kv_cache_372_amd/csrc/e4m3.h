// The E4M3 encoding of fp8 KV pools, shared by the quantising cache write
// and the decode launch that appends the new tokens itself: both must store
// the same code for the same value and scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// fp32 -> OCP E4M3 code: round to nearest (ties to even mantissa), saturate
// at +-448; the sign of zero is kept.  Written out from the format (1 sign,
// 4 exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9) with
// integer operations, so the result is fixed bit for bit.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.f);
    if (a < 0.015625f)                                   // below 2^-6: multiples of 2^-9
        return sign | (uint32_t)__builtin_rintf(a * 512.f);  // exact scaling, rint rounds to even
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = (ab >> 20) & 7u;                  // top 3 mantissa bits
    const uint32_t rem = ab & 0xFFFFFu;                  // the 20 dropped bits
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ? 1u : 0u;
    const uint32_t code = ((((ab >> 23) - 120u) << 3) | r) + up;  // exponent bias 127 -> 7; a carry bumps it
    return sign | (code < 0x7Eu ? code : 0x7Eu);
}

// The code the pools hold for value x (bf16 or fp32 bits widened to fp32)
// of a KV head with dequantisation scale `scale`: E4M3(fp32(x / scale)),
// with the correctly rounded fp32 division.
__device__ __forceinline__ uint32_t e4m3_encode(float x, float scale) { return e4m3_rne_sat(x / scale); }

}  // namespace pkv
