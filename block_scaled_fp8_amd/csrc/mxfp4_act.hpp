// MXFP4 quantisation of bf16 activations (OCP microscaling rule): each run of
// 32 consecutive elements shares the E8M0 exponent X = floor(log2 amax) - 2,
// clamped to [-127, 127] (an all-zero run takes -127), so the run's largest
// magnitude lands in [4, 8); each element becomes the nearest E2M1 value of
// |x| / 2^X (a tie to the even code, saturating at 6) with the sign bit of x.
// A run holding a NaN or an infinity takes the E8M0 NaN byte 255 and zero
// codes.  Sources: "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter
// PR #5988), description (activations quantised to MXFP4 on the fly); the
// weights' MXFP4 format, "NKI Library Supported Kernel Reference", Quantize
// MXFP8 / Blockwise MM Block MX (E8M0 scale per 32 elements).
#pragma once

#include "common.hpp"

namespace moe {

// The largest magnitude of 8 bf16 values (raw bits, two a word) as bf16
// magnitude bits: finite values order as integers, and NaN or infinity give
// a value >= 0x7F80.
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(u32x4 v) {
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = max(m, max(v[w] & 0x7FFFu, (v[w] >> 16) & 0x7FFFu));
    return m;
}

// The run exponent X from the run's largest magnitude bits (finite): the
// bf16 exponent field less 129, at least -127 (a zero or subnormal largest
// value gives -127).
__device__ __forceinline__ int mxfp4_run_exponent(uint32_t amax_bits) {
    return max((int)(amax_bits >> 7) - 129, -127);
}

// E2M1 codes of 8 bf16 values at the run exponent X, element e in bits
// 4e .. 4e+3 (the byte order of packed MXFP4: element 2j in the low nibble of
// byte j).  |x| * 2^-X is exact in fp32 (bf16 significands, a power-of-two
// factor within range), and the code counts the E2M1 midpoints below it: at
// a midpoint the even code wins, so 1/4, 5/4, 5/2 and 5 round down and 3/4,
// 7/4 and 7/2 up.
__device__ __forceinline__ uint32_t mxfp4_encode8(u32x4 v, int X) {
    const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, 127 - X in [2, 254]
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t b = (v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
        const float a = __uint_as_float((b & 0x7FFFu) << 16) * inv;
        const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                           (uint32_t)(a > 5.0f);
        word |= (c | ((b >> 12) & 8u)) << (4 * e);
    }
    return word;
}

}  // namespace moe
