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
// byte j), by gfx950's scaled conversion: each pair of bf16 values divided by
// the fp32 2^X (X = -127: the subnormal 2^-127) and rounded to the nearest
// E2M1 value, a tie to the even code, saturating at 6 and keeping the sign.
// Checked on the GPU over every bf16 pattern whose quotient is below 8 (all a
// run's elements: its largest lands in [4, 8)) at X = -127, -126, -10, -1,
// 0, 1, 10, 125 and 127: identical to counting the E2M1 midpoints below
// |x| / 2^X (1/4, 5/4, 5/2 and 5 round down, 3/4, 7/4 and 7/2 up).
__device__ __forceinline__ uint32_t mxfp4_encode8(u32x4 v, int X) {
    const float sc = __uint_as_float(X >= -126 ? (uint32_t)(X + 127) << 23 : 0x00400000u);
    // (each word through a scalar first: a bit cast of an ext-vector
    //  element has compiled to element 0)
    const uint32_t p0 = v[0], p1 = v[1], p2 = v[2], p3 = v[3];
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p0), sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p1), sc, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p2), sc, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p3), sc, 3);
    return w;
}

}  // namespace moe
