// Per-token E4M3 quantisation of the activations, for the prefill gate/up
// GEMM on the FP8 MFMA (the "second precision": FP8 weights and FP8
// activations).  Source for the format: "Gated DeltaNet (+ FP8 MoE) -- AWS
// Neuron (NKI) kernels for Trainium2", section "FP8 MoE decode kernel": the
// official E4M3FN format with a scale of the block maximum over 448 (the
// weights' recipe); here one scale per token row of x.
//
// Row t:  s = amax_h |x[t][h]| / 448            (fp32, correctly rounded)
//         code[h] = E4M3FN_RNE(min(max(x / s, -448), 448))   (fp32 quotient)
// A row of zeros gets s = 0 and all-zero codes; a row holding a NaN or an
// infinity gets a NaN scale and zero codes.  The encoder is written from
// the format: below the smallest normal 2^-6 the step is 2^-9 (subnormals),
// above it 2^(E-3) with E the fp32 exponent; both round half to even, and a
// carry out of the 3-bit mantissa moves into the exponent field.
#include "common.hpp"
#include "plan.hpp"
#include "mxfp4_act.hpp"

namespace moe {

__device__ __forceinline__ uint32_t e4m3fn_encode_rne(float v) {
    v = fminf(fmaxf(v, -448.0f), 448.0f);
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);  // 0..8; 8 is the smallest normal (0x08)
    } else {
        const int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // -6..8
        const float m = ldexpf(a, -E);                                   // [1, 2), exact
        code = (uint32_t)((E + 7) << 3) + (uint32_t)rintf((m - 1.0f) * 8.0f);
    }
    return sign | code;
}

// One wave per token row, four rows per workgroup, no barrier.  Lane l takes
// the 8-element chunks l, l + 64, ...; rows of up to NCH * 512 elements stay
// in registers between the maximum and the encoding (NCH = 0: any width, the
// row is read twice, the second time from the cache).  H % 8 == 0.
template <int NCH>
__global__ __launch_bounds__(256) void quant_rows_e4m3_kernel(const uint16_t* __restrict__ x,
                                                              int T, int H,
                                                              uint8_t* __restrict__ xq,
                                                              float* __restrict__ xs) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole waves
    const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
    const int nc = H / 8;
    // the row maximum on |x| as bf16 bits: finite magnitudes order as
    // integers, and a NaN (above every other pattern) makes the maximum, and
    // so the row's scale, NaN instead of being dropped as fmaxf would
    auto chunk_max = [](const u32x4& v, uint32_t m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
        return m;
    };
    uint32_t amax = 0u;
    u32x4 v[NCH > 0 ? NCH : 1];
    if constexpr (NCH > 0) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = lane + 64 * j;
            v[j] = c < nc ? row[c] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j) amax = chunk_max(v[j], amax);
    } else {
        for (int c = lane; c < nc; c += 64) amax = chunk_max(row[c], amax);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, MOE_WAVE));
    // a row holding a NaN or an infinity: NaN scale (the quiet NaN 0x7FC00000)
    // and zero codes
    const float s = amax >= 0x7F80u ? __uint_as_float(0x7FC00000u) : __fdiv_rn(__uint_as_float(amax << 16), 448.0f);
    if (lane == 0) xs[t] = s;
    uint2* out = reinterpret_cast<uint2*>(xq + (size_t)t * H);
    auto encode_chunk = [&](const u32x4& c8) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t b = (c8[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            const uint32_t q = s > 0.0f ? e4m3fn_encode_rne(__fdiv_rn(__uint_as_float(b << 16), s)) : 0u;
            w[j >> 2] |= q << ((j & 3) * 8);
        }
        return uint2{w[0], w[1]};
    };
    if constexpr (NCH > 0) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = lane + 64 * j;
            if (c < nc) out[c] = encode_chunk(v[j]);
        }
    } else {
        for (int c = lane; c < nc; c += 64) out[c] = encode_chunk(row[c]);
    }
}

int launch_quant_rows_e4m3(const uint16_t* x, int T, int H, uint8_t* xq, float* xs,
                           hipStream_t stream) {
    if (H % 8) {
        set_error("activation quantisation needs H %% 8 == 0 (got %d)", H);
        return MOE_EUNSUPPORTED;
    }
    if (T == 0) return MOE_OK;
    const int nc = H / 8;
    const dim3 grid((T + 3) / 4), block(256);
    prof_begin("quant_rows_e4m3", stream);
    if (nc <= 64)
        quant_rows_e4m3_kernel<1><<<grid, block, 0, stream>>>(x, T, H, xq, xs);
    else if (nc <= 128)
        quant_rows_e4m3_kernel<2><<<grid, block, 0, stream>>>(x, T, H, xq, xs);
    else if (nc <= 256)
        quant_rows_e4m3_kernel<4><<<grid, block, 0, stream>>>(x, T, H, xq, xs);
    else if (nc <= 512)
        quant_rows_e4m3_kernel<8><<<grid, block, 0, stream>>>(x, T, H, xq, xs);
    else if (nc <= 1024)
        quant_rows_e4m3_kernel<16><<<grid, block, 0, stream>>>(x, T, H, xq, xs);
    else
        quant_rows_e4m3_kernel<0><<<grid, block, 0, stream>>>(x, T, H, xq, xs);
    prof_end(stream);
    return check_launch("quant_rows_e4m3_kernel");
}

// MXFP4 quantisation of activation rows for the E2M1 x E2M1 gate/up GEMM
// ("Add gfx950 Q256 fused MXFP4 prefill pipeline": its producer quantises the
// activations to MXFP4; the rule is the OCP Microscaling one).  Four lanes
// per run of 32 elements of a row, 8 elements (16 bytes) a lane, so that a
// wave reads 1 KB and writes 256 code bytes contiguously:
//   X = floor(log2 max|x|) - 2, clamped to [-127, 127]: with e the bf16
//       exponent field of the run's largest magnitude (the maximum of |x| as
//       bf16 bits, shared over the lane quad), X = max(e - 129, -127) (an
//       all-zero or subnormal run clamps to -127); scale byte X + 127;
//   v = |x| * 2^-X, exact in fp32 (a power-of-two scaling of a bf16 value,
//       at least 2^-6 and below 8);
//   code = the number of E2M1 midpoints below v, a tie going to the even
//       code (0.25, 1.25, 2.5 and 5 round down; 0.75, 1.75 and 3.5 up), 7
//       for everything above 5 (saturation at 6), plus the sign bit of x.
// A run holding a NaN or an infinity (exponent field all ones) gets the E8M0
// NaN byte 255 and zero codes.  Element 2j of a run goes to the low nibble of
// its byte j.
__global__ __launch_bounds__(256) void quant_rows_mxfp4_kernel(const uint16_t* __restrict__ x, long nruns,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;  // 8-element group
    const long run = g >> 2;
    // (whole quads: nruns * 4 threads are rounded up to whole waves, and a
    //  quad past the end only takes part in the shuffles)
    const bool live = run < nruns;
    const u32x4 v = live ? reinterpret_cast<const u32x4*>(x)[g] : u32x4{0u, 0u, 0u, 0u};
    uint32_t m = bf16x8_absmax_bits(v);
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, MOE_WAVE));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, MOE_WAVE));
    if (!live) return;
    const bool bad = m >= 0x7F80u;
    const int X = mxfp4_run_exponent(m);
    const uint32_t word = mxfp4_encode8(v, X);
    reinterpret_cast<uint32_t*>(codes)[g] = bad ? 0u : word;
    if ((g & 3) == 0) scales[run] = bad ? (uint8_t)255 : (uint8_t)(X + 127);
}

int launch_quant_rows_mxfp4(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
    if (H % 32) {
        set_error("MXFP4 activation quantisation needs H %% 32 == 0 (got %d)", H);
        return MOE_EUNSUPPORTED;
    }
    if (T == 0) return MOE_OK;
    const long nruns = (long)T * (H / 32);
    prof_begin("quant_rows_mxfp4", stream);
    quant_rows_mxfp4_kernel<<<(unsigned)((4 * nruns + 255) / 256), 256, 0, stream>>>(x, nruns, codes, scales);
    prof_end(stream);
    return check_launch("quant_rows_mxfp4_kernel");
}

}  // namespace moe
