// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_w8a16.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MOE_WAVE 64

namespace moe {

// ---------------------------------------------------------------- FP8 decode
// Two E4M3FN bytes (byte 0/1 of `w` when hi == false, 2/3 when true) to two
// bf16 values with the gfx950 scaled converter at scale 1.0.  Every finite
// E4M3FN value (4 significant bits, |v| in [2^-9, 448]) is a bf16 value, so
// this is exact.
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

// 8 FP8 bytes (two dwords, little-endian byte order) -> 8 bf16, element i = byte i.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// The same conversion times 2^e, where e is the exponent of `pow2` (the
// converter uses only the exponent field of its scale operand, an E8M0
// scale: 0.0f means 2^-127).  Exact while every product is a normal bf16
// value (e >= -117); smaller results are flushed to zero.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8_scaled(uint32_t lo, uint32_t hi, float pow2) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, pow2, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, pow2, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, pow2, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, pow2, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// Eight E2M1 (FP4) codes (one dword: element 2b in the low nibble of byte b,
// 2b + 1 in its high nibble) to eight bf16 times 2^e, e the exponent of
// `pow2` (an E8M0 scale given as fp32: only the exponent field is used).
// Every E2M1 value times 2^e is a bf16 value while it stays in the normal
// range, so this is exact there.  Each conversion's two results are read as
// one 32-bit word: reading the second bf16 element of this builtin's result
// on its own was measured to return the first one.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8_scaled(uint32_t w, float pow2) {
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 3));
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------- weight layouts
// A weight matrix [rows, K] of FP8 bytes (rows % 16 == 0, K % 64 == 0) is
// consumed in 16-row tiles and 64-wide K chunks; lane l of a wave takes the 16
// bytes of row 16*t + l%16, columns 64*c + 16*(l/16) .. +15.
//  - row-major: those 16 bytes sit at row * K + column;
//  - tiled:     tile t, chunk c is one contiguous kilobyte, lane l at byte 16*l,
//               so a wave's load of one chunk is a single 1 KB burst.
enum { LAYOUT_ROWMAJOR = MOE_LAYOUT_ROWMAJOR, LAYOUT_TILED = MOE_LAYOUT_TILED };

template <int LAYOUT>
__device__ __forceinline__ const uint8_t* tile_lane_ptr(const uint8_t* W, int row0, int K, int lane) {
    if (LAYOUT == LAYOUT_TILED) return W + (size_t)(row0 >> 4) * 16 * K + lane * 16;
    return W + (size_t)(row0 + (lane & 15)) * K + (lane >> 4) * 16;
}

template <int LAYOUT>
__device__ __forceinline__ constexpr int chunk_stride() { return LAYOUT == LAYOUT_TILED ? 1024 : 64; }

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    // a NaN stays a (quiet) NaN: rounding its payload could carry into the
    // exponent or the sign
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? (uint16_t)((u >> 16) | 0x0040u) : (uint16_t)(r >> 16);
}

// ---------------------------------------------------------------- SwiGLU
// silu(g) * u with silu(g) = g / (1 + exp(-g)).
// Prefill contributions leave the down GEMM in a block floating-point form:
// each run of 8 consecutive values of a row shares one exponent byte ex (the
// fp32 exponent field of the run's largest magnitude) and each value keeps a
// 16-bit signed mantissa m = rint(v * 2^(141 - ex)) saturated to |m| <= 32767,
// so that v = m * 2^(ex - 141) to within 2^-15 of the run's largest magnitude
// (2^-14 where the rounding saturates).  A row of H values is a mantissa
// plane (2*H bytes) then an exponent plane (H/8 bytes).  Non-finite values
// stay non-finite: the unused mantissa -32768 marks a NaN, and an infinity
// sets the run's exponent to 255, whose saturated mantissa decodes to inf.
__device__ __forceinline__ void bfp16x8_encode(f32x4 a, f32x4 b, u32x4& mant, uint32_t& ex) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(a[j]), fabsf(b[j])));
    ex = (__float_as_uint(amax) >> 23) & 0xFFu;
    const int sh = 141 - (int)ex;
    uint32_t m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float v = j < 4 ? a[j] : b[j - 4];
        const float q = fminf(fmaxf(rintf(ldexpf(v, sh)), -32767.0f), 32767.0f);
        m[j] = v != v ? 0x8000u : (uint32_t)(int32_t)q & 0xFFFFu;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) mant[j] = m[2 * j] | (m[2 * j + 1] << 16);
}
// The same form for the values ldexp(a_j * sm, se) (an accumulator run, its
// fp32 unit mantissa sm and power of two se), in about four VALU operations a
// value.  Let f be the exponent field of fl(max |a_j| * sm): the run's
// exponent byte is then f + se, and its mantissas rint(a_j * sm * 2^(141 - f))
// depend on a and sm only.  One FMA forms a_j * c + 1.5 * 2^23 with
// c = sm * 2^(141 - f): |a_j * c| < 2^15, so the sum is rounded to the nearest
// integer n (ties to even) in the binade [2^23, 2^24), whose low 16 bits are
// n as a 16-bit two's complement; a clamp at 1.5 * 2^23 +- 32767 saturates n.
// (One rounding of the exact product, where bfp16x8_encode of the separately
// rounded a_j * sm may differ by one unit on a near-tie.)  Runs this cannot
// hold exactly -- a non-finite or zero largest magnitude, f < 14 (c not a
// normal float) or an exponent byte outside 1..254 -- take bfp16x8_encode of
// ldexp(a_j * sm, se).
// The common case alone, with no branch: returns whether it holds the run
// exactly (when it does not, mant and ex are meaningless and the run must be
// encoded by bfp16x8_encode_scaled).
__device__ __forceinline__ bool bfp16x8_encode_scaled_fast(f32x4 a, f32x4 b, float sm, int se,
                                                           u32x4& mant, uint32_t& ex) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        mx = max(mx, max(__float_as_uint(a[j]) & 0x7FFFFFFFu, __float_as_uint(b[j]) & 0x7FFFFFFFu));
    const int f = (int)((__float_as_uint(__uint_as_float(mx) * sm) >> 23) & 0xFFu);
    const int e = f + se;
    constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
    const float c = sm * __uint_as_float((uint32_t)(268 - f) << 23);  // sm * 2^(141 - f)
    uint32_t m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float y = __builtin_fmaf(j < 4 ? a[j] : b[j - 4], c, MAGIC);
        m[j] = __float_as_uint(__builtin_amdgcn_fmed3f(y, MAGIC - 32767.0f, MAGIC + 32767.0f));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) mant[j] = __builtin_amdgcn_perm(m[2 * j + 1], m[2 * j], 0x05040100u);
    ex = (uint32_t)e;
    return (mx < 0x7F800000u) & (f >= 14) & (f <= 254) & (e >= 1) & (e <= 254);
}
__device__ __forceinline__ void bfp16x8_encode_scaled(f32x4 a, f32x4 b, float sm, int se, u32x4& mant,
                                                      uint32_t& ex) {
    if (!bfp16x8_encode_scaled_fast(a, b, sm, se, mant, ex)) {
        f32x4 va, vb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            va[j] = ldexpf(a[j] * sm, se);
            vb[j] = ldexpf(b[j] * sm, se);
        }
        bfp16x8_encode(va, vb, mant, ex);
    }
}
// value j of a run: the sign-extended 16-bit mantissa times 2^(ex - 141)
__device__ __forceinline__ float bfp16_value(u32x4 mant, uint32_t ex, int j) {
    const int m = (int)(int16_t)((mant[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    return m == -32768 ? __builtin_nanf("") : ldexpf((float)m, (int)ex - 141);
}

__device__ __forceinline__ float swiglu(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

// relu(u)^2, the activation of non-gated (relu-squared) experts.
__device__ __forceinline__ float relu2(float u) {
    const float r = fmaxf(u, 0.0f);
    return r * r;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & (MOE_WAVE - 1); }

// Wave index inside the workgroup, marked wave-uniform so that values derived
// from it (tile rows, scale addresses) live in SGPRs and scale reads become
// scalar loads that never wait on the vector-memory counter.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
}

// 16-byte load of data the call reads exactly once (decode weight streams):
// non-temporal, so the stream does not evict lines that other loads reuse
// from L2 and the last-level cache.  Measured on the decode workload: the
// fused expert kernel 125.8 -> 114.7 us, the router after it 7.7 -> 6.4 us.
__device__ __forceinline__ u32x4 load_stream16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

// Inclusive scan over the wave (lane order).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
        int n = __shfl_up(v, o, MOE_WAVE);
        if (l >= o) v += n;
    }
    return v;
}

__device__ __forceinline__ size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe

// Host-side helpers (defined in api.hip).
namespace moe {
void set_error(const char* fmt, ...);
int check_launch(const char* what);
inline size_t halign(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }
}  // namespace moe
