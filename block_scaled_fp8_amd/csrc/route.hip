// Router: softmax over E experts -> top-k -> renormalised affinities.
//
// Source: "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for
// Trainium2", section "FP8 MoE decode kernel (moe_fused_w8_35b)", Serving
// contract: the router is softmax -> top-8 -> norm.
//
// One wave64 per token; lane l holds experts l, l+64, ... (NPL per lane).
// Selection runs k wave-wide arg-max passes over 64-bit keys
//     key = (order-preserving bits of the fp32 logit) << 32 | ~expert
// so a larger logit wins and, between equal logits, the lower expert index
// wins.  -0.0 is canonicalised to +0.0 first (they tie); NaN maps to the
// lowest key.  Softmax is strictly increasing, so choosing on logits picks
// the same experts as choosing on probabilities, without exp() rounding
// ever reordering them.  The renormalised affinity of slot j is
//     p_j / sum_sel p = exp(l_j - M) / sum_sel exp(l - M),
// since the full-softmax denominator cancels (M = the largest logit).
#include "common.hpp"
#include "plan.hpp"

namespace moe {

__device__ __forceinline__ uint64_t route_key(float v, int e) {
    uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
    uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    if (v != v) o = 0u;
    return ((uint64_t)o << 32) | (uint64_t)(~(uint32_t)e);
}

__device__ __forceinline__ float key_logit(uint64_t key) {
    uint32_t o = (uint32_t)(key >> 32);
    uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(b);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, o, MOE_WAVE);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, MOE_WAVE);
        uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w > v ? w : v;
    }
    return v;
}

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_softmax_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ aff, int32_t* __restrict__ status) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;

    uint64_t key[NPL];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + MOE_WAVE * i;
        if (e < E) {
            const float v = row[e];
            bad |= !__builtin_isfinite(v);
            key[i] = route_key(v, e);
        } else {
            key[i] = 0ull;  // padding: below every real key
        }
    }
    if (status && __ballot(bad) != 0ull && lane == 0) atomicOr(status, MOE_STATUS_NONFINITE_LOGIT);

    float my_logit = 0.0f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (key[i] == best) key[i] = 0ull;  // keys are unique (index in low bits)
        if (lane == j) {
            my_id = (int)(~(uint32_t)best);
            my_logit = key_logit(best);
        }
    }
    const float M = __shfl(my_logit, 0, MOE_WAVE);
    const float w = lane < k ? expf(my_logit - M) : 0.0f;
    const float s = wave_sum_f32(w);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        aff[(size_t)t * k + lane] = w / s;
    }
}

int launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* aff,
                 int32_t* status, hipStream_t stream) {
    const int npl = (E + MOE_WAVE - 1) / MOE_WAVE;
    const dim3 grid((T + 3) / 4), block(256);
    prof_begin("route_topk_softmax", stream);
    if (npl <= 1)
        route_topk_softmax_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, ids, aff, status);
    else if (npl <= 2)
        route_topk_softmax_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, ids, aff, status);
    else if (npl <= 4)
        route_topk_softmax_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, ids, aff, status);
    else if (npl <= 8)
        route_topk_softmax_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, ids, aff, status);
    else
        route_topk_softmax_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, ids, aff, status);
    prof_end(stream);
    return check_launch("route_topk_softmax_kernel");
}

}  // namespace moe
