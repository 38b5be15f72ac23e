// Router: softmax over E experts -> top-k -> renormalised affinities.
//
// Source: "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for
// Trainium2", section "FP8 MoE decode kernel (moe_fused_w8_35b)", Serving
// contract: the router is softmax -> top-8 -> norm.
//
// One wave64 per token; lane l holds experts l, l+64, ... (NPL per lane).
// Selection runs k wave-wide arg-max passes: a larger logit wins and, between
// equal logits, the lower expert index wins.  -0.0 is canonicalised to +0.0
// first (they tie); NaN ranks below every other value.  Softmax is strictly increasing, so choosing on logits picks
// the same experts as choosing on probabilities, without exp() rounding
// ever reordering them.  The renormalised affinity of slot j is
//     p_j / sum_sel p = exp(l_j - M) / sum_sel exp(l - M),
// since the full-softmax denominator cancels (M = the largest logit).
#include "common.hpp"
#include "plan.hpp"

namespace moe {

// Order-preserving unsigned image of a float: larger float -> larger value;
// -0.0 maps like +0.0 and NaN to 0 (below -inf).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    const uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return v != v ? 0u : o;
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// DPP controls (gfx9): quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_ror:4, row_ror:8.
#define MOE_DPP_QP_1032 0xB1
#define MOE_DPP_QP_2301 0x4E
#define MOE_DPP_ROR4 0x124
#define MOE_DPP_ROR8 0x128

template <bool MAX>
__device__ __forceinline__ uint32_t dpp_red(uint32_t v, int ctrl) {
    uint32_t o = 0;
    switch (ctrl) {  // the control must be a literal
        case MOE_DPP_QP_1032: o = __builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_QP_1032, 0xF, 0xF, false); break;
        case MOE_DPP_QP_2301: o = __builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_QP_2301, 0xF, 0xF, false); break;
        case MOE_DPP_ROR4: o = __builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_ROR4, 0xF, 0xF, false); break;
        default: o = __builtin_amdgcn_update_dpp(0, (int)v, MOE_DPP_ROR8, 0xF, 0xF, false); break;
    }
    return MAX ? (o > v ? o : v) : (o < v ? o : v);
}

// Wave-wide maximum (MAX) or minimum, returned as a wave-uniform value: a
// butterfly inside each 16-lane row (DPP), then the four row results read as
// scalars.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_red_u32(uint32_t v) {
    v = dpp_red<MAX>(v, MOE_DPP_QP_1032);
    v = dpp_red<MAX>(v, MOE_DPP_QP_2301);
    v = dpp_red<MAX>(v, MOE_DPP_ROR4);
    v = dpp_red<MAX>(v, MOE_DPP_ROR8);
    const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = __builtin_amdgcn_readlane((int)v, 48);
    if (MAX) {
        const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
        return a > b ? a : b;
    }
    const uint32_t a = r0 < r1 ? r0 : r1, b = r2 < r3 ? r2 : r3;
    return a < b ? a : b;
}

// Selection.  Each lane first orders its own NPL entries (slot i holds expert
// 64*i + lane) by key, larger first and lower slot first among equal keys, so
// its head is its best remaining candidate.  Each of the k passes then takes
// the wave-wide maximum of the lane heads; when one lane holds it, that
// lane's head is the choice, and when several lanes tie, the lowest expert
// index among their heads (a wave minimum).  Either way the chosen entry is
// the largest key with the lowest expert index, and it leaves its lane's list.
// Padding entries (expert >= E) are never candidates.
//
// SLABS: the logits arrive as nslab (<= RT_MAX_SLABS) partial sums
// logits[s][t][e] of a K-split projection; they are added in slice order (all
// loads issued first, a clamped duplicate masked out) and, when logits_out is
// given, the sums are written there.
//
// SIGMOID: the affinity of a kept expert is scale * sigma(l_j), or with
// `normalize` scale * sigma(l_j) / sum over the kept sigma (see
// launch_route_sigmoid); the selection is the same, sigma being increasing.
constexpr int RT_MAX_SLABS = 8;

template <int NPL, bool SLABS, bool SIGMOID>
__global__ __launch_bounds__(256) void route_topk_softmax_kernel(
    const float* __restrict__ logits, int nslab, float* __restrict__ logits_out, int T, int E,
    int k, int normalize, float scale, int32_t* __restrict__ ids, float* __restrict__ aff,
    int32_t* __restrict__ status) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;

    float lv[NPL];
    if (SLABS) {
        const size_t slab = (size_t)T * E;
        float pv[RT_MAX_SLABS][NPL];
#pragma unroll
        for (int s = 0; s < RT_MAX_SLABS; ++s)
#pragma unroll
            for (int i = 0; i < NPL; ++i) {
                const int e = min(lane + MOE_WAVE * i, E - 1);
                pv[s][i] = row[(size_t)min(s, nslab - 1) * slab + e];
            }
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            float v = pv[0][i];
#pragma unroll
            for (int s = 1; s < RT_MAX_SLABS; ++s) v += s < nslab ? pv[s][i] : 0.0f;
            lv[i] = v;
            const int e = lane + MOE_WAVE * i;
            if (logits_out && e < E) logits_out[(size_t)t * E + e] = v;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int e = lane + MOE_WAVE * i;
            lv[i] = e < E ? row[e] : 0.0f;
        }
    }

    uint32_t key[NPL];
    int slot[NPL];  // -1: no candidate
    bool bad = false;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + MOE_WAVE * i;
        const bool in = e < E;
        const float v = lv[i];
        bad |= in && !__builtin_isfinite(v);
        key[i] = in ? ordered_bits(v) : 0u;
        slot[i] = in ? i : -1;
    }
    if (status && __ballot(bad) != 0ull && lane == 0) atomicOr(status, MOE_STATUS_NONFINITE_LOGIT);
    // insertion order of (key desc, slot asc); empty entries (slot -1) last
#pragma unroll
    for (int a = 1; a < NPL; ++a)
#pragma unroll
        for (int b = a; b > 0; --b) {
            const bool lo_empty = slot[b - 1] < 0, hi_full = slot[b] >= 0;
            const bool sw = hi_full && (lo_empty || key[b] > key[b - 1] ||
                                        (key[b] == key[b - 1] && slot[b] < slot[b - 1]));
            const uint32_t k0 = key[b - 1], k1 = key[b];
            const int s0 = slot[b - 1], s1 = slot[b];
            key[b - 1] = sw ? k1 : k0;
            key[b] = sw ? k0 : k1;
            slot[b - 1] = sw ? s1 : s0;
            slot[b] = sw ? s0 : s1;
        }

    uint32_t my_o = 0, top_o = 0;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        const bool has = slot[0] >= 0;
        const uint32_t gmax = wave_red_u32<true>(has ? key[0] : 0u);
        const bool at = has && key[0] == gmax;
        const uint64_t hit = __ballot(at);
        int sel;
        if (__popcll(hit) == 1) {
            const int wl = (int)__builtin_ctzll(hit);
            sel = __builtin_amdgcn_readlane(slot[0], wl) * MOE_WAVE + wl;
        } else {  // equal keys in several lanes: the lowest expert index
            sel = (int)wave_red_u32<false>(at ? (uint32_t)(slot[0] * MOE_WAVE + lane) : 0xFFFFFFFFu);
        }
        if (lane == (sel & (MOE_WAVE - 1))) {  // the winner drops its head
#pragma unroll
            for (int i = 0; i + 1 < NPL; ++i) {
                key[i] = key[i + 1];
                slot[i] = slot[i + 1];
            }
            slot[NPL - 1] = -1;
        }
        if (j == 0) top_o = gmax;
        if (lane == j) {
            my_id = sel;
            my_o = gmax;
        }
    }
    float a;
    if (SIGMOID) {
        // log sigma(l) = min(l, 0) - log(1 + exp(-|l|)): finite for every finite l
        const float lj = from_ordered(my_o);
        const float ls = fminf(lj, 0.0f) - log1pf(expf(-fabsf(lj)));
        if (normalize) {
            // sigma_j / sum of the kept sigma, as a softmax over log sigma (slot
            // 0, in lane 0, holds the largest), so tiny sigmas never divide 0 by 0
            const float lm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), 0));
            const float w = lane < k ? expf(ls - lm) : 0.0f;
            a = w / wave_sum_f32(w);
        } else {
            a = expf(ls);
        }
        a *= scale;
    } else {
        const float M = from_ordered(top_o);
        const float w = lane < k ? expf(from_ordered(my_o) - M) : 0.0f;
        a = w / wave_sum_f32(w);
    }
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        aff[(size_t)t * k + lane] = a;
    }
}

template <bool SLABS, bool SIGMOID>
static int launch_route_impl(const float* logits, int nslab, float* logits_out, int T, int E,
                             int k, int normalize, float scale, int32_t* ids, float* aff,
                             int32_t* status, hipStream_t stream) {
    const int npl = (E + MOE_WAVE - 1) / MOE_WAVE;
    const dim3 grid((T + 3) / 4), block(256);
    prof_begin(SIGMOID ? "route_topk_sigmoid" : "route_topk_softmax", stream);
#define MOE_ROUTE_LAUNCH(N)                                                                       \
    route_topk_softmax_kernel<N, SLABS, SIGMOID><<<grid, block, 0, stream>>>(                     \
        logits, nslab, logits_out, T, E, k, normalize, scale, ids, aff, status)
    if (npl <= 1)
        MOE_ROUTE_LAUNCH(1);
    else if (npl <= 2)
        MOE_ROUTE_LAUNCH(2);
    else if (npl <= 4)
        MOE_ROUTE_LAUNCH(4);
    else if (npl <= 8)
        MOE_ROUTE_LAUNCH(8);
    else
        MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
    prof_end(stream);
    return check_launch("route_topk_softmax_kernel");
}

int launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* aff,
                 int32_t* status, hipStream_t stream) {
    return launch_route_impl<false, false>(logits, 1, nullptr, T, E, k, 0, 1.0f, ids, aff, status,
                                           stream);
}

// Sigmoid routing: the k largest logits (as for softmax), affinity
// scale * sigma(l_j), or scale * sigma(l_j) / sum of the kept sigma when
// normalize is set.
int launch_route_sigmoid(const float* logits, int T, int E, int k, int normalize, float scale,
                         int32_t* ids, float* aff, int32_t* status, hipStream_t stream) {
    return launch_route_impl<false, true>(logits, 1, nullptr, T, E, k, normalize ? 1 : 0, scale,
                                          ids, aff, status, stream);
}

int launch_route_slabs(const float* part, int nslab, float* logits_out, int T, int E, int k,
                       int32_t* ids, float* aff, int32_t* status, hipStream_t stream) {
    if (nslab < 1 || nslab > RT_MAX_SLABS) {
        set_error("router: %d partial slabs (1..%d supported)", nslab, RT_MAX_SLABS);
        return MOE_EINVAL;
    }
    if (nslab == 1 && !logits_out)
        return launch_route_impl<false, false>(part, 1, nullptr, T, E, k, 0, 1.0f, ids, aff,
                                               status, stream);
    return launch_route_impl<true, false>(part, nslab, logits_out, T, E, k, 0, 1.0f, ids, aff,
                                          status, stream);
}

}  // namespace moe
