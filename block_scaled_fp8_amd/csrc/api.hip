// C ABI of the block-scaled FP8 routed MoE expert FFN (see include/moe_w8a16.h).
//
// Host-side contract checks follow "spark_model/layers/nemotron_moe.rs" (the
// layer constructor validates top_k against 1..=E and the expert count
// against a maximum, failing with a message) and the AITER PR page (tensor
// contracts validated in the launcher, caller-provided outputs, scratch kept
// below the dispatch, unsupported geometry rejected).  Nothing here allocates,
// synchronises or reads device memory back.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.hpp"
#include "plan.hpp"

namespace moe {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: launch failed: %s", what, hipGetErrorString(e));
        return MOE_EHIP;
    }
    return MOE_OK;
}

// Workspace carve-up for moe_fused_w8a16 (256-byte aligned pieces).
struct FusedLayout {
    size_t counts, offsets, sorted_route, inv_route, seg_n, seg_expert, seg_row0, seg_rows,
        seg_tile0, tile_info, tile_n, sort_scratch, abuf, ybuf, xq, xs, total;
};

// The pieces before ybuf do not depend on the variant.  ybuf holds one
// contribution row per route (+ shared rows + a trash row): fp32 for the
// decode variant, block floating point (2 bytes a value + one exponent byte
// per 8) for the prefill ones; AUTO is sized for either.  The fp8-activation
// variant appends the E4M3 codes and per-token scales of x, the MXFP4 ones
// its E2M1 codes and E8M0 bytes (MOE_VARIANT_PREFILL_FP4 keeps the MXFP4
// hidden activation inside abuf).
static FusedLayout fused_layout(int T, int H, int I, int E, int k, int has_shared, int variant) {
    const bool fp8_x = variant == MOE_VARIANT_PREFILL_A8;
    const bool fp4_x = variant == MOE_VARIANT_PREFILL_A4 || variant == MOE_VARIANT_PREFILL_FP4;
    const bool compact = variant == MOE_VARIANT_PREFILL || fp8_x || fp4_x;
    FusedLayout L;
    const size_t R = (size_t)T * k;
    const size_t rows = R + (has_shared ? (size_t)T : 0);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += halign(bytes);
        return at;
    };
    L.counts = take(sizeof(int32_t) * E);
    L.offsets = take(sizeof(int32_t) * (E + 1));
    L.sorted_route = take(sizeof(int32_t) * R);
    L.inv_route = take(sizeof(int32_t) * R);
    L.seg_n = take(sizeof(int32_t));
    L.seg_expert = take(sizeof(int32_t) * (E + 1));
    L.seg_row0 = take(sizeof(int32_t) * (E + 1));
    L.seg_rows = take(sizeof(int32_t) * (E + 1));
    L.seg_tile0 = take(sizeof(int32_t) * (E + 2));
    // row tiles (prefill: 128 rows; the sorted decode kernel: 16 or 32): at
    // most ceil(R / tile) + one partial tile per segment, sized for 16 rows
    const size_t max_tiles = decode_fused_tile_capacity(T, k, E, has_shared, 16);
    L.tile_info = take(sizeof(int4) * max_tiles);
    L.tile_n = take(sizeof(int32_t));
    L.sort_scratch = take(sort_scratch_bytes((int)R, E));
    L.abuf = take(sizeof(uint16_t) * rows * I);
    const size_t yrow = compact ? 2 * (size_t)H + (size_t)H / 8 : sizeof(float) * (size_t)H;
    L.ybuf = take(yrow * (rows + 1));  // + one trash row for padded stores
    L.xq = fp8_x ? take((size_t)T * H) : fp4_x ? take((size_t)T * H / 2) : 0;
    L.xs = fp8_x ? take(sizeof(float) * (size_t)T) : fp4_x ? take((size_t)T * (H / 32)) : 0;
    L.total = o;
    return L;
}

// AUTO: the decode variant up to 16 routes per expert and the self-routed
// batch size, the prefill GEMMs above.  Measured at H = 2048, I = 512,
// E = 256, k = 8: T = 512 decode 172 / prefill 195 us, T = 768 267 / 204,
// T = 1024 296 / 218 (past 4096 routes decode needs the sort and a second
// M tile).
static int resolve_variant(int T, int H, int I, int E, int k, int act, int variant) {
    if (variant != MOE_VARIANT_AUTO) return variant;
    const long long R = (long long)T * k;
    return (R <= 16LL * E && R <= decode_self_routed_max_routes()) || !prefill_supported(H, I, act)
               ? MOE_VARIANT_DECODE
               : MOE_VARIANT_PREFILL;
}

static int check_route_args(int T, int E, int k) {
    if (T < 0) {
        set_error("T must be >= 0 (got %d)", T);
        return MOE_EINVAL;
    }
    if (E < 1 || E > MOE_MAX_EXPERTS) {
        set_error("E must be in 1..%d (got %d)", MOE_MAX_EXPERTS, E);
        return MOE_EINVAL;
    }
    if (k < 1 || k > E || k > MOE_MAX_TOPK) {
        set_error("k must be in 1..min(E, %d) (got k=%d, E=%d)", MOE_MAX_TOPK, k, E);
        return MOE_EINVAL;
    }
    if ((long long)T * k > (1LL << 30)) {
        set_error("T*k too large (%lld)", (long long)T * k);
        return MOE_EINVAL;
    }
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_route(const float* logits, int T, int E, int k, int32_t* ids, float* aff,
              int32_t* status, void* stream) {
    g_err[0] = 0;
    if (int rc = check_route_args(T, E, k)) return rc;
    if (T == 0) return MOE_OK;
    if (!logits || !ids || !aff) {
        set_error("moe_route: logits, ids and aff must be non-NULL");
        return MOE_EINVAL;
    }
    return launch_route(logits, T, E, k, ids, aff, status, (hipStream_t)stream);
}

int moe_route_sigmoid(const float* logits, int T, int E, int k, int normalize, float scale,
                      int32_t* ids, float* aff, int32_t* status, void* stream) {
    g_err[0] = 0;
    if (int rc = check_route_args(T, E, k)) return rc;
    if (normalize != 0 && normalize != 1) {
        set_error("moe_route_sigmoid: normalize must be 0 or 1 (got %d)", normalize);
        return MOE_EINVAL;
    }
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) {
        set_error("moe_route_sigmoid: scale must be finite");
        return MOE_EINVAL;
    }
    if (T == 0) return MOE_OK;
    if (!logits || !ids || !aff) {
        set_error("moe_route_sigmoid: logits, ids and aff must be non-NULL");
        return MOE_EINVAL;
    }
    return launch_route_sigmoid(logits, T, E, k, normalize, scale, ids, aff, status,
                                (hipStream_t)stream);
}

size_t moe_route_proj_workspace_bytes(int T, int H, int E) {
    if (T < 1 || H < 64 || H % 64 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    return route_proj_workspace_bytes(T, H, E);
}

int moe_route_proj(const void* x, const void* wg, int T, int H, int E, int k, float* logits,
                   int32_t* ids, float* aff, int32_t* status, void* ws, size_t ws_bytes,
                   void* stream) {
    g_err[0] = 0;
    if (int rc = check_route_args(T, E, k)) return rc;
    if (H < 64 || H % 64) {
        set_error("moe_route_proj: H must be a positive multiple of 64 (got %d)", H);
        return MOE_EUNSUPPORTED;
    }
    if (T == 0) return MOE_OK;
    if (!x || !wg || !ids || !aff) {
        set_error("moe_route_proj: x, wg, ids and aff must be non-NULL");
        return MOE_EINVAL;
    }
    if (((uintptr_t)x | (uintptr_t)wg) & 15) {
        set_error("moe_route_proj: x and wg must be 16-byte aligned");
        return MOE_EINVAL;
    }
    const bool direct = route_proj_splits(T, H, E) == 1 && logits;  // no slab needed
    const size_t need = route_proj_workspace_bytes(T, H, E);
    if (!direct && (!ws || ws_bytes < need)) {
        set_error("moe_route_proj: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
        return MOE_EINVAL;
    }
    return launch_route_proj(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), T,
                             H, E, k, logits, ids, aff, status, static_cast<float*>(ws),
                             (hipStream_t)stream);
}

size_t moe_sort_workspace_bytes(int T, int k, int E) {
    if (T < 0 || k < 1 || E < 1) return 0;
    return sort_scratch_bytes(T * k, E);
}

int moe_sort(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
             int32_t* sorted_route, int32_t* inv_route, int32_t* status, void* ws,
             size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (int rc = check_route_args(T, E, k)) return rc;
    if (!counts || !offsets) {
        set_error("moe_sort: counts and offsets must be non-NULL");
        return MOE_EINVAL;
    }
    if (T > 0 && (!ids || !sorted_route || !inv_route)) {
        set_error("moe_sort: ids, sorted_route and inv_route must be non-NULL");
        return MOE_EINVAL;
    }
    const size_t need = sort_scratch_bytes(T * k, E);
    if (need && (!ws || ws_bytes < need)) {
        set_error("moe_sort: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
        return MOE_EINVAL;
    }
    Plan p{};
    p.counts = counts;
    p.offsets = offsets;
    p.sorted_route = sorted_route;
    p.inv_route = inv_route;
    if (T == 0) {
        // empty input: zero counts and offsets
        if (int rc = launch_fill_i32(counts, 0, E, (hipStream_t)stream)) return rc;
        return launch_fill_i32(offsets, 0, E + 1, (hipStream_t)stream);
    }
    return launch_sort(ids, T, k, E, p, 0, 1, status, ws, (hipStream_t)stream);
}

size_t moe_fused_workspace_bytes(int T, int H, int I, int E, int k, int has_shared,
                                 int variant) {
    if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1) return 0;
    if (variant < MOE_VARIANT_AUTO || variant > MOE_VARIANT_PREFILL_FP4) return 0;
    return fused_layout(T, H, I, E, k, has_shared ? 1 : 0, variant).total;
}

}  // extern "C"

namespace moe {
// The fused call for both stored weight formats.  `who` names the entry point
// in error messages; `sh` is the shared expert (w13 == nullptr: none).
static int fused_impl(const char* who, const void* x, const uint8_t* w13, const void* w13_scale,
                      const uint8_t* w2, const void* w2_scale, const int32_t* ids, const float* aff,
                      int T, int H, int I, int E, int k, const SharedW* shared, float* out,
                      int32_t* status, void* ws, size_t ws_bytes, int weight_layout, int variant,
                      int activation, int wfmt, void* stream) {
    g_err[0] = 0;
    const bool mx4 = wfmt == WFMT_MXFP4;
    if (activation != MOE_ACT_SWIGLU && activation != MOE_ACT_RELU2) {
        set_error("unknown activation %d", activation);
        return MOE_EINVAL;
    }
    const int act = activation == MOE_ACT_RELU2 ? ACT_RELU2 : ACT_SWIGLU;
    if (int rc = check_route_args(T, E, k)) return rc;
    if (H < 128 || I < 128 || H % 128 || I % 128) {
        set_error("H and I must be positive multiples of 128 (got H=%d, I=%d)", H, I);
        return MOE_EUNSUPPORTED;
    }
    if ((long long)H * I * 3 > (1LL << 40)) {
        set_error("expert too large (H=%d, I=%d)", H, I);
        return MOE_EUNSUPPORTED;
    }
    if (weight_layout != MOE_LAYOUT_ROWMAJOR && weight_layout != MOE_LAYOUT_TILED) {
        set_error("unknown weight layout %d", weight_layout);
        return MOE_EINVAL;
    }
    if (variant < MOE_VARIANT_AUTO || variant > MOE_VARIANT_PREFILL_FP4) {
        set_error("unknown variant %d", variant);
        return MOE_EINVAL;
    }
    if ((variant == MOE_VARIANT_PREFILL_A4 || variant == MOE_VARIANT_PREFILL_FP4) && !mx4) {
        set_error("%s: MXFP4 activations (MOE_VARIANT_PREFILL_A4, MOE_VARIANT_PREFILL_FP4) need MXFP4 weights",
                  who);
        return MOE_EUNSUPPORTED;
    }
    if (T == 0) return MOE_OK;
    if (!x || !w13 || !w13_scale || !w2 || !w2_scale || !ids || !aff || !out) {
        set_error("%s: x, weights, scales, ids, aff and out must be non-NULL", who);
        return MOE_EINVAL;
    }
    if (shared && (!shared->w13 || !shared->w13_scale || !shared->w2 || !shared->w2_scale)) {
        set_error("%s: shared expert descriptor has a NULL member", who);
        return MOE_EINVAL;
    }
    if ((const void*)out == x) {
        set_error("%s: out must not alias x", who);
        return MOE_EINVAL;
    }
    // 16-byte vector loads and stores (and direct-to-LDS loads) on x, the
    // weights, out and the workspace; 4-byte ones on the fp32 scales, ids and
    // aff (E8M0 scales are read a byte at a time)
    {
        uintptr_t a16 = (uintptr_t)x | (uintptr_t)w13 | (uintptr_t)w2 | (uintptr_t)out |
                        (uintptr_t)ws;
        uintptr_t a4 = (uintptr_t)ids | (uintptr_t)aff;
        if (!mx4) a4 |= (uintptr_t)w13_scale | (uintptr_t)w2_scale;
        if (shared) {
            a16 |= (uintptr_t)shared->w13 | (uintptr_t)shared->w2;
            if (!mx4) a4 |= (uintptr_t)shared->w13_scale | (uintptr_t)shared->w2_scale;
        }
        if ((a16 & 15) || (a4 & 3)) {
            set_error("%s: x, w13, w2, out and ws must be 16-byte aligned, the %sids and aff "
                      "4-byte aligned", who, mx4 ? "" : "scales, ");
            return MOE_EINVAL;
        }
    }
    const int has_shared = shared ? 1 : 0;
    const bool fp8_x = variant == MOE_VARIANT_PREFILL_A8;
    const bool fp4_h = variant == MOE_VARIANT_PREFILL_FP4;
    const bool fp4_x = variant == MOE_VARIANT_PREFILL_A4 || fp4_h;
    // the prefill GEMMs stage MXFP4 scales with 4-byte loads
    const bool mx_sc4 = !mx4 || ((((uintptr_t)w13_scale | (uintptr_t)w2_scale |
                                  (shared ? (uintptr_t)shared->w13_scale | (uintptr_t)shared->w2_scale : 0)) &
                                 3) == 0);
    if (mx4 && (variant == MOE_VARIANT_PREFILL || fp8_x || fp4_x) && !mx_sc4) {
        set_error("%s: the prefill variants need 4-byte aligned MXFP4 scale arrays", who);
        return MOE_EINVAL;
    }
    const int auto_pick = variant == MOE_VARIANT_AUTO;
    variant = resolve_variant(T, H, I, E, k, act, variant);
    if (auto_pick && mx4 && !mx_sc4) variant = MOE_VARIANT_DECODE;
    const FusedLayout L = fused_layout(T, H, I, E, k, has_shared, variant);
    if (!ws || ws_bytes < L.total) {
        set_error("%s: workspace of %zu bytes needed (got %zu)", who, L.total, ws_bytes);
        return MOE_EINVAL;
    }
    if (variant == MOE_VARIANT_PREFILL || fp8_x || fp4_x) {
        if (int rc = prefill_check(T, H, I, E, k, has_shared, act)) return rc;
    }
    // MXFP4 weights, decode variant: the weight-streaming kernel (self-routed
    // or on row tiles of the sort)
    const long long R = (long long)T * k;
    const bool mx_self = R <= decode_self_routed_max_routes();
    if (mx4 && variant == MOE_VARIANT_DECODE &&
        (decode_fused_lds_bytes(decode_mt(T, k, E), I, mx_self ? (int)R : 0) > 64 * 1024 ||
         (long long)T * H >= (1LL << 32))) {
        set_error("%s: MXFP4 weights need the activations of one expert pass in 64 KB of LDS "
                  "and T*H < 2^32 (got T=%d, H=%d, I=%d)", who, T, H, I);
        return MOE_EUNSUPPORTED;
    }

    char* base = static_cast<char*>(ws);
    Plan p;
    p.counts = reinterpret_cast<int32_t*>(base + L.counts);
    p.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    p.sorted_route = reinterpret_cast<int32_t*>(base + L.sorted_route);
    p.inv_route = reinterpret_cast<int32_t*>(base + L.inv_route);
    p.seg_n = reinterpret_cast<int32_t*>(base + L.seg_n);
    p.seg_expert = reinterpret_cast<int32_t*>(base + L.seg_expert);
    p.seg_row0 = reinterpret_cast<int32_t*>(base + L.seg_row0);
    p.seg_rows = reinterpret_cast<int32_t*>(base + L.seg_rows);
    p.seg_tile0 = reinterpret_cast<int32_t*>(base + L.seg_tile0);
    const bool pf = variant == MOE_VARIANT_PREFILL || fp8_x || fp4_x;
    p.tile_info = reinterpret_cast<int4*>(base + L.tile_info);
    p.tile_n = reinterpret_cast<int32_t*>(base + L.tile_n);
    uint16_t* abuf = reinterpret_cast<uint16_t*>(base + L.abuf);
    float* ybuf = reinterpret_cast<float*>(base + L.ybuf);
    hipStream_t s = (hipStream_t)stream;
    const SharedW sh = shared ? *shared : SharedW{nullptr, nullptr, nullptr, nullptr};
    const float* w13f = static_cast<const float*>(w13_scale);
    const float* w2f = static_cast<const float*>(w2_scale);

    const uint16_t* xb = static_cast<const uint16_t*>(x);
    int rc;
    if (variant == MOE_VARIANT_DECODE &&
        (mx4 ? mx_self : decode_fused_fits(T, k, E, H, I, has_shared, true))) {
        // small decode batch: each expert's workgroup finds its own routes
        rc = launch_decode_fused_self(weight_layout, decode_mt(T, k, E), xb, w13, w13_scale, w2,
                                      w2_scale, sh, ids, aff, T, H, I, E, k, ybuf, act, wfmt, s);
    } else {
        // (the sorted decode kernel takes one row tile of its pass height per workgroup)
        const int tile_m = pf ? prefill_tile_m() : 16 * decode_mt(T, k, E);
        if ((rc = launch_sort(ids, T, k, E, p, has_shared, tile_m, status, base + L.sort_scratch, s)))
            return rc;
        if (mx4 && variant == MOE_VARIANT_DECODE)
            rc = launch_decode_fused(weight_layout, decode_mt(T, k, E), xb, w13, w13_scale, w2,
                                     w2_scale, sh, p, aff, T, H, I, E, k, ybuf, act, wfmt, s);
        else if (variant == MOE_VARIANT_DECODE)
            rc = launch_decode_ffn(weight_layout, xb, w13, w13f, w2, w2f, sh, p, aff, T, H, I, E,
                                   k, abuf, ybuf, act, s);
        else {
            uint8_t* xq = fp8_x || fp4_x ? reinterpret_cast<uint8_t*>(base + L.xq) : nullptr;
            void* xsc = fp8_x || fp4_x ? static_cast<void*>(base + L.xs) : nullptr;
            if (fp8_x && (rc = launch_quant_rows_e4m3(xb, T, H, xq, static_cast<float*>(xsc), s))) return rc;
            if (fp4_x && (rc = launch_quant_rows_mxfp4(xb, T, H, xq, static_cast<uint8_t*>(xsc), s)))
                return rc;
            rc = launch_prefill_ffn(weight_layout, xb, w13, w13_scale, w2, w2_scale, sh, p, T, H, I,
                                    E, k, abuf, ybuf, act, xq, xsc,
                                    fp4_h ? AFMT_MXFP4_H4 : fp4_x ? AFMT_MXFP4 : fp8_x ? AFMT_E4M3 : AFMT_BF16,
                                    wfmt, s);
        }
    }
    if (rc) return rc;
    const bool gathered = pf;
    return launch_combine(ybuf, ids, gathered ? p.inv_route : nullptr,
                          gathered ? aff : nullptr, T, H, k, E,
                          has_shared, status, out, s);
}
}  // namespace moe

extern "C" {

int moe_fused_w8a16_ex(const void* x, const uint8_t* w13, const float* w13_scale,
                       const uint8_t* w2, const float* w2_scale, const int32_t* ids,
                       const float* aff, int T, int H, int I, int E, int k,
                       const moe_expert_w8* shared, float* out, int32_t* status, void* ws,
                       size_t ws_bytes, int weight_layout, int variant, int activation,
                       void* stream) {
    SharedW sh{};
    if (shared) sh = SharedW{shared->w13, shared->w13_scale, shared->w2, shared->w2_scale};
    return fused_impl("moe_fused_w8a16", x, w13, w13_scale, w2, w2_scale, ids, aff, T, H, I, E, k,
                      shared ? &sh : nullptr, out, status, ws, ws_bytes, weight_layout, variant,
                      activation, WFMT_E4M3_128, stream);
}

int moe_fused_mxfp4(const void* x, const uint8_t* w13, const uint8_t* w13_scale,
                    const uint8_t* w2, const uint8_t* w2_scale, const int32_t* ids,
                    const float* aff, int T, int H, int I, int E, int k,
                    const moe_expert_mx4* shared, float* out, int32_t* status, void* ws,
                    size_t ws_bytes, int weight_layout, int variant, int activation,
                    void* stream) {
    SharedW sh{};
    if (shared) sh = SharedW{shared->w13, shared->w13_scale, shared->w2, shared->w2_scale};
    return fused_impl("moe_fused_mxfp4", x, w13, w13_scale, w2, w2_scale, ids, aff, T, H, I, E, k,
                      shared ? &sh : nullptr, out, status, ws, ws_bytes, weight_layout, variant,
                      activation, WFMT_MXFP4, stream);
}

int moe_fused_w8a16(const void* x, const uint8_t* w13, const float* w13_scale,
                    const uint8_t* w2, const float* w2_scale, const int32_t* ids,
                    const float* aff, int T, int H, int I, int E, int k,
                    const moe_expert_w8* shared, float* out, int32_t* status, void* ws,
                    size_t ws_bytes, int weight_layout, int variant, void* stream) {
    return moe_fused_w8a16_ex(x, w13, w13_scale, w2, w2_scale, ids, aff, T, H, I, E, k, shared,
                              out, status, ws, ws_bytes, weight_layout, variant, MOE_ACT_SWIGLU,
                              stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation entry
// The workspace of moe_fused_w8a16_noalloc: one file-scope device array.  Each
// GPU the library runs on holds its own copy until the process ends; host
// code never uses the array's name as an address (it is a host-side stand-in
// there), only the device address taken once per device below.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (the device must be
// current), taken on its first use and kept.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_error("moe_fused_w8a16_noalloc: no usable current device (%s)",
                  e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
        return MOE_EHIP;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_error("moe_fused_w8a16_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                      hipGetErrorString(e));
            return MOE_EHIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" {

int moe_fused_w8a16_noalloc(const void* x, const uint8_t* w13, const float* w13_scale,
                            const uint8_t* w2, const float* w2_scale, const int32_t* ids,
                            const float* aff, int T, int H, int I, int E, int k,
                            const moe_expert_w8* shared, float* out, int32_t* status,
                            int weight_layout, int variant, int activation, void* stream) {
    g_err[0] = 0;
    if (activation != MOE_ACT_SWIGLU && activation != MOE_ACT_RELU2) {
        set_error("unknown activation %d", activation);
        return MOE_EINVAL;
    }
    if (int rc = check_route_args(T, E, k)) return rc;
    if (H < 128 || I < 128 || H % 128 || I % 128) {
        set_error("H and I must be positive multiples of 128 (got H=%d, I=%d)", H, I);
        return MOE_EUNSUPPORTED;
    }
    if (variant < MOE_VARIANT_AUTO || variant > MOE_VARIANT_PREFILL_FP4) {
        set_error("unknown variant %d", variant);
        return MOE_EINVAL;
    }
    if (variant == MOE_VARIANT_PREFILL_A4 || variant == MOE_VARIANT_PREFILL_FP4) {
        set_error("moe_fused_w8a16_noalloc: MXFP4 activations need MXFP4 weights");
        return MOE_EUNSUPPORTED;
    }
    if (T == 0) return MOE_OK;
    const int act = activation == MOE_ACT_RELU2 ? ACT_RELU2 : ACT_SWIGLU;
    const int v = resolve_variant(T, H, I, E, k, act, variant);
    const size_t need = fused_layout(T, H, I, E, k, shared ? 1 : 0, v).total;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) {
        set_error("moe_fused_w8a16_noalloc: this call needs %zu bytes of workspace, more than the "
                  "%zu-byte device scratch array (use moe_fused_w8a16 with a workspace)",
                  need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
        return MOE_EUNSUPPORTED;
    }
    void* ws = nullptr;
    if (int rc = scratch_address(&ws)) return rc;
    return moe_fused_w8a16_ex(x, w13, w13_scale, w2, w2_scale, ids, aff, T, H, I, E, k, shared,
                              out, status, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, weight_layout, v,
                              activation, stream);
}

int moe_pack_w8(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                void* stream) {
    g_err[0] = 0;
    if (n_mats < 0 || rows < 0 || cols < 0 || rows % 16 || cols % 64) {
        set_error("moe_pack_w8: need n_mats, rows, cols >= 0, rows %% 16 == 0, cols %% 64 == 0 "
                  "(got %lld, %d, %d)", (long long)n_mats, rows, cols);
        return MOE_EINVAL;
    }
    if (n_mats == 0 || rows == 0 || cols == 0) return MOE_OK;
    if (!src || !dst) {
        set_error("moe_pack_w8: src and dst must be non-NULL");
        return MOE_EINVAL;
    }
    const size_t bytes = (size_t)n_mats * rows * cols;
    const char* a = reinterpret_cast<const char*>(src);
    const char* b = reinterpret_cast<const char*>(dst);
    if (a < b + bytes && b < a + bytes) {
        set_error("moe_pack_w8: src and dst overlap");
        return MOE_EINVAL;
    }
    return launch_pack_w8(src, dst, n_mats, rows, cols, (hipStream_t)stream);
}

int moe_pack_mx_scales(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                       void* stream) {
    g_err[0] = 0;
    if (n_mats < 0 || rows < 0 || cols < 0 || rows % 16 || cols % 4) {
        set_error("moe_pack_mx_scales: need n_mats, rows, cols >= 0, rows %% 16 == 0, "
                  "cols %% 4 == 0 (got %lld, %d, %d)", (long long)n_mats, rows, cols);
        return MOE_EINVAL;
    }
    if (n_mats == 0 || rows == 0 || cols == 0) return MOE_OK;
    if (!src || !dst) {
        set_error("moe_pack_mx_scales: src and dst must be non-NULL");
        return MOE_EINVAL;
    }
    const size_t bytes = (size_t)n_mats * rows * cols;
    const char* a = reinterpret_cast<const char*>(src);
    const char* b = reinterpret_cast<const char*>(dst);
    if (a < b + bytes && b < a + bytes) {
        set_error("moe_pack_mx_scales: src and dst overlap");
        return MOE_EINVAL;
    }
    return launch_pack_mx_scales(src, dst, n_mats, rows, cols, (hipStream_t)stream);
}

int moe_quant_e4m3_rows(const void* x, int T, int H, uint8_t* codes, float* scales,
                        void* stream) {
    g_err[0] = 0;
    if (T < 0 || H < 8 || H % 8) {
        set_error("moe_quant_e4m3_rows: need T >= 0 and H a positive multiple of 8 (got %d, %d)", T, H);
        return MOE_EINVAL;
    }
    if (T == 0) return MOE_OK;
    if (!x || !codes || !scales) {
        set_error("moe_quant_e4m3_rows: x, codes and scales must be non-NULL");
        return MOE_EINVAL;
    }
    if ((uintptr_t)x & 15 || (uintptr_t)codes & 7) {
        set_error("moe_quant_e4m3_rows: x must be 16-byte and codes 8-byte aligned");
        return MOE_EINVAL;
    }
    return launch_quant_rows_e4m3(static_cast<const uint16_t*>(x), T, H, codes, scales,
                                  (hipStream_t)stream);
}

int moe_quant_mxfp4_rows(const void* x, int T, int H, uint8_t* codes, uint8_t* scales, void* stream) {
    g_err[0] = 0;
    if (T < 0 || H < 32 || H % 32) {
        set_error("moe_quant_mxfp4_rows: need T >= 0 and H a positive multiple of 32 (got %d, %d)", T, H);
        return MOE_EINVAL;
    }
    if (T == 0) return MOE_OK;
    if (!x || !codes || !scales) {
        set_error("moe_quant_mxfp4_rows: x, codes and scales must be non-NULL");
        return MOE_EINVAL;
    }
    if ((uintptr_t)x & 15 || (uintptr_t)codes & 15) {
        set_error("moe_quant_mxfp4_rows: x and codes must be 16-byte aligned");
        return MOE_EINVAL;
    }
    return launch_quant_rows_mxfp4(static_cast<const uint16_t*>(x), T, H, codes, scales,
                                   (hipStream_t)stream);
}

int moe_decode_e4m3fn(const uint8_t* codes, uint16_t* out, int64_t n, void* stream) {
    g_err[0] = 0;
    if (n < 0) {
        set_error("moe_decode_e4m3fn: n must be >= 0");
        return MOE_EINVAL;
    }
    if (n == 0) return MOE_OK;
    if (!codes || !out) {
        set_error("moe_decode_e4m3fn: codes and out must be non-NULL");
        return MOE_EINVAL;
    }
    return launch_decode_e4m3fn(codes, out, n, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------- profiling
#include <mutex>
#include <string>
#include <vector>

namespace moe {
namespace {
struct ProfRecord {
    const char* name;
    hipEvent_t start, stop;
};
struct ProfStat {
    std::string name;
    int64_t launches = 0;
    double total_ms = 0.0;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<hipEvent_t> g_prof_pool;
std::vector<ProfRecord> g_prof_open;   // begun, not yet ended (per call, at most one)
std::vector<ProfRecord> g_prof_done;
std::vector<ProfStat> g_prof_stats;
constexpr size_t kMaxPending = 1 << 16;

hipEvent_t prof_event() {
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

void prof_begin(const char* name, hipStream_t stream) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on || g_prof_done.size() >= kMaxPending) return;
    hipEvent_t a = prof_event(), b = prof_event();
    if (!a || !b) return;
    if (hipEventRecord(a, stream) != hipSuccess) {
        g_prof_pool.push_back(a);
        g_prof_pool.push_back(b);
        return;
    }
    g_prof_open.push_back(ProfRecord{name, a, b});
}

void prof_end(hipStream_t stream) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_open.empty()) return;
    ProfRecord r = g_prof_open.back();
    g_prof_open.pop_back();
    if (hipEventRecord(r.stop, stream) != hipSuccess) {
        g_prof_pool.push_back(r.start);
        g_prof_pool.push_back(r.stop);
        return;
    }
    g_prof_done.push_back(r);
}

}  // namespace moe

extern "C" {

int moe_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(moe::g_prof_mu);
    if (on) moe::g_prof_stats.clear();
    moe::g_prof_on = on != 0;
    return MOE_OK;
}

int moe_profile_collect(void) {
    std::lock_guard<std::mutex> lk(moe::g_prof_mu);
    int rc = MOE_OK;
    for (const auto& r : moe::g_prof_done) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
            moe::set_error("moe_profile_collect: event query failed");
            rc = MOE_EHIP;
        } else {
            moe::ProfStat* st = nullptr;
            for (auto& s : moe::g_prof_stats)
                if (s.name == r.name) st = &s;
            if (!st) {
                moe::g_prof_stats.push_back(moe::ProfStat{r.name, 0, 0.0});
                st = &moe::g_prof_stats.back();
            }
            st->launches += 1;
            st->total_ms += ms;
        }
        moe::g_prof_pool.push_back(r.start);
        moe::g_prof_pool.push_back(r.stop);
    }
    moe::g_prof_done.clear();
    return rc;
}

int moe_profile_count(void) {
    std::lock_guard<std::mutex> lk(moe::g_prof_mu);
    return (int)moe::g_prof_stats.size();
}

int moe_profile_stat(int i, char* name, int name_len, int64_t* launches, double* total_ms) {
    std::lock_guard<std::mutex> lk(moe::g_prof_mu);
    if (i < 0 || i >= (int)moe::g_prof_stats.size() || !name || name_len < 1 || !launches ||
        !total_ms) {
        moe::set_error("moe_profile_stat: bad index or NULL output");
        return MOE_EINVAL;
    }
    const auto& s = moe::g_prof_stats[i];
    snprintf(name, (size_t)name_len, "%s", s.name.c_str());
    *launches = s.launches;
    *total_ms = s.total_ms;
    return MOE_OK;
}

}  // extern "C"
