// The routing plan: sort maps plus the segment list consumed by the FFN kernels.
//
// A segment is a run of rows of the sorted route space that share one weight
// set: an active routed expert (rows offsets[e] .. offsets[e+1]-1) or the
// shared expert (rows R .. R+T-1 with R = T*k, token t at row R + t).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct Plan {
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E+1]
    int32_t* sorted_route;  // [R]
    int32_t* inv_route;     // [R]
    int32_t* seg_n;         // [1]   number of segments
    int32_t* seg_expert;    // [E+1] expert id, -1 = shared expert
    int32_t* seg_row0;      // [E+1] first row in sorted space
    int32_t* seg_rows;      // [E+1] rows in the segment
    int32_t* seg_tile0;     // [E+2] prefix of ceil(rows / tile_m)
    // Tile list of the prefill variant, or null (not built): every full tile
    // of every segment in segment order, then the partial last tiles (in
    // segment order).  tile_info[i] = {expert (-1 = shared), first sorted row
    // of the tile, rows in the tile (1 .. tile_m), 0}; tile_n[0] = tiles.
    int4* tile_info;        // [at most ceil(R / tile_m) + E + shared tiles]
    int32_t* tile_n;        // [1]
};

// Stored weight formats: E4M3FN codes with fp32 128x128 block scales, or
// MXFP4 (E2M1 codes two a byte, E8M0 scale bytes per 32 elements of a row).
enum { WFMT_E4M3_128 = 0, WFMT_MXFP4 = 1 };
// activation operand of the prefill gate/up GEMM: bf16 x, x quantised to
// E4M3 per token (fp32 scale a row), or x quantised to MXFP4 (E8M0 a run of 32)
enum { AFMT_BF16 = 0, AFMT_E4M3 = 1, AFMT_MXFP4 = 2, AFMT_MXFP4_H4 = 3 };

// One expert's weights outside the routed arrays (the shared expert); the
// scales are fp32 (WFMT_E4M3_128) or E8M0 bytes (WFMT_MXFP4).
struct SharedW {
    const uint8_t* w13;
    const void* w13_scale;
    const uint8_t* w2;
    const void* w2_scale;
};

// Sort entry used by moe_sort and moe_fused_w8a16 (sort.hip).  `plan.seg_*`
// may be null when no segment list is wanted.
size_t sort_scratch_bytes(int R, int E);
int launch_sort(const int32_t* ids, int T, int k, int E, const Plan& plan, int has_shared,
                int tile_m, int32_t* status, void* scratch, hipStream_t stream);

// Expert activation (the values of MOE_ACT_*): SwiGLU on gate and up rows of
// w13 [2I, H], or relu(u)^2 on the up rows of a non-gated expert's w13 [I, H].
enum { ACT_SWIGLU = 0, ACT_RELU2 = 1 };

// Kernel launchers (route.hip, ffn_decode.hip, ffn_prefill.hip, misc).
int launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* aff,
                 int32_t* status, hipStream_t stream);
int launch_route_sigmoid(const float* logits, int T, int E, int k, int normalize, float scale,
                         int32_t* ids, float* aff, int32_t* status, hipStream_t stream);
// The router on nslab partial-logit slabs [nslab][T][E] added in slab order;
// the sums go to logits_out when it is not NULL.
int launch_route_slabs(const float* part, int nslab, float* logits_out, int T, int E, int k,
                       int32_t* ids, float* aff, int32_t* status, hipStream_t stream);
// Router projection (route_proj.hip): logits = x * wg^T, then the router.
int route_proj_splits(int T, int H, int E);
size_t route_proj_workspace_bytes(int T, int H, int E);
int launch_route_proj(const uint16_t* x, const uint16_t* wg, int T, int H, int E, int k,
                      float* logits, int32_t* ids, float* aff, int32_t* status, float* ws,
                      hipStream_t stream);
// Both FFN variants write, for every valid route r = t*k + j, the row
// aff[r] * MLP_e(x_t) (fp32, H wide): the decode variant at y[r], the prefill
// variant at its sorted position y[inv_route[r]]; the shared expert's row of
// token t is y[R + t] in both.  The combine then sums the k rows of a token.
int launch_decode_ffn(int layout, const uint16_t* x, const uint8_t* w13, const float* w13s,
                      const uint8_t* w2, const float* w2s, const SharedW& sh, const Plan& plan,
                      const float* aff, int T, int H, int I, int E, int k, uint16_t* abuf,
                      float* ybuf, int act, hipStream_t stream);
// Writes y (without the affinity) of every route at its sorted row of ybuf,
// in a block floating-point form: 16-bit mantissas at byte 2*col and one
// exponent byte per run of 8 columns at byte 2*H + col/8, row stride
// 2*H + H/8 bytes (common.hpp, bfp16x8_encode).  Weight scales are fp32
// 128x128 blocks, or (wfmt WFMT_MXFP4) E8M0 bytes, 4-byte aligned.  afmt
// AFMT_E4M3: xq [T, H] codes, xs fp32 [T]; AFMT_MXFP4 (MXFP4 weights only):
// xq [T, H/2], xs E8M0 bytes [T, H/32]; AFMT_MXFP4_H4: the same x, and the
// hidden activation quantised to MXFP4 too (codes and E8M0 bytes in abuf)
// for an E2M1 x E2M1 down GEMM; AFMT_BF16: both unused.
int launch_prefill_ffn(int layout, const uint16_t* x, const uint8_t* w13, const void* w13s,
                       const uint8_t* w2, const void* w2s, const SharedW& sh, const Plan& plan,
                       int T, int H, int I, int E, int k, uint16_t* abuf, float* ybuf, int act,
                       const uint8_t* xq, const void* xs, int afmt, int wfmt, hipStream_t stream);
// Per-token E4M3 quantisation of x [T, H] bf16 -> codes [T, H], scales [T] (quant.hip).
int launch_quant_rows_e4m3(const uint16_t* x, int T, int H, uint8_t* xq, float* xs,
                           hipStream_t stream);
// MXFP4 quantisation of x [T, H] bf16 -> codes [T, H/2] (two E2M1 a byte),
// E8M0 scales [T, H/32] (quant.hip).  H % 32 == 0.
int launch_quant_rows_mxfp4(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream);
int launch_pack_w8(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                   hipStream_t stream);
int launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                          hipStream_t stream);
int prefill_tile_m();
int prefill_supported(int H, int I, int act);
// MOE_OK, or MOE_EUNSUPPORTED with the error message set.
int prefill_check(int T, int H, int I, int E, int k, int has_shared, int act);
// Sums, per token, the k route rows whose id is valid (plus the shared row at
// R + t).  Decode producers write aff * y at row r (inv_route and aff null);
// prefill producers write y at the route's sorted position in the block
// floating-point layout of launch_prefill_ffn, and the sum takes aff[r] * y widened to fp32.
// Ids outside [0, E) set
// MOE_STATUS_BAD_EXPERT_ID in *status (if not NULL).
int launch_combine(const float* ybuf, const int32_t* ids, const int32_t* inv_route,
                   const float* aff, int T, int H, int k, int E, int has_shared, int32_t* status,
                   float* out, hipStream_t stream);
// Decode variant helpers: the M tile, whether the fused one-workgroup-per-
// expert kernel applies, and its self-routed form (no sort: each workgroup
// scans the ids for its expert; at most decode_self_routed_max_routes() routes).
int decode_mt(int T, int k, int E);
bool decode_fused_fits(int T, int k, int E, int H, int I, int has_shared, bool self_routed);
size_t decode_fused_lds_bytes(int MT, int I, int self_routes, int H = 0, bool alias = false);
bool decode_fused_x_in_lds(int MT, int H, int I, int self_routes);
int decode_self_routed_max_routes();
// Row tiles of tile_m rows over all segments, at most (the sort's tile list
// holds this many records when built with tile_m >= the given size).
size_t decode_fused_tile_capacity(int T, int k, int E, int has_shared, int tile_m);
int launch_decode_fused_self(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                             const void* w13s, const uint8_t* w2, const void* w2s,
                             const SharedW& sh, const int32_t* ids, const float* aff, int T,
                             int H, int I, int E, int k, float* ybuf, int act, int wfmt,
                             hipStream_t stream);
// The same kernel after the sort (one workgroup per segment of the plan).
int launch_decode_fused(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                        const void* w13s, const uint8_t* w2, const void* w2s, const SharedW& sh,
                        const Plan& plan, const float* aff, int T, int H, int I, int E, int k,
                        float* ybuf, int act, int wfmt, hipStream_t stream);
int launch_decode_e4m3fn(const uint8_t* codes, uint16_t* out, int64_t n, hipStream_t stream);
int launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t stream);

// Optional per-kernel timing events around each launch (api.hip).
void prof_begin(const char* name, hipStream_t stream);
void prof_end(hipStream_t stream);

}  // namespace moe
