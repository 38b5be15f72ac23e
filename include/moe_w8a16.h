/*
 * moe_w8a16.h -- C ABI of the block-scaled FP8 (W8A16) routed MoE expert FFN
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the pages' titles and sections):
 *
 *  - "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for Trainium2",
 *    section "FP8 MoE decode kernel (moe_fused_w8_35b)": the routed experts
 *    run gate/up GEMM -> SwiGLU -> down GEMM -> affinity scale -> expert-sum on
 *    E4M3FN weights with one scale per 128x128 block, decoded to BF16 tile by
 *    tile; the router is softmax -> top-k -> normalise; a shared expert is
 *    added after the routed sum; the result is [tokens, hidden] fp32.
 *  - "spark_model/layers/nemotron_moe.rs", module documentation: expert
 *    dispatch stays on the device, with no device-to-host synchronisation; the
 *    layer constructor rejects a top-k outside 1..E.
 *  - "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter PR #5988):
 *    tokens sorted by expert with an inverse route map, a grouped producer
 *    for gate/up + SiLU + down, an FP32 route reduction, one shared expert,
 *    caller-provided output buffers and graph replay.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    the `shared` descriptor struct itself, which is read on the host during
 *    the call (its members are device pointers).  Nothing is allocated,
 *    freed, synchronised or read back by the library: every call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns, so calls can be captured into a HIP graph.
 *  - Arrays are dense and row-major (last index contiguous).
 *  - Route r of token t, slot j, is r = t*k + j.
 *  - Return value: MOE_OK, or a negative moe_status; on failure nothing has
 *    been enqueued and moe_last_error() describes the reason.
 *  - Data faults found on the device (an expert id outside [0, E), a
 *    non-finite router logit) do not stop the kernels: they OR a bit into
 *    `*status` when `status` is not NULL (the caller zeroes it), and the
 *    faulty route is dropped from the sort and from the sum.
 *  - Calls on different streams must use different workspaces.
 */
#ifndef MOE_W8A16_H
#define MOE_W8A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad argument: NULL pointer, size or workspace */
    MOE_EUNSUPPORTED = -2,  /* valid but unsupported geometry (e.g. H % 128) */
    MOE_EHIP = -3           /* the HIP runtime refused a launch */
} moe_status;

enum {
    MOE_STATUS_BAD_EXPERT_ID = 1,   /* an id outside [0, E) was dropped */
    MOE_STATUS_NONFINITE_LOGIT = 2  /* a router logit was NaN or +-inf */
};

enum {
    MOE_MAX_EXPERTS = 1024,  /* E */
    MOE_MAX_TOPK = 16        /* k */
};

enum {
    MOE_VARIANT_AUTO = 0,     /* decode for T*k <= 16E and T*k <= 4096, else prefill */
    MOE_VARIANT_DECODE = 1,   /* weight-streaming kernels: one workgroup per active expert
                                 (or per 16/32-row tile of its routes past 4096 routes), or per
                                 (expert, N tile) with few active experts */
    MOE_VARIANT_PREFILL = 2,  /* grouped bf16-MFMA GEMM over 128-row tiles of sorted routes */
    MOE_VARIANT_PREFILL_A8 = 3, /* the prefill GEMMs with x quantised to E4M3 per token (as
                                   moe_quant_e4m3_rows) for the gate/up (or up) GEMM on the
                                   FP8 MFMA; the down GEMM as PREFILL; never chosen by AUTO */
    MOE_VARIANT_PREFILL_A4 = 4, /* MXFP4 weights only (moe_fused_mxfp4): the prefill GEMMs with
                                   x quantised to MXFP4 (as moe_quant_mxfp4_rows) for the
                                   gate/up (or up) GEMM as E2M1 x E2M1 products on the scaled
                                   MFMA; the down GEMM as PREFILL; never chosen by AUTO */
    MOE_VARIANT_PREFILL_FP4 = 5 /* MXFP4 weights only: PREFILL_A4, and the hidden activation
                                   (rounded to bf16) quantised to MXFP4 by the same rule in the
                                   gate/up epilogue, so that the down GEMM also runs E2M1 x
                                   E2M1; never chosen by AUTO */
};

enum {
    MOE_ACT_SWIGLU = 0,  /* silu(gate) * up; w13 = [gate; up] rows, [2I, H] per expert */
    MOE_ACT_RELU2 = 1    /* relu(up)^2, non-gated experts; w13 = up rows only, [I, H] */
};

enum {
    MOE_LAYOUT_ROWMAJOR = 0,  /* FP8 weights as [rows, K], K contiguous */
    MOE_LAYOUT_TILED = 1      /* tile-coalesced, see moe_pack_w8 */
};

/* Message describing the most recent failure on the calling thread ("" if none).
 * Interface plumbing, not from the pages: a thread-local buffer owned by the
 * library, valid until the thread's next call into it; never NULL. */
const char* moe_last_error(void);

/*
 * moe_route -- router: softmax over E experts, top-k, renormalised affinities.
 * Source: NKI page above, section "FP8 MoE decode kernel", Serving contract
 * ("softmax -> top-8 -> norm").
 *   logits  [T, E] fp32                (in)
 *   ids     [T, k] int32               (out) slot j = the j-th largest logit;
 *                                       equal logits go to the lower expert
 *                                       index and -0.0 equals +0.0
 *   aff     [T, k] fp32                (out) p_j / sum of the k selected p
 *   status  int32 or NULL              (in/out) MOE_STATUS_NONFINITE_LOGIT
 * Requires 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS, T >= 0.
 * T == 0 is a successful no-op.
 */
int moe_route(const float* logits, int T, int E, int k,
              int32_t* ids, float* aff, int32_t* status, void* stream);

/*
 * moe_route_sigmoid -- sigmoid top-k routing with a routed scaling factor.
 * Source: "spark_model/layers/nemotron_moe.rs", module documentation and
 * prefill forward: the gate logits go through sigmoid top-K routing, and the
 * routed experts' weighted sum is scaled by the routed scaling factor of the
 * model configuration.
 *   logits    [T, E] fp32                                         (in)
 *   normalize 0: aff = scale * sigma(l_j), sigma(l) = 1 / (1 + exp(-l));
 *             1: aff = scale * sigma(l_j) / (sum of the k kept sigma)
 *   scale     routed scaling factor, finite; folded into aff, so the expert
 *             sum of moe_fused_w8a16 carries it
 *   ids       [T, k] int32 (out): the k largest logits, ordered and tied as
 *             in moe_route (sigma is strictly increasing, so these are the
 *             k largest sigmoid scores)
 *   aff       [T, k] fp32 (out); status as for moe_route.
 * Requires the moe_route conditions, normalize in {0, 1} and a finite scale
 * (else MOE_EINVAL).  T == 0 is a no-op.
 */
int moe_route_sigmoid(const float* logits, int T, int E, int k, int normalize, float scale,
                      int32_t* ids, float* aff, int32_t* status, void* stream);

/*
 * moe_route_proj -- router projection followed by the router:
 *     logits[t][e] = sum_h x[t][h] * wg[e][h]   (bf16 x bf16 products, fp32 sums)
 * then exactly what moe_route computes on those fp32 logits.
 * Sources: "spark_model/layers/nemotron_moe.rs", prefill forward (a batched
 * gate GEMM [N, H] x [H, E]^T -> [N, E] feeds the top-K routing); "NKI
 * Library Supported Kernel Reference", Router Top-K (router logits and top-K
 * selection in one kernel).
 *   x       [T, H] bf16 (raw 16-bit patterns), 16-byte aligned      (in)
 *   wg      [E, H] bf16 gate weights, 16-byte aligned               (in)
 *   logits  [T, E] fp32, or NULL when not wanted                     (out)
 *   ids, aff, status: as for moe_route                               (out)
 *   ws, ws_bytes: device scratch of moe_route_proj_workspace_bytes(T, H, E)
 *           bytes; it may be NULL/0 when that shape runs as one K slice
 *           and logits is given (the workspace function still returns the
 *           size to pass in general).
 * H must be a positive multiple of 64 (else MOE_EUNSUPPORTED); T, E and k as
 * for moe_route; T == 0 is a no-op.  The sum over h is split into at most 8
 * consecutive K slices whose partial sums are added in slice order, so the
 * logits are the same from call to call.
 */
size_t moe_route_proj_workspace_bytes(int T, int H, int E);
int moe_route_proj(const void* x, const void* wg, int T, int H, int E, int k, float* logits,
                   int32_t* ids, float* aff, int32_t* status, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * moe_sort_workspace_bytes -- device scratch that moe_sort needs for (T, k, E);
 * interface plumbing, not from the pages.  0 for invalid sizes (T < 0, k < 1,
 * E < 1) or when no scratch is needed.
 *
 * moe_sort -- per-expert histogram, exclusive scan, stable sorted route map
 * and its inverse.  Sources: nemotron_moe.rs page (sort by expert before the
 * grouped GEMM, unpermute-reduce after); AITER PR page (sorting and inverse
 * route map).
 *   ids          [T*k] int32   (in)
 *   counts       [E]   int32   (out) routes per expert
 *   offsets      [E+1] int32   (out) exclusive scan of counts; offsets[E] =
 *                               number of valid routes (no padding)
 *   sorted_route [T*k] int32   (out) expert-major, ascending r inside an
 *                               expert; entries past offsets[E] are -1
 *   inv_route    [T*k] int32   (out) position of route r in sorted_route,
 *                               -1 for a dropped route
 *   status       int32 or NULL (in/out) MOE_STATUS_BAD_EXPERT_ID
 *   ws, ws_bytes: device scratch of at least moe_sort_workspace_bytes(T,k,E).
 */
size_t moe_sort_workspace_bytes(int T, int k, int E);
int moe_sort(const int32_t* ids, int T, int k, int E,
             int32_t* counts, int32_t* offsets,
             int32_t* sorted_route, int32_t* inv_route,
             int32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_pack_w8 -- offline weight preparation: reorder FP8 weight bytes into the
 * tile-coalesced layout the decode kernels stream.  Source: NKI page, file
 * table (moe_w8.py: offline weight prep that packs coalesced operands).
 * For each of n_mats matrices W[rows, cols] (row-major, rows % 16 == 0,
 * cols % 64 == 0) the packed matrix P holds, for tile t < rows/16, chunk
 * c < cols/64, lane l < 64 and byte b < 16,
 *     P[((t * (cols/64) + c) * 64 + l) * 16 + b] = W[16t + l%16][64c + 16(l/16) + b],
 * so one wave's 16-byte-per-lane load of a tile chunk is one contiguous 1 KB.
 * The byte count and the block scales are unchanged.  src and dst are device
 * pointers of n_mats*rows*cols bytes each and must not overlap.
 */
int moe_pack_w8(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                void* stream);

/* One expert's block-scaled FP8 weights (same H and I as the routed experts). */
typedef struct {
    const uint8_t* w13;        /* [2I, H] E4M3FN: rows 0..I-1 gate, I..2I-1 up (relu^2: [I, H] up) */
    const float* w13_scale;    /* [2I/128, H/128] fp32 (relu^2: [I/128, H/128]) */
    const uint8_t* w2;         /* [H, I] E4M3FN */
    const float* w2_scale;     /* [H/128, I/128] fp32 */
} moe_expert_w8;

/*
 * moe_fused_w8a16 -- sort + routed expert FFN + affinity-weighted fp32 sum
 * (+ optional always-on shared expert with affinity 1.0).
 * Sources: NKI page, section "FP8 MoE decode kernel" (fused path, weight
 * format, fp32 [B, H] result, shared expert added after the routed sum);
 * AITER PR page (sorted routes, fp32 route reduction, one shared expert).
 *   x          [T, H] bf16 (raw 16-bit patterns)                   (in)
 *   w13        [E, 2I, H] E4M3FN bytes, w13_scale [E, 2I/128, H/128] fp32
 *   w2         [E, H, I]  E4M3FN bytes, w2_scale  [E, H/128, I/128]  fp32
 *              weight value = E4M3FN(code) * scale of its 128x128 block
 *   ids, aff   [T, k] int32 / fp32 (e.g. from moe_route)            (in)
 *   shared     host pointer to a moe_expert_w8, or NULL for none    (in)
 *   out        [T, H] fp32, overwritten (must not alias x)          (out)
 *   status     int32 or NULL                                        (in/out)
 *   ws         device scratch of moe_fused_workspace_bytes(...) bytes
 *   weight_layout  MOE_LAYOUT_ROWMAJOR or MOE_LAYOUT_TILED (moe_pack_w8
 *              output); applies to w13, w2 and the shared expert alike
 *   variant    MOE_VARIANT_*
 * H and I must be multiples of 128 (else MOE_EUNSUPPORTED); T >= 0; T == 0
 * is a no-op.  MOE_VARIANT_PREFILL_A4 and MOE_VARIANT_PREFILL_FP4 take MXFP4
 * weights only and give MOE_EUNSUPPORTED here (and in the _ex and _noalloc
 * forms).
 * MOE_VARIANT_PREFILL also needs H and 2I to be multiples of
 * 256 (else MOE_EUNSUPPORTED); MOE_VARIANT_AUTO picks the decode variant for
 * such shapes and for batches of at most 16 routes per expert and 4096 routes
 * in all, the prefill variant otherwise.  The expert FFN computes in bf16 x
 * bf16 products with fp32 accumulation; the SwiGLU output is rounded to bf16
 * before the down GEMM.
 * Block scales: any finite fp32 value (zero, subnormal or negative included;
 * NaN and infinity are out of contract).  Each 128-wide K block is weighted
 * by its own scale: a zero-scale block adds exactly 0 whatever its codes.
 * The decode variant multiplies each block's fp32 partial sum by its scale.
 * The prefill variants fold the scale's power of two exactly into the bf16
 * (or fp8) weight operand and apply its mantissa to the fp32 accumulators;
 * this is exact while a block's scale is at most 2^117 below the largest
 * scale of its 128-row scale row, and beyond that the block's smallest
 * codes are flushed to zero.
 * Alignment: x, w13, w2, out, ws and the shared expert's w13 and w2 must be
 * 16-byte aligned; the scales, ids and aff 4-byte aligned (else MOE_EINVAL).
 */
/* MOE_VARIANT_PREFILL_A8 computes every expert from x_hat[t] = decode(code) * scale
 * of moe_quant_e4m3_rows instead of x[t] (gate/up on fp8 x fp8 products, exact
 * in fp32, with fp32 sums); the rest of the path is that of MOE_VARIANT_PREFILL,
 * with the same shape rules.  Its workspace holds the codes and scales too.
 *
 * moe_fused_workspace_bytes -- device scratch of a moe_fused_w8a16(_ex) call
 * with these sizes and this variant (interface plumbing, not from the pages):
 * the sort maps, the row-tile list, the activations between the GEMMs and
 * one contribution row per route (fp32 for the decode variant, 2.125 bytes a
 * value for the prefill ones; AUTO is sized for either).  0 for invalid
 * sizes.  A call checks ws_bytes against the size of the variant it runs. */
size_t moe_fused_workspace_bytes(int T, int H, int I, int E, int k,
                                 int has_shared, int variant);
int moe_fused_w8a16(const void* x,
                    const uint8_t* w13, const float* w13_scale,
                    const uint8_t* w2, const float* w2_scale,
                    const int32_t* ids, const float* aff,
                    int T, int H, int I, int E, int k,
                    const moe_expert_w8* shared, float* out,
                    int32_t* status, void* ws, size_t ws_bytes,
                    int weight_layout, int variant, void* stream);

/*
 * moe_fused_w8a16_ex -- moe_fused_w8a16 with a choice of expert activation.
 * Source for MOE_ACT_RELU2: "spark_model/layers/nemotron_moe.rs", module
 * documentation: the routed experts run an up projection, then a fused
 * relu^2 + down projection, and the shared expert runs up + relu^2 + down.
 *   activation MOE_ACT_SWIGLU: exactly moe_fused_w8a16.
 *              MOE_ACT_RELU2: expert e computes y = W2[e] relu(W1[e] x)^2 with
 *              w13 [E, I, H] holding W1 (and w13_scale [E, I/128, H/128]); the
 *              shared expert's w13 is [I, H] likewise.  The relu^2 output is
 *              rounded to bf16 before the down GEMM, as the SwiGLU output is.
 *              The prefill variant then needs I % 256 == 0 instead of 2I % 256.
 * Every other argument, the workspace size and the error behaviour are those
 * of moe_fused_w8a16; an unknown activation gives MOE_EINVAL.
 */
int moe_fused_w8a16_ex(const void* x,
                       const uint8_t* w13, const float* w13_scale,
                       const uint8_t* w2, const float* w2_scale,
                       const int32_t* ids, const float* aff,
                       int T, int H, int I, int E, int k,
                       const moe_expert_w8* shared, float* out,
                       int32_t* status, void* ws, size_t ws_bytes,
                       int weight_layout, int variant, int activation, void* stream);

/*
 * moe_fused_w8a16_noalloc -- moe_fused_w8a16_ex for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same call, kernels and results, with
 * no workspace argument.  Its workspace is one device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library; each GPU it runs on holds its
 * own copy from the first call on that device until the process ends.
 *   Every argument means what it means for moe_fused_w8a16_ex; the call runs
 *   on the current device, and `stream` must belong to it.
 *   A call whose workspace (moe_fused_workspace_bytes of the variant it runs;
 *   AUTO resolved as moe_fused_w8a16 resolves it) exceeds the array returns
 *   MOE_EUNSUPPORTED before anything is enqueued, with moe_last_error()
 *   saying so.  The array keeps the last call's contents; nothing in it needs
 *   to start at zero.  Calls on one GPU share the array, so calls that
 *   overlap on one GPU (other streams, or other threads) race: serialise
 *   them.  Nothing is allocated or freed: not by this call, its kernels or
 *   the library routines it uses.  At 64 MiB the array fits, for example,
 *   the decode variant at T = 512, H = 2048, I = 512, E = 256, k = 8.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_fused_w8a16_noalloc(const void* x,
                            const uint8_t* w13, const float* w13_scale,
                            const uint8_t* w2, const float* w2_scale,
                            const int32_t* ids, const float* aff,
                            int T, int H, int I, int E, int k,
                            const moe_expert_w8* shared, float* out,
                            int32_t* status, int weight_layout, int variant, int activation,
                            void* stream);

/*
 * moe_pack_mx_scales -- offline preparation of MXFP4 scales for
 * MOE_LAYOUT_TILED (interface plumbing for the tiled layout, not from the
 * pages): for each of n_mats matrices S[rows, cols] of E8M0 bytes (cols =
 * K/32; rows % 16 == 0, cols % 4 == 0) the packed matrix P holds, for tile
 * t < rows/16, chunk c < cols/4 and lane l < 64,
 *     P[(t * (cols/4) + c) * 64 + l] = S[16t + l%16][4c + l/16],
 * so that one wave's scale bytes of a 16-row, 128-element chunk are one
 * 64-byte line.  src and dst are device pointers of n_mats*rows*cols bytes
 * and must not overlap.
 */
int moe_pack_mx_scales(const uint8_t* src, uint8_t* dst, int64_t n_mats, int rows, int cols,
                       void* stream);

/* One expert's MXFP4 weights (same H and I as the routed experts). */
typedef struct {
    const uint8_t* w13;        /* [2I, H/2] E2M1 codes two a byte (relu^2: [I, H/2]) */
    const uint8_t* w13_scale;  /* [2I, H/32] E8M0 (relu^2: [I, H/32]) */
    const uint8_t* w2;         /* [H, I/2] */
    const uint8_t* w2_scale;   /* [H, I/32] */
} moe_expert_mx4;

/*
 * moe_fused_mxfp4 -- moe_fused_w8a16_ex with MXFP4 expert weights (W4A16).
 * Sources: "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter
 * PR #5988), description: the experts' weights are MXFP4; "NKI Library
 * Supported Kernel Reference", Blockwise MM Block MX (MXFP4/MXFP8 MoE).  The
 * pages do not spell the encoding out; the OCP Microscaling definition is
 * taken: each element an E2M1 code (1 sign, 2 exponent bits with bias 1,
 * 1 mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), each run of 32
 * consecutive elements of a row sharing one E8M0 scale byte s (2^(s - 127);
 * 255 = NaN is out of contract).
 *   w13        [E, 2I, H/2] bytes: element 2j of a row in the low nibble of
 *              byte j, element 2j+1 in its high nibble (relu^2: [E, I, H/2])
 *   w13_scale  [E, 2I, H/32] E8M0 bytes (relu^2: [E, I, H/32])
 *   w2         [E, H, I/2], w2_scale [E, H, I/32], likewise
 *              weight value = E2M1(code) * 2^(scale - 127)
 *   shared     host pointer to a moe_expert_mx4, or NULL
 *   weight_layout  MOE_LAYOUT_TILED: the code bytes packed by moe_pack_w8
 *              (rows, cols = K/2) and the scales by moe_pack_mx_scales
 *              (rows, cols = K/32); MOE_LAYOUT_ROWMAJOR: both as above
 * Everything else as moe_fused_w8a16_ex, including the workspace
 * (moe_fused_workspace_bytes with the same variant) and AUTO's choice:
 *   MOE_VARIANT_DECODE   the weight-streaming kernel (one workgroup per
 *              active expert up to 4096 routes, above that one per 16- or
 *              32-row tile of an expert's sorted routes); shapes whose
 *              activation pass does not fit 64 KB of LDS (16 or 32 *
 *              (I + 8) * 2 bytes, plus 4 bytes a route when T*k <= 4096) or
 *              with T*H >= 2^32 give MOE_EUNSUPPORTED
 *   MOE_VARIANT_PREFILL  the grouped GEMMs (same shape limits as the E4M3FN
 *              weights); the E8M0 arrays (routed and shared) must then be
 *              4-byte aligned, else MOE_EINVAL -- AUTO takes the decode
 *              kernels for unaligned scale arrays instead
 *   MOE_VARIANT_PREFILL_A8  likewise, with x quantised to E4M3 per token as
 *              for E4M3FN weights; the gate/up (relu^2: up) GEMM multiplies
 *              E4M3 by E2M1 codes on the scaled FP8 MFMA, each 32-element
 *              block's E8M0 byte as the MFMA's weight scale, and the down
 *              GEMM stays bf16 x MXFP4
 *   MOE_VARIANT_PREFILL_A4  likewise, with x quantised to MXFP4 as
 *              moe_quant_mxfp4_rows does ("Add gfx950 Q256 fused MXFP4
 *              prefill pipeline", description: the producer quantises the
 *              activations and the GEMMs run in MXFP4); gate/up as E2M1 x
 *              E2M1 products with both operands' E8M0 bytes as the MFMA's
 *              scales; every expert then computes from x_hat of
 *              moe_quant_mxfp4_rows instead of x (the SwiGLU output stays
 *              bf16, the down GEMM bf16 x MXFP4); the workspace also holds
 *              the codes and scales of x.  A token whose row holds a NaN or
 *              an infinity gets a NaN output row.
 *   MOE_VARIANT_PREFILL_FP4  PREFILL_A4, and the hidden activation (the
 *              SwiGLU or relu^2 output, rounded to bf16) quantised to MXFP4
 *              by the same rule in the gate/up (up) epilogue (same page:
 *              the producer quantises the hidden activation in registers and
 *              runs the down projection in MXFP4), so the down GEMM also
 *              multiplies E2M1 by E2M1 with both E8M0 bytes as the MFMA's
 *              scales.  The quantisation decision is taken from the fp32
 *              sums, so a hidden element within a rounding error of an E2M1
 *              midpoint (or of a power of two that sets its run's exponent)
 *              may land on either neighbour.  A run of 32 hidden values
 *              holding a NaN or an infinity gives NaN outputs for its token.
 * The E8M0 scale is applied exactly in the conversion to bf16 (every E2M1
 * value times a power of two is a bf16 value while it stays in bf16's normal
 * range; smaller products are flushed to zero), products are summed in fp32
 * and the SwiGLU output is rounded to bf16 before the down GEMM.
 */
int moe_fused_mxfp4(const void* x,
                    const uint8_t* w13, const uint8_t* w13_scale,
                    const uint8_t* w2, const uint8_t* w2_scale,
                    const int32_t* ids, const float* aff,
                    int T, int H, int I, int E, int k,
                    const moe_expert_mx4* shared, float* out,
                    int32_t* status, void* ws, size_t ws_bytes,
                    int weight_layout, int variant, int activation, void* stream);

/*
 * moe_quant_e4m3_rows -- the per-token activation quantisation that
 * MOE_VARIANT_PREFILL_A8 applies to x, exposed so it can be checked on its
 * own.  For each row t:
 *     scales[t] = max_h |x[t][h]| / 448                    (fp32, correctly rounded)
 *     codes[t][h] = E4M3FN round-half-even of min(max(x[t][h] / scales[t], -448), 448)
 * with the quotient in fp32; a row of zeros gets scale 0 and zero codes, a row
 * holding a NaN or an infinity a NaN scale and zero codes.  The
 * value the GEMM then uses is decode(code) * scale.  Source of the format and
 * of the amax / 448 rule: NKI page, section "FP8 MoE decode kernel" (official
 * E4M3FN weights, block scale = block maximum / 448), applied per token row.
 *   x [T, H] bf16 (16-byte aligned), codes [T, H] uint8 (8-byte aligned),
 *   scales [T] fp32; H % 8 == 0 (else MOE_EINVAL); T == 0 is a no-op.
 */
int moe_quant_e4m3_rows(const void* x, int T, int H, uint8_t* codes, float* scales,
                        void* stream);

/*
 * moe_quant_mxfp4_rows -- the MXFP4 quantisation of x that
 * MOE_VARIANT_PREFILL_A4 applies, exposed so it can be checked on its own.
 * Source: "Add gfx950 Q256 fused MXFP4 prefill pipeline" (description: the
 * producer quantises the activations to MXFP4); the pages give no rule, and
 * the OCP Microscaling one is taken (as for the MXFP4 weights).  For each run
 * of 32 consecutive elements of a row:
 *     X = floor(log2 max |x|) - 2, clamped to [-127, 127] (an all-zero run:
 *         -127), so the run's largest magnitude maps into [4, 8);
 *     scales[t][r] = X + 127 (E8M0);
 *     code = the E2M1 value nearest to |x| / 2^X (a tie to the even code,
 *         magnitudes above 6 saturating to 6) with the sign bit of x.
 * Every step is exact for bf16 inputs.  A run holding a NaN or an infinity
 * gets the E8M0 NaN byte 255 and zero codes.  The value the GEMM uses is
 * E2M1(code) * 2^(scale - 127).
 *   x [T, H] bf16 (16-byte aligned), codes [T, H/2] uint8 (two a byte,
 *   element 2j in the low nibble of byte j; 16-byte aligned), scales
 *   [T, H/32] uint8; H % 32 == 0 (else MOE_EINVAL); T == 0 is a no-op.
 */
int moe_quant_mxfp4_rows(const void* x, int T, int H, uint8_t* codes, uint8_t* scales,
                         void* stream);

/*
 * moe_decode_e4m3fn -- decode n E4M3FN bytes to bf16 bit patterns with the
 * same on-chip conversion the FFN kernels use (scale 1, exact: every finite
 * E4M3FN value is a bf16 value).  Exposed so the decode step can be checked
 * on its own.  Source: NKI page, file table ("decode official E4M3FN").
 *   codes [n] uint8 (in), out [n] uint16 (out); n >= 0.
 */
int moe_decode_e4m3fn(const uint8_t* codes, uint16_t* out, int64_t n, void* stream);

/*
 * Per-kernel timing, for measurement only (not from the pages).  While
 * enabled, every kernel the library launches is bracketed by two HIP timing
 * events recorded on that kernel's own stream.  moe_profile_collect() waits
 * on the host for the recorded events and folds their elapsed times into
 * per-kernel statistics, so it must not be called under graph capture, and
 * profiling must be off while a graph is being captured.
 *   moe_profile_enable(1) clears the statistics and starts recording;
 *   moe_profile_enable(0) stops recording (statistics are kept).
 *   moe_profile_stat(i, ...) reports kernel i < moe_profile_count(): its name
 *   (NUL-terminated, truncated to name_len), launches and total milliseconds.
 * All return MOE_OK or a negative moe_status (MOE_EHIP if an event call
 * fails, MOE_EINVAL for a bad index or NULL output).
 */
int moe_profile_enable(int on);
int moe_profile_collect(void);
int moe_profile_count(void);
int moe_profile_stat(int i, char* name, int name_len, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W8A16_H */
