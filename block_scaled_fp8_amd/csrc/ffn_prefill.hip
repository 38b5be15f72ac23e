// Prefill variant of the expert FFN: grouped bf16-MFMA GEMMs over 128-row
// tiles of the expert-sorted routes.
//
// Sources: "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter
// PR #5988): a prefill producer over expert-sorted tokens does the gate/up
// projection, SiLU and down projection, then an FP32 route reduction sums the
// routed contributions (one always-on shared expert included);
// "spark_model/layers/nemotron_moe.rs": the sorted prefill path runs one
// grouped GEMM per projection over tokens sorted by expert and unpermutes with
// a reduction.  The weights stay block-scaled E4M3FN ("Gated DeltaNet (+ FP8
// MoE) -- AWS Neuron (NKI) kernels for Trainium2", FP8 MoE decode kernel
// section) and are decoded to bf16 on chip.
//
// gfx950 design.  Kernel 1 (gate/up): each workgroup computes a 128-row x
// (128 gate + 128 up) tile of one segment, applies SwiGLU in registers and
// writes bf16 activations (abuf, sorted row order).  Kernel 2 (down): each
// workgroup computes a 128-row x 256-column tile of y = a W2^T and writes its
// rows at their sorted position (a tile's rows are contiguous) in a block
// floating-point form (8 values share an exponent byte, 16-bit mantissas:
// common.hpp, bfp16x8_encode); the final combine
// gathers the k rows of a token through the inverse route map, widens them
// and applies the affinities in fp32.
//
//  * Workgroup tile 128 rows x 256 columns (gate/up: 128 gate + the matching
//    128 up columns), 4 waves (2 x 2), each a 64 x 128 tile with 128 fp32
//    accumulators: gate/up as 4 x 8 tiles of v_mfma_f32_16x16x32_bf16, down
//    as 2 x 4 tiles of v_mfma_f32_32x32x16_bf16.
//    Two workgroups share a CU (64 KB of stages each, 2 waves per SIMD), so
//    one workgroup's prologue, epilogue and barrier waits overlap the other's
//    MFMAs; measured, this beats one 8-wave 128 x 512 workgroup per CU.
//  * Operands are staged through LDS with 16-byte direct-to-LDS loads
//    (global_load_lds_dwordx4: a wave instruction fills one contiguous 1 KB),
//    two stages of 64-wide K, one barrier per K step; the next step's loads
//    are in flight while a step is multiplied, and the LDS reads of the next
//    half step overlap the MFMAs of the current one.
//  * Activation tiles: 8 rows x 128 bytes per wave instruction, the 16-byte
//    pieces of each row XOR-swizzled by (row / 2) % 8, so that the 16 rows read
//    by one 16-lane phase of ds_read_b128 cover all 64 LDS banks.
//    Weight tiles: one 16-row x 64-byte chunk per instruction, stored in lane
//    order (the tile-coalesced layout is this chunk order in memory).
//  * FP8 is converted exactly to bf16 after the LDS read; the fp32 block scale
//    of each 128-wide K block is never rounded into bf16: its power of two is
//    folded exactly into the conversion, and its mantissa is applied by
//    rescaling the accumulators when the block starts (running scale); a
//    zero-scale block's MFMAs are skipped.
//  * Work list: the sort lists every full 128-row tile first and the partial
//    last tiles after them; the list is cut into runs of 8 row tiles dealt
//    round-robin to the 8 XCDs (all column blocks of a row tile on one XCD,
//    so consecutive tiles of one expert share its weights in L2), and the
//    last round of workgroups holds the cheap partial tiles, whose empty
//    MFMA row groups (16 rows gate/up, 32 down) are skipped.  The grid covers
//    the worst case and idle workgroups exit.
//  * Epilogue: gate/up applies SwiGLU (up: relu^2) and down encodes its
//    contributions; both turn the accumulators into row pieces through LDS
//    so that a lane stores 16 contiguous bytes of a row.
//  * MXFP4 weights ("Add gfx950 Q256 fused MXFP4 prefill pipeline": E2M1
//    codes with an E8M0 scale per 32 elements of a row) run the same
//    kernels on 32x32 tiles: a stage holds 32 code bytes a weight row and
//    the scale bytes of its 128-wide K chunk; each lane's 16 code bytes of a
//    step are exactly one scale block, whose power of two the bf16
//    conversion applies, so no running scale is needed.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "plan.hpp"
#include "mxfp4_act.hpp"

namespace moe {

constexpr int PF_BK = 64;  // K per stage
constexpr int PF_XCD_RUN = 8;  // consecutive row tiles an XCD takes at a time

// Workgroup tile BM rows x BN columns, WM x WN waves of 64 x 128 each (2 x 4
// MFMA tiles of 32 x 32), STAGES LDS stages of 64-wide K, OCC workgroups per
// CU (the register budget follows from it).
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int OCC_, int M16_ = 0, int A8_ = 0,
          int MX4_ = 0, int A4_ = 0, int H4_ = 0>
struct PfCfg {
    static constexpr int OCC = OCC_;
    // MFMA shape: v_mfma_f32_16x16x32_bf16 (M16) or v_mfma_f32_32x32x16_bf16;
    // A8: the activation operand is E4M3 (per-token scale) and the product
    // runs on v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales, fp8 x fp8
    static constexpr bool M16 = M16_ != 0;
    static constexpr bool A8 = A8_ != 0;
    static_assert(!(M16 && A8), "the fp8 path uses 32x32 tiles");
    // MX4: MXFP4 weights (E2M1 codes, two a byte, one E8M0 scale per 32
    // elements of a row); a stage holds 32 code bytes of each weight row and
    // the scale bytes of the 128-wide K chunk the step lies in.  With A8 the
    // product is E4M3 x E2M1 on the scaled MFMA, the lane's E8M0 byte its B
    // scale.
    static constexpr bool MX4 = MX4_ != 0;
    static_assert(!(MX4 && M16), "MXFP4 weights use 32x32 tiles");
    // A4 (with A8 and MX4): the activation operand is MXFP4 too (E2M1 codes,
    // 32 bytes a row per stage), E2M1 x E2M1 on the scaled MFMA with per-lane
    // scales on both sides.  A4_ = 1: each stage also stages its rows' E8M0
    // bytes of the 128-K chunk; A4_ = 2 (XT): the tile's rows' E8M0 bytes
    // for all of K are staged once, in a table after the stages
    static constexpr bool A4 = A4_ != 0;
    static constexpr bool XT = A4_ == 2;
    static_assert(!A4 || (A8 && MX4), "MXFP4 activations pair with MXFP4 weights");
    // H4 (gate/up and up, with A4): the hidden activation leaves as MXFP4,
    // E2M1 codes [rows][I/2] and E8M0 bytes [rows][I/32], for a down GEMM
    // that takes MXFP4 activations (A4 with MODE PF_DOWN)
    static constexpr bool H4 = H4_ != 0;
    static_assert(!H4 || A4, "the MXFP4 hidden activation belongs to the MXFP4 pipeline");
    static constexpr int MS = M16 ? 16 : 32;  // rows = columns of one MFMA tile
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int THREADS = WM * WN * MOE_WAVE;
    static constexpr int WAVES = WM * WN;
    static constexpr int STAGES = STAGES_;
    static constexpr int A_BYTES = A4 ? BM * PF_BK / 2 : BM * PF_BK * (A8 ? 1 : 2);  // bf16, E4M3 or E2M1
    static constexpr int B_BYTES = BN * PF_BK / (MX4 ? 2 : 1);  // fp8 or E2M1
    static constexpr int TB = MX4 ? 512 : 1024;    // bytes of a 16-row weight tile per stage
    static constexpr int S_BYTES = MX4 ? BN * 4 : 0;  // E8M0: 4 scale bytes a row
    static constexpr int SA_BYTES = A4 && !XT ? WAVES * 256 : 0;  // 4 scale bytes a row (staged twice with 4 waves)
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES + SA_BYTES;
    static constexpr int A_INSTR = A_BYTES / 1024 / WAVES;  // 1 KB loads per wave per stage
    static constexpr int B_INSTR = B_BYTES / 1024 / WAVES;
    static constexpr int S_INSTR = (MX4 ? 1 : 0) + (A4 && !XT ? 1 : 0);  // 256-byte scale loads per wave per stage
    static_assert(!MX4 || S_BYTES == WAVES * 256, "each wave stages the scales of 64 rows");
    static_assert(!A4 || WAVES * 64 >= BM, "the activation rows' scales fit one load a wave");
    static constexpr int MT = BM / WM / MS;
    static constexpr int NT = BN / WN / MS;
    static constexpr int WROWS = BM / WM;  // rows of a wave tile
    static constexpr int WCOLS = BN / WN;  // columns of a wave tile
    // 64 x 128, 128 fp32 accumulators per lane: the running-scale rescale
    // needs them in architectural VGPRs beside the operand fragments, so a
    // 128 x 128 wave tile does not fit; 128 x 64 (each weight converted by one
    // wave instead of two, activations read twice as often) measured slower.
    // Gate/up: a wave's columns are 64 gate and the matching 64 up columns,
    // each half inside one 128-column scale block.
    static_assert(WROWS == 64 && WCOLS == 128, "wave tile is 64 x 128");
    static_assert(BM == 128, "tile prefixes are built for 128-row tiles");
    static_assert(A_INSTR >= 1 && B_INSTR >= 1, "every wave issues loads");
};
// 4 waves and 64 KB of stages: two workgroups share a CU, so one's prologue,
// epilogue and barrier waits overlap the other's MFMAs.  Gate/up multiplies
// with 16x16x32 MFMAs: on random operands the chip holds a higher clock for
// them than for 32x32x16 (register-only loops: 1.94 against 1.71 PFLOP/s),
// and the kernel measured 2.5% faster.  Down keeps 32x32x16 (it measured 4%
// faster when its fp32 rows left the accumulators directly, in 128-byte row
// pieces instead of 64-byte ones; they now pass through LDS).
using PfGateUp = PfCfg<128, 256, 2, 2, 2, 2, 1>;
using PfDown = PfCfg<128, 256, 2, 2, 2, 2, 0>;
using PfGateUpA8 = PfCfg<128, 256, 2, 2, 3, 2, 0, 1>;
// relu^2 up projections whose I is an odd multiple of 128: 128-column tiles
// of two waves (the 256-column tile would run past the matrix)
using PfUpNarrow = PfCfg<128, 128, 2, 1, 2, 2, 1>;
using PfUpNarrowA8 = PfCfg<128, 128, 2, 1, 3, 2, 0, 1>;
// MXFP4 weights: the same tiles on 32x32x16 MFMAs (a lane's 16 code bytes
// of a step are one scale block; with 16x16 tiles the per-half code and scale
// operands spilled registers)
using PfGateUpMx = PfCfg<128, 256, 2, 2, 2, 2, 0, 0, 1>;
using PfDownMx = PfCfg<128, 256, 2, 2, 2, 2, 0, 0, 1>;
using PfUpNarrowMx = PfCfg<128, 128, 2, 1, 2, 2, 0, 0, 1>;
using PfGateUpMxA8 = PfCfg<128, 256, 2, 2, 3, 2, 0, 1, 1>;
using PfUpNarrowMxA8 = PfCfg<128, 128, 2, 1, 3, 2, 0, 1, 1>;
using PfGateUpMxA4 = PfCfg<128, 256, 2, 2, 3, 2, 0, 1, 1, 1>;
using PfUpNarrowMxA4 = PfCfg<128, 128, 2, 1, 3, 2, 0, 1, 1, 1>;
using PfGateUpMxA4T = PfCfg<128, 256, 2, 2, 3, 2, 0, 1, 1, 2>;
using PfUpNarrowMxA4T = PfCfg<128, 128, 2, 1, 3, 2, 0, 1, 1, 2>;
// ... and the hidden activation quantised to MXFP4 in the epilogue, for the
// down GEMM on MXFP4 activations (per-step scales of the hidden rows)
using PfGateUpMxA4H = PfCfg<128, 256, 2, 2, 3, 2, 0, 1, 1, 1, 1>;
using PfUpNarrowMxA4H = PfCfg<128, 128, 2, 1, 3, 2, 0, 1, 1, 1, 1>;
using PfGateUpMxA4TH = PfCfg<128, 256, 2, 2, 3, 2, 0, 1, 1, 2, 1>;
using PfUpNarrowMxA4TH = PfCfg<128, 128, 2, 1, 3, 2, 0, 1, 1, 2, 1>;
using PfDownMxA4 = PfCfg<128, 256, 2, 2, 3, 2, 0, 1, 1, 1>;
// the x-scale table (XT): 128 rows of H/32 bytes, at most 32 KB; a row is a
// power-of-two number of 16-byte pieces (the slot swizzle XORs piece indices)
constexpr int PF_XT_MAX_H = 8192;
static bool prefill_xscale_table(int H) {
    const int pieces = H / 512;
    return H % 512 == 0 && H <= PF_XT_MAX_H && (pieces & (pieces - 1)) == 0;
}
constexpr int PF_BM = 128;

int prefill_tile_m() { return PF_BM; }

// Widths the grouped GEMMs tile exactly (K % 128 holds for every valid call);
// the per-tile scale table (2 rows of K / 128 floats, padded to 64) must fit
// in LDS beside the stages, which holds for K <= 65536.  Down tiles H in
// 256-column blocks; relu^2 experts tile their I up columns in 256-column
// blocks, or 128-column ones when I is an odd multiple of 128.
int prefill_supported(int H, int I, int act) {
    const int ncols = act == ACT_RELU2 ? I : 2 * I;
    return H % 256 == 0 && ncols % 128 == 0 && (act == ACT_RELU2 || ncols % 256 == 0) && H <= 65536 &&
           I <= 65536;
}

// PF_GATEUP: gate and up columns side by side, SwiGLU epilogue into abuf;
// PF_UP:     the up projection of a non-gated expert, relu^2 epilogue into abuf;
// PF_DOWN:   the down projection, block floating-point rows into ybuf.
enum { PF_GATEUP = 0, PF_DOWN = 1, PF_UP = 2 };

// LDS the epilogue passes a tile's results through (from byte 0; the launch
// gives the kernel at least this much): fp32 32-row slabs of 128 columns a
// wave (down), or the wave's bf16 activation rows.
template <int MODE, class C>
constexpr int pf_epilogue_lds() {
    return MODE == PF_DOWN ? C::WAVES * 32 * 128 * 4
                           : C::WAVES * C::WROWS * (MODE == PF_GATEUP ? C::WCOLS / 2 : C::WCOLS) * 2;
}

// silu(g) * u with the hardware reciprocal (about 1 ulp) in place of an IEEE
// divide; exp(-g) overflowing to +inf gives the correct limit 0.
__device__ __forceinline__ float swiglu_fast(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Two floats to two bf16 bit patterns (low half: a) by gfx950's packed
// conversion: round to nearest even, as f32_to_bf16_bits, and a NaN stays a
// NaN.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
    typedef float pf_f32x2 __attribute__((ext_vector_type(2)));
    const pf_f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float uniform_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Two 16-byte operand pieces as the 32-byte register operand of the fp8 MFMA.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x8 cat_i32x8(u32x4 a, u32x4 b) {
    const i32x4v ai = __builtin_bit_cast(i32x4v, a), bi = __builtin_bit_cast(i32x4v, b);
    return __builtin_shufflevector(ai, bi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void lds_load16(const void* g, uint32_t lds_byte_addr_uniform, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, reinterpret_cast<char*>(lds_base) + lds_byte_addr_uniform, 16,
                                     0, 0);
}

// s_waitcnt vmcnt(n) (n < 64), leaving the other counters unconstrained.  The
// gfx9 encoding splits vmcnt into bits 3:0 and 15:14; expcnt is bits 6:4 and
// lgkmcnt bits 11:8.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for the K loop.  A __syncthreads() fence would also wait
// for every direct-to-LDS load in flight (they write LDS), which drains the
// prefetch pipeline; here the caller has already waited (vmcnt) for the loads
// other waves will read, and this wave's own LDS reads are waited for before
// the barrier so that a buffer can be refilled after it.  The asm statement
// also keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_after_lds_reads() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

template <int MODE, int LAYOUT, class C>
__global__ __launch_bounds__(C::THREADS, C::OCC) void prefill_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ abuf_in,
    const uint8_t* __restrict__ wexp, const void* __restrict__ sexp,
    const uint8_t* __restrict__ wsh, const void* __restrict__ ssh, Plan plan,
    int T, int H, int I, int k, int nblk, int max_tiles,
    uint16_t* __restrict__ abuf_out, float* __restrict__ ybuf, const void* __restrict__ xscale,
    uint8_t* __restrict__ hscale_out) {
    constexpr int BM = C::BM, BN = C::BN;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ int row_tok[BM];  // gate/up: token row of x
    constexpr bool XS_ROW = C::A8 && !C::A4;  // a per-token fp32 x scale (E4M3 activations)
    __shared__ __attribute__((aligned(16))) float row_xs[XS_ROW ? BM : 1];  // the row's x scale

    // ---- which tile.  Workgroups are dealt round-robin over the 8 XCDs
    //      (id % 8).  The sort's tile list is cut into blocks of PF_XCD_RUN
    //      consecutive row tiles, dealt round-robin to the XCDs; XCD x walks
    //      its blocks in order, each row tile with all its column blocks.  So
    //      every XCD gets an equal share of the full tiles (listed first, to
    //      within one block) before the partial ones (listed last: the last
    //      round of workgroups is the cheapest), while consecutive tiles of
    //      one expert stay on one XCD and share its weights in L2.  (Dealing
    //      the trailing tiles one at a time instead measured slower: the last
    //      full tiles lose that sharing.)  The grid covers the worst case; the
    //      rest exit.
    const int bid = blockIdx.x;
    const int jx = bid >> 3, q = jx / nblk;
    const int tile = (q / PF_XCD_RUN) * (8 * PF_XCD_RUN) + (bid & 7) * PF_XCD_RUN + q % PF_XCD_RUN;
    const int nb = jx - q * nblk;
    // the tile's record is read together with the tile count (one round trip;
    // the index is clamped to the list's capacity, the record then unused)
    const int ntiles = plan.tile_n[0];
    const int4 ti = plan.tile_info[min(tile, max_tiles - 1)];
    if (tile >= ntiles) return;
    const int e = ti.x;          // expert, -1 = shared
    const int p0 = ti.y;         // first sorted row of the tile
    const int rows_here = ti.z;  // rows in the tile (1 .. BM)

    constexpr bool GATHER = MODE != PF_DOWN;   // operand rows gathered from x
    constexpr bool PAIRED = MODE == PF_GATEUP; // gate and up columns side by side
    const int K = GATHER ? H : I;
    const int Nrows = MODE == PF_GATEUP ? 2 * I : (MODE == PF_UP ? I : H);  // weight rows
    // weight rows of KB bytes; scales: fp32 [Nrows/128][K/128] blocks, or
    // (MX4) E8M0 bytes [Nrows][K/32]
    const int KB = C::MX4 ? K / 2 : K;
    const uint8_t* W = e >= 0 ? wexp + (size_t)e * Nrows * KB : wsh;
    const float* S = e >= 0 ? static_cast<const float*>(sexp) + (size_t)e * (Nrows / 128) * (K / 128)
                            : static_cast<const float*>(ssh);
    const uint8_t* SX = e >= 0 ? static_cast<const uint8_t*>(sexp) + (size_t)e * Nrows * (K / 32)
                               : static_cast<const uint8_t*>(ssh);
    const int R = T * k;

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    // Rows of the tile: row m is sorted row p0 + m (m < rows_here); padding
    // rows read a valid row and are never stored.  Gate/up gathers token rows
    // of x through the sorted route map (shared expert: token p - R); down
    // reads the activations at the sorted rows themselves, so its loads need
    // no table.  Both write at the sorted row.
    if (GATHER) {
        if (tid < BM) {
            const int p = p0 + tid;
            const bool valid = tid < rows_here;
            row_tok[tid] = valid ? (e >= 0 ? plan.sorted_route[p] / k : p - R) : 0;
            if constexpr (XS_ROW) row_xs[tid] = valid ? static_cast<const float*>(xscale)[row_tok[tid]] : 0.0f;
        }
        __syncthreads();
    }

    // ---- per-lane global sources of the staged tiles
    // activations: instruction q of wave w fills rows (w*A_INSTR + q)*8 .. +8,
    // 128 B each; the lane's source is a 32-bit byte offset from the matrix
    // (the launcher checks that the matrix is under 4 GB), so the loads
    // address through a scalar base
    // (A8: E4M3 rows of 64 bytes per stage, 16 rows per instruction, pieces
    //  swizzled by (row / 4) % 4 so that the MFMA reads of 8 rows fall on
    //  distinct banks)
    // (A4: E2M1 rows of 32 bytes per stage, 32 rows per instruction, the two
    //  pieces swapped on rows 8..15 of each 16 so that the reads of 16 rows
    //  fall on distinct banks)
    constexpr int APR = C::A4 ? 2 : (C::A8 ? 4 : 8);  // 16-byte pieces per row per stage
    constexpr int AROW = APR * 16;                    // bytes of an activation row per stage
    const int ar_sub = lane / APR, apiece = lane % APR;
    const char* abase = GATHER ? reinterpret_cast<const char*>(x)
                               : reinterpret_cast<const char*>(abuf_in);
    uint32_t asrc[C::A_INSTR];
#pragma unroll
    for (int q = 0; q < C::A_INSTR; ++q) {
        const int row = (wave * C::A_INSTR + q) * (64 / APR) + ar_sub;
        const int sw = C::A4 ? apiece ^ ((row >> 3) & 1) : C::A8 ? apiece ^ ((row >> 2) & 3) : apiece ^ ((row >> 1) & 7);
        const uint32_t src_row = GATHER ? (uint32_t)row_tok[row]
                                        : (uint32_t)(p0 + (row < rows_here ? row : 0));
        const uint32_t kdim = GATHER ? H : I;
        asrc[q] = src_row * (C::A4 ? kdim / 2 : (C::A8 ? 1u : 2u) * kdim) + sw * 16;
    }
    // weights: instruction q of wave w fills 16-row tile w*B_INSTR + q (MX4:
    // the step's 512 bytes of tiles 2 (w*B_INSTR + q) and the next one, from
    // lanes 0-31 and 32-63; a 16-row tile's staged piece holds 32-K quarter j
    // of its row r at 16-byte position 16 j + r, as in a 64-byte chunk of
    // the tiled layout)
    constexpr int HALF_T = BN / 2 / 16;  // gate tiles in a gate/up tile (MODE 0)
    // weight row of the WG's 16-row tile t (MODE 0: gate tiles, then up)
    auto tile_row = [&](int t) {
        return PAIRED ? (t < HALF_T ? 0 : I) + nb * (BN / 2) + (t % HALF_T) * 16 : nb * BN + t * 16;
    };
    // (a wave-uniform tile base plus one per-lane offset, so the loads address
    //  through a scalar base; the lane's 16 bytes follow tile_lane_ptr)
    const uint8_t* bbase[C::B_INSTR];
#pragma unroll
    for (int q = 0; q < C::B_INSTR; ++q) {
        const int t16 = (C::MX4 ? 2 : 1) * (wave * C::B_INSTR + q);
        // the tiled layout keeps whole 16-row tiles in place
        bbase[q] = W + (size_t)tile_row(t16) * KB;
    }
    uint32_t blane;
    if constexpr (C::MX4)
        blane = (lane >> 5) * 16u * KB +
                (LAYOUT == LAYOUT_TILED ? (lane & 31) * 16 : (lane & 15) * KB + ((lane >> 4) & 1) * 16);
    else
        blane = LAYOUT == LAYOUT_TILED ? lane * 16 : (lane & 15) * K + (lane >> 4) * 16;
    // bytes from one step's weight piece to the next
    constexpr int CS = C::MX4 ? (LAYOUT == LAYOUT_TILED ? 512 : 32) : chunk_stride<LAYOUT>();
    // MX4 scales of the 128-wide K chunk the step lies in (both steps of a
    // chunk stage the same bytes): lanes 16 i .. 16 i + 15 of wave w stage the
    // 64 bytes of 16-row tile 4 w + i at byte 64 (4 w + i) of the scale area,
    // 4 bytes a lane -- the tiled layout's scale chunk of the tile as it is
    // (byte 16 j + r: 32-K quarter j, row r), or row-major the 4 bytes of row
    // r (byte 4 r + j).
    uint32_t ssrc = 0;
    if constexpr (C::MX4) {
        const int tw = 4 * wave + (lane >> 4), r = lane & 15;
        ssrc = LAYOUT == LAYOUT_TILED ? (uint32_t)(tile_row(tw) >> 4) * (uint32_t)(K / 128) * 64u + r * 4
                                      : (uint32_t)(tile_row(tw) + r) * (uint32_t)(K / 32);
    }
    constexpr uint32_t SCS = LAYOUT == LAYOUT_TILED ? 64 : 4;  // per 128-K chunk
    // A4: lane l of wave w stages the 4 E8M0 bytes of activation row
    // (64 w + l) % BM (row-major [T][H/32]; down: the hidden rows
    // [rows][I/32] at the sorted rows, padding rows reading the tile's first)
    // for the step's 128-K chunk, at byte 4 row of the stage's
    // activation-scale area (with four waves the rows are staged twice, the
    // second copy unused)
    uint32_t xsrc = 0;
    if constexpr (C::A4 && !C::XT) {
        const int r = (64 * wave + lane) % BM;
        xsrc = GATHER ? (uint32_t)row_tok[r] * (uint32_t)(H / 32)
                      : (uint32_t)(p0 + (r < rows_here ? r : 0)) * (uint32_t)(I / 32);
    }

    auto issue_stage = [&](int st, int kc) {
        const uint32_t sbase = st * C::STAGE;
#pragma unroll
        for (int q = 0; q < C::A_INSTR; ++q)
            lds_load16(abase + (asrc[q] + (uint32_t)kc * AROW),
                       sbase + (wave * C::A_INSTR + q) * 1024, smem);
#pragma unroll
        for (int q = 0; q < C::B_INSTR; ++q)
            lds_load16(bbase[q] + (size_t)kc * CS + blane, sbase + C::A_BYTES + (wave * C::B_INSTR + q) * 1024,
                       smem);
        if constexpr (C::MX4)
            __builtin_amdgcn_global_load_lds(SX + (ssrc + (uint32_t)(kc >> 1) * SCS),
                                             smem + sbase + C::A_BYTES + C::B_BYTES + wave * 256, 4, 0, 0);
        if constexpr (C::A4 && !C::XT)
            __builtin_amdgcn_global_load_lds(static_cast<const uint8_t*>(xscale) + (xsrc + (uint32_t)(kc >> 1) * 4),
                                             smem + sbase + C::A_BYTES + C::B_BYTES + C::S_BYTES + wave * 256, 4,
                                             0, 0);
    };

    // ---- wave tile: rows wm*WROWS .. +WROWS, columns wn*WCOLS .. +WCOLS of
    //      the WG tile
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;
    const int ln = lane & 31, lg = lane >> 5;
    // LDS byte offsets of this lane's operand pieces inside a stage, for the
    // first 32-row / 32-column MFMA tile; the others sit at constant distances
    // (a_step, b_step), which the LDS reads take as immediate offsets.
    // Activation piece s (16 K) of row r: the swizzle (r / 2) % 8 is the same
    // for rows 32 apart.
    //
    // K order inside a 64-wide step (any order works if both operands use it;
    // each lane's 8 K values are one 8-K block kb of the step):
    //   32x32x16: sub-step s (16 K, four per step), lane half lg: kb = 4 lg + s;
    //   16x16x32: sub-step s (32 K, two per step), lane quarter g: kb = 2 g + s,
    //   so that one 16-byte weight read serves both sub-steps.
    // An activation piece (16 bytes) is one kb of a row; a weight lane of the
    // staged 1 KB chunk holds kbs 2 (L / 16), 2 (L / 16) + 1 of row L % 16.
    //
    // MX4 (32 code bytes a row per step, 32x32 tiles): the lane's 16 bytes
    // are quarter lg of its row, K [32 lg, 32 lg + 32), one scale block;
    // sub-step s takes bytes 4s .. 4s + 3 (element 2i of a byte is its low
    // nibble), so K block 4 lg + s as above.  The lane's scale byte sits at
    // s_off + s_step(nt) in the stage, plus 32 (tiled) or 2 (row-major) for
    // the second step of a chunk.
    const int l16 = lane & 15, g16 = lane >> 4;
    uint32_t a_off[4];
    uint32_t b_off, s_off = 0;
    const int t16 = PAIRED ? wn * (C::WCOLS / 32) : wn * (C::WCOLS / 16);
    constexpr uint32_t S_AREA = C::A_BYTES + C::B_BYTES;
    if constexpr (C::M16) {
        const int row = wm * C::WROWS + l16;
#pragma unroll
        for (int s = 0; s < 2; ++s) a_off[s] = row * 128 + (((2 * g16 + s) ^ ((row >> 1) & 7)) * 16);
        a_off[2] = a_off[3] = 0;  // (two sub-steps per step)
        // 16-column tile nt is 16-row weight tile t16(nt); the lane's 16
        // bytes (sub-step 0 then 1) are piece g16 of row l16: lane order
        b_off = C::A_BYTES + t16 * 1024 + lane * 16;
    } else {
        const int row = wm * C::WROWS + ln;
#pragma unroll
        for (int s = 0; s < 4; ++s) a_off[s] = row * 128 + (((4 * lg + s) ^ ((row >> 1) & 7)) * 16);
        // 32-column tile nt spans 16-row tiles t16(nt), t16(nt) + 1; the
        // lane's 16 bytes for half p sit p * 256 bytes further on
        const int tt = t16 + (ln >> 4), r = ln & 15;
        if constexpr (C::MX4) {
            b_off = C::A_BYTES + tt * 512 + (lg * 16 + r) * 16;
            s_off = S_AREA + tt * 64 + (LAYOUT == LAYOUT_TILED ? lg * 16 + r : r * 4 + lg);
        } else {
            b_off = C::A_BYTES + tt * 1024 + (2 * lg * 16 + r) * 16;
        }
    }
    constexpr uint32_t S_PAR = LAYOUT == LAYOUT_TILED ? 32 : 2;
    // (MODE 0: the first NT/2 MFMA column tiles are gate columns, the rest the
    // matching up columns)
    auto a_step = [](int mt) { return mt * C::MS * 128; };
    auto t_step = [](int nt) {  // first 16-row weight tile of column tile nt, from t16
        constexpr int T16 = C::MS / 16;  // 16-row weight tiles per MFMA column tile
        if (PAIRED) return (nt < C::NT / 2 ? 0 : HALF_T) + (nt % (C::NT / 2)) * T16;
        return nt * T16;
    };
    auto b_step = [&](int nt) { return t_step(nt) * C::TB; };
    auto s_step = [&](int nt) { return t_step(nt) * 64; };
    // ---- block scales of the workgroup's columns, staged once in LDS by
    //      direct-to-LDS loads issued before the first operand stages (so the
    //      first stage wait covers them).  Table row j < NR/2 (MODE 0: gate;
    //      MODE 1: all NR rows) holds the 128-row scale block (col0 >> 7) + j
    //      over all K blocks, MODE 0 rows NR/2.. the matching up blocks; rows
    //      are padded to 64 floats and the padding repeats the last block.
    constexpr int NR = BN / 128;
    const int kblocks = K >> 7;
    const int kbp = (kblocks + 63) & ~63;
    float* sc_tab = reinterpret_cast<float*>(smem + C::STAGES * C::STAGE);
    if constexpr (!C::MX4) {
        const int nchunk = kbp >> 6;
        for (int it = wave; it < NR * nchunk; it += C::WAVES) {
            const int j = it / nchunk, c = it - j * nchunk;
            int sr;
            if (PAIRED)
                sr = j < NR / 2 ? ((nb * (BN / 2)) >> 7) + j : ((I + nb * (BN / 2)) >> 7) + j - NR / 2;
            else
                sr = ((nb * BN) >> 7) + j;
            const int kb = min(c * 64 + lane, kblocks - 1);
            __builtin_amdgcn_global_load_lds(S + (size_t)sr * kblocks + kb, sc_tab + j * kbp + c * 64, 4, 0, 0);
        }
    }
    // XT: the tile's E8M0 bytes of x for all of K, [128 rows][H/32 bytes] at
    // byte STAGES * STAGE, staged once with 16-byte direct-to-LDS loads that
    // the first stage wait covers.  Row r's 16-byte piece p sits at slot
    // p ^ (r % pieces) of the row, so that the 32 rows of a wave reading
    // the same block fall on different banks (two rows a bank at H = 8192).
    if constexpr (C::XT) {
        const int rowb = H / 32, pieces = rowb / 16;  // H % 512 == 0: whole pieces
        const int n = BM * pieces;                    // 16-byte loads, a multiple of 64
        for (int it = wave; it * 64 < n; it += C::WAVES) {
            const int d = it * 64 + lane, r = d / pieces, slot = d - r * pieces;
            const int p = slot ^ (r & (pieces - 1));
            // (through the device helper: a 16-byte direct load written in the
            //  kernel body itself left the kernel's host launch stub undefined)
            lds_load16(static_cast<const uint8_t*>(xscale) + ((size_t)row_tok[r] * rowb + p * 16),
                       C::STAGES * C::STAGE + it * 1024, smem);
        }
    }
    // this wave's table rows: g = 0 its gate (or only) columns, g = 1 its up columns
    int sj[2];
    if (PAIRED) {
        sj[0] = (wn * (C::WCOLS / 2)) >> 7;
        sj[1] = NR / 2 + sj[0];
    } else {
        sj[0] = sj[1] = (wn * C::WCOLS) >> 7;
    }

    using Acc = std::conditional_t<C::M16, f32x4, f32x16>;
    constexpr int AR = C::M16 ? 4 : 16;  // accumulator registers per MFMA tile
    Acc acc[C::MT][C::NT];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
            for (int i = 0; i < AR; ++i) acc[mt][nt][i] = 0.0f;

    // ---- block scales.  Group g (g = 0 the wave's gate or only columns, g = 1
    //      its up columns) sums over K blocks b with scales s_b.  Each s_b is
    //      split as m_b * 2^(eref + d_b), 1 <= |m_b| < 2, where eref is the
    //      largest exponent among the group's nonzero scales (so d_b <= 0):
    //      the power of two 2^d_b is folded exactly into the weight operand
    //      (the bf16 conversion's exponent-only scale, or the fp8 MFMA's E8M0
    //      B scale), and the accumulators are kept in units of m_cur * 2^eref,
    //      rescaled by m_old / m_new (a ratio in (1/2, 2), so it can neither
    //      overflow nor lose the sum) when a block starts.  A block whose scale
    //      is zero adds exactly nothing: its MFMAs are skipped (a wave-uniform
    //      branch).  Weights stay exact while d_b >= -117 (E4M3FN times 2^d_b
    //      then stays a normal bf16 value); a block more than 2^117 below the
    //      group's largest scale has its smallest codes flushed to zero.
    float mcur[2] = {1.0f, 1.0f};  // mantissa of the accumulator unit
    int eref[2] = {0, 0};
    float csc[2] = {1.0f, 1.0f};   // 2^d of the current block as a conversion scale
    int bsc[2] = {127, 127};       // the same as an E8M0 byte
    bool zs[2] = {false, false};   // the current block's scale is zero
    // (once the scale table is in LDS) the largest exponent of each group
    auto scale_prologue = [&]() {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            int mx = -1000;
            for (int c = 0; c < kbp; c += 64) {
                const float v = sc_tab[sj[g] * kbp + c + lane];
                int ex;
                (void)frexpf(v, &ex);
                mx = v != 0.0f ? max(mx, ex - 1) : mx;
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, MOE_WAVE));
            eref[g] = __builtin_amdgcn_readfirstlane(mx == -1000 ? 0 : mx);
        }
    };
    // a K block starts: its scales sn[g] give the rescale factors rr[g]
    auto enter_block = [&](const float (&sn)[2], float (&rr)[2]) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const float s = sn[g];
            const bool z = s == 0.0f;
            int ex;
            const float m = 2.0f * frexpf(s, &ex);
            const int byte = max(ex - 1 - eref[g] + 127, 0);
            // (wave-uniform: kept in scalar registers)
            rr[g] = uniform_f32(z ? 1.0f : mcur[g] * __builtin_amdgcn_rcpf(m));
            mcur[g] = uniform_f32(z ? mcur[g] : m);
            bsc[g] = __builtin_amdgcn_readfirstlane(byte);
            csc[g] = __builtin_bit_cast(float, (uint32_t)bsc[g] << 23);
            zs[g] = __builtin_amdgcn_readfirstlane((int)z) != 0;
        }
    };

    // ---- K loop, software-pipelined by half steps.  Half p of a 64-wide step
    //      covers sub-steps 2p, 2p+1 (16 K each): A pieces 2p, 2p+1 and 16-byte
    //      weight piece p.  The LDS reads of the next half are in flight while
    //      the MFMAs of the current half run; the LDS stages hold step kc
    //      (being read) and the following ones (landing), and the buffer of
    //      step kc is refilled with step kc+STAGES once every wave has read
    //      it.  The body
    //      covers the two steps of one 128-wide K block and is branch-free
    //      around the LDS reads, so their waits stay partial.
    const int nk = K / PF_BK;  // even and >= 2 since K % 128 == 0
    constexpr int PER_STAGE = C::A_INSTR + C::B_INSTR + C::S_INSTR;  // loads per wave per stage
    // MFMA row groups (32 rows) of this wave that hold rows of the segment:
    // a partial last tile skips the empty ones (their rows are never stored)
    const int mt_active = __builtin_amdgcn_readfirstlane(
        min(C::MT, max(0, rows_here - wm * C::WROWS + C::MS - 1) / C::MS));
    auto kloop = [&](auto mta_c) {
    constexpr int MTA = decltype(mta_c)::value;
    // operand registers of a half step (32 K): 32x32 -- two activation
    // pieces per row group and 16 weight bytes per column tile; 16x16 -- one
    // activation piece per row group and 8 weight bytes per column tile
    constexpr int AP = C::M16 ? 1 : 2;
    using BFrag = std::conditional_t<C::M16, u32x2, u32x4>;
    u32x4 ah[2][C::MT][AP];
    BFrag bh[2][C::NT];
    // the second half's weight operands, read with the first half's: 16x16 --
    // sub-step 1's bytes; MX4 -- sub-steps 2, 3 and the scale
    BFrag bz[C::NT];
    // MX4 operands {codes, codes, scale, -}: the scale is its E8M0 byte as the
    // exponent field of an fp32 (the converter reads only that field).  par:
    // the step's position in its 128-K chunk.
    auto read_half = [&](int stage, int p, u32x4 (&a)[C::MT][AP], BFrag (&b)[C::NT], int par) {
        const char* st = smem + stage * C::STAGE;
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
            for (int j = 0; j < AP; ++j)
                a[mt][j] = *reinterpret_cast<const u32x4*>(st + a_off[AP * p + j] + a_step(mt));
        if (MTA > 0) {
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) {
                if constexpr (C::MX4) {
                    if (p == 0) {
                        const uint32_t sc = (uint32_t)*reinterpret_cast<const uint8_t*>(
                                                st + s_off + par * S_PAR + s_step(nt)) << 23;
                        const u32x4 w = *reinterpret_cast<const u32x4*>(st + b_off + b_step(nt));
                        b[nt] = BFrag{w[0], w[1], sc, 0u};
                        bz[nt] = BFrag{w[2], w[3], sc, 0u};
                    } else {
                        b[nt] = bz[nt];
                    }
                } else if constexpr (C::M16) {
                    if (p == 0) {
                        const u32x4 w = *reinterpret_cast<const u32x4*>(st + b_off + b_step(nt));
                        b[nt] = BFrag{w[0], w[1]};
                        bz[nt] = BFrag{w[2], w[3]};
                    } else {
                        b[nt] = bz[nt];
                    }
                } else {
                    b[nt] = *reinterpret_cast<const BFrag*>(st + b_off + p * 256 + b_step(nt));
                }
            }
        }
    };
    // Part j of a half: 32x32 -- sub-step j (16 K) of every tile; 16x16 --
    // the half's 32 K for column tiles j*NT/2 .. (j+1)*NT/2 - 1 (gate/up: j = 0
    // the gate tiles, j = 1 the up tiles).  rescale: the half opens a new K
    // block, and each accumulator is multiplied by its group's factor right
    // before its first MFMA of the block.
    auto mma_sub = [&](const u32x4 (&a)[C::MT][AP], const BFrag (&b)[C::NT], int j, bool rescale,
                       const float (&rr)[2]) {
        if (MTA == 0) return;
        if (C::MX4) rescale = false;  // (the scales are in the operands)
        if (C::M16 && rescale) {
            // 16x16: every accumulator of the block's first half is rescaled
            // before part 0's MFMAs
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) {
                const float f = PAIRED ? rr[nt / (C::NT / 2)] : rr[0];
#pragma unroll
                for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
                    for (int i = 0; i < AR; ++i) acc[mt][nt][i] *= f;
            }
            rescale = false;
        }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
            if (C::M16 && nt / (C::NT / 2) != j) continue;
            const int gi = PAIRED ? nt / (C::NT / 2) : 0;
            if (zs[gi]) continue;  // a zero block scale: nothing to add
            bf16x8 bf;
            if constexpr (C::MX4)
                bf = fp4x8_to_bf16x8_scaled(b[nt][j], __uint_as_float(b[nt][2]));
            else if constexpr (C::M16)
                bf = fp8x8_to_bf16x8_scaled(b[nt][0], b[nt][1], csc[gi]);
            else
                bf = j == 0 ? fp8x8_to_bf16x8_scaled(b[nt][0], b[nt][1], csc[gi])
                            : fp8x8_to_bf16x8_scaled(b[nt][2], b[nt][3], csc[gi]);
            const float f = rr[gi];
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt) {
                if (rescale)
#pragma unroll
                    for (int i = 0; i < AR; ++i) acc[mt][nt][i] *= f;
                if constexpr (C::M16)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[mt][0]), bf, acc[mt][nt], 0, 0, 0);
                else
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[mt][j]), bf, acc[mt][nt], 0, 0, 0);
            }
            // (16x16: one converted weight fragment live at a time)
            if constexpr (C::M16) __builtin_amdgcn_sched_barrier(0);
        }
    };
    // step kc + 1 landed (with three stages step kc + 2 may still be in
    // flight); the barrier also orders every wave's reads of buffer kc before
    // its refill
    // (par: the position of step kc + 1 in its 128-K chunk)
    auto next_step = [&](int kc, int par) {
        if (C::STAGES >= 3 && kc + 2 < nk) wait_vmcnt<(C::STAGES >= 3 ? PER_STAGE : 0)>();
        else wait_vmcnt<0>();
        barrier_after_lds_reads();
        if (kc + C::STAGES < nk) issue_stage(kc % C::STAGES, kc + C::STAGES);
        // past the last step this reads a stale buffer whose values are unused
        read_half((kc + 1) % C::STAGES, 0, ah[0], bh[0], par);
    };

#pragma unroll
    for (int st = 0; st < C::STAGES; ++st)
        if (st < nk) issue_stage(st, st);
    if (nk >= C::STAGES) wait_vmcnt<(C::STAGES - 1) * PER_STAGE>();
    else wait_vmcnt<PER_STAGE>();  // nk == 2: stages 0 and 1 issued
    barrier_after_lds_reads();     // stage 0 and the scale table landed in every wave
    float snext[2] = {1.0f, 1.0f};
    if constexpr (!C::MX4) {
        scale_prologue();
        snext[0] = sc_tab[sj[0] * kbp];
        snext[1] = sc_tab[sj[1] * kbp];
    }
    read_half(0, 0, ah[0], bh[0], 0);
    const float one[2] = {1.0f, 1.0f};
    for (int kb = 0; kb < kblocks; ++kb) {
        const int kc = 2 * kb;
        float rr[2] = {1.0f, 1.0f};
        if constexpr (!C::MX4) {
            enter_block(snext, rr);
            const int kn = kb + 1 < kblocks ? kb + 1 : kb;
            snext[0] = sc_tab[sj[0] * kbp + kn];
            snext[1] = sc_tab[sj[1] * kbp + kn];
        }

        // the reads of the second half go out after the first sub-step's MFMAs,
        // whose operands were read a whole half earlier
        mma_sub(ah[0], bh[0], 0, true, rr);
        __builtin_amdgcn_sched_barrier(0);
        read_half(kc % C::STAGES, 1, ah[1], bh[1], 0);
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(ah[0], bh[0], 1, false, one);
        __builtin_amdgcn_sched_barrier(0);
        next_step(kc, 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(ah[1], bh[1], 0, false, one);
        mma_sub(ah[1], bh[1], 1, false, one);
        __builtin_amdgcn_sched_barrier(0);

        mma_sub(ah[0], bh[0], 0, false, one);
        __builtin_amdgcn_sched_barrier(0);
        read_half((kc + 1) % C::STAGES, 1, ah[1], bh[1], 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(ah[0], bh[0], 1, false, one);
        __builtin_amdgcn_sched_barrier(0);
        next_step(kc + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(ah[1], bh[1], 0, false, one);
        mma_sub(ah[1], bh[1], 1, false, one);
        __builtin_amdgcn_sched_barrier(0);
    }
    };
    if constexpr (C::A8) {
        // ---- A8 K loop: one v_mfma_scale_f32_32x32x64_f8f6f4 per tile per stage
        //      (unit scales).  Lane l feeds row (or weight row) l % 32 of a 32-row
        //      tile with bytes [32 h, 32 h + 32) of the stage's 64 K, h = l / 32,
        //      for both operands alike, so each product sums exactly over K.  The
        //      weight operand's pieces sit where the 32x32 bf16 path reads them
        //      (b_off, b_step); the activation rows are 64 bytes.
        //      MX4: the lane's 32 K of its weight row are its 16 E2M1 code
        //      bytes, one scale block, whose E8M0 byte is the MFMA's B scale
        //      for the lane.  With an E2M1 B operand the MFMA pairs B lane half
        //      h's codes 0-15 with A lane half 0's bytes 16h .. 16h + 15 and
        //      codes 16-31 with A lane half 1's (measured on gfx950 with
        //      one-hot operands), so A lane half h carries the 16-K pieces h
        //      and h + 2 of the step.
        auto kloop_a8 = [&](auto mta_c) {
            constexpr int MTA = decltype(mta_c)::value;
            const int r32 = lane & 31, h8 = lane >> 5;
            uint32_t a8_off[2];
    #pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wm * C::WROWS + r32;
                const int piece = C::MX4 ? h8 + 2 * j : 2 * h8 + j;
                a8_off[j] = row * 64 + ((piece ^ ((row >> 2) & 3)) * 16);
            }
            // A4: E2M1 x E2M1 pairs A lane (row, h) with B lane (column, h) in
            // the natural order (measured like the E4M3 pairing), so the lane
            // reads piece h of its 32-byte row; its E8M0 byte for the step's
            // block h sits at byte 4 row + 2 par + h of the scale area
            const int arow = wm * C::WROWS + r32;
            const uint32_t a4_off = arow * 32 + ((h8 ^ ((arow >> 3) & 1)) * 16);
            const uint32_t sa_off = C::A_BYTES + C::B_BYTES + C::S_BYTES + arow * 4 + h8;
            // XT: block 2 kc + h of row arow is byte 2 (kc % 8) + h of piece
            // kc / 8, stored at slot (kc / 8) ^ (arow % pieces); the row
            // groups mt sit 32 rows apart (the same slot order)
            const int xt_rowb = H / 32, xt_mask = xt_rowb / 16 - 1;
            const uint32_t xt_row = C::STAGES * C::STAGE + arow * xt_rowb + h8;
            // (par: the stage's position in its 128-K chunk, for the MX4 scales)
            auto stage_mma = [&](int stage, bool rescale, const float (&rr)[2], int par, int kc) {
                const char* st = smem + stage * C::STAGE;
                i32x8 av[C::MT], bv[C::NT];
                int bs[C::NT];  // MX4: the lane's E8M0 byte of each column tile
                int sa[C::MT];  // A4: the lane's E8M0 byte of each row group
    #pragma unroll
                for (int mt = 0; mt < MTA; ++mt) {
                    if constexpr (C::A4) {
                        av[mt] = cat_i32x8(*reinterpret_cast<const u32x4*>(st + a4_off + mt * 32 * 32),
                                           u32x4{0u, 0u, 0u, 0u});
                        if constexpr (C::XT)
                            sa[mt] = *reinterpret_cast<const uint8_t*>(
                                smem + xt_row + ((((kc >> 3) ^ (arow & xt_mask)) * 16) + 2 * (kc & 7)) +
                                mt * 32 * xt_rowb);
                        else
                            sa[mt] = *reinterpret_cast<const uint8_t*>(st + sa_off + par * 2 + mt * 32 * 4);
                    } else {
                        av[mt] = cat_i32x8(*reinterpret_cast<const u32x4*>(st + a8_off[0] + mt * 32 * 64),
                                           *reinterpret_cast<const u32x4*>(st + a8_off[1] + mt * 32 * 64));
                    }
                }
                if (MTA > 0)
    #pragma unroll
                    for (int nt = 0; nt < C::NT; ++nt) {
                        if constexpr (C::MX4) {
                            bv[nt] = cat_i32x8(*reinterpret_cast<const u32x4*>(st + b_off + b_step(nt)),
                                               u32x4{0u, 0u, 0u, 0u});
                            bs[nt] = *reinterpret_cast<const uint8_t*>(st + s_off + par * S_PAR + s_step(nt));
                        } else {
                            bv[nt] = cat_i32x8(*reinterpret_cast<const u32x4*>(st + b_off + b_step(nt)),
                                               *reinterpret_cast<const u32x4*>(st + b_off + b_step(nt) + 256));
                        }
                    }
    #pragma unroll
                for (int nt = 0; nt < C::NT; ++nt) {
                    if constexpr (C::A4) {
    #pragma unroll
                        for (int mt = 0; mt < MTA; ++mt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                av[mt], bv[nt], acc[mt][nt], 4, 4, 0, sa[mt], 0, bs[nt]);
                        continue;
                    }
                    if constexpr (C::MX4) {
    #pragma unroll
                        for (int mt = 0; mt < MTA; ++mt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                av[mt], bv[nt], acc[mt][nt], 0, 4, 0, 127, 0, bs[nt]);
                        continue;
                    }
                    const int gi = PAIRED ? nt / (C::NT / 2) : 0;
                    if (zs[gi]) continue;  // a zero block scale: nothing to add
                    const float f = rr[gi];
    #pragma unroll
                    for (int mt = 0; mt < MTA; ++mt) {
                        if (rescale)
    #pragma unroll
                            for (int i = 0; i < AR; ++i) acc[mt][nt][i] *= f;
                        // (the block's power of two as the B operand's E8M0 scale)
                        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            av[mt], bv[nt], acc[mt][nt], 0, 0, 0, 127, 0, bsc[gi]);
                    }
                }
            };
            auto next_stage = [&](int kc) {
                // stage kc + 1 landed in this wave (with three stages, kc + 2 may
                // still be in flight)
                if (C::STAGES >= 3 && kc + 2 < nk) wait_vmcnt<(C::STAGES >= 3 ? PER_STAGE : 0)>();
                else wait_vmcnt<0>();
                barrier_after_lds_reads();   // ... in every wave; stage kc read by every wave
                if (kc + C::STAGES < nk) issue_stage(kc % C::STAGES, kc + C::STAGES);
            };
    #pragma unroll
            for (int st = 0; st < C::STAGES; ++st)
                if (st < nk) issue_stage(st, st);
            // stage 0 and the scale table landed (with fewer K stages than
            // buffers, e.g. K = 128 on three stages, wait for everything)
            if (nk >= C::STAGES) wait_vmcnt<(C::STAGES - 1) * PER_STAGE>();
            else wait_vmcnt<0>();
            barrier_after_lds_reads();  // ... in every wave
            float snext[2] = {1.0f, 1.0f};
            if constexpr (!C::MX4) {
                scale_prologue();
                snext[0] = sc_tab[sj[0] * kbp];
                snext[1] = sc_tab[sj[1] * kbp];
            }
            const float one[2] = {1.0f, 1.0f};
            for (int kb = 0; kb < kblocks; ++kb) {
                const int kc = 2 * kb;
                float rr[2] = {1.0f, 1.0f};
                if constexpr (!C::MX4) {
                    enter_block(snext, rr);
                    const int kn = kb + 1 < kblocks ? kb + 1 : kb;
                    snext[0] = sc_tab[sj[0] * kbp + kn];
                    snext[1] = sc_tab[sj[1] * kbp + kn];
                }
                stage_mma(kc % C::STAGES, true, rr, 0, kc);
                next_stage(kc);
                stage_mma((kc + 1) % C::STAGES, false, one, 1, kc + 1);
                next_stage(kc + 1);
            }
        };
        if (mt_active >= 2) kloop_a8(std::integral_constant<int, 2>{});
        else if (mt_active == 1) kloop_a8(std::integral_constant<int, 1>{});
        else kloop_a8(std::integral_constant<int, 0>{});
    } else if constexpr (C::MT == 4) {
        // three active groups run the full loop (cheaper than another copy)
        if (mt_active >= 3) kloop(std::integral_constant<int, 4>{});
        else if (mt_active == 2) kloop(std::integral_constant<int, 2>{});
        else if (mt_active == 1) kloop(std::integral_constant<int, 1>{});
        else kloop(std::integral_constant<int, 0>{});
    } else {
        if (mt_active >= 2) kloop(std::integral_constant<int, 2>{});
        else if (mt_active == 1) kloop(std::integral_constant<int, 1>{});
        else kloop(std::integral_constant<int, 0>{});
    }

    // ---- epilogue.  Accumulator layouts: 32x32 -- lane l holds column l%32
    //      and, for register i, row 8*(i/4) + 4*(l/32) + i%4; 16x16 -- column
    //      l%16, row 4*(l/16) + i.  Row m of the tile goes to sorted row p0 + m
    //      (m < rows_here).  Both epilogues pass a wave tile's results through
    //      LDS (the stage buffers, free once every wave has left the K loop) so
    //      that a lane stores a run of consecutive columns of one row.
    if constexpr (MODE == PF_DOWN) {
        // Down: the tile's rows are the sorted rows p0 .. p0 + rows_here - 1,
        // written in the block floating-point form of bfp16x8_encode (16-bit
        // mantissas at byte 2*col, one exponent byte per 8 columns at byte
        // 2*H + col/8; row stride 2*H + H/8; the combine widens them and
        // multiplies by the affinity).  The MFMA layout gives a lane one
        // column of many rows, so each 32-row slab of a wave tile goes through
        // LDS (the stage buffers, free once every wave has left the K loop): a
        // lane then holds 8 consecutive columns of one row, encodes them as
        // one run and writes a 16-byte and a 1-byte streaming store, 16 lanes
        // covering a row's 128 columns (256 + 16 contiguous bytes).
        static_assert(!C::M16 && C::MS == 32 && C::WCOLS == 128 && C::MT * 32 == C::WROWS,
                      "down epilogue: 64 x 128 wave tiles of 32 x 32 MFMAs");
        __syncthreads();  // every wave is done reading the K stages
        float* slab = reinterpret_cast<float*>(smem) + wave * (32 * 128);
        uint8_t* ybytes = reinterpret_cast<uint8_t*>(ybuf);
        const size_t rowb = (size_t)H * 2 + (size_t)(H / 8);
        const int col0 = nb * BN + wn * C::WCOLS;  // first column of the wave tile
        // the accumulator unit is mcur * 2^eref: the slab holds the raw
        // accumulators and the encoder applies the unit (the power of two
        // goes into the exponent byte)
        const float sm = mcur[0];
        const int se = eref[0];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
                for (int i = 0; i < AR; ++i)
                    slab[(8 * (i >> 2) + 4 * lg + (i & 3)) * 128 + nt * 32 + ln] = acc[mt][nt][i];
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slab is written
            __builtin_amdgcn_wave_barrier();
            // Each run is first encoded by the branch-free common case and
            // stored; a run that case cannot hold (a largest value that is
            // not finite, zero or near the ends of the exponent range: rare)
            // is encoded again by the full encoder and stored over it, after
            // all eight, so the eight runs' LDS reads, encodes and stores
            // carry no branch and can interleave.
            uint32_t redo = 0;  // runs to encode again (bit q)
            const int c = 8 * (lane & 15);  // the lane's first column
            auto ld = [&](int q, f32x4& v0, f32x4& v1) {
                const int r = 4 * q + (lane >> 4);  // row of the slab
                v0 = *reinterpret_cast<const f32x4*>(slab + r * 128 + c);
                v1 = *reinterpret_cast<const f32x4*>(slab + r * 128 + c + 4);
            };
            auto put = [&](int q, f32x4 v0, f32x4 v1, bool guarded, bool full) {
                const int m = wm * C::WROWS + mt * 32 + 4 * q + (lane >> 4);  // row of the tile
                if (!guarded || m < rows_here) {
                    u32x4 mant;
                    uint32_t ex;
                    if (full)
                        bfp16x8_encode_scaled(v0, v1, sm, se, mant, ex);
                    else if (!bfp16x8_encode_scaled_fast(v0, v1, sm, se, mant, ex))
                        redo |= 1u << q;
                    uint8_t* rowp = ybytes + (size_t)(p0 + m) * rowb;
                    __builtin_nontemporal_store(mant, reinterpret_cast<u32x4*>(rowp + 2 * (size_t)(col0 + c)));
                    __builtin_nontemporal_store((uint8_t)ex, rowp + 2 * (size_t)H + (col0 + c) / 8);
                }
            };
            // a slab whose 32 rows are all real stores with no per-row branch,
            // each run's LDS reads issued one run ahead; a partial slab checks
            // each row
            if (wm * C::WROWS + mt * 32 + 32 <= rows_here) {
                f32x4 a0, a1, b0, b1;
                ld(0, a0, a1);
#pragma unroll
                for (int q = 0; q < 8; q += 2) {
                    ld(q + 1, b0, b1);
                    put(q, a0, a1, false, false);
                    if (q + 2 < 8) ld(q + 2, a0, a1);
                    put(q + 1, b0, b1, false, false);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    f32x4 v0, v1;
                    ld(q, v0, v1);
                    put(q, v0, v1, true, false);
                }
            }
            if (__ballot(redo != 0) != 0ull) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (redo & (1u << q)) {
                        f32x4 v0, v1;
                        ld(q, v0, v1);
                        put(q, v0, v1, true, true);
                    }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // the slab is read before it is rewritten
            __builtin_amdgcn_wave_barrier();
        }
        return;
    }
    // Gate/up (SwiGLU of the paired gate and up columns) and up (relu^2):
    // bf16 activations, OUTC per wave row, into the wave's slab, then 8
    // consecutive columns (16 bytes) per lane and store, OUTC/8 lanes per row.
    constexpr int OUTC = MODE == PF_GATEUP ? C::WCOLS / 2 : C::WCOLS;
    constexpr int LPR = OUTC / 8;              // lanes per row
    constexpr int RPS = MOE_WAVE / LPR;        // rows per store step
    static_assert(C::WAVES * C::WROWS * OUTC * 2 == pf_epilogue_lds<MODE, C>(), "slab size");
    __syncthreads();  // every wave is done reading the K stages
    uint16_t* slab = reinterpret_cast<uint16_t*>(smem) + wave * (C::WROWS * OUTC);
    const int ocol = C::M16 ? l16 : ln;  // the lane's column in an MFMA tile
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int r = mt * C::MS + (C::M16 ? 4 * g16 + i : 8 * (i >> 2) + 4 * lg + (i & 3));
            // A8: the row's activation scale joins the weight block's
            float xsv = 1.0f;
            if constexpr (XS_ROW) xsv = row_xs[wm * C::WROWS + r];
            // value = acc * mcur * x scale * 2^eref, the power of two last (an
            // exact exponent shift unless the result is subnormal)
            const float s0 = mcur[0] * xsv, s1 = mcur[1] * xsv;
            // two values at a time through the packed bf16 conversion
            if constexpr (MODE == PF_GATEUP) {
                static_assert(C::NT % 4 == 0, "pairs of gate tiles");
                auto g = [&](int nt) {
                    return swiglu_fast(ldexpf(acc[mt][nt][i] * s0, eref[0]),
                                       ldexpf(acc[mt][nt + C::NT / 2][i] * s1, eref[1]));
                };
#pragma unroll
                for (int nt = 0; nt < C::NT / 2; nt += 2) {
                    const uint32_t w = f32x2_to_bf16x2_bits(g(nt), g(nt + 1));
                    slab[r * OUTC + nt * C::MS + ocol] = (uint16_t)w;
                    slab[r * OUTC + (nt + 1) * C::MS + ocol] = (uint16_t)(w >> 16);
                }
            } else {
                static_assert(C::NT % 2 == 0, "pairs of tiles");
#pragma unroll
                for (int nt = 0; nt < C::NT; nt += 2) {
                    const uint32_t w = f32x2_to_bf16x2_bits(relu2(ldexpf(acc[mt][nt][i] * s0, eref[0])),
                                                            relu2(ldexpf(acc[mt][nt + 1][i] * s0, eref[0])));
                    slab[r * OUTC + nt * C::MS + ocol] = (uint16_t)w;
                    slab[r * OUTC + (nt + 1) * C::MS + ocol] = (uint16_t)(w >> 16);
                }
            }
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slab is written
    __builtin_amdgcn_wave_barrier();
    const int colbase = MODE == PF_GATEUP ? nb * (BN / 2) + wn * (C::WCOLS / 2) : nb * BN + wn * C::WCOLS;
    auto put = [&](int q, bool guarded) {
        const int r = q * RPS + lane / LPR;
        const int c = 8 * (lane % LPR);
        const int m = wm * C::WROWS + r;  // row of the tile
        const u32x4 v = *reinterpret_cast<const u32x4*>(slab + r * OUTC + c);
        if constexpr (C::H4) {
            // MXFP4: a lane quad holds one 32-column run of a row (OUTC is a
            // multiple of 32 and colbase of 32), its largest magnitude shared
            // by shuffles; a lane writes its 8 codes (4 bytes), the quad's
            // first lane the E8M0 byte
            uint32_t mx = bf16x8_absmax_bits(v);
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, MOE_WAVE));
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, MOE_WAVE));
            const bool bad = mx >= 0x7F80u;
            const int X = mxfp4_run_exponent(mx);
            const uint32_t word = bad ? 0u : mxfp4_encode8(v, X);
            if (!guarded || m < rows_here) {
                const int col = colbase + c;
                uint8_t* hq = reinterpret_cast<uint8_t*>(abuf_out);
                *reinterpret_cast<uint32_t*>(hq + (size_t)(p0 + m) * (I / 2) + col / 2) = word;
                if ((lane & 3) == 0)
                    hscale_out[(size_t)(p0 + m) * (I / 32) + col / 32] = bad ? (uint8_t)255 : (uint8_t)(X + 127);
            }
        } else if (!guarded || m < rows_here) {
            *reinterpret_cast<u32x4*>(abuf_out + (size_t)(p0 + m) * I + colbase + c) = v;
        }
    };
    // a wave tile whose rows are all real stores with no per-row branch, so
    // that its row pieces' LDS reads and stores can interleave; a partial one
    // checks each row
    if (wm * C::WROWS + C::WROWS <= rows_here) {
#pragma unroll
        for (int q = 0; q < C::WROWS / RPS; ++q) put(q, false);
    } else {
#pragma unroll
        for (int q = 0; q < C::WROWS / RPS; ++q) put(q, true);
    }
}

template <int MODE>
static inline int K_of(int H, int I) { return MODE == PF_DOWN ? I : H; }

template <int MODE, int LAYOUT, class C>
static int launch_pf(const uint16_t* x, const uint16_t* abuf_in, const uint8_t* wexp,
                     const void* sexp, const uint8_t* wsh, const void* ssh, const Plan& plan,
                     int T, int H, int I, int E, int k, int has_shared, uint16_t* abuf_out,
                     float* ybuf, hipStream_t stream, const void* xscale = nullptr,
                     uint8_t* hscale_out = nullptr) {
    const int nblk = MODE == PF_GATEUP ? 2 * I / C::BN : (MODE == PF_UP ? I : H) / C::BN;
    const long R = (long)T * k;
    const long max_tiles = (R + C::BM - 1) / C::BM + E + (has_shared ? (T + C::BM - 1) / C::BM : 0);
    // (the sort's tile list has room for at least this many records)
    // XCD x's workgroup j handles the (j / nblk)-th row tile of its blocks
    const long grid = 8L * nblk * PF_XCD_RUN * ((max_tiles + 8 * PF_XCD_RUN - 1) / (8 * PF_XCD_RUN));
    if (grid > 0x7FFFFFFFL) {
        set_error("prefill: too many tiles");
        return MOE_EUNSUPPORTED;
    }
    // activation rows are addressed by 32-bit byte offsets
    const size_t a_bytes = MODE != PF_DOWN ? (C::A4 ? (size_t)T * H / 2 : (size_t)T * H * (C::A8 ? 1 : 2))
                                           : (size_t)(R + (has_shared ? T : 0)) * I * 2;
    if (a_bytes > 0xFFFFFFFFull) {
        set_error("prefill: activation matrix over 4 GB");
        return MOE_EUNSUPPORTED;
    }
    const size_t kbp = ((size_t)K_of<MODE>(H, I) / 128 + 63) / 64 * 64;
    // stages, the fp32 scale table (MX4: none) and at least the epilogue's slabs
    // (XT: the x-scale table instead)
    const size_t tab = C::XT ? (size_t)C::BM * (H / 32) : C::MX4 ? 0 : (size_t)(C::BN / 128) * kbp * 4;
    const size_t lds = std::max((size_t)C::STAGES * C::STAGE + tab, (size_t)pf_epilogue_lds<MODE, C>());
    if (C::XT && !prefill_xscale_table(H)) {
        set_error("prefill: x-scale table needs H = 512 * 2^j <= %d", PF_XT_MAX_H);
        return MOE_EINVAL;
    }
    static_assert(!C::H4 || MODE != PF_DOWN, "H4 is an epilogue of the first GEMM");
    static_assert(!C::H4 || (MODE == PF_GATEUP ? C::WCOLS / 2 : C::WCOLS) % 32 == 0, "whole MXFP4 runs a wave");
    if (C::H4 && !hscale_out) {
        set_error("prefill: the MXFP4 hidden activation needs its scale array");
        return MOE_EINVAL;
    }
    if (C::A4 && !xscale) {
        set_error("prefill: MXFP4 activations need their scale array");
        return MOE_EINVAL;
    }
    const char* pname =
        MODE == PF_DOWN ? (C::A4 ? "prefill_down_mxfp4_a4" : C::MX4 ? "prefill_down_mxfp4" : "prefill_down")
        : MODE == PF_UP
            ? (C::H4 ? "prefill_up_relu2_mxfp4_a4h4"
               : C::A4 ? "prefill_up_relu2_mxfp4_a4"
               : C::A8 ? (C::MX4 ? "prefill_up_relu2_mxfp4_a8" : "prefill_up_relu2_a8")
                       : (C::MX4 ? "prefill_up_relu2_mxfp4" : "prefill_up_relu2"))
            : (C::H4 ? "prefill_gateup_swiglu_mxfp4_a4h4"
               : C::A4 ? "prefill_gateup_swiglu_mxfp4_a4"
               : C::A8 ? (C::MX4 ? "prefill_gateup_swiglu_mxfp4_a8" : "prefill_gateup_swiglu_a8")
                       : (C::MX4 ? "prefill_gateup_swiglu_mxfp4" : "prefill_gateup_swiglu"));
    prof_begin(pname, stream);
    prefill_gemm_kernel<MODE, LAYOUT, C><<<(unsigned)grid, C::THREADS, lds, stream>>>(
        x, abuf_in, wexp, sexp, wsh, ssh, plan, T, H, I, k, nblk, (int)max_tiles, abuf_out, ybuf,
        xscale, hscale_out);
    prof_end(stream);
    return check_launch(MODE == PF_GATEUP ? "prefill_gemm_kernel<gateup>"
                                          : (MODE == PF_UP ? "prefill_gemm_kernel<up>" : "prefill_gemm_kernel<down>"));
}

// The first GEMM on MXFP4 activations: gate/up (SwiGLU), or the up
// projection (relu^2) on the wide tile CW or, where I % 256 != 0, the
// narrow tile CN.
template <int LAYOUT, class CW, class CN>
static int launch_first_a4(const uint16_t* xa, const uint8_t* w13, const void* w13s, const SharedW& sh,
                           const Plan& plan, int T, int H, int I, int E, int k, int hs, uint16_t* abuf,
                           float* ybuf, int act, bool narrow, const void* xs, uint8_t* hsc,
                           hipStream_t stream) {
    const void* ss = sh.w13_scale;
    if (act != ACT_RELU2)
        return launch_pf<PF_GATEUP, LAYOUT, CW>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k, hs,
                                                abuf, ybuf, stream, xs, hsc);
    if (narrow)
        return launch_pf<PF_UP, LAYOUT, CN>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k, hs, abuf,
                                            ybuf, stream, xs, hsc);
    return launch_pf<PF_UP, LAYOUT, CW>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k, hs, abuf,
                                        ybuf, stream, xs, hsc);
}

template <int LAYOUT>
static int launch_prefill_c(const uint16_t* x, const uint8_t* w13, const void* w13s,
                            const uint8_t* w2, const void* w2s, const SharedW& sh,
                            const Plan& plan, int T, int H, int I, int E, int k, uint16_t* abuf,
                            float* ybuf, int act, const uint8_t* xq, const void* xs, int afmt, bool mx4,
                            hipStream_t stream) {
    const int hs = sh.w13 != nullptr;
    int rc;
    const void* ss = sh.w13_scale;
    const bool narrow = act == ACT_RELU2 && I % 256 != 0;  // (I % 128 == 0)
    if (mx4 && (afmt == AFMT_MXFP4 || afmt == AFMT_MXFP4_H4)) {
        // MXFP4 weights and activations: E2M1 x E2M1 gate/up, the x scales
        // from a per-tile table where H allows it
        const uint16_t* xa = reinterpret_cast<const uint16_t*>(xq);
        const bool xt = prefill_xscale_table(H);
        if (afmt == AFMT_MXFP4_H4) {
            // ... and the hidden activation to MXFP4 for an E2M1 x E2M1 down:
            // its codes [rows][I/2] from the start of abuf, its E8M0 bytes
            // [rows][I/32] after them (256-byte aligned; within abuf's
            // rows * I * 2 bytes)
            const size_t rows = (size_t)T * k + (hs ? (size_t)T : 0);
            uint8_t* hsc = reinterpret_cast<uint8_t*>(abuf) + ((rows * (I / 2) + 255) & ~(size_t)255);
            rc = xt ? launch_first_a4<LAYOUT, PfGateUpMxA4TH, PfUpNarrowMxA4TH>(
                          xa, w13, w13s, sh, plan, T, H, I, E, k, hs, abuf, ybuf, act, narrow, xs, hsc, stream)
                    : launch_first_a4<LAYOUT, PfGateUpMxA4H, PfUpNarrowMxA4H>(
                          xa, w13, w13s, sh, plan, T, H, I, E, k, hs, abuf, ybuf, act, narrow, xs, hsc, stream);
            if (rc == MOE_OK)
                rc = launch_pf<PF_DOWN, LAYOUT, PfDownMxA4>(x, abuf, w2, w2s, sh.w2, sh.w2_scale, plan, T, H, I,
                                                            E, k, hs, abuf, ybuf, stream, hsc);
            return rc;
        }
        rc = xt ? launch_first_a4<LAYOUT, PfGateUpMxA4T, PfUpNarrowMxA4T>(
                      xa, w13, w13s, sh, plan, T, H, I, E, k, hs, abuf, ybuf, act, narrow, xs, nullptr, stream)
                : launch_first_a4<LAYOUT, PfGateUpMxA4, PfUpNarrowMxA4>(
                      xa, w13, w13s, sh, plan, T, H, I, E, k, hs, abuf, ybuf, act, narrow, xs, nullptr, stream);
        if (rc == MOE_OK)
            rc = launch_pf<PF_DOWN, LAYOUT, PfDownMx>(x, abuf, w2, w2s, sh.w2, sh.w2_scale, plan, T, H, I, E, k,
                                                      hs, abuf, ybuf, stream);
        return rc;
    }
    if (mx4 && xq) {  // MXFP4 weights, E4M3 activations: gate/up on the scaled MFMA
        const uint16_t* xa = reinterpret_cast<const uint16_t*>(xq);
        if (act != ACT_RELU2)
            rc = launch_pf<PF_GATEUP, LAYOUT, PfGateUpMxA8>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I,
                                                            E, k, hs, abuf, ybuf, stream, xs);
        else if (narrow)
            rc = launch_pf<PF_UP, LAYOUT, PfUpNarrowMxA8>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E,
                                                          k, hs, abuf, ybuf, stream, xs);
        else
            rc = launch_pf<PF_UP, LAYOUT, PfGateUpMxA8>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k,
                                                        hs, abuf, ybuf, stream, xs);
        if (rc == MOE_OK)
            rc = launch_pf<PF_DOWN, LAYOUT, PfDownMx>(x, abuf, w2, w2s, sh.w2, sh.w2_scale, plan, T, H, I, E, k,
                                                      hs, abuf, ybuf, stream);
        return rc;
    }
    if (mx4) {  // MXFP4 weights, bf16 activations
        if (act != ACT_RELU2)
            rc = launch_pf<PF_GATEUP, LAYOUT, PfGateUpMx>(x, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E,
                                                          k, hs, abuf, ybuf, stream);
        else if (narrow)
            rc = launch_pf<PF_UP, LAYOUT, PfUpNarrowMx>(x, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k,
                                                        hs, abuf, ybuf, stream);
        else
            rc = launch_pf<PF_UP, LAYOUT, PfGateUpMx>(x, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k,
                                                      hs, abuf, ybuf, stream);
        if (rc == MOE_OK)
            rc = launch_pf<PF_DOWN, LAYOUT, PfDownMx>(x, abuf, w2, w2s, sh.w2, sh.w2_scale, plan, T, H, I, E, k,
                                                      hs, abuf, ybuf, stream);
        return rc;
    }
    if (xq) {  // E4M3 activations with per-token scales: the fp8 x fp8 MFMA
        const uint16_t* xa = reinterpret_cast<const uint16_t*>(xq);
        if (act != ACT_RELU2)
            rc = launch_pf<PF_GATEUP, LAYOUT, PfGateUpA8>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I,
                                                          E, k, hs, abuf, ybuf, stream, xs);
        else if (narrow)
            rc = launch_pf<PF_UP, LAYOUT, PfUpNarrowA8>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E,
                                                        k, hs, abuf, ybuf, stream, xs);
        else
            rc = launch_pf<PF_UP, LAYOUT, PfGateUpA8>(xa, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k,
                                                      hs, abuf, ybuf, stream, xs);
    } else {
        if (act != ACT_RELU2)
            rc = launch_pf<PF_GATEUP, LAYOUT, PfGateUp>(x, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k,
                                                        hs, abuf, ybuf, stream);
        else if (narrow)
            rc = launch_pf<PF_UP, LAYOUT, PfUpNarrow>(x, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k,
                                                      hs, abuf, ybuf, stream);
        else
            rc = launch_pf<PF_UP, LAYOUT, PfGateUp>(x, nullptr, w13, w13s, sh.w13, ss, plan, T, H, I, E, k, hs,
                                                    abuf, ybuf, stream);
    }
    if (rc == MOE_OK)
        rc = launch_pf<PF_DOWN, LAYOUT, PfDown>(x, abuf, w2, w2s, sh.w2, sh.w2_scale, plan, T, H, I, E, k, hs,
                                                abuf, ybuf, stream);
    return rc;
}

// Host-side checks of a prefill call, before anything is launched.
int prefill_check(int T, int H, int I, int E, int k, int has_shared, int act) {
    if (!prefill_supported(H, I, act)) {
        set_error("prefill variant needs H %% 256 == 0, %s and H, I <= 65536 (got H=%d, I=%d)",
                  act == ACT_RELU2 ? "I % 128 == 0" : "2I % 256 == 0", H, I);
        return MOE_EUNSUPPORTED;
    }
    const long R = (long)T * k, rows = R + (has_shared ? T : 0);
    if ((long)T * H * 2 > 0xFFFFFFFFL || rows * I * 2 > 0xFFFFFFFFL) {
        set_error("prefill: activation matrix over 4 GB");
        return MOE_EUNSUPPORTED;
    }
    const long tiles = (R + PF_BM - 1) / PF_BM + E + (has_shared ? (T + PF_BM - 1) / PF_BM : 0);
    const long nblk = std::max(std::max(2L * I, (long)H) / 256, (long)I / 128);
    if (8L * nblk * PF_XCD_RUN * ((tiles + 8 * PF_XCD_RUN - 1) / (8 * PF_XCD_RUN)) > 0x7FFFFFFFL) {
        set_error("prefill: too many tiles");
        return MOE_EUNSUPPORTED;
    }
    return MOE_OK;
}

int launch_prefill_ffn(int layout, const uint16_t* x, const uint8_t* w13, const void* w13s,
                       const uint8_t* w2, const void* w2s, const SharedW& sh, const Plan& plan,
                       int T, int H, int I, int E, int k, uint16_t* abuf, float* ybuf,
                       int act, const uint8_t* xq, const void* xs, int afmt, int wfmt, hipStream_t stream) {
    if ((afmt == AFMT_MXFP4 || afmt == AFMT_MXFP4_H4) && wfmt != WFMT_MXFP4) {
        set_error("prefill variant: MXFP4 activations need MXFP4 weights");
        return MOE_EUNSUPPORTED;
    }
    if (afmt != AFMT_BF16 && !(xq && xs)) {
        set_error("prefill variant: quantised activations missing");
        return MOE_EINVAL;
    }

    if (!prefill_supported(H, I, act)) {
        set_error("prefill variant needs H %% 256 == 0, %s and H, I <= 65536 (got H=%d, I=%d)",
                  act == ACT_RELU2 ? "I % 128 == 0" : "2I % 256 == 0", H, I);
        return MOE_EUNSUPPORTED;
    }
    if (!plan.tile_info || !plan.tile_n || !plan.sorted_route) {
        set_error("prefill variant needs the tile list of the sort");
        return MOE_EINVAL;
    }
    if (layout == LAYOUT_TILED)
        return launch_prefill_c<LAYOUT_TILED>(x, w13, w13s, w2, w2s, sh, plan, T, H, I, E, k, abuf,
                                              ybuf, act, xq, xs, afmt, wfmt == WFMT_MXFP4, stream);
    return launch_prefill_c<LAYOUT_ROWMAJOR>(x, w13, w13s, w2, w2s, sh, plan, T, H, I, E, k, abuf,
                                             ybuf, act, xq, xs, afmt, wfmt == WFMT_MXFP4, stream);
}

}  // namespace moe
