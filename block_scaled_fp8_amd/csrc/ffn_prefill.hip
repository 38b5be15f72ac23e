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
//    of each 128-wide K block is applied by rescaling the accumulators when the
//    block starts (running scale), never by rounding it into bf16.
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
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "plan.hpp"

namespace moe {

constexpr int PF_BK = 64;  // K per stage
constexpr int PF_XCD_RUN = 8;  // consecutive row tiles an XCD takes at a time

// Workgroup tile BM rows x BN columns, WM x WN waves of 64 x 128 each (2 x 4
// MFMA tiles of 32 x 32), STAGES LDS stages of 64-wide K, OCC workgroups per
// CU (the register budget follows from it).
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int OCC_, int M16_ = 0, int A8_ = 0>
struct PfCfg {
    static constexpr int OCC = OCC_;
    // MFMA shape: v_mfma_f32_16x16x32_bf16 (M16) or v_mfma_f32_32x32x16_bf16;
    // A8: the activation operand is E4M3 (per-token scale) and the product
    // runs on v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales, fp8 x fp8
    static constexpr bool M16 = M16_ != 0;
    static constexpr bool A8 = A8_ != 0;
    static_assert(!(M16 && A8), "the fp8 path uses 32x32 tiles");
    static constexpr int MS = M16 ? 16 : 32;  // rows = columns of one MFMA tile
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int THREADS = WM * WN * MOE_WAVE;
    static constexpr int WAVES = WM * WN;
    static constexpr int STAGES = STAGES_;
    static constexpr int A_BYTES = BM * PF_BK * (A8 ? 1 : 2);  // bf16 or E4M3
    static constexpr int B_BYTES = BN * PF_BK;      // fp8
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_INSTR = A_BYTES / 1024 / WAVES;  // 1 KB loads per wave per stage
    static constexpr int B_INSTR = B_BYTES / 1024 / WAVES;
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
constexpr int PF_BM = 128;

int prefill_tile_m() { return PF_BM; }

// Widths the grouped GEMMs tile exactly (K % 128 holds for every valid call);
// the per-tile scale table (2 rows of K / 128 floats, padded to 64) must fit
// in LDS beside the stages, which holds for K <= 65536.
// relu^2 experts tile their I up columns in 256-wide blocks.
int prefill_supported(int H, int I, int act) {
    const int ncols = act == ACT_RELU2 ? I : 2 * I;
    return H % 256 == 0 && ncols % 256 == 0 && H <= 65536 && I <= 65536;
}

// PF_GATEUP: gate and up columns side by side, SwiGLU epilogue into abuf;
// PF_UP:     the up projection of a non-gated expert, relu^2 epilogue into abuf;
// PF_DOWN:   the down projection, block floating-point rows into ybuf.
enum { PF_GATEUP = 0, PF_DOWN = 1, PF_UP = 2 };

// silu(g) * u with the hardware reciprocal (about 1 ulp) in place of an IEEE
// divide; exp(-g) overflowing to +inf gives the correct limit 0.
__device__ __forceinline__ float swiglu_fast(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
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
    const uint8_t* __restrict__ wexp, const float* __restrict__ sexp,
    const uint8_t* __restrict__ wsh, const float* __restrict__ ssh, Plan plan,
    int T, int H, int I, int k, int nblk, int max_tiles,
    uint16_t* __restrict__ abuf_out, float* __restrict__ ybuf, const float* __restrict__ xscale) {
    constexpr int BM = C::BM, BN = C::BN;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ int row_tok[BM];  // gate/up: token row of x
    __shared__ __attribute__((aligned(16))) float row_xs[C::A8 ? BM : 1];  // A8: the row's x scale

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
    const uint8_t* W = e >= 0 ? wexp + (size_t)e * Nrows * K : wsh;
    const float* S = e >= 0 ? sexp + (size_t)e * (Nrows / 128) * (K / 128) : ssh;
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
            if constexpr (C::A8) row_xs[tid] = valid ? xscale[row_tok[tid]] : 0.0f;
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
    constexpr int APR = C::A8 ? 4 : 8;  // 16-byte pieces per row per stage
    const int ar_sub = lane / APR, apiece = lane % APR;
    const char* abase = GATHER ? reinterpret_cast<const char*>(x)
                               : reinterpret_cast<const char*>(abuf_in);
    uint32_t asrc[C::A_INSTR];
#pragma unroll
    for (int q = 0; q < C::A_INSTR; ++q) {
        const int row = (wave * C::A_INSTR + q) * (64 / APR) + ar_sub;
        const int sw = C::A8 ? apiece ^ ((row >> 2) & 3) : apiece ^ ((row >> 1) & 7);
        const uint32_t src_row = GATHER ? (uint32_t)row_tok[row]
                                        : (uint32_t)(p0 + (row < rows_here ? row : 0));
        asrc[q] = src_row * (uint32_t)((C::A8 ? 1 : 2) * (GATHER ? H : I)) + sw * 16;
    }
    // weights: instruction q of wave w fills 16-row tile w*B_INSTR + q
    constexpr int HALF_T = BN / 2 / 16;  // gate tiles in a gate/up tile (MODE 0)
    // (a wave-uniform tile base plus one per-lane offset, so the loads address
    //  through a scalar base; the lane's 16 bytes follow tile_lane_ptr)
    const uint8_t* bbase[C::B_INSTR];
#pragma unroll
    for (int q = 0; q < C::B_INSTR; ++q) {
        const int t16 = wave * C::B_INSTR + q;
        int wrow;
        if (PAIRED)
            wrow = (t16 < HALF_T ? 0 : I) + nb * (BN / 2) + (t16 % HALF_T) * 16;
        else
            wrow = nb * BN + t16 * 16;
        bbase[q] = W + (size_t)wrow * K;  // the tiled layout keeps whole 16-row tiles in place
    }
    const uint32_t blane = LAYOUT == LAYOUT_TILED ? lane * 16 : (lane & 15) * K + (lane >> 4) * 16;
    constexpr int CS = chunk_stride<LAYOUT>();

    auto issue_stage = [&](int st, int kc) {
        const uint32_t sbase = st * C::STAGE;
#pragma unroll
        for (int q = 0; q < C::A_INSTR; ++q)
            lds_load16(abase + (asrc[q] + (uint32_t)kc * (PF_BK * (C::A8 ? 1 : 2))),
                       sbase + (wave * C::A_INSTR + q) * 1024, smem);
#pragma unroll
        for (int q = 0; q < C::B_INSTR; ++q)
            lds_load16(bbase[q] + (size_t)kc * CS + blane, sbase + C::A_BYTES + (wave * C::B_INSTR + q) * 1024,
                       smem);
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
    //   16x16x32: sub-step s (32 K, two per step), lane quarter g: kb = 4 s + g.
    // An activation piece (16 bytes) is one kb of a row; a weight lane of the
    // staged 1 KB chunk holds kbs 2 (L / 16), 2 (L / 16) + 1 of row L % 16.
    const int l16 = lane & 15, g16 = lane >> 4;
    uint32_t a_off[4];
    uint32_t b_off;
    const int t16 = PAIRED ? wn * (C::WCOLS / 32) : wn * (C::WCOLS / 16);
    if constexpr (C::M16) {
        const int row = wm * C::WROWS + l16;
#pragma unroll
        for (int s = 0; s < 2; ++s) a_off[s] = row * 128 + (((4 * s + g16) ^ ((row >> 1) & 7)) * 16);
        a_off[2] = a_off[3] = 0;  // (two sub-steps per step)
        // 16-column tile nt is 16-row weight tile t16(nt); sub-step s's 8
        // bytes sit s * 512 bytes further on
        b_off = C::A_BYTES + t16 * 1024 + ((g16 >> 1) * 16 + l16) * 16 + (g16 & 1) * 8;
    } else {
        const int row = wm * C::WROWS + ln;
#pragma unroll
        for (int s = 0; s < 4; ++s) a_off[s] = row * 128 + (((4 * lg + s) ^ ((row >> 1) & 7)) * 16);
        // 32-column tile nt spans 16-row tiles t16(nt), t16(nt) + 1; the
        // lane's 16 bytes for half p sit p * 256 bytes further on
        const int tt = t16 + (ln >> 4), r = ln & 15;
        b_off = C::A_BYTES + tt * 1024 + (2 * lg * 16 + r) * 16;
    }
    // (MODE 0: the first NT/2 MFMA column tiles are gate columns, the rest the
    // matching up columns)
    auto a_step = [](int mt) { return mt * C::MS * 128; };
    auto b_step = [](int nt) {
        constexpr int T16 = C::MS / 16;  // 16-row weight tiles per MFMA column tile
        if (PAIRED)
            return ((nt < C::NT / 2 ? 0 : HALF_T) + (nt % (C::NT / 2)) * T16) * 1024;
        return nt * T16 * 1024;
    };
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
    {
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
    float seff[2] = {0.0f, 0.0f};

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
    constexpr int PER_STAGE = C::A_INSTR + C::B_INSTR;
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
    auto read_half = [&](int stage, int p, u32x4 (&a)[C::MT][AP], BFrag (&b)[C::NT]) {
        const char* st = smem + stage * C::STAGE;
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
            for (int j = 0; j < AP; ++j)
                a[mt][j] = *reinterpret_cast<const u32x4*>(st + a_off[AP * p + j] + a_step(mt));
        if (MTA > 0)
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
                b[nt] = *reinterpret_cast<const BFrag*>(st + b_off + p * (C::M16 ? 512 : 256) + b_step(nt));
    };
    // Part j of a half: 32x32 -- sub-step j (16 K) of every tile; 16x16 --
    // the half's 32 K for column tiles j*NT/2 .. (j+1)*NT/2 - 1 (gate/up: j = 0
    // the gate tiles, j = 1 the up tiles).  rescale: the half opens a new K
    // block, and each accumulator is multiplied by its group's factor right
    // before its first MFMA of the block.
    auto mma_sub = [&](const u32x4 (&a)[C::MT][AP], const BFrag (&b)[C::NT], int j, bool rescale,
                       const float (&rr)[2]) {
        if (MTA == 0) return;
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
            bf16x8 bf;
            if constexpr (C::M16)
                bf = fp8x8_to_bf16x8(b[nt][0], b[nt][1]);
            else
                bf = j == 0 ? fp8x8_to_bf16x8(b[nt][0], b[nt][1]) : fp8x8_to_bf16x8(b[nt][2], b[nt][3]);
            const float f = PAIRED ? rr[nt / (C::NT / 2)] : rr[0];
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
    auto next_step = [&](int kc) {
        if (C::STAGES >= 3 && kc + 2 < nk) wait_vmcnt<(C::STAGES >= 3 ? PER_STAGE : 0)>();
        else wait_vmcnt<0>();
        barrier_after_lds_reads();
        if (kc + C::STAGES < nk) issue_stage(kc % C::STAGES, kc + C::STAGES);
        // past the last step this reads a stale buffer whose values are unused
        read_half((kc + 1) % C::STAGES, 0, ah[0], bh[0]);
    };

#pragma unroll
    for (int st = 0; st < C::STAGES; ++st)
        if (st < nk) issue_stage(st, st);
    if (nk >= C::STAGES) wait_vmcnt<(C::STAGES - 1) * PER_STAGE>();
    else wait_vmcnt<PER_STAGE>();  // nk == 2: stages 0 and 1 issued
    barrier_after_lds_reads();     // stage 0 and the scale table landed in every wave
    float snext[2] = {sc_tab[sj[0] * kbp], sc_tab[sj[1] * kbp]};
    read_half(0, 0, ah[0], bh[0]);
    const float one[2] = {1.0f, 1.0f};
    for (int kb = 0; kb < kblocks; ++kb) {
        const int kc = 2 * kb;
        // running scale: a zero scale (all-zero block) keeps the current one
        float rr[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const float sn = snext[g];
            const bool take = sn != 0.0f;
            // (wave-uniform: kept in scalar registers)
            rr[g] = uniform_f32(take && seff[g] != 0.0f ? seff[g] * __builtin_amdgcn_rcpf(sn) : 1.0f);
            seff[g] = uniform_f32(take ? sn : seff[g]);
        }
        const int kn = kb + 1 < kblocks ? kb + 1 : kb;
        snext[0] = sc_tab[sj[0] * kbp + kn];
        snext[1] = sc_tab[sj[1] * kbp + kn];

        // the reads of the second half go out after the first sub-step's MFMAs,
        // whose operands were read a whole half earlier
        mma_sub(ah[0], bh[0], 0, true, rr);
        __builtin_amdgcn_sched_barrier(0);
        read_half(kc % C::STAGES, 1, ah[1], bh[1]);
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(ah[0], bh[0], 1, false, one);
        __builtin_amdgcn_sched_barrier(0);
        next_step(kc);
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(ah[1], bh[1], 0, false, one);
        mma_sub(ah[1], bh[1], 1, false, one);
        __builtin_amdgcn_sched_barrier(0);

        mma_sub(ah[0], bh[0], 0, false, one);
        __builtin_amdgcn_sched_barrier(0);
        read_half((kc + 1) % C::STAGES, 1, ah[1], bh[1]);
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(ah[0], bh[0], 1, false, one);
        __builtin_amdgcn_sched_barrier(0);
        next_step(kc + 1);
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
        auto kloop_a8 = [&](auto mta_c) {
            constexpr int MTA = decltype(mta_c)::value;
            const int r32 = lane & 31, h8 = lane >> 5;
            uint32_t a8_off[2];
    #pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wm * C::WROWS + r32;
                a8_off[j] = row * 64 + (((2 * h8 + j) ^ ((row >> 2) & 3)) * 16);
            }
            auto stage_mma = [&](int stage, bool rescale, const float (&rr)[2]) {
                const char* st = smem + stage * C::STAGE;
                i32x8 av[C::MT], bv[C::NT];
    #pragma unroll
                for (int mt = 0; mt < MTA; ++mt)
                    av[mt] = cat_i32x8(*reinterpret_cast<const u32x4*>(st + a8_off[0] + mt * 32 * 64),
                                       *reinterpret_cast<const u32x4*>(st + a8_off[1] + mt * 32 * 64));
                if (MTA > 0)
    #pragma unroll
                    for (int nt = 0; nt < C::NT; ++nt)
                        bv[nt] = cat_i32x8(*reinterpret_cast<const u32x4*>(st + b_off + b_step(nt)),
                                           *reinterpret_cast<const u32x4*>(st + b_off + b_step(nt) + 256));
    #pragma unroll
                for (int nt = 0; nt < C::NT; ++nt) {
                    const float f = PAIRED ? rr[nt / (C::NT / 2)] : rr[0];
    #pragma unroll
                    for (int mt = 0; mt < MTA; ++mt) {
                        if (rescale)
    #pragma unroll
                            for (int i = 0; i < AR; ++i) acc[mt][nt][i] *= f;
                        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            av[mt], bv[nt], acc[mt][nt], 0, 0, 0, 127, 0, 127);
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
            float snext[2] = {sc_tab[sj[0] * kbp], sc_tab[sj[1] * kbp]};
            const float one[2] = {1.0f, 1.0f};
            for (int kb = 0; kb < kblocks; ++kb) {
                const int kc = 2 * kb;
                float rr[2];
    #pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const float sn = snext[g];
                    const bool take = sn != 0.0f;
                    rr[g] = uniform_f32(take && seff[g] != 0.0f ? seff[g] * __builtin_amdgcn_rcpf(sn) : 1.0f);
                    seff[g] = uniform_f32(take ? sn : seff[g]);
                }
                const int kn = kb + 1 < kblocks ? kb + 1 : kb;
                snext[0] = sc_tab[sj[0] * kbp + kn];
                snext[1] = sc_tab[sj[1] * kbp + kn];
                stage_mma(kc % C::STAGES, true, rr);
                next_stage(kc);
                stage_mma((kc + 1) % C::STAGES, false, one);
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
        static_assert(C::WAVES * 32 * 128 * 4 <= C::STAGES * C::STAGE, "slabs fit the stages");
        __syncthreads();  // every wave is done reading the K stages
        float* slab = reinterpret_cast<float*>(smem) + wave * (32 * 128);
        uint8_t* ybytes = reinterpret_cast<uint8_t*>(ybuf);
        const size_t rowb = (size_t)H * 2 + (size_t)(H / 8);
        const int col0 = nb * BN + wn * C::WCOLS;  // first column of the wave tile
        const float sc = seff[0];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
                for (int i = 0; i < AR; ++i)
                    slab[(8 * (i >> 2) + 4 * lg + (i & 3)) * 128 + nt * 32 + ln] = acc[mt][nt][i] * sc;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slab is written
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int r = 4 * q + (lane >> 4);   // row of the slab
                const int c = 8 * (lane & 15);       // the lane's first column
                const int m = wm * C::WROWS + mt * 32 + r;  // row of the tile
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(slab + r * 128 + c);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(slab + r * 128 + c + 4);
                if (m < rows_here) {
                    u32x4 mant;
                    uint32_t ex;
                    bfp16x8_encode(v0, v1, mant, ex);
                    uint8_t* rowp = ybytes + (size_t)(p0 + m) * rowb;
                    __builtin_nontemporal_store(mant, reinterpret_cast<u32x4*>(rowp + 2 * (size_t)(col0 + c)));
                    __builtin_nontemporal_store((uint8_t)ex, rowp + 2 * (size_t)H + (col0 + c) / 8);
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
    static_assert(C::WAVES * C::WROWS * OUTC * 2 <= C::STAGES * C::STAGE, "slabs fit the stages");
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
            if constexpr (C::A8) xsv = row_xs[wm * C::WROWS + r];
            if constexpr (MODE == PF_GATEUP) {
                const float s0 = seff[0] * xsv, s1 = seff[1] * xsv;
#pragma unroll
                for (int nt = 0; nt < C::NT / 2; ++nt)
                    slab[r * OUTC + nt * C::MS + ocol] = f32_to_bf16_bits(
                        swiglu_fast(acc[mt][nt][i] * s0, acc[mt][nt + C::NT / 2][i] * s1));
            } else {
                const float s0 = seff[0] * xsv;
#pragma unroll
                for (int nt = 0; nt < C::NT; ++nt)
                    slab[r * OUTC + nt * C::MS + ocol] = f32_to_bf16_bits(relu2(acc[mt][nt][i] * s0));
            }
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slab is written
    __builtin_amdgcn_wave_barrier();
    const int colbase = MODE == PF_GATEUP ? nb * (BN / 2) + wn * (C::WCOLS / 2) : nb * BN + wn * C::WCOLS;
#pragma unroll
    for (int q = 0; q < C::WROWS / RPS; ++q) {
        const int r = q * RPS + lane / LPR;
        const int c = 8 * (lane % LPR);
        const int m = wm * C::WROWS + r;  // row of the tile
        const u32x4 v = *reinterpret_cast<const u32x4*>(slab + r * OUTC + c);
        if (m < rows_here)
            *reinterpret_cast<u32x4*>(abuf_out + (size_t)(p0 + m) * I + colbase + c) = v;
    }
}

template <int MODE>
static inline int K_of(int H, int I) { return MODE == PF_DOWN ? I : H; }

template <int MODE, int LAYOUT, class C>
static int launch_pf(const uint16_t* x, const uint16_t* abuf_in, const uint8_t* wexp,
                     const float* sexp, const uint8_t* wsh, const float* ssh, const Plan& plan,
                     int T, int H, int I, int E, int k, int has_shared, uint16_t* abuf_out,
                     float* ybuf, hipStream_t stream, const float* xscale = nullptr) {
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
    const size_t a_bytes = MODE != PF_DOWN ? (size_t)T * H * (C::A8 ? 1 : 2)
                                           : (size_t)(R + (has_shared ? T : 0)) * I * 2;
    if (a_bytes > 0xFFFFFFFFull) {
        set_error("prefill: activation matrix over 4 GB");
        return MOE_EUNSUPPORTED;
    }
    const size_t kbp = ((size_t)K_of<MODE>(H, I) / 128 + 63) / 64 * 64;
    const size_t lds = (size_t)C::STAGES * C::STAGE + (size_t)(C::BN / 128) * kbp * 4;
    const char* pname = MODE == PF_DOWN ? "prefill_down"
                        : MODE == PF_UP ? (C::A8 ? "prefill_up_relu2_a8" : "prefill_up_relu2")
                                        : (C::A8 ? "prefill_gateup_swiglu_a8" : "prefill_gateup_swiglu");
    prof_begin(pname, stream);
    prefill_gemm_kernel<MODE, LAYOUT, C><<<(unsigned)grid, C::THREADS, lds, stream>>>(
        x, abuf_in, wexp, sexp, wsh, ssh, plan, T, H, I, k, nblk, (int)max_tiles, abuf_out, ybuf,
        xscale);
    prof_end(stream);
    return check_launch(MODE == PF_GATEUP ? "prefill_gemm_kernel<gateup>"
                                          : (MODE == PF_UP ? "prefill_gemm_kernel<up>" : "prefill_gemm_kernel<down>"));
}

template <int LAYOUT>
static int launch_prefill_c(const uint16_t* x, const uint8_t* w13, const float* w13s,
                            const uint8_t* w2, const float* w2s, const SharedW& sh,
                            const Plan& plan, int T, int H, int I, int E, int k, uint16_t* abuf,
                            float* ybuf, int act, const uint8_t* xq, const float* xs,
                            hipStream_t stream) {
    const int hs = sh.w13 != nullptr;
    int rc;
    if (xq) {  // E4M3 activations with per-token scales: the fp8 x fp8 MFMA
        const uint16_t* xa = reinterpret_cast<const uint16_t*>(xq);
        rc = act == ACT_RELU2
                 ? launch_pf<PF_UP, LAYOUT, PfGateUpA8>(xa, nullptr, w13, w13s, sh.w13,
                                                        sh.w13_scale, plan, T, H, I, E, k, hs,
                                                        abuf, ybuf, stream, xs)
                 : launch_pf<PF_GATEUP, LAYOUT, PfGateUpA8>(xa, nullptr, w13, w13s, sh.w13,
                                                            sh.w13_scale, plan, T, H, I, E, k, hs,
                                                            abuf, ybuf, stream, xs);
    } else {
        rc = act == ACT_RELU2
                 ? launch_pf<PF_UP, LAYOUT, PfGateUp>(x, nullptr, w13, w13s, sh.w13, sh.w13_scale,
                                                      plan, T, H, I, E, k, hs, abuf, ybuf, stream)
                 : launch_pf<PF_GATEUP, LAYOUT, PfGateUp>(x, nullptr, w13, w13s, sh.w13,
                                                          sh.w13_scale, plan, T, H, I, E, k, hs,
                                                          abuf, ybuf, stream);
    }
    if (rc == MOE_OK)
        rc = launch_pf<PF_DOWN, LAYOUT, PfDown>(x, abuf, w2, w2s, sh.w2, sh.w2_scale, plan, T, H, I,
                                                E, k, hs, abuf, ybuf, stream);
    return rc;
}

// Host-side checks of a prefill call, before anything is launched.
int prefill_check(int T, int H, int I, int E, int k, int has_shared, int act) {
    if (!prefill_supported(H, I, act)) {
        set_error("prefill variant needs H %% 256 == 0, %s %% 256 == 0 and H, I <= 65536 (got H=%d, I=%d)",
                  act == ACT_RELU2 ? "I" : "2I", H, I);
        return MOE_EUNSUPPORTED;
    }
    const long R = (long)T * k, rows = R + (has_shared ? T : 0);
    if ((long)T * H * 2 > 0xFFFFFFFFL || rows * I * 2 > 0xFFFFFFFFL) {
        set_error("prefill: activation matrix over 4 GB");
        return MOE_EUNSUPPORTED;
    }
    const long tiles = (R + PF_BM - 1) / PF_BM + E + (has_shared ? (T + PF_BM - 1) / PF_BM : 0);
    const long nblk = std::max(2L * I, (long)H) / 256;
    if (8L * nblk * PF_XCD_RUN * ((tiles + 8 * PF_XCD_RUN - 1) / (8 * PF_XCD_RUN)) > 0x7FFFFFFFL) {
        set_error("prefill: too many tiles");
        return MOE_EUNSUPPORTED;
    }
    return MOE_OK;
}

int launch_prefill_ffn(int layout, const uint16_t* x, const uint8_t* w13, const float* w13s,
                       const uint8_t* w2, const float* w2s, const SharedW& sh, const Plan& plan,
                       int T, int H, int I, int E, int k, uint16_t* abuf, float* ybuf,
                       int act, const uint8_t* xq, const float* xs, hipStream_t stream) {
    if (!prefill_supported(H, I, act)) {
        set_error("prefill variant needs H %% 256 == 0, %s %% 256 == 0 and H, I <= 65536 (got H=%d, I=%d)",
                  act == ACT_RELU2 ? "I" : "2I", H, I);
        return MOE_EUNSUPPORTED;
    }
    if (!plan.tile_info || !plan.tile_n || !plan.sorted_route) {
        set_error("prefill variant needs the tile list of the sort");
        return MOE_EINVAL;
    }
    if (layout == LAYOUT_TILED)
        return launch_prefill_c<LAYOUT_TILED>(x, w13, w13s, w2, w2s, sh, plan, T, H, I, E, k, abuf,
                                              ybuf, act, xq, xs, stream);
    return launch_prefill_c<LAYOUT_ROWMAJOR>(x, w13, w13s, w2, w2s, sh, plan, T, H, I, E, k, abuf,
                                             ybuf, act, xq, xs, stream);
}

}  // namespace moe
