// Decode variant, one workgroup per active expert (or, after the sort, per
// row tile of an expert's routes): gate/up GEMM -> SwiGLU -> down GEMM in a
// single launch, the SwiGLU activations kept in LDS.
//
// Source: "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for
// Trainium2", section "FP8 MoE decode kernel (moe_fused_w8_35b)": the fused
// local routed experts (gate/up GEMM -> SwiGLU -> down GEMM -> affinity scale
// -> expert-sum) on E4M3FN weights with 128x128 block scales, decoded to BF16
// tile by tile.
//
// gfx950 design.  At decode every active expert moves the same 3*H*I weight
// bytes and does little arithmetic, so giving each active expert one
// workgroup balances HBM traffic across the CUs with no inter-workgroup
// dependency: phase 1 streams W13 (gate and matching up rows in the same
// wave, SwiGLU in registers, bf16 result into LDS), one barrier, phase 2
// streams W2 against the LDS activations and writes fp32 rows of the routes.
// Each wave streams 4 tiles of 16 weight rows per pass; lane l loads 16 consecutive
// FP8 bytes of row l%16 at K offset 16*(l/16) of each 64-wide chunk
// (global_load_dwordx4), which is the operand layout of
// v_mfma_f32_16x16x32_bf16 after an exact FP8 -> bf16 conversion; the token
// operand uses the same K permutation, so every MFMA computes exact K sums.
//
// Block scales: the MFMAs of each 128-wide K block accumulate a fresh fp32
// partial, which joins the tile's total as total += scale * partial when the
// block ends.  Every block is therefore weighted by exactly its own fp32
// scale, whatever the scales of its neighbours: a zero scale adds exactly 0
// (for finite activations), and subnormal or widely different scales are
// multiplied in as they are.  The scale is never rounded into bf16.
#include "common.hpp"
#include "plan.hpp"

namespace moe {

constexpr int DF_THREADS = 512;
constexpr int DF_WAVES = DF_THREADS / MOE_WAVE;
constexpr int DF_NT = 4;  // weight tiles (16 rows each) per wave pass

// Per wave, the weight tiles of both phases form ONE stream of 64-wide K
// chunks: its phase-1 groups (HALF gate tiles + the matching HALF up tiles),
// then its phase-2 groups (NT row tiles of W2).  DEPTH chunks are always in
// flight: the refill for position p+DEPTH is issued right after position p is
// consumed, across group ends and across the phase boundary (phase-2 weights
// do not depend on the activations, so they are fetched before the barrier).
//
// Every wave runs the same, static sequence: all chunk counts are even
// (K % 128 == 0); a wave with fewer real groups than the others re-streams a
// valid tile and writes its results into LDS padding columns or a trash row of
// y; rows past the workgroup's routes write to the trash row too.  With no conditional
// loads or stores (global stores also count on the vector-memory counter of
// gfx9-class GPUs), the compiler's wait counts stay partial and the pipeline
// never drains mid-stream.
constexpr int DF_HALF = DF_NT / 2;
constexpr int DF_XCD_RUN = 8;  // sorted form: consecutive row tiles an XCD takes at a time

// Self-routed mode (decode batches of at most DF_SELF_MAX_ROUTES routes): the
// workgroup of expert e finds its own routes by scanning the ids (wave ballots,
// ascending route order, the same order as the stable sort), so the step needs
// no separate sort launch.  Workgroup E is the shared expert.
constexpr int DF_SELF_MAX_ROUTES = 4096;
constexpr int DF_SELF_IDS_PER_THREAD = DF_SELF_MAX_ROUTES / DF_THREADS;
// dynamic LDS a workgroup may take: 160 KB less room for the kernel's static
// arrays (the route scan's per-round wave counts)
constexpr size_t DF_LDS_DYNAMIC_MAX = 160 * 1024 - 1024;

// LDS: the SwiGLU activations [16 MT][I + 8], then (x staged) the pass's
// token rows of x [16 MT][H + 8], then (self-routed) the expert's routes.
// alias: x and the activations share one region (the activations are written
// once phase 1 has read all of x).
size_t decode_fused_lds_bytes(int MT, int I, int self_routes, int H, bool alias) {
    const size_t a = sizeof(uint16_t) * (size_t)(16 * MT) * (I + 8);
    const size_t xb = H > 0 ? sizeof(uint16_t) * (size_t)(16 * MT) * (H + 8) : 0;
    return (alias ? std::max(a, xb) : a + xb) + sizeof(int32_t) * (size_t)self_routes;
}

// The pass's x rows go to LDS (and every wave reads its operands there
// instead of re-reading them from L2 for each weight chunk) when a row is a
// whole number of 1 KB wave loads and everything fits one workgroup's LDS.
bool decode_fused_x_in_lds(int MT, int H, int I, int self_routes) {
    return H % 512 == 0 && decode_fused_lds_bytes(MT, I, self_routes, H) <= DF_LDS_DYNAMIC_MAX;
}

// Phase-1 groups per wave (as the kernel counts them).
static int decode_fused_groups1(int H, int I, bool relu2, bool mx4) {
    const int nch1 = H / (mx4 ? 128 : 64);
    const int G1 = I / (16 * (relu2 ? DF_NT : DF_HALF));
    int n1 = (G1 + DF_WAVES - 1) / DF_WAVES;
    return n1 + (nch1 & n1 & 1);
}

// RELU2: a non-gated expert, w13 = the up projection [I, H] alone; a phase-1
// group is NT up tiles (64 rows, inside one 128-row scale block) and the
// activation is relu(u)^2.
//
// MX4: MXFP4 weights (two E2M1 codes a byte, element 2j in the low nibble of
// byte j; one E8M0 scale per 32 consecutive elements of a row).  A chunk is
// then 128 K (the same 16 bytes a lane, 64 bytes a row): lane quarter g holds
// K [32g, 32g + 32) of the chunk, exactly one scale block, and its scale,
// a power of two, is applied exactly by the bf16 conversion (converter scale
// operand), so the MFMAs accumulate over all of K with no rescaling.  Four
// MFMA sub-steps per chunk, sub-step s taking K [32g + 8s, 32g + 8s + 8) of
// both operands.  Scales are void pointers: fp32 [rows/128][K/128] blocks, or
// E8M0 bytes [rows][K/32] for MX4.
//
// XLDS: the token rows of each pass are staged in LDS once (direct-to-LDS
// wave loads), and phase 1 reads its activation operands there.
// XA (with XLDS; at most two phase-1 groups a wave): x and the activations
// share LDS.  Phase 1 keeps its SwiGLU results in registers, and they go to
// LDS once every wave has read the last of x.
template <int MT, int DEPTH, int LAYOUT, bool SELF, bool RELU2, bool MX4, bool XLDS, bool XA = false>
__global__ __launch_bounds__(DF_THREADS) void decode_fused_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13,
    const void* __restrict__ w13s, const uint8_t* __restrict__ w2,
    const void* __restrict__ w2s, const uint8_t* __restrict__ sh_w13,
    const void* __restrict__ sh_w13s, const uint8_t* __restrict__ sh_w2,
    const void* __restrict__ sh_w2s, Plan plan, const int32_t* __restrict__ ids, int E,
    const float* __restrict__ aff, int T, int H, int I, int k, float* __restrict__ ybuf,
    int ytrash_row, int tile_cap) {
    // two 64-wide chunks per 128-wide scale block, two in flight: the chunk
    // in flight slot d is the block's first (d = 0) or second (d = 1) half
    static_assert(DEPTH == 2, "chunks per 128-wide scale block");
    static_assert(!XA || XLDS, "the shared region holds staged x rows");
    constexpr int MROWS = 16 * MT, NT = DF_NT, HALF = DF_HALF;
    constexpr int CS = chunk_stride<LAYOUT>();
    extern __shared__ uint16_t a_lds[];  // [MROWS][I + 8] bf16 SwiGLU activations
    const int astride = I + 8;  // +16 bytes per row: conflict-free 16-byte column reads
    const int xstride = H + 8;  // (XLDS) x rows, padded likewise
    uint16_t* x_lds = XA ? a_lds : a_lds + (size_t)MROWS * astride;
    const size_t region = XA ? (size_t)MROWS * (size_t)max(astride, xstride)
                             : (size_t)MROWS * astride + (XLDS ? (size_t)MROWS * xstride : 0);
    const int lane = lane_id(), wave = wave_id();
    const int R = T * k;
    int e, row0, rows;
    int32_t* rlist = reinterpret_cast<int32_t*>(a_lds + region);  // SELF: routes of e
    if (SELF) {
        const int b = blockIdx.x;
        if (b > E || (b == E && sh_w13 == nullptr)) return;
        e = b < E ? b : -1;
        row0 = 0;
        rows = T;
        if (e >= 0) {
            // every round's per-wave counts first (one barrier), then the
            // positions: round c, wave w's hits follow all earlier rounds'
            // and round c's earlier waves'
            __shared__ int wcnt[DF_SELF_IDS_PER_THREAD][DF_WAVES];
            int idv[DF_SELF_IDS_PER_THREAD];
            uint64_t hm[DF_SELF_IDS_PER_THREAD];
#pragma unroll
            for (int c = 0; c < DF_SELF_IDS_PER_THREAD; ++c) {
                const int r = c * DF_THREADS + (int)threadIdx.x;
                idv[c] = r < R ? ids[r] : -1;
            }
#pragma unroll
            for (int c = 0; c < DF_SELF_IDS_PER_THREAD; ++c) {
                if (c * DF_THREADS >= R) break;  // uniform
                hm[c] = __ballot(idv[c] == e);
                if (lane == 0) wcnt[c][wave] = (int)__popcll(hm[c]);
            }
            __syncthreads();
            int base = 0;
#pragma unroll
            for (int c = 0; c < DF_SELF_IDS_PER_THREAD; ++c) {
                if (c * DF_THREADS >= R) break;  // uniform
                int woff = 0, tot = 0;
#pragma unroll
                for (int w = 0; w < DF_WAVES; ++w) {
                    const int cw = wcnt[c][w];
                    woff += w < wave ? cw : 0;
                    tot += cw;
                }
                if (idv[c] == e)
                    rlist[base + woff + (int)__popcll(hm[c] & lanemask_lt())] = c * DF_THREADS + (int)threadIdx.x;
                base += tot;
            }
            __syncthreads();  // rlist complete
            rows = base;
            if (rows == 0) return;  // the same value in every thread
        }
    } else {
        // one row tile of the sort's list (at most MROWS rows of one
        // segment).  Runs of DF_XCD_RUN consecutive tiles go to one XCD
        // (workgroups are dealt round-robin over the 8 XCDs), so the tiles of
        // one expert re-read its weights from that XCD's L2.  The record and
        // the tile count load together, so one memory latency passes before
        // the weights are known (the index is clamped to the list's
        // capacity, the record then unused).
        const int b = blockIdx.x, j = b >> 3;
        const int tile = (j / DF_XCD_RUN) * (8 * DF_XCD_RUN) + (b & 7) * DF_XCD_RUN + j % DF_XCD_RUN;
        const int ntiles = plan.tile_n[0];
        const int4 ti = plan.tile_info[min(tile, tile_cap - 1)];
        if (tile >= ntiles) return;
        e = ti.x;
        row0 = ti.y;
        rows = ti.z;
    }
    // route index of the m-th row of this workgroup (shared expert: R + token)
    auto route_of = [&](int m) -> int {
        if (e < 0) return (SELF ? R : row0) + m;
        return SELF ? rlist[m] : plan.sorted_route[row0 + m];
    };
    const int n13 = RELU2 ? I : 2 * I;  // rows of the expert's first matrix
    constexpr int KC = MX4 ? 128 : 64;  // K per 64-byte chunk of a weight row
    constexpr int NS = KC / 32;         // MFMA sub-steps (16-byte activation pieces) per chunk
    const int H8 = MX4 ? H / 2 : H, I8 = MX4 ? I / 2 : I;  // weight row strides in bytes
    const uint8_t* W13 = e >= 0 ? w13 + (size_t)e * n13 * H8 : sh_w13;
    const uint8_t* W2 = e >= 0 ? w2 + (size_t)e * H * I8 : sh_w2;
    // fp32 128x128 block scales, or (MX4) E8M0 bytes per 32 elements of a row
    const size_t s13n = MX4 ? (size_t)n13 * (H / 32) : (size_t)(n13 / 128) * (H / 128);
    const size_t s2n = MX4 ? (size_t)H * (I / 32) : (size_t)(H / 128) * (I / 128);
    const void* S13v = e >= 0 ? static_cast<const char*>(w13s) + (MX4 ? 1 : 4) * (size_t)e * s13n : sh_w13s;
    const void* S2v = e >= 0 ? static_cast<const char*>(w2s) + (MX4 ? 1 : 4) * (size_t)e * s2n : sh_w2s;
    const float* S13 = static_cast<const float*>(S13v);
    const float* S2 = static_cast<const float*>(S2v);
    const uint8_t* M13 = static_cast<const uint8_t*>(S13v);
    const uint8_t* M2 = static_cast<const uint8_t*>(S2v);

    const int ln = lane & 15, lg = lane >> 4;

    const int nch1 = H / KC, nch2 = I / KC;  // chunks per group (even unless MX4)
    const int kb1 = H >> 7, kb2 = I >> 7;    // 128-wide scale blocks along K
    const int G1 = I / (16 * (RELU2 ? NT : HALF)), G2 = H / (16 * NT);
    int n1 = (G1 + DF_WAVES - 1) / DF_WAVES, n2 = (G2 + DF_WAVES - 1) / DF_WAVES;
    // the stream advances DEPTH = 2 positions at a time, so each phase takes an
    // even number of chunks: with an odd chunk count (MX4, K = 128 * odd) a
    // wave streams one more spare group, whose results go to padding
    n1 += (nch1 & n1 & 1);
    n2 += (nch2 & n2 & 1);
    const int tot1 = n1 * nch1, tot2 = n2 * nch2;

    for (int mp = 0; mp < rows; mp += MROWS) {
        if (mp > 0) __syncthreads();  // the previous pass has finished reading a_lds
        // (32-bit offsets and indices keep the registers for the block totals)
        uint32_t xoff[MT];   // element offset of this lane's x row piece (x is under 4 GB)
        bool xvalid[MT];
        uint32_t aoff[MT];   // element offset of this lane's activation row piece in a_lds
        int yrow[MT][4];     // y row of this lane's output rows (the trash row if padded)
        float yaff[MT][4];   // affinity of each of those routes
        u32x4 bq[DEPTH][NT];
        uint32_t sq[DEPTH][NT];  // MX4: the lane's E8M0 scale byte of each tile's chunk
        u32x4 aq[DEPTH][MT][NS];
        f32x4 acc[MT][NT];  // partial sums of the current 128-wide K block
        f32x4 tot[MT][NT];  // scaled totals of the finished blocks
        // XA: the bf16 activations of the wave's first and second phase-1
        // groups, two a register, until x has been read
        constexpr int JN = RELU2 ? NT : HALF;
        uint32_t hold0[MT][JN][2], hold1[MT][JN][2];
        float sc0 = 0.0f, sc1 = 0.0f;  // scales of the current block (phase 1: gate, up; phase 2: sc0)
        auto reset = [&]() {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    tot[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        };
        // the block ends: its partial, times its own scale, joins the total
        // (the block's first MFMAs start the next partial from zero)
        auto fold = [&](float sc, int j0, int j1) {
#pragma unroll
            for (int j = j0; j < j1; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) tot[mt][j] += sc * acc[mt][j];
        };
        // av(mt, s): the activation operand of row tile mt, sub-step s (read
        // at its sub-step, so only one sub-step's pieces are live at a time)
        auto mfma_chunk = [&](int d, auto&& av) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                u32x4 a[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) a[mt] = av(mt, s);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    bf16x8 b;
                    if constexpr (MX4)
                        b = fp4x8_to_bf16x8_scaled(bq[d][j][s], __uint_as_float(sq[d][j] << 23));
                    else
                        b = s == 0 ? fp8x8_to_bf16x8(bq[d][j][0], bq[d][j][1])
                                   : fp8x8_to_bf16x8(bq[d][j][2], bq[d][j][3]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(a[mt]), b,
                            !MX4 && d == 0 && s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mt][j],
                            0, 0, 0);
                }
                // (MX4: keeps the scheduler from hoisting every sub-step's
                // operand reads, which spilled the 32-row passes)
                if constexpr (MX4) __builtin_amdgcn_sched_barrier(0);
            }
        };

        // ---- issue side: phase-1 group g has gate tiles g*HALF+j and up tiles
        //      I/16 + g*HALF + j; phase-2 group g has W2 row tiles g*NT + j.
        //      Groups past the real count re-stream group g % G.
        int ig = wave, ic = 0;  // issue cursor (group, chunk)
        // (MX4: row r's scale of K [KC c + 32 lg, +32) is byte r * K/32 + 4c + lg,
        //  or in the tiled layout byte ((r / 16) * K/128 + c) * 64 + lane)
        auto issue1_b = [&](int d, int g, int c) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int r = RELU2 ? (g * NT + j) * 16 : (j < HALF ? 0 : I) + (g * HALF + (j % HALF)) * 16;
                bq[d][j] = load_stream16(tile_lane_ptr<LAYOUT>(W13, r, H8, lane) + (size_t)c * CS);
                if constexpr (MX4)
                    sq[d][j] = LAYOUT == LAYOUT_TILED
                                   ? M13[((size_t)(r >> 4) * (H / 128) + c) * 64 + lane]
                                   : M13[(size_t)(r + ln) * (H / 32) + 4 * c + lg];
            }
        };
        auto issue1_a = [&](int d, int c) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4* q = reinterpret_cast<const u32x4*>(x + xoff[mt] + c * KC);
#pragma unroll
                for (int s = 0; s < NS; ++s) aq[d][mt][s] = q[s];
            }
        };
        auto issue1 = [&](int d) {
            issue1_b(d, ig % G1, ic);
            if (!XLDS) issue1_a(d, ic);
            if (++ic == nch1) { ic = 0; ig += DF_WAVES; }
        };
        auto issue2 = [&](int d) {
            const int g = ig % G2;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                bq[d][j] = load_stream16(tile_lane_ptr<LAYOUT>(W2, (g * NT + j) * 16, I8, lane) +
                                         (size_t)ic * CS);
                if constexpr (MX4)
                    sq[d][j] = LAYOUT == LAYOUT_TILED
                                   ? M2[((size_t)(g * NT + j) * (I / 128) + ic) * 64 + lane]
                                   : M2[(size_t)((g * NT + j) * 16 + ln) * (I / 32) + 4 * ic + lg];
            }
            if (++ic == nch2) { ic = 0; ig += DF_WAVES; }
        };

        // a tile's result at the end of its group: the scaled block totals,
        // or (MX4, scales applied in the conversion) the accumulator itself
        auto res = [&](int mt, int j, int i) -> float { return MX4 ? acc[mt][j][i] : tot[mt][j][i]; };

        // ---- process side
        int pg = wave, pc = 0;
        auto proc1 = [&](int d) {
            const int g = pg % G1;
            if (!MX4 && d == 0) {  // a block starts: its scales
                const int kb = pc >> 1;
                if (RELU2) {
                    const int ui = __builtin_amdgcn_readfirstlane(((g * NT * 16) >> 7) * kb1 + kb);
                    sc0 = S13[ui];
                } else {
                    const int gi = __builtin_amdgcn_readfirstlane(((g * HALF * 16) >> 7) * kb1 + kb);
                    const int ui = __builtin_amdgcn_readfirstlane(((I + g * HALF * 16) >> 7) * kb1 + kb);
                    sc0 = S13[gi];
                    sc1 = S13[ui];
                }
            }
            mfma_chunk(d, [&](int mt, int s) -> u32x4 {
                if (!xvalid[mt]) return u32x4{0u, 0u, 0u, 0u};
                if constexpr (XLDS)
                    return reinterpret_cast<const u32x4*>(x_lds + xoff[mt] + pc * KC)[s];
                else
                    return aq[d][mt][s];
            });
            if (!MX4 && d == 1) {  // the block's second chunk: fold it
                if (RELU2) {
                    fold(sc0, 0, NT);
                } else {
                    fold(sc0, 0, HALF);
                    fold(sc1, HALF, NT);
                }
            }
            if (pc == nch1 - 1) {  // group done: activations into LDS (padding columns if spare)
                const bool real = pg < G1;
                // activation (mt, j, i) of the group, as bf16 bits
                auto act = [&](int mt, int j, int i) -> uint32_t {
                    return RELU2 ? f32_to_bf16_bits(relu2(res(mt, j, i)))
                                 : f32_to_bf16_bits(swiglu(res(mt, j, i), res(mt, HALF + j, i)));
                };
                if constexpr (XA) {
                    const bool first = pg < DF_WAVES;  // (the wave's groups are wave, wave + 8)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int j = 0; j < JN; ++j)
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                const uint32_t v = act(mt, j, 2 * h) | (act(mt, j, 2 * h + 1) << 16);
                                if (first) hold0[mt][j][h] = v;
                                else hold1[mt][j][h] = v;
                            }
                } else {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int j = 0; j < JN; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int m = mt * 16 + lg * 4 + i;
                                const int col = real ? (g * JN + j) * 16 + ln : I + (ln & 7);
                                a_lds[m * astride + col] = (uint16_t)act(mt, j, i);
                            }
                }
                reset();
                pc = 0;
                pg += DF_WAVES;
            } else {
                ++pc;
            }
        };
        auto proc2 = [&](int d) {
            const int g = pg % G2;
            if (!MX4 && d == 0) {
                const int si = __builtin_amdgcn_readfirstlane(((g * NT * 16) >> 7) * kb2 + (pc >> 1));
                sc0 = S2[si];
            }
            mfma_chunk(d, [&](int mt, int s) -> u32x4 {
                return reinterpret_cast<const u32x4*>(a_lds + aoff[mt] + pc * KC)[s];
            });
            if (!MX4 && d == 1) fold(sc0, 0, NT);
            if (pc == nch2 - 1) {  // group done: fp32 rows of the routes (trash if spare)
                const bool real = pg < G2;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float* dst = ybuf + (size_t)(real ? yrow[mt][i] : ytrash_row) * H +
                                     (real ? g * NT * 16 : 0) + ln;
                        const float a = yaff[mt][i];
#pragma unroll
                        for (int j = 0; j < NT; ++j) dst[j * 16] = res(mt, j, i) * a;
                    }
                reset();
                pc = 0;
                pg += DF_WAVES;
            } else {
                ++pc;
            }
        };

        reset();
        // weight prologue first (it needs only the expert), then the token ids;
        // the first DEPTH stream positions may cross a group end (one chunk a
        // group: MX4 with K = 128)
        int pcd[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            pcd[d] = ic;
            issue1_b(d, ig % G1, ic);
            if (++ic == nch1) { ic = 0; ig += DF_WAVES; }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mp + mt * 16 + ln;
            int t = -1;
            if (m < rows) t = e >= 0 ? route_of(m) / k : route_of(m) - R;
            xvalid[mt] = t >= 0;
            xoff[mt] = (uint32_t)(t >= 0 ? t : 0) * (uint32_t)H + lg * (KC / 4);
            aoff[mt] = (uint32_t)((mt * 16 + ln) * astride + lg * (KC / 4));
            // (XLDS: the phase-1 operand offset in x_lds, from x_lds)
            if (XLDS) xoff[mt] = (uint32_t)((mt * 16 + ln) * xstride + lg * (KC / 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mi = mp + mt * 16 + lg * 4 + i;
                int r = -1;
                float a = 0.0f;
                if (mi < rows) {
                    r = route_of(mi);
                    a = e >= 0 ? aff[r] : 1.0f;
                }
                yrow[mt][i] = r >= 0 ? r : ytrash_row;
                yaff[mt][i] = a;
            }
        }
        if constexpr (XLDS) {
            // stage the pass's token rows: wave w loads rows w, w + 8, ...; a
            // wave load moves 1 KB of one row (padding rows read token 0)
            const int per_row = H / 512;
            for (int r = wave; r < MROWS; r += DF_WAVES) {
                const int m = mp + r;
                int t = 0;
                if (m < rows) t = e >= 0 ? route_of(m) / k : route_of(m) - R;
                t = __builtin_amdgcn_readfirstlane(t < 0 ? 0 : t);
                const uint16_t* src = x + (size_t)t * H + lane * 8;
                char* dst = reinterpret_cast<char*>(x_lds) + (size_t)r * xstride * 2;
                for (int i = 0; i < per_row; ++i)
                    __builtin_amdgcn_global_load_lds(src + i * 512, dst + i * 1024, 16, 0, 0);
            }
            __syncthreads();  // (waits for the loads too) every x row is in LDS
        } else {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) issue1_a(d, pcd[d]);
        }
        int p0 = 0;
        for (; p0 + DEPTH < tot1; p0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                proc1(d);
                issue1(d);
            }
        }
        ig = wave;
        ic = 0;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {  // last phase-1 chunks; refills start phase 2
            proc1(d);
            issue2(d);
        }
        if constexpr (XA) {
            __syncthreads();  // every wave has read the last of x: its region takes the activations
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int pgh = wave + hh * DF_WAVES;
                if (pgh >= n1 * DF_WAVES) break;  // (uniform) the wave's groups
                const int g = pgh % G1;
                const bool real = pgh < G1;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int j = 0; j < JN; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t v = (hh == 0 ? hold0 : hold1)[mt][j][i >> 1];
                            const int m = mt * 16 + lg * 4 + i;
                            const int col = real ? (g * JN + j) * 16 + ln : I + (ln & 7);
                            a_lds[m * astride + col] = (uint16_t)((i & 1) ? v >> 16 : v & 0xFFFFu);
                        }
            }
        }
        __syncthreads();  // every activation column is in LDS
        pg = wave;
        pc = 0;
        for (int q0 = 0; q0 + DEPTH < tot2; q0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                proc2(d);
                issue2(d);
            }
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) proc2(d);
    }
}

template <int LAYOUT, bool SELF, bool RELU2, bool MX4>
static int launch_decode_fused_l(int MT, const uint16_t* x, const uint8_t* w13, const void* w13s,
                                 const uint8_t* w2, const void* w2s, const SharedW& sh,
                                 const Plan& plan, const int32_t* ids, const float* aff, int T,
                                 int H, int I, int E, int k, float* ybuf, hipStream_t stream) {
    // self-routed: one workgroup per possible segment (E routed + shared);
    // sorted: one per row tile of 16 MT rows (a segment longer than one
    // pass spreads over several workgroups).  Workgroups past the real
    // count exit at once.
    // (sorted: the grid is the capacity rounded up to whole rounds of
    // 8 * DF_XCD_RUN, so that the tile dealing covers every index below it)
    const size_t cap = SELF ? 0 : decode_fused_tile_capacity(T, k, E, sh.w13 ? 1 : 0, 16 * MT);
    const size_t nwg = SELF ? (size_t)E + (sh.w13 ? 1 : 0)
                            : (cap + 8 * DF_XCD_RUN - 1) / (8 * DF_XCD_RUN) * (8 * DF_XCD_RUN);
    if (!SELF && (!plan.tile_info || !plan.tile_n)) {
        set_error("decode: the sorted fused kernel needs the sort's tile list");
        return MOE_EINVAL;
    }
    if (nwg > 0x7FFFFFFFu) {
        set_error("decode: too many row tiles");
        return MOE_EUNSUPPORTED;
    }
    const int routes = SELF ? T * k : 0;
    // (x rows in LDS: MXFP4 16-row passes whose rows fit; see
    // decode_fused_x_in_lds.  Measured on decode64: MXFP4 72.4 -> 70.3 us,
    // while the E4M3FN stream went from 115.9 to 117.8 us, so it keeps its
    // operand loads from L2)
    const bool xlds = MX4 && MT == 1 && decode_fused_x_in_lds(MT, H, I, routes);
    // (32-row SwiGLU passes: x and the activations share LDS when a row is
    // whole 1 KB wave loads, a wave holds at most two phase-1 groups and it
    // fits.  Each chunk's x operand is then read from LDS instead of L2:
    // measured on decode512, MXFP4 124.6 -> 100.8 us, E4M3FN 154.6 -> 151.8 us.
    // relu^2 keeps four tiles a group in registers and spills too much.)
    const bool xa = !xlds && !RELU2 && MT == 2 && H % 512 == 0 &&
                    decode_fused_groups1(H, I, RELU2, MX4) <= 2 &&
                    decode_fused_lds_bytes(MT, I, routes, H, true) <= DF_LDS_DYNAMIC_MAX;
    const size_t lds = decode_fused_lds_bytes(MT, I, routes, (xlds || xa) ? H : 0, xa);
    // the trash row sits right after the last real row of y
    const int ytrash = T * k + (sh.w13 ? T : 0);
    prof_begin(MX4 ? "decode_fused_expert_mxfp4" : "decode_fused_expert", stream);
#define MOE_DF_KERNEL(MTV, XL, XAV)                                                                       \
    decode_fused_kernel<MTV, 2, LAYOUT, SELF, RELU2, MX4, XL, XAV><<<(unsigned)nwg, DF_THREADS, lds, stream>>>( \
        x, w13, w13s, w2, w2s, sh.w13, sh.w13_scale, sh.w2, sh.w2_scale, plan, ids, E, aff, T, H, I,      \
        k, ybuf, ytrash, (int)cap)
    if (MX4 && MT == 1 && xlds)
        MOE_DF_KERNEL(1, MX4, false);
    else if (MT == 1)
        MOE_DF_KERNEL(1, false, false);
    else if (xa)
        MOE_DF_KERNEL(2, true, true);
    else
        MOE_DF_KERNEL(2, false, false);
#undef MOE_DF_KERNEL
    prof_end(stream);
    return check_launch("decode_fused_kernel");
}

template <bool SELF>
static int launch_decode_fused_any(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                                   const void* w13s, const uint8_t* w2, const void* w2s,
                                   const SharedW& sh, const Plan& plan, const int32_t* ids,
                                   const float* aff, int T, int H, int I, int E, int k,
                                   float* ybuf, int act, int wfmt, hipStream_t stream) {
#define MOE_DF_LAUNCH(L, R, M)                                                                      \
    launch_decode_fused_l<L, SELF, R, M>(MT, x, w13, w13s, w2, w2s, sh, plan, ids, aff, T, H, I, E, \
                                         k, ybuf, stream)
#define MOE_DF_LAYOUT(L, M) \
    (act == ACT_RELU2 ? MOE_DF_LAUNCH(L, true, M) : MOE_DF_LAUNCH(L, false, M))
    if (wfmt == WFMT_MXFP4)
        return layout == LAYOUT_TILED ? MOE_DF_LAYOUT(LAYOUT_TILED, true)
                                      : MOE_DF_LAYOUT(LAYOUT_ROWMAJOR, true);
    return layout == LAYOUT_TILED ? MOE_DF_LAYOUT(LAYOUT_TILED, false)
                                  : MOE_DF_LAYOUT(LAYOUT_ROWMAJOR, false);
#undef MOE_DF_LAYOUT
#undef MOE_DF_LAUNCH
}

size_t decode_fused_tile_capacity(int T, int k, int E, int has_shared, int tile_m) {
    const size_t R = (size_t)T * k, tm = (size_t)tile_m;
    return (R + tm - 1) / tm + (size_t)E + 1 + (has_shared ? ((size_t)T + tm - 1) / tm : 0);
}

// The sorted form: one workgroup per row tile of the sort's list.
int launch_decode_fused(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                        const void* w13s, const uint8_t* w2, const void* w2s, const SharedW& sh,
                        const Plan& plan, const float* aff, int T, int H, int I, int E, int k,
                        float* ybuf, int act, int wfmt, hipStream_t stream) {
    return launch_decode_fused_any<false>(layout, MT, x, w13, w13s, w2, w2s, sh, plan, nullptr,
                                          aff, T, H, I, E, k, ybuf, act, wfmt, stream);
}

// The self-routed form: no sort beforehand; workgroup e scans the ids.
int launch_decode_fused_self(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                             const void* w13s, const uint8_t* w2, const void* w2s,
                             const SharedW& sh, const int32_t* ids, const float* aff, int T,
                             int H, int I, int E, int k, float* ybuf, int act, int wfmt,
                             hipStream_t stream) {
    const Plan none{};
    return launch_decode_fused_any<true>(layout, MT, x, w13, w13s, w2, w2s, sh, none, ids, aff, T,
                                         H, I, E, k, ybuf, act, wfmt, stream);
}

int decode_self_routed_max_routes() { return DF_SELF_MAX_ROUTES; }

}  // namespace moe
