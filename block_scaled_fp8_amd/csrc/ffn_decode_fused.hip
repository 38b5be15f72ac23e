// Decode variant, one workgroup per active expert: gate/up GEMM -> SwiGLU ->
// down GEMM in a single launch, the SwiGLU activations kept in LDS.
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
// Block scales: the accumulator of a tile is kept in units of the scale of
// the 128-wide K block being summed; entering a new block multiplies it by
// s_old / s_new, and the final value is multiplied by the last scale.  The
// scale is therefore applied in fp32 and never rounded into bf16, with one
// accumulator set instead of a partial plus a total.  A block whose scale is
// zero holds only zero weights and leaves the running scale unchanged.
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
// y; rows past the segment write to the trash row too.  With no conditional
// loads or stores (global stores also count on the vector-memory counter of
// gfx9-class GPUs), the compiler's wait counts stay partial and the pipeline
// never drains mid-stream.
constexpr int DF_HALF = DF_NT / 2;

// Self-routed mode (decode batches of at most DF_SELF_MAX_ROUTES routes): the
// workgroup of expert e finds its own routes by scanning the ids (wave ballots,
// ascending route order, the same order as the stable sort), so the step needs
// no separate sort launch.  Workgroup E is the shared expert.
constexpr int DF_SELF_MAX_ROUTES = 4096;
constexpr int DF_SELF_IDS_PER_THREAD = DF_SELF_MAX_ROUTES / DF_THREADS;

size_t decode_fused_lds_bytes(int MT, int I, int self_routes) {
    return sizeof(uint16_t) * (size_t)(16 * MT) * (I + 8) + sizeof(int32_t) * (size_t)self_routes;
}

// RELU2: a non-gated expert, w13 = the up projection [I, H] alone; a phase-1
// group is NT up tiles (64 rows, inside one 128-row scale block) and the
// activation is relu(u)^2.
template <int MT, int DEPTH, int LAYOUT, bool SELF, bool RELU2>
__global__ __launch_bounds__(DF_THREADS) void decode_fused_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13,
    const float* __restrict__ w13s, const uint8_t* __restrict__ w2,
    const float* __restrict__ w2s, const uint8_t* __restrict__ sh_w13,
    const float* __restrict__ sh_w13s, const uint8_t* __restrict__ sh_w2,
    const float* __restrict__ sh_w2s, Plan plan, const int32_t* __restrict__ ids, int E,
    const float* __restrict__ aff, int T, int H, int I, int k, float* __restrict__ ybuf,
    float* __restrict__ ytrash) {
    static_assert(DEPTH == 1 || DEPTH == 2, "chunks per 128-wide scale block");
    constexpr int MROWS = 16 * MT, NT = DF_NT, HALF = DF_HALF;
    constexpr int CS = chunk_stride<LAYOUT>();
    extern __shared__ uint16_t a_lds[];  // [MROWS][I + 8] bf16 SwiGLU activations
    const int astride = I + 8;  // +16 bytes per row: conflict-free 16-byte column reads
    const int lane = lane_id(), wave = wave_id();
    const int R = T * k;
    int e, row0, rows;
    int32_t* rlist = reinterpret_cast<int32_t*>(a_lds + (size_t)MROWS * astride);  // SELF: routes of e
    if (SELF) {
        const int b = blockIdx.x;
        if (b > E || (b == E && sh_w13 == nullptr)) return;
        e = b < E ? b : -1;
        row0 = 0;
        rows = T;
        if (e >= 0) {
            __shared__ int wcnt[DF_WAVES];
            int idv[DF_SELF_IDS_PER_THREAD];
#pragma unroll
            for (int c = 0; c < DF_SELF_IDS_PER_THREAD; ++c) {
                const int r = c * DF_THREADS + (int)threadIdx.x;
                idv[c] = r < R ? ids[r] : -1;
            }
            int base = 0;
#pragma unroll
            for (int c = 0; c < DF_SELF_IDS_PER_THREAD; ++c) {
                if (c * DF_THREADS >= R) break;  // uniform
                const bool hit = idv[c] == e;
                const uint64_t m = __ballot(hit);
                if (lane == 0) wcnt[wave] = (int)__popcll(m);
                __syncthreads();
                int woff = 0, tot = 0;
#pragma unroll
                for (int w = 0; w < DF_WAVES; ++w) {
                    const int cw = wcnt[w];
                    woff += w < wave ? cw : 0;
                    tot += cw;
                }
                if (hit) rlist[base + woff + (int)__popcll(m & lanemask_lt())] = c * DF_THREADS + (int)threadIdx.x;
                base += tot;
                __syncthreads();  // wcnt is rewritten next round; rlist complete after the last
            }
            rows = base;
            if (rows == 0) return;  // the same value in every thread
        }
    } else {
        // the segment fields are loaded together (arrays hold E+1 >= gridDim.x
        // entries), so one memory latency passes before the weights are known
        const int seg = blockIdx.x;
        const int nseg = plan.seg_n[0];
        e = plan.seg_expert[seg];
        row0 = plan.seg_row0[seg];
        rows = plan.seg_rows[seg];
        if (seg >= nseg) return;
    }
    // route index of the m-th row of this workgroup (shared expert: R + token)
    auto route_of = [&](int m) -> int {
        if (e < 0) return (SELF ? R : row0) + m;
        return SELF ? rlist[m] : plan.sorted_route[row0 + m];
    };
    const int n13 = RELU2 ? I : 2 * I;  // rows of the expert's first matrix
    const uint8_t* W13 = e >= 0 ? w13 + (size_t)e * n13 * H : sh_w13;
    const float* S13 = e >= 0 ? w13s + (size_t)e * (n13 / 128) * (H / 128) : sh_w13s;
    const uint8_t* W2 = e >= 0 ? w2 + (size_t)e * H * I : sh_w2;
    const float* S2 = e >= 0 ? w2s + (size_t)e * (H / 128) * (I / 128) : sh_w2s;

    const int ln = lane & 15, lg = lane >> 4;

    const int nch1 = H >> 6, nch2 = I >> 6;  // chunks per group, both even
    const int kb1 = H >> 7, kb2 = I >> 7;    // scale blocks along K
    const int G1 = I / (16 * (RELU2 ? NT : HALF)), G2 = H / (16 * NT);
    const int n1 = (G1 + DF_WAVES - 1) / DF_WAVES, n2 = (G2 + DF_WAVES - 1) / DF_WAVES;
    const int tot1 = n1 * nch1, tot2 = n2 * nch2;

    for (int mp = 0; mp < rows; mp += MROWS) {
        if (mp > 0) __syncthreads();  // the previous pass has finished reading a_lds
        const uint16_t* xp[MT];
        bool xvalid[MT];
        const uint16_t* ap[MT];
        float* yrow[MT][4];  // y destination of this lane's output rows (trash row if padded)
        float yaff[MT][4];   // affinity of each of those routes
        u32x4 bq[DEPTH][NT];
        u32x4 aq[DEPTH][MT][2];
        f32x4 acc[MT][NT];
        float seff0 = 0.0f, seff1 = 0.0f;  // running scales (phase 1: gate, up; phase 2: seff0)
        auto reset = [&]() {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            seff0 = 0.0f;
            seff1 = 0.0f;
        };
        auto rescale = [&](float& seff, float sn, int j0, int j1) {
            if (sn != 0.0f) {
                if (seff != 0.0f) {
                    const float r = seff * __builtin_amdgcn_rcpf(sn);
#pragma unroll
                    for (int j = j0; j < j1; ++j)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc[mt][j] *= r;
                }
                seff = sn;
            }
        };
        auto mfma_chunk = [&](int d, const u32x4 (&av)[MT][2]) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const bf16x8 b = s == 0 ? fp8x8_to_bf16x8(bq[d][j][0], bq[d][j][1])
                                            : fp8x8_to_bf16x8(bq[d][j][2], bq[d][j][3]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[mt][s]),
                                                                             b, acc[mt][j], 0, 0, 0);
                }
        };

        // ---- issue side: phase-1 group g has gate tiles g*HALF+j and up tiles
        //      I/16 + g*HALF + j; phase-2 group g has W2 row tiles g*NT + j.
        //      Groups past the real count re-stream group g % G.
        int ig = wave, ic = 0;  // issue cursor (group, chunk)
        auto issue1_b = [&](int d, int g, int c) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int r = RELU2 ? (g * NT + j) * 16 : (j < HALF ? 0 : I) + (g * HALF + (j % HALF)) * 16;
                bq[d][j] = load_stream16(tile_lane_ptr<LAYOUT>(W13, r, H, lane) + (size_t)c * CS);
            }
        };
        auto issue1_a = [&](int d, int c) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4* q = reinterpret_cast<const u32x4*>(xp[mt] + c * 64);
                aq[d][mt][0] = q[0];
                aq[d][mt][1] = q[1];
            }
        };
        auto issue1 = [&](int d) {
            issue1_b(d, ig % G1, ic);
            issue1_a(d, ic);
            if (++ic == nch1) { ic = 0; ig += DF_WAVES; }
        };
        auto issue2 = [&](int d) {
            const int g = ig % G2;
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bq[d][j] = load_stream16(tile_lane_ptr<LAYOUT>(W2, (g * NT + j) * 16, I, lane) +
                                         (size_t)ic * CS);
            if (++ic == nch2) { ic = 0; ig += DF_WAVES; }
        };

        // ---- process side
        int pg = wave, pc = 0;
        auto proc1 = [&](int d) {
            const int g = pg % G1;
            if ((pc & 1) == 0) {
                const int kb = pc >> 1;
                if (RELU2) {
                    const int ui = __builtin_amdgcn_readfirstlane(((g * NT * 16) >> 7) * kb1 + kb);
                    rescale(seff0, S13[ui], 0, NT);
                } else {
                    const int gi = __builtin_amdgcn_readfirstlane(((g * HALF * 16) >> 7) * kb1 + kb);
                    const int ui = __builtin_amdgcn_readfirstlane(((I + g * HALF * 16) >> 7) * kb1 + kb);
                    rescale(seff0, S13[gi], 0, HALF);
                    rescale(seff1, S13[ui], HALF, NT);
                }
            }
            u32x4 av[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                av[mt][0] = xvalid[mt] ? aq[d][mt][0] : u32x4{0u, 0u, 0u, 0u};
                av[mt][1] = xvalid[mt] ? aq[d][mt][1] : u32x4{0u, 0u, 0u, 0u};
            }
            mfma_chunk(d, av);
            if (pc == nch1 - 1) {  // group done: activations into LDS (padding columns if spare)
                const bool real = pg < G1;
                if (RELU2) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int j = 0; j < NT; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int m = mt * 16 + lg * 4 + i;
                                const int col = real ? (g * NT + j) * 16 + ln : I + (ln & 7);
                                a_lds[m * astride + col] = f32_to_bf16_bits(relu2(acc[mt][j][i] * seff0));
                            }
                } else {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int j = 0; j < HALF; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float gv = acc[mt][j][i] * seff0;
                                const float uv = acc[mt][HALF + j][i] * seff1;
                                const int m = mt * 16 + lg * 4 + i;
                                const int col = real ? (g * HALF + j) * 16 + ln : I + (ln & 7);
                                a_lds[m * astride + col] = f32_to_bf16_bits(swiglu(gv, uv));
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
            if ((pc & 1) == 0) {
                const int si = __builtin_amdgcn_readfirstlane(((g * NT * 16) >> 7) * kb2 + (pc >> 1));
                rescale(seff0, S2[si], 0, NT);
            }
            u32x4 av[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4* q = reinterpret_cast<const u32x4*>(ap[mt] + pc * 64);
                av[mt][0] = q[0];
                av[mt][1] = q[1];
            }
            mfma_chunk(d, av);
            if (pc == nch2 - 1) {  // group done: fp32 rows of the routes (trash if spare)
                const bool real = pg < G2;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float* dst = real ? yrow[mt][i] + g * NT * 16 + ln : ytrash + ln;
                        const float sc = seff0 * yaff[mt][i];
#pragma unroll
                        for (int j = 0; j < NT; ++j) dst[j * 16] = acc[mt][j][i] * sc;
                    }
                reset();
                pc = 0;
                pg += DF_WAVES;
            } else {
                ++pc;
            }
        };

        reset();
        // weight prologue first (it needs only the expert), then the token ids
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) issue1_b(d, ig % G1, d);
        ic = DEPTH;
        if (ic == nch1) { ic = 0; ig += DF_WAVES; }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mp + mt * 16 + ln;
            int t = -1;
            if (m < rows) t = e >= 0 ? route_of(m) / k : route_of(m) - R;
            xvalid[mt] = t >= 0;
            xp[mt] = x + (size_t)(t >= 0 ? t : 0) * H + lg * 16;
            ap[mt] = a_lds + (mt * 16 + ln) * astride + lg * 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mi = mp + mt * 16 + lg * 4 + i;
                int r = -1;
                float a = 0.0f;
                if (mi < rows) {
                    r = route_of(mi);
                    a = e >= 0 ? aff[r] : 1.0f;
                }
                yrow[mt][i] = r >= 0 ? ybuf + (size_t)r * H : ytrash;
                yaff[mt][i] = a;
            }
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) issue1_a(d, d);
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

template <int LAYOUT, bool SELF, bool RELU2>
static int launch_decode_fused_l(int MT, const uint16_t* x, const uint8_t* w13, const float* w13s,
                                 const uint8_t* w2, const float* w2s, const SharedW& sh,
                                 const Plan& plan, const int32_t* ids, const float* aff, int T,
                                 int H, int I, int E, int k, float* ybuf, hipStream_t stream) {
    const int nseg_max = E + (sh.w13 ? 1 : 0);
    const size_t lds = decode_fused_lds_bytes(MT, I, SELF ? T * k : 0);
    // the trash row sits right after the last real row of y
    float* ytrash = ybuf + ((size_t)T * k + (sh.w13 ? (size_t)T : 0)) * H;
    prof_begin("decode_fused_expert", stream);
    if (MT == 1)
        decode_fused_kernel<1, 2, LAYOUT, SELF, RELU2><<<nseg_max, DF_THREADS, lds, stream>>>(
            x, w13, w13s, w2, w2s, sh.w13, sh.w13_scale, sh.w2, sh.w2_scale, plan, ids, E, aff, T,
            H, I, k, ybuf, ytrash);
    else
        decode_fused_kernel<2, 2, LAYOUT, SELF, RELU2><<<nseg_max, DF_THREADS, lds, stream>>>(
            x, w13, w13s, w2, w2s, sh.w13, sh.w13_scale, sh.w2, sh.w2_scale, plan, ids, E, aff, T,
            H, I, k, ybuf, ytrash);
    prof_end(stream);
    return check_launch("decode_fused_kernel");
}

template <bool SELF>
static int launch_decode_fused_any(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                                   const float* w13s, const uint8_t* w2, const float* w2s,
                                   const SharedW& sh, const Plan& plan, const int32_t* ids,
                                   const float* aff, int T, int H, int I, int E, int k,
                                   float* ybuf, int act, hipStream_t stream) {
#define MOE_DF_LAUNCH(L, R)                                                                      \
    launch_decode_fused_l<L, SELF, R>(MT, x, w13, w13s, w2, w2s, sh, plan, ids, aff, T, H, I, E, \
                                      k, ybuf, stream)
    const bool relu2 = act == ACT_RELU2;
    if (layout == LAYOUT_TILED)
        return relu2 ? MOE_DF_LAUNCH(LAYOUT_TILED, true) : MOE_DF_LAUNCH(LAYOUT_TILED, false);
    return relu2 ? MOE_DF_LAUNCH(LAYOUT_ROWMAJOR, true) : MOE_DF_LAUNCH(LAYOUT_ROWMAJOR, false);
#undef MOE_DF_LAUNCH
}

// One workgroup per possible segment (E routed + shared); workgroups past the
// number of active segments exit at once.
int launch_decode_fused(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                        const float* w13s, const uint8_t* w2, const float* w2s, const SharedW& sh,
                        const Plan& plan, const float* aff, int T, int H, int I, int E, int k,
                        float* ybuf, int act, hipStream_t stream) {
    return launch_decode_fused_any<false>(layout, MT, x, w13, w13s, w2, w2s, sh, plan, nullptr,
                                          aff, T, H, I, E, k, ybuf, act, stream);
}

// The self-routed form: no sort beforehand; workgroup e scans the ids.
int launch_decode_fused_self(int layout, int MT, const uint16_t* x, const uint8_t* w13,
                             const float* w13s, const uint8_t* w2, const float* w2s,
                             const SharedW& sh, const int32_t* ids, const float* aff, int T,
                             int H, int I, int E, int k, float* ybuf, int act,
                             hipStream_t stream) {
    const Plan none{};
    return launch_decode_fused_any<true>(layout, MT, x, w13, w13s, w2, w2s, sh, none, ids, aff, T,
                                         H, I, E, k, ybuf, act, stream);
}

int decode_self_routed_max_routes() { return DF_SELF_MAX_ROUTES; }

}  // namespace moe
