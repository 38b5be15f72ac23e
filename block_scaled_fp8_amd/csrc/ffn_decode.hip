// Decode variant of the expert FFN: weight-bandwidth-bound streaming kernels.
//
// Source: "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for
// Trainium2", section "FP8 MoE decode kernel (moe_fused_w8_35b)": gate/up GEMM
// -> SwiGLU -> down GEMM -> affinity scale -> expert-sum, E4M3FN weights with
// 128x128 block scales decoded to BF16 tile by tile; at decode the expert
// weights dominate the bytes moved.
//
// Design (gfx950): one workgroup per (segment, N tile) with segments = active
// experts (plus the shared expert), so each active expert's weights are read
// from HBM once.  The 4 waves of a workgroup split the contraction dimension;
// each wave streams 16-byte FP8 fragments directly in the register layout of
// v_mfma_f32_16x16x32_bf16 (lane l: weight row l%16, 16 consecutive K bytes
// at 16*(l/16) inside each 64-wide K chunk), converts them exactly to bf16
// and multiplies against the token rows (M = 16 per MFMA tile).  The same K
// permutation is used for the token operand, so the dot products are exact
// sums over K.  Each 128-wide K block accumulates into a fresh fp32 partial
// that is multiplied by the block's fp32 scale before joining the total, so
// the scale is never rounded into bf16.
#include <algorithm>

#include "common.hpp"
#include "plan.hpp"

namespace moe {

enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_UP = 2 };

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = 4;
constexpr int DEC_NTILE = 4;   // 16-row weight tiles per workgroup
constexpr int DEC_DEPTH = 4;   // 64-K chunks in flight per wave

// MODE_GATEUP: rows = 32 gate rows + the 32 matching up rows, K = H,
//              A = x rows of the segment's tokens, out = bf16 SwiGLU into abuf.
// MODE_UP:     rows = 64 rows of the up projection of a non-gated expert,
//              K = H, A = x rows, out = bf16 relu(u)^2 into abuf.
// MODE_DOWN:   rows = 64 rows of W2, K = I, A = abuf rows, out = fp32 ybuf.
template <int MODE, int MT, int LAYOUT>
__global__ __launch_bounds__(DEC_THREADS) void decode_ffn_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13,
    const float* __restrict__ w13s, const uint8_t* __restrict__ w2,
    const float* __restrict__ w2s, const uint8_t* __restrict__ sh_w13,
    const float* __restrict__ sh_w13s, const uint8_t* __restrict__ sh_w2,
    const float* __restrict__ sh_w2s, Plan plan, const float* __restrict__ aff, int T, int H,
    int I, int k, uint16_t* __restrict__ abuf, float* __restrict__ ybuf) {
    constexpr int MROWS = 16 * MT;
    constexpr bool GATHER = MODE != MODE_DOWN;  // A rows are token rows of x
    const int K = GATHER ? H : I;
    const int ntile_per_seg = MODE == MODE_GATEUP ? I / 32 : (MODE == MODE_UP ? I / 64 : H / 64);
    const int seg = blockIdx.x / ntile_per_seg;
    const int nt = blockIdx.x % ntile_per_seg;
    if (seg >= plan.seg_n[0]) return;
    const int e = plan.seg_expert[seg];
    const int row0 = plan.seg_row0[seg];
    const int rows = plan.seg_rows[seg];

    const uint8_t* W;
    const float* S;
    if (GATHER) {
        const int n13 = MODE == MODE_GATEUP ? 2 * I : I;  // rows of the expert's first matrix
        W = e >= 0 ? w13 + (size_t)e * n13 * H : sh_w13;
        S = e >= 0 ? w13s + (size_t)e * (n13 / 128) * (H / 128) : sh_w13s;
    } else {
        W = e >= 0 ? w2 + (size_t)e * H * I : sh_w2;
        S = e >= 0 ? w2s + (size_t)e * (H / 128) * (I / 128) : sh_w2s;
    }
    const int kblocks = K / 128;

    const int lane = lane_id(), wave = wave_id();
    const int ln = lane & 15, lg = lane >> 4;

    // weight rows of the 4 tiles
    int brow[DEC_NTILE];
#pragma unroll
    for (int j = 0; j < DEC_NTILE; ++j) {
        if (MODE == MODE_GATEUP)
            brow[j] = (j < 2 ? 0 : I) + nt * 32 + (j & 1) * 16;
        else
            brow[j] = nt * 64 + j * 16;
    }
    const uint8_t* bptr[DEC_NTILE];
#pragma unroll
    for (int j = 0; j < DEC_NTILE; ++j) bptr[j] = tile_lane_ptr<LAYOUT>(W, brow[j], K, lane);

    // this wave's 64-K chunks
    const int nchunk = K / 64;
    const int per = (nchunk + DEC_WAVES - 1) / DEC_WAVES;
    const int cb = min(nchunk, wave * per), ce = min(nchunk, cb + per);

    __shared__ float red[DEC_WAVES][MT][DEC_NTILE][4][MOE_WAVE];
    __shared__ int tok_s[MROWS];

    const size_t R = (size_t)T * k;
    for (int mp = 0; mp < rows; mp += MROWS) {
        // token (or abuf row) of each of the MROWS rows of this pass
        __syncthreads();
        if (threadIdx.x < MROWS) {
            const int m = mp + threadIdx.x;
            int src = -1;
            if (m < rows) {
                const int p = row0 + m;
                if (GATHER)
                    src = e >= 0 ? plan.sorted_route[p] / k : p - (int)R;
                else
                    src = p;
            }
            tok_s[threadIdx.x] = src;
        }
        __syncthreads();
        const uint16_t* aptr[MT];
        bool avalid[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int src = tok_s[mt * 16 + ln];
            avalid[mt] = src >= 0;
            const int s = src >= 0 ? src : 0;
            aptr[mt] = (GATHER ? x + (size_t)s * H : abuf + (size_t)s * I) + lg * 16;
        }

        f32x4 acc[MT][DEC_NTILE], part[MT][DEC_NTILE];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < DEC_NTILE; ++j) {
                acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                part[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }

        u32x4 bq[DEC_DEPTH][DEC_NTILE];
        u32x4 aq[DEC_DEPTH][MT][2];
        auto issue = [&](int d, int c) {
#pragma unroll
            for (int j = 0; j < DEC_NTILE; ++j)
                bq[d][j] = load_stream16(bptr[j] + (size_t)c * chunk_stride<LAYOUT>());
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4* ap = reinterpret_cast<const u32x4*>(aptr[mt] + (size_t)c * 64);
                aq[d][mt][0] = ap[0];
                aq[d][mt][1] = ap[1];
            }
        };
#pragma unroll
        for (int d = 0; d < DEC_DEPTH; ++d)
            if (cb + d < ce) issue(d, cb + d);

        for (int c0 = cb; c0 < ce; c0 += DEC_DEPTH) {
#pragma unroll
            for (int d = 0; d < DEC_DEPTH; ++d) {
                const int c = c0 + d;
                if (c < ce) {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        bf16x8 bfrag[DEC_NTILE];
#pragma unroll
                        for (int j = 0; j < DEC_NTILE; ++j)
                            bfrag[j] = s == 0 ? fp8x8_to_bf16x8(bq[d][j][0], bq[d][j][1])
                                              : fp8x8_to_bf16x8(bq[d][j][2], bq[d][j][3]);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            u32x4 av = aq[d][mt][s];
                            if (!avalid[mt]) av = u32x4{0u, 0u, 0u, 0u};
                            const bf16x8 afrag = as_bf16x8(av);
#pragma unroll
                            for (int j = 0; j < DEC_NTILE; ++j)
                                part[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    afrag, bfrag[j], part[mt][j], 0, 0, 0);
                        }
                    }
                    if (c + DEC_DEPTH < ce) issue(d, c + DEC_DEPTH);
                    if ((c & 1) == 1 || c == ce - 1) {
                        const int kb = c >> 1;
#pragma unroll
                        for (int j = 0; j < DEC_NTILE; ++j) {
                            // uniform index -> scalar load (no wait on in-flight weight loads)
                        const int sidx = __builtin_amdgcn_readfirstlane((brow[j] >> 7) * kblocks + kb);
                        const float sc = S[sidx];
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                acc[mt][j] += sc * part[mt][j];
                                part[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                            }
                        }
                    }
                }
            }
        }

        // cross-wave reduction of the K split
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < DEC_NTILE; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wave][mt][j][i][lane] = acc[mt][j][i];
        __syncthreads();

        if (MODE == MODE_GATEUP) {
            // items: (mt, pair p) with gate tile p and up tile 2 + p
            for (int item = wave; item < MT * 2; item += DEC_WAVES) {
                const int mt = item >> 1, p = item & 1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float g = 0.f, u = 0.f;
#pragma unroll
                    for (int v = 0; v < DEC_WAVES; ++v) {
                        g += red[v][mt][p][i][lane];
                        u += red[v][mt][2 + p][i][lane];
                    }
                    const int m = mp + mt * 16 + lg * 4 + i;
                    if (m < rows) {
                        const int col = nt * 32 + p * 16 + ln;
                        abuf[(size_t)(row0 + m) * I + col] = f32_to_bf16_bits(swiglu(g, u));
                    }
                }
            }
        } else if (MODE == MODE_UP) {
            for (int item = wave; item < MT * DEC_NTILE; item += DEC_WAVES) {
                const int mt = item / DEC_NTILE, j = item % DEC_NTILE;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float u = 0.f;
#pragma unroll
                    for (int v = 0; v < DEC_WAVES; ++v) u += red[v][mt][j][i][lane];
                    const int m = mp + mt * 16 + lg * 4 + i;
                    if (m < rows) abuf[(size_t)(row0 + m) * I + brow[j] + ln] = f32_to_bf16_bits(relu2(u));
                }
            }
        } else {
            for (int item = wave; item < MT * DEC_NTILE; item += DEC_WAVES) {
                const int mt = item / DEC_NTILE, j = item % DEC_NTILE;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float y = 0.f;
#pragma unroll
                    for (int v = 0; v < DEC_WAVES; ++v) y += red[v][mt][j][i][lane];
                    const int m = mp + mt * 16 + lg * 4 + i;
                    if (m < rows) {
                        const int p = row0 + m;
                        const int r = e >= 0 ? plan.sorted_route[p] : p;
                        const float a = e >= 0 ? aff[r] : 1.0f;
                        ybuf[(size_t)r * H + brow[j] + ln] = y * a;
                    }
                }
            }
        }
    }
}

// out[t] = sum_j y[t*k + j] over the valid routes (inv_route >= 0), in slot
// order, + y[R + t] for the shared expert; fp32.  The producers have already
// multiplied each row by its affinity.  Source: AITER PR page (FP32 route
// reduction); NKI page (affinity scale -> expert-sum, shared expert added after
// the routed sum).
// Sum of the k route rows of a token (slot order) plus its shared-expert row,
// decode form: route r's row aff[r] * y is fp32 row r of ybuf.  All loads are
// issued before any is used: the ids only select (a row of an invalid route
// was never written and may hold anything, so it is masked, not multiplied),
// which keeps one memory round trip per thread.  ybuf is read once, so its
// loads bypass the caches' retention (non-temporal).
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ybuf,
                                                      const int32_t* __restrict__ ids,
                                                      int T, int H, int k, int E, int has_shared,
                                                      int32_t* __restrict__ status,
                                                      float* __restrict__ out) {
    const int t = blockIdx.y;
    const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (h >= H) return;
    f32x4 v[KMAX];
    int id[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
            const size_t r = (size_t)t * k + j;
            id[j] = ids[r];
            v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ybuf + r * H + h));
        }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (has_shared) {
        const size_t R = (size_t)T * k;
        acc = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ybuf + (R + t) * H + h));
    }
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    bool bad = false;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
            const bool ok = id[j] >= 0 && id[j] < E;  // an invalid id's route is dropped
            bad |= !ok;
#pragma unroll
            for (int c = 0; c < 4; ++c) sum[c] += ok ? v[j][c] : 0.0f;
        }
    }
    if (bad && status && h == 0) atomicOr(status, MOE_STATUS_BAD_EXPERT_ID);
    // routed sum in slot order first, then the shared expert
    *reinterpret_cast<f32x4*>(out + (size_t)t * H + h) = sum + acc;
}

// Prefill form: the producers write y of route r (no affinity) at its sorted
// row inv_route[r] in the block floating-point form of bfp16x8_encode (16-bit
// mantissas at byte 2*col, one exponent byte per 8 columns at byte
// 2*H + col/8; row stride 2*H + H/8; the shared row of token t is row R + t).
// A thread owns one run of 8 columns (a 16-byte and a 1-byte load per row),
// widens it to fp32 and adds aff[r] * y over the slots in order, eight slots'
// loads in flight at a time, then the shared row.
constexpr int COMBINE_G_THREADS = 256;
__global__ __launch_bounds__(COMBINE_G_THREADS) void combine_gather_kernel(
    const uint8_t* __restrict__ ybytes, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ inv_route, const float* __restrict__ aff, int T, int H, int k,
    int E, int has_shared, int32_t* __restrict__ status, float* __restrict__ out) {
    constexpr int G = 8;  // slots per batch of loads
    const int t = blockIdx.y;
    const int h = (blockIdx.x * COMBINE_G_THREADS + threadIdx.x) * 8;
    if (h >= H) return;
    const size_t rowb = (size_t)H * 2 + (size_t)(H / 8);
    auto load_row = [&](size_t row, u32x4& mant, uint32_t& ex) {
        const uint8_t* p = ybytes + row * rowb;
        mant = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 2 * (size_t)h));
        ex = __builtin_nontemporal_load(p + 2 * (size_t)H + h / 8);
    };
    float sum[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) sum[c] = 0.0f;
    bool bad = false;
    for (int j0 = 0; j0 < k; j0 += G) {
        u32x4 vh[G];
        uint32_t vl[G];
        int id[G];
        float a[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (j0 + j < k) {
                const size_t r = (size_t)t * k + j0 + j;
                id[j] = ids[r];
                a[j] = aff[r];
                const int p = inv_route[r];
                load_row(p >= 0 ? (size_t)p : 0, vh[j], vl[j]);  // a dropped route: masked below
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (j0 + j < k) {
                const bool ok = id[j] >= 0 && id[j] < E;  // an invalid id's route is dropped
                bad |= !ok;
#pragma unroll
                for (int c = 0; c < 8; ++c) sum[c] += ok ? a[j] * bfp16_value(vh[j], vl[j], c) : 0.0f;
            }
        }
    }
    if (has_shared) {
        u32x4 sh;
        uint32_t se;
        load_row((size_t)T * k + t, sh, se);
#pragma unroll
        for (int c = 0; c < 8; ++c) sum[c] += bfp16_value(sh, se, c);
    }
    if (bad && status && h == 0) atomicOr(status, MOE_STATUS_BAD_EXPERT_ID);
    f32x4* o = reinterpret_cast<f32x4*>(out + (size_t)t * H + h);
    o[0] = f32x4{sum[0], sum[1], sum[2], sum[3]};
    o[1] = f32x4{sum[4], sum[5], sum[6], sum[7]};
}

template <int MODE, int LAYOUT>
static int launch_decode_mode_l(int MT, int nseg_max, const uint16_t* x, const uint8_t* w13,
                                const float* w13s, const uint8_t* w2, const float* w2s,
                                const SharedW& sh, const Plan& plan, const float* aff, int T,
                                int H, int I, int k, uint16_t* abuf, float* ybuf,
                                hipStream_t stream) {
    const int ntile = MODE == MODE_GATEUP ? I / 32 : (MODE == MODE_UP ? I / 64 : H / 64);
    const dim3 grid((unsigned)nseg_max * ntile), block(DEC_THREADS);
    prof_begin(MODE == MODE_GATEUP ? "decode_gateup_swiglu" : (MODE == MODE_UP ? "decode_up_relu2" : "decode_down"),
               stream);
    if (MT == 1)
        decode_ffn_kernel<MODE, 1, LAYOUT><<<grid, block, 0, stream>>>(
            x, w13, w13s, w2, w2s, sh.w13, static_cast<const float*>(sh.w13_scale), sh.w2,
            static_cast<const float*>(sh.w2_scale), plan, aff, T, H, I, k,
            abuf, ybuf);
    else
        decode_ffn_kernel<MODE, 2, LAYOUT><<<grid, block, 0, stream>>>(
            x, w13, w13s, w2, w2s, sh.w13, static_cast<const float*>(sh.w13_scale), sh.w2,
            static_cast<const float*>(sh.w2_scale), plan, aff, T, H, I, k,
            abuf, ybuf);
    prof_end(stream);
    return check_launch(MODE == MODE_GATEUP ? "decode_ffn_kernel<gateup>"
                                            : (MODE == MODE_UP ? "decode_ffn_kernel<up>" : "decode_ffn_kernel<down>"));
}

template <int MODE>
static int launch_decode_mode(int layout, int MT, int nseg_max, const uint16_t* x,
                              const uint8_t* w13, const float* w13s, const uint8_t* w2,
                              const float* w2s, const SharedW& sh, const Plan& plan,
                              const float* aff, int T, int H, int I, int k, uint16_t* abuf,
                              float* ybuf, hipStream_t stream) {
    if (layout == LAYOUT_TILED)
        return launch_decode_mode_l<MODE, LAYOUT_TILED>(MT, nseg_max, x, w13, w13s, w2, w2s, sh,
                                                        plan, aff, T, H, I, k, abuf, ybuf, stream);
    return launch_decode_mode_l<MODE, LAYOUT_ROWMAJOR>(MT, nseg_max, x, w13, w13s, w2, w2s, sh,
                                                       plan, aff, T, H, I, k, abuf, ybuf, stream);
}

// At most min(E, T*k) routed experts are active.  When that fills most of the
// chip, one workgroup per active expert (ffn_decode_fused.hip) streams every
// weight byte once with no inter-workgroup dependency; with few active
// experts the work is split into (expert, N tile) workgroups over two kernels
// so that all CUs still stream.
int decode_mt(int T, int k, int E) { return ((long)T * k <= 4L * E) ? 1 : 2; }

// The fused one-workgroup-per-expert kernel pays off once most CUs get an
// expert, and needs its activations (and, self-routed, the route list) in LDS;
// it addresses x by 32-bit element offsets.
bool decode_fused_fits(int T, int k, int E, int H, int I, int has_shared, bool self_routed) {
    const long R = (long)T * k;
    const long max_active = std::min<long>(E, R) + has_shared;
    if (max_active < 128) return false;
    if ((long long)T * H >= (1LL << 32)) return false;
    if (self_routed && R > decode_self_routed_max_routes()) return false;
    return decode_fused_lds_bytes(decode_mt(T, k, E), I, self_routed ? (int)R : 0) <= 64 * 1024;
}

int launch_decode_ffn(int layout, const uint16_t* x, const uint8_t* w13, const float* w13s,
                      const uint8_t* w2, const float* w2s, const SharedW& sh, const Plan& plan,
                      const float* aff, int T, int H, int I, int E, int k, uint16_t* abuf,
                      float* ybuf, int act, hipStream_t stream) {
    const int has_shared = sh.w13 != nullptr;
    const int nseg_max = E + has_shared;
    const int MT = decode_mt(T, k, E);
    if (decode_fused_fits(T, k, E, H, I, has_shared, false))
        return launch_decode_fused(layout, MT, x, w13, w13s, w2, w2s, sh, plan, aff, T, H, I, E,
                                   k, ybuf, act, WFMT_E4M3_128, stream);
    const int rc = act == ACT_RELU2
                       ? launch_decode_mode<MODE_UP>(layout, MT, nseg_max, x, w13, w13s, w2, w2s,
                                                     sh, plan, aff, T, H, I, k, abuf, ybuf, stream)
                       : launch_decode_mode<MODE_GATEUP>(layout, MT, nseg_max, x, w13, w13s, w2,
                                                         w2s, sh, plan, aff, T, H, I, k, abuf,
                                                         ybuf, stream);
    if (rc) return rc;
    return launch_decode_mode<MODE_DOWN>(layout, MT, nseg_max, x, w13, w13s, w2, w2s, sh, plan,
                                         aff, T, H, I, k, abuf, ybuf, stream);
}

int launch_combine(const float* ybuf, const int32_t* ids, const int32_t* inv_route,
                   const float* aff, int T, int H, int k, int E, int has_shared, int32_t* status,
                   float* out, hipStream_t stream) {
    if (inv_route && !aff) {
        set_error("combine: the gathered form needs the affinities");
        return MOE_EINVAL;
    }
    prof_begin("combine", stream);
    if (inv_route) {
        // (H % 256 == 0 on the prefill path, so a thread's 8 columns are whole)
        const dim3 grid((H / 8 + COMBINE_G_THREADS - 1) / COMBINE_G_THREADS, T);
        combine_gather_kernel<<<grid, COMBINE_G_THREADS, 0, stream>>>(
            reinterpret_cast<const uint8_t*>(ybuf), ids, inv_route, aff, T, H, k, E, has_shared,
            status, out);
    } else {
        const dim3 grid((H / 4 + 255) / 256, T), block(256);
        if (k <= 8)
            combine_kernel<8><<<grid, block, 0, stream>>>(ybuf, ids, T, H, k, E, has_shared, status, out);
        else
            combine_kernel<MOE_MAX_TOPK><<<grid, block, 0, stream>>>(ybuf, ids, T, H, k, E, has_shared,
                                                                    status, out);
    }
    prof_end(stream);
    return check_launch("combine_kernel");
}

// n E4M3FN bytes -> bf16 bit patterns, with the FFN kernels' converter.
__global__ __launch_bounds__(256) void decode_e4m3fn_kernel(const uint8_t* __restrict__ codes,
                                                            uint16_t* __restrict__ out, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
    if (i >= n) return;
    const uint32_t w = (uint32_t)codes[i] | (i + 1 < n ? (uint32_t)codes[i + 1] << 8 : 0u);
    // split the converted pair as one 32-bit word (element 0 in the low half)
    const uint32_t v = __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2(w, false));
    out[i] = (uint16_t)(v & 0xFFFFu);
    if (i + 1 < n) out[i + 1] = (uint16_t)(v >> 16);
}

int launch_decode_e4m3fn(const uint8_t* codes, uint16_t* out, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + 511) / 512;
    prof_begin("decode_e4m3fn", stream);
    decode_e4m3fn_kernel<<<(unsigned)blocks, 256, 0, stream>>>(codes, out, n);
    prof_end(stream);
    return check_launch("decode_e4m3fn_kernel");
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int32_t v,
                                                       int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// A fill kernel rather than hipMemsetAsync, so callers may capture it in a graph.
int launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t stream) {
    if (n <= 0) return MOE_OK;
    prof_begin("fill_i32", stream);
    fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(p, v, n);
    prof_end(stream);
    return check_launch("fill_i32_kernel");
}

}  // namespace moe
