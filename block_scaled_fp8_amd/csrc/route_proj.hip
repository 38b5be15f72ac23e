// Router projection: logits = x * W_g^T from bf16 operands with fp32
// accumulation, then the router (softmax -> top-k -> normalise) on them.
//
// Sources: "spark_model/layers/nemotron_moe.rs", prefill forward: a batched
// gate GEMM takes the normalised hidden states [N, H] and the gate weights
// [E, H] to gate logits [N, E], which the top-K routing then consumes;
// "NKI Library Supported Kernel Reference", Router Top-K: one kernel computes
// the router logits and performs the top-K selection.
//
// gfx950 design.  The projection is a small dense GEMM (M = T tokens,
// N = E experts, K = H) whose weight operand is shared by every token: at
// decode sizes it is bound by memory latency, at prefill sizes by L2 and LDS
// bandwidth.  A workgroup computes a 64-token x 64-expert tile over a slice
// of K with four waves of 32 x 32 (2 x 2 tiles of v_mfma_f32_16x16x32_bf16).
// Operands go global -> registers -> LDS (two buffers whose rows are padded by
// 16 bytes, so that the 16-byte column reads of 16 consecutive rows fall on
// distinct banks), with a ring of up to four 64-wide K stages of loads in
// flight per thread.  When the tiles alone cannot fill the chip, K is split
// into S slices; each slice writes its fp32 partial logits to a slab of its
// own and the router kernel adds the slabs in slice order, a fixed order, so
// the logits do not depend on scheduling.  The tiles are laid out so that
// each XCD computes a contiguous run of them, every expert tile of a token
// tile on one XCD: the activation rows then cross the fabric to an XCD's L2
// once instead of once per expert tile (measured at T = 8192, H = 2048,
// E = 256: 31 -> 21 us).
#include "common.hpp"
#include "plan.hpp"

namespace moe {

constexpr int RP_THREADS = 256;
constexpr int RP_TM = 64;                       // tokens per tile
constexpr int RP_TN = 64;                       // experts per tile
constexpr int RP_KC = 64;                       // K per stage
constexpr int RP_ROW = RP_KC * 2 + 16;          // LDS bytes per operand row (+16-byte pad)
constexpr int RP_STAGE = (RP_TM + RP_TN) * RP_ROW;
constexpr int RP_LOADS = (RP_TM + RP_TN) * RP_KC * 2 / 16 / RP_THREADS;  // 16-byte loads per thread
static_assert(RP_LOADS * RP_THREADS * 16 == (RP_TM + RP_TN) * RP_KC * 2, "stage load mapping");

// Workgroup barrier that waits for this wave's LDS accesses only: the global
// loads of later stages stay in flight across it.  The asm statement keeps
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void rp_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

// part[z][t][e] = sum over k in slice z of x[t][k] * wg[e][k]  (fp32).
// One workgroup per (slice z, token tile, expert tile), in a 1-D grid rounded
// up to a multiple of 8; slice z covers K [z*ks, (z+1)*ks) and ks is a
// multiple of D*64.  Rows past T or E read a clamped valid row (an MFMA
// output row or column depends only on its own operand row) and are not
// stored.
template <int D>
__global__ __launch_bounds__(RP_THREADS) void router_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int T, int H, int E, int ks,
    int ntx, int nty, int nslice, float* __restrict__ part) {
    __shared__ __align__(16) uint8_t lds[2 * RP_STAGE];
    const int lane = lane_id(), wave = wave_id();
    // Workgroups are dealt round-robin over the 8 XCDs; tile q = (slice z,
    // token tile y, expert tile x), x fastest, and XCD c takes tiles
    // [c*per, (c+1)*per), so the expert tiles of a token tile share one L2
    // and its activation rows cross the fabric once.
    const int ntiles = ntx * nty * nslice;
    const int per = (ntiles + 7) / 8;
    const int q = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (q >= ntiles) return;  // the whole workgroup, before any barrier
    const int tx = q % ntx, ty = (q / ntx) % nty, tz = q / (ntx * nty);
    const int t0 = ty * RP_TM, e0 = tx * RP_TN;
    const int kbeg = tz * ks;
    const int nk = ks / RP_KC;

    // stage loads: piece p = tid + 256*i is operand row p/8 (tokens 0..63,
    // then experts 0..63) and its 16-byte piece p%8
    const uint16_t* src[RP_LOADS];
    uint32_t dst[RP_LOADS];
#pragma unroll
    for (int i = 0; i < RP_LOADS; ++i) {
        const int p = (int)threadIdx.x + RP_THREADS * i;
        const int r = p >> 3, c = p & 7;
        if (r < RP_TM) {
            const int t = min(t0 + r, T - 1);
            src[i] = x + (size_t)t * H + kbeg + c * 8;
        } else {
            const int e = min(e0 + r - RP_TM, E - 1);
            src[i] = wg + (size_t)e * H + kbeg + c * 8;
        }
        dst[i] = (uint32_t)(r * RP_ROW + c * 16);
    }
    u32x4 ring[D][RP_LOADS];
    auto fetch = [&](int d, int kc) {
#pragma unroll
        for (int i = 0; i < RP_LOADS; ++i)
            ring[d][i] = *reinterpret_cast<const u32x4*>(src[i] + (size_t)kc * RP_KC);
    };
    auto stash = [&](int d, int buf) {
#pragma unroll
        for (int i = 0; i < RP_LOADS; ++i)
            *reinterpret_cast<u32x4*>(lds + buf * RP_STAGE + dst[i]) = ring[d][i];
    };

    // MFMA operands: lane group lg supplies K 8*lg..8*lg+7 of each 32-wide
    // sub-step for row ln of a 16-row tile (tokens for A, experts for B)
    const int ln = lane & 15, lg = lane >> 4;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
    uint32_t a_off[2], b_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        a_off[j] = (uint32_t)((wm + j * 16 + ln) * RP_ROW + lg * 16);
        b_off[j] = (uint32_t)((RP_TM + wn + j * 16 + ln) * RP_ROW + lg * 16);
    }
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < RP_KC / 32; ++s) {
            u32x4 a[2], b[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                a[j] = *reinterpret_cast<const u32x4*>(lds + buf * RP_STAGE + a_off[j] + s * 64);
                b[j] = *reinterpret_cast<const u32x4*>(lds + buf * RP_STAGE + b_off[j] + s * 64);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i]),
                                                                        as_bf16x8(b[j]), acc[i][j],
                                                                        0, 0, 0);
        }
    };

    // Stage kc: its loads (issued D stages earlier) go to LDS buffer kc&1, the
    // loads of stage kc+D are issued, one barrier, then the MFMAs.  A wave
    // refills a buffer two stages after reading it, and the barrier between
    // proves every wave has finished that read.  Loads past the slice re-read
    // its last stage, so every stage runs the same instruction stream.
#pragma unroll
    for (int d = 0; d < D; ++d) fetch(d, min(d, nk - 1));
    for (int kc0 = 0; kc0 < nk; kc0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int kc = kc0 + d;
            stash(d, kc & 1);
            fetch(d, min(kc + D, nk - 1));
            rp_barrier();
            compute(kc & 1);
        }
    }

    float* out = part + (size_t)tz * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = e0 + wn + j * 16 + ln;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + wm + i * 16 + lg * 4 + r;
                if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][r];
            }
        }
}

// Number of K slices (at most 8, what the router kernel adds): doubled while
// the tile grid has fewer than 512 workgroups and every slice keeps at least
// four stages.
int route_proj_splits(int T, int H, int E) {
    const long long tiles = (long long)((T + RP_TM - 1) / RP_TM) * ((E + RP_TN - 1) / RP_TN);
    const int nk = H / RP_KC;
    int S = 1;
    while (tiles * S < 512 && 2 * S <= 8 && nk % (2 * S) == 0 && nk / (2 * S) >= 4) S *= 2;
    return S;
}

size_t route_proj_workspace_bytes(int T, int H, int E) {
    return sizeof(float) * (size_t)route_proj_splits(T, H, E) * (size_t)T * (size_t)E;
}

int launch_route_proj(const uint16_t* x, const uint16_t* wg, int T, int H, int E, int k,
                      float* logits, int32_t* ids, float* aff, int32_t* status, float* ws,
                      hipStream_t stream) {
    const int S = route_proj_splits(T, H, E);
    const int ks = H / S;
    const int nk = ks / RP_KC;
    // one slice writing straight into the caller's logits needs no slab
    float* part = (S == 1 && logits) ? logits : ws;
    const int ntx = (E + RP_TN - 1) / RP_TN, nty = (T + RP_TM - 1) / RP_TM;
    const long long ntiles = (long long)ntx * nty * S;
    if (ntiles > (1LL << 30)) {
        set_error("moe_route_proj: T=%d gives too many tiles", T);
        return MOE_EUNSUPPORTED;
    }
    const dim3 grid((unsigned)(8 * ((ntiles + 7) / 8))), block(RP_THREADS);
    prof_begin("router_gemm", stream);
    if (nk % 4 == 0)
        router_gemm_kernel<4><<<grid, block, 0, stream>>>(x, wg, T, H, E, ks, ntx, nty, S, part);
    else if (nk % 2 == 0)
        router_gemm_kernel<2><<<grid, block, 0, stream>>>(x, wg, T, H, E, ks, ntx, nty, S, part);
    else
        router_gemm_kernel<1><<<grid, block, 0, stream>>>(x, wg, T, H, E, ks, ntx, nty, S, part);
    prof_end(stream);
    if (int rc = check_launch("router_gemm_kernel")) return rc;
    return launch_route_slabs(part, S, S > 1 ? logits : nullptr, T, E, k, ids, aff, status,
                              stream);
}

}  // namespace moe
