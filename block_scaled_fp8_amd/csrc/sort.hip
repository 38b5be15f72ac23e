// Sort routes by expert: per-expert histogram, exclusive scan, stable sorted
// route map and inverse map (plus the FFN's segment list).
//
// Sources: "spark_model/layers/nemotron_moe.rs" (the sorted prefill path sorts
// routes by expert, runs a grouped GEMM per expert and unpermutes with a
// reduction), and "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter
// PR #5988), description (sorting plus an inverse route map feed the producer
// and the FP32 route reduction).
//
// Determinism: LDS atomics only ever build histograms (their result does not
// depend on arrival order).  Ranks inside an expert never come from atomic
// return values: each wave walks its contiguous range of routes in order, 64
// at a time, and ranks equal ids inside a step by comparing against every
// lane's id, on top of per-(block, wave, expert) bases from exclusive scans.  So route r sits at
//     offsets[e] + #{ r' < r : ids[r'] == e },
// the stable expert-major order.
#include "common.hpp"
#include "plan.hpp"

namespace moe {

constexpr int SORT_SMALL_THREADS = 1024;      // single-workgroup path
constexpr int SORT_SMALL_MAX_ROUTES = 4096;  // measured: one workgroup is as fast up to here, slower above
constexpr int SORT_CHUNK = 1024;              // routes per workgroup, multi-workgroup path (measured at
                                              // R = 65536: 2048 -> 18.3 us, 1024 -> 13.7, 512 -> 15.6)
constexpr int SORT_THREADS = 256;
constexpr int SORT_SCAN_MIN_CHUNKS = 128;  // from this many chunks on, sort_scan runs first

// Exclusive scan of arr[0..n) held in LDS, in place; returns the total.
// Every thread of the block must call it.  tmp holds NT/64 + 1 ints.
template <int NT>
__device__ int lds_excl_scan(int* arr, int n, int* tmp) {
    constexpr int NW = NT / MOE_WAVE;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / MOE_WAVE;
    const int G = (n + NT - 1) / NT;
    const int b = tid * G;
    int local = 0;
    for (int i = 0; i < G; ++i)
        if (b + i < n) local += arr[b + i];
    const int incl = wave_incl_scan_i32(local);
    if (lane == MOE_WAVE - 1) tmp[w] = incl;
    __syncthreads();
    if (tid < MOE_WAVE) {
        const int v = tid < NW ? tmp[tid] : 0;
        const int s = wave_incl_scan_i32(v);
        if (tid < NW) tmp[tid] = s - v;
        if (tid == NW - 1) tmp[NW] = s;
    }
    __syncthreads();
    int run = tmp[w] + incl - local;
    for (int i = 0; i < G; ++i)
        if (b + i < n) {
            const int v = arr[b + i];
            arr[b + i] = run;
            run += v;
        }
    const int total = tmp[NW];
    __syncthreads();
    return total;
}

// Count the ids of [r0, r1) into hist (LDS atomics); returns true if any id
// was out of range.
__device__ bool count_range(const int32_t* __restrict__ ids, int r0, int r1, int stride, int E,
                            int* hist) {
    bool bad = false;
    for (int r = r0; r < r1; r += stride) {
        const int id = ids[r];
        if (id >= 0 && id < E)
            atomicAdd(&hist[id], 1);
        else
            bad = true;
    }
    return bad;
}

// One wave places routes [r_begin, r_end) in order, 64 at a time.  wcnt[e] is
// the position of this wave's next route of expert e (LDS, touched by this
// wave only).  Inside a step, the rank of a lane among the lanes holding the
// same id is counted against every lane's id read as a scalar (readlane), so
// the step costs a fixed, short sequence of ALU instructions.
__device__ void wave_place(const int32_t* __restrict__ ids, int r_begin, int r_end, int E, int* wcnt,
                           int32_t* __restrict__ sorted_route, int32_t* __restrict__ inv_route) {
    const int lane = lane_id();
    for (int r0 = r_begin; r0 < r_end; r0 += MOE_WAVE) {
        const int r = r0 + lane;
        const bool in = r < r_end;
        const int raw = in ? ids[r] : -1;
        const bool valid = in && raw >= 0 && raw < E;
        const int id = valid ? raw : -1;
        int rank = 0, cnt = 0;
#pragma unroll
        for (int l = 0; l < MOE_WAVE; ++l) {
            const int other = __builtin_amdgcn_readlane(id, l);
            const int same = (other == id) ? 1 : 0;
            rank += (l < lane) ? same : 0;
            cnt += same;
        }
        int pos = -1;
        if (valid) pos = wcnt[id] + rank;
        // every lane has read its base before the group's first lane bumps it
        if (valid && rank == 0) wcnt[id] += cnt;
        if (in) {
            if (valid) {
                sorted_route[pos] = r;
                inv_route[r] = pos;
            } else {
                inv_route[r] = -1;
            }
        }
    }
}

// Segment list from counts/offsets held in LDS (one block, all threads).
// flags, tiles, fulls, segx: LDS scratch of E+2 ints each.
template <int NT>
__device__ void build_segments(const int* cnt, const int* off, int E, int R, int T, int has_shared,
                               int tile_m, int* flags, int* tiles, int* fulls, int* segx, int* tmp,
                               const Plan& plan) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += NT) flags[e] = cnt[e] > 0 ? 1 : 0;
    __syncthreads();
    const int nrouted = lds_excl_scan<NT>(flags, E, tmp);
    const int nseg = nrouted + (has_shared ? 1 : 0);
    for (int e = tid; e < E; e += NT)
        if (cnt[e] > 0) {
            const int i = flags[e];
            plan.seg_expert[i] = e;
            plan.seg_row0[i] = off[e];
            plan.seg_rows[i] = cnt[e];
            segx[i] = e;
            tiles[i] = (cnt[e] + tile_m - 1) / tile_m;
            fulls[i] = cnt[e] / tile_m;
        }
    if (has_shared && tid == 0) {
        plan.seg_expert[nrouted] = -1;
        plan.seg_row0[nrouted] = R;
        plan.seg_rows[nrouted] = T;
        segx[nrouted] = -1;
        tiles[nrouted] = (T + tile_m - 1) / tile_m;
        fulls[nrouted] = T / tile_m;
    }
    __syncthreads();
    const int ntiles = lds_excl_scan<NT>(tiles, nseg, tmp);
    const int nfull = lds_excl_scan<NT>(fulls, nseg, tmp);
    for (int i = tid; i < nseg; i += NT) plan.seg_tile0[i] = tiles[i];
    if (tid == 0) {
        plan.seg_tile0[nseg] = ntiles;
        plan.seg_n[0] = nseg;
    }
    if (plan.tile_info) {
        // ordered tile list: full tiles first (segment s's at fulls[s] ..),
        // then the partial ones (segment s's at nfull + #partials before s,
        // which is tiles[s] - fulls[s] with both as exclusive prefixes)
        // (one thread per segment: most segments hold a few tiles, and a wave
        // per segment made this block the sort's longest)
        for (int s = tid; s < nseg; s += NT) {
            const int e = segx[s];
            const int row0 = e >= 0 ? off[e] : R, rows = e >= 0 ? cnt[e] : T;
            const int f0 = fulls[s], f1 = s + 1 < nseg ? fulls[s + 1] : nfull;
            const int t0 = tiles[s], t1 = s + 1 < nseg ? tiles[s + 1] : ntiles;
            for (int j = 0; j < f1 - f0; ++j)
                plan.tile_info[f0 + j] = make_int4(e, row0 + j * tile_m, tile_m, 0);
            if (t1 - t0 > f1 - f0) {
                const int done = (f1 - f0) * tile_m;
                plan.tile_info[nfull + (t0 - f0)] = make_int4(e, row0 + done, rows - done, 0);
            }
        }
        if (tid == 0) plan.tile_n[0] = ntiles;
    }
}

// ------------------------------------------------------------------ small R
// Everything in one workgroup: per-wave histograms, scans, placement.
__global__ __launch_bounds__(SORT_SMALL_THREADS) void sort_small_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, Plan plan, int want_segments,
    int has_shared, int tile_m, int32_t* __restrict__ status) {
    constexpr int NT = SORT_SMALL_THREADS, NW = NT / MOE_WAVE;
    extern __shared__ int lds[];
    int* whist = lds;                    // [NW][E]
    int* cnt = whist + NW * E;           // [E]
    int* off = cnt + E;                  // [E+1]
    int* flags = off + E + 1;            // [E+2]
    int* tiles = flags + E + 2;          // [E+2]
    int* fulls = tiles + E + 2;          // [E+2]
    int* segx = fulls + E + 2;           // [E+2]
    int* tmp = segx + E + 2;             // [NW+1]
    const int R = T * k;
    const int tid = threadIdx.x, w = tid / MOE_WAVE, lane = lane_id();
    const int sub = ((R + NW - 1) / NW + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
    const int r0 = min(R, w * sub), r1 = min(R, r0 + sub);

    for (int i = tid; i < NW * E; i += NT) whist[i] = 0;
    __syncthreads();
    const bool bad = count_range(ids, r0 + lane, r1, MOE_WAVE, E, whist + w * E);
    if (status && __ballot(bad) != 0ull && lane == 0) atomicOr(status, MOE_STATUS_BAD_EXPERT_ID);
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
        int run = 0;
        for (int v = 0; v < NW; ++v) {
            const int c = whist[v * E + e];
            whist[v * E + e] = run;
            run += c;
        }
        cnt[e] = run;
        off[e] = run;
    }
    __syncthreads();
    const int total = lds_excl_scan<NT>(off, E, tmp);
    for (int e = tid; e < E; e += NT) {
        for (int v = 0; v < NW; ++v) whist[v * E + e] += off[e];
        plan.counts[e] = cnt[e];
        plan.offsets[e] = off[e];
    }
    if (tid == 0) {
        plan.offsets[E] = total;
        off[E] = total;
    }
    for (int p = total + tid; p < R; p += NT) plan.sorted_route[p] = -1;
    __syncthreads();
    wave_place(ids, r0, r1, E, whist + w * E, plan.sorted_route, plan.inv_route);
    if (want_segments) {
        __syncthreads();
        build_segments<NT>(cnt, off, E, R, T, has_shared, tile_m, flags, tiles, fulls, segx, tmp, plan);
    }
}

// ------------------------------------------------------------------ large R
__global__ __launch_bounds__(SORT_THREADS) void sort_count_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nb, int32_t* __restrict__ ghist,
    int32_t* __restrict__ status) {
    extern __shared__ int hist[];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += SORT_THREADS) hist[e] = 0;
    __syncthreads();
    const int r0 = blockIdx.x * SORT_CHUNK, r1 = min(R, r0 + SORT_CHUNK);
    const bool bad = count_range(ids, r0 + tid, r1, SORT_THREADS, E, hist);
    if (status && __ballot(bad) != 0ull && lane_id() == 0) atomicOr(status, MOE_STATUS_BAD_EXPERT_ID);
    __syncthreads();
    for (int e = tid; e < E; e += SORT_THREADS) ghist[(size_t)e * nb + blockIdx.x] = hist[e];
}

// One wave per expert e: the row ghist[e][0 .. nb) of per-chunk counts
// becomes its exclusive prefix over the chunks (in place: the routes of
// expert e in earlier chunks), and totals[e] the expert's count.
__global__ __launch_bounds__(SORT_THREADS) void sort_scan_kernel(int32_t* __restrict__ ghist, int E,
                                                                 int nb, int32_t* __restrict__ totals) {
    constexpr int NW = SORT_THREADS / MOE_WAVE;
    const int lane = lane_id();
    const int e = blockIdx.x * NW + wave_id();
    if (e >= E) return;
    int32_t* row = ghist + (size_t)e * nb;
    int carry = 0;
    for (int j0 = 0; j0 < nb; j0 += MOE_WAVE) {
        const int j = j0 + lane;
        const int v = j < nb ? row[j] : 0;
        const int incl = wave_incl_scan_i32(v);
        if (j < nb) row[j] = carry + incl - v;
        carry += __builtin_amdgcn_readlane(incl, MOE_WAVE - 1);
    }
    if (lane == 0) totals[e] = carry;
}

// Blocks 0 .. nb-1 place the routes of their chunk; block nb writes the
// counts, offsets, tail fill and the segment list.  Every block needs the
// expert totals (and derives the offsets, their exclusive scan) and, for
// placement block b, the routes of each expert in earlier chunks: with
// `totals`, from sort_scan's results (one column of the table); without, by
// summing the rows of the count table itself (cheaper than a third launch
// while the table is short).
__global__ __launch_bounds__(SORT_THREADS) void sort_place_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int nb,
    const int32_t* __restrict__ ghist, const int32_t* __restrict__ totals, Plan plan,
    int want_segments, int has_shared, int tile_m) {
    constexpr int NT = SORT_THREADS, NW = NT / MOE_WAVE;
    constexpr int SUB = SORT_CHUNK / NW;
    extern __shared__ int lds[];
    int* whist = lds;               // [NW][E]
    int* cnt = whist + NW * E;      // [E]
    int* off = cnt + E;             // [E+1]
    int* pre = off + E + 1;         // [E]
    int* flags = pre + E;           // [E+2]
    int* tiles = flags + E + 2;     // [E+2]
    int* fulls = tiles + E + 2;     // [E+2]
    int* segx = fulls + E + 2;      // [E+2]
    int* tmp = segx + E + 2;        // [NW+1]
    const int R = T * k, tid = threadIdx.x, w = tid / MOE_WAVE, lane = lane_id();
    const int b = blockIdx.x;
    for (int e = tid; e < E; e += NT) {
        int tot = 0, before = 0;
        if (totals) {
            tot = totals[e];
            before = b < nb ? ghist[(size_t)e * nb + b] : 0;
        } else {
            const int32_t* row = ghist + (size_t)e * nb;
#pragma unroll 8
            for (int j = 0; j < nb; ++j) {
                const int v = row[j];
                before += j < b ? v : 0;
                tot += v;
            }
        }
        cnt[e] = tot;
        off[e] = tot;
        pre[e] = before;
    }
    __syncthreads();
    const int total = lds_excl_scan<NT>(off, E, tmp);
    if (b == nb) {
        for (int e = tid; e < E; e += NT) {
            plan.counts[e] = cnt[e];
            plan.offsets[e] = off[e];
        }
        if (tid == 0) {
            plan.offsets[E] = total;
            off[E] = total;
        }
        for (int p = total + tid; p < R; p += NT) plan.sorted_route[p] = -1;
        if (want_segments) {
            __syncthreads();
            build_segments<NT>(cnt, off, E, R, T, has_shared, tile_m, flags, tiles, fulls, segx, tmp,
                               plan);
        }
        return;
    }
    for (int i = tid; i < NW * E; i += NT) whist[i] = 0;
    __syncthreads();
    const int c0 = b * SORT_CHUNK;
    const int r0 = min(R, c0 + w * SUB), r1 = min(R, r0 + SUB);
    count_range(ids, r0 + lane, r1, MOE_WAVE, E, whist + w * E);
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
        int run = off[e] + pre[e];
        for (int v = 0; v < NW; ++v) {
            const int c = whist[v * E + e];
            whist[v * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    wave_place(ids, r0, r1, E, whist + w * E, plan.sorted_route, plan.inv_route);
}

// The per-(expert, chunk) count table, then the expert totals.
size_t sort_scratch_bytes(int R, int E) {
    if (R <= SORT_SMALL_MAX_ROUTES) return 0;
    const size_t nb = (size_t)(R + SORT_CHUNK - 1) / SORT_CHUNK;
    return halign(nb * (size_t)E * sizeof(int32_t)) + halign((size_t)E * sizeof(int32_t));
}

int launch_sort(const int32_t* ids, int T, int k, int E, const Plan& plan, int has_shared,
                int tile_m, int32_t* status, void* scratch, hipStream_t stream) {
    const int R = T * k;
    const int want_segments = plan.seg_n != nullptr;
    if (R <= SORT_SMALL_MAX_ROUTES) {
        constexpr int NW = SORT_SMALL_THREADS / MOE_WAVE;
        const size_t lds = sizeof(int) * ((size_t)NW * E + E + (E + 1) + 4 * (E + 2) + NW + 1);
        prof_begin("sort_small", stream);
        sort_small_kernel<<<1, SORT_SMALL_THREADS, lds, stream>>>(ids, T, k, E, plan, want_segments,
                                                                  has_shared, tile_m, status);
        prof_end(stream);
        return check_launch("sort_small_kernel");
    }
    const int nb = (R + SORT_CHUNK - 1) / SORT_CHUNK;
    int32_t* ghist = static_cast<int32_t*>(scratch);
    int32_t* totals = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) +
                                                 halign((size_t)nb * E * sizeof(int32_t)));
    prof_begin("sort_count", stream);
    sort_count_kernel<<<nb, SORT_THREADS, sizeof(int) * E, stream>>>(ids, R, E, nb, ghist, status);
    prof_end(stream);
    if (int rc = check_launch("sort_count_kernel")) return rc;
    constexpr int NW = SORT_THREADS / MOE_WAVE;
    // (measured: at 64 chunks the scan's launch costs more than the sums it
    // saves; at 160 chunks the placement went from 50 to 16 us with it)
    if (nb >= SORT_SCAN_MIN_CHUNKS) {
        prof_begin("sort_scan", stream);
        sort_scan_kernel<<<(E + NW - 1) / NW, SORT_THREADS, 0, stream>>>(ghist, E, nb, totals);
        prof_end(stream);
        if (int rc = check_launch("sort_scan_kernel")) return rc;
    } else {
        totals = nullptr;
    }
    const size_t lds = sizeof(int) * ((size_t)NW * E + E + (E + 1) + E + 4 * (E + 2) + NW + 1);
    prof_begin("sort_place", stream);
    sort_place_kernel<<<nb + 1, SORT_THREADS, lds, stream>>>(ids, T, k, E, nb, ghist, totals, plan,
                                                             want_segments, has_shared, tile_m);
    prof_end(stream);
    return check_launch("sort_place_kernel");
}

}  // namespace moe
