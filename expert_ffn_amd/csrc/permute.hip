// Stable grouping of routes by expert: one workgroup of 1024 threads for up
// to 1024 routes (below), one per block of 1024 routes above that
// (permute_multi_kernel).
//
// Winery-Strata's RemoteExperts::begin lists, per expert group, its routes in
// route order; rlx_runtime/expert_pool.rs count_hits is the per-expert
// histogram.  Here: an LDS histogram (integer atomics; counts do not depend on
// their order), a wave scan into group offsets, then blocks of 1024 routes in
// order: each wave finds the lanes sharing its expert with one ballot per bit
// of the expert id, writes one per-(wave, expert) count, and every route's
// position is
//   base[e] + counts of earlier waves in the block + rank among equal lanes.
// No position depends on thread timing, so the result is deterministic.  The
// cross-lane steps use ballots, DPP and lane reads only (no LDS round trips),
// since the kernel is a chain of short dependent steps.
#include "common.h"
#include "kernels.h"
#include "route.h"

namespace moe {

constexpr int PERM_THREADS = 1024;
constexpr int PERM_WAVES = PERM_THREADS / 64;
constexpr int PERM_MAX_E = 512;
static_assert(PERM_MAX_E <= PERM_THREADS, "one expert per thread at set-up");

// inclusive prefix sum over the 64 lanes of a wave: DPP shifts inside rows of
// 16, then the totals of the lower rows (lane reads)
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

struct PermLds {
    int count[PERM_MAX_E];
    int base[PERM_MAX_E];
    int res[PERM_MAX_E];
    int wcnt[PERM_WAVES][PERM_MAX_E];   // per (wave, expert) count of the current block
    int drop;
    int total;
};

// Steps of the grouping for one workgroup of PERM_THREADS threads.  res: is
// expert tid resident (tid < E); id0: the expert of route tid (tid < R, else
// -1); routes of later blocks of 1024 are read from ids.  Each thread holds its
// routes of IB blocks at a time (one load each, all requested at once), so for
// up to IB blocks neither the histogram nor the positions wait for memory once
// per block.  With wpre ([PERM_WAVES][PERM_MAX_E] in LDS, IB > 1) a block's
// per-expert wave offsets are formed once by the expert's thread; without it
// each route adds up the counts of the earlier waves itself (fewer steps for a
// single block).
template <int PERM_IB>
__device__ __forceinline__ void permute_steps(PermLds& S, int (*wpre)[PERM_MAX_E], const int* __restrict__ ids, int id0,
                                              int res, int R, int E, int* __restrict__ offsets,
                                              int* __restrict__ sorted_route, int* __restrict__ route_pos,
                                              int* __restrict__ n_dropped) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < E) {
        S.count[tid] = 0;
        S.res[tid] = res;
        for (int v = 0; v < PERM_WAVES; ++v) S.wcnt[v][tid] = 0;
    }
    if (tid == 0) S.drop = 0;
    __syncthreads();

    // the kept expert (or -1) of route b0 + 1024 j + tid, j < PERM_IB
    auto load_batch = [&](int b0, int* ev) {
        int raw[PERM_IB];
#pragma unroll
        for (int j = 0; j < PERM_IB; ++j) {
            const int i = b0 + j * PERM_THREADS + tid;
            raw[j] = (b0 == 0 && j == 0) ? id0 : (i < R ? ids[i] : -1);
        }
#pragma unroll
        for (int j = 0; j < PERM_IB; ++j) {
            const int v = raw[j];
            ev[j] = (v >= 0 && v < E && S.res[v]) ? v : -1;
        }
    };
    constexpr int BATCH = PERM_IB * PERM_THREADS;
    int ev0[PERM_IB];   // the first batch, kept for the positions

    // 1. histogram of kept routes, count of dropped ones
    for (int b0 = 0; b0 < R; b0 += BATCH) {
        int ev[PERM_IB];
        load_batch(b0, ev);
        int nd = 0;
#pragma unroll
        for (int j = 0; j < PERM_IB; ++j) {
            const int i = b0 + j * PERM_THREADS + tid;
            if (ev[j] >= 0) atomicAdd(&S.count[ev[j]], 1);
            nd += __popcll(__ballot(i < R && ev[j] < 0));
            if (b0 == 0) ev0[j] = ev[j];
        }
        if (lane == 0 && nd) atomicAdd(&S.drop, nd);
    }
    __syncthreads();

    // 2. exclusive scan of the counts (wave 0, 64 experts per step)
    if (wave == 0) {
        int carry = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int c = e < E ? S.count[e] : 0;
            const int incl = wave_incl_scan(c);
            if (e < E) {
                S.base[e] = carry + incl - c;
                offsets[e] = carry + incl - c;
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
        if (lane == 0) {
            offsets[E] = carry;
            S.total = carry;
            *n_dropped = S.drop;
        }
    }
    __syncthreads();

    // 3. stable positions, one block of 1024 routes at a time: the lanes of a
    // wave with the same kept expert (one ballot per bit of the id) give each
    // route its rank and the wave's count; a route's position is base[e] plus
    // the counts of earlier waves plus its rank, and base[e] then moves past
    // the block
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;   // bits of an expert id
    for (int b0 = 0; b0 < R; b0 += BATCH) {
        int ev[PERM_IB];
        if (b0 == 0) {
#pragma unroll
            for (int j = 0; j < PERM_IB; ++j) ev[j] = ev0[j];
        } else {
            load_batch(b0, ev);
        }
#pragma unroll
        for (int j = 0; j < PERM_IB; ++j) {
            const int blk = b0 + j * PERM_THREADS;
            if (blk >= R) break;
            const int i = blk + tid, e = ev[j];
            uint64_t peers = __ballot(e >= 0);
            for (int bit = 0; bit < nbits; ++bit) {
                const bool mine = (e >> bit) & 1;
                const uint64_t bb = __ballot(mine);
                peers &= mine ? bb : ~bb;
            }
            const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(peers >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(peers), 0));
            if (e >= 0 && rank == 0) S.wcnt[wave][e] = __popcll(peers);
            __syncthreads();   // counts of the block in; positions of the last block read
            if constexpr (PERM_IB > 1) {
                for (int ee = tid; ee < E; ee += PERM_THREADS) {
                    int run = S.base[ee];
#pragma unroll
                    for (int v = 0; v < PERM_WAVES; ++v) {
                        const int c = S.wcnt[v][ee];
                        wpre[v][ee] = run;
                        S.wcnt[v][ee] = 0;
                        run += c;
                    }
                    S.base[ee] = run;
                }
                __syncthreads();
                if (e >= 0) {
                    const int pos = wpre[wave][e] + rank;
                    sorted_route[pos] = i;
                    route_pos[i] = pos;
                } else if (i < R) {
                    route_pos[i] = -1;
                }
                continue;
            }
            if (e >= 0) {
                int pos = S.base[e] + rank;
                for (int v = 0; v < wave; ++v) pos += S.wcnt[v][e];
                sorted_route[pos] = i;
                route_pos[i] = pos;
            } else if (i < R) {
                route_pos[i] = -1;
            }
            if (blk + PERM_THREADS < R) {   // set up the next block
                __syncthreads();
                for (int ee = tid; ee < E; ee += PERM_THREADS) {
                    int sum = 0;
                    for (int v = 0; v < PERM_WAVES; ++v) {
                        sum += S.wcnt[v][ee];
                        S.wcnt[v][ee] = 0;
                    }
                    S.base[ee] += sum;
                }
                __syncthreads();
            }
        }
    }
    // 4. positions past the kept routes
    for (int p = S.total + tid; p < R; p += PERM_THREADS) sorted_route[p] = -1;
}

__global__ __launch_bounds__(PERM_THREADS) void permute_kernel(
    const int* __restrict__ ids, int R, int E, const int* __restrict__ slot_of,
    int* __restrict__ offsets, int* __restrict__ sorted_route, int* __restrict__ route_pos,
    int* __restrict__ n_dropped) {
    __shared__ PermLds S;
    __shared__ int wpre[PERM_WAVES][PERM_MAX_E];
    const int tid = threadIdx.x;
    // both inputs requested at once: the residency of expert tid and route tid
    const int res = tid < E ? (slot_of[tid] >= 0) : 0;
    const int id0 = tid < R ? ids[tid] : -1;
    permute_steps<8>(S, wpre, ids, id0, res, R, E, offsets, sorted_route, route_pos, n_dropped);
}

// The same grouping for R > 1024 by ceil(R / 1024) workgroups with no
// exchange between them: workgroup b histograms all R routes (kept routes
// per expert, and those before its block of 1024), so every workgroup forms
// the same offsets, and its block's routes start at offset[e] + the count of
// earlier routes to e; inside the block the positions come from the wave
// ballots above.  Workgroup 0 writes offsets and n_dropped; each writes the
// -1 tail positions of its own range.  The positions equal the
// single-workgroup ones.
__global__ __launch_bounds__(PERM_THREADS) void permute_multi_kernel(
    const int* __restrict__ ids, int R, int E, const int* __restrict__ slot_of,
    int* __restrict__ offsets, int* __restrict__ sorted_route, int* __restrict__ route_pos,
    int* __restrict__ n_dropped) {
    constexpr int IB = 8;
    __shared__ int cnt_all[PERM_MAX_E], cnt_before[PERM_MAX_E], base[PERM_MAX_E], res_s[PERM_MAX_E];
    __shared__ int wcnt[PERM_WAVES][PERM_MAX_E];
    __shared__ int drop, total;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int blk0 = blockIdx.x * PERM_THREADS;
    const int res = tid < E ? (slot_of[tid] >= 0) : 0;
    const int own = blk0 + tid < R ? ids[blk0 + tid] : -1;   // this thread's route of the block
    if (tid < E) {
        cnt_all[tid] = 0;
        cnt_before[tid] = 0;
        res_s[tid] = res;
        for (int v = 0; v < PERM_WAVES; ++v) wcnt[v][tid] = 0;
    }
    if (tid == 0) drop = 0;
    __syncthreads();
    // 1. histograms of the kept routes: all, and those before this block
    for (int b0 = 0; b0 < R; b0 += IB * PERM_THREADS) {
        int raw[IB];
#pragma unroll
        for (int j = 0; j < IB; ++j) {
            const int i = b0 + j * PERM_THREADS + tid;
            raw[j] = i < R ? ids[i] : -1;
        }
        int nd = 0;
#pragma unroll
        for (int j = 0; j < IB; ++j) {
            const int i = b0 + j * PERM_THREADS + tid, v = raw[j];
            const int e = (v >= 0 && v < E && res_s[v]) ? v : -1;
            if (e >= 0) {
                atomicAdd(&cnt_all[e], 1);
                if (i < blk0) atomicAdd(&cnt_before[e], 1);
            }
            nd += __popcll(__ballot(i < R && e < 0));
        }
        if (lane == 0 && nd) atomicAdd(&drop, nd);
    }
    __syncthreads();
    // 2. offsets (wave 0, 64 experts per step); this block starts past the earlier routes
    if (wave == 0) {
        int carry = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int c = e < E ? cnt_all[e] : 0;
            const int incl = wave_incl_scan(c);
            if (e < E) {
                base[e] = carry + incl - c + cnt_before[e];
                if (blockIdx.x == 0) offsets[e] = carry + incl - c;
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
        if (lane == 0) {
            total = carry;
            if (blockIdx.x == 0) {
                offsets[E] = carry;
                *n_dropped = drop;
            }
        }
    }
    __syncthreads();
    // 3. positions of this block's routes
    const int i = blk0 + tid;
    const int e = (own >= 0 && own < E && res_s[own]) ? own : -1;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    uint64_t peers = __ballot(e >= 0);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool mine = (e >> bit) & 1;
        const uint64_t bb = __ballot(mine);
        peers &= mine ? bb : ~bb;
    }
    const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(peers >> 32),
                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(peers), 0));
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
        int pos = base[e] + rank;
        for (int v = 0; v < wave; ++v) pos += wcnt[v][e];
        sorted_route[pos] = i;
        route_pos[i] = pos;
    } else if (i < R) {
        route_pos[i] = -1;
    }
    // 4. positions past the kept routes, in this block's range
    if (i < R && i >= total) sorted_route[i] = -1;
}

// Router top-k and grouping in one workgroup, for R = T k <= 1024: wave w
// routes tokens w, w + 16, ...; the ids also go to LDS, and the grouping reads
// them there, so the two steps cost one launch and no round trip through
// memory between them.
template <int NPL>
__global__ __launch_bounds__(PERM_THREADS) void route_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, const int* __restrict__ slot_of,
    int* __restrict__ ids, float* __restrict__ w, int* __restrict__ offsets, int* __restrict__ sorted_route,
    int* __restrict__ route_pos, int* __restrict__ n_dropped) {
    __shared__ PermLds S;
    __shared__ int s_ids[PERM_THREADS];
    const int tid = threadIdx.x, R = T * k;
    const int res = tid < E ? (slot_of[tid] >= 0) : 0;
    for (int t = tid >> 6; t < T; t += PERM_WAVES) route_token<NPL>(logits, t, E, k, renorm, ids, w, s_ids);
    __syncthreads();
    const int id0 = tid < R ? s_ids[tid] : -1;
    permute_steps<1>(S, nullptr, ids, id0, res, R, E, offsets, sorted_route, route_pos, n_dropped);
}

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int renorm, const int* slot_of,
                                int* ids, float* w, int* offsets, int* sorted_route, int* route_pos,
                                int* n_dropped, hipStream_t s) {
    if (T * k > PERM_THREADS || T > 4 * PERM_WAVES) {
        const hipError_t e = launch_route_topk(logits, T, E, k, renorm, ids, w, s);
        if (e != hipSuccess) return e;
        return launch_permute(ids, T * k, E, slot_of, offsets, sorted_route, route_pos, n_dropped, s);
    }
    const dim3 grid(1), block(PERM_THREADS);
    if (E <= 64)
        hipLaunchKernelGGL(route_permute_kernel<1>, grid, block, 0, s, logits, T, E, k, renorm, slot_of, ids, w,
                           offsets, sorted_route, route_pos, n_dropped);
    else if (E <= 128)
        hipLaunchKernelGGL(route_permute_kernel<2>, grid, block, 0, s, logits, T, E, k, renorm, slot_of, ids, w,
                           offsets, sorted_route, route_pos, n_dropped);
    else if (E <= 256)
        hipLaunchKernelGGL(route_permute_kernel<4>, grid, block, 0, s, logits, T, E, k, renorm, slot_of, ids, w,
                           offsets, sorted_route, route_pos, n_dropped);
    else
        hipLaunchKernelGGL(route_permute_kernel<8>, grid, block, 0, s, logits, T, E, k, renorm, slot_of, ids, w,
                           offsets, sorted_route, route_pos, n_dropped);
    return hipGetLastError();
}

hipError_t launch_permute(const int* ids, int R, int E, const int* slot_of, int* offsets,
                          int* sorted_route, int* route_pos, int* n_dropped, hipStream_t s) {
    if (R > PERM_THREADS)
        hipLaunchKernelGGL(permute_multi_kernel, dim3((R + PERM_THREADS - 1) / PERM_THREADS), dim3(PERM_THREADS), 0,
                           s, ids, R, E, slot_of, offsets, sorted_route, route_pos, n_dropped);
    else
        hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_THREADS), 0, s, ids, R, E, slot_of,
                           offsets, sorted_route, route_pos, n_dropped);
    return hipGetLastError();
}

}  // namespace moe
