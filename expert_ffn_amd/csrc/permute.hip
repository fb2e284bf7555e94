// Stable grouping of routes by expert in one workgroup of 1024 threads.
//
// Winery-Strata's RemoteExperts::begin lists, per expert group, its routes in
// route order; rlx_runtime/expert_pool.rs count_hits is the per-expert
// histogram.  Here: an LDS histogram (integer atomics; counts do not depend on
// their order), a wave scan into group offsets, then blocks of 1024 routes in
// order: each wave finds the lanes sharing its expert with ballots, writes one
// per-(wave, expert) count, and every route's position is
//   base[e] + counts of earlier waves in the block + rank among equal lanes.
// No position depends on thread timing, so the result is deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PERM_THREADS = 1024;
constexpr int PERM_WAVES = PERM_THREADS / 64;
constexpr int PERM_MAX_E = 512;

__global__ __launch_bounds__(PERM_THREADS) void permute_kernel(
    const int* __restrict__ ids, int R, int E, const int* __restrict__ slot_of,
    int* __restrict__ offsets, int* __restrict__ sorted_route, int* __restrict__ route_pos,
    int* __restrict__ n_dropped) {
    __shared__ int s_count[PERM_MAX_E];
    __shared__ int s_base[PERM_MAX_E];
    __shared__ int s_res[PERM_MAX_E];
    __shared__ int s_wcnt[PERM_WAVES][PERM_MAX_E];
    __shared__ int s_drop;
    __shared__ int s_total;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < E; e += PERM_THREADS) {
        s_count[e] = 0;
        s_res[e] = slot_of[e] >= 0;
        for (int v = 0; v < PERM_WAVES; ++v) s_wcnt[v][e] = 0;
    }
    if (tid == 0) s_drop = 0;
    __syncthreads();

    // 1. histogram of kept routes, count of dropped ones
    int mydrop = 0;
    for (int i = tid; i < R; i += PERM_THREADS) {
        const int e = ids[i];
        if (e >= 0 && e < E && s_res[e])
            atomicAdd(&s_count[e], 1);
        else
            ++mydrop;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mydrop += __shfl_xor(mydrop, m, 64);
    if (lane == 0 && mydrop) atomicAdd(&s_drop, mydrop);
    __syncthreads();

    // 2. exclusive scan of the counts (wave 0, 64 experts per step)
    if (wave == 0) {
        int carry = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int c = e < E ? s_count[e] : 0;
            int incl = c;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d, 64);
                if (lane >= d) incl += o;
            }
            if (e < E) {
                s_base[e] = carry + incl - c;
                offsets[e] = carry + incl - c;
            }
            carry += __shfl(incl, 63, 64);
        }
        if (lane == 0) {
            offsets[E] = carry;
            s_total = carry;
            *n_dropped = s_drop;
        }
    }
    __syncthreads();

    // 3. stable positions, one block of 1024 routes at a time
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int blk = 0; blk < R; blk += PERM_THREADS) {
        const int i = blk + tid;
        int e = -1;
        if (i < R) {
            const int v = ids[i];
            if (v >= 0 && v < E && s_res[v]) e = v;
        }
        uint64_t peers = 0ull;
        uint64_t rem = __ballot(e >= 0);
        while (rem) {
            const int leader = __ffsll(static_cast<unsigned long long>(rem)) - 1;
            const int le = __shfl(e, leader, 64);
            const uint64_t m = __ballot(e == le);
            if (e == le) peers = m;
            rem &= ~m;
        }
        const int rank = __popcll(peers & lt_mask);
        if (e >= 0 && rank == 0) s_wcnt[wave][e] = __popcll(peers);
        __syncthreads();
        if (e >= 0) {
            int pos = s_base[e] + rank;
            for (int v = 0; v < wave; ++v) pos += s_wcnt[v][e];
            sorted_route[pos] = i;
            route_pos[i] = pos;
        } else if (i < R) {
            route_pos[i] = -1;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += PERM_THREADS) {
            int sum = 0;
            for (int v = 0; v < PERM_WAVES; ++v) {
                sum += s_wcnt[v][ee];
                s_wcnt[v][ee] = 0;
            }
            s_base[ee] += sum;
        }
        __syncthreads();
    }
    // 4. positions past the kept routes
    for (int p = s_total + tid; p < R; p += PERM_THREADS) sorted_route[p] = -1;
}

hipError_t launch_permute(const int* ids, int R, int E, const int* slot_of, int* offsets,
                          int* sorted_route, int* route_pos, int* n_dropped, hipStream_t s) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_THREADS), 0, s, ids, R, E, slot_of,
                       offsets, sorted_route, route_pos, n_dropped);
    return hipGetLastError();
}

}  // namespace moe
