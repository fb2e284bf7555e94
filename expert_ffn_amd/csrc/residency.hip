// Residency refresh from the device's own routing (rlx_runtime expert_pool.rs,
// TIDE-style placement: hit counts, the gpu_budget most-hit experts as target,
// paired promote/demote), one workgroup of 512 threads (E, S <= 512).
//
//  1. hit counts of the step's routes (LDS atomics: integer, order-free);
//  2. rank of expert e = experts with more hits, or as many and a lower id;
//     the target is ranks < budget among experts with hits > 0;
//  3. promotions: target entries not resident, in rank order; demotions: the
//     resident experts outside the target in ascending id, as many as there
//     are promotions; free slots in ascending order -- each an exclusive
//     prefix count of a flag (ballots within a wave, wave totals in LDS);
//  4. promotion j takes the slot of demotion j, or free slot j - demotions;
//     the table is read whole before it is rewritten (it may be updated in
//     place).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RR_THREADS = 512, RR_MAX = 512;

// exclusive prefix count of f over the 512 threads, and the total
__device__ __forceinline__ int block_excl_count(bool f, int* wtot, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t b = __ballot(f);
    const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
    __syncthreads();   // wtot free for reuse
    if (lane == 0) wtot[wave] = __popcll(b);
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < RR_THREADS / 64; ++w) {
        before += w < wave ? wtot[w] : 0;
        all += wtot[w];
    }
    total = all;
    return before + in_wave;
}

__global__ __launch_bounds__(RR_THREADS) void residency_refresh_kernel(const int* __restrict__ ids, int64_t R, int E,
                                                                       int budget, int S, int* slot_of,
                                                                       int* __restrict__ hits, int* __restrict__ target,
                                                                       int* __restrict__ promote,
                                                                       int* __restrict__ promote_slot,
                                                                       int* __restrict__ demote,
                                                                       int* __restrict__ counts) {
    __shared__ int hist[RR_MAX], slot_in[RR_MAX], tgt[RR_MAX], in_t[RR_MAX], used[RR_MAX];
    __shared__ int prom[RR_MAX], dem[RR_MAX], freeslot[RR_MAX], newslot[RR_MAX], wtot[RR_THREADS / 64];
    const int tid = threadIdx.x;
    if (tid < E) {
        hist[tid] = 0;
        in_t[tid] = 0;
        newslot[tid] = -2;   // not promoted
        slot_in[tid] = slot_of[tid];
    }
    if (tid < S) used[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < R; i += RR_THREADS) {
        const int e = ids[i];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    if (tid < E && slot_in[tid] >= 0 && slot_in[tid] < S) used[slot_in[tid]] = 1;
    __syncthreads();
    // 2. ranks and the target
    bool sel = false;
    if (tid < E) {
        const int h = hist[tid];
        int rank = 0;
        for (int e2 = 0; e2 < E; ++e2) {
            const int h2 = hist[e2];
            rank += (h2 > h) || (h2 == h && e2 < tid);
        }
        hits[tid] = h;
        sel = h > 0 && rank < budget;
        if (sel) {
            tgt[rank] = tid;
            in_t[tid] = 1;
        }
    }
    int nt;
    (void)block_excl_count(sel, wtot, nt);
    __syncthreads();
    // 3. promotions in rank order, demotions in id order, free slots in order
    const bool pf = tid < nt && slot_in[tgt[tid]] < 0;
    int np;
    const int pi = block_excl_count(pf, wtot, np);
    if (pf) prom[pi] = tgt[tid];
    const bool df = tid < E && slot_in[tid] >= 0 && !in_t[tid];
    int ncan;
    const int di = block_excl_count(df, wtot, ncan);
    const int nd = min(np, ncan);
    if (df && di < nd) dem[di] = tid;
    const bool ff = tid < S && !used[tid];
    int nfree;
    const int fi = block_excl_count(ff, wtot, nfree);
    if (ff && fi < np - nd) freeslot[fi] = tid;
    __syncthreads();
    // 4. slots of the promotions, then the new table
    if (tid < np) {
        const int sl = tid < nd ? slot_in[dem[tid]] : (tid - nd < nfree ? freeslot[tid - nd] : -1);
        promote[tid] = prom[tid];
        promote_slot[tid] = sl;
        newslot[prom[tid]] = sl;
    }
    if (tid < nd) demote[tid] = dem[tid];
    if (tid < budget) target[tid] = tid < nt ? tgt[tid] : -1;
    __syncthreads();
    if (tid < nd) newslot[dem[tid]] = -1;
    __syncthreads();
    if (tid < E) slot_of[tid] = newslot[tid] == -2 ? slot_in[tid] : newslot[tid];
    if (tid == 0) {
        counts[0] = nt;
        counts[1] = np;
        counts[2] = nd;
    }
}

hipError_t launch_residency_refresh(const int* ids, int64_t R, int E, int budget, int S, int* slot_of, int* hits,
                                    int* target, int* promote, int* promote_slot, int* demote, int* counts,
                                    hipStream_t s) {
    hipLaunchKernelGGL(residency_refresh_kernel, dim3(1), dim3(RR_THREADS), 0, s, ids, R, E, budget, S, slot_of, hits,
                       target, promote, promote_slot, demote, counts);
    return hipGetLastError();
}

}  // namespace moe
