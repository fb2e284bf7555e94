// Router top-k with softmax weights: one wavefront per token.
//
// Each lane holds NPL = ceil(E / 64) logits in registers with their
// order-preserving 32-bit images.  A round takes the wave maximum of the
// images (DPP and lane swaps, no LDS) and then the lowest expert id holding it
// (ballots), which is the tie rule of rlx_runtime/expert_pool.rs
// (target_gpu_from_counts).  k rounds give the ids in rank order; lanes j < k
// then compute the softmax weights (prain README, "Trading quality for speed").
#include "common.h"
#include "kernels.h"
#include "route.h"

namespace moe {

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         int* __restrict__ ids,
                                                         float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    route_token<NPL>(logits, t, E, k, renorm, ids, w);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int renorm, int* ids,
                             float* w, hipStream_t s) {
    const dim3 grid((T + 3) / 4), block(256);
    if (E <= 64)
        hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (E <= 128)
        hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (E <= 256)
        hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    return hipGetLastError();
}

// min_weight partial routing (prain README, "Trading quality for speed"), one
// thread per token.  Resident routes are kept; the non-resident ones are taken
// heaviest first (equal weights: lower j) while the kept weight is below
// min_weight times the token's weight W; the rest are skipped (id -1, weight
// 0) and the kept weights scaled by W / kept.  min_weight >= 1 keeps every
// valid route unchanged.  Ids outside [0, E) are skipped and not part of W.
// fp32 throughout, sums in route order (resident first, then the order of
// taking), so the decisions are reproducible.  Reads a token's routes before
// writing them: ids_out / w_out may alias ids / w.
__global__ __launch_bounds__(256) void min_weight_kernel(const int* ids, const float* w, int T, int k, int E,
                                                         const int* __restrict__ slot_of, float share, int* ids_out,
                                                         float* w_out, int* __restrict__ miss) {
#pragma clang fp contract(off)
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const int* id = ids + static_cast<int64_t>(t) * k;
    const float* wt = w + static_cast<int64_t>(t) * k;
    uint32_t valid = 0, res = 0;
    float W = 0.0f;
    for (int j = 0; j < k; ++j) {
        const int e = id[j];
        if (e < 0 || e >= E) continue;
        valid |= 1u << j;
        W += wt[j];
        if (slot_of[e] >= 0) res |= 1u << j;
    }
    uint32_t keep = valid;
    float c = 0.0f;
    if (!(share >= 1.0f)) {
        keep = res;
        for (int j = 0; j < k; ++j)
            if ((res >> j) & 1u) c += wt[j];
        const float target = share * W;
        for (uint32_t todo = valid & ~res; todo;) {
            int b = -1;
            for (int j = 0; j < k; ++j)
                if (((todo >> j) & 1u) && (b < 0 || wt[j] > wt[b])) b = j;
            todo &= ~(1u << b);
            if (c >= target) continue;
            keep |= 1u << b;
            c += wt[b];
        }
    }
    const bool skipped = (valid & ~keep) != 0;
    const float scale = (skipped && c > 0.0f) ? W / c : 1.0f;
    for (int j = 0; j < k; ++j) {
        const int e = id[j];
        const float wj = wt[j];
        const bool kj = (keep >> j) & 1u;
        ids_out[static_cast<int64_t>(t) * k + j] = kj ? e : -1;
        w_out[static_cast<int64_t>(t) * k + j] = kj ? (skipped ? wj * scale : wj) : 0.0f;
        if (kj && !((res >> j) & 1u)) atomicAdd(miss + e, 1);
    }
}

__global__ void zero_counts_kernel(int* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

hipError_t launch_min_weight(const int* ids, const float* w, int T, int k, int E, const int* slot_of, float share,
                             int* ids_out, float* w_out, int* miss, hipStream_t s) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, s, miss, E);
    if (T > 0)
        hipLaunchKernelGGL(min_weight_kernel, dim3((T + 255) / 256), dim3(256), 0, s, ids, w, T, k, E, slot_of,
                           share, ids_out, w_out, miss);
    return hipGetLastError();
}

}  // namespace moe
