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
// wave per token, lane j holding route j.  Resident routes are kept; the
// non-resident ones are taken heaviest first (equal weights: lower j) while
// the kept weight is below min_weight times the token's weight W; the rest are
// skipped (id -1, weight 0) and the kept weights scaled by W / kept.
// min_weight >= 1 keeps every valid route unchanged.  Ids outside [0, E) are
// skipped and not part of W.  fp32 throughout; the sums run in route order
// (resident first, then the order of taking) as a wave-uniform loop over lane
// reads, so the decisions are reproducible.  Every lane loads its route
// before any lane writes: ids_out / w_out may alias ids / w.
__device__ __forceinline__ float lane_f(float v, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

__global__ __launch_bounds__(256) void min_weight_kernel(const int* ids, const float* w, int T, int k, int E,
                                                         const int* __restrict__ slot_of, float share, int* ids_out,
                                                         float* w_out, int* __restrict__ miss) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // wave-uniform
    const int64_t r = static_cast<int64_t>(t) * k + lane;
    int e = -1;
    float wj = 0.0f;
    bool v = false, rs = false;
    if (lane < k) {
        e = ids[r];
        wj = w[r];
        v = e >= 0 && e < E;
        rs = v && slot_of[e] >= 0;
    }
    const uint32_t valid = static_cast<uint32_t>(__ballot(v)), res = static_cast<uint32_t>(__ballot(rs));
    float W = 0.0f;
    for (int j = 0; j < k; ++j)
        if ((valid >> j) & 1u) W += lane_f(wj, j);
    uint32_t keep = valid;
    float c = 0.0f;
    if (!(share >= 1.0f)) {
        keep = res;
        for (int j = 0; j < k; ++j)
            if ((res >> j) & 1u) c += lane_f(wj, j);
        const float target = share * W;
        for (uint32_t todo = valid & ~res; todo;) {
            int b = -1;
            float wb = 0.0f;
            for (int j = 0; j < k; ++j) {
                const float x = lane_f(wj, j);
                if (((todo >> j) & 1u) && (b < 0 || x > wb)) {
                    b = j;
                    wb = x;
                }
            }
            todo &= ~(1u << b);
            if (c >= target) continue;
            keep |= 1u << b;
            c += wb;
        }
    }
    const bool skipped = (valid & ~keep) != 0;
    const float scale = (skipped && c > 0.0f) ? W / c : 1.0f;
    if (lane < k) {
        const bool kj = (keep >> lane) & 1u;
        ids_out[r] = kj ? e : -1;
        w_out[r] = kj ? (skipped ? wj * scale : wj) : 0.0f;
        if (kj && !rs) atomicAdd(miss + e, 1);
    }
}

__global__ void zero_counts_kernel(int* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

hipError_t launch_min_weight(const int* ids, const float* w, int T, int k, int E, const int* slot_of, float share,
                             int* ids_out, float* w_out, int* miss, hipStream_t s) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, s, miss, E);
    if (T > 0)
        hipLaunchKernelGGL(min_weight_kernel, dim3((T + 3) / 4), dim3(256), 0, s, ids, w, T, k, E, slot_of,
                           share, ids_out, w_out, miss);
    return hipGetLastError();
}

}  // namespace moe
