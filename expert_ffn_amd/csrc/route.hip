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

}  // namespace moe
