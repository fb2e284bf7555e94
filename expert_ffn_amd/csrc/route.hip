// Router top-k with softmax weights: one wavefront per token.
//
// Each lane holds NPL = ceil(E / 64) logits in registers as 64-bit keys
// (order-preserving image of the logit << 32 | ~expert), so one wave-wide max
// picks the best remaining expert with the lower id winning ties (the tie rule
// of rlx_runtime/expert_pool.rs, target_gpu_from_counts).  k rounds of a
// 6-step butterfly max give the ids in rank order; lanes j < k then compute the
// softmax weights (prain README, "Trading quality for speed").
#include "common.h"
#include "kernels.h"

namespace moe {

// Order-preserving map of an fp32 logit to uint32: NaN -> 0 (below -inf),
// -0 -> +0, otherwise the usual sign-flip trick.  Key 0 = taken / no expert.
__device__ __forceinline__ uint64_t logit_key(float v, int e) {
    uint32_t b = __float_as_uint(v);
    uint32_t ord;
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) {
        ord = 0u;
    } else {
        if (b == 0x80000000u) b = 0u;
        ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
        uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
        uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         int* __restrict__ ids,
                                                         float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* l = logits + static_cast<int64_t>(t) * E;
    uint64_t key[NPL];
    float val[NPL];
#pragma unroll
    for (int s = 0; s < NPL; ++s) {
        const int e = lane + 64 * s;
        val[s] = e < E ? l[e] : 0.0f;
        key[s] = e < E ? logit_key(val[s], e) : 0ull;
    }
    int my_id = -1;
    float my_logit = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0ull;
#pragma unroll
        for (int s = 0; s < NPL; ++s) best = key[s] > best ? key[s] : best;
        best = wave_max_u64(best);
        const int e = static_cast<int>(~static_cast<uint32_t>(best));
        // the owner lane retires the winner
#pragma unroll
        for (int s = 0; s < NPL; ++s)
            if (lane + 64 * s == e) key[s] = 0ull;
        if (lane == j) my_id = e;
    }
    if (lane < k) my_logit = l[my_id];
    const float m = __shfl(my_logit, 0, 64);
    const float ex = lane < k ? expf(my_logit - m) : 0.0f;
    float den;
    if (renorm) {
        den = wave_sum_f32(ex);
    } else {
        float part = 0.0f;
#pragma unroll
        for (int s = 0; s < NPL; ++s)
            if (lane + 64 * s < E) part += expf(val[s] - m);
        den = wave_sum_f32(part);
    }
    if (lane < k) {
        ids[static_cast<int64_t>(t) * k + lane] = my_id;
        w[static_cast<int64_t>(t) * k + lane] = ex / den;
    }
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
