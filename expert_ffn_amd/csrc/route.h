// Router top-k on one wave per token.  Keys order logits descending, NaN below
// -inf, -0 == +0, equal logits by ascending expert id (prain README, "Trading
// quality for speed": top-k with renormalised softmax weights;
// rlx_runtime/expert_pool.rs ranks equal counts by the lower id).
#pragma once

#include "common.h"

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

// Top-k of one token's logits on one wave (t < T): ids in rank order (larger
// logit first, equal logits: lower expert id first), softmax weights over the
// k chosen (renorm) or over all E.
template <int NPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k, int renorm,
                                            int* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
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
        // the owner lane retires the winner and hands its logit to lane j
        float ve = val[0];
#pragma unroll
        for (int s = 0; s < NPL; ++s) {
            if (lane + 64 * s == e) key[s] = 0ull;
            if (s == (e >> 6)) ve = val[s];
        }
        ve = __shfl(ve, e & 63, 64);
        if (lane == j) {
            my_id = e;
            my_logit = ve;
        }
    }
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

}  // namespace moe
