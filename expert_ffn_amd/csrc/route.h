// Router top-k on one wave per token.  Logits order descending, NaN below
// -inf, -0 == +0, equal logits by ascending expert id (prain README, "Trading
// quality for speed": top-k with renormalised softmax weights;
// rlx_runtime/expert_pool.rs ranks equal counts by the lower id).
#pragma once

#include "common.h"

namespace moe {

// Order-preserving map of an fp32 logit to uint32: 0 = taken / no expert,
// NaN -> 1 (below -inf), -0 -> +0, otherwise the sign-flip image (>= 0x007FFFFF).
__device__ __forceinline__ uint32_t logit_ord(float v) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 1u;
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Cross-lane steps without LDS: DPP inside rows of 16, then the gfx950 row
// and half-wave swaps.  Every lane ends with the same result (the pairings
// are symmetric, and fp32 addition is commutative).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
// v_permlane16_swap / v_permlane32_swap of a register with itself: the two
// results hold, per lane, the lane's own value and its partner's (lane ^ 16,
// lane ^ 32), in an order that depends on the lane.
__device__ __forceinline__ uint32_t max16(uint32_t v) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max(p[0], p[1]);
}
__device__ __forceinline__ uint32_t max32(uint32_t v) {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(p[0], p[1]);
}
__device__ __forceinline__ float sum16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
constexpr int DPP_QUAD_1032 = 0xB1, DPP_QUAD_2301 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<DPP_QUAD_1032>(v));
    v = max(v, dpp_u32<DPP_QUAD_2301>(v));
    v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
    v = max(v, dpp_u32<DPP_ROW_MIRROR>(v));
    return max32(max16(v));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += __uint_as_float(dpp_u32<DPP_QUAD_1032>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<DPP_QUAD_2301>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<DPP_ROW_HALF_MIRROR>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<DPP_ROW_MIRROR>(__float_as_uint(v)));
    return sum32(sum16(v));
}

// Top-k of one token's logits on one wave (t < T): ids in rank order (larger
// logit first, equal logits: lower expert id first), softmax weights over the
// k chosen (renorm) or over all E, ids also to lds_ids if given.  Lane l holds
// experts l + 64 s.  A round
// takes the wave maximum of the ordered logits, then the lowest expert id
// holding it (ballots, lowest s first, then lowest lane).  The logits are in
// registers: val[s] = logit of expert lane + 64 s (ignored for experts >= E).
template <int NPL>
__device__ __forceinline__ void route_token_vals(const float (&val)[NPL], int t, int E, int k, int renorm,
                                                 int* __restrict__ ids, float* __restrict__ w,
                                                 int* lds_ids = nullptr) {
    const int lane = threadIdx.x & 63;
    uint32_t key[NPL];
#pragma unroll
    for (int s = 0; s < NPL; ++s) key[s] = lane + 64 * s < E ? logit_ord(val[s]) : 0u;
    int my_id = -1;
    float my_logit = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t best = key[0];
#pragma unroll
        for (int s = 1; s < NPL; ++s) best = max(best, key[s]);
        best = __builtin_amdgcn_readfirstlane(wave_max_u32(best));
        int e = 0;
        float ve = 0.0f;
#pragma unroll
        for (int s = NPL - 1; s >= 0; --s) {   // ends at the lowest s holding the maximum
            const uint64_t b = __ballot(key[s] == best);
            if (b != 0ull) {
                const int ln = __ffsll(static_cast<unsigned long long>(b)) - 1;
                e = ln + 64 * s;
                ve = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(val[s]), ln));
            }
        }
        // retire the winner; lane j keeps it
#pragma unroll
        for (int s = 0; s < NPL; ++s)
            if (lane + 64 * s == e) key[s] = 0u;
        if (lane == j) {
            my_id = e;
            my_logit = ve;
        }
    }
    const float m = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(my_logit)));
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
        if (lds_ids != nullptr) lds_ids[t * k + lane] = my_id;
    }
}

// The same, loading row t of logits [T, E] first.
template <int NPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k, int renorm,
                                            int* __restrict__ ids, float* __restrict__ w, int* lds_ids = nullptr) {
    const int lane = threadIdx.x & 63;
    const float* l = logits + static_cast<int64_t>(t) * E;
    float val[NPL];
#pragma unroll
    for (int s = 0; s < NPL; ++s) val[s] = lane + 64 * s < E ? l[lane + 64 * s] : 0.0f;
    route_token_vals<NPL>(val, t, E, k, renorm, ids, w, lds_ids);
}

}  // namespace moe
