// Launch functions of the HIP kernels (internal; the C ABI is in include/expert_ffn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int renorm, int* ids,
                             float* w, hipStream_t s);
// router GEMV + top-k: x [T, H] (fp32 or bf16), wr fp32 [E, H]; logits fp32 [T, E] out;
// part fp32 [router_part_floats(T, H, E)] scratch (partial logits per H slice)
int64_t router_part_floats(int T, int H, int E);
hipError_t launch_router_topk(const void* x, bool xf32, const float* wr, int T, int H, int E, int k, int renorm,
                              float* logits, float* part, int* ids, float* w, hipStream_t s);
// residency refresh: one workgroup, E <= 512, budget <= S <= 512; slot_of updated in place
hipError_t launch_residency_refresh(const int* ids, int64_t R, int E, int budget, int S, int* slot_of, int* hits,
                                    int* target, int* promote, int* promote_slot, int* demote, int* counts,
                                    hipStream_t s);
// min_weight partial routing: ids_out / w_out (may alias ids / w), miss [E] (zeroed here)
hipError_t launch_min_weight(const int* ids, const float* w, int T, int k, int E, const int* slot_of, float share,
                             int* ids_out, float* w_out, int* miss, hipStream_t s);
hipError_t launch_permute(const int* ids, int R, int E, const int* slot_of, int* offsets,
                          int* sorted_route, int* route_pos, int* n_dropped, hipStream_t s);
// route + permute: one fused launch for T k <= 1024 (and T <= 64), else the two
hipError_t launch_route_permute(const float* logits, int T, int E, int k, int renorm, const int* slot_of,
                                int* ids, float* w, int* offsets, int* sorted_route, int* route_pos,
                                int* n_dropped, hipStream_t s);
hipError_t launch_combine(const void* out_routes, int out_dt, const float* w, const int* route_pos,
                          int T, int k, int H, void* y, int y_dt, hipStream_t s);
// canonical blob (int4 codes row-major) at src (device, or with host_src the
// device mapping of pinned host memory) -> slot blob (int4 codes tiled);
// off: the blob layout (5 entries, host)
hipError_t launch_fill_slot(int fmt, const void* src, bool host_src, int H, int FF, const uint64_t* off, void* slot,
                            hipStream_t s);
// n (<= FILL_MAX) canonical blobs back to back at src (device) -> slots[j] (host array of device pointers)
constexpr int FILL_MAX = 64;
hipError_t launch_fill_slots(int fmt, const void* src, int n, int H, int FF, const uint64_t* off, void* const* slots,
                             hipStream_t s);
// mismatches (device): 16-byte chunks of slot that differ from the canonical blob src
hipError_t launch_verify_slot(int fmt, const void* src, int H, int FF, const uint64_t* off, const void* slot,
                              int32_t* mismatches, hipStream_t s);
// tiled: int4 codes in the blob's 32-row tiles (N a multiple of 32), else row-major
hipError_t launch_quantize(int fmt, const uint16_t* w, int N, int K, void* q, void* scales, bool tiled,
                           hipStream_t s);

// Everything the expert-FFN kernels read and write.
struct FfnParams {
    const uint8_t* pool;
    uint64_t slot_bytes;
    const int* slot_of;
    int E, H, FF, fmt, act, T, k;
    const int* offsets;       // [E+1]
    const int* sorted_route;  // [T*k]
    const void* x;            // [T, H] fp32 or bf16 (x_dt)
    int x_dt;
    const uint16_t* xq;       // [T, H] bf16 in the w13 operand order (may alias x)
    uint16_t* xq_out;         // where the preparation kernel writes xq (workspace)
    float* xsum;              // group sums of xq per (token, 64-group) as bf16 hi [T, H/64] then lo; int4 fast gate/up
    float* xsum_out;          // where the preparation kernel may write them (workspace)
    uint16_t* xqg_out;        // the grouped GEMM's copy of x (M32 operand order) and its group
    uint16_t* xsumg_out;      //   sums (workspace; both kernel families can run in one call)
    uint16_t* h;              // [T*k, FF] bf16 in the w2 operand order (workspace)
    uint16_t* hsum;           // group sums of h per (route, 64-group of FF), bf16 hi then lo (int4 GEMM path)
    void* out;                // [T*k, H] fp32 or bf16 (out_dt)
    int out_dt;
    uint64_t o13, os13, o2, os2;  // blob sub-block offsets
    uint64_t kmul;            // ceil(2^32 / k): route -> token by a multiply (route_token)
    int gmin;                 // int4: groups of more than gmin routes belong to the grouped GEMM,
                              // the others to the streaming kernels (INT_MAX: no GEMM)
};

// token of route i = t * k + j (i < 2^30, k <= 32): q = (i * ceil(2^32 / k)) >> 32
// is t or t + 1 (the error i * (ceil - 2^32 / k) / 2^32 stays below 1/4), so one
// comparison corrects it; scalar multiplies instead of an integer division
__host__ __device__ __forceinline__ int route_token(int i, uint64_t kmul, int k) {
    const int q = static_cast<int>((static_cast<uint64_t>(static_cast<uint32_t>(i)) * kmul) >> 32);
    return q * k > i ? q - 1 : q;
}
inline uint64_t token_multiplier(int k) { return ((1ull << 32) + static_cast<uint64_t>(k) - 1) / static_cast<uint64_t>(k); }

// Workspace layout of the expert FFN.
struct FfnWorkspace {
    size_t xq_off, xsum_off, xqg_off, xsumg_off, h_off, hsum_off, bytes;
};
FfnWorkspace ffn_workspace(int T, int k, int H, int FF);

// Kernel family per expert group (int4): a group of m_e routes takes the
// grouped GEMM when m_e > GEMM_GROUP_MIN, else the streaming kernels (which
// take the routes 4 at a time against weights held in registers).  The GEMM
// family is launched only when T > GEMM_T_MIN (m_e <= T, and at decode sizes
// its launches would find no work); it runs on a second stream, beside the
// streaming kernels.  Measured at the Gemma shape, T = 64 to 1024, per layer:
// with the two families overlapped, 8 beat 16 by 17-27 % at T = 128-256 and by
// 7 % at T = 1024 with Zipf routing (a group of 9-16 routes is 3-4 sequential
// route tiles for the streaming kernels); 4 and 6 were no better, and 4 was
// 4 % slower at T = 1024.  Launching the GEMM from T > 32 rather than T > 64
// took a T = 64 layer with Zipf routing from 179 to 140 us.
#ifndef GEMM_GROUP_MIN_DEF
#define GEMM_GROUP_MIN_DEF 8
#endif
constexpr int GEMM_GROUP_MIN = GEMM_GROUP_MIN_DEF;
#ifndef GEMM_T_MIN_DEF
#define GEMM_T_MIN_DEF 32
#endif
constexpr int GEMM_T_MIN = GEMM_GROUP_MIN > GEMM_T_MIN_DEF ? GEMM_GROUP_MIN : GEMM_T_MIN_DEF;

// int4 grouped-GEMM path (large token groups): shape and LDS fit, checked
// before anything is launched
bool int4_gemm_eligible(const FfnParams& p);
hipError_t launch_int4_gemm(const FfnParams& p, int phases, hipStream_t s);

// fork: the grouped GEMM may run on a second stream of the device, joined
// back into s before the call returns (0 for callers that must create nothing)
hipError_t launch_ffn(const FfnParams& p, int phases /*1 gate_up, 2 down, 3 both*/, hipStream_t s, bool fork);

}  // namespace moe
