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

typedef __attribute__((ext_vector_type(16))) float f32x16;

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

// Router GEMV and top-k (prain README, "int4 experts on RDNA2": the router is
// an fp32 GEMV whose logits feed the top-k): logits[t][e] = x_t . Wr_e in fp32,
// then the top-k above.  Two launches; the kernel boundary is the only
// synchronisation.
//
// router_part_kernel: workgroup (b, s, c) takes experts 8b .. 8b+7, the
// 256-element slice s of H and tokens 16c .. 16c+15.  One round of 16-byte
// loads stages the eight router row slices (fp32) and the tokens' x slices
// (widened to fp32) in LDS; lane l of wave w sums 64 products for token l / 4
// and experts l % 4 and l % 4 + 4 over elements 64w .. 64w+63 of the slice;
// the four wave sums are added in wave order and the slice's partial logits
// written to part [slice][T][E].
//
// router_topk_part_kernel: one wave per token adds the partials of the slices
// in slice order (a fixed order: reproducible logits), writes the logits and
// runs the top-k from registers.
constexpr int RT_TB = 16, RT_EB = 8, RT_HL = 256;

template <bool XF32>
__global__ __launch_bounds__(256) void router_part_kernel(const void* __restrict__ x, const float* __restrict__ wr,
                                                          int T, int H, int E, float* __restrict__ part) {
    __shared__ float xs[RT_TB][RT_HL + 4];
    __shared__ float ws[RT_EB][RT_HL + 4];
    __shared__ float red[4][128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e0 = blockIdx.x * RT_EB, h0 = blockIdx.y * RT_HL, t0 = blockIdx.z * RT_TB;
    const int nT = min(RT_TB, T - t0);
    const int hl = min(RT_HL, H - h0);   // a multiple of 64
    // loads first (clamped addresses, zeros outside), then the LDS writes
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const float* xf = static_cast<const float*>(x);
    f32x4 wv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {   // router rows: 8 x 256 fp32 = 512 chunks of 16 B
        const int q = tid + 256 * i, r = q >> 6, c = (q & 63) * 4;
        const bool ok = e0 + r < E && c < hl;
        wv[i] = *reinterpret_cast<const f32x4*>(wr + static_cast<int64_t>(ok ? e0 + r : 0) * H + (ok ? h0 + c : 0));
        if (!ok) wv[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (XF32) {   // 16 x 256 fp32 = 1024 chunks of 16 B
        f32x4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i, r = q >> 6, c = (q & 63) * 4;
            const bool ok = r < nT && c < hl;
            xv[i] = *reinterpret_cast<const f32x4*>(xf + static_cast<int64_t>(ok ? t0 + r : t0) * H + (ok ? h0 + c : 0));
            if (!ok) xv[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            *reinterpret_cast<f32x4*>(&xs[q >> 6][(q & 63) * 4]) = xv[i];
        }
    } else {      // 16 x 256 bf16 = 512 chunks of 16 B
        u32x4 xv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + 256 * i, r = q >> 5, c = (q & 31) * 8;
            const bool ok = r < nT && c < hl;
            xv[i] = *reinterpret_cast<const u32x4*>(xb + static_cast<int64_t>(ok ? t0 + r : t0) * H + (ok ? h0 + c : 0));
            if (!ok) xv[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + 256 * i, r = q >> 5, c = (q & 31) * 8;
            const u32x4 v = xv[i];
            f32x4 lo, hi;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lo[2 * j] = __uint_as_float(v[j] << 16);
                lo[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
                hi[2 * j] = __uint_as_float(v[2 + j] << 16);
                hi[2 * j + 1] = __uint_as_float(v[2 + j] & 0xFFFF0000u);
            }
            *reinterpret_cast<f32x4*>(&xs[r][c]) = lo;
            *reinterpret_cast<f32x4*>(&xs[r][c + 4]) = hi;
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + 256 * i;
        *reinterpret_cast<f32x4*>(&ws[q >> 6][(q & 63) * 4]) = wv[i];
    }
    __syncthreads();
    const int pt = lane >> 2, pe = lane & 3, hb = 64 * wave;
    float a0 = 0.0f, a1 = 0.0f;
    if (hb < hl) {
#pragma unroll 4
        for (int j = 0; j < 64; j += 4) {
            const f32x4 xv = *reinterpret_cast<const f32x4*>(&xs[pt][hb + j]);
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(&ws[pe][hb + j]);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(&ws[pe + 4][hb + j]);
            a0 += xv[0] * w0[0] + xv[1] * w0[1] + xv[2] * w0[2] + xv[3] * w0[3];
            a1 += xv[0] * w1[0] + xv[1] * w1[1] + xv[2] * w1[2] + xv[3] * w1[3];
        }
    }
    red[wave][lane] = a0;
    red[wave][64 + lane] = a1;
    __syncthreads();
    if (tid < 128) {
        const int l = tid & 63, t = l >> 2, e = (l & 3) + 4 * (tid >> 6);
        const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        if (t < nT && e0 + e < E) part[(static_cast<int64_t>(blockIdx.y) * T + t0 + t) * E + e0 + e] = v;
    }
}

// Larger tiles for T > 64: workgroup (b, s, c) takes experts 64b .. 64b+63,
// the 128-element slice s of H and tokens 64c .. 64c+63, staged in LDS as
// fp32.  Wave w computes the 32 x 32 block of tokens 32 (w / 2) .. and experts
// 32 (w % 2) .. with fp32 MFMA (v_mfma_f32_32x32x2f32: lane l gives row l % 32
// of A, a token, and column l % 32 of B, an expert, at k = l / 32).  Per 8
// elements of K, lane half h reads elements 4h .. 4h + 3 of both rows (one
// 16-byte LDS read each) and feeds them to 4 MFMAs: MFMA j's k = 0, 1 are
// elements j and 4 + j.  No cross-wave sum.
constexpr int RL_TB = 64, RL_EB = 64, RL_HL = 128;

template <bool XF32>
__global__ __launch_bounds__(256) void router_part_large_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ wr, int T, int H, int E,
                                                                float* __restrict__ part) {
    __shared__ float xs[RL_TB][RL_HL + 4];
    __shared__ float ws[RL_EB][RL_HL + 4];
    const int tid = threadIdx.x;
    const int e0 = blockIdx.x * RL_EB, h0 = blockIdx.y * RL_HL, t0 = blockIdx.z * RL_TB;
    const int nT = min(RL_TB, T - t0);
    const int hl = min(RL_HL, H - h0);   // a multiple of 64
    // Every load is issued (chunks outside the matrices read a valid address
    // and are replaced by zeros), then every LDS write: no branch between a
    // load and its use, so the loads are in flight together.
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const float* xf = static_cast<const float*>(x);
    f32x4 wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // router rows: 64 x 128 fp32 = 2048 chunks of 16 B
        const int q = tid + 256 * i, r = q >> 5, c = (q & 31) * 4;
        const bool ok = e0 + r < E && c < hl;
        wv[i] = *reinterpret_cast<const f32x4*>(wr + static_cast<int64_t>(ok ? e0 + r : 0) * H + (ok ? h0 + c : 0));
        if (!ok) wv[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (XF32) {   // 64 x 128 fp32 = 2048 chunks of 16 B
        f32x4 xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = tid + 256 * i, r = q >> 5, c = (q & 31) * 4;
            const bool ok = r < nT && c < hl;
            xv[i] = *reinterpret_cast<const f32x4*>(xf + static_cast<int64_t>(ok ? t0 + r : t0) * H + (ok ? h0 + c : 0));
            if (!ok) xv[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = tid + 256 * i;
            *reinterpret_cast<f32x4*>(&xs[q >> 5][(q & 31) * 4]) = xv[i];
        }
    } else {      // 64 x 128 bf16 = 1024 chunks of 16 B
        u32x4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i, r = q >> 4, c = (q & 15) * 8;
            const bool ok = r < nT && c < hl;
            xv[i] = *reinterpret_cast<const u32x4*>(xb + static_cast<int64_t>(ok ? t0 + r : t0) * H + (ok ? h0 + c : 0));
            if (!ok) xv[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i, r = q >> 4, c = (q & 15) * 8;
            const u32x4 v = xv[i];
            f32x4 lo, hi;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lo[2 * j] = __uint_as_float(v[j] << 16);
                lo[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
                hi[2 * j] = __uint_as_float(v[2 + j] << 16);
                hi[2 * j + 1] = __uint_as_float(v[2 + j] & 0xFFFF0000u);
            }
            *reinterpret_cast<f32x4*>(&xs[r][c]) = lo;
            *reinterpret_cast<f32x4*>(&xs[r][c + 4]) = hi;
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = tid + 256 * i;
        *reinterpret_cast<f32x4*>(&ws[q >> 5][(q & 31) * 4]) = wv[i];
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63, h = lane >> 5;
    const int tr = 32 * (wave >> 1) + (lane & 31), er = 32 * (wave & 1) + (lane & 31);
    f32x16 acc = {};
    for (int k8 = 0; k8 < hl; k8 += 8) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(&xs[tr][k8 + 4 * h]);
        const f32x4 wv = *reinterpret_cast<const f32x4*>(&ws[er][k8 + 4 * h]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xv[j], wv[j], acc, 0, 0, 0);
    }
    // lane: expert column er, token rows 8 (v / 4) + 4 h + (v % 4) of the wave's 32
    const int ecol = e0 + er;
    if (ecol < E) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = 32 * (wave >> 1) + 8 * (v >> 2) + 4 * h + (v & 3);
            if (t < nT) part[(static_cast<int64_t>(blockIdx.y) * T + t0 + t) * E + ecol] = acc[v];
        }
    }
}

template <int NPL>
__global__ __launch_bounds__(256) void router_topk_part_kernel(const float* __restrict__ part, int HS, int T, int E,
                                                               int k, int renorm, float* __restrict__ logits,
                                                               int* __restrict__ ids, float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= T) return;
    float val[NPL];
#pragma unroll
    for (int s = 0; s < NPL; ++s) {
        const int e = lane + 64 * s;
        float v = 0.0f;
        if (e < E) {
            // eight slices' loads in flight at a time, added in slice order
            const float* p = part + static_cast<int64_t>(t) * E + e;
            const int64_t stride = static_cast<int64_t>(T) * E;
            for (int s0 = 0; s0 < HS; s0 += 8) {
                float b[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) b[j] = s0 + j < HS ? p[(s0 + j) * stride] : 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (s0 + j < HS) v = s0 + j == 0 ? b[j] : v + b[j];
            }
            logits[static_cast<int64_t>(t) * E + e] = v;
        }
        val[s] = v;
    }
    route_token_vals<NPL>(val, t, E, k, renorm, ids, w);
}

static bool router_large(int T) { return T > 64; }

int64_t router_part_floats(int T, int H, int E) {
    const int hl = router_large(T) ? RL_HL : RT_HL;
    return static_cast<int64_t>((H + hl - 1) / hl) * T * E;
}

hipError_t launch_router_topk(const void* x, bool xf32, const float* wr, int T, int H, int E, int k, int renorm,
                              float* logits, float* part, int* ids, float* w, hipStream_t s) {
    const dim3 block(256);
    int HS;
    if (router_large(T)) {
        HS = (H + RL_HL - 1) / RL_HL;
        const dim3 grid((E + RL_EB - 1) / RL_EB, HS, (T + RL_TB - 1) / RL_TB);
        auto pk = xf32 ? router_part_large_kernel<true> : router_part_large_kernel<false>;
        hipLaunchKernelGGL(pk, grid, block, 0, s, x, wr, T, H, E, part);
    } else {
        HS = (H + RT_HL - 1) / RT_HL;
        const dim3 grid((E + RT_EB - 1) / RT_EB, HS, (T + RT_TB - 1) / RT_TB);
        auto pk = xf32 ? router_part_kernel<true> : router_part_kernel<false>;
        hipLaunchKernelGGL(pk, grid, block, 0, s, x, wr, T, H, E, part);
    }
    const dim3 g2((T + 3) / 4);   // the slice sums run in slice order either way
    auto tk = E <= 64 ? router_topk_part_kernel<1>
                      : E <= 128 ? router_topk_part_kernel<2>
                                 : E <= 256 ? router_topk_part_kernel<4> : router_topk_part_kernel<8>;
    hipLaunchKernelGGL(tk, g2, block, 0, s, part, HS, T, E, k, renorm, logits, ids, w);
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
