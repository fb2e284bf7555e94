// Weighted scatter-combine back to token order (Winery-Strata
// RemoteExperts::finish; prain README, "Trading quality for speed").
// One thread per 8 consecutive outputs of a token; the k routes are summed in
// ascending j in fp32, dropped routes (position -1) skipped.  Routes are taken
// CMB_CH at a time: their positions (uniform, scalar loads) and rows are all
// requested before the first is added, so a thread waits for one round trip
// per chunk instead of one per route.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int CMB_THREADS = 64;
constexpr int CMB_CH = 8;

template <int OT>
__device__ __forceinline__ void load_row8(const void* __restrict__ out_routes, int64_t base, u32x4 (&r)[2]) {
    if (OT == F32) {
        const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(out_routes) + base);
        r[0] = src[0];
        r[1] = src[1];
    } else {
        r[0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(out_routes) + base);
        r[1] = r[0];
    }
}

template <int OT, int YT>
__global__ __launch_bounds__(CMB_THREADS) void combine_kernel(const void* __restrict__ out_routes,
                                                              const float* __restrict__ w,
                                                              const int* __restrict__ route_pos, int k,
                                                              int H, void* __restrict__ y) {
    const int t = blockIdx.x;
    const int n0 = (blockIdx.y * CMB_THREADS + threadIdx.x) * 8;
    if (n0 >= H) return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += CMB_CH) {
        int pj[CMB_CH];
        float wj[CMB_CH];
        u32x4 rows[CMB_CH][2];
#pragma unroll
        for (int c = 0; c < CMB_CH; ++c) {
            const int j = min(j0 + c, k - 1);
            pj[c] = route_pos[static_cast<int64_t>(t) * k + j];
            wj[c] = w[static_cast<int64_t>(t) * k + j];
        }
#pragma unroll
        for (int c = 0; c < CMB_CH; ++c)
            load_row8<OT>(out_routes, static_cast<int64_t>(max(pj[c], 0)) * H + n0, rows[c]);
#pragma unroll
        for (int c = 0; c < CMB_CH; ++c) {
            if (j0 + c >= k || pj[c] < 0) continue;
            if (OT == F32) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc[v] += wj[c] * __uint_as_float(rows[c][0][v]);
                    acc[4 + v] += wj[c] * __uint_as_float(rows[c][1][v]);
                }
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc[2 * v] += wj[c] * __uint_as_float(rows[c][0][v] << 16);
                    acc[2 * v + 1] += wj[c] * __uint_as_float(rows[c][0][v] & 0xFFFF0000u);
                }
            }
        }
    }
    const int64_t ob = static_cast<int64_t>(t) * H + n0;
    if (YT == F32) {
        f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(y) + ob);
        dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
        dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
        u32x4 o;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            o[v] = static_cast<uint32_t>(f32_to_bf16(acc[2 * v])) |
                   (static_cast<uint32_t>(f32_to_bf16(acc[2 * v + 1])) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + ob) = o;
    }
}

hipError_t launch_combine(const void* out_routes, int out_dt, const float* w, const int* route_pos,
                          int T, int k, int H, void* y, int y_dt, hipStream_t s) {
    const dim3 grid(T, (H / 8 + CMB_THREADS - 1) / CMB_THREADS), block(CMB_THREADS);
    if (out_dt == F32 && y_dt == F32)
        hipLaunchKernelGGL((combine_kernel<F32, F32>), grid, block, 0, s, out_routes, w, route_pos, k, H, y);
    else if (out_dt == F32)
        hipLaunchKernelGGL((combine_kernel<F32, BF16>), grid, block, 0, s, out_routes, w, route_pos, k, H, y);
    else if (y_dt == F32)
        hipLaunchKernelGGL((combine_kernel<BF16, F32>), grid, block, 0, s, out_routes, w, route_pos, k, H, y);
    else
        hipLaunchKernelGGL((combine_kernel<BF16, BF16>), grid, block, 0, s, out_routes, w, route_pos, k, H, y);
    return hipGetLastError();
}

}  // namespace moe
