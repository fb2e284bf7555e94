// Weighted scatter-combine back to token order (Winery-Strata
// RemoteExperts::finish; prain README, "Trading quality for speed").
// One thread per 8 consecutive outputs of a token; the k routes are summed in
// ascending j in fp32, dropped routes (position -1) skipped.
#include "common.h"
#include "kernels.h"

namespace moe {

template <int OT, int YT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ out_routes,
                                                      const float* __restrict__ w,
                                                      const int* __restrict__ route_pos, int k,
                                                      int H, void* __restrict__ y) {
    const int t = blockIdx.x;
    const int n0 = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (n0 >= H) return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
        const int p = route_pos[static_cast<int64_t>(t) * k + j];
        if (p < 0) continue;
        const float wj = w[static_cast<int64_t>(t) * k + j];
        const int64_t base = static_cast<int64_t>(p) * H + n0;
        if (OT == F32) {
            const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(out_routes) + base);
            const f32x4 a = src[0], b = src[1];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                acc[v] += wj * a[v];
                acc[4 + v] += wj * b[v];
            }
        } else {
            const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(out_routes) + base);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                acc[2 * v] += wj * __uint_as_float(a[v] << 16);
                acc[2 * v + 1] += wj * __uint_as_float(a[v] & 0xFFFF0000u);
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
    const dim3 grid(T, (H / 8 + 255) / 256), block(256);
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
