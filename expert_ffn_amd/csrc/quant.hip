// Bit-exact quantisers for the two packed expert formats (prain README,
// "Expert formats": int8 with an fp32 scale per row; int4 with a bf16 scale per
// 64 elements chosen by an MSE clip search), and the expert blob writer.
//
// Every floating-point step is one IEEE operation rounded to nearest even:
// hipcc's fp32 division is correctly rounded, rintf is round-half-even, and
// FMA contraction is switched off below so that products and sums round
// separately, as the format's definition states them.
#include "common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace moe {

// int8: one wavefront per row; absmax by a wave max (exact in any order).
__global__ __launch_bounds__(256) void quant_int8_kernel(const uint16_t* __restrict__ w, int N,
                                                         int K, int8_t* __restrict__ q,
                                                         float* __restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= N) return;
    const uint16_t* row = w + static_cast<int64_t>(r) * K;
    float a = 0.0f;
    for (int c = lane; c < K; c += 64) a = fmaxf(a, fabsf(bf16_to_f32(row[c])));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
    const float sc = (a == 0.0f) ? 0.0f : a / 127.0f;
    if (lane == 0) s[r] = sc;
    for (int c = lane; c < K; c += 64) {
        float code = 0.0f;
        if (sc != 0.0f) code = fminf(fmaxf(rintf(bf16_to_f32(row[c]) / sc), -127.0f), 127.0f);
        q[static_cast<int64_t>(r) * K + c] = static_cast<int8_t>(code);
    }
}

// int4: one thread per (row, group of 64).  Candidate i has scale
// s_i = bf16(fp32(a * (20 - i)) / 140), i.e. clip alpha = (20 - i) / 20 of a / 7.
__global__ __launch_bounds__(256) void quant_int4_kernel(const uint16_t* __restrict__ w, int N,
                                                         int K, uint8_t* __restrict__ q,
                                                         uint16_t* __restrict__ s, int tiled) {
    const int G = K / 64;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= static_cast<int64_t>(N) * G) return;
    const int r = static_cast<int>(gid / G), g = static_cast<int>(gid % G);
    const uint16_t* src = w + static_cast<int64_t>(r) * K + static_cast<int64_t>(g) * 64;
    float v[64];
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < 64; ++c) {
        v[c] = bf16_to_f32(src[c]);
        a = fmaxf(a, fabsf(v[c]));
    }
    double best_err = 0.0;
    uint16_t best_s = 0;
    for (int i = 0; i < 10; ++i) {
        const uint16_t sb = f32_to_bf16((a * static_cast<float>(20 - i)) / 140.0f);
        const float sc = bf16_to_f32(sb);
        double err = 0.0;
        for (int c = 0; c < 64; ++c) {
            const float code = (sc == 0.0f) ? 0.0f : fminf(fmaxf(rintf(v[c] / sc), -8.0f), 7.0f);
            const double d = static_cast<double>(v[c]) - static_cast<double>(sc) * static_cast<double>(code);
            err = err + d * d;
        }
        if (i == 0 || err < best_err) {
            best_err = err;
            best_s = sb;
        }
    }
    s[gid] = best_s;
    const float sc = bf16_to_f32(best_s);
    // the group's 32 bytes: row-major codes, or the blob's 32-row tiles
    uint8_t* out = q + (tiled ? int4_code_off(r, G, 32 * g) : static_cast<int64_t>(r) * (K / 2) + static_cast<int64_t>(g) * 32);
    for (int b = 0; b < 32; ++b) {
        int lo = 0, hi = 0;
        if (sc != 0.0f) {
            lo = static_cast<int>(fminf(fmaxf(rintf(v[2 * b] / sc), -8.0f), 7.0f));
            hi = static_cast<int>(fminf(fmaxf(rintf(v[2 * b + 1] / sc), -8.0f), 7.0f));
        }
        out[b] = static_cast<uint8_t>(((lo + 8) & 0xF) | (((hi + 8) & 0xF) << 4));
    }
}

hipError_t launch_quantize(int fmt, const uint16_t* w, int N, int K, void* q, void* scales, bool tiled,
                           hipStream_t s) {
    if (N <= 0 || K <= 0) return hipSuccess;
    if (fmt == W_INT8) {
        hipLaunchKernelGGL(quant_int8_kernel, dim3((N + 3) / 4), dim3(256), 0, s, w, N, K,
                           static_cast<int8_t*>(q), static_cast<float*>(scales));
    } else {
        const int64_t groups = static_cast<int64_t>(N) * (K / 64);
        hipLaunchKernelGGL(quant_int4_kernel, dim3(static_cast<uint32_t>((groups + 255) / 256)),
                           dim3(256), 0, s, w, N, K, static_cast<uint8_t*>(q),
                           static_cast<uint16_t*>(scales), tiled ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace moe
