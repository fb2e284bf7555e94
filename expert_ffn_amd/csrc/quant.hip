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

// Canonical expert -> slot (prain README, "int4 experts on RDNA2": one unpack
// kernel per expert copy): one pass over the blob in 16-byte chunks.  A chunk
// of an int4 nibble block (rows of K / 2 bytes, a multiple of 32, so a chunk
// never crosses a row or a 64-group) moves to its place in the 32-row tiles;
// every other chunk (scales, padding, bf16 and int8 weights) keeps its offset.
struct SlotMap {
    uint32_t nchunks;     // blob bytes / 16
    uint32_t o13, e13;    // w13 nibble block [o13, e13) (empty unless int4)
    uint32_t rb13;        // its row bytes (H / 2)
    uint32_t o2, e2, rb2; // the same for w2 (row bytes FF / 2)
};

__device__ __forceinline__ uint32_t slot_chunk(const SlotMap& m, uint32_t i) {
    const uint32_t b = i * 16;
    if (b >= m.o13 && b < m.e13) {
        const uint32_t r = b - m.o13, n = r / m.rb13;
        return (m.o13 + static_cast<uint32_t>(int4_code_off(n, m.rb13 / 32, r - n * m.rb13))) / 16;
    }
    if (b >= m.o2 && b < m.e2) {
        const uint32_t r = b - m.o2, n = r / m.rb2;
        return (m.o2 + static_cast<uint32_t>(int4_code_off(n, m.rb2 / 32, r - n * m.rb2))) / 16;
    }
    return i;
}

// HOST_SRC: src is the device mapping of pinned host memory (same code; a
// separate instance so that traces tell the bus-bound fills apart)
template <bool HOST_SRC>
__global__ __launch_bounds__(256) void fill_slot_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        SlotMap m) {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i < m.nchunks) dst[slot_chunk(m, i)] = src[i];
}

// several experts at once: blockIdx.y picks the expert, its canonical blob at
// src + y * blob bytes and its slot at dst.p[y]
struct SlotPtrs {
    u32x4* p[FILL_MAX];
};

__global__ __launch_bounds__(256) void fill_slots_kernel(const u32x4* __restrict__ src, SlotPtrs dst, SlotMap m) {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i < m.nchunks) dst.p[blockIdx.y][slot_chunk(m, i)] = src[static_cast<uint64_t>(blockIdx.y) * m.nchunks + i];
}

// count of 16-byte chunks of the slot that differ from the canonical blob
__global__ __launch_bounds__(256) void verify_slot_kernel(const u32x4* __restrict__ src,
                                                          const u32x4* __restrict__ slot, SlotMap m,
                                                          int32_t* __restrict__ bad) {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    bool diff = false;
    if (i < m.nchunks) {
        const u32x4 a = src[i], c = slot[slot_chunk(m, i)];
        diff = a[0] != c[0] || a[1] != c[1] || a[2] != c[2] || a[3] != c[3];
    }
    const uint64_t v = __ballot(diff);
    if (v && (threadIdx.x & 63) == 0) atomicAdd(bad, __popcll(v));
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

static SlotMap slot_map(int fmt, int H, int FF, const uint64_t* off) {
    SlotMap m{};
    m.nchunks = static_cast<uint32_t>(off[4] / 16);
    if (fmt == W_INT4) {
        m.o13 = static_cast<uint32_t>(off[0]);
        m.e13 = m.o13 + static_cast<uint32_t>(FF) * H;   // 2FF rows of H / 2 bytes
        m.rb13 = H / 2;
        m.o2 = static_cast<uint32_t>(off[2]);
        m.e2 = m.o2 + static_cast<uint32_t>(H) * (FF / 2);
        m.rb2 = FF / 2;
    } else {
        m.rb13 = m.rb2 = 32;
    }
    return m;
}

hipError_t launch_fill_slot(int fmt, const void* src, bool host_src, int H, int FF, const uint64_t* off, void* slot,
                            hipStream_t s) {
    const SlotMap m = slot_map(fmt, H, FF, off);
    hipLaunchKernelGGL(host_src ? fill_slot_kernel<true> : fill_slot_kernel<false>, dim3((m.nchunks + 255) / 256),
                       dim3(256), 0, s, static_cast<const u32x4*>(src), static_cast<u32x4*>(slot), m);
    return hipGetLastError();
}

hipError_t launch_fill_slots(int fmt, const void* src, int n, int H, int FF, const uint64_t* off, void* const* slots,
                             hipStream_t s) {
    const SlotMap m = slot_map(fmt, H, FF, off);
    SlotPtrs d{};
    for (int j = 0; j < n; ++j) d.p[j] = static_cast<u32x4*>(slots[j]);
    hipLaunchKernelGGL(fill_slots_kernel, dim3((m.nchunks + 255) / 256, n), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), d, m);
    return hipGetLastError();
}

hipError_t launch_verify_slot(int fmt, const void* src, int H, int FF, const uint64_t* off, const void* slot,
                              int32_t* mismatches, hipStream_t s) {
    const SlotMap m = slot_map(fmt, H, FF, off);
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, mismatches);
    hipLaunchKernelGGL(verify_slot_kernel, dim3((m.nchunks + 255) / 256), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), static_cast<const u32x4*>(slot), m, mismatches);
    return hipGetLastError();
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
