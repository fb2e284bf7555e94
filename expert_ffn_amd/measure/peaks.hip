// Measurement kernels for the benchmark (not part of the expert FFN path):
// the achieved peaks that the roofline fractions are also quoted against, and
// the load pattern of the decode gate/up kernel without its compute.
//
//   peak_stream_read   plain streaming read of a large buffer: each thread
//                      keeps UNR 16-byte loads in flight, grid-stride
//   peak_tile_loads    the decode gate/up kernel's weight loads only: one
//                      workgroup of 4 waves per (expert, 16-row tile of the
//                      gate/up rows), each wave requesting its 11 fragments of
//                      16 bytes per lane (one K half of the 16 rows) from the
//                      tiled int4 codes of an expert blob in the slot pool;
//                      experts without routes leave at once
//   peak_mfma_bf16     back-to-back v_mfma_f32_32x32x16_bf16 on CH independent
//                      accumulator chains per wave
// Each kernel folds what it reads into a value that is stored only when it
// equals an unlikely constant, so no load is removed and nearly nothing is
// written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr uint32_t MAGIC = 0x9E3779B9u;

template <int UNR>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                          uint32_t* __restrict__ sink) {
    const uint64_t nth = static_cast<uint64_t>(gridDim.x) * 256;
    const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    u32x4 acc = {0, 0, 0, 0};
    uint64_t i = tid;
    for (; i + (UNR - 1) * nth < n16; i += UNR * nth) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) v[u] = src[i + u * nth];
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= v[u];
    }
    for (; i < n16; i += nth) acc ^= src[i];
    const uint32_t h = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (h == MAGIC) sink[tid & 1023] = h;
}

// rows: gate rows t*FF + 16u .. +15 (t = wave / 2), K half (wave % 2) of H;
// the int4 code block is tiled [N/32][H/64][32 rows][32 bytes]
__global__ __launch_bounds__(256) void tile_loads_kernel(const uint8_t* __restrict__ pool, uint64_t slot_bytes,
                                                         const int* __restrict__ slot_of,
                                                         const int* __restrict__ offsets, int H, int FF,
                                                         uint32_t* __restrict__ sink) {
    const int ntile = FF / 16;
    const int e = blockIdx.y, u = blockIdx.x;
    if (offsets[e] >= offsets[e + 1]) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const int t = wave >> 1, part = wave & 1;
    const int G = H / 64;
    const int row = t * FF + 16 * u + r;
    const int kb = part * (H / 4) + 16 * q;   // byte of the row: K half, lane group
    const uint8_t* a = pool + static_cast<uint64_t>(slot_of[e]) * slot_bytes +
                       ((static_cast<int64_t>(row >> 5) * G + (kb >> 5)) << 10) + ((row & 31) << 5) + (kb & 31);
    constexpr int NF = 11;
    u32x4 v[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) v[i] = *reinterpret_cast<const u32x4*>(a + 2048 * i);
    u32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NF; ++i) acc ^= v[i];
    const uint32_t h = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (h == MAGIC) sink[(blockIdx.y * ntile + blockIdx.x) & 1023] = h;
}

template <int CH>
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, uint32_t seed, float* __restrict__ sink) {
    const uint32_t s = seed ^ threadIdx.x;
    const u32x4 av = {s, s * 3u, s * 5u, s * 7u}, bv = {s * 11u, s * 13u, s * 17u, s * 19u};
    const bf16x8 a = __builtin_bit_cast(bf16x8, av & u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    const bf16x8 b = __builtin_bit_cast(bf16x8, bv & u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    f32x16 acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) sum += acc[c][j];
    if (sum == 1.2345678f) sink[threadIdx.x] = sum;
}

}  // namespace

extern "C" {

// every function enqueues one launch on stream and returns hipGetLastError()
int peak_stream_read(const void* src, uint64_t bytes, int blocks, uint32_t* sink, void* stream) {
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    return static_cast<int>(hipGetLastError());
}

int peak_tile_loads(const void* pool, uint64_t slot_bytes, const int* slot_of, const int* offsets, int E, int H,
                    int FF, uint32_t* sink, void* stream) {
    if (H != 2816 || FF % 16) return static_cast<int>(hipErrorInvalidValue);   // 11 fragments per wave: H = 2816
    hipLaunchKernelGGL(tile_loads_kernel, dim3(FF / 16, E), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(pool), slot_bytes, slot_of, offsets, H, FF, sink);
    return static_cast<int>(hipGetLastError());
}

// flops per launch: blocks * 4 waves * iters * 4 chains * 32768
int peak_mfma_bf16(int blocks, int iters, float* sink, void* stream) {
    hipLaunchKernelGGL(mfma_bf16_kernel<4>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       0x1234u, sink);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
