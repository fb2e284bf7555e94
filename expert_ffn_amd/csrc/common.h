// Internal helpers shared by the HIP kernels of the routed expert FFN (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// format / dtype / activation codes (same values as the public enums)
enum { F32 = 0, BF16 = 1 };
enum { W_BF16 = 0, W_INT8 = 1, W_INT4 = 2 };
enum { ACT_GELU_TANH = 0, ACT_SILU = 1 };

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// bf16 <-> fp32 on bit patterns.  Narrowing is round to nearest, ties to even;
// NaN becomes the quiet NaN 0x7FC0.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
// two fp32 -> packed bf16x2 (RNE) with the gfx950 conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Raw buffer loads: a lane whose byte offset is at or past num_records reads
// zeros without touching memory, so lanes without work pass NO_LANE.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t NO_LANE = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// with a wave-uniform byte offset in an SGPR (soff) added to the lane's
__device__ __forceinline__ u32x4 bload16s(rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ uint32_t bload_u16(rsrc_t r, uint32_t off, uint32_t soff) {
    return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0));
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Gated activations.  GELU (tanh form) uses 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)):
//   gelu(g) = g / (1 + exp(-2 sqrt(2/pi) (g + 0.044715 g^3)));  silu(g) = g / (1 + exp(-g)).
// One exponential and one hardware reciprocal (v_rcp_f32, 1 ulp); both limits are
// exact (exp overflow gives 0: the reciprocal of +inf is 0).
__device__ __forceinline__ float act_fn(int act, float g) {
    const float z = act == ACT_SILU ? -g : -1.5957691216057308f * (g + 0.044715f * g * g * g);
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(z));
}

// int4 codes of a matrix [N rows][K] inside an expert blob: 32-row blocks,
// and inside a block one [32 rows][32 bytes] piece per 64-element group, so
// that one group of 32 consecutive rows is 1 KB of contiguous memory.  Offset
// of byte kb (of the row's K/2 bytes, element 2 kb in the low nibble) of row n,
// G = K / 64; N is a multiple of 32.
__host__ __device__ __forceinline__ int64_t int4_code_off(int n, int G, int kb) {
    return ((static_cast<int64_t>(n >> 5) * G + (kb >> 5)) << 10) + ((n & 31) << 5) + (kb & 31);
}

// slot j of an int4 operand dword holds element perm8(j): 0,4,1,5,2,6,3,7
__device__ __forceinline__ int perm8(int j) { return (j >> 1) | ((j & 1) << 2); }

// int4 codes -> bf16 (128 + u): (d >> 4j) & 0x000F000F | 0x43004300.  The
// constants pass through empty asm statements so that they stay in registers:
// a literal cannot be a VOP3 operand here, and with one the compiler splits
// each dword into v_and + v_or.  With the mask in an SGPR and the magic in a
// VGPR it emits one v_and_or_b32 per dword and tracks the VALU -> MFMA operand
// hazards itself (it does not for VGPRs written by inline asm instructions).
// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory
// operations of the wave are outstanding, leaving the LDS/scalar and export
// counters unwaited: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
__host__ __device__ constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
static_assert(waitcnt_vm(8) == 0x0F78 && waitcnt_vm(0) == 0x0F70 && waitcnt_vm(24) == 0x4F78, "s_waitcnt encoding");

__device__ __forceinline__ u32x4 deq_int4(uint32_t d) {
    uint32_t M = 0x000F000Fu, C = 0x43004300u;
    asm("" : "+s"(M));
    asm("" : "+v"(C));
    u32x4 r;
    r[0] = (d & M) | C;
    r[1] = ((d >> 4) & M) | C;
    r[2] = ((d >> 8) & M) | C;
    r[3] = ((d >> 12) & M) | C;
    return r;
}

}  // namespace moe
