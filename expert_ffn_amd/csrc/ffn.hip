// Expert FFN kernels (prain README, "Expert formats": an expert is its w13 --
// gate and up projections stacked -- and its w2 down projection; int8 and int4
// weights are dequantised inside the kernel, w8a16 / w4a16).
//
// Both halves are grouped GEMMs on bf16 MFMA (v_mfma_f32_16x16x32_bf16):
//   A operand = 16 weight rows x 32 K, read from the packed blob and expanded
//               to bf16 in registers;
//   B operand = 32 K x 16 routes of one expert (bf16 activations);
//   D         = 16 rows x 16 routes, fp32.
// Lane l holds A row (l & 15) and B/D column (l & 15); lane group q = l >> 4
// holds the K slots 8q..8q+7 of A and B and the D rows 4q..4q+3.  Only the
// pairing of A and B slots matters, so each format picks the slot -> K map
// that expands cheapest:
//   int4: a dword of 8 nibbles (elements K..K+7, low nibble first) becomes four
//         bf16 pairs (d >> 4s) & 0x000F000F | 0x43004300 = 128 + (q + 8), i.e.
//         elements {0,4}, {1,5}, {2,6}, {3,7}; activations are stored in that
//         slot order.  The +136 bias is removed by one MFMA with a constant
//         A = -136 (shared by every row tile), the bf16 group scale is applied
//         to each group's fp32 partial sum.
//   int8: bytes ^ 0x80 = q + 128 -> fp32 -> bf16 (exact); bias removed by a
//         constant A = -128 MFMA; the fp32 row scale is applied at the end.
//   bf16: the weights are the operand.
// Lane group q covers K = 64 s + 16 q .. +15 of step s for int4/int8 (so a row's
// 64-element group is one step), K = 32 s + 8 q .. +7 for bf16.
//
// Streaming kernels (small groups, decode): one wavefront per 16-row tile and
// K range, no LDS for operands; the first half splits K over the workgroup's
// waves and reduces the partial sums in LDS.  Expert groups with no routes
// leave their workgroups idle at once.
#include "common.h"
#include "kernels.h"

namespace moe {

// slot j of an int4 operand dword holds element perm8(j): 0,4,1,5,2,6,3,7
__device__ __forceinline__ int perm8(int j) { return (j >> 1) | ((j & 1) << 2); }

template <int FMT> struct Geo;
template <> struct Geo<W_INT4> { static constexpr int KSTEP = 64, MF = 2; using A = u32x2; };
template <> struct Geo<W_INT8> { static constexpr int KSTEP = 64, MF = 2; using A = u32x4; };
template <> struct Geo<W_BF16> { static constexpr int KSTEP = 32, MF = 1; using A = u32x4; };

// bytes of one weight row of K elements
template <int FMT> __host__ __device__ __forceinline__ int64_t row_bytes(int K) {
    return FMT == W_INT4 ? K / 2 : (FMT == W_INT8 ? K : 2 * K);
}
// byte offset of lane group q's A fragment of step s inside a row
template <int FMT> __device__ __forceinline__ int a_off(int s, int q) {
    return FMT == W_INT4 ? s * 32 + q * 8 : (FMT == W_INT8 ? s * 64 + q * 16 : (s * 32 + q * 8) * 2);
}
// element offset of lane group q's B fragment of step s inside an activation row
template <int FMT> __device__ __forceinline__ int b_off(int s, int q) {
    return FMT == W_BF16 ? s * 32 + q * 8 : s * 64 + q * 16;
}

__device__ __forceinline__ u32x4 deq_int4(uint32_t d) {
    u32x4 r;
    r[0] = (d & 0x000F000Fu) | 0x43004300u;
    r[1] = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
    r[2] = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
    r[3] = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
    return r;
}

__device__ __forceinline__ u32x4 deq_int8(uint32_t d0, uint32_t d1) {
    d0 ^= 0x80808080u;
    d1 ^= 0x80808080u;
    u32x4 r;
    r[0] = pack_bf16x2(static_cast<float>(d0 & 0xFFu), static_cast<float>((d0 >> 8) & 0xFFu));
    r[1] = pack_bf16x2(static_cast<float>((d0 >> 16) & 0xFFu), static_cast<float>(d0 >> 24));
    r[2] = pack_bf16x2(static_cast<float>(d1 & 0xFFu), static_cast<float>((d1 >> 8) & 0xFFu));
    r[3] = pack_bf16x2(static_cast<float>((d1 >> 16) & 0xFFu), static_cast<float>(d1 >> 24));
    return r;
}

__device__ __forceinline__ u32x4 splat(uint32_t v) { return u32x4{v, v, v, v}; }

// ----------------------------------------------------------- preparation --
// xq[t][8b + j] = bf16(x[t][8b + perm(j)]), perm = perm8 for int4 w13, identity
// otherwise.  One thread per 8 elements.
template <int XT, bool PERM>
__global__ __launch_bounds__(256) void prep_x_kernel(const void* __restrict__ x, int64_t nblk,
                                                     uint16_t* __restrict__ xq) {
    const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (b >= nblk) return;
    float v[8];
    if (XT == F32) {
        const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + b * 8);
        const f32x4 a = src[0], c = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = c[j];
        }
    } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + b * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(a[j] << 16);
            v[2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
        }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i0 = PERM ? perm8(2 * j) : 2 * j, i1 = PERM ? perm8(2 * j + 1) : 2 * j + 1;
        o[j] = static_cast<uint32_t>(f32_to_bf16(v[i0])) | (static_cast<uint32_t>(f32_to_bf16(v[i1])) << 16);
    }
    *reinterpret_cast<u32x4*>(xq + b * 8) = o;
}

// ------------------------------------------------- gate/up (first half) --
// Workgroup = KSPLIT waves on one (expert, 16-row tile of FF); wave w covers
// steps [w*spw, (w+1)*spw) of K = H for the gate rows n0.. and the up rows
// FF+n0.. of that tile.  For int4 w2 the tile's rows are taken in the order
// (i & 8) | perm8(i & 7), so that the four h values a lane ends with are four
// consecutive entries of h in the w2 operand order.
template <int FMT, int KSPLIT, int NGC>
__global__ __launch_bounds__(64 * KSPLIT) void gate_up_stream_kernel(FfnParams P) {
    using G = Geo<FMT>;
    using AF = typename G::A;
    constexpr bool PERM_H = (FMT == W_INT4);
    extern __shared__ float smem[];
    const int ntile = P.FF >> 4;
    const int e = blockIdx.x / ntile, tile = blockIdx.x - e * ntile;
    const int beg = P.offsets[e], end = P.offsets[e + 1];
    if (beg >= end) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
    const int n0 = tile << 4;
    const int rho = PERM_H ? ((r & 8) | perm8(r & 7)) : r;
    const int64_t rs = row_bytes<FMT>(P.H);
    const uint8_t* ag_row = blob + P.o13 + static_cast<int64_t>(n0 + rho) * rs;
    const uint8_t* au_row = blob + P.o13 + static_cast<int64_t>(P.FF + n0 + rho) * rs;
    const int nsteps = P.H / G::KSTEP, spw = nsteps / KSPLIT, s0 = wave * spw;

    float* s_sc = smem + wave * (2 * spw * 16);               // int4: [2][spw][16]
    float* s_red = smem + (FMT == W_INT4 ? KSPLIT * 2 * spw * 16 : 0);  // [KSPLIT-1][8][64]
    f32x4 sg_row = {0, 0, 0, 0}, su_row = {0, 0, 0, 0};
    if (FMT == W_INT4) {
        const int Gr = P.H / 64;
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + P.os13);
        for (int idx = lane; idx < 32 * spw; idx += 64) {
            const int tl = idx / (16 * spw), rem = idx - tl * 16 * spw;
            const int i = rem / spw, gg = rem - i * spw;
            const int row = tl * P.FF + n0 + ((i & 8) | perm8(i & 7));
            s_sc[(tl * spw + gg) * 16 + i] = bf16_to_f32(sc[static_cast<int64_t>(row) * Gr + s0 + gg]);
        }
    } else if (FMT == W_INT8) {
        const float* sc = reinterpret_cast<const float*>(blob + P.os13);
        sg_row = *reinterpret_cast<const f32x4*>(sc + n0 + 4 * q);
        su_row = *reinterpret_cast<const f32x4*>(sc + P.FF + n0 + 4 * q);
    }
    __syncthreads();

    const f32x4 zero = {0, 0, 0, 0};
    const u32x4 kbias = splat(FMT == W_INT4 ? 0xC308C308u : 0xC300C300u);  // bf16 -136 / -128
    for (int c0 = beg; c0 < end; c0 += 16) {
        const int p = c0 + r;
        const bool valid = p < end;
        const int tok = valid ? P.sorted_route[p] / P.k : 0;
        const uint16_t* xrow = P.xq + static_cast<int64_t>(tok) * P.H;
        f32x4 accg = zero, accu = zero, cc = zero;
        for (int sc0 = 0; sc0 < spw; sc0 += NGC) {
            AF ag[NGC], au[NGC];
            u32x4 b[NGC][G::MF];
#pragma unroll
            for (int j = 0; j < NGC; ++j) {
                if (sc0 + j < spw) {
                    const int s = s0 + sc0 + j;
                    ag[j] = *reinterpret_cast<const AF*>(ag_row + a_off<FMT>(s, q));
                    au[j] = *reinterpret_cast<const AF*>(au_row + a_off<FMT>(s, q));
#pragma unroll
                    for (int m = 0; m < G::MF; ++m)
                        b[j][m] = valid ? *reinterpret_cast<const u32x4*>(xrow + b_off<FMT>(s, q) + 8 * m)
                                        : splat(0u);
                }
            }
#pragma unroll
            for (int j = 0; j < NGC; ++j) {
                if (sc0 + j < spw) {
                    if constexpr (FMT == W_INT4) {
                        f32x4 c = mfma16x16x32(kbias, b[j][0], zero);
                        c = mfma16x16x32(kbias, b[j][1], c);
                        f32x4 t = mfma16x16x32(deq_int4(ag[j][0]), b[j][0], c);
                        t = mfma16x16x32(deq_int4(ag[j][1]), b[j][1], t);
                        const f32x4 sg = *reinterpret_cast<const f32x4*>(s_sc + (sc0 + j) * 16 + 4 * q);
                        accg += sg * t;
                        t = mfma16x16x32(deq_int4(au[j][0]), b[j][0], c);
                        t = mfma16x16x32(deq_int4(au[j][1]), b[j][1], t);
                        const f32x4 su = *reinterpret_cast<const f32x4*>(s_sc + (spw + sc0 + j) * 16 + 4 * q);
                        accu += su * t;
                    } else if constexpr (FMT == W_INT8) {
                        cc = mfma16x16x32(kbias, b[j][0], cc);
                        cc = mfma16x16x32(kbias, b[j][1], cc);
                        accg = mfma16x16x32(deq_int8(ag[j][0], ag[j][1]), b[j][0], accg);
                        accg = mfma16x16x32(deq_int8(ag[j][2], ag[j][3]), b[j][1], accg);
                        accu = mfma16x16x32(deq_int8(au[j][0], au[j][1]), b[j][0], accu);
                        accu = mfma16x16x32(deq_int8(au[j][2], au[j][3]), b[j][1], accu);
                    } else {
                        accg = mfma16x16x32(ag[j], b[j][0], accg);
                        accu = mfma16x16x32(au[j], b[j][0], accu);
                    }
                }
            }
        }
        if (FMT == W_INT8) {
            accg = sg_row * (accg + cc);
            accu = su_row * (accu + cc);
        }
        if constexpr (KSPLIT > 1) {
            if (wave > 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s_red[((wave - 1) * 8 + j) * 64 + lane] = accg[j];
                    s_red[((wave - 1) * 8 + 4 + j) * 64 + lane] = accu[j];
                }
            }
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int w = 1; w < KSPLIT; ++w)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        accg[j] += s_red[((w - 1) * 8 + j) * 64 + lane];
                        accu[j] += s_red[((w - 1) * 8 + 4 + j) * 64 + lane];
                    }
            }
            __syncthreads();
        }
        if (wave == 0 && valid) {
            const uint32_t h0 = pack_bf16x2(act_fn(P.act, accg[0]) * accu[0], act_fn(P.act, accg[1]) * accu[1]);
            const uint32_t h1 = pack_bf16x2(act_fn(P.act, accg[2]) * accu[2], act_fn(P.act, accg[3]) * accu[3]);
            *reinterpret_cast<u32x2*>(P.h + static_cast<int64_t>(p) * P.FF + n0 + 4 * q) = u32x2{h0, h1};
        }
    }
}

// ----------------------------------------------------- down (second half) --
// Workgroup = 4 waves on one (expert, 64 rows of H); wave w owns 16 rows and
// the whole K = FF.  B rows are the h rows of the expert's route positions.
template <int FMT, int NGC>
__global__ __launch_bounds__(256) void down_stream_kernel(FfnParams P) {
    using G = Geo<FMT>;
    using AF = typename G::A;
    extern __shared__ float smem[];
    const int nblk = P.H >> 6;
    const int e = blockIdx.x / nblk, blk = blockIdx.x - e * nblk;
    const int beg = P.offsets[e], end = P.offsets[e + 1];
    if (beg >= end) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
    const int m0 = blk * 64 + wave * 16;
    const uint8_t* a_row = blob + P.o2 + static_cast<int64_t>(m0 + r) * row_bytes<FMT>(P.FF);
    const int nsteps = P.FF / G::KSTEP;

    float* s_sc = smem + wave * (nsteps * 16);  // int4: [nsteps][16]
    f32x4 s_row = {0, 0, 0, 0};
    if (FMT == W_INT4) {
        const int Gr = P.FF / 64;
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + P.os2);
        for (int idx = lane; idx < 16 * nsteps; idx += 64) {
            const int i = idx / nsteps, gg = idx - i * nsteps;
            s_sc[gg * 16 + i] = bf16_to_f32(sc[static_cast<int64_t>(m0 + i) * Gr + gg]);
        }
    } else if (FMT == W_INT8) {
        s_row = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(blob + P.os2) + m0 + 4 * q);
    }
    __syncthreads();

    const f32x4 zero = {0, 0, 0, 0};
    const u32x4 kbias = splat(FMT == W_INT4 ? 0xC308C308u : 0xC300C300u);
    for (int c0 = beg; c0 < end; c0 += 16) {
        const int p = c0 + r;
        const bool valid = p < end;
        const uint16_t* hrow = P.h + static_cast<int64_t>(valid ? p : beg) * P.FF;
        f32x4 acc = zero, cc = zero;
        for (int sc0 = 0; sc0 < nsteps; sc0 += NGC) {
            AF a[NGC];
            u32x4 b[NGC][G::MF];
#pragma unroll
            for (int j = 0; j < NGC; ++j) {
                if (sc0 + j < nsteps) {
                    const int s = sc0 + j;
                    a[j] = *reinterpret_cast<const AF*>(a_row + a_off<FMT>(s, q));
#pragma unroll
                    for (int m = 0; m < G::MF; ++m)
                        b[j][m] = valid ? *reinterpret_cast<const u32x4*>(hrow + b_off<FMT>(s, q) + 8 * m)
                                        : splat(0u);
                }
            }
#pragma unroll
            for (int j = 0; j < NGC; ++j) {
                if (sc0 + j < nsteps) {
                    if constexpr (FMT == W_INT4) {
                        f32x4 t = mfma16x16x32(kbias, b[j][0], zero);
                        t = mfma16x16x32(kbias, b[j][1], t);
                        t = mfma16x16x32(deq_int4(a[j][0]), b[j][0], t);
                        t = mfma16x16x32(deq_int4(a[j][1]), b[j][1], t);
                        const f32x4 s = *reinterpret_cast<const f32x4*>(s_sc + (sc0 + j) * 16 + 4 * q);
                        acc += s * t;
                    } else if constexpr (FMT == W_INT8) {
                        cc = mfma16x16x32(kbias, b[j][0], cc);
                        cc = mfma16x16x32(kbias, b[j][1], cc);
                        acc = mfma16x16x32(deq_int8(a[j][0], a[j][1]), b[j][0], acc);
                        acc = mfma16x16x32(deq_int8(a[j][2], a[j][3]), b[j][1], acc);
                    } else {
                        acc = mfma16x16x32(a[j], b[j][0], acc);
                    }
                }
            }
        }
        if (FMT == W_INT8) acc = s_row * (acc + cc);
        if (valid) {
            const int64_t o = static_cast<int64_t>(p) * P.H + m0 + 4 * q;
            if (P.out_dt == F32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(P.out) + o) = acc;
            } else {
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.out) + o) =
                    u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            }
        }
    }
}

// ------------------------------------------------------------------ host --
FfnWorkspace ffn_workspace(int T, int k, int H, int FF) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    FfnWorkspace w;
    w.xq_off = 0;
    w.h_off = up(static_cast<size_t>(T) * H * 2);
    w.bytes = w.h_off + up(static_cast<size_t>(T) * k * FF * 2);
    return w;
}

template <int FMT, int KSPLIT>
static void launch_gate_up_stream(const FfnParams& P, hipStream_t s) {
    constexpr int KSTEP = Geo<FMT>::KSTEP;
    const int spw = P.H / KSTEP / KSPLIT;
    size_t smem = (KSPLIT - 1) * 8 * 64 * sizeof(float);
    if (FMT == W_INT4) smem += static_cast<size_t>(KSPLIT) * 2 * spw * 16 * sizeof(float);
    const dim3 grid(P.E * (P.FF / 16)), block(64 * KSPLIT);
    hipLaunchKernelGGL((gate_up_stream_kernel<FMT, KSPLIT, 4>), grid, block, smem, s, P);
}

template <int FMT>
static void launch_phases(const FfnParams& P, int phases, hipStream_t s) {
    constexpr int KSTEP = Geo<FMT>::KSTEP;
    if (phases & 1) {
        const int nsteps = P.H / KSTEP;
        if (nsteps % 4 == 0)
            launch_gate_up_stream<FMT, 4>(P, s);
        else if (nsteps % 2 == 0)
            launch_gate_up_stream<FMT, 2>(P, s);
        else
            launch_gate_up_stream<FMT, 1>(P, s);
    }
    if (phases & 2) {
        const int nsteps = P.FF / KSTEP;
        const size_t smem = FMT == W_INT4 ? 4 * static_cast<size_t>(nsteps) * 16 * sizeof(float) : 0;
        hipLaunchKernelGGL((down_stream_kernel<FMT, 4>), dim3(P.E * (P.H / 64)), dim3(256), smem, s, P);
    }
}

hipError_t launch_ffn(const FfnParams& P0, int phases, int path, hipStream_t s) {
    (void)path;
    FfnParams P = P0;
    if (phases & 1) {
        const bool perm = (P.fmt == W_INT4);
        if (perm || P.x_dt == F32) {
            const int64_t nblk = static_cast<int64_t>(P.T) * P.H / 8;
            const dim3 grid(static_cast<uint32_t>((nblk + 255) / 256)), block(256);
            if (P.x_dt == F32 && perm)
                hipLaunchKernelGGL((prep_x_kernel<F32, true>), grid, block, 0, s, P.x, nblk, P.xq_out);
            else if (P.x_dt == F32)
                hipLaunchKernelGGL((prep_x_kernel<F32, false>), grid, block, 0, s, P.x, nblk, P.xq_out);
            else
                hipLaunchKernelGGL((prep_x_kernel<BF16, true>), grid, block, 0, s, P.x, nblk, P.xq_out);
            P.xq = P.xq_out;
        } else {
            P.xq = static_cast<const uint16_t*>(P.x);
        }
    }
    if (P.fmt == W_INT4)
        launch_phases<W_INT4>(P, phases, s);
    else if (P.fmt == W_INT8)
        launch_phases<W_INT8>(P, phases, s);
    else
        launch_phases<W_BF16>(P, phases, s);
    return hipGetLastError();
}

}  // namespace moe
