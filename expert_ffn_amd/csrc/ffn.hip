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
// K range, the weights in registers; the first half splits K over the
// workgroup's waves and reduces the partial sums in LDS.  Activations reach
// the MFMAs through LDS where they fit (the h rows of down's 16-route tile,
// the x rows of a gate/up tile of at most 4 routes), copied there before the
// weights are requested, so that no activation load issued after the weights
// waits for them in the in-order vector-memory counter.  Expert groups with
// no routes leave their workgroups idle at once.
#include <climits>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

template <int FMT> struct Geo;
template <> struct Geo<W_INT8> { static constexpr int KSTEP = 64, MF = 2; using A = u32x4; };
template <> struct Geo<W_BF16> { static constexpr int KSTEP = 32, MF = 1; using A = u32x4; };

// bytes of one weight row of K elements
template <int FMT> __host__ __device__ __forceinline__ int64_t row_bytes(int K) {
    return FMT == W_INT8 ? K : 2 * K;
}
// byte offset of lane group q's A fragment of step s inside a row
template <int FMT> __device__ __forceinline__ int a_off(int s, int q) {
    return FMT == W_INT8 ? s * 64 + q * 16 : (s * 32 + q * 8) * 2;
}
// element offset of lane group q's B fragment of step s inside an activation row
template <int FMT> __device__ __forceinline__ int b_off(int s, int q) {
    return FMT == W_BF16 ? s * 32 + q * 8 : s * 64 + q * 16;
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
// FF+n0.. of that tile (bf16 and int8 weights; int4 has kernels of its own).
template <int FMT, int KSPLIT, int NGC>
__global__ __launch_bounds__(64 * KSPLIT) void gate_up_generic_kernel(FfnParams P) {
    using G = Geo<FMT>;
    using AF = typename G::A;
    extern __shared__ float smem[];
    const int ntile = P.FF >> 4;
    const int e = blockIdx.x / ntile, tile = blockIdx.x - e * ntile;
    const int beg = P.offsets[e], end = P.offsets[e + 1];
    if (beg >= end) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
    const int n0 = tile << 4;
    const int64_t rs = row_bytes<FMT>(P.H);
    const uint8_t* ag_row = blob + P.o13 + static_cast<int64_t>(n0 + r) * rs;
    const uint8_t* au_row = blob + P.o13 + static_cast<int64_t>(P.FF + n0 + r) * rs;
    const int nsteps = P.H / G::KSTEP, spw = nsteps / KSPLIT, s0 = wave * spw;

    float* s_red = smem;   // [KSPLIT-1][8][64]
    f32x4 sg_row = {0, 0, 0, 0}, su_row = {0, 0, 0, 0};
    if (FMT == W_INT8) {
        const float* sc = reinterpret_cast<const float*>(blob + P.os13);
        sg_row = *reinterpret_cast<const f32x4*>(sc + n0 + 4 * q);
        su_row = *reinterpret_cast<const f32x4*>(sc + P.FF + n0 + 4 * q);
    }
    __syncthreads();

    const f32x4 zero = {0, 0, 0, 0};
    const u32x4 kbias = splat(0xC300C300u);  // bf16 -128
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
                    if constexpr (FMT == W_INT8) {
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
__global__ __launch_bounds__(256) void down_generic_kernel(FfnParams P) {
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

    f32x4 s_row = {0, 0, 0, 0};
    if (FMT == W_INT8)
        s_row = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(blob + P.os2) + m0 + 4 * q);

    const f32x4 zero = {0, 0, 0, 0};
    const u32x4 kbias = splat(0xC300C300u);   // bf16 -128
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
                    if constexpr (FMT == W_INT8) {
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

// ------------------------------------------------- streaming, prefetched --
// The decode kernels (at most 64 tokens, so no expert has more than four
// tiles of 16 routes; blockIdx.y picks the tile).  A wavefront owns NG steps
// of K for its row tiles and issues every weight load of that range at once;
// the route index is loaded first so that the activation loads can follow, D
// steps ahead of the MFMAs.  Scale staging into LDS happens while the weight
// loads are in flight.  Lanes past the group's last route read the group's
// first route: their D columns are computed and never stored.

// one step of the gate/up MFMAs for both tiles
template <int FMT>
__device__ __forceinline__ void step_gu(const typename Geo<FMT>::A& ag, const typename Geo<FMT>::A& au,
                                        const u32x4* b, f32x4& accg, f32x4& accu, f32x4& cc) {
    if constexpr (FMT == W_INT8) {
        const u32x4 kb = splat(0xC300C300u);  // bf16 -128
        cc = mfma16x16x32(kb, b[0], cc);
        cc = mfma16x16x32(kb, b[1], cc);
        accg = mfma16x16x32(deq_int8(ag[0], ag[1]), b[0], accg);
        accg = mfma16x16x32(deq_int8(ag[2], ag[3]), b[1], accg);
        accu = mfma16x16x32(deq_int8(au[0], au[1]), b[0], accu);
        accu = mfma16x16x32(deq_int8(au[2], au[3]), b[1], accu);
    } else {
        accg = mfma16x16x32(ag, b[0], accg);
        accu = mfma16x16x32(au, b[0], accu);
    }
}

// A tile of at most SMALL_RT routes (the usual case in decode) copies its
// tokens' x rows into LDS by LDS DMA, issued before the weights, and the K
// loop takes its B fragments there; larger tiles read each lane's activation
// row from L2 D steps ahead of the MFMAs (16 rows of H would not fit in LDS).
constexpr int SMALL_RT = 4;
template <int FMT, int NG, int KSPLIT>
__host__ __device__ constexpr size_t gate_up_fast_lds() {
    return SMALL_RT * NG * KSPLIT * Geo<FMT>::KSTEP * 2 + (KSPLIT - 1) * 8 * 64 * sizeof(float);
}

template <int FMT, int NG, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) __attribute__((amdgpu_waves_per_eu(4)))
void gate_up_fast_kernel(FfnParams P) {
    using G = Geo<FMT>;
    using AF = typename G::A;
    constexpr int MF = G::MF;
    constexpr int D = NG < 3 ? NG : 3;             // activation prefetch depth (steps), larger tiles
    constexpr int HC = NG * KSPLIT * G::KSTEP;     // H of this instantiation
    constexpr int NCH = SMALL_RT * HC / 8;         // 16-byte chunks of SMALL_RT x rows
    constexpr int NCP = (NCH + 63) / 64;           // 1 KB LDS DMA copies of them
    constexpr int NCW = (NCP + KSPLIT - 1) / KSPLIT;   // per wave
    extern __shared__ float smem[];
    const int ntile = P.FF >> 4;
    const int e = blockIdx.x / ntile, tile = blockIdx.x - e * ntile;
    const int beg = P.offsets[e] + 16 * static_cast<int>(blockIdx.y), end = P.offsets[e + 1];
    if (beg >= end) return;
    // the wave index as a scalar: the LDS DMA destinations go through M0
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15,
              q = lane >> 4;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
    const int n0 = tile << 4;
    const int s0 = wave * NG;
    const int64_t rs = row_bytes<FMT>(HC);
    const uint8_t* ag_row = blob + P.o13 + static_cast<int64_t>(n0 + r) * rs;
    const uint8_t* au_row = ag_row + static_cast<int64_t>(P.FF) * rs;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                 // [SMALL_RT][HC] bf16
    float* s_red = reinterpret_cast<float*>(xs + SMALL_RT * HC);      // [KSPLIT-1][8][64]

    // The vector-memory counter retires loads in issue order, so the loads go
    // out in the order they are needed: the activations (they sit in L2 and
    // arrive long before the weights), then every weight fragment of the
    // wave's K range in the order of use, then the int8 row scales.
    // 1. the tile's 16 route indices by uniform (scalar) loads, read before
    //    any store; column r is route beg + r (columns past the group repeat
    //    the last route: computed from real data and never stored)
    const int p = beg + r;
    const bool valid = p < end;
    const int nr = min(end - beg, 16);
    const bool small = nr <= SMALL_RT;   // uniform
    int route, tk[SMALL_RT];
    {
        int rt[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) rt[i] = P.sorted_route[min(beg + i, end - 1)];
        route = rt[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) route = r == i ? rt[i] : route;
#pragma unroll
        for (int i = 0; i < SMALL_RT; ++i) tk[i] = route_token(rt[i], P.kmul, P.k);
    }
    // 2. activations (a small tile's x rows, else this lane's row D steps
    //    ahead of the MFMAs), 3. the weights, 4. int8 row scales, then the K
    //    loop.  The two cases are separate paths (the branch is uniform), so
    //    that the large tiles' staging registers are not live in the other.
    AF ag[NG], au[NG];
    f32x4 sg_row = {0, 0, 0, 0}, su_row = {0, 0, 0, 0};
    auto load_weights = [&]() {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            ag[g] = *reinterpret_cast<const AF*>(ag_row + a_off<FMT>(s0 + g, q));
            au[g] = *reinterpret_cast<const AF*>(au_row + a_off<FMT>(s0 + g, q));
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FMT == W_INT8) {
            const float* sc = reinterpret_cast<const float*>(blob + P.os13);
            sg_row = *reinterpret_cast<const f32x4*>(sc + n0 + 4 * q);
            su_row = *reinterpret_cast<const f32x4*>(sc + P.FF + n0 + 4 * q);
        }
    };
    const f32x4 zero = {0, 0, 0, 0};
    f32x4 accg = zero, accu = zero, cc = zero;
    if (small) {
        // copy b = i KSPLIT + wave: lane l takes 16-byte chunk 64 b + l of the
        // rows (row j at chunk j HC / 8; rows past nr are not read)
        const rsrc_t xres = make_rsrc(P.xq, static_cast<uint32_t>(P.T) * HC * 2);
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
            const int cp = i * KSPLIT + wave;
            if (NCP % KSPLIT == 0 || cp < NCP) {
                const int c = 64 * cp + lane, j = c / (HC / 8), col = c - j * (HC / 8);
                const int t = j == 0 ? tk[0] : (j == 1 ? tk[1] : (j == 2 ? tk[2] : tk[3]));
                const uint32_t off = (NCH % 64 == 0 || c < NCH) && j < nr ? static_cast<uint32_t>(t * HC + 8 * col) * 2 : NO_LANE;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xres, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(xs + 512 * cp)),
                    16, off, 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_weights();
        // the copies are this wave's oldest vector-memory operations: 2 NG
        // weight loads (and 2 scale loads for int8) follow them.  The compiler
        // does not track LDS DMA completion, so the wait is explicit.
        constexpr int NAFTER = 2 * NG + (FMT == W_INT8 ? 2 : 0);
        static_assert(NAFTER < 64, "vmcnt holds 6 bits");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NAFTER));
        __syncthreads();
        // fragments read one step ahead (fenced: the compiler would otherwise
        // read every step's at once and hold them in registers)
        const uint16_t* xl = xs + min(r, nr - 1) * HC;
        u32x4 bn[MF];
#pragma unroll
        for (int m = 0; m < MF; ++m) bn[m] = *reinterpret_cast<const u32x4*>(xl + b_off<FMT>(s0, q) + 8 * m);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            u32x4 bg[MF];
#pragma unroll
            for (int m = 0; m < MF; ++m) bg[m] = bn[m];
            if (g + 1 < NG) {
#pragma unroll
                for (int m = 0; m < MF; ++m) bn[m] = *reinterpret_cast<const u32x4*>(xl + b_off<FMT>(s0 + g + 1, q) + 8 * m);
            }
            step_gu<FMT>(ag[g], au[g], bg, accg, accu, cc);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        const uint16_t* xrow = P.xq + static_cast<int64_t>(route_token(route, P.kmul, P.k)) * HC;
        u32x4 b[D][MF];
#pragma unroll
        for (int g = 0; g < D; ++g)
#pragma unroll
            for (int m = 0; m < MF; ++m) b[g][m] = *reinterpret_cast<const u32x4*>(xrow + b_off<FMT>(s0 + g, q) + 8 * m);
        __builtin_amdgcn_sched_barrier(0);
        load_weights();
        __syncthreads();
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            step_gu<FMT>(ag[g], au[g], b[g % D], accg, accu, cc);
            if (g + D < NG) {
#pragma unroll
                for (int m = 0; m < MF; ++m)
                    b[g % D][m] = *reinterpret_cast<const u32x4*>(xrow + b_off<FMT>(s0 + g + D, q) + 8 * m);
            }
        }
    }
    if constexpr (FMT == W_INT8) {
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
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < KSPLIT; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                accg[j] += s_red[((w - 1) * 8 + j) * 64 + lane];
                accu[j] += s_red[((w - 1) * 8 + 4 + j) * 64 + lane];
            }
    }
    if (valid) {
        const uint32_t h0 = pack_bf16x2(act_fn(P.act, accg[0]) * accu[0], act_fn(P.act, accg[1]) * accu[1]);
        const uint32_t h1 = pack_bf16x2(act_fn(P.act, accg[2]) * accu[2], act_fn(P.act, accg[3]) * accu[3]);
        *reinterpret_cast<u32x2*>(P.h + static_cast<int64_t>(p) * P.FF + n0 + 4 * q) = u32x2{h0, h1};
    }
}

// Workgroup = 4 waves = (4 / KS) tiles of 16 rows of H x KS parts of K = FF,
// one tile of 16 routes (blockIdx.y).  With KS = 1 every wave multiplies the
// same 16 h rows over the whole FF, so the workgroup copies them (16 x FF
// bf16) into LDS once, with loads issued before the weights, and the K loop
// reads its B fragments there: no activation load waits behind the weights in
// the in-order vector-memory counter, and each h row is read from L2 once per
// workgroup, not per wave (int8: 21.7 -> 15.7 us per layer under Zipf routing
// at T = 16).  With K split (bf16) each lane reads its row from L2 D steps
// ahead of the MFMAs, which measured 1-3 % faster there.
template <int KS>
__host__ __device__ constexpr bool down_fast_stage() { return KS == 1; }
template <int FMT, int NG, int KS>
__host__ __device__ constexpr int down_fast_hs() { return NG * KS * Geo<FMT>::KSTEP + 8; }   // LDS row stride
template <int FMT, int NG, int KS>
__host__ __device__ constexpr size_t down_fast_lds() {
    return (down_fast_stage<KS>() ? 16 * down_fast_hs<FMT, NG, KS>() * 2 : 0) + (KS > 1 ? 3 * 4 * 64 * sizeof(float) : 0);
}

template <int FMT, int NG, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void down_fast_kernel(FfnParams P) {
    using G = Geo<FMT>;
    using AF = typename G::A;
    constexpr int MF = G::MF;
    constexpr int RTW = 4 / KS;
    constexpr int FFC = NG * KS * G::KSTEP;          // FF of this instantiation
    constexpr int HS = down_fast_hs<FMT, NG, KS>();  // row stride 16 bytes past a multiple of 128: rows on distinct banks
    constexpr bool STAGE = down_fast_stage<KS>();
    constexpr int NCH = 16 * FFC / 8;                // 16-byte chunks of the tile's h rows
    constexpr int NPT = STAGE ? (NCH + 255) / 256 : 1;
    constexpr int D = NG < 3 ? NG : 3;               // prefetch depth (steps) without staging
    extern __shared__ float smem[];
    const int nblk = P.H / (16 * RTW);
    const int e = blockIdx.x / nblk, blk = blockIdx.x - e * nblk;
    const int beg = P.offsets[e] + 16 * static_cast<int>(blockIdx.y), end = P.offsets[e + 1];
    if (beg >= end) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
    const int rt = wave / KS, kp = wave - rt * KS;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
    const int m0 = (blk * RTW + rt) * 16;
    const int s0 = kp * NG;
    const uint8_t* a_row = blob + P.o2 + static_cast<int64_t>(m0 + r) * row_bytes<FMT>(FFC);
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);                        // [16][HS] bf16 (staging)
    float* s_red = reinterpret_cast<float*>(hs + (STAGE ? 16 * HS : 0));     // [3][4][64] when K is split

    const int p = beg + r;
    const bool valid = p < end;
    // loads in the order of need: the tile's h rows (in L2; rows past the
    // group repeat its last row: computed, never stored) or this lane's row
    // D steps ahead, then the weights in the order of use, then the row scales
    u32x4 hr[NPT];
    u32x4 b[D][MF];
    const uint16_t* hg = P.h + static_cast<int64_t>(valid ? p : beg) * FFC;
    if constexpr (STAGE) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int idx = tid + 256 * i;
            if (NCH % 256 == 0 || idx < NCH) {
                const int row = idx / (FFC / 8), c = idx - row * (FFC / 8);
                hr[i] = *reinterpret_cast<const u32x4*>(P.h + static_cast<int64_t>(min(beg + row, end - 1)) * FFC + 8 * c);
            }
        }
    } else {
#pragma unroll
        for (int g = 0; g < D; ++g)
#pragma unroll
            for (int m = 0; m < MF; ++m) b[g][m] = *reinterpret_cast<const u32x4*>(hg + b_off<FMT>(s0 + g, q) + 8 * m);
    }
    __builtin_amdgcn_sched_barrier(0);
    AF a[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        a[g] = *reinterpret_cast<const AF*>(a_row + a_off<FMT>(s0 + g, q));
        __builtin_amdgcn_sched_barrier(0);
    }
    f32x4 s_row = {0, 0, 0, 0};
    if constexpr (FMT == W_INT8) {
        s_row = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(blob + P.os2) + m0 + 4 * q);
    }
    if constexpr (STAGE) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int idx = tid + 256 * i;
            if (NCH % 256 == 0 || idx < NCH) {
                const int row = idx / (FFC / 8), c = idx - row * (FFC / 8);
                *reinterpret_cast<u32x4*>(hs + row * HS + 8 * c) = hr[i];
            }
        }
    }
    __syncthreads();

    const f32x4 zero = {0, 0, 0, 0};
    f32x4 acc = zero, cc = zero;
    const uint16_t* hrow = hs + r * HS;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        u32x4 bg[MF];
        if constexpr (STAGE) {
#pragma unroll
            for (int m = 0; m < MF; ++m) bg[m] = *reinterpret_cast<const u32x4*>(hrow + b_off<FMT>(s0 + g, q) + 8 * m);
        } else {
#pragma unroll
            for (int m = 0; m < MF; ++m) bg[m] = b[g % D][m];
            if (g + D < NG) {
#pragma unroll
                for (int m = 0; m < MF; ++m)
                    b[g % D][m] = *reinterpret_cast<const u32x4*>(hg + b_off<FMT>(s0 + g + D, q) + 8 * m);
            }
        }
        if constexpr (FMT == W_INT8) {
            const u32x4 kb = splat(0xC300C300u);
            cc = mfma16x16x32(kb, bg[0], cc);
            cc = mfma16x16x32(kb, bg[1], cc);
            acc = mfma16x16x32(deq_int8(a[g][0], a[g][1]), bg[0], acc);
            acc = mfma16x16x32(deq_int8(a[g][2], a[g][3]), bg[1], acc);
        } else {
            acc = mfma16x16x32(a[g], bg[0], acc);
        }
    }
    if constexpr (FMT == W_INT8) acc = s_row * (acc + cc);
    if constexpr (KS > 1) {
        if (kp > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) s_red[((wave - 1) * 4 + j) * 64 + lane] = acc[j];
        }
        __syncthreads();
        if (kp != 0) return;
#pragma unroll
        for (int w = 1; w < KS; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += s_red[((wave + w - 1) * 4 + j) * 64 + lane];
    }
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

// ------------------------------------------------------------ int4 paths --
// An int4 lane loads 16 bytes = 32 elements of its row per instruction, so a
// 16-row tile moves 64 contiguous bytes per row (two 64-element groups).  Two
// v_permlane32_swap exchanges then give every lane two dwords of each group:
// dwords 0,1 hold group A (elements 0..63 of the 128-element block), dwords
// 2,3 group B.  MFMA m uses dword m of every lane, so lane group q supplies
// block elements 64(m/2) + 8(m%2) + 16(q/2) + 32(q%2) + perm8(0..7).  A row
// whose length K is an odd number of groups ends with one 64-element group
// read the plain way (8 bytes per lane, elements 16q + 8m + perm8(0..7)).
// Activations and h are stored in this position order ("operand order"):
// position p = 128 G + 32 q + 8 m + j holds element int4_pos_to_k(p, K).
__host__ __device__ __forceinline__ int perm8h(int j) { return (j >> 1) | ((j & 1) << 2); }
__host__ __device__ __forceinline__ int int4_pos_to_k(int p, int K) {
    const int full = K & ~127;
    if (p < full) {
        const int w = p & 127, q = w >> 5, m = (w >> 3) & 3, j = w & 7;
        return (p & ~127) + ((m >> 1) << 6) + ((m & 1) << 3) + ((q >> 1) << 4) + ((q & 1) << 5) + perm8h(j);
    }
    const int w = p - full, q = w >> 4, m = (w >> 3) & 1, j = w & 7;
    return full + (q << 4) + (m << 3) + perm8h(j);
}
// rows of the 16 positions [16u, 16u+16): base + (i & 8) + perm8(i & 7)
__device__ __forceinline__ int int4_tile_base(int u, int K) { return int4_pos_to_k(16 * u, K) & ~15; }

__device__ __forceinline__ u32x4 regroup(u32x4 v) {
    const auto x = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    const auto y = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    return u32x4{x[0], y[0], x[1], y[1]};
}

// acc += s_grp * (A . B - 136 * sum B) for one 64-element group given as two
// MFMA operands (one per dword)
__device__ __forceinline__ void int4_group(uint32_t d0, uint32_t d1, const u32x4& b0, const u32x4& b1,
                                           const f32x4& s, f32x4& acc) {
    const f32x4 zero = {0, 0, 0, 0};
    const u32x4 kb = splat(0xC308C308u);  // bf16 -136
    f32x4 t = mfma16x16x32(kb, b0, zero);
    t = mfma16x16x32(kb, b1, t);
    t = mfma16x16x32(deq_int4(d0), b0, t);
    t = mfma16x16x32(deq_int4(d1), b1, t);
    acc += s * t;
}

// One wave: 16 rows of a w13 or w2 tile over the K range [k0, k0 + Kw) of a
// row of K elements; codes a_lane (this lane's 16 bytes of double step 0: row,
// byte k0 / 2 + 16 q, in the blob's tiled layout, so double step i is 2 KB
// further), a_tail (its 8 bytes of the tail group), activations brow (this
// lane's column, at position k0), scales s_sc [group][16].
template <int CH>
__device__ __forceinline__ f32x4 int4_tile(const uint8_t* a_lane, const uint8_t* a_tail, rsrc_t bres, uint32_t boff,
                                           const float* s_sc, int nds, bool tail, int q) {
    // boff: byte offset of this lane's activation row at the K range start, or NO_LANE
    f32x4 acc = {0, 0, 0, 0};
    for (int c = 0; c < nds; c += CH) {
        u32x4 a[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (c + i < nds) a[i] = *reinterpret_cast<const u32x4*>(a_lane + 2048 * (c + i));
        u32x4 b[2][4];
#pragma unroll
        for (int m = 0; m < 4; ++m) b[0][m] = bload16(bres, boff + 2 * (128 * c + 32 * q + 8 * m));
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (c + i < nds) {
                if (i + 1 < CH && c + i + 1 < nds) {
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        b[(i + 1) & 1][m] = bload16(bres, boff + 2 * (128 * (c + i + 1) + 32 * q + 8 * m));
                }
                const u32x4 v = regroup(a[i]);
                const u32x4* bb = b[i & 1];
                const int g = 2 * (c + i);
                int4_group(v[0], v[1], bb[0], bb[1], *reinterpret_cast<const f32x4*>(s_sc + g * 16 + 4 * q), acc);
                int4_group(v[2], v[3], bb[2], bb[3], *reinterpret_cast<const f32x4*>(s_sc + (g + 1) * 16 + 4 * q), acc);
            }
        }
    }
    if (tail) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(a_tail);
        const u32x4 b0 = bload16(bres, boff + 2 * (128 * nds + 16 * q));
        const u32x4 b1 = bload16(bres, boff + 2 * (128 * nds + 16 * q + 8));
        int4_group(a[0], a[1], b0, b1, *reinterpret_cast<const f32x4*>(s_sc + 2 * nds * 16 + 4 * q), acc);
    }
    return acc;
}

// stage the scales of 16 rows (rows16[i]) x ng groups starting at group g0
// into s_sc[g][i] as fp32.  SPL > 0: all loads first (SPL per lane, so
// 16 * ng <= 64 * SPL), then the LDS stores; SPL == 0: a plain loop.
template <int SPL>
__device__ __forceinline__ void stage_scales(const uint16_t* sc_rows, int row_stride, int g0, int ng,
                                             const int* rows16, float* s_sc, int lane) {
    if constexpr (SPL > 0) {
        float sv[SPL];
#pragma unroll
        for (int m = 0; m < SPL; ++m) {
            const int idx = lane + 64 * m;
            sv[m] = 0.0f;
            if (idx < 16 * ng) {
                const int i = idx / ng, g = idx - i * ng;
                sv[m] = bf16_to_f32(sc_rows[static_cast<int64_t>(rows16[i]) * row_stride + g0 + g]);
            }
        }
#pragma unroll
        for (int m = 0; m < SPL; ++m) {
            const int idx = lane + 64 * m;
            if (idx < 16 * ng) {
                const int i = idx / ng, g = idx - i * ng;
                s_sc[g * 16 + i] = sv[m];
            }
        }
    } else {
        for (int idx = lane; idx < 16 * ng; idx += 64) {
            const int i = idx / ng, g = idx - i * ng;
            s_sc[g * 16 + i] = bf16_to_f32(sc_rows[static_cast<int64_t>(rows16[i]) * row_stride + g0 + g]);
        }
    }
}

// gate/up, int4: workgroup = 2*KH waves on one (expert, 16 positions of h,
// 16 routes); wave w = (tile t = w / KH: gate or up, K part w % KH).
template <int KH, int CH, int SPL>
__global__ __launch_bounds__(128 * KH) void gate_up_int4_kernel(FfnParams P) {
    extern __shared__ float smem[];
    const int ntile = P.FF >> 4;
    const int e = blockIdx.x / ntile, u = blockIdx.x - e * ntile;
    const int b0 = P.offsets[e], end = P.offsets[e + 1], beg = b0 + 16 * static_cast<int>(blockIdx.y);
    if (beg >= end || end - b0 > P.gmin) return;   // no routes here, or the group is the GEMM's
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const int t = wave / KH, hp = wave - t * KH;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
    const int n0 = int4_tile_base(u, P.FF);
    const int Kw = P.H / KH, k0 = hp * Kw;
    const int rowbase = t * P.FF + n0;
    const int arow = rowbase + (r & 8) + perm8(r & 7);
    const uint8_t* a_lane = blob + P.o13 + int4_code_off(arow, P.H / 64, k0 / 2 + 16 * q);
    const uint8_t* a_tail = blob + P.o13 + int4_code_off(arow, P.H / 64, k0 / 2 + 64 * (Kw >> 7) + 8 * q);
    const int p = beg + r;
    const bool valid = p < end;
    const int route = P.sorted_route[valid ? p : beg];
    const int ngw = Kw / 64;   // groups per wave
    float* s_sc = smem + wave * (16 * ngw);
    float* s_red = smem + 2 * KH * 16 * ngw;
    {
        int rows16[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) rows16[i] = rowbase + (i & 8) + perm8(i & 7);
        stage_scales<SPL>(reinterpret_cast<const uint16_t*>(blob + P.os13), P.H / 64, k0 / 64, Kw / 64, rows16,
                           s_sc, lane);
    }
    __syncthreads();
    const rsrc_t xres = make_rsrc(P.xq, static_cast<uint32_t>(P.T) * P.H * 2);
    const uint32_t xoff = valid ? static_cast<uint32_t>(((route / P.k) * P.H + k0) * 2) : NO_LANE;
    const f32x4 acc = int4_tile<CH>(a_lane, a_tail, xres, xoff, s_sc, Kw >> 7, (Kw & 127) != 0, q);
    if (wave > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) s_red[((wave - 1) * 4 + j) * 64 + lane] = acc[j];
    }
    __syncthreads();
    if (wave != 0) return;
    f32x4 g = acc, uu = {0, 0, 0, 0};
#pragma unroll
    for (int w = 1; w < 2 * KH; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = s_red[((w - 1) * 4 + j) * 64 + lane];
            if (w < KH) g[j] += v; else uu[j] += v;
        }
    if (valid) {
        const uint32_t h0 = pack_bf16x2(act_fn(P.act, g[0]) * uu[0], act_fn(P.act, g[1]) * uu[1]);
        const uint32_t h1 = pack_bf16x2(act_fn(P.act, g[2]) * uu[2], act_fn(P.act, g[3]) * uu[3]);
        *reinterpret_cast<u32x2*>(P.h + static_cast<int64_t>(p) * P.FF + 16 * u + 4 * q) = u32x2{h0, h1};
    }
}

// down, int4: workgroup = 4 waves x 16 rows of H, whole K = FF, 16 routes.
template <int CH, int SPL>
__global__ __launch_bounds__(256) void down_int4_kernel(FfnParams P) {
    extern __shared__ float smem[];
    const int nblk = P.H >> 6;
    const int e = blockIdx.x / nblk, blk = blockIdx.x - e * nblk;
    const int b0 = P.offsets[e], end = P.offsets[e + 1], beg = b0 + 16 * static_cast<int>(blockIdx.y);
    if (beg >= end || end - b0 > P.gmin) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
    const int m0 = blk * 64 + wave * 16;
    const uint8_t* a_lane = blob + P.o2 + int4_code_off(m0 + r, P.FF / 64, 16 * q);
    const uint8_t* a_tail = blob + P.o2 + int4_code_off(m0 + r, P.FF / 64, 64 * (P.FF >> 7) + 8 * q);
    const int p = beg + r;
    const bool valid = p < end;
    float* s_sc = smem + wave * (16 * (P.FF / 64));
    {
        int rows16[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) rows16[i] = m0 + i;
        stage_scales<SPL>(reinterpret_cast<const uint16_t*>(blob + P.os2), P.FF / 64, 0, P.FF / 64, rows16, s_sc,
                           lane);
    }
    __syncthreads();
    const rsrc_t hres = make_rsrc(P.h, static_cast<uint32_t>(P.T) * P.k * P.FF * 2);
    const uint32_t hoff = valid ? static_cast<uint32_t>(p) * P.FF * 2 : NO_LANE;
    const f32x4 acc = int4_tile<CH>(a_lane, a_tail, hres, hoff, s_sc, P.FF >> 7, (P.FF & 127) != 0, q);
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

// ------------------------------------------------ int4 gate/up, decode --
// One workgroup of 4 waves per (expert, GUD_TPW 16-row tiles of h): wave
// (t, part) = (gate or up) x (half of K), so a wave holds the 11 weight
// fragments per tile of its rows in registers, all requested at once (16 bytes
// per lane each).  The
// expert's routes are taken 4 at a time: their activations, already in the
// operand order (preparation kernel), and their 64-group sums (bf16 hi + lo)
// are copied into LDS, then every wave runs its MFMAs against the same weight
// registers.  Experts without
// routes leave at once; many small workgroups per CU keep enough loads in
// flight to stream the weights at close to the HBM rate.
constexpr int GUD_RT = 4;   // routes per route tile
constexpr int GUD_TPW = 1;  // 16-row tiles per workgroup

struct GudLds {             // offsets (bytes) into dynamic LDS
    int xs, xsum, sc, red, total;
};
__host__ __device__ inline GudLds gud_lds(int H) {
    GudLds L;
    const int G = H / 64, GS = (G + 39) & ~7, NGW = 2 * ((H / 128 + 1) / 2);
    L.xs = 0;                                             // bf16 [RT][H + 8] (rows 16 bytes apart in bank order)
    L.xsum = GUD_RT * (H + 8) * 2;                        // bf16 [2][RT][GS] hi, lo (zero past G)
    L.sc = (L.xsum + 2 * GUD_RT * GS * 2 + 15) & ~15;     // float [4 waves][TPW][NGW][16]
    L.red = L.sc + 4 * GUD_TPW * NGW * 16 * 4;            // float [TPW][3][4][64]
    L.total = L.red + GUD_TPW * 3 * 4 * 64 * 4;
    return L;
}

// XT = BF16: x rows are copied as they are and put into the operand order in
// LDS; XT = F32: the preparation kernel has converted them (P.xq, P.xsum).
template <int NDT, int XT>
__global__ __launch_bounds__(256) void gate_up_int4_dec_kernel(FfnParams P) {
    constexpr int KS = 2;
    constexpr int NDW = (NDT + KS - 1) / KS;   // double steps of one wave
    constexpr int NGW = 2 * NDW;
    static_assert(NGW <= 32, "the bias MFMA takes 32 groups");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // grid (tile, expert).  The group bounds and the expert's slot are
    // requested together (one round trip), before the exit test.
    const int e = blockIdx.y, u0 = blockIdx.x * GUD_TPW;
    const int beg = P.offsets[e], end = P.offsets[e + 1];
    const int slot = P.slot_of[e];
    // no routes, or the group is the GEMM's (a resident expert has slot >= 0;
    // the test on it makes the slot load part of the same round trip)
    if ((beg >= end) | (end - beg > P.gmin) | (slot < 0)) return;
    const int H = P.H, G = H / 64, GS = (G + 39) & ~7;
    const GudLds L = gud_lds(H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds + L.xs);
    uint16_t* xsum = reinterpret_cast<uint16_t*>(lds + L.xsum);
    float* s_sc = reinterpret_cast<float*>(lds + L.sc) + wave * (GUD_TPW * NGW * 16);
    float* s_red = reinterpret_cast<float*>(lds + L.red);
    const int t = wave >> 1, part = wave & 1;
    const int ds0 = part * NDT / KS, nds = (part + 1) * NDT / KS - ds0;
    const int ng = 2 * nds, k0 = 128 * ds0;

    // The activations of a route tile come from L2 and arrive long before the
    // weights, so they are requested first (tokens by uniform scalar loads,
    // read before any global store): waiting for them in the in-order vector
    // load counter does not wait for the weights.  A thread takes up to NSB of
    // the tile's 4 x H/8 blocks of 8 elements; bf16 x is read as it is and put
    // into the operand order in registers, fp32 x was converted by the
    // preparation kernel (xq and its group sums).
    constexpr int NSB = (GUD_RT * NDT * 16 + 255) / 256;
    static_assert(GUD_RT == 4, "four route tokens");
    const uint8_t* blob = P.pool + static_cast<uint64_t>(slot) * P.slot_bytes;
    constexpr int HC = 128 * NDT;   // H of this instantiation
    constexpr int nb = HC / 8;      // blocks per row, a multiple of 16
    // the first tile's 4 route indices, requested together, then their tokens
    int tk0 = P.sorted_route[beg], tk1 = P.sorted_route[beg + min(1, end - beg - 1)];
    int tk2 = P.sorted_route[beg + min(2, end - beg - 1)], tk3 = P.sorted_route[beg + min(3, end - beg - 1)];
    tk0 = route_token(tk0, P.kmul, P.k);
    tk1 = route_token(tk1, P.kmul, P.k);
    tk2 = route_token(tk2, P.kmul, P.k);
    tk3 = route_token(tk3, P.kmul, P.k);
    u32x4 xr[NSB];
    // Blocks past the tile's rows are neither read nor converted (nr * nb is
    // uniform, so the skips are scalar branches).
    auto load_x = [&](int nr) {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            if (256 * sb >= nr * nb) continue;
            const int i = min(tid + 256 * sb, nr * nb - 1);
            const int j = i / nb, blk = i - j * nb;
            const int tj = j >= 3 ? tk3 : (j == 2 ? tk2 : (j == 1 ? tk1 : tk0));
            if (XT == BF16)
                xr[sb] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(P.x) + static_cast<int64_t>(tj) * HC +
                                                         int4_pos_to_k(8 * blk, HC));
            else
                xr[sb] = *reinterpret_cast<const u32x4*>(P.xq + static_cast<int64_t>(tj) * HC + 8 * blk);
        }
    };
    auto store_x = [&](int nr) {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            if (256 * sb >= nr * nb) continue;
            const int i = tid + 256 * sb;
            const bool ok = i < nr * nb;   // nr * nb is a multiple of 16: whole 16-lane groups agree
            const int ic = min(i, nr * nb - 1), j = ic / nb, blk = ic - j * nb;
            if (XT == BF16) {
                // operand dword m = (element m, element m + 4) of the 8 read: a byte permute
                const u32x4 v = xr[sb];
                const u32x4 o = {__builtin_amdgcn_perm(v[2], v[0], 0x05040100u), __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                                 __builtin_amdgcn_perm(v[3], v[1], 0x05040100u), __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
                // sum of the 8 bf16 values in fp32
                float sum = 0.0f;
#pragma unroll
                for (int m = 0; m < 4; ++m) sum += __uint_as_float(v[m] << 16) + __uint_as_float(v[m] & 0xFFFF0000u);
                // the 8 blocks of a 64-group: block indices differing in bits 0, 2, 3
                sum += __shfl_xor(sum, 1, 64);
                sum += __shfl_xor(sum, 4, 64);
                sum += __shfl_xor(sum, 8, 64);
                if (ok) {
                    *reinterpret_cast<u32x4*>(xs + j * (HC + 8) + 8 * blk) = o;
                    if ((blk & 13) == 0) {
                        const int gi = j * GS + (blk >> 4) * 2 + ((blk >> 1) & 1);
                        const uint32_t shi = pack_bf16x2(sum, 0.0f) & 0xFFFFu;
                        xsum[gi] = static_cast<uint16_t>(shi);
                        xsum[GUD_RT * GS + gi] = static_cast<uint16_t>(pack_bf16x2(sum - __uint_as_float(shi << 16), 0.0f));
                    }
                }
            } else if (ok) {
                *reinterpret_cast<u32x4*>(xs + j * (HC + 8) + 8 * blk) = xr[sb];
            }
        }
        if (XT != BF16) {
            const uint16_t* xsg = reinterpret_cast<const uint16_t*>(P.xsum);
            for (int i = tid; i < 2 * nr * G; i += 256) {
                const int hl = i / (nr * G), rem = i - hl * (nr * G), j = rem / G, g = rem - j * G;
                const int tj = j >= 3 ? tk3 : (j == 2 ? tk2 : (j == 1 ? tk1 : tk0));
                xsum[(hl * GUD_RT + j) * GS + g] = xsg[(static_cast<int64_t>(hl) * P.T + tj) * G + g];
            }
        }
    };
    load_x(min(GUD_RT, end - beg));

    // then the weights: the scale dwords of this lane's row (groups 8q..8q+7 of
    // the wave's range) and its 11 fragments
    u32x4 sa[GUD_TPW];
    u32x4 a[GUD_TPW][NDW];
#pragma unroll
    for (int tt = 0; tt < GUD_TPW; ++tt) {
        const int row = t * P.FF + int4_tile_base(u0 + tt, P.FF) + (r & 8) + perm8(r & 7);
        const uint32_t* srow = reinterpret_cast<const uint32_t*>(blob + P.os13) + (row * G + k0 / 64) / 2;
        sa[tt] = *reinterpret_cast<const u32x4*>(srow + 4 * (8 * q < ng ? q : 0));
        const uint8_t* a_lane = blob + P.o13 + int4_code_off(row, G, k0 / 2 + 16 * q);   // tiled: double step i 2 KB further
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            a[tt][i] = *reinterpret_cast<const u32x4*>(a_lane + 2048 * min(i, nds - 1));
            __builtin_amdgcn_sched_barrier(0);   // issue order = order of use
        }
    }

    for (int i = tid; i < 2 * GUD_RT * GS; i += 256) xsum[i] = 0;
    __syncthreads();   // padding zero before any group sum lands
    auto compute_tile = [&](int rt, int nr) {
        // column r of the MFMA is token slot r % RT (slots past nr are discarded)
        const int slot = r & (GUD_RT - 1);
        const uint16_t* xrow = xs + slot * (H + 8) + k0 + 32 * q;   // 4 route rows on different banks
        const uint32_t* shi = reinterpret_cast<const uint32_t*>(xsum + slot * GS + k0 / 64 + 8 * q);
        const uint32_t* slo = reinterpret_cast<const uint32_t*>(xsum + GUD_RT * GS + slot * GS + k0 / 64 + 8 * q);
        const u32x4 xhi = {shi[0], shi[1], shi[2], shi[3]};
        const u32x4 xlo = {slo[0], slo[1], slo[2], slo[3]};
        const f32x4 zero = {0, 0, 0, 0};
        f32x4 acc[GUD_TPW];
#pragma unroll
        for (int tt = 0; tt < GUD_TPW; ++tt) {
            f32x4 corr = mfma16x16x32(sa[tt], xhi, zero);
            corr = mfma16x16x32(sa[tt], xlo, corr);
            acc[tt] = corr * -136.0f;
        }
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            if (i < nds) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 b0 = *reinterpret_cast<const u32x4*>(xrow + 128 * i + 16 * h);
                    const u32x4 b1 = *reinterpret_cast<const u32x4*>(xrow + 128 * i + 16 * h + 8);
#pragma unroll
                    for (int tt = 0; tt < GUD_TPW; ++tt) {
                        const u32x4 vv = regroup(a[tt][i]);
                        f32x4 d = mfma16x16x32(deq_int4(vv[2 * h]), b0, zero);
                        d = mfma16x16x32(deq_int4(vv[2 * h + 1]), b1, d);
                        acc[tt] += *reinterpret_cast<const f32x4*>(s_sc + (tt * NGW + 2 * i + h) * 16 + 4 * q) * d;
                    }
                }
            }
        }
        if (wave > 0) {
#pragma unroll
            for (int tt = 0; tt < GUD_TPW; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) s_red[((tt * 3 + wave - 1) * 4 + j) * 64 + lane] = acc[tt][j];
        }
        __syncthreads();
        if (wave == 0 && r < nr) {
            // gate = this wave + wave 1 (other K half); up = waves 2 + 3
            const int p = rt + r;
#pragma unroll
            for (int tt = 0; tt < GUD_TPW; ++tt) {
                f32x4 g = acc[tt], uu;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g[j] += s_red[((tt * 3 + 0) * 4 + j) * 64 + lane];
                    uu[j] = s_red[((tt * 3 + 1) * 4 + j) * 64 + lane] + s_red[((tt * 3 + 2) * 4 + j) * 64 + lane];
                }
                const uint32_t h0 = pack_bf16x2(act_fn(P.act, g[0]) * uu[0], act_fn(P.act, g[1]) * uu[1]);
                const uint32_t h1 = pack_bf16x2(act_fn(P.act, g[2]) * uu[2], act_fn(P.act, g[3]) * uu[3]);
                *reinterpret_cast<u32x2*>(P.h + static_cast<int64_t>(p) * P.FF + 16 * (u0 + tt) + 4 * q) = u32x2{h0, h1};
            }
        }
    };

    // first route tile: its activations were requested before the weights
    const int nr0 = min(GUD_RT, end - beg);
    store_x(nr0);
#pragma unroll
    for (int tt = 0; tt < GUD_TPW; ++tt) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (8 * q + 2 * j >= ng) sa[tt][j] = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = 8 * q + 2 * j;
            if (g < ng) {
                s_sc[(tt * NGW + g) * 16 + r] = __uint_as_float(sa[tt][j] << 16);
                s_sc[(tt * NGW + g + 1) * 16 + r] = __uint_as_float(sa[tt][j] & 0xFFFF0000u);
            }
        }
    }
    __syncthreads();
    compute_tile(beg, nr0);
    // further route tiles (groups of more than 4 routes)
    for (int rt = beg + GUD_RT; rt < end; rt += GUD_RT) {
        const int nr = min(GUD_RT, end - rt);
        tk0 = P.sorted_route[rt];
        tk1 = P.sorted_route[rt + min(1, nr - 1)];
        tk2 = P.sorted_route[rt + min(2, nr - 1)];
        tk3 = P.sorted_route[rt + min(3, nr - 1)];
        tk0 = route_token(tk0, P.kmul, P.k);
        tk1 = route_token(tk1, P.kmul, P.k);
        tk2 = route_token(tk2, P.kmul, P.k);
        tk3 = route_token(tk3, P.kmul, P.k);
        __syncthreads();   // the previous tile's readers of xs, xsum and s_red are done
        load_x(nr);
        store_x(nr);
        __syncthreads();
        compute_tile(rt, nr);
    }
}

// ------------------------------------------------------ int4 down, decode --
// One workgroup of 4 waves per (expert, 64 TPW rows of H); a wave owns TPW
// tiles of 16 rows and the whole K = FF (NDS double steps and, when
// FF % 128 == 64, a tail group).  The expert's routes are taken 4 at a time.
// The first tile's h rows are requested before the weights (h sits in L2), so
// waiting for them in the in-order vector load counter does not wait for the
// weights; all weight fragments and row scales of the wave are then requested
// at once.  More rows per wave keep more bytes in flight per workgroup; the
// h fragments read from LDS serve every tile of the wave.
#ifndef DND_TPW
#define DND_TPW 1
#endif
template <int NDS, bool TAIL, int TPW>
__global__ __launch_bounds__(256) void down_int4_dec_kernel(FfnParams P) {
    constexpr int NG = 2 * NDS + (TAIL ? 1 : 0);   // groups per row
    constexpr int SPL = (16 * NG + 63) / 64;       // scale values per lane and tile
    constexpr int RT = GUD_RT;
    // [RT][FF + 8] bf16: rows 16 bytes apart in bank order, so that the 4 route
    // rows of a fragment read sit on different banks (FF + 8 <= 128 (NDS + 1))
    __shared__ __attribute__((aligned(16))) uint16_t hs[RT * 128 * (NDS + 1)];
    __shared__ float s_scs[4][TPW][NG * 16];
    const int FF = P.FF;
    // grid (64 TPW-row block of H, expert); group bounds and slot in one round trip
    const int e = blockIdx.y, blk = blockIdx.x;
    const int beg = P.offsets[e], end = P.offsets[e + 1];
    const int slot = P.slot_of[e];
    if ((beg >= end) | (end - beg > P.gmin) | (slot < 0)) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
    const uint8_t* blob = P.pool + static_cast<uint64_t>(slot) * P.slot_bytes;
    const int m0 = (blk * 4 + wave) * 16 * TPW;   // first row of the wave; tile tt is rows m0 + 16 tt
    constexpr int NHB = (RT * 128 * (NDS + 1) / 8 + 255) / 256;   // blocks of 8 per thread (upper bound)
    const int nbr = FF / 8;                                         // blocks per h row

    // blocks past the tile's rows are neither read nor stored (nr * nbr is
    // uniform, so the skips are scalar branches)
    u32x4 hr[NHB];
    auto load_h = [&](int rt, int nr) {
#pragma unroll
        for (int sb = 0; sb < NHB; ++sb) {
            if (256 * sb >= nr * nbr) continue;
            const int i = min(tid + 256 * sb, nr * nbr - 1);
            const int j = i / nbr, c = i - j * nbr;
            hr[sb] = *reinterpret_cast<const u32x4*>(P.h + static_cast<int64_t>(rt + j) * FF + 8 * c);
        }
    };
    auto store_h = [&](int nr) {
#pragma unroll
        for (int sb = 0; sb < NHB; ++sb) {
            if (256 * sb >= nr * nbr) continue;
            const int i = tid + 256 * sb;
            if (i < nr * nbr) {
                const int j = i / nbr, c = i - j * nbr;
                *reinterpret_cast<u32x4*>(hs + j * (FF + 8) + 8 * c) = hr[sb];
            }
        }
    };
    const int nr0 = min(RT, end - beg);
    load_h(beg, nr0);

    // the scales of the wave's TPW tiles of 16 rows (needed in LDS before any
    // MFMA), then the weights in the order of use, the tail group last
    u32x4 a[TPW][NDS];
    u32x2 at[TPW];
    float sv[TPW][SPL];
    {
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + P.os2);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int m = 0; m < SPL; ++m) {
                const int idx = min(lane + 64 * m, 16 * NG - 1);
                const int i = idx / NG, g = idx - i * NG;
                sv[tt][m] = bf16_to_f32(sc[static_cast<int64_t>(m0 + 16 * tt + i) * NG + g]);
            }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int arow = m0 + 16 * tt + r;
        const uint8_t* a_lane = blob + P.o2 + int4_code_off(arow, FF / 64, 16 * q);   // tiled: double step i 2 KB further
#pragma unroll
        for (int i = 0; i < NDS; ++i) {
            a[tt][i] = *reinterpret_cast<const u32x4*>(a_lane + 2048 * i);
            __builtin_amdgcn_sched_barrier(0);
        }
        at[tt] = u32x2{0u, 0u};
        if (TAIL) at[tt] = *reinterpret_cast<const u32x2*>(blob + P.o2 + int4_code_off(arow, FF / 64, 64 * NDS + 8 * q));
    }

    auto compute_tile = [&](int rt, int nr) {
        const int slot = r & (RT - 1);
        const uint16_t* hrow = hs + slot * (FF + 8) + 32 * q;
        f32x4 acc[TPW];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) acc[tt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NDS; ++i) {
            u32x4 b[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) b[m] = *reinterpret_cast<const u32x4*>(hrow + 128 * i + 8 * m);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const float* s_sc = &s_scs[wave][tt][0];
                const u32x4 v = regroup(a[tt][i]);
                int4_group(v[0], v[1], b[0], b[1], *reinterpret_cast<const f32x4*>(s_sc + (2 * i) * 16 + 4 * q), acc[tt]);
                int4_group(v[2], v[3], b[2], b[3], *reinterpret_cast<const f32x4*>(s_sc + (2 * i + 1) * 16 + 4 * q), acc[tt]);
            }
        }
        if (TAIL) {
            const uint16_t* tr = hs + slot * (FF + 8) + 128 * NDS + 16 * q;
            const u32x4 b0 = *reinterpret_cast<const u32x4*>(tr), b1 = *reinterpret_cast<const u32x4*>(tr + 8);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
                int4_group(at[tt][0], at[tt][1], b0, b1, *reinterpret_cast<const f32x4*>(&s_scs[wave][tt][0] + 2 * NDS * 16 + 4 * q),
                           acc[tt]);
        }
        if (r < nr) {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int64_t o = static_cast<int64_t>(rt + r) * P.H + m0 + 16 * tt + 4 * q;
                if (P.out_dt == F32) {
                    *reinterpret_cast<f32x4*>(static_cast<float*>(P.out) + o) = acc[tt];
                } else {
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.out) + o) =
                        u32x2{pack_bf16x2(acc[tt][0], acc[tt][1]), pack_bf16x2(acc[tt][2], acc[tt][3])};
                }
            }
        }
    };

    store_h(nr0);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int m = 0; m < SPL; ++m) {
            const int idx = lane + 64 * m;
            if (idx < 16 * NG) {
                const int i = idx / NG, g = idx - i * NG;
                s_scs[wave][tt][g * 16 + i] = sv[tt][m];
            }
        }
    __syncthreads();
    compute_tile(beg, nr0);
    for (int rt = beg + RT; rt < end; rt += RT) {
        const int nr = min(RT, end - rt);
        __syncthreads();   // readers of the previous tile's h are done
        load_h(rt, nr);
        store_h(nr);
        __syncthreads();
        compute_tile(rt, nr);
    }
}

// x -> xq in the int4 operand order of K = H (one thread per 8 positions)
template <int XT>
__global__ __launch_bounds__(256) void prep_x_int4_kernel(const void* __restrict__ x, int T, int H,
                                                          uint16_t* __restrict__ xq, float* __restrict__ xsum) {
    // xsum (H % 128 == 0 only): per token and 64-element group, the sum of the
    // bf16 values in that group, as bf16 hi [T, H/64] followed by bf16 lo [T, H/64]
    const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (b >= static_cast<int64_t>(T) * (H / 8)) return;   // T * H / 8 is a multiple of 16: whole groups exit together
    const int64_t t = b / (H / 8);
    const int p0 = static_cast<int>(b - t * (H / 8)) * 8;
    const int k0 = int4_pos_to_k(p0, H);   // elements k0 + perm8(j), j = 0..7
    float v[8];
    if (XT == F32) {
        const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + t * H + k0);
        const f32x4 a = src[0], c = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = c[j];
        }
    } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + t * H + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(a[j] << 16);
            v[2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
        }
    }
    u32x4 o;
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint16_t lo = f32_to_bf16(v[perm8(2 * j)]), hi = f32_to_bf16(v[perm8(2 * j + 1)]);
        o[j] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
        sum += bf16_to_f32(lo) + bf16_to_f32(hi);
    }
    *reinterpret_cast<u32x4*>(xq + t * H + p0) = o;
    if (xsum != nullptr) {
        // the 8 blocks of a 64-element group are lanes whose block index differs
        // in bits 0, 2 and 3 (bit 1 selects group A or B of the double step)
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 4, 64);
        sum += __shfl_xor(sum, 8, 64);
        const int blk = p0 >> 3;
        if ((blk & 13) == 0) {
            // stored as bf16 hi + lo (hi + lo = sum to ~16 bits) for a bf16 MFMA
            const int64_t gi = t * (H / 64) + (blk >> 4) * 2 + ((blk >> 1) & 1);
            const uint16_t hi = f32_to_bf16(sum);
            uint16_t* xs = reinterpret_cast<uint16_t*>(xsum);
            xs[gi] = hi;
            xs[static_cast<int64_t>(T) * (H / 64) + gi] = f32_to_bf16(sum - bf16_to_f32(hi));
        }
    }
}

static void launch_int4(const FfnParams& P, int phases, hipStream_t s) {
    const unsigned tiles_y = (P.T + 15) / 16;
    if (phases & 1) {
        if (P.xq == nullptr) {
            // the decode kernel has run the first half
        } else if (P.H % 256 == 0 && P.H <= 2816) {   // two K halves of <= 11 double steps, <= 22 groups each
            const int ngw = P.H / 128;
            const size_t smem = (4 * 16 * ngw + 3 * 4 * 64) * sizeof(float);
            hipLaunchKernelGGL((gate_up_int4_kernel<2, 11, 6>), dim3(P.E * (P.FF / 16), tiles_y), dim3(256), smem, s, P);
        } else {
            const int ngw = P.H / 64;
            const size_t smem = (2 * 16 * ngw + 1 * 4 * 64) * sizeof(float);
            hipLaunchKernelGGL((gate_up_int4_kernel<1, 4, 0>), dim3(P.E * (P.FF / 16), tiles_y), dim3(128), smem, s, P);
        }
    }
    if (phases & 2) {
        const size_t smem = 4 * 16 * (P.FF / 64) * sizeof(float);
        if (P.FF == 704) {   // decode: 5 double steps and a tail group
            if (P.H % (64 * DND_TPW) == 0)
                hipLaunchKernelGGL((down_int4_dec_kernel<5, true, DND_TPW>), dim3(P.H / (64 * DND_TPW), P.E), dim3(256), 0, s, P);
            else
                hipLaunchKernelGGL((down_int4_dec_kernel<5, true, 1>), dim3(P.H / 64, P.E), dim3(256), 0, s, P);
            return;
        }
        if (P.FF <= 704)   // <= 5 double steps and a tail, <= 11 groups
            hipLaunchKernelGGL((down_int4_kernel<5, 3>), dim3(P.E * (P.H / 64), tiles_y), dim3(256), smem, s, P);
        else
            hipLaunchKernelGGL((down_int4_kernel<4, 0>), dim3(P.E * (P.H / 64), tiles_y), dim3(256), smem, s, P);
    }
}

// ------------------------------------------------------------------ host --
FfnWorkspace ffn_workspace(int T, int k, int H, int FF) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    FfnWorkspace w;
    w.xq_off = 0;
    // group sums: bf16 hi + lo per (row, 64-group), rows padded to 16 groups
    const size_t gx = static_cast<size_t>((H / 64 + 15) & ~15), gh = static_cast<size_t>((FF / 64 + 15) & ~15);
    w.xsum_off = up(static_cast<size_t>(T) * H * 2);
    w.xqg_off = w.xsum_off + up(static_cast<size_t>(T) * gx * 4);
    // the grouped GEMM's own x copy and sums, only when that family can run
    const size_t tg = T > GEMM_T_MIN ? static_cast<size_t>(T) : 0;
    w.xsumg_off = w.xqg_off + up(tg * H * 2);
    w.h_off = w.xsumg_off + up(tg * gx * 4);
    w.hsum_off = w.h_off + up(static_cast<size_t>(T) * k * FF * 2);
    w.bytes = w.hsum_off + up(static_cast<size_t>(T) * k * gh * 4);
    return w;
}

template <int FMT, int KSPLIT>
static void launch_gate_up_generic(const FfnParams& P, hipStream_t s) {
    const size_t smem = (KSPLIT - 1) * 8 * 64 * sizeof(float);
    const dim3 grid(P.E * (P.FF / 16)), block(64 * KSPLIT);
    hipLaunchKernelGGL((gate_up_generic_kernel<FMT, KSPLIT, 4>), grid, block, smem, s, P);
}

// fast-path shapes: (steps per wave, waves splitting K) with steps * waves = the step count
template <int FMT, int NG, int KSPLIT>
static void launch_gate_up_fast(const FfnParams& P, hipStream_t s) {
    const size_t smem = gate_up_fast_lds<FMT, NG, KSPLIT>();
    hipLaunchKernelGGL((gate_up_fast_kernel<FMT, NG, KSPLIT>), dim3(P.E * (P.FF / 16), (P.T + 15) / 16), dim3(64 * KSPLIT),
                       smem, s, P);
}

template <int FMT, int NG, int KS>
static void launch_down_fast(const FfnParams& P, hipStream_t s) {
    const size_t smem = down_fast_lds<FMT, NG, KS>();
    hipLaunchKernelGGL((down_fast_kernel<FMT, NG, KS>), dim3(P.E * (P.H / (16 * (4 / KS))), (P.T + 15) / 16), dim3(256),
                       smem, s, P);
}

template <int FMT>
static bool try_fast(const FfnParams& P, int phases, hipStream_t s) {
    constexpr int KSTEP = Geo<FMT>::KSTEP;
    const int n1 = P.H / KSTEP, n2 = P.FF / KSTEP;
    const bool ok1 = !(phases & 1) || (FMT == W_BF16 ? n1 == 88 : n1 == 44);
    const bool ok2 = !(phases & 2) || (FMT == W_BF16 ? n2 == 22 : n2 == 11);
    if (!ok1 || !ok2 || P.T > 64) return false;
    if (phases & 1) {
        if (FMT == W_BF16) launch_gate_up_fast<FMT, 11, 8>(P, s);
        else launch_gate_up_fast<FMT, 11, 4>(P, s);
    }
    if (phases & 2) {
        if (FMT == W_BF16) launch_down_fast<FMT, 11, 2>(P, s);
        else launch_down_fast<FMT, 11, 1>(P, s);
    }
    return true;
}

template <int FMT>
static void launch_phases(const FfnParams& P, int phases, hipStream_t s) {
    static_assert(FMT != W_INT4, "int4 blobs hold tiled codes: the int4 kernels read them");
    constexpr int KSTEP = Geo<FMT>::KSTEP;
    if (try_fast<FMT>(P, phases, s)) return;
    if (phases & 1) {
        const int nsteps = P.H / KSTEP;
        if (nsteps % 4 == 0)
            launch_gate_up_generic<FMT, 4>(P, s);
        else if (nsteps % 2 == 0)
            launch_gate_up_generic<FMT, 2>(P, s);
        else
            launch_gate_up_generic<FMT, 1>(P, s);
    }
    if (phases & 2) {
        hipLaunchKernelGGL((down_generic_kernel<FMT, 4>), dim3(P.E * (P.H / 64)), dim3(256), 0, s, P);
    }
}

// A second stream per device for the grouped GEMM, with the two events that
// fork it from and join it back into the caller's stream; created on the
// first use outside graph capture and kept until the process ends.  nullptr
// before that, or if creation failed (the call then runs on one stream).
namespace {
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;   // also orders the event records of concurrent calls
SideStream* side_stream_locked(hipStream_t s) {
    static SideStream side[64];
    static bool tried[64];
    int dev = 0, sdev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    // the caller's stream must belong to the current device (the side stream
    // is that device's); otherwise the call stays on the caller's stream
    if (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (!tried[dev]) {
        // not while s is being captured into a graph (creating a stream or an
        // event there is not a stream operation); such a call runs on one stream
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
            (void)hipGetLastError();
            return nullptr;
        }
        tried[dev] = true;
        SideStream t;
        if (hipStreamCreateWithFlags(&t.s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&t.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&t.join, hipEventDisableTiming) == hipSuccess)
            side[dev] = t;
        (void)hipGetLastError();
    }
    return side[dev].join ? &side[dev] : nullptr;
}
}  // namespace

static hipError_t launch_streaming(FfnParams P, int phases, hipStream_t s);

hipError_t launch_ffn(const FfnParams& P0, int phases, hipStream_t s, bool fork) {
    FfnParams P = P0;
    P.gmin = INT_MAX;
    if (P.fmt == W_INT4 && P.T > GEMM_T_MIN && int4_gemm_eligible(P)) {
        // per expert group: more than GEMM_GROUP_MIN routes -> grouped GEMM,
        // the rest -> the streaming kernels.  The two families touch disjoint
        // groups (and disjoint parts of the workspace), so the GEMM runs on a
        // second stream, forked from s and joined back: at mid-size batches
        // neither family fills the GPU alone.
        P.gmin = GEMM_GROUP_MIN;
        std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
        SideStream* side = nullptr;
        if (fork) {
            lk.lock();
            side = side_stream_locked(s);
        }
        hipError_t err = hipSuccess;
        if (side) {
            if ((err = hipEventRecord(side->fork, s)) != hipSuccess) return err;
            if ((err = hipStreamWaitEvent(side->s, side->fork, 0)) != hipSuccess) return err;
        }
        if ((err = launch_int4_gemm(P, phases, side ? side->s : s)) != hipSuccess) return err;
        err = launch_streaming(P, phases, s);
        if (side) {
            const hipError_t e1 = hipEventRecord(side->join, side->s);
            const hipError_t e2 = hipStreamWaitEvent(s, side->join, 0);
            if (err == hipSuccess) err = e1 != hipSuccess ? e1 : e2;
        }
        return err;
    }
    return launch_streaming(P, phases, s);
}

// the streaming kernels of every group that P.gmin leaves them
static hipError_t launch_streaming(FfnParams P, int phases, hipStream_t s) {
    if ((phases & 1) && P.fmt == W_INT4 && P.H == 2816 && P.FF % (16 * GUD_TPW) == 0) {
        const GudLds L = gud_lds(P.H);
        const dim3 grid(P.FF / 16 / GUD_TPW, P.E);
        if (P.x_dt == F32) {
            const int64_t nblk = static_cast<int64_t>(P.T) * P.H / 8;
            P.xq = P.xq_out;
            P.xsum = P.xsum_out;
            hipLaunchKernelGGL((prep_x_int4_kernel<F32>), dim3(static_cast<uint32_t>((nblk + 255) / 256)), dim3(256), 0, s,
                               P.x, P.T, P.H, P.xq_out, P.xsum);
            hipLaunchKernelGGL((gate_up_int4_dec_kernel<22, F32>), grid, dim3(256), L.total, s, P);
        } else {
            hipLaunchKernelGGL((gate_up_int4_dec_kernel<22, BF16>), grid, dim3(256), L.total, s, P);
        }
        P.xq = nullptr;   // tells launch_int4 the first half is done
        if (phases == 1) return hipGetLastError();
        launch_int4(P, 2, s);
        return hipGetLastError();
    }
    if (phases & 1) {
        const bool perm = (P.fmt == W_INT4);
        if (perm || P.x_dt == F32) {
            const int64_t nblk = static_cast<int64_t>(P.T) * P.H / 8;
            const dim3 grid(static_cast<uint32_t>((nblk + 255) / 256)), block(256);
            if (P.x_dt == F32 && perm)
                hipLaunchKernelGGL((prep_x_int4_kernel<F32>), grid, block, 0, s, P.x, P.T, P.H, P.xq_out, P.xsum);
            else if (P.x_dt == F32)
                hipLaunchKernelGGL((prep_x_kernel<F32, false>), grid, block, 0, s, P.x, nblk, P.xq_out);
            else
                hipLaunchKernelGGL((prep_x_int4_kernel<BF16>), grid, block, 0, s, P.x, P.T, P.H, P.xq_out, P.xsum);
            P.xq = P.xq_out;
        } else {
            P.xq = static_cast<const uint16_t*>(P.x);
        }
    }
    if (P.fmt == W_INT4)
        launch_int4(P, phases, s);
    else if (P.fmt == W_INT8)
        launch_phases<W_INT8>(P, phases, s);
    else
        launch_phases<W_BF16>(P, phases, s);
    return hipGetLastError();
}

}  // namespace moe
