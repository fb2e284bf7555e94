// int4 expert FFN for large token groups (prefill chunks): per expert, the
// routes of the expert form the rows of a grouped GEMM against its packed
// weights (prain README, "Expert formats": w13 = gate and up stacked, w2 down;
// int4 with a bf16 scale per 64-element group, dequantised in the kernel).
//
// MFMA v_mfma_f32_32x32x16_bf16, operands:
//   A = 32 routes x 16 K of bf16 activations, staged through LDS;
//   B = 16 K x 32 weight rows, expanded from int4 in registers;
//   D = 32 routes x 32 weight rows, fp32.  Lane l holds D column (l & 31) and
//       rows 8 (v / 4) + 4 (l >> 5) + (v & 3) of its 16 values v.
// Lane l holds A row / B column (l & 31) and the K slots 8 (l >> 5) + j.
// A lane's 16-byte weight load covers the 32 codes 32 h + 0..31 of one
// 64-group of its row (h = l >> 5): dword s feeds K step s, and its expansion
// (d >> 4i) & 0x000F000F | 0x43004300 puts code 8 s + perm8(j) in slot j.
// The activations are therefore stored in "M32 operand order": inside each
// 64-group, position 16 s + 8 h + j holds element 32 h + 8 s + perm8(j), so an
// A fragment is one 16-byte read.
//
// The expanded codes are 128 + (q + 8): each group's fp32 partial sum is
// scaled by the group's bf16 scale, and the offset is removed once per tile
// by an MFMA of the row scales with the activations' group sums (bf16 hi + lo),
// -136 * sum_g s[n][g] * X[m][g].
//
// Work items are (expert, route tile, N tile); two workgroups of 4 waves per
// CU walk the items (one of 8 waves is a build option).  Wave (mh, nq): routes
// 64 mh .. 64 mh + 63 of the tile (two 32-route blocks) times 64 weight rows
// (two 32-row blocks).  The K loop runs over 64-groups: a group's activations
// (a 128-byte piece of each route row of the tile) are copied by LDS DMA two
// groups ahead into a ring of three stages, whole cache lines per copy, XOR
// swizzled in LDS; each wave keeps the weights of the next 2*DC groups in flight
// in registers, one 1 KB load per group and 32 rows from the blob's tiled codes.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
}

// position of element f (0..63) of a 64-group in the M32 operand order
__host__ __device__ __forceinline__ int m32_pos(int f) {
    const int h = f >> 5, s = (f >> 3) & 3, e = f & 7;
    return 16 * s + 8 * h + (((e & 3) << 1) | (e >> 2));   // slot j with perm8(j) = e
}

constexpr int GM_ROWS = 128;   // routes per narrow tile
// Groups of at most GEMM_WIDE_MAX routes take wide tiles (64 routes, an N
// tile twice as wide: half the activation traffic per weight byte); larger
// ones take 128-route narrow tiles.
#ifndef GEMM_WIDE_MAX
#define GEMM_WIDE_MAX 96
#endif
constexpr int GM_GBUF = 16384; // one group of a stage: [4 K steps][4 route blocks] x 1 KB
// A workgroup of NW waves (4 or 8): wave (mh, nq), NQ = NW / 2 column blocks
// per narrow tile; a stage holds NW / 4 groups.

// ---------------------------------------------------------------- prep ----
// x [T, H] (fp32 or bf16) -> xq [T, H] bf16 in M32 operand order, and the
// per-(token, 64-group) sums of the bf16 values as bf16 hi + lo:
// xs [0][T][GP] hi, xs [1][T][GP] lo, GP = H/64 rounded up to 16, padding 0.
template <int XT>
__global__ __launch_bounds__(256) void prep_x_m32_kernel(const void* __restrict__ x, int T, int H,
                                                         uint16_t* __restrict__ xq, uint16_t* __restrict__ xs) {
    const int nb = H / 8;   // a multiple of 8: the 8 threads of a group are lanes 8i..8i+7
    const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (b >= static_cast<int64_t>(T) * nb) return;
    const int t = static_cast<int>(b / nb), p0 = static_cast<int>(b - static_cast<int64_t>(t) * nb) * 8;
    const int g = p0 >> 6, s = (p0 >> 4) & 3, h = (p0 >> 3) & 1;
    const int k0 = 64 * g + 32 * h + 8 * s;
    float v[8];
    if (XT == F32) {
        const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + static_cast<int64_t>(t) * H + k0);
        const f32x4 a = src[0], c = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = c[j];
        }
    } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + static_cast<int64_t>(t) * H + k0);
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
    *reinterpret_cast<u32x4*>(xq + static_cast<int64_t>(t) * H + p0) = o;
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    sum += __shfl_xor(sum, 4, 64);
    if ((p0 & 63) == 0) {
        const int G = H / 64, GP = (G + 15) & ~15;
        uint16_t* rh = xs + static_cast<int64_t>(t) * GP;
        uint16_t* rl = xs + (static_cast<int64_t>(T) + t) * GP;
        const uint16_t shi = f32_to_bf16(sum);
        rh[g] = shi;
        rl[g] = f32_to_bf16(sum - bf16_to_f32(shi));
        if (g == G - 1)
            for (int i = G; i < GP; ++i) rh[i] = rl[i] = 0;
    }
}

// ---------------------------------------------------------------- GEMM ----
// MODE 0: gate/up.  K = H.  N tile = 128 gate rows + the matching 128 up rows;
//         wave nq owns gate rows n0 + 32 nq + c and up rows FF + n0 + 32 nq + c.
//         Epilogue: h = act(gate) * up as bf16 in M32 operand order over FF,
//         and the group sums of h (bf16 hi + lo) for the second half.
// MODE 1: down.  K = FF.  N tile = 256 rows of w2; wave nq owns rows
//         n0 + 64 nq + 32 nb + c.  Epilogue: the route rows of out (fp32/bf16).
template <int MODE, int NW>
struct GemmShape {
    int K, G, GP, NC, NT, nrows, gp_a;
};

template <int MODE, int NW>
__device__ __forceinline__ GemmShape<MODE, NW> gemm_shape(const FfnParams& P) {
    constexpr int NQ = NW / 2, SG = NW / 4;
    GemmShape<MODE, NW> S;
    S.K = MODE == 0 ? P.H : P.FF;
    S.G = S.K / 64;
    S.GP = (S.G + 15) & ~15;
    S.NC = (S.G + SG - 1) / SG;
    S.NT = MODE == 0 ? (P.FF + 32 * NQ - 1) / (32 * NQ) : (P.H + 64 * NQ - 1) / (64 * NQ);
    S.nrows = MODE == 0 ? 2 * P.FF : P.H;   // rows of the weight matrix
    return S;
}

// stages of activations in LDS: 4-wave workgroups copy them with LDS DMA
// into a ring of 3 (two groups of prefetch), 8-wave ones through registers
// into 2
__host__ __device__ constexpr int gemm_nstage(int NW) { return NW == 4 ? 3 : 2; }

__host__ __device__ inline size_t gemm_lds_bytes(int E, int G, int NW) {
    return gemm_nstage(NW) * static_cast<size_t>(NW / 4) * GM_GBUF + static_cast<size_t>(64 * NW) * G * 2 + 16 +
           static_cast<size_t>(E + 1) * 4;
}

template <int MODE, int DC, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void ffn_int4_gemm_kernel(FfnParams P) {
    constexpr int NQ = NW / 2;                      // column blocks of a narrow tile
    constexpr int SG = NW / 4;                      // groups per stage
    constexpr int XBUF = SG * GM_GBUF;              // bytes of one stage
    constexpr int NTH = 64 * NW;                    // threads
    constexpr int D = 2 * DC;                       // weight groups in flight per wave
    constexpr int U = (D / SG) > 2 ? (D / SG) : 2;  // chunks per unrolled body: static slots and stage parity
    constexpr bool XD = NW == 4;                    // activations by LDS DMA (3-stage ring)
    constexpr int NSTG = gemm_nstage(NW);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const GemmShape<MODE, NW> S = gemm_shape<MODE, NW>(P);
    const int E = P.E, G = S.G, GP = S.GP, NC = S.NC, NT = S.NT;
    uint8_t* xbuf = lds;                                                   // [NSTG][XBUF]
    uint16_t* ssc = reinterpret_cast<uint16_t*>(lds + NSTG * XBUF);        // [NTH][G] bf16 scales of the tile
    int* pre = reinterpret_cast<int*>(lds + NSTG * XBUF + ((NTH * G * 2 + 15) & ~15));   // [E+1]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, c32 = lane & 31, hh = lane >> 5;
    const int mh = wave / NQ, nq = wave % NQ;

    // Items per expert -> prefix sums (wave 0).  An expert with at most 64
    // routes is one "wide" row tile: the two wave halves take different
    // columns (an N tile twice as wide), so that both waves of each SIMD work.
    // Larger groups take 128-route tiles, the halves splitting the routes.
    const int NTW = MODE == 0 ? (P.FF + 32 * NW - 1) / (32 * NW) : (P.H + 64 * NW - 1) / (64 * NW);
    if (wave == 0) {
        int run = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int me = e < E ? P.offsets[e + 1] - P.offsets[e] : 0;
            const int cnt = me == 0 ? 0 : (me <= GEMM_WIDE_MAX ? (me + 63) / 64 * NTW : (me + GM_ROWS - 1) / GM_ROWS * NT);
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d, 64);
                if (lane >= d) incl += o;
            }
            if (e < E) pre[e + 1] = run + incl;
            run += __shfl(incl, 63, 64);
        }
        if (lane == 0) pre[0] = 0;
    }
    __syncthreads();
    const int nitems = pre[E];

    const uint64_t o_codes = MODE == 0 ? P.o13 : P.o2, o_scales = MODE == 0 ? P.os13 : P.os2;
    const int arow_stride = MODE == 0 ? P.H : P.FF;                 // elements per A row
    const uint16_t* abase = MODE == 0 ? P.xq : P.h;
    const uint16_t* asum = MODE == 0 ? reinterpret_cast<const uint16_t*>(P.xsum) : P.hsum;
    const int asum_rows = MODE == 0 ? P.T : P.T * P.k;

    // XCD-aware order: workgroups are dealt to the 8 XCDs round robin, so the
    // workgroups of one XCD (blockIdx % 8) take one contiguous eighth of the
    // item list.  An expert's N tiles then run on one XCD and its activation
    // rows are fetched into that XCD's L2 once.  (A mapping that differs only
    // costs locality, not correctness: every item is still taken once.)
    const int nxcd = gridDim.x % 8 == 0 ? 8 : 1;
    const int xcd = blockIdx.x % nxcd, wpx = gridDim.x / nxcd, wj = blockIdx.x / nxcd;
    const int ibeg = static_cast<int>(static_cast<int64_t>(nitems) * xcd / nxcd);
    const int iend = static_cast<int>(static_cast<int64_t>(nitems) * (xcd + 1) / nxcd);
    for (int item = ibeg + wj; item < iend; item += wpx) {
        int lo = 0, hi = E;   // largest e with pre[e] <= item
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= item) lo = mid; else hi = mid;
        }
        const int e = lo, li = item - pre[e];
        const bool wide = P.offsets[e + 1] - P.offsets[e] <= GEMM_WIDE_MAX;
        const int nw = wide ? 2 : 1;                        // N tile width in narrow tiles
        const int ntl = wide ? NTW : NT, rows = wide ? 64 : GM_ROWS;
        const int mt = li / ntl, nt = li - mt * ntl;
        const int beg = P.offsets[e] + rows * mt;
        const int end = min(P.offsets[e + 1], beg + rows);
        const uint8_t* blob = P.pool + static_cast<uint64_t>(P.slot_of[e]) * P.slot_bytes;
        const int n0 = (MODE == 0 ? 32 * NQ : 64 * NQ) * nw * nt;
        const int nsub = wide ? wave : nq;                  // this wave's column block of the tile
        const int mbase = wide ? 0 : 64 * mh;               // this wave's first route row of the tile

        // ---- scales of the tile's 256 rows -> LDS (16-byte copies; rows past the matrix read as 0)
        {
            const uint8_t* sblk = blob + o_scales;
            const int half = (MODE == 0 ? 32 * NQ : 64 * NQ) * nw * G * 2;    // bytes of one contiguous row run
            const int nruns = MODE == 0 ? 2 : 1;
            // batches of up to 3 chunks per thread: the loads of a batch, then its stores
            const int nch = nruns * half / 16;
            for (int i0 = 0; i0 < nch; i0 += 3 * NTH) {
                u32x4 v[3];
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int i = i0 + tid + NTH * j;
                    const int run = i / (half / 16), o = (i - run * (half / 16)) * 16;
                    const int r0 = MODE == 0 ? run * P.FF + n0 : n0;            // first matrix row of the run
                    const int64_t src = static_cast<int64_t>(r0) * G * 2 + o;
                    const bool ok = i < nch && src + 16 <= static_cast<int64_t>(S.nrows) * G * 2;
                    v[j] = ok ? *reinterpret_cast<const u32x4*>(sblk + src) : u32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int i = i0 + tid + NTH * j;
                    const int run = i / (half / 16), o = (i - run * (half / 16)) * 16;
                    if (i < nch) *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(ssc) + run * half + o) = v[j];
                }
            }
        }

        // ---- this wave's weight rows and activation rows
        const bool nact = MODE == 0 ? (n0 + 32 * nsub < P.FF) : (n0 + 64 * nsub < P.H);
        const bool mact = beg + mbase < end;
        int wrow[2], lrow[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            if (MODE == 0) {
                const int n = min(n0 + 32 * nsub + c32, P.FF - 1);
                wrow[nb] = nb * P.FF + n;
                lrow[nb] = 32 * NQ * nw * nb + 32 * nsub + c32;
            } else {
                wrow[nb] = min(n0 + 64 * nsub + 32 * nb + c32, P.H - 1);
                lrow[nb] = 64 * nsub + 32 * nb + c32;
            }
        }
        // codes in the blob's tiled layout: group g of the lane's row 1 KB * g further
        const uint8_t* wp0 = blob + o_codes + int4_code_off(wrow[0], G, 16 * hh);
        const uint8_t* wp1 = blob + o_codes + int4_code_off(wrow[1], G, 16 * hh);
        // Register staging (8-wave workgroups): a stage is [group][K step s]
        // [route block] 1 KB fragment blocks; wave w copies (group gi, K step s) =
        // (w >> 2, w & 3) of the 4 route blocks.  Rows past the tile (and blocks
        // 2, 3 of a wide tile) read zeros without a memory access.
        const int sgi = wave >> 2, ss = wave & 3;
        const rsrc_t ares = make_rsrc(abase, static_cast<uint32_t>(asum_rows) * arow_stride * 2);
        uint32_t aoff[4];
#pragma unroll
        for (int mb4 = 0; mb4 < 4; ++mb4) {
            const int p = beg + 32 * mb4 + c32;
            const bool ok = p < end && (!wide || mb4 < 2);
            const int r = ok ? (MODE == 0 ? P.sorted_route[p] / P.k : p) : 0;
            aoff[mb4] = ok ? static_cast<uint32_t>((r * arow_stride + 16 * ss + 8 * hh) * 2) : NO_LANE;
        }
        // LDS DMA staging (4-wave workgroups): a stage is [128 tile rows][128 B]
        // (one 64-group of K), the 16-byte chunk j of row R at position
        // j ^ swz(R), swz(R) = (R & 7) ^ ((R >> 3) & 3): fragment reads of 8 or 16
        // consecutive rows hit distinct banks.  Wave w copies rows 32 w .. 32 w + 31,
        // 8 rows (whole 128-byte lines) per copy: lane l takes row 32 w + 8 i + l / 8,
        // position l % 8.
        uint32_t adm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int R = 32 * (wave & 3) + 8 * i + (lane >> 3);
            const int p = beg + R;
            const bool ok = p < end && (!wide || R < 64);
            const int r = ok ? (MODE == 0 ? P.sorted_route[p] / P.k : p) : 0;
            const int j = (lane & 7) ^ ((lane >> 3) & 7) ^ i;
            adm[i] = ok ? static_cast<uint32_t>((r * arow_stride + 8 * j) * 2) : NO_LANE;
        }
        // fragment (row c32 of a 32-row block, chunk 2 s + hh) in that layout
        uint32_t aro[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) aro[s4] = c32 * 128 + (((2 * s4 + hh) ^ (c32 & 7) ^ ((c32 >> 3) & 3)) * 16);
        auto load_stage = [&](int c, u32x4* xr) {
            const uint32_t g = static_cast<uint32_t>(min(SG * c + sgi, G - 1)) * 128;
#pragma unroll
            for (int mb4 = 0; mb4 < 4; ++mb4) xr[mb4] = bload16(ares, aoff[mb4] + g);
        };
        auto store_stage = [&](int buf, const u32x4* xr) {
#pragma unroll
            for (int mb4 = 0; mb4 < 4; ++mb4)
                *reinterpret_cast<u32x4*>(xbuf + buf * XBUF + ((sgi * 4 + ss) * 4 + mb4) * 1024 + lane * 16) = xr[mb4];
        };
        // the same copy by LDS DMA: 4 loads per wave straight into the stage
        // buffer (each writes 64 lanes x 16 bytes, the block layout above);
        // lanes past the tile write zeros
        auto dma_stage = [&](int c, int buf) {
            const uint32_t g = static_cast<uint32_t>(min(SG * c + sgi, G - 1)) * 128;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ares, reinterpret_cast<__attribute__((address_space(3))) void*>(
                              reinterpret_cast<uintptr_t>(xbuf + buf * XBUF + (32 * (wave & 3) + 8 * i) * 128)),
                    16, adm[i], g, 0, 0);
        };

        // Load order = order of need, as in the K loop below (stage c + 1, then
        // the last two groups of the ring), so that the in-order load counter
        // gives the same waits on the first pass as on later ones.
        u32x4 xr[4];
        if (!XD) load_stage(0, xr);
        u32x4 wr[D][2];
        auto fill = [&](int d) {
            const int g = min(d, G - 1);
            wr[d][0] = *reinterpret_cast<const u32x4*>(wp0 + 1024 * g);
            wr[d][1] = *reinterpret_cast<const u32x4*>(wp1 + 1024 * g);
        };
#pragma unroll
        for (int d = 0; d < D - 2; ++d) fill(d);
        if (!XD) store_stage(0, xr);
        __syncthreads();   // scales (and stage 0) in LDS

        // ---- bias of the expanded codes: acc = -136 * sum_g X[m][g] s[n][g]
        f32x16 acc[2][2];
        {
            const f32x16 z = {};
            f32x16 corr[2][2] = {{z, z}, {z, z}};
            for (int t = 0; t < GP / 16; ++t) {
                u32x4 bs[2];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const uint16_t* sr = ssc + lrow[nb] * G;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int g0 = 16 * t + 8 * hh + 2 * j;
                        const uint32_t a = g0 < G ? sr[g0] : 0u, b = g0 + 1 < G ? sr[g0 + 1] : 0u;
                        bs[nb][j] = a | (b << 16);
                    }
                }
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int p = min(beg + mbase + 32 * mb + c32, end - 1);
                    const int r = MODE == 0 ? P.sorted_route[p] / P.k : p;
                    const uint16_t* sh = asum + static_cast<int64_t>(r) * GP + 16 * t + 8 * hh;
                    const uint16_t* sl = sh + static_cast<int64_t>(asum_rows) * GP;
                    u32x4 ah = *reinterpret_cast<const u32x4*>(sh), al = *reinterpret_cast<const u32x4*>(sl);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {   // groups past G: zero (the padding is not trusted)
                        const int g0 = 16 * t + 8 * hh + 2 * j;
                        const uint32_t m = g0 >= G ? 0u : (g0 + 1 >= G ? 0x0000FFFFu : 0xFFFFFFFFu);
                        ah[j] &= m;
                        al[j] &= m;
                    }
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        corr[mb][nb] = mfma32(ah, bs[nb], corr[mb][nb]);
                        corr[mb][nb] = mfma32(al, bs[nb], corr[mb][nb]);
                    }
                }
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = corr[mb][nb] * -136.0f;
        }
        if (XD) {
            // stage 0, weight group D - 2, stage 1, weight group D - 1: the
            // same order as in the loop, so each chunk's wait below is exact
            dma_stage(0, 0);
            __builtin_amdgcn_sched_barrier(0);
            fill(D - 2);
            __builtin_amdgcn_sched_barrier(0);
            dma_stage(1, 1);
            __builtin_amdgcn_sched_barrier(0);
            fill(D - 1);
        } else {
            load_stage(1, xr);
            __builtin_amdgcn_sched_barrier(0);   // keep the issue order
            fill(D - 2);
            fill(D - 1);
        }

        // ---- K loop: U chunks per unrolled body
        const int ncu = (NC + U - 1) / U * U;
        int bcur = 0;   // LDS DMA ring: the buffer of stage c is c % 3
        for (int c0 = 0; c0 < ncu; c0 += U) {
#pragma unroll
            for (int cu = 0; cu < U; ++cu) {
                const int c = c0 + cu;
                const uint8_t* xb = xbuf + (XD ? bcur : (cu & 1)) * XBUF;
                if (XD) {
                    // Stage c was requested two chunks ago; after it this wave
                    // issued 8 vector-memory operations (the 2 weight loads of
                    // that chunk, stage c + 1's 4 copies, the next 2 weight
                    // loads; likewise in the prologue), so vmcnt <= 8 means its
                    // copies have landed.  The barrier makes that true for every
                    // wave, and also ends the reads of stage c - 1, whose buffer
                    // stage c + 2 now takes.  (The compiler does not track LDS DMA
                    // completion itself.)
                    __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8), lgkm/exp not waited
                    __builtin_amdgcn_s_barrier();
                    dma_stage(min(c + 2, NC - 1), bcur == 0 ? 2 : bcur - 1);
                } else {
                    // stage c + 1 (loaded one chunk ago) into the other buffer, whose
                    // readers finished at the last barrier; then start stage c + 2,
                    // ahead of this chunk's weight loads so that the in-order load
                    // counter never makes a wait cover weights needed later
                    store_stage((cu + 1) & 1, xr);
                    load_stage(min(c + 2, NC - 1), xr);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int gi = 0; gi < SG; ++gi) {
                    const int g = SG * c + gi;
                    const int slot = (SG * cu + gi) % D;
                    if (nact && mact && g < G) {
                        // K steps software-pipelined: the next step's activation
                        // fragments are read and its weights expanded while this
                        // step's MFMAs run
                        const int mblk = wide ? 0 : 2 * mh;
                        const uint8_t* xa = XD ? xb + mblk * 4096 : xb + (gi * 16 + mblk) * 1024 + lane * 16;
                        const float sc0 = bf16_to_f32(ssc[lrow[0] * G + g]), sc1 = bf16_to_f32(ssc[lrow[1] * G + g]);
                        f32x16 part[2][2];
                        u32x4 a0 = *reinterpret_cast<const u32x4*>(xa + (XD ? aro[0] : 0));
                        u32x4 a1 = *reinterpret_cast<const u32x4*>(xa + (XD ? aro[0] + 4096 : 1024));
                        u32x4 b0 = deq_int4(wr[slot][0][0]), b1 = deq_int4(wr[slot][1][0]);
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            u32x4 na0, na1, nb0, nb1;
                            if (s < 3) {
                                na0 = *reinterpret_cast<const u32x4*>(xa + (XD ? aro[s + 1] : (s + 1) * 4096));
                                na1 = *reinterpret_cast<const u32x4*>(xa + (XD ? aro[s + 1] + 4096 : (s + 1) * 4096 + 1024));
                            }
                            if (s == 0) {
                                const f32x16 z = {};
                                part[0][0] = mfma32(a0, b0, z);
                                part[0][1] = mfma32(a0, b1, z);
                                part[1][0] = mfma32(a1, b0, z);
                                part[1][1] = mfma32(a1, b1, z);
                            } else {
                                part[0][0] = mfma32(a0, b0, part[0][0]);
                                part[0][1] = mfma32(a0, b1, part[0][1]);
                                part[1][0] = mfma32(a1, b0, part[1][0]);
                                part[1][1] = mfma32(a1, b1, part[1][1]);
                            }
                            if (s < 3) {
                                nb0 = deq_int4(wr[slot][0][s + 1]);
                                nb1 = deq_int4(wr[slot][1][s + 1]);
                                a0 = na0;
                                a1 = na1;
                                b0 = nb0;
                                b1 = nb1;
                            }
                        }
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb) {
                            acc[mb][0] += sc0 * part[mb][0];
                            acc[mb][1] += sc1 * part[mb][1];
                        }
                    }
                    // refill the slot with group g + D (past the end: the last group again)
                    const int gn = min(g + D, G - 1);
                    wr[slot][0] = *reinterpret_cast<const u32x4*>(wp0 + 1024 * gn);
                    wr[slot][1] = *reinterpret_cast<const u32x4*>(wp1 + 1024 * gn);
                }
                if (XD)
                    bcur = bcur == 2 ? 0 : bcur + 1;
                else
                    __syncthreads();
            }
        }
        if (XD) {
            // every copy into the ring has landed before the epilogue reuses it
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            __syncthreads();
        }

        // ---- epilogue
        if (MODE == 0) {
            // [128 / nw routes][128 nw columns] bf16, M32 order inside each 64-group
            uint16_t* tile = reinterpret_cast<uint16_t*>(xbuf);
            const int tw = 32 * NQ * nw;
            if (nact && mact) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = mbase + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
                        const int col = 32 * nsub + c32;
                        const float hv = act_fn(P.act, acc[mb][0][v]) * acc[mb][1][v];
                        tile[r * tw + 64 * (col >> 6) + m32_pos(col & 63)] = f32_to_bf16(hv);
                    }
            }
            __syncthreads();
            const int ncol = min(tw, P.FF - n0);
            for (int i = tid; i < 512 * NQ; i += NTH) {   // (128 / nw rows) x (tw / 8 blocks)
                const int r = i / (4 * NQ * nw), c8 = i - r * (4 * NQ * nw);
                if (beg + r < end && 8 * c8 < ncol)
                    *reinterpret_cast<u32x4*>(P.h + static_cast<int64_t>(beg + r) * P.FF + n0 + 8 * c8) =
                        *reinterpret_cast<const u32x4*>(tile + r * tw + 8 * c8);
            }
            {
                // group sums of the stored h: 2 threads per (route row, 64-group)
                const int pr = tid >> 1, hf = tid & 1, r = pr / (NQ * nw / 2), gg = pr - r * (NQ * nw / 2);
                float sum = 0.0f;
                const uint16_t* src = tile + r * tw + 64 * gg + 32 * hf;
#pragma unroll
                for (int j = 0; j < 32; ++j) sum += bf16_to_f32(src[j]);
                sum += __shfl_xor(sum, 1, 64);
                if (hf == 0 && beg + r < end && 64 * gg < ncol) {
                    const int G2 = P.FF / 64, GP2 = (G2 + 15) & ~15, R = P.T * P.k;
                    const uint16_t shi = f32_to_bf16(sum);
                    const int gidx = n0 / 64 + gg;
                    P.hsum[static_cast<int64_t>(beg + r) * GP2 + gidx] = shi;
                    P.hsum[(static_cast<int64_t>(R) + beg + r) * GP2 + gidx] = f32_to_bf16(sum - bf16_to_f32(shi));
                }
            }
        } else if (nact && mact) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int p = beg + mbase + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
                    if (p < end) {
#pragma unroll
                        for (int nb = 0; nb < 2; ++nb) {
                            const int64_t o = static_cast<int64_t>(p) * P.H + n0 + 64 * nsub + 32 * nb + c32;
                            if (P.out_dt == F32)
                                static_cast<float*>(P.out)[o] = acc[mb][nb][v];
                            else
                                static_cast<uint16_t*>(P.out)[o] = f32_to_bf16(acc[mb][nb][v]);
                        }
                    }
                }
        }
        __syncthreads();   // LDS is rewritten by the next item
    }
}

// true if the int4 GEMM path takes this call
bool int4_gemm_eligible(const FfnParams& P) {
    // the tiles handle any H, FF that are multiples of 64 (ragged last N tile,
    // odd group counts); E bounds the prefix table in LDS
    return P.fmt == W_INT4 && P.H % 64 == 0 && P.FF % 64 == 0 && P.E <= 4096;
}

#ifndef GEMM_NW
#define GEMM_NW 4
#endif
hipError_t launch_int4_gemm(const FfnParams& P0, int phases, hipStream_t s) {
    FfnParams P = P0;
    int dev = 0, cus = 0, maxlds = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return err;
    if ((err = hipDeviceGetAttribute(&maxlds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess) return err;
    constexpr int DC0 = 2, DC1 = 3, NW = GEMM_NW;   // weight prefetch depth (2 DC groups) per half
    // persistent: 8 waves per CU, as one workgroup of 8 or two of 4 (which then
    // run out of step with each other)
    const dim3 grid(static_cast<uint32_t>(cus * (8 / NW))), block(64 * NW);
    if (phases & 1) {
        const int64_t nblk = static_cast<int64_t>(P.T) * P.H / 8;
        P.xq = P.xq_out;
        P.xsum = P.xsum_out;
        if (P.x_dt == F32)
            hipLaunchKernelGGL((prep_x_m32_kernel<F32>), dim3(static_cast<uint32_t>((nblk + 255) / 256)), dim3(256), 0, s,
                               P.x, P.T, P.H, P.xq_out, reinterpret_cast<uint16_t*>(P.xsum_out));
        else
            hipLaunchKernelGGL((prep_x_m32_kernel<BF16>), dim3(static_cast<uint32_t>((nblk + 255) / 256)), dim3(256), 0, s,
                               P.x, P.T, P.H, P.xq_out, reinterpret_cast<uint16_t*>(P.xsum_out));
        const size_t lds = gemm_lds_bytes(P.E, P.H / 64, NW);
        if (static_cast<int>(lds) > maxlds) return hipErrorInvalidConfiguration;
        static bool attr = false;
        if (!attr)
            attr = hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_int4_gemm_kernel<0, DC0, NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, maxlds) == hipSuccess;
        hipLaunchKernelGGL((ffn_int4_gemm_kernel<0, DC0, NW>), grid, block, lds, s, P);
    }
    if (phases & 2) {
        const size_t lds = gemm_lds_bytes(P.E, P.FF / 64, NW);
        if (static_cast<int>(lds) > maxlds) return hipErrorInvalidConfiguration;
        static bool attr = false;
        if (!attr)
            attr = hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_int4_gemm_kernel<1, DC1, NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, maxlds) == hipSuccess;
        hipLaunchKernelGGL((ffn_int4_gemm_kernel<1, DC1, NW>), grid, block, lds, s, P);
    }
    return hipGetLastError();
}

}  // namespace moe
