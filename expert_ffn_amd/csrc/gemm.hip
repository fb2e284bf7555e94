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
// CU walk the items (one of 8 waves is a build option).  A group of up to 64
// routes is one route tile, each wave taking all of it (one or two blocks of
// 32 routes) times its own 64 weight rows (two 32-row blocks); a group of 65
// to 96 routes is one three-block tile when the items outnumber the
// workgroups, else a 64-route tile and the rest; a larger group takes
// 128-route tiles, wave (mh, nq) taking routes 64 mh .. 64 mh + 63 times 64
// rows.  Each (route block, row block) pair is a chain of 4 MFMAs per
// 64-group whose partial sum is scaled into the accumulator; with three route
// blocks this happens block by block, so that only two partial tiles are
// live.  The K loop runs over 64-groups: a group's activations
// (a 128-byte piece of each route row of the tile) are copied by LDS DMA two
// groups ahead into a ring of three stages, whole cache lines per copy, XOR
// swizzled in LDS; each wave keeps the weights of the next 2*DC groups in flight
// in registers, one 1 KB load per group and 32 rows from the blob's tiled codes.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
}

// fp32 -> bf16 (round to nearest even) by the gfx950 conversion instruction:
// one VALU where f32_to_bf16 takes five; the two differ only in NaN payloads
__device__ __forceinline__ uint16_t bf16_cvt(float f) { return static_cast<uint16_t>(pack_bf16x2(f, 0.0f)); }

// position of element f (0..63) of a 64-group in the M32 operand order
__host__ __device__ __forceinline__ int m32_pos(int f) {
    const int h = f >> 5, s = (f >> 3) & 3, e = f & 7;
    return 16 * s + 8 * h + (((e & 3) << 1) | (e >> 2));   // slot j with perm8(j) = e
}

constexpr int GM_ROWS = 128;   // routes per narrow tile
// Groups of at most GEMM_WIDE_MAX routes take one wide tile (all the group's
// routes, up to three 32-route blocks per wave, and an N tile twice as wide:
// less activation traffic per weight byte); larger ones take 128-route
// narrow tiles.
#ifndef GEMM_WIDE_MAX
#define GEMM_WIDE_MAX 96
#endif
static_assert(GEMM_WIDE_MAX > 64 && GEMM_WIDE_MAX <= 96, "a wide tile holds at most three 32-route blocks per wave");
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
           static_cast<size_t>(E + 1) * 20;   // prefix arrays [3][E+1], offsets [E+1], slots [E]
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
    int* pre = reinterpret_cast<int*>(lds + NSTG * XBUF + ((NTH * G * 2 + 15) & ~15));   // [3][E+1]
    int* offs = pre + 3 * (E + 1);    // [E+1] group offsets, copied by the prefix pass
    int* slots = offs + (E + 1);      // [E] expert slots, likewise
    // the wave index as a scalar: the LDS DMA copies take wave-derived offsets
    // in SGPRs and M0, which the compiler must know to be uniform (else each
    // copy becomes a loop over the lanes' values)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, c32 = lane & 31,
              hh = lane >> 5;
    const int mh = wave / NQ, nq = wave % NQ;

    // Items: (expert, row tile, N tile).  A group of at most GEMM_WIDE_MAX
    // routes takes "wide" row tiles of up to 64 routes: every wave takes all
    // the tile's routes (MB = 1 or 2 blocks of 32), and the four waves take
    // different columns (an N tile twice as wide as a narrow one).  Larger
    // groups take 128-route narrow tiles, the two wave halves splitting the
    // routes (two blocks each).  When those items outnumber the workgroups, a
    // group of 65 to 96 routes takes one three-block tile instead of two
    // ("class A": one item of about 1.35 times the time of the others, in
    // place of two); with fewer items the two tiles run side by side and the
    // split is faster.  Groups of at most 32 routes are one-block tiles
    // ("class C", about 0.6 of a two-block item: half the MFMAs and scaling).
    // Class-A items are listed first, class C last: pre / preB / preC are
    // per-expert prefix sums of the three classes' item counts (wave 0).
    // Measured per layer at T = 1024 (gate/up + down): 146 + 87 -> 131 + 79 us
    // under uniform routing; Zipf routing (few such groups) and T = 128 to 512
    // unchanged within 3 us.
    const int NTW = MODE == 0 ? (P.FF + 32 * NW - 1) / (32 * NW) : (P.H + 64 * NW - 1) / (64 * NW);
    int* preB = pre + (E + 1);
    int* preC = pre + 2 * (E + 1);
    // items of a group of me routes with 64-route wide tiles (groups of at
    // most gmin routes are the streaming kernels')
    auto split_items = [&](int me) {
        return me <= P.gmin ? 0 : (me <= GEMM_WIDE_MAX ? (me + 63) / 64 * NTW : (me + GM_ROWS - 1) / GM_ROWS * NT);
    };
    if (wave == 0) {
        // one round of global loads: the group sizes wait in pre[] for the
        // second pass, which overwrites each entry after reading it; the
        // offsets and slots stay in LDS for the items' headers
        int tot = 0, elig = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int o0 = e < E ? P.offsets[e] : 0, o1 = e < E ? P.offsets[e + 1] : 0;
            const int sl = e < E ? P.slot_of[e] : 0;
            const int me = o1 - o0;
            if (e < E) {
                pre[e + 1] = me;
                offs[e] = o0;
                slots[e] = sl;
                if (e == E - 1) offs[E] = o1;
            }
            int c = split_items(me), ce = me > 64 && me <= GEMM_WIDE_MAX ? c : 0;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                c += __shfl_xor(c, d, 64);
                ce += __shfl_xor(ce, d, 64);
            }
            tot += c;
            elig += ce;
        }
        // merge when the split items outnumber the workgroups and the groups
        // of 65-96 routes hold at least a quarter of them (a few three-block
        // items among many others lengthen the rounds they fall in)
        const bool merge = tot > static_cast<int>(gridDim.x) && 4 * elig >= tot;
        int runA = 0, runB = 0, runC = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int me = e < E ? pre[e + 1] : 0;
            const bool three = merge && me > 64 && me <= GEMM_WIDE_MAX, one = me <= 32;
            const int cnt = three ? NTW : split_items(me);
            int ia = three ? cnt : 0, ic = one ? cnt : 0, ib = cnt - ia - ic;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int oa = __shfl_up(ia, d, 64), ob = __shfl_up(ib, d, 64), oc = __shfl_up(ic, d, 64);
                if (lane >= d) {
                    ia += oa;
                    ib += ob;
                    ic += oc;
                }
            }
            if (e < E) {
                pre[e + 1] = runA + ia;
                preB[e + 1] = runB + ib;
                preC[e + 1] = runC + ic;
            }
            runA += __shfl(ia, 63, 64);
            runB += __shfl(ib, 63, 64);
            runC += __shfl(ic, 63, 64);
        }
        if (lane == 0) pre[0] = preB[0] = preC[0] = 0;
    }
    __syncthreads();
    const int nA = pre[E], nB = preB[E], nC = preC[E];

    const uint64_t o_codes = MODE == 0 ? P.o13 : P.o2, o_scales = MODE == 0 ? P.os13 : P.os2;
    const int arow_stride = MODE == 0 ? P.H : P.FF;                 // elements per A row
    const uint16_t* abase = MODE == 0 ? P.xq : P.h;
    const uint16_t* asum = MODE == 0 ? reinterpret_cast<const uint16_t*>(P.xsum) : P.hsum;
    const int asum_rows = MODE == 0 ? P.T : P.T * P.k;

    // XCD-aware order: workgroups are dealt to the 8 XCDs round robin, so the
    // workgroups of one XCD (blockIdx % 8) take one contiguous eighth of each
    // class's item list, class A first.  An expert's N tiles then mostly run
    // on one XCD and its activation rows are fetched into that XCD's L2 once.
    // Inside an XCD workgroup j takes position r W + j in round r; for gate/up
    // with class-A items the odd rounds run backwards (r W + W - 1 - j), so
    // that the workgroups which started with a class-A item take their next
    // item last (measured: 133 -> 126 us per gate/up layer at T = 1024; down,
    // with 11 N tiles per expert and nearly 3 items per workgroup, is 2.5 us
    // faster without it, and so is gate/up without class-A items).
    // (A mapping of workgroups to XCDs that differs only costs locality: every
    // item is still taken once.)
    const int nxcd = gridDim.x % 8 == 0 ? 8 : 1;
    const int xcd = blockIdx.x % nxcd, wpx = gridDim.x / nxcd, wj = blockIdx.x / nxcd;
    const int a0i = static_cast<int>(static_cast<int64_t>(nA) * xcd / nxcd);
    const int na = static_cast<int>(static_cast<int64_t>(nA) * (xcd + 1) / nxcd) - a0i;
    const int b0i = static_cast<int>(static_cast<int64_t>(nB) * xcd / nxcd);
    const int nb = static_cast<int>(static_cast<int64_t>(nB) * (xcd + 1) / nxcd) - b0i;
    const int c0i = static_cast<int>(static_cast<int64_t>(nC) * xcd / nxcd);
    const int nmine = na + nb + static_cast<int>(static_cast<int64_t>(nC) * (xcd + 1) / nxcd) - c0i;
    const bool snake = MODE == 0 && nA > 0;
    // One item at list position pos.  MBC = the route blocks its K loop
    // computes: 3 for class A, 2 for class B (a second tile of at most 32
    // routes computes a second block of zero rows), 1 for class C.  The
    // classes are three inlined copies of the whole item, run one after the
    // other, so that no large state is live across a branch between K loops
    // (with the choice made per item, the register allocator spilled).
    auto do_item = [&](auto mbc, int pos) {
        constexpr int MBC = decltype(mbc)::value;
        constexpr bool inA = MBC == 3;
        const int item = inA ? a0i + pos : (MBC == 2 ? b0i + pos - na : c0i + pos - na - nb);
        const int* pc = inA ? pre : (MBC == 2 ? preB : preC);
        int lo = 0, hi = E;   // largest e with pc[e] <= item
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pc[mid] <= item) lo = mid; else hi = mid;
        }
        const int e = lo, li = item - pc[e];
        const int o0 = offs[e], o1 = offs[e + 1];
        const int me = o1 - o0;
        const bool wide = me <= GEMM_WIDE_MAX;
        const int nw = wide ? 2 : 1;                        // N tile width in narrow tiles
        const int ntl = wide ? NTW : NT;
        const int mt = li / ntl, nt = li - mt * ntl;
        const int rows = wide ? (inA ? 96 : 64) : GM_ROWS;  // route rows of the tile
        const int beg = o0 + rows * mt;
        const int end = min(o1, beg + rows);
        const int MB = MBC == 2 ? (wide ? (end - beg + 31) / 32 : 2) : MBC;   // route blocks of each wave (uniform)
        const uint8_t* blob = P.pool + static_cast<uint64_t>(slots[e]) * P.slot_bytes;
        const int n0 = (MODE == 0 ? 32 * NQ : 64 * NQ) * nw * nt;
        // the tile's route indices (gate/up), requested together before the
        // scales, as tokens: rows beg + 32 mb4 + c32 (bias, register staging)
        // and the LDS DMA rows; rows past the group read the group's last route
        int srt[4], srd[4];
        if (MODE == 0) {
#pragma unroll
            for (int mb4 = 0; mb4 < 4; ++mb4) srt[mb4] = P.sorted_route[min(beg + 32 * mb4 + c32, end - 1)];
            if (XD) {
#pragma unroll
                for (int i = 0; i < 4; ++i) srd[i] = P.sorted_route[min(beg + 32 * (wave & 3) + 8 * i + (lane >> 3), end - 1)];
            }
            // routes -> tokens (a multiply, not a division by k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                srt[i] = route_token(srt[i], P.kmul, P.k);
                if (XD) srd[i] = route_token(srd[i], P.kmul, P.k);
            }
        }
        const int nsub = wide ? wave : nq;                  // this wave's column block of the tile
        const int mbase = wide ? 0 : 64 * mh;               // this wave's first route row of the tile
        // ---- scales of the tile's 256 rows -> LDS (16-byte copies; rows past
        // the matrix read as 0): the first batch of loads now, its stores after
        // the bias and weight requests below, so that one wait covers them
        const uint8_t* sblk = blob + o_scales;
        const int shalf = (MODE == 0 ? 32 * NQ : 64 * NQ) * nw * G * 2;   // bytes of one contiguous row run
        const int cpr = shalf / 16, nch = (MODE == 0 ? 2 : 1) * cpr;   // chunks per run, in all
        constexpr int SB = MODE == 0 ? 6 : 2;   // chunks per thread and batch (one batch at the Gemma shapes)
        // chunk i (< nch) of the tile: run i / cpr, byte 16 (i % cpr) of it;
        // chunks past the matrix (or the tile) read as 0 without a memory access
        const rsrc_t sres = make_rsrc(sblk, static_cast<uint32_t>(S.nrows) * G * 2);
        auto scale_src = [&](int i) {
            const int run = MODE == 0 && i >= cpr ? 1 : 0;   // (i < 2 cpr)
            const int r0 = MODE == 0 ? run * P.FF + n0 : n0;  // first matrix row of the run
            const int src = r0 * G * 2 + (i - run * cpr) * 16;
            return i < nch && src + 16 <= S.nrows * G * 2 ? static_cast<uint32_t>(src) : NO_LANE;
        };
        u32x4 sv[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) sv[j] = bload16(sres, scale_src(tid + NTH * j));
        // the LDS copy is contiguous: chunk i at byte 16 i
        auto scale_stores = [&]() {
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int i = tid + NTH * j;
                if (i < nch) *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(ssc) + 16 * i) = sv[j];
            }
            for (int i = SB * NTH + tid; i < nch; i += NTH)   // shapes beyond one batch
                *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(ssc) + 16 * i) = bload16(sres, scale_src(i));
        };

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
        // (w >> 2, w & 3) of the 4 route blocks.  Rows past the group read zeros
        // without a memory access.
        const int sgi = wave >> 2, ss = wave & 3;
        const rsrc_t ares = make_rsrc(abase, static_cast<uint32_t>(asum_rows) * arow_stride * 2);
        uint32_t aoff[4];
#pragma unroll
        for (int mb4 = 0; mb4 < 4; ++mb4) {
            const int p = beg + 32 * mb4 + c32;
            const bool ok = p < end;
            const int r = MODE == 0 ? srt[mb4] : p;
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
            const bool ok = p < end;
            const int r = MODE == 0 ? srd[i] : p;
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
        // group sums of the bias for 16-group step t: the rows of the wave's
        // MBC blocks, clamped to the group
        const int GPT = GP / 16;
        auto bias_loads = [&](int t, u32x4* h, u32x4* l) {
#pragma unroll
            for (int mb = 0; mb < MBC; ++mb) {
                const int sb = (wide ? 0 : 2 * mh) + mb;   // the block's index among srt
                const int r = MODE == 0 ? (sb == 0 ? srt[0] : sb == 1 ? srt[1] : sb == 2 ? srt[2] : srt[3])
                                        : min(beg + mbase + 32 * mb + c32, end - 1);
                const uint16_t* sh = asum + static_cast<int64_t>(r) * GP + 16 * t + 8 * hh;
                h[mb] = *reinterpret_cast<const u32x4*>(sh);
                l[mb] = *reinterpret_cast<const u32x4*>(sh + static_cast<int64_t>(asum_rows) * GP);
            }
        };
        u32x4 ah[MBC], al[MBC];
        bias_loads(0, ah, al);
#pragma unroll
        for (int d = 0; d < D - 2; ++d) fill(d);
        scale_stores();
        if (!XD) store_stage(0, xr);
        __syncthreads();   // scales (and stage 0) in LDS

        // ---- bias of the expanded codes: acc = -136 * sum_g X[m][g] s[n][g]
        // (acc[mb][nb] for the wave's MB route blocks; the group sums of all
        // MBC blocks are loaded from clamped rows, the MFMAs run for mb < MB)
        f32x16 acc[MBC][2];
        {
            const f32x16 z = {};
#pragma unroll
            for (int mb = 0; mb < MBC; ++mb) acc[mb][0] = acc[mb][1] = z;
#pragma unroll 1
            for (int t = 0; t < GPT; ++t) {
                u32x4 nh[MBC], nl[MBC];
                if (t + 1 < GPT) bias_loads(t + 1, nh, nl);   // the next step's, one step ahead
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
                for (int mb = 0; mb < MBC; ++mb) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {   // groups past G: zero (the padding is not trusted)
                        const int g0 = 16 * t + 8 * hh + 2 * j;
                        const uint32_t m = g0 >= G ? 0u : (g0 + 1 >= G ? 0x0000FFFFu : 0xFFFFFFFFu);
                        ah[mb][j] &= m;
                        al[mb][j] &= m;
                    }
                    if (mb < MB) {
#pragma unroll
                        for (int nb = 0; nb < 2; ++nb) {
                            acc[mb][nb] = mfma32(ah[mb], bs[nb], acc[mb][nb]);
                            acc[mb][nb] = mfma32(al[mb], bs[nb], acc[mb][nb]);
                        }
                    }
                }
#pragma unroll
                for (int mb = 0; mb < MBC; ++mb) {
                    ah[mb] = nh[mb];
                    al[mb] = nl[mb];
                }
            }
#pragma unroll
            for (int mb = 0; mb < MBC; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = acc[mb][nb] * -136.0f;
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

        // ---- K loop, U chunks per unrolled body, for MBC route blocks
        int bcur = 0;   // LDS DMA ring: the buffer of stage c is c % 3
        auto kloop = [&](auto) {
            const int ncu = (NC + U - 1) / U * U;
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
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
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
                            const int mblk = wide ? 0 : 2 * mh;
                            const uint8_t* xa = XD ? xb + mblk * 4096 : xb + (gi * 16 + mblk) * 1024 + lane * 16;
                            const float sc0 = bf16_to_f32(ssc[lrow[0] * G + g]), sc1 = bf16_to_f32(ssc[lrow[1] * G + g]);
                            if constexpr (MBC == 2) {
                                // two route blocks: all four chains per K step, the next
                                // step's activation fragments read and its weights
                                // expanded while this step's MFMAs run; then the scaling
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
                            } else {
                                // three route blocks: the group's weights expanded once,
                                // then per block two chains of 4 MFMAs scaled into the
                                // accumulators as soon as they end
                                u32x4 bq[2][4];
    #pragma unroll
                                for (int s = 0; s < 4; ++s) {
                                    bq[0][s] = deq_int4(wr[slot][0][s]);
                                    bq[1][s] = deq_int4(wr[slot][1][s]);
                                }
    #pragma unroll
                                for (int mb = 0; mb < MBC; ++mb) {
                                    // fragment (route block mb, K step s)
                                    auto afrag = [&](int s) {
                                        return *reinterpret_cast<const u32x4*>(
                                            XD ? xa + mb * 4096 + aro[s] : xa + s * 4096 + mb * 1024);
                                    };
                                    u32x4 a = afrag(0);
                                    const f32x16 z = {};
                                    f32x16 p0 = z, p1 = z;
    #pragma unroll
                                    for (int s = 0; s < 4; ++s) {
                                        u32x4 na;
                                        if (s < 3) na = afrag(s + 1);
                                        p0 = mfma32(a, bq[0][s], p0);
                                        p1 = mfma32(a, bq[1][s], p1);
                                        if (s < 3) a = na;
                                    }
                                    acc[mb][0] += sc0 * p0;
                                    acc[mb][1] += sc1 * p1;
                                }
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
        };
        kloop(mbc);
        if (XD) {
            // every copy into the ring has landed before the epilogue reuses it
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __syncthreads();
        }

        // ---- epilogue
        if (MODE == 0) {
            // [tile rows][128 nw columns] bf16, M32 order inside each 64-group;
            // tile rows: 32 MB (wide) or 128 (narrow)
            uint16_t* tile = reinterpret_cast<uint16_t*>(xbuf);
            const int tw = 32 * NQ * nw, trows = wide ? 32 * MB : GM_ROWS;
            if (nact && mact) {
#pragma unroll
                for (int mb = 0; mb < MBC; ++mb) {
                    if (mb < MB) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int r = mbase + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
                            const int col = 32 * nsub + c32;
                            const float hv = act_fn(P.act, acc[mb][0][v]) * acc[mb][1][v];
                            tile[r * tw + 64 * (col >> 6) + m32_pos(col & 63)] = bf16_cvt(hv);
                        }
                    }
                }
            }
            __syncthreads();
            const int ncol = min(tw, P.FF - n0);
            for (int i = tid; i < trows * (tw / 8); i += NTH) {   // trows x (tw / 8 blocks)
                const int r = i / (tw / 8), c8 = i - r * (tw / 8);
                if (beg + r < end && 8 * c8 < ncol)
                    *reinterpret_cast<u32x4*>(P.h + static_cast<int64_t>(beg + r) * P.FF + n0 + 8 * c8) =
                        *reinterpret_cast<const u32x4*>(tile + r * tw + 8 * c8);
            }
            // group sums of the stored h: 2 threads (adjacent lanes) per (route
            // row, 64-group); trows * tw / 32 is a multiple of 64, so every
            // wave runs the same number of passes
            for (int i0 = 0; i0 < trows * (tw / 32); i0 += NTH) {
                const int i = i0 + tid;
                const int pr = i >> 1, hf = i & 1, r = pr / (tw / 64), gg = pr - r * (tw / 64);
                float sum = 0.0f;
                if (r < trows) {
                    const uint16_t* src = tile + r * tw + 64 * gg + 32 * hf;
#pragma unroll
                    for (int j = 0; j < 32; ++j) sum += bf16_to_f32(src[j]);
                }
                sum += __shfl_xor(sum, 1, 64);
                if (hf == 0 && r < trows && beg + r < end && 64 * gg < ncol) {
                    const int G2 = P.FF / 64, GP2 = (G2 + 15) & ~15, R = P.T * P.k;
                    const uint16_t shi = f32_to_bf16(sum);
                    const int gidx = n0 / 64 + gg;
                    P.hsum[static_cast<int64_t>(beg + r) * GP2 + gidx] = shi;
                    P.hsum[(static_cast<int64_t>(R) + beg + r) * GP2 + gidx] = f32_to_bf16(sum - bf16_to_f32(shi));
                }
            }
        } else if (NW == 4 && P.out_dt != F32) {
            // bf16 rows of out: the tile [tile rows][64 NQ nw columns] (at most
            // 96 x 256, 48 KB) through LDS (the activation ring is free), then
            // 16-byte stores along the rows; per-element 2-byte stores cost down
            // about a fifth of its time
            uint16_t* tile = reinterpret_cast<uint16_t*>(xbuf);
            const int tw = 64 * NQ * nw, trows = wide ? 32 * MB : GM_ROWS;
            if (nact && mact) {
#pragma unroll
                for (int mb = 0; mb < MBC; ++mb) {
                    if (mb < MB) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int r = mbase + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
#pragma unroll
                            for (int nb = 0; nb < 2; ++nb)
                                tile[r * tw + 64 * nsub + 32 * nb + c32] = bf16_cvt(acc[mb][nb][v]);
                        }
                    }
                }
            }
            __syncthreads();
            const int ncol = min(tw, P.H - n0);
            for (int i = tid; i < trows * (tw / 8); i += NTH) {
                const int r = i / (tw / 8), c8 = i - r * (tw / 8);
                if (beg + r < end && 8 * c8 < ncol)
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(P.out) + static_cast<int64_t>(beg + r) * P.H + n0 + 8 * c8) =
                        *reinterpret_cast<const u32x4*>(tile + r * tw + 8 * c8);
            }
        } else if (nact && mact) {
#pragma unroll
            for (int mb = 0; mb < MBC; ++mb) {
                if (mb < MB) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int p = beg + mbase + 32 * mb + 8 * (v >> 2) + 4 * hh + (v & 3);
                        if (p < end) {
#pragma unroll
                            for (int nb = 0; nb < 2; ++nb)
                                static_cast<float*>(P.out)[static_cast<int64_t>(p) * P.H + n0 + 64 * nsub + 32 * nb + c32] =
                                    acc[mb][nb][v];
                        }
                    }
                }
            }
        }
        __syncthreads();   // LDS is rewritten by the next item
    };
    // the classes' positions come in list order in every workgroup's
    // sequence (a workgroup's positions grow with the round)
    int rnd = 0;
    for (;; ++rnd) {
        const int pos = rnd * wpx + ((snake && (rnd & 1)) ? wpx - 1 - wj : wj);
        if (pos >= na) break;
        do_item(std::integral_constant<int, 3>{}, pos);
    }
    for (;; ++rnd) {
        const int pos = rnd * wpx + ((snake && (rnd & 1)) ? wpx - 1 - wj : wj);
        if (pos >= na + nb) break;
        do_item(std::integral_constant<int, 2>{}, pos);
    }
    for (;; ++rnd) {
        const int pos = rnd * wpx + ((snake && (rnd & 1)) ? wpx - 1 - wj : wj);
        if (pos >= nmine) break;   // every later round's positions are larger
        do_item(std::integral_constant<int, 1>{}, pos);
    }
}

#ifndef GEMM_NW
#define GEMM_NW 4
#endif

// LDS the device allows a workgroup, per device (queried once)
static int max_lds_bytes() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// true if the int4 GEMM can take this call's large groups: the tiles handle
// any H, FF that are multiples of 64 (ragged last N tile, odd group counts);
// E bounds the prefix table, and both halves' LDS must fit (checked here, so
// that nothing is launched when it does not)
bool int4_gemm_eligible(const FfnParams& P) {
    if (P.fmt != W_INT4 || P.H % 64 || P.FF % 64 || P.E > 4096) return false;
    const size_t lim = static_cast<size_t>(max_lds_bytes());
    return gemm_lds_bytes(P.E, P.H / 64, GEMM_NW) <= lim && gemm_lds_bytes(P.E, P.FF / 64, GEMM_NW) <= lim;
}

hipError_t launch_int4_gemm(const FfnParams& P0, int phases, hipStream_t s) {
    FfnParams P = P0;
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return err;
    const int maxlds = max_lds_bytes();
    constexpr int DC0 = 2, DC1 = 2, NW = GEMM_NW;   // weight prefetch depth (2 DC groups) per half
    // persistent: 8 waves per CU, as one workgroup of 8 or two of 4 (which then
    // run out of step with each other)
    const dim3 grid(static_cast<uint32_t>(cus * (8 / NW))), block(64 * NW);
    if (phases & 1) {
        const int64_t nblk = static_cast<int64_t>(P.T) * P.H / 8;
        P.xq = P.xqg_out;
        P.xsum = reinterpret_cast<float*>(P.xsumg_out);
        if (P.x_dt == F32)
            hipLaunchKernelGGL((prep_x_m32_kernel<F32>), dim3(static_cast<uint32_t>((nblk + 255) / 256)), dim3(256), 0, s,
                               P.x, P.T, P.H, P.xqg_out, P.xsumg_out);
        else
            hipLaunchKernelGGL((prep_x_m32_kernel<BF16>), dim3(static_cast<uint32_t>((nblk + 255) / 256)), dim3(256), 0, s,
                               P.x, P.T, P.H, P.xqg_out, P.xsumg_out);
        const size_t lds = gemm_lds_bytes(P.E, P.H / 64, NW);
        static bool attr = false;
        if (!attr)
            attr = hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_int4_gemm_kernel<0, DC0, NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, maxlds) == hipSuccess;
        hipLaunchKernelGGL((ffn_int4_gemm_kernel<0, DC0, NW>), grid, block, lds, s, P);
    }
    if (phases & 2) {
        const size_t lds = gemm_lds_bytes(P.E, P.FF / 64, NW);
        static bool attr = false;
        if (!attr)
            attr = hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_int4_gemm_kernel<1, DC1, NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, maxlds) == hipSuccess;
        hipLaunchKernelGGL((ffn_int4_gemm_kernel<1, DC1, NW>), grid, block, lds, s, P);
    }
    return hipGetLastError();
}

}  // namespace moe
