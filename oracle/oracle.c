/*
 * oracle.c -- plain, slow CPU oracle of one MoE layer's routed expert FFN.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg load this library.  It shares no source,
 * header, table or helper with the HIP library under expert_ffn_amd/csrc, and
 * it never reads anything that library produced.
 *
 * Every routine is the plain definition of its step, written out with scalar
 * loops: fp32 storage, fp64 accumulation, no blocking, no fusion, no reordering.
 * It is compiled with -O2 -ffp-contract=off (no FMA contraction, no fast-math),
 * so every fp32/fp64 operation below is one IEEE-754 operation rounded to
 * nearest-even, exactly as written.
 *
 * Sources (titles of the pages the method is taken from):
 *   [prain]  prain/README.md -- sections "Expert formats", "int4 experts on
 *            RDNA2", "Trading quality for speed", "Profile".
 *   [rlx]    rlx_runtime/expert_pool.rs (docs.rs, rlx-runtime 0.2.2) --
 *            count_hits, target_gpu_from_counts, apply_target_placement and
 *            their unit tests.
 *   [strata] Winery-Strata src/core/remote_experts.cpp -- RemoteExperts::begin
 *            and RemoteExperts::finish.
 * Where the pages leave a step open, the reading taken is stated at the
 * routine that implements it.
 *
 * Parity pins: every routine here is pinned by the CPU tests in tests/ against
 * brute force, closed forms, library routines or the numbers the pages print.
 * No routine is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_OK 0
#define ORA_EARG 1

enum { ORA_W_BF16 = 0, ORA_W_INT8_ROW = 1, ORA_W_INT4_G64 = 2 };
enum { ORA_ACT_GELU_TANH = 0, ORA_ACT_SILU = 1 };

/* ------------------------------------------------------------------ bf16 --
 * bf16 is the upper half of an fp32 bit pattern.  Widening is exact.
 * Narrowing is round-to-nearest, ties to the even bf16 (the IEEE default;
 * the pages never state a rounding mode).  NaN becomes the quiet NaN 0x7FC0.
 */
static float bf16_bits_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return 0x7FC0;
    uint32_t lo = u >> 16;          /* the candidate below (truncation)      */
    uint32_t rem = u & 0xFFFFu;     /* the discarded lower 16 bits           */
    if (rem > 0x8000u) return (uint16_t)(lo + 1);   /* above half: round up  */
    if (rem < 0x8000u) return (uint16_t)lo;         /* below half: truncate  */
    return (uint16_t)((lo & 1u) ? lo + 1 : lo);     /* tie: to even          */
}

void oracle_f32_to_bf16(const float* src, uint16_t* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = f32_to_bf16_bits(src[i]);
}

void oracle_bf16_to_f32(const uint16_t* src, float* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = bf16_bits_to_f32(src[i]);
}

/* ------------------------------------------------------------- routing --
 * Router top-k ([prain] "Trading quality for speed": each token has a router
 * weight spread over its experts; [strata] RemoteExperts::begin: k routes per
 * token, route i belongs to token i / k).
 *
 * Order of experts for one token: larger logit first; equal logits go to the
 * lower expert id first (the tie rule of [rlx] target_gpu_from_counts and its
 * test "tie-break: lower expert id first").  NaN ranks below every number,
 * -0 and +0 are equal.  ids are written in rank order.
 *
 * Weights: softmax.  With renorm = 1 the softmax over all E experts is
 * renormalised over the chosen k, which equals the softmax over the chosen k
 * logits: w_j = exp(l_j - m) / sum_{i<k} exp(l_i - m), m = the top logit.
 * With renorm = 0 the denominator runs over all E logits.  fp64, stored fp32.
 */
static int logit_above(float a, float b)
{
    if (isnan(a)) return 0;
    if (isnan(b)) return 1;
    return a > b;
}

int oracle_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                      int32_t* ids, float* w)
{
    if (!logits || !ids || !w || T < 0 || E < 1 || k < 1 || k > E) return ORA_EARG;
    char* taken = (char*)malloc((size_t)E);
    for (int32_t t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                /* scanning e upward and replacing only on a strictly better
                   logit keeps the lower id on ties */
                if (best < 0 || logit_above(l[e], l[best])) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        const double m = (double)l[ids[(int64_t)t * k]];
        double den = 0.0;
        if (renorm) {
            for (int32_t j = 0; j < k; ++j) den += exp((double)l[ids[(int64_t)t * k + j]] - m);
        } else {
            for (int32_t e = 0; e < E; ++e) den += exp((double)l[e] - m);
        }
        for (int32_t j = 0; j < k; ++j)
            w[(int64_t)t * k + j] = (float)(exp((double)l[ids[(int64_t)t * k + j]] - m) / den);
    }
    free(taken);
    return ORA_OK;
}

/* ----------------------------------------------------------- permutation --
 * Grouping routes by expert ([strata] RemoteExperts::begin builds, per expert
 * group, the list of its routes in route order, each with token i / k;
 * [rlx] count_hits is the per-expert histogram, ignoring ids out of range).
 *
 * A route i = t*k + j is kept when 0 <= ids[i] < E and slot_of[ids[i]] >= 0
 * (the expert is resident); otherwise it is dropped and counted.
 * Groups are in expert-id order; inside a group routes keep ascending i.
 *   counts[e]      = number of kept routes with ids[i] == e
 *   offsets[0]     = 0, offsets[e+1] = offsets[e] + counts[e]
 *   sorted_route[p] = the route at position p (p < offsets[E]); -1 after
 *   route_pos[i]   = p with sorted_route[p] == i, or -1 for a dropped route
 */
int oracle_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, const int32_t* slot_of,
                   int32_t* offsets, int32_t* sorted_route, int32_t* route_pos, int32_t* n_dropped)
{
    if (!ids || !slot_of || !offsets || !sorted_route || !route_pos || !n_dropped || T < 0 ||
        k < 1 || E < 1)
        return ORA_EARG;
    const int64_t R = (int64_t)T * k;
    int32_t dropped = 0;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t c = 0;
        if (slot_of[e] >= 0)
            for (int64_t i = 0; i < R; ++i) c += (ids[i] == e);
        offsets[e + 1] = offsets[e] + c;
    }
    for (int64_t i = 0; i < R; ++i) {
        route_pos[i] = -1;
        sorted_route[i] = -1;
    }
    int32_t p = 0;
    for (int32_t e = 0; e < E; ++e) {
        if (slot_of[e] < 0) continue;
        for (int64_t i = 0; i < R; ++i) {
            if (ids[i] != e) continue;
            sorted_route[p] = (int32_t)i;
            route_pos[i] = p;
            ++p;
        }
    }
    for (int64_t i = 0; i < R; ++i) dropped += (route_pos[i] < 0);
    *n_dropped = dropped;
    return ORA_OK;
}

/* --------------------------------------------------------- router GEMV --
 * [prain] "int4 experts on RDNA2" (the router is an fp32 GEMV whose logits feed
 * the top-k): logits[t][e] = sum_h x[t][h] * Wr[e][h], x the token's hidden state
 * (its fp32 value), Wr the fp32 router weight [E, H]; summed in fp64.
 */
int oracle_router_logits(const float* x, const float* wr, int32_t T, int32_t H, int32_t E, double* logits)
{
    if (!x || !wr || !logits || T < 0 || H < 1 || E < 1) return ORA_EARG;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h) acc += (double)x[(int64_t)t * H + h] * (double)wr[(int64_t)e * H + h];
            logits[(int64_t)t * E + e] = acc;
        }
    return ORA_OK;
}

/* ---------------------------------------------------- residency refresh --
 * [rlx_runtime expert_pool.rs] (TIDE-style placement): count the hits of
 * each expert in a step's routes, take the gpu_budget experts with the most
 * hits (hits > 0; equal counts: lower expert id first) as the target, promote
 * the target experts that are not resident (in target order) and demote as
 * many resident experts outside the target (paired promote/demote); resident
 * experts outside the target beyond that stay.  Readings (the page's set
 * iteration has no order, and it keeps no slots):
 *   - the experts that may be demoted are taken in ascending expert id;
 *   - promotion j takes the slot of demotion j; promotions beyond the pairs
 *     take the lowest free slots of [0, S) in ascending order (slots no
 *     resident expert holds).  S >= budget guarantees enough.
 * slot_of_out: demoted experts -1, promoted ones their slot, others as in
 * slot_of_in.  counts = {targets, promotions, demotions}.
 */
int oracle_residency_refresh(const int32_t* ids, int64_t R, int32_t E, int32_t budget, int32_t S,
                             const int32_t* slot_of_in, int32_t* hits, int32_t* target, int32_t* promote,
                             int32_t* promote_slot, int32_t* demote, int32_t* counts, int32_t* slot_of_out)
{
    if (!ids || !slot_of_in || !hits || !target || !promote || !promote_slot || !demote || !counts ||
        !slot_of_out || R < 0 || E < 1 || budget < 0 || budget > E || S < budget)
        return ORA_EARG;
    for (int32_t e = 0; e < E; ++e) hits[e] = 0;
    for (int64_t i = 0; i < R; ++i)
        if (ids[i] >= 0 && ids[i] < E) hits[ids[i]] += 1;
    /* target: repeatedly the unpicked expert with the most hits (> 0), lowest id on ties */
    int32_t* picked = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    int32_t* in_target = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    int32_t* used = (int32_t*)calloc((size_t)S + 1, sizeof(int32_t));
    if (!picked || !in_target || !used) { free(picked); free(in_target); free(used); return ORA_EARG; }
    int32_t nt = 0;
    while (nt < budget) {
        int32_t b = -1;
        for (int32_t e = 0; e < E; ++e)
            if (!picked[e] && hits[e] > 0 && (b < 0 || hits[e] > hits[b])) b = e;
        if (b < 0) break;
        picked[b] = 1;
        in_target[b] = 1;
        target[nt++] = b;
    }
    for (int32_t r = nt; r < budget; ++r) target[r] = -1;
    int32_t np = 0;
    for (int32_t r = 0; r < nt; ++r)
        if (slot_of_in[target[r]] < 0) promote[np++] = target[r];
    int32_t nd = 0;
    for (int32_t e = 0; e < E && nd < np; ++e)
        if (slot_of_in[e] >= 0 && !in_target[e]) demote[nd++] = e;
    for (int32_t e = 0; e < E; ++e)
        if (slot_of_in[e] >= 0 && slot_of_in[e] < S) used[slot_of_in[e]] = 1;
    int32_t next_free = 0;
    int rc = ORA_OK;
    for (int32_t j = 0; j < np; ++j) {
        if (j < nd) {
            promote_slot[j] = slot_of_in[demote[j]];
        } else {
            while (next_free < S && used[next_free]) ++next_free;
            if (next_free >= S) { rc = ORA_EARG; break; }
            promote_slot[j] = next_free++;
        }
    }
    for (int32_t e = 0; e < E; ++e) slot_of_out[e] = slot_of_in[e];
    for (int32_t j = 0; j < nd; ++j) slot_of_out[demote[j]] = -1;
    for (int32_t j = 0; j < np && rc == ORA_OK; ++j) slot_of_out[promote[j]] = promote_slot[j];
    counts[0] = nt;
    counts[1] = np;
    counts[2] = nd;
    free(picked);
    free(in_target);
    free(used);
    return rc;
}

/* ------------------------------------------------- min_weight routing --
 * [prain] "Trading quality for speed": min_weight is the share of a token's
 * router weight that must be computed.  Below 1 the token skips its lightest
 * experts that are not resident once the share is reached, and the routes it
 * keeps are scaled up to its full weight.  Readings (the page states the rule,
 * not its arithmetic):
 *   - the token's weight W = sum of its k weights; resident routes are always
 *     kept; the others are taken heaviest first (equal weights: lower j first)
 *     while the kept weight c is below min_weight * W, the rest skipped;
 *   - kept routes are scaled by W / c when something was skipped; min_weight
 *     >= 1 keeps every route unchanged (the hot path);
 *   - routes with ids outside [0, E) are skipped and not counted in W;
 *   - all of it in fp32 (the decision is a float comparison; both sides take
 *     it in the kernel's precision), sums in the order just stated.
 * Outputs: ids_out (skipped: -1), w_out (skipped: 0), and miss_count[e], the
 * number of kept routes to a non-resident expert e (the copies a step needs).
 */
int oracle_min_weight(const int32_t* ids, const float* w, int32_t T, int32_t k, int32_t E, const int32_t* slot_of,
                      float min_weight, int32_t* ids_out, float* w_out, int32_t* miss_count)
{
    if (!ids || !w || !slot_of || !ids_out || !w_out || !miss_count || T < 0 || k < 1 || k > 32 || E < 1)
        return ORA_EARG;
    for (int32_t e = 0; e < E; ++e) miss_count[e] = 0;
    for (int32_t t = 0; t < T; ++t) {
        const int32_t* id = ids + (int64_t)t * k;
        const float* wt = w + (int64_t)t * k;
        int valid[32], res[32], keep[32];
        float W = 0.0f, c = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            valid[j] = id[j] >= 0 && id[j] < E;
            res[j] = valid[j] && slot_of[id[j]] >= 0;
            keep[j] = res[j];
            if (valid[j]) W += wt[j];
        }
        if (min_weight >= 1.0f) {
            for (int32_t j = 0; j < k; ++j) keep[j] = valid[j];
        } else {
            for (int32_t j = 0; j < k; ++j)
                if (res[j]) c += wt[j];
            const float target = min_weight * W;
            int done[32] = {0};
            for (;;) {   /* the heaviest non-resident route not yet decided */
                int32_t b = -1;
                for (int32_t j = 0; j < k; ++j)
                    if (valid[j] && !res[j] && !done[j] && (b < 0 || wt[j] > wt[b])) b = j;
                if (b < 0) break;
                done[b] = 1;
                if (c >= target) continue;   /* share reached: skip */
                keep[b] = 1;
                c += wt[b];
            }
        }
        int skipped = 0;
        for (int32_t j = 0; j < k; ++j) skipped |= valid[j] && !keep[j];
        const float scale = (skipped && c > 0.0f) ? W / c : 1.0f;
        for (int32_t j = 0; j < k; ++j) {
            ids_out[(int64_t)t * k + j] = keep[j] ? id[j] : -1;
            w_out[(int64_t)t * k + j] = keep[j] ? (skipped ? wt[j] * scale : wt[j]) : 0.0f;
            if (keep[j] && !res[j]) miss_count[id[j]] += 1;
        }
    }
    return ORA_OK;
}

/* --------------------------------------------------------- quantisation --
 * [prain] "Expert formats": int8 experts carry an fp32 scale per row; int4
 * experts carry a bf16 scale per 64 elements, chosen by an MSE clip search;
 * activations stay 16-bit (w8a16 / w4a16).  Readings taken (the pages name the
 * formats and their sizes, not the algorithm):
 *   - symmetric codes, no zero point (a zero point would not fit the sizes the
 *     table prints); rows run along the reduction dimension K, groups are 64
 *     consecutive elements of a row;
 *   - int8: absmax scale s = a / 127, codes in [-127, 127];
 *   - int4: codes in [-8, 7], stored as u = q + 8, the low nibble of byte b
 *     holding element 2b and the high nibble element 2b+1; the clip search
 *     tries alpha = (20 - i) / 20 for i = 0..9 (1.00, 0.95, ..., 0.55) with
 *     s_i = bf16(a * (20 - i) / 140) = bf16(alpha * a / 7) and keeps the first
 *     candidate with the smallest squared error.
 */
void oracle_quantize_int8(const uint16_t* w, int32_t N, int32_t K, int8_t* q, float* s)
{
    for (int32_t r = 0; r < N; ++r) {
        const uint16_t* row = w + (int64_t)r * K;
        float a = 0.0f;
        for (int32_t c = 0; c < K; ++c) {
            float v = fabsf(bf16_bits_to_f32(row[c]));
            if (v > a) a = v;
        }
        float sc = (a == 0.0f) ? 0.0f : a / 127.0f;
        s[r] = sc;
        for (int32_t c = 0; c < K; ++c) {
            float code = 0.0f;
            if (sc != 0.0f) {
                code = rintf(bf16_bits_to_f32(row[c]) / sc);
                if (code > 127.0f) code = 127.0f;
                if (code < -127.0f) code = -127.0f;
            }
            q[(int64_t)r * K + c] = (int8_t)code;
        }
    }
}

/* one candidate scale's codes for one group of 64 */
static void int4_codes(const float* v, float sc, int32_t* code)
{
    for (int c = 0; c < 64; ++c) {
        if (sc == 0.0f) { code[c] = 0; continue; }
        float x = rintf(v[c] / sc);
        if (x > 7.0f) x = 7.0f;
        if (x < -8.0f) x = -8.0f;
        code[c] = (int32_t)x;
    }
}

/* Clip candidate i of a 64-element group v with absmax a: its bf16 scale and
 * its squared error summed in element order (fp64, no FMA). */
static double int4_candidate(const float* v, float a, int i, uint16_t* sb_out, int32_t* code)
{
    const uint16_t sb = f32_to_bf16_bits((a * (float)(20 - i)) / 140.0f);
    const float sc = bf16_bits_to_f32(sb);
    int4_codes(v, sc, code);
    double err = 0.0;
    for (int c = 0; c < 64; ++c) {
        double d = (double)v[c] - (double)sc * (double)code[c];
        err = err + d * d;
    }
    *sb_out = sb;
    return err;
}

static float group_absmax(const uint16_t* grp, float* v)
{
    float a = 0.0f;
    for (int c = 0; c < 64; ++c) {
        v[c] = bf16_bits_to_f32(grp[c]);
        if (fabsf(v[c]) > a) a = fabsf(v[c]);
    }
    return a;
}

/* Every clip candidate of one 64-element group (bf16 bits): scale bits and
 * squared error of each i = 0..9 (for pinning the candidates that never win). */
void oracle_int4_candidates(const uint16_t* grp, uint16_t* scales, double* errs)
{
    float v[64];
    int32_t code[64];
    const float a = group_absmax(grp, v);
    for (int i = 0; i < 10; ++i) errs[i] = int4_candidate(v, a, i, &scales[i], code);
}

void oracle_quantize_int4(const uint16_t* w, int32_t N, int32_t K, uint8_t* q, uint16_t* s)
{
    const int32_t G = K / 64;
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < N; ++r) {
        float v[64];
        int32_t code[64], best_code[64];
        for (int32_t g = 0; g < G; ++g) {
            const uint16_t* grp = w + (int64_t)r * K + (int64_t)g * 64;
            const float a = group_absmax(grp, v);
            double best_err = 0.0;
            uint16_t best_s = 0;
            for (int i = 0; i < 10; ++i) {
                uint16_t sb;
                const double err = int4_candidate(v, a, i, &sb, code);
                if (i == 0 || err < best_err) {
                    best_err = err;
                    best_s = sb;
                    memcpy(best_code, code, sizeof(code));
                }
            }
            s[(int64_t)r * G + g] = best_s;
            uint8_t* out = q + (int64_t)r * (K / 2) + (int64_t)g * 32;
            for (int b = 0; b < 32; ++b)
                out[b] = (uint8_t)(((best_code[2 * b] + 8) & 0xF) | (((best_code[2 * b + 1] + 8) & 0xF) << 4));
        }
    }
}

/* ------------------------------------------------------------- the pack --
 * One expert's blob ([prain] "Expert formats": an expert is its w13 (gate and
 * up stacked, [2FF, H]) and its w2 ([H, FF]), with the format's scales).
 * Sub-blocks in this order, each starting on a 256-byte boundary, the blob
 * size rounded up to 256:
 *   bf16: w13 bf16 [2FF,H] | w2 bf16 [H,FF]
 *   int8: w13 int8 [2FF,H] | w13 scale fp32 [2FF] | w2 int8 [H,FF] | w2 scale fp32 [H]
 *   int4: w13 nibbles [2FF,H/2] | w13 scale bf16 [2FF,H/64] | w2 nibbles [H,FF/2] |
 *         w2 scale bf16 [H,FF/64]
 *         The nibble blocks are tiled (a storage order of this library, not
 *         of the pages): rows in blocks of 32, and within a block the 32 bytes
 *         of each 64-element group of the 32 rows stored together, so byte b
 *         (element 2b low, 2b+1 high) of row n sits at
 *         ((n / 32) * (K / 64) + b / 32) * 1024 + (n % 32) * 32 + b % 32.
 * off[0..3] = start of w13 codes, w13 scales, w2 codes, w2 scales (for bf16 the
 * scale entries equal the next block's start); off[4] = blob bytes.
 */
static uint64_t up256(uint64_t x) { return (x + 255u) / 256u * 256u; }

/* offset of byte b of row n in a tiled int4 nibble block of K columns */
static int64_t int4_tiled(int32_t n, int32_t K, int32_t b)
{
    return ((int64_t)(n / 32) * (K / 64) + b / 32) * 1024 + (int64_t)(n % 32) * 32 + b % 32;
}

/* quantise W [N, K] (N a multiple of 32) into a tiled nibble block */
static int quantize_int4_tiled(const uint16_t* w, int32_t N, int32_t K, uint8_t* q, uint16_t* s)
{
    uint8_t* rm = (uint8_t*)malloc((size_t)N * (size_t)(K / 2));
    if (!rm) return ORA_EARG;
    oracle_quantize_int4(w, N, K, rm, s);
    for (int32_t n = 0; n < N; ++n)
        for (int32_t b = 0; b < K / 2; ++b) q[int4_tiled(n, K, b)] = rm[(int64_t)n * (K / 2) + b];
    free(rm);
    return ORA_OK;
}

int oracle_blob_layout(int32_t fmt, int32_t H, int32_t FF, uint64_t* off)
{
    const uint64_t n13 = 2ull * (uint64_t)FF * (uint64_t)H, n2 = (uint64_t)H * (uint64_t)FF;
    if (H < 1 || FF < 1) return ORA_EARG;
    if (fmt == ORA_W_BF16) {
        off[0] = 0;
        off[1] = off[2] = up256(n13 * 2);
        off[3] = off[4] = up256(off[2] + n2 * 2);
    } else if (fmt == ORA_W_INT8_ROW) {
        off[0] = 0;
        off[1] = up256(n13);
        off[2] = up256(off[1] + 2ull * FF * 4);
        off[3] = up256(off[2] + n2);
        off[4] = up256(off[3] + (uint64_t)H * 4);
    } else if (fmt == ORA_W_INT4_G64) {
        if (H % 64 || FF % 64) return ORA_EARG;
        off[0] = 0;
        off[1] = up256(n13 / 2);
        off[2] = up256(off[1] + 2ull * FF * (H / 64) * 2);
        off[3] = up256(off[2] + n2 / 2);
        off[4] = up256(off[3] + (uint64_t)H * (FF / 64) * 2);
    } else {
        return ORA_EARG;
    }
    return ORA_OK;
}

int oracle_pack_expert(int32_t fmt, const uint16_t* w13, const uint16_t* w2, int32_t H, int32_t FF,
                       uint8_t* blob)
{
    uint64_t off[5];
    if (oracle_blob_layout(fmt, H, FF, off) != ORA_OK) return ORA_EARG;
    memset(blob, 0, off[4]);
    if (fmt == ORA_W_BF16) {
        memcpy(blob + off[0], w13, 2ull * FF * H * 2);
        memcpy(blob + off[2], w2, (uint64_t)H * FF * 2);
    } else if (fmt == ORA_W_INT8_ROW) {
        oracle_quantize_int8(w13, 2 * FF, H, (int8_t*)(blob + off[0]), (float*)(blob + off[1]));
        oracle_quantize_int8(w2, H, FF, (int8_t*)(blob + off[2]), (float*)(blob + off[3]));
    } else {
        if (quantize_int4_tiled(w13, 2 * FF, H, blob + off[0], (uint16_t*)(blob + off[1])) != ORA_OK ||
            quantize_int4_tiled(w2, H, FF, blob + off[2], (uint16_t*)(blob + off[3])) != ORA_OK)
            return ORA_EARG;
    }
    return ORA_OK;
}

/* ------------------------------------------------------------ slot fill --
 * [prain] "int4 experts on RDNA2": an expert copied into a cache slot goes
 * through a staging buffer and one unpack step.  The canonical form of an
 * expert is the blob layout above with the int4 nibble blocks row-major (byte b
 * of row n at n * K/2 + b, as oracle_quantize_int4 writes them); the slot form
 * is the tiled one.  bf16 and int8 blobs are the same in both forms.
 */
int oracle_pack_expert_canonical(int32_t fmt, const uint16_t* w13, const uint16_t* w2, int32_t H, int32_t FF,
                                 uint8_t* blob)
{
    uint64_t off[5];
    if (oracle_blob_layout(fmt, H, FF, off) != ORA_OK) return ORA_EARG;
    if (fmt != ORA_W_INT4_G64) return oracle_pack_expert(fmt, w13, w2, H, FF, blob);
    memset(blob, 0, off[4]);
    oracle_quantize_int4(w13, 2 * FF, H, blob + off[0], (uint16_t*)(blob + off[1]));
    oracle_quantize_int4(w2, H, FF, blob + off[2], (uint16_t*)(blob + off[3]));
    return ORA_OK;
}

/* canonical blob -> slot blob: the nibble blocks tiled, every other byte as it is */
int oracle_fill_slot(int32_t fmt, const uint8_t* canonical, int32_t H, int32_t FF, uint8_t* slot)
{
    uint64_t off[5];
    if (oracle_blob_layout(fmt, H, FF, off) != ORA_OK) return ORA_EARG;
    memcpy(slot, canonical, off[4]);
    if (fmt != ORA_W_INT4_G64) return ORA_OK;
    for (int which = 0; which < 2; ++which) {
        const int32_t N = which ? H : 2 * FF, K = which ? FF : H;
        const uint64_t o = which ? off[2] : off[0];
        for (int32_t n = 0; n < N; ++n)
            for (int32_t b = 0; b < K / 2; ++b) slot[o + int4_tiled(n, K, b)] = canonical[o + (int64_t)n * (K / 2) + b];
    }
    return ORA_OK;
}

/* ---------------------------------------------------------- dequantised --
 * The weight a packed blob stands for, as the format defines it:
 *   bf16: the bf16 value;  int8: s_row * q;  int4: s_(row,group) * (u - 8).
 * which = 0 reads w13 [2FF, H], which = 1 reads w2 [H, FF].
 */
static double weight_at(const uint8_t* blob, const uint64_t* off, int32_t fmt, int which,
                        int32_t K, int32_t row, int32_t col)
{
    const uint8_t* codes = blob + (which ? off[2] : off[0]);
    const uint8_t* scales = blob + (which ? off[3] : off[1]);
    if (fmt == ORA_W_BF16) {
        uint16_t h;
        memcpy(&h, codes + 2 * ((int64_t)row * K + col), 2);
        return (double)bf16_bits_to_f32(h);
    }
    if (fmt == ORA_W_INT8_ROW) {
        float sc;
        memcpy(&sc, scales + 4 * (int64_t)row, 4);
        return (double)sc * (double)(int8_t)codes[(int64_t)row * K + col];
    }
    uint16_t sb;
    memcpy(&sb, scales + 2 * ((int64_t)row * (K / 64) + col / 64), 2);
    uint8_t byte = codes[int4_tiled(row, K, col / 2)];
    int32_t u = (col & 1) ? (byte >> 4) : (byte & 0xF);
    return (double)bf16_bits_to_f32(sb) * (double)(u - 8);
}

/* expose single-matrix dequantisation for the tests: out [rows, K] fp64 */
int oracle_dequant(const uint8_t* blob, int32_t fmt, int32_t H, int32_t FF, int32_t which, double* out)
{
    uint64_t off[5];
    if (oracle_blob_layout(fmt, H, FF, off) != ORA_OK) return ORA_EARG;
    const int32_t rows = which ? H : 2 * FF, K = which ? FF : H;
    for (int32_t r = 0; r < rows; ++r)
        for (int32_t c = 0; c < K; ++c)
            out[(int64_t)r * K + c] = weight_at(blob, off, fmt, which, K, r, c);
    return ORA_OK;
}

/* --------------------------------------------------------- activations --
 * The pages never name the gated activation.  Two are provided:
 *   GELU, tanh form: 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3)))
 *   SiLU:            g / (1 + exp(-g))
 */
static double act_fn(int32_t act, double g)
{
    if (act == ORA_ACT_SILU) return g / (1.0 + exp(-g));
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * g * (1.0 + tanh(c * (g + 0.044715 * g * g * g)));
}

void oracle_act(int32_t act, const double* g, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = act_fn(act, g[i]);
}

/* ---------------------------------------------------------- expert FFN --
 * For a route i (token t = i / k, expert e = ids[i], blob at pool + slot_of[e] *
 * slot_bytes): with W13 = [W1; W3] (gate rows 0..FF-1, up rows FF..2FF-1 -- a
 * reading; the pages only name the w13/w2 split),
 *   g_n = sum_h W1[n][h] x[t][h],  u_n = sum_h W3[n][h] x[t][h],
 *   h_n = act(g_n) * u_n,          o[m] = sum_n W2[m][n] h_n.
 * All in fp64.  routes[0..n_routes) lists which routes to evaluate; o is
 * [n_routes, H].  Routes whose expert is out of range or not resident are
 * left as zeros and flagged in ok[] (0).
 */
int oracle_expert_ffn(const uint8_t* pool, uint64_t slot_bytes, const int32_t* slot_of, int32_t E,
                      int32_t H, int32_t FF, int32_t fmt, int32_t act, const float* x, int32_t T,
                      int32_t k, const int32_t* ids, const int32_t* routes, int32_t n_routes,
                      double* o, int32_t* ok)
{
    uint64_t off[5];
    if (oracle_blob_layout(fmt, H, FF, off) != ORA_OK) return ORA_EARG;
    if (!pool || !slot_of || !x || !ids || !routes || !o || !ok || k < 1 || T < 0) return ORA_EARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < n_routes; ++r) {
        const int32_t i = routes[r];
        double* orow = o + (int64_t)r * H;
        for (int32_t m = 0; m < H; ++m) orow[m] = 0.0;
        ok[r] = 0;
        if (i < 0 || (int64_t)i >= (int64_t)T * k) continue;
        const int32_t e = ids[i], t = i / k;
        if (e < 0 || e >= E || slot_of[e] < 0) continue;
        ok[r] = 1;
        const uint8_t* blob = pool + (uint64_t)slot_of[e] * slot_bytes;
        const float* xt = x + (int64_t)t * H;
        double* hv = (double*)malloc(sizeof(double) * (size_t)FF);
        for (int32_t n = 0; n < FF; ++n) {
            double g = 0.0, u = 0.0;
            for (int32_t c = 0; c < H; ++c) {
                g += weight_at(blob, off, fmt, 0, H, n, c) * (double)xt[c];
                u += weight_at(blob, off, fmt, 0, H, FF + n, c) * (double)xt[c];
            }
            hv[n] = act_fn(act, g) * u;
        }
        for (int32_t m = 0; m < H; ++m) {
            double acc = 0.0;
            for (int32_t n = 0; n < FF; ++n) acc += weight_at(blob, off, fmt, 1, FF, m, n) * hv[n];
            orow[m] = acc;
        }
        free(hv);
    }
    return ORA_OK;
}

/* ------------------------------------------------------------- combine --
 * Weighted scatter-combine back to token order ([strata] RemoteExperts::finish
 * scatters each computed row back to its route; [prain] "Trading quality for
 * speed": a token's output is its routes weighted by their router share).
 *   y[t][m] = sum_{j=0..k-1, route t*k+j kept} w[t][j] * o_(t*k+j)[m]
 * in ascending j, fp64.  Dropped routes add nothing and the rest are not
 * rescaled.  o_rows[q] holds route routes_of[q]'s output; tokens[] lists the
 * tokens to produce; y is [n_tokens, H].
 */
int oracle_combine(const double* o_rows, const int32_t* route_row, const float* w, int32_t k,
                   int32_t H, const int32_t* tokens, int32_t n_tokens, double* y)
{
    /* route_row[t*k + j] = row of o_rows holding that route, or -1 (dropped) */
    if (!o_rows || !route_row || !w || !tokens || !y || k < 1 || H < 1) return ORA_EARG;
    for (int32_t q = 0; q < n_tokens; ++q) {
        const int32_t t = tokens[q];
        double* yr = y + (int64_t)q * H;
        for (int32_t m = 0; m < H; ++m) yr[m] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            const int32_t row = route_row[(int64_t)q * k + j];
            if (row < 0) continue;
            const double wj = (double)w[(int64_t)t * k + j];
            const double* orow = o_rows + (int64_t)row * H;
            for (int32_t m = 0; m < H; ++m) yr[m] += wj * orow[m];
        }
    }
    return ORA_OK;
}

/* ------------------------------------------------------------- threads --
 * Worker threads of the parallel loops above (for timing the oracle at a
 * chosen thread count); returns the count that later loops will use. */
int oracle_set_threads(int32_t n)
{
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}
