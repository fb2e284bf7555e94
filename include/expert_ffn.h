/*
 * expert_ffn.h -- C ABI of the MI355X (gfx950) routed expert FFN library
 * (expert_ffn_amd/libexpert_ffn.so).
 *
 * One MoE layer's routed expert FFN, as the prain README describes the serving
 * problem (sections "Expert formats" and "int4 experts on RDNA2"): each token
 * picks its top-k experts from router logits; routes are grouped per expert;
 * each expert applies a gated FFN (w13 = gate and up projections stacked,
 * then the w2 down projection); the outputs are combined back into token
 * order, weighted by the router's renormalised softmax.  Expert weights are
 * bf16, int8 with an fp32 scale per row, or int4 with a bf16 scale per 64
 * elements; experts are found through a per-layer expert -> slot table into a
 * pool of equally sized slots (prain's VRAM cache slots; Winery-Strata's
 * RemoteExperts::begin looks experts up the same way, slot_of / device_slot).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library keeps no pointer after a call returns and never allocates or
 *     frees device memory in any call.  "host" pointers are host memory:
 *     the layout query, the slot bookkeeping (moe_slot_admit) and the
 *     sources of the slot fills (pinned memory, read by the copy engine or
 *     the unpack kernel until the stream reaches them).
 *   - stream is a hipStream_t (NULL = the legacy default stream).  Every call
 *     only enqueues work on that stream and returns; nothing synchronises.
 *     (The int4 expert FFN calls may also run their grouped GEMM on a second
 *     stream the library keeps per device, created with its two events on the
 *     first such call: it waits for `stream` through one event and `stream`
 *     waits for it through the other before the call returns, so the work
 *     stays ordered on `stream`, and under HIP graph capture it is a fork and
 *     join inside the captured graph.)
 *   - Arguments are checked on the host before anything is enqueued.  A call
 *     that returns a status other than MOE_OK has enqueued nothing, and
 *     moe_last_error() describes why as "<function>: <what>".  MOE_E_HIP
 *     reports a failed launch with the HIP runtime's error string.
 *   - Shape rules: 1 <= k <= min(E, 32), E <= 512, T >= 0 (T = 0 enqueues
 *     nothing), H % 64 == 0, FF % 32 == 0 (bf16 weights) or FF % 64 == 0
 *     (int8/int4 weights).
 */
#ifndef EXPERT_FFN_H
#define EXPERT_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_E_ARG = 1,          /* a null pointer, negative size or unknown enum    */
    MOE_E_SHAPE = 2,        /* sizes that break a shape rule above              */
    MOE_E_UNSUPPORTED = 3,  /* a combination the library does not implement     */
    MOE_E_WORKSPACE = 4,    /* workspace smaller than moe_workspace_bytes()     */
    MOE_E_HIP = 5           /* the HIP runtime reported an error                */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Expert weight formats (prain README, "Expert formats" table). */
typedef enum {
    MOE_W_BF16 = 0,      /* weights as trained                                   */
    MOE_W_INT8_ROW = 1,  /* int8 codes, one fp32 scale per output row (w8a16)    */
    MOE_W_INT4_G64 = 2   /* int4 codes, one bf16 scale per 64 elements (w4a16)   */
} moe_wfmt;

/* Gated activation applied to the gate projection (the pages do not name it). */
typedef enum { MOE_ACT_GELU_TANH = 0, MOE_ACT_SILU = 1 } moe_act;

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* moe_last_error(void);

/*
 * Bytes of one packed expert blob (the slot size a pool needs), 0 if the shape
 * is invalid for the format.  Gemma-4-26B-A4B (H = 2816, FF = 704): 11,894,784
 * (bf16), 5,964,288 (int8), 3,159,552 (int4) -- 11.34 / 5.69 / 3.01 MiB, the
 * sizes of prain's "Expert formats" table.
 */
uint64_t moe_expert_bytes(int32_t wfmt, int32_t H, int32_t FF);

/*
 * Layout of a blob (host call).  off (host, 5 entries) receives the byte
 * offsets of: w13 codes, w13 scales, w2 codes, w2 scales, and the blob size.
 * Each sub-block starts on a 256-byte boundary; the size is rounded up to 256.
 *   bf16: w13 bf16 [2FF, H] | w2 bf16 [H, FF]  (the scale offsets equal the
 *         next block's start)
 *   int8: w13 int8 [2FF, H] | fp32 [2FF] | w2 int8 [H, FF] | fp32 [H]
 *   int4: w13 [2FF, H/2] | bf16 [2FF, H/64] | w2 [H, FF/2] | bf16 [H, FF/64]
 * Rows are K-contiguous (K = H for w13, FF for w2).  w13 rows 0..FF-1 are the
 * gate projection, FF..2FF-1 the up projection.  int4 byte b of a row holds
 * element 2b in its low nibble and 2b+1 in its high nibble, each as q + 8;
 * the int4 code blocks are stored in tiles of 32 rows: byte b of row n is at
 * ((n / 32) * (K / 64) + b / 32) * 1024 + (n % 32) * 32 + b % 32, so that the
 * 32 bytes of one 64-element group of 32 consecutive rows are 1 KB of
 * contiguous memory (one wide load for the kernels).  moe_quantize writes the
 * codes row-major; moe_pack_expert writes them tiled.
 */
moe_status moe_blob_layout(int32_t wfmt, int32_t H, int32_t FF, uint64_t* off);

/*
 * Workspace bytes moe_expert_ffn / moe_ffn_gate_up / moe_ffn_down need for T
 * tokens with top-k routing (bf16 activations in the kernels' operand layout
 * and the gated hidden rows h [T*k, FF]).
 */
size_t moe_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t FF, int32_t wfmt);

/*
 * Router top-k with softmax weights (prain README, "Trading quality for speed":
 * a token's router weight is shared among its experts; the tie rule is that of
 * rlx_runtime/expert_pool.rs, target_gpu_from_counts: equal values go to the
 * lower expert id first).
 *   logits   device fp32 [T, E], row-major.  Larger logit = preferred.  NaN
 *            ranks below every number; -0 equals +0.  Logits should be finite
 *            for meaningful weights.
 *   topk_ids device int32 [T, k] out: the k chosen experts, best first.
 *   topk_w   device fp32 [T, k] out: renorm != 0: softmax over the chosen k
 *            logits (the full softmax renormalised over the chosen experts);
 *            renorm == 0: the full softmax over E at the chosen experts.
 */
moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                          int32_t* topk_ids, float* topk_w, void* stream);

/*
 * Group routes by expert (Winery-Strata remote_experts.cpp, RemoteExperts::
 * begin: per expert group, the routes in route order, token = route / k;
 * rlx_runtime/expert_pool.rs count_hits: the per-expert histogram).
 * Route i = t*k + j is kept when 0 <= topk_ids[i] < E and slot_of[that] >= 0;
 * otherwise it is dropped (its expert is not resident) and counted.
 *   topk_ids       device int32 [T*k]
 *   slot_of        device int32 [E], the layer's expert -> slot table, -1 =
 *                  not resident
 *   expert_offsets device int32 [E+1] out: group e is positions
 *                  [offsets[e], offsets[e+1]); offsets[E] = kept routes
 *   sorted_route   device int32 [T*k] out: route index at each position,
 *                  experts ascending, route index ascending inside a group;
 *                  -1 from offsets[E] on
 *   route_pos      device int32 [T*k] out: position of each route, -1 if dropped
 *   n_dropped      device int32 [1] out: number of dropped routes
 * Deterministic: no result depends on thread timing.
 */
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       const int32_t* slot_of, int32_t* expert_offsets, int32_t* sorted_route,
                       int32_t* route_pos, int32_t* n_dropped, void* stream);

/*
 * moe_route_topk followed by moe_permute on the same routes, with the same
 * arguments and results as those two calls (the definitions above).  For
 * T*k <= 1024 and T <= 64 both run in one workgroup of one launch and the ids
 * never make a round trip through memory between them; larger T falls back
 * to the two launches.  topk_ids and topk_w are written as by moe_route_topk.
 */
moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                             const int32_t* slot_of, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                             int32_t* sorted_route, int32_t* route_pos, int32_t* n_dropped, void* stream);

/*
 * Router GEMV fused with the top-k (prain README, "int4 experts on RDNA2":
 * the router is an fp32 GEMV, tried there as a separate kernel): logits[t][e] =
 * sum_h x[t][h] * w_router[e][h] in fp32 (bf16 x widened exactly), then the
 * top-k and softmax weights of moe_route_topk on those logits: two launches
 * (partial sums over 256-element slices of H, then per token the sum of the
 * slices and the top-k), the full logits written once.
 *   x         device [T, H], fp32 or bf16 (x_dtype), 16-byte aligned
 *   w_router  device fp32 [E, H], 16-byte aligned
 *   logits    device fp32 [T, E] out (the router logits)
 *   ws        device workspace of ws_bytes >= moe_router_ws_bytes(T, H, E),
 *             16-byte aligned (partial sums; no state between calls)
 *   topk_ids, topk_w: as moe_route_topk.
 * H % 64 == 0.  The sums run in a fixed order (per 256-element slice of H,
 * then the slices in order), so results are reproducible; the logits differ
 * from an fp64 product by fp32 rounding, and so may the order of experts whose
 * logits tie within it.
 */
size_t moe_router_ws_bytes(int32_t T, int32_t H, int32_t E);
moe_status moe_router_topk(const void* x, int32_t x_dtype, int32_t T, int32_t H, const float* w_router, int32_t E,
                           int32_t k, int32_t renorm, float* logits, void* ws, size_t ws_bytes, int32_t* topk_ids,
                           float* topk_w, void* stream);

/*
 * Residency refresh from the device's routing (rlx_runtime expert_pool.rs,
 * TIDE-style placement: count token hits per expert, take the budget most-hit
 * experts, promote and demote in pairs to limit copies).  One launch:
 *   hits[e]   (device int32 [E] out) routes of ids (device int32 [R], e.g. a
 *             step's topk_ids) with id e; ids outside [0, E) are not counted
 *   target    (device int32 [budget] out) the experts with hits > 0, most
 *             hits first, equal counts lower id first, at most budget; the
 *             rest -1
 *   promote   (device int32 [E] out) the target experts not resident
 *             (slot_of < 0), in target order; promote_slot the slot each
 *             takes: the slot of the paired demotion, then the lowest slots
 *             of [0, n_slots) that no resident expert holds
 *   demote    (device int32 [E] out) resident experts outside the target, in
 *             ascending id, as many as there are promotions (residents
 *             beyond that stay)
 *   counts    (device int32 [3] out) {targets, promotions, demotions}
 *   slot_of   (device int32 [E], in and out) the layer's table, rewritten:
 *             demoted -1, promoted their slot.  The caller copies each
 *             promoted expert into its slot (moe_fill_slot) before the table
 *             is used by a step.
 * 1 <= E <= 512, 0 <= budget <= E, budget <= n_slots <= 512; the resident
 * experts must hold distinct slots below n_slots.
 */
moe_status moe_residency_refresh(const int32_t* ids, int64_t R, int32_t E, int32_t budget, int32_t n_slots,
                                 int32_t* slot_of, int32_t* hits, int32_t* target, int32_t* promote,
                                 int32_t* promote_slot, int32_t* demote, int32_t* counts, void* stream);

/*
 * When to refresh (host; rlx_runtime expert_pool.rs, should_refresh): never
 * without offload (budget < E); always for a prefill block or with every <= 1;
 * otherwise on steps that are multiples of every.
 */
int32_t moe_refresh_due(int32_t every, int64_t step, int32_t prefill_block, int32_t offload);

/*
 * Experts per layer that fit in memory (host; rlx_runtime expert_pool.rs,
 * gpu_expert_budget_from_vram): (free - reserve) / (expert_bytes * layers),
 * at most min(max_per_layer, E); min(max_per_layer, E) when expert_bytes or
 * layers is 0.
 */
int32_t moe_budget_from_memory(uint64_t free_bytes, uint64_t reserve_bytes, uint64_t expert_bytes, int32_t layers,
                               int32_t max_per_layer, int32_t E);

/*
 * min_weight partial routing (prain README, "Trading quality for speed": the
 * share of each token's router weight that must be computed; below 1 a token
 * skips its lightest experts that are not resident once it has that share,
 * and the routes it keeps are scaled up to its full weight).  For token t
 * with routes j (topk_ids / topk_w device [T, k], as moe_route_topk writes
 * them), in fp32:
 *   W = sum of w_j over routes with 0 <= id_j < E (in j order); resident
 *   routes (slot_of[id_j] >= 0) are kept; the non-resident ones are taken
 *   heaviest first (equal weights: lower j first) while the kept weight c
 *   (resident sum in j order, then each taken weight) is below
 *   min_weight * W; the rest, and ids outside [0, E), are skipped.
 *   If a valid route was skipped, kept weights become w_j * (W / c).
 *   min_weight >= 1 keeps every valid route unchanged (the full routing).
 * ids_out (device int32 [T, k]): the id, or -1 for a skipped route (which
 * moe_permute then drops); w_out (device fp32 [T, k]): the weight, 0 for a
 * skipped route.  They may alias topk_ids / topk_w.  miss_count (device int32
 * [E], overwritten): per expert, the kept routes that need it while it is not
 * resident -- the experts to copy in (moe_fill_slot) before the FFN.
 * 1 <= k <= 32, E <= 512; NaN min_weight returns MOE_E_ARG.  T = 0 only
 * zeroes miss_count (the route pointers may then be NULL).
 */
moe_status moe_min_weight(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k, int32_t E,
                          const int32_t* slot_of, float min_weight, int32_t* ids_out, float* w_out,
                          int32_t* miss_count, void* stream);

/*
 * The expert FFN of every kept route (prain README, "Expert formats": an
 * expert is its w13 and w2; weights are dequantised inside the kernels):
 *   for the route at position p (route i = sorted_route[p], token t = i / k,
 *   expert e):  g = W1_e x_t,  u = W3_e x_t,  h = act(g) * u,  o_p = W2_e h.
 *   pool        device, the slot pool; expert e's blob starts at
 *               pool + slot_of[e] * slot_bytes (slot_bytes >= moe_expert_bytes,
 *               a multiple of 256)
 *   slot_of     device int32 [E] (the table moe_permute was given)
 *   x           device [T, H], fp32 or bf16 (x_dtype); the kernels multiply in
 *               bf16 with fp32 accumulation (fp32 x is rounded to bf16)
 *   expert_offsets, sorted_route: device, from moe_permute
 *   out_routes  device [T*k, H] out, fp32 or bf16 (out_dtype): row p is the
 *               output of the route at position p; rows from offsets[E] on are
 *               not written
 *   ws          device workspace of ws_bytes >= moe_workspace_bytes(...)
 * moe_ffn_gate_up and moe_ffn_down are its two halves, for callers that time
 * or schedule them apart: gate_up leaves h in ws, down reads it from there;
 * gate_up ignores out_routes, down ignores x (both accept NULL for them).
 * int4 weights: each expert group is computed by one of two kernel families
 * chosen on the device from its size (more than 8 routes, when T > 32: the
 * grouped MFMA GEMM; otherwise the streaming kernels); the result does not
 * depend on the stream arrangement above.
 */
moe_status moe_expert_ffn(const void* pool, uint64_t slot_bytes, const int32_t* slot_of, int32_t E,
                          int32_t H, int32_t FF, int32_t wfmt, int32_t act, const void* x,
                          int32_t x_dtype, int32_t T, int32_t k, const int32_t* expert_offsets,
                          const int32_t* sorted_route, void* out_routes, int32_t out_dtype,
                          void* ws, size_t ws_bytes, void* stream);

moe_status moe_ffn_gate_up(const void* pool, uint64_t slot_bytes, const int32_t* slot_of, int32_t E,
                           int32_t H, int32_t FF, int32_t wfmt, int32_t act, const void* x,
                           int32_t x_dtype, int32_t T, int32_t k, const int32_t* expert_offsets,
                           const int32_t* sorted_route, void* out_routes, int32_t out_dtype,
                           void* ws, size_t ws_bytes, void* stream);

moe_status moe_ffn_down(const void* pool, uint64_t slot_bytes, const int32_t* slot_of, int32_t E,
                        int32_t H, int32_t FF, int32_t wfmt, int32_t act, const void* x,
                        int32_t x_dtype, int32_t T, int32_t k, const int32_t* expert_offsets,
                        const int32_t* sorted_route, void* out_routes, int32_t out_dtype,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn without a workspace argument, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments (minus ws
 * and ws_bytes), results and errors as moe_expert_ffn.  The workspace is a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES (32 MiB) inside the
 * library, one per GPU, held from the first call on that GPU until the
 * process ends; its address is looked up once per device.  Calls whose
 * moe_workspace_bytes(T, k, E, H, FF, wfmt) exceeds the array return
 * MOE_E_WORKSPACE and enqueue nothing (at the Gemma-4-26B-A4B shape, up to
 * T = 1024 with top-8 fits).  The call allocates nothing.  Every call on one
 * GPU shares that GPU's array and nothing in it needs to start zeroed: calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_expert_ffn_noalloc(const void* pool, uint64_t slot_bytes, const int32_t* slot_of, int32_t E,
                                  int32_t H, int32_t FF, int32_t wfmt, int32_t act, const void* x,
                                  int32_t x_dtype, int32_t T, int32_t k, const int32_t* expert_offsets,
                                  const int32_t* sorted_route, void* out_routes, int32_t out_dtype,
                                  void* stream);

/*
 * Weighted scatter-combine back to token order (Winery-Strata
 * RemoteExperts::finish scatters each computed row back to its route; prain
 * README, "Trading quality for speed": a token's result is its routes weighted
 * by their router share):
 *   y[t] = sum over j = 0..k-1 with route_pos[t*k+j] >= 0 of
 *          topk_w[t*k+j] * out_routes[route_pos[t*k+j]]
 * accumulated in fp32 in ascending j; dropped routes add nothing and the
 * others are not rescaled.
 *   out_routes device [T*k, H] fp32 or bf16 (out_dtype)
 *   topk_w     device fp32 [T*k];  route_pos device int32 [T*k]
 *   y          device [T, H] out, fp32 or bf16 (y_dtype, rounded to nearest
 *              even)
 */
moe_status moe_combine(const void* out_routes, int32_t out_dtype, const float* topk_w,
                       const int32_t* route_pos, int32_t T, int32_t k, int32_t H, void* y,
                       int32_t y_dtype, void* stream);

/*
 * Quantise a bf16 matrix W [N, K] (device, row-major) into a packed format,
 * bit-exactly as the format defines (prain README, "Expert formats": int8 with
 * an fp32 scale per row; int4 with a bf16 scale per 64 elements chosen by an
 * MSE clip search).
 *   MOE_W_INT8_ROW: a = max |row|; s = a / 127 (fp32, IEEE division; 0 for a
 *     zero row); q = clamp(rint(w / s), -127, 127).  q device int8 [N, K],
 *     scales device fp32 [N].
 *   MOE_W_INT4_G64 (K % 64 == 0): per 64-element group with absmax a, try
 *     s_i = bf16(fp32(a * (20 - i)) / 140) for i = 0..9 (clip 1.00 down to
 *     0.55 of a / 7), codes q = clamp(rint(w / s_i), -8, 7) (0 if s_i = 0),
 *     squared error summed in fp64 in element order; keep the first smallest.
 *     q device uint8 [N, K/2] (low nibble = even element, value q + 8),
 *     scales device bf16 bits [N, K/64].
 */
moe_status moe_quantize(int32_t wfmt, const uint16_t* w_bf16, int32_t N, int32_t K, void* q,
                        void* scales, void* stream);

/*
 * Write one expert's blob (layout of moe_blob_layout) from its bf16 w13
 * [2FF, H] and w2 [H, FF] (device), quantising as moe_quantize does.  blob is
 * device memory of moe_expert_bytes() bytes; padding bytes are zeroed.
 */
moe_status moe_pack_expert(int32_t wfmt, const uint16_t* w13_bf16, const uint16_t* w2_bf16,
                           int32_t H, int32_t FF, void* blob, void* stream);

/*
 * Slot fill: make an expert resident (prain README, "int4 experts on RDNA2":
 * each int4 expert copy is one DMA through a pinned staging buffer and one
 * unpack kernel; Winery-Strata's ExpertCache fills and checks slots the same
 * way, admit / fill_slot_blocking / verify_slot).
 *
 * The canonical form of an expert -- what a pack file or host cache holds --
 * is the blob layout of moe_blob_layout with the int4 code blocks row-major
 * (byte b of row n at n * K/2 + b, as moe_quantize writes them); bf16 and int8
 * blobs are the same in both forms.  moe_fill_slot writes the slot form:
 *   src_on_host != 0: src is the canonical blob in host memory (pinned,
 *     hipHostMalloc, for an asynchronous copy; pageable memory works but the
 *     runtime copies it synchronously); one host-to-device copy of
 *     moe_expert_bytes() bytes into staging (device, caller-owned, at least
 *     that size, 16-byte aligned, not overlapping slot), then one kernel that
 *     writes slot from staging.
 *   src_on_host == 2: src is the canonical blob in pinned host memory
 *     (hipHostMalloc; anything else returns MOE_E_ARG); no copy: the kernel
 *     reads it over the bus through its device mapping.  staging is unused.
 *   src_on_host == 0: src is the canonical blob in device memory (16-byte
 *     aligned, not overlapping slot); staging is unused and may be NULL.
 * slot (device, 16-byte aligned, moe_expert_bytes() bytes) receives the blob
 * byte for byte as moe_pack_expert would write it from the same weights.
 * src and staging must stay valid until the stream reaches the copy and the
 * kernel.  Blobs of 2 GiB or more return MOE_E_SHAPE.
 */
moe_status moe_fill_slot(int32_t wfmt, const void* src, int32_t src_on_host, int32_t H, int32_t FF,
                         void* staging, void* slot, void* stream);

/*
 * n experts at once (0 <= n <= 64), as moe_fill_slot with src_on_host = 1 for
 * each: srcs (host array of n host pointers, pinned for asynchronous copies)
 * are copied back to back into staging (device, n * moe_expert_bytes() bytes,
 * 16-byte aligned), then one kernel unpacks all n into slots (host array of n
 * device pointers, 16-byte aligned, none overlapping staging).  The copy
 * engine runs the n copies without a hand-off to the compute queue between
 * them.  Same formats, layout rules and errors as moe_fill_slot.
 */
moe_status moe_fill_slots(int32_t wfmt, int32_t n, const void* const* srcs, int32_t H, int32_t FF, void* staging,
                          void* const* slots, void* stream);

/*
 * Check a filled slot against the canonical blob src (both device, 16-byte
 * aligned): *mismatches (device int32, overwritten) receives the number of
 * 16-byte chunks of the slot that differ from what moe_fill_slot writes.
 */
moe_status moe_verify_slot(int32_t wfmt, const void* src, int32_t H, int32_t FF, const void* slot,
                           int32_t* mismatches, void* stream);

/*
 * Host bookkeeping of a layer's expert -> slot table (host arrays): slot_of
 * [E] (-1 = not resident) and owner [S] (the expert in each slot, -1 = free).
 * Returns expert's slot when it is already resident, else claims the lowest
 * free slot (updating both tables), else returns -1 (moe_last_error says why;
 * also -1 for bad arguments).  Eviction is the caller's: set owner[j] and
 * slot_of[owner[j]] to -1.  The device copy of slot_of is the caller's.
 */
int32_t moe_slot_admit(int32_t* slot_of, int32_t E, int32_t* owner, int32_t S, int32_t expert);

#ifdef __cplusplus
}
#endif

#endif /* EXPERT_FFN_H */
