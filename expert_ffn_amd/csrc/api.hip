// C ABI of the routed expert FFN library: argument checks on the host, then
// one or more kernel launches on the caller's stream.  Nothing is enqueued when
// a check fails; the reason is kept per thread for moe_last_error().
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/expert_ffn.h"
#include "common.h"
#include "kernels.h"
#include <algorithm>

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fn, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(fn) + ": " + buf;
    return st;
}

moe_status hip_status(const char* fn, hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_E_HIP, fn, "%s", hipGetErrorString(e));
}

bool fmt_ok(int32_t f) { return f == MOE_W_BF16 || f == MOE_W_INT8_ROW || f == MOE_W_INT4_G64; }
bool dt_ok(int32_t d) { return d == MOE_F32 || d == MOE_BF16; }

uint64_t up256(uint64_t x) { return (x + 255u) / 256u * 256u; }

bool overlap(const void* a, const void* b, uint64_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + n && y < x + n;
}
bool al16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// layout of a blob; false if the shape does not fit the format
bool layout(int32_t wfmt, int32_t H, int32_t FF, uint64_t* off) {
    if (H < 1 || FF < 1 || !fmt_ok(wfmt)) return false;
    const uint64_t n13 = 2ull * FF * H, n2 = static_cast<uint64_t>(H) * FF;
    if (wfmt == MOE_W_BF16) {
        off[0] = 0;
        off[1] = off[2] = up256(n13 * 2);
        off[3] = off[4] = up256(off[2] + n2 * 2);
    } else if (wfmt == MOE_W_INT8_ROW) {
        off[0] = 0;
        off[1] = up256(n13);
        off[2] = up256(off[1] + 2ull * FF * 4);
        off[3] = up256(off[2] + n2);
        off[4] = up256(off[3] + static_cast<uint64_t>(H) * 4);
    } else {
        if (H % 64 || FF % 64) return false;
        off[0] = 0;
        off[1] = up256(n13 / 2);
        off[2] = up256(off[1] + 2ull * FF * (H / 64) * 2);
        off[3] = up256(off[2] + n2 / 2);
        off[4] = up256(off[3] + static_cast<uint64_t>(H) * (FF / 64) * 2);
    }
    return true;
}

// shape rules of the expert FFN kernels
moe_status check_ffn_shape(const char* fn, int32_t E, int32_t H, int32_t FF, int32_t wfmt,
                           int32_t T, int32_t k) {
    if (!fmt_ok(wfmt)) return fail(MOE_E_ARG, fn, "unknown weight format %d", wfmt);
    if (E < 1 || E > 512) return fail(MOE_E_SHAPE, fn, "E=%d outside [1, 512]", E);
    if (k < 1 || k > 32 || k > E) return fail(MOE_E_SHAPE, fn, "k=%d outside [1, min(E=%d, 32)]", k, E);
    if (T < 0) return fail(MOE_E_SHAPE, fn, "T=%d < 0", T);
    if (H < 64 || H % 64) return fail(MOE_E_SHAPE, fn, "H=%d is not a positive multiple of 64", H);
    const int ffq = wfmt == MOE_W_BF16 ? 32 : 64;
    if (FF < ffq || FF % ffq)
        return fail(MOE_E_SHAPE, fn, "FF=%d is not a positive multiple of %d for this format", FF, ffq);
    if (static_cast<int64_t>(T) * k > (1ll << 30)) return fail(MOE_E_SHAPE, fn, "T*k too large");
    // the kernels address activations and h with 31-bit buffer offsets
    if (static_cast<int64_t>(T) * H * 2 >= (1ll << 31) || static_cast<int64_t>(T) * k * FF * 2 >= (1ll << 31))
        return fail(MOE_E_SHAPE, fn, "T=%d too large for this H/FF (activation or h buffer >= 2 GiB)", T);
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

uint64_t moe_expert_bytes(int32_t wfmt, int32_t H, int32_t FF) {
    uint64_t off[5];
    return layout(wfmt, H, FF, off) ? off[4] : 0;
}

moe_status moe_blob_layout(int32_t wfmt, int32_t H, int32_t FF, uint64_t* off) {
    if (!off) return fail(MOE_E_ARG, "moe_blob_layout", "off is NULL");
    if (!fmt_ok(wfmt)) return fail(MOE_E_ARG, "moe_blob_layout", "unknown weight format %d", wfmt);
    if (!layout(wfmt, H, FF, off))
        return fail(MOE_E_SHAPE, "moe_blob_layout", "H=%d FF=%d invalid for format %d", H, FF, wfmt);
    return MOE_OK;
}

size_t moe_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t FF, int32_t wfmt) {
    (void)E;
    (void)wfmt;
    if (T < 0 || k < 1 || H < 1 || FF < 1) return 0;
    return moe::ffn_workspace(T, k, H, FF).bytes;
}

moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                          int32_t* topk_ids, float* topk_w, void* stream) {
    const char* fn = "moe_route_topk";
    if (!logits || !topk_ids || !topk_w) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (T < 0) return fail(MOE_E_SHAPE, fn, "T=%d < 0", T);
    if (E < 1 || E > 512) return fail(MOE_E_SHAPE, fn, "E=%d outside [1, 512]", E);
    if (k < 1 || k > 32 || k > E) return fail(MOE_E_SHAPE, fn, "k=%d outside [1, min(E=%d, 32)]", k, E);
    if (T == 0) return MOE_OK;
    return hip_status(fn, moe::launch_route_topk(logits, T, E, k, renorm, topk_ids, topk_w,
                                                 static_cast<hipStream_t>(stream)));
}

size_t moe_router_ws_bytes(int32_t T, int32_t H, int32_t E) {
    if (T <= 0 || H < 1 || E < 1) return 256;
    return up256(static_cast<uint64_t>(moe::router_part_floats(T, H, E)) * 4);
}

moe_status moe_router_topk(const void* x, int32_t x_dtype, int32_t T, int32_t H, const float* w_router, int32_t E,
                           int32_t k, int32_t renorm, float* logits, void* ws, size_t ws_bytes, int32_t* topk_ids,
                           float* topk_w, void* stream) {
    const char* fn = "moe_router_topk";
    if (T < 0) return fail(MOE_E_SHAPE, fn, "T=%d < 0", T);
    if (T > 0 && (!x || !w_router || !logits || !ws || !topk_ids || !topk_w))
        return fail(MOE_E_ARG, fn, "null pointer argument");
    if (!dt_ok(x_dtype)) return fail(MOE_E_ARG, fn, "unknown dtype %d", x_dtype);
    if (E < 1 || E > 512) return fail(MOE_E_SHAPE, fn, "E=%d outside [1, 512]", E);
    if (k < 1 || k > 32 || k > E) return fail(MOE_E_SHAPE, fn, "k=%d outside [1, min(E=%d, 32)]", k, E);
    if (H < 64 || H % 64) return fail(MOE_E_SHAPE, fn, "H=%d is not a positive multiple of 64", H);
    if (static_cast<int64_t>(T) * H >= (1ll << 31) || moe::router_part_floats(T, H, E) >= (1ll << 31))
        return fail(MOE_E_SHAPE, fn, "T=%d too large", T);
    if (T == 0) return MOE_OK;
    if (ws_bytes < moe_router_ws_bytes(T, H, E))
        return fail(MOE_E_WORKSPACE, fn, "ws_bytes=%zu < %zu", ws_bytes, moe_router_ws_bytes(T, H, E));
    if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(w_router) % 16 ||
        reinterpret_cast<uintptr_t>(ws) % 16)
        return fail(MOE_E_ARG, fn, "x, w_router and ws must be 16-byte aligned");
    return hip_status(fn, moe::launch_router_topk(x, x_dtype == MOE_F32, w_router, T, H, E, k, renorm, logits,
                                                  static_cast<float*>(ws), topk_ids, topk_w,
                                                  static_cast<hipStream_t>(stream)));
}

moe_status moe_residency_refresh(const int32_t* ids, int64_t R, int32_t E, int32_t budget, int32_t n_slots,
                                 int32_t* slot_of, int32_t* hits, int32_t* target, int32_t* promote,
                                 int32_t* promote_slot, int32_t* demote, int32_t* counts, void* stream) {
    const char* fn = "moe_residency_refresh";
    if (!slot_of || !hits || !target || !promote || !promote_slot || !demote || !counts || (R > 0 && !ids))
        return fail(MOE_E_ARG, fn, "null pointer argument");
    if (R < 0) return fail(MOE_E_SHAPE, fn, "R=%lld < 0", static_cast<long long>(R));
    if (E < 1 || E > 512) return fail(MOE_E_SHAPE, fn, "E=%d outside [1, 512]", E);
    if (budget < 0 || budget > E) return fail(MOE_E_SHAPE, fn, "budget=%d outside [0, E=%d]", budget, E);
    if (n_slots < budget || n_slots > 512)
        return fail(MOE_E_SHAPE, fn, "n_slots=%d outside [budget=%d, 512]", n_slots, budget);
    return hip_status(fn, moe::launch_residency_refresh(ids, R, E, budget, n_slots, slot_of, hits, target, promote,
                                                        promote_slot, demote, counts,
                                                        static_cast<hipStream_t>(stream)));
}

int32_t moe_refresh_due(int32_t every, int64_t step, int32_t prefill_block, int32_t offload) {
    if (!offload) return 0;
    if (prefill_block || every <= 1) return 1;
    return step % every == 0 ? 1 : 0;
}

int32_t moe_budget_from_memory(uint64_t free_bytes, uint64_t reserve_bytes, uint64_t expert_bytes, int32_t layers,
                               int32_t max_per_layer, int32_t E) {
    const int64_t cap = std::min<int64_t>(max_per_layer, E);
    if (expert_bytes == 0 || layers <= 0) return static_cast<int32_t>(std::max<int64_t>(cap, 0));
    const uint64_t usable = free_bytes > reserve_bytes ? free_bytes - reserve_bytes : 0;
    const uint64_t per_layer = usable / (expert_bytes * static_cast<uint64_t>(layers));
    return static_cast<int32_t>(std::max<int64_t>(std::min<int64_t>(static_cast<int64_t>(std::min<uint64_t>(per_layer, 1u << 30)), cap), 0));
}

moe_status moe_min_weight(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k, int32_t E,
                          const int32_t* slot_of, float min_weight, int32_t* ids_out, float* w_out,
                          int32_t* miss_count, void* stream) {
    const char* fn = "moe_min_weight";
    if (!slot_of || !miss_count || (T > 0 && (!topk_ids || !topk_w || !ids_out || !w_out)))
        return fail(MOE_E_ARG, fn, "null pointer argument");
    if (T < 0) return fail(MOE_E_SHAPE, fn, "T=%d < 0", T);
    if (E < 1 || E > 512) return fail(MOE_E_SHAPE, fn, "E=%d outside [1, 512]", E);
    if (k < 1 || k > 32) return fail(MOE_E_SHAPE, fn, "k=%d outside [1, 32]", k);
    if (min_weight != min_weight) return fail(MOE_E_ARG, fn, "min_weight is NaN");
    return hip_status(fn, moe::launch_min_weight(topk_ids, topk_w, T, k, E, slot_of, min_weight, ids_out, w_out,
                                                 miss_count, static_cast<hipStream_t>(stream)));
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       const int32_t* slot_of, int32_t* expert_offsets, int32_t* sorted_route,
                       int32_t* route_pos, int32_t* n_dropped, void* stream) {
    const char* fn = "moe_permute";
    if (!slot_of || !expert_offsets || !n_dropped) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (T < 0) return fail(MOE_E_SHAPE, fn, "T=%d < 0", T);
    if (T > 0 && (!topk_ids || !sorted_route || !route_pos)) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (E < 1 || E > 512) return fail(MOE_E_SHAPE, fn, "E=%d outside [1, 512]", E);
    if (k < 1 || k > 32 || k > E) return fail(MOE_E_SHAPE, fn, "k=%d outside [1, min(E=%d, 32)]", k, E);
    if (static_cast<int64_t>(T) * k > (1ll << 30)) return fail(MOE_E_SHAPE, fn, "T*k too large");
    return hip_status(fn, moe::launch_permute(topk_ids, T * k, E, slot_of, expert_offsets, sorted_route,
                                              route_pos, n_dropped, static_cast<hipStream_t>(stream)));
}

moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                             const int32_t* slot_of, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                             int32_t* sorted_route, int32_t* route_pos, int32_t* n_dropped, void* stream) {
    const char* fn = "moe_route_permute";
    if (!slot_of || !expert_offsets || !n_dropped) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (T < 0) return fail(MOE_E_SHAPE, fn, "T=%d < 0", T);
    if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_route || !route_pos))
        return fail(MOE_E_ARG, fn, "null pointer argument");
    if (E < 1 || E > 512) return fail(MOE_E_SHAPE, fn, "E=%d outside [1, 512]", E);
    if (k < 1 || k > 32 || k > E) return fail(MOE_E_SHAPE, fn, "k=%d outside [1, min(E=%d, 32)]", k, E);
    if (static_cast<int64_t>(T) * k > (1ll << 30)) return fail(MOE_E_SHAPE, fn, "T*k too large");
    if (T == 0)   // offsets and the dropped count are still written
        return hip_status(fn, moe::launch_permute(topk_ids, 0, E, slot_of, expert_offsets, sorted_route, route_pos,
                                                  n_dropped, static_cast<hipStream_t>(stream)));
    return hip_status(fn, moe::launch_route_permute(logits, T, E, k, renorm, slot_of, topk_ids, topk_w,
                                                    expert_offsets, sorted_route, route_pos, n_dropped,
                                                    static_cast<hipStream_t>(stream)));
}

static moe_status ffn_entry(const char* fn, int phases, const void* pool, uint64_t slot_bytes,
                            const int32_t* slot_of, int32_t E, int32_t H, int32_t FF, int32_t wfmt,
                            int32_t act, const void* x, int32_t x_dtype, int32_t T, int32_t k,
                            const int32_t* expert_offsets, const int32_t* sorted_route,
                            void* out_routes, int32_t out_dtype, void* ws, size_t ws_bytes,
                            void* stream, bool fork = true) {
    moe_status st = check_ffn_shape(fn, E, H, FF, wfmt, T, k);
    if (st != MOE_OK) return st;
    if (!pool || !slot_of || !expert_offsets || !sorted_route || !ws)
        return fail(MOE_E_ARG, fn, "null pointer argument");
    if ((phases & 1) && !x) return fail(MOE_E_ARG, fn, "x is NULL");
    if ((phases & 2) && !out_routes) return fail(MOE_E_ARG, fn, "out_routes is NULL");
    if (act != MOE_ACT_GELU_TANH && act != MOE_ACT_SILU) return fail(MOE_E_ARG, fn, "unknown activation %d", act);
    if (!dt_ok(x_dtype) || !dt_ok(out_dtype)) return fail(MOE_E_ARG, fn, "unknown dtype");
    uint64_t off[5];
    layout(wfmt, H, FF, off);
    if (slot_bytes < off[4] || slot_bytes % 256)
        return fail(MOE_E_ARG, fn, "slot_bytes=%llu must be a multiple of 256 and >= %llu",
                    static_cast<unsigned long long>(slot_bytes), static_cast<unsigned long long>(off[4]));
    if (reinterpret_cast<uintptr_t>(pool) % 256) return fail(MOE_E_ARG, fn, "pool is not 256-byte aligned");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MOE_E_ARG, fn, "ws is not 256-byte aligned");
    if ((phases & 1) && reinterpret_cast<uintptr_t>(x) % 16) return fail(MOE_E_ARG, fn, "x is not 16-byte aligned");
    if ((phases & 2) && reinterpret_cast<uintptr_t>(out_routes) % 16)
        return fail(MOE_E_ARG, fn, "out_routes is not 16-byte aligned");
    const moe::FfnWorkspace wl = moe::ffn_workspace(T, k, H, FF);
    if (ws_bytes < wl.bytes)
        return fail(MOE_E_WORKSPACE, fn, "ws_bytes=%zu < %zu needed", ws_bytes, wl.bytes);
    if (T == 0) return MOE_OK;
    moe::FfnParams P{};
    P.pool = static_cast<const uint8_t*>(pool);
    P.slot_bytes = slot_bytes;
    P.slot_of = slot_of;
    P.E = E; P.H = H; P.FF = FF; P.fmt = wfmt; P.act = act; P.T = T; P.k = k;
    P.kmul = moe::token_multiplier(k);
    P.offsets = expert_offsets;
    P.sorted_route = sorted_route;
    P.x = x;
    P.x_dt = x_dtype;
    P.xq = nullptr;
    P.xq_out = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + wl.xq_off);
    P.xsum = nullptr;
    P.xsum_out = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + wl.xsum_off);
    P.xqg_out = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + wl.xqg_off);
    P.xsumg_out = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + wl.xsumg_off);
    P.h = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + wl.h_off);
    P.hsum = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + wl.hsum_off);
    P.out = out_routes;
    P.out_dt = out_dtype;
    P.o13 = off[0]; P.os13 = off[1]; P.o2 = off[2]; P.os2 = off[3];
    return hip_status(fn, moe::launch_ffn(P, phases, static_cast<hipStream_t>(stream), fork));
}

#define FFN_ARGS pool, slot_bytes, slot_of, E, H, FF, wfmt, act, x, x_dtype, T, k, expert_offsets, \
                 sorted_route, out_routes, out_dtype, ws, ws_bytes, stream
#define FFN_PARAMS const void *pool, uint64_t slot_bytes, const int32_t *slot_of, int32_t E, int32_t H, \
                   int32_t FF, int32_t wfmt, int32_t act, const void *x, int32_t x_dtype, int32_t T,  \
                   int32_t k, const int32_t *expert_offsets, const int32_t *sorted_route,             \
                   void *out_routes, int32_t out_dtype, void *ws, size_t ws_bytes, void *stream

moe_status moe_expert_ffn(FFN_PARAMS) { return ffn_entry("moe_expert_ffn", 3, FFN_ARGS); }
moe_status moe_ffn_gate_up(FFN_PARAMS) { return ffn_entry("moe_ffn_gate_up", 1, FFN_ARGS); }
moe_status moe_ffn_down(FFN_PARAMS) { return ffn_entry("moe_ffn_down", 2, FFN_ARGS); }

}  // extern "C"

// Workspace of moe_expert_ffn_noalloc: one array per device, allocated when the
// library's code object is loaded on it and held until the process ends.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
// Device address of this device's scratch array, looked up once per device
// (the array's name is a host-side stand-in; kernels get this address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

extern "C" {

moe_status moe_expert_ffn_noalloc(const void* pool, uint64_t slot_bytes, const int32_t* slot_of, int32_t E,
                                  int32_t H, int32_t FF, int32_t wfmt, int32_t act, const void* x,
                                  int32_t x_dtype, int32_t T, int32_t k, const int32_t* expert_offsets,
                                  const int32_t* sorted_route, void* out_routes, int32_t out_dtype,
                                  void* stream) {
    const char* fn = "moe_expert_ffn_noalloc";
    moe_status st = check_ffn_shape(fn, E, H, FF, wfmt, T, k);
    if (st != MOE_OK) return st;
    const size_t need = moe::ffn_workspace(T, k, H, FF).bytes;
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_E_WORKSPACE, fn, "T=%d k=%d H=%d FF=%d needs %zu workspace bytes > the %u-byte scratch array",
                    T, k, H, FF, need, static_cast<unsigned>(MOE_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_status(fn, e);
    // one stream only: a second stream and its events would be created on the first call
    return ffn_entry(fn, 3, pool, slot_bytes, slot_of, E, H, FF, wfmt, act, x, x_dtype, T, k, expert_offsets,
                     sorted_route, out_routes, out_dtype, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, false);
}

moe_status moe_combine(const void* out_routes, int32_t out_dtype, const float* topk_w,
                       const int32_t* route_pos, int32_t T, int32_t k, int32_t H, void* y,
                       int32_t y_dtype, void* stream) {
    const char* fn = "moe_combine";
    if (!out_routes || !topk_w || !route_pos || !y) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (!dt_ok(out_dtype) || !dt_ok(y_dtype)) return fail(MOE_E_ARG, fn, "unknown dtype");
    if (T < 0) return fail(MOE_E_SHAPE, fn, "T=%d < 0", T);
    if (k < 1 || k > 32) return fail(MOE_E_SHAPE, fn, "k=%d outside [1, 32]", k);
    if (H < 8 || H % 8) return fail(MOE_E_SHAPE, fn, "H=%d is not a positive multiple of 8", H);
    if (reinterpret_cast<uintptr_t>(out_routes) % 16 || reinterpret_cast<uintptr_t>(y) % 16)
        return fail(MOE_E_ARG, fn, "out_routes and y must be 16-byte aligned");
    if (T == 0) return MOE_OK;
    return hip_status(fn, moe::launch_combine(out_routes, out_dtype, topk_w, route_pos, T, k, H, y,
                                              y_dtype, static_cast<hipStream_t>(stream)));
}

moe_status moe_quantize(int32_t wfmt, const uint16_t* w_bf16, int32_t N, int32_t K, void* q,
                        void* scales, void* stream) {
    const char* fn = "moe_quantize";
    if (!w_bf16 || !q || !scales) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (wfmt != MOE_W_INT8_ROW && wfmt != MOE_W_INT4_G64)
        return fail(MOE_E_ARG, fn, "format %d is not a quantised format", wfmt);
    if (N < 0 || K < 1) return fail(MOE_E_SHAPE, fn, "N=%d K=%d", N, K);
    if (wfmt == MOE_W_INT4_G64 && K % 64) return fail(MOE_E_SHAPE, fn, "K=%d is not a multiple of 64", K);
    return hip_status(fn, moe::launch_quantize(wfmt, w_bf16, N, K, q, scales, false,
                                               static_cast<hipStream_t>(stream)));
}

moe_status moe_pack_expert(int32_t wfmt, const uint16_t* w13_bf16, const uint16_t* w2_bf16,
                           int32_t H, int32_t FF, void* blob, void* stream) {
    const char* fn = "moe_pack_expert";
    if (!w13_bf16 || !w2_bf16 || !blob) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (!fmt_ok(wfmt)) return fail(MOE_E_ARG, fn, "unknown weight format %d", wfmt);
    uint64_t off[5];
    if (!layout(wfmt, H, FF, off)) return fail(MOE_E_SHAPE, fn, "H=%d FF=%d invalid for format %d", H, FF, wfmt);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* b = static_cast<uint8_t*>(blob);
    hipError_t e = hipMemsetAsync(blob, 0, off[4], s);
    if (e != hipSuccess) return hip_status(fn, e);
    if (wfmt == MOE_W_BF16) {
        e = hipMemcpyAsync(b + off[0], w13_bf16, 2ull * FF * H * 2, hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(b + off[2], w2_bf16, static_cast<uint64_t>(H) * FF * 2, hipMemcpyDeviceToDevice, s);
        return hip_status(fn, e);
    }
    e = moe::launch_quantize(wfmt, w13_bf16, 2 * FF, H, b + off[0], b + off[1], true, s);
    if (e == hipSuccess) e = moe::launch_quantize(wfmt, w2_bf16, H, FF, b + off[2], b + off[3], true, s);
    return hip_status(fn, e);
}

moe_status moe_fill_slot(int32_t wfmt, const void* src, int32_t src_on_host, int32_t H, int32_t FF,
                         void* staging, void* slot, void* stream) {
    const char* fn = "moe_fill_slot";
    if (!src || !slot) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (!fmt_ok(wfmt)) return fail(MOE_E_ARG, fn, "unknown weight format %d", wfmt);
    uint64_t off[5];
    if (!layout(wfmt, H, FF, off)) return fail(MOE_E_SHAPE, fn, "H=%d FF=%d invalid for format %d", H, FF, wfmt);
    if (off[4] >= (1ull << 31)) return fail(MOE_E_SHAPE, fn, "blob of %llu bytes is not below 2 GiB",
                                            static_cast<unsigned long long>(off[4]));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const void* dev = src;
    if (src_on_host == 2) {
        // the kernel reads the pinned host blob itself (its device-side mapping)
        void* mapped = nullptr;
        if (hipHostGetDevicePointer(&mapped, const_cast<void*>(src), 0) != hipSuccess || !mapped) {
            (void)hipGetLastError();
            return fail(MOE_E_ARG, fn, "src is not pinned (hipHostMalloc) host memory");
        }
        if (!al16(mapped) || !al16(slot)) return fail(MOE_E_ARG, fn, "src and slot must be 16-byte aligned");
        dev = mapped;
    } else if (src_on_host) {
        if (!staging) return fail(MOE_E_ARG, fn, "a host source needs a device staging buffer");
        if (!al16(staging) || !al16(slot)) return fail(MOE_E_ARG, fn, "staging and slot must be 16-byte aligned");
        if (overlap(staging, slot, off[4])) return fail(MOE_E_ARG, fn, "staging overlaps the slot");
        const hipError_t e = hipMemcpyAsync(staging, src, off[4], hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(fn, e);
        dev = staging;
    } else {
        if (!al16(src) || !al16(slot)) return fail(MOE_E_ARG, fn, "src and slot must be 16-byte aligned");
        if (overlap(src, slot, off[4])) return fail(MOE_E_ARG, fn, "src overlaps the slot");
    }
    return hip_status(fn, moe::launch_fill_slot(wfmt, dev, src_on_host == 2, H, FF, off, slot, s));
}

moe_status moe_fill_slots(int32_t wfmt, int32_t n, const void* const* srcs, int32_t H, int32_t FF, void* staging,
                          void* const* slots, void* stream) {
    const char* fn = "moe_fill_slots";
    if (n < 0 || n > moe::FILL_MAX) return fail(MOE_E_SHAPE, fn, "n=%d outside [0, %d]", n, moe::FILL_MAX);
    if (!fmt_ok(wfmt)) return fail(MOE_E_ARG, fn, "unknown weight format %d", wfmt);
    uint64_t off[5];
    if (!layout(wfmt, H, FF, off)) return fail(MOE_E_SHAPE, fn, "H=%d FF=%d invalid for format %d", H, FF, wfmt);
    if (off[4] >= (1ull << 31)) return fail(MOE_E_SHAPE, fn, "blob of %llu bytes is not below 2 GiB",
                                            static_cast<unsigned long long>(off[4]));
    if (n == 0) return MOE_OK;
    if (!srcs || !slots || !staging) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (!al16(staging)) return fail(MOE_E_ARG, fn, "staging must be 16-byte aligned");
    for (int32_t j = 0; j < n; ++j) {
        if (!srcs[j] || !slots[j]) return fail(MOE_E_ARG, fn, "null pointer for expert %d", j);
        if (!al16(slots[j])) return fail(MOE_E_ARG, fn, "slot %d is not 16-byte aligned", j);
        const uintptr_t a = reinterpret_cast<uintptr_t>(slots[j]), b = reinterpret_cast<uintptr_t>(staging);
        if (a < b + n * off[4] && b < a + off[4]) return fail(MOE_E_ARG, fn, "slot %d overlaps the staging buffer", j);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* st = static_cast<uint8_t*>(staging);
    for (int32_t j = 0; j < n; ++j) {
        const hipError_t e = hipMemcpyAsync(st + j * off[4], srcs[j], off[4], hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(fn, e);
    }
    return hip_status(fn, moe::launch_fill_slots(wfmt, staging, n, H, FF, off, slots, s));
}

moe_status moe_verify_slot(int32_t wfmt, const void* src, int32_t H, int32_t FF, const void* slot,
                           int32_t* mismatches, void* stream) {
    const char* fn = "moe_verify_slot";
    if (!src || !slot || !mismatches) return fail(MOE_E_ARG, fn, "null pointer argument");
    if (!fmt_ok(wfmt)) return fail(MOE_E_ARG, fn, "unknown weight format %d", wfmt);
    uint64_t off[5];
    if (!layout(wfmt, H, FF, off)) return fail(MOE_E_SHAPE, fn, "H=%d FF=%d invalid for format %d", H, FF, wfmt);
    if (off[4] >= (1ull << 31)) return fail(MOE_E_SHAPE, fn, "blob of %llu bytes is not below 2 GiB",
                                            static_cast<unsigned long long>(off[4]));
    if (!al16(src) || !al16(slot)) return fail(MOE_E_ARG, fn, "src and slot must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(mismatches) % 4) return fail(MOE_E_ARG, fn, "mismatches must be 4-byte aligned");
    return hip_status(fn, moe::launch_verify_slot(wfmt, src, H, FF, off, slot, mismatches,
                                                  static_cast<hipStream_t>(stream)));
}

int32_t moe_slot_admit(int32_t* slot_of, int32_t E, int32_t* owner, int32_t S, int32_t expert) {
    const char* fn = "moe_slot_admit";
    if (!slot_of || !owner) return fail(MOE_E_ARG, fn, "null pointer argument"), -1;
    if (E < 1 || S < 0 || expert < 0 || expert >= E)
        return fail(MOE_E_ARG, fn, "expert=%d outside [0, E=%d) or S=%d < 0", expert, E, S), -1;
    const int32_t cur = slot_of[expert];
    if (cur >= 0 && cur < S && owner[cur] == expert) return cur;
    for (int32_t j = 0; j < S; ++j)
        if (owner[j] < 0) {
            owner[j] = expert;
            slot_of[expert] = j;
            return j;
        }
    return fail(MOE_E_ARG, fn, "no free slot among %d", S), -1;
}

}  // extern "C"
