"""Python binding of libexpert_ffn.so (the C ABI in include/expert_ffn.h).

Argument marshalling only: every function passes torch tensors' device
pointers, sizes and torch's current HIP stream to the C entry point of the same
name and raises MoeError on a non-OK status.  There is no fallback: without the
built library, importing the first entry point raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libexpert_ffn.so")

F32, BF16 = 0, 1
W_BF16, W_INT8_ROW, W_INT4_G64 = 0, 1, 2
ACT_GELU_TANH, ACT_SILU = 0, 1
FMT_NAMES = {"bf16": W_BF16, "int8": W_INT8_ROW, "int4": W_INT4_G64}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"status {status}: {message}")
        self.status = status


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_expert_bytes.argtypes = [i32, i32, i32]
        L.moe_expert_bytes.restype = u64
        L.moe_blob_layout.argtypes = [i32, i32, i32, P]
        L.moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_route_topk.argtypes = [P, i32, i32, i32, i32, P, P, P]
        L.moe_permute.argtypes = [P, i32, i32, i32, P, P, P, P, P, P]
        L.moe_route_permute.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
        ffn = [P, u64, P, i32, i32, i32, i32, i32, P, i32, i32, i32, P, P, P, i32, P, sz, P]
        for name in ("moe_expert_ffn", "moe_ffn_gate_up", "moe_ffn_down"):
            getattr(L, name).argtypes = ffn
        L.moe_expert_ffn_noalloc.argtypes = ffn[:16] + [P]
        L.moe_combine.argtypes = [P, i32, P, P, i32, i32, i32, P, i32, P]
        L.moe_quantize.argtypes = [i32, P, i32, i32, P, P, P]
        L.moe_pack_expert.argtypes = [i32, P, P, i32, i32, P, P]
        L.moe_router_ws_bytes.argtypes = [i32, i32, i32]
        L.moe_router_ws_bytes.restype = sz
        L.moe_router_topk.argtypes = [P, i32, i32, i32, P, i32, i32, i32, P, P, sz, P, P, P]
        L.moe_residency_refresh.argtypes = [P, ctypes.c_int64, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.moe_refresh_due.argtypes = [i32, ctypes.c_int64, i32, i32]
        L.moe_refresh_due.restype = i32
        L.moe_budget_from_memory.argtypes = [u64, u64, u64, i32, i32, i32]
        L.moe_budget_from_memory.restype = i32
        L.moe_min_weight.argtypes = [P, P, i32, i32, i32, P, ctypes.c_float, P, P, P, P]
        L.moe_fill_slot.argtypes = [i32, P, i32, i32, i32, P, P, P]
        L.moe_fill_slots.argtypes = [i32, i32, P, i32, i32, P, P, P]
        L.moe_verify_slot.argtypes = [i32, P, i32, i32, P, P, P]
        L.moe_slot_admit.argtypes = [P, i32, P, i32, i32]
        for name in ("moe_blob_layout", "moe_route_topk", "moe_permute", "moe_route_permute", "moe_expert_ffn",
                     "moe_ffn_gate_up", "moe_ffn_down", "moe_expert_ffn_noalloc", "moe_combine", "moe_quantize",
                     "moe_pack_expert", "moe_router_topk", "moe_residency_refresh", "moe_min_weight", "moe_fill_slot", "moe_fill_slots", "moe_verify_slot",
                     "moe_slot_admit"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------ host queries --
def expert_bytes(fmt: int, H: int, FF: int) -> int:
    return int(lib().moe_expert_bytes(fmt, H, FF))


def blob_layout(fmt: int, H: int, FF: int):
    off = (ctypes.c_uint64 * 5)()
    _check(lib().moe_blob_layout(fmt, H, FF, off))
    return [int(v) for v in off]


def workspace_bytes(T: int, k: int, E: int, H: int, FF: int, fmt: int) -> int:
    return int(lib().moe_workspace_bytes(T, k, E, H, FF, fmt))


# ------------------------------------------------------------- the steps --
def route_topk(logits, k: int, topk_ids, topk_w, renorm: int = 1, stream=None):
    T, E = logits.shape
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, renorm, _ptr(topk_ids), _ptr(topk_w),
                                _stream(stream)))


def permute(topk_ids, E: int, slot_of, expert_offsets, sorted_route, route_pos, n_dropped,
            stream=None):
    T, k = topk_ids.shape
    _check(lib().moe_permute(_ptr(topk_ids), T, k, E, _ptr(slot_of), _ptr(expert_offsets),
                             _ptr(sorted_route), _ptr(route_pos), _ptr(n_dropped), _stream(stream)))


def route_permute(logits, k: int, slot_of, topk_ids, topk_w, expert_offsets, sorted_route, route_pos,
                  n_dropped, renorm: int = 1, stream=None):
    T, E = logits.shape
    _check(lib().moe_route_permute(_ptr(logits), T, E, k, renorm, _ptr(slot_of), _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(expert_offsets), _ptr(sorted_route), _ptr(route_pos), _ptr(n_dropped),
                                   _stream(stream)))


def _ffn(name, pool, slot_bytes, slot_of, E, H, FF, fmt, act, x, T, k, expert_offsets,
         sorted_route, out_routes, ws, stream):
    x_dt = _dt(x) if x is not None else BF16
    o_dt = _dt(out_routes) if out_routes is not None else F32
    _check(getattr(lib(), name)(_ptr(pool), slot_bytes, _ptr(slot_of), E, H, FF, fmt, act, _ptr(x),
                                x_dt, T, k, _ptr(expert_offsets), _ptr(sorted_route),
                                _ptr(out_routes), o_dt, _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)))


def expert_ffn(pool, slot_bytes, slot_of, E, H, FF, fmt, act, x, k, expert_offsets, sorted_route,
               out_routes, ws, stream=None):
    _ffn("moe_expert_ffn", pool, slot_bytes, slot_of, E, H, FF, fmt, act, x, x.shape[0], k,
         expert_offsets, sorted_route, out_routes, ws, stream)


def expert_ffn_noalloc(pool, slot_bytes, slot_of, E, H, FF, fmt, act, x, k, expert_offsets, sorted_route,
                       out_routes, stream=None):
    """moe_expert_ffn_noalloc: the library's static scratch array is the workspace."""
    _check(lib().moe_expert_ffn_noalloc(_ptr(pool), slot_bytes, _ptr(slot_of), E, H, FF, fmt, act, _ptr(x),
                                        _dt(x), x.shape[0], k, _ptr(expert_offsets), _ptr(sorted_route),
                                        _ptr(out_routes), _dt(out_routes), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def ffn_gate_up(pool, slot_bytes, slot_of, E, H, FF, fmt, act, x, k, expert_offsets,
                sorted_route, ws, stream=None):
    _ffn("moe_ffn_gate_up", pool, slot_bytes, slot_of, E, H, FF, fmt, act, x, x.shape[0], k,
         expert_offsets, sorted_route, None, ws, stream)


def ffn_down(pool, slot_bytes, slot_of, E, H, FF, fmt, T, k, expert_offsets, sorted_route,
             out_routes, ws, stream=None):
    _ffn("moe_ffn_down", pool, slot_bytes, slot_of, E, H, FF, fmt, ACT_GELU_TANH, None, T, k,
         expert_offsets, sorted_route, out_routes, ws, stream)


def combine(out_routes, topk_w, route_pos, y, stream=None):
    T, H = y.shape
    k = topk_w.numel() // T if T else 1
    _check(lib().moe_combine(_ptr(out_routes), _dt(out_routes), _ptr(topk_w), _ptr(route_pos), T, k,
                             H, _ptr(y), _dt(y), _stream(stream)))


def quantize(fmt: int, w_bf16, q, scales, stream=None):
    N, K = w_bf16.shape
    _check(lib().moe_quantize(fmt, _ptr(w_bf16), N, K, _ptr(q), _ptr(scales), _stream(stream)))


def pack_expert(fmt: int, w13_bf16, w2_bf16, blob, stream=None):
    H = w13_bf16.shape[1]
    FF = w2_bf16.shape[1]
    _check(lib().moe_pack_expert(fmt, _ptr(w13_bf16), _ptr(w2_bf16), H, FF, _ptr(blob),
                                 _stream(stream)))


def fill_slot(fmt: int, src, H: int, FF: int, slot, staging=None, stream=None, direct=False):
    """Canonical blob src (host: one copy into staging, then the unpack kernel,
    or with direct=True the kernel reading the pinned blob itself; device: the
    kernel alone) -> slot, byte for byte the packed blob."""
    on_host = 0 if src.is_cuda else (2 if direct else 1)
    _check(lib().moe_fill_slot(fmt, _ptr(src), on_host, H, FF, _ptr(staging), _ptr(slot), _stream(stream)))


def fill_slots(fmt: int, srcs, H: int, FF: int, slots, staging, stream=None):
    """Canonical blobs srcs (host tensors) -> slots (device tensors): the
    copies back to back into staging, then one unpack kernel for all."""
    n = len(srcs)
    assert len(slots) == n
    src_arr = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in srcs])
    dst_arr = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in slots])
    _check(lib().moe_fill_slots(fmt, n, src_arr, H, FF, _ptr(staging), dst_arr, _stream(stream)))


def verify_slot(fmt: int, src, H: int, FF: int, slot, mismatches, stream=None):
    """mismatches[0] <- 16-byte chunks of slot that differ from the fill of src."""
    _check(lib().moe_verify_slot(fmt, _ptr(src), H, FF, _ptr(slot), _ptr(mismatches), _stream(stream)))


def slot_admit(slot_of, owner, expert: int) -> int:
    """Host int32 tables slot_of [E], owner [S]: expert's slot, claiming the
    lowest free one if it is not resident; raises when none is free."""
    import torch
    assert slot_of.dtype == torch.int32 and owner.dtype == torch.int32
    assert not slot_of.is_cuda and not owner.is_cuda and slot_of.is_contiguous() and owner.is_contiguous()
    j = lib().moe_slot_admit(_ptr(slot_of), slot_of.numel(), _ptr(owner), owner.numel(), expert)
    if j < 0:
        raise MoeError(1, lib().moe_last_error().decode())
    return j


def min_weight(ids, w, E: int, slot_of, share: float, ids_out, w_out, miss_count, stream=None):
    """min_weight partial routing of topk ids/w [T, k] (outputs may alias them)."""
    T, k = ids.shape
    _check(lib().moe_min_weight(_ptr(ids), _ptr(w), T, k, E, _ptr(slot_of), ctypes.c_float(share), _ptr(ids_out),
                                _ptr(w_out), _ptr(miss_count), _stream(stream)))


def router_ws_bytes(T: int, H: int, E: int) -> int:
    """Bytes of the workspace router_topk needs for T tokens."""
    return int(lib().moe_router_ws_bytes(T, H, E))


def router_topk(x, w_router, k: int, logits, ws, ids, w, renorm: int = 1, stream=None):
    """fp32 router GEMV of x [T, H] with w_router [E, H], then the top-k (two launches)."""
    T, H = x.shape
    E = w_router.shape[0]
    _check(lib().moe_router_topk(_ptr(x), _dt(x), T, H, _ptr(w_router), E, k, renorm, _ptr(logits), _ptr(ws),
                                 ws.numel() * ws.element_size(), _ptr(ids), _ptr(w), _stream(stream)))


def residency_refresh(ids, E: int, budget: int, n_slots: int, slot_of, hits, target, promote, promote_slot, demote,
                      counts, stream=None):
    """Hit counts, top-budget target and paired promote/demote; slot_of is rewritten in place."""
    _check(lib().moe_residency_refresh(_ptr(ids), ids.numel(), E, budget, n_slots, _ptr(slot_of), _ptr(hits),
                                       _ptr(target), _ptr(promote), _ptr(promote_slot), _ptr(demote), _ptr(counts),
                                       _stream(stream)))


def refresh_due(every: int, step: int, prefill_block: bool, offload: bool) -> bool:
    return bool(lib().moe_refresh_due(every, step, int(prefill_block), int(offload)))


def budget_from_memory(free_bytes: int, reserve_bytes: int, expert_bytes: int, layers: int, max_per_layer: int,
                       E: int) -> int:
    return int(lib().moe_budget_from_memory(free_bytes, reserve_bytes, expert_bytes, layers, max_per_layer, E))
