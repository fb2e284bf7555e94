"""Python face of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
and the benchmark's CPU-baseline leg import this module.  It shares no code
with the HIP library in ``expert_ffn_amd`` and never imports it.

The wrappers below only marshal numpy arrays into the C routines; every step of
the method is computed in ``oracle.c``.  Enumerations are this module's own
(same numbering as the library's public header, which is a format both sides
state independently).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

W_BF16, W_INT8_ROW, W_INT4_G64 = 0, 1, 2
ACT_GELU_TANH, ACT_SILU = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=False)
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


def _declare(L):
    P = ctypes.c_void_p
    i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    L.oracle_int4_candidates.argtypes = [P, P, P]
    L.oracle_int4_candidates.restype = None
    L.oracle_set_threads.argtypes = [i32]
    L.oracle_set_threads.restype = ctypes.c_int
    L.oracle_f32_to_bf16.argtypes = [P, P, i64]
    L.oracle_bf16_to_f32.argtypes = [P, P, i64]
    L.oracle_route_topk.argtypes = [P, i32, i32, i32, i32, P, P]
    L.oracle_route_topk.restype = ctypes.c_int
    L.oracle_permute.argtypes = [P, i32, i32, i32, P, P, P, P, P]
    L.oracle_permute.restype = ctypes.c_int
    L.oracle_quantize_int8.argtypes = [P, i32, i32, P, P]
    L.oracle_quantize_int4.argtypes = [P, i32, i32, P, P]
    L.oracle_blob_layout.argtypes = [i32, i32, i32, P]
    L.oracle_blob_layout.restype = ctypes.c_int
    L.oracle_pack_expert.argtypes = [i32, P, P, i32, i32, P]
    L.oracle_pack_expert.restype = ctypes.c_int
    L.oracle_pack_expert_canonical.argtypes = [i32, P, P, i32, i32, P]
    L.oracle_pack_expert_canonical.restype = ctypes.c_int
    L.oracle_fill_slot.argtypes = [i32, P, i32, i32, P]
    L.oracle_fill_slot.restype = ctypes.c_int
    L.oracle_router_logits.argtypes = [P, P, i32, i32, i32, P]
    L.oracle_router_logits.restype = ctypes.c_int
    L.oracle_residency_refresh.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P, P, P, P]
    L.oracle_residency_refresh.restype = ctypes.c_int
    L.oracle_min_weight.argtypes = [P, P, i32, i32, i32, P, ctypes.c_float, P, P, P]
    L.oracle_min_weight.restype = ctypes.c_int
    L.oracle_dequant.argtypes = [P, i32, i32, i32, i32, P]
    L.oracle_dequant.restype = ctypes.c_int
    L.oracle_act.argtypes = [i32, P, P, i64]
    L.oracle_expert_ffn.argtypes = [P, u64, P, i32, i32, i32, i32, i32, P, i32, i32, P, P, i32, P, P]
    L.oracle_expert_ffn.restype = ctypes.c_int
    L.oracle_combine.argtypes = [P, P, P, i32, i32, P, i32, P]
    L.oracle_combine.restype = ctypes.c_int


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {rc})")


# ---------------------------------------------------------------- bf16 ----
def f32_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16(_p(x), _p(out), x.size)
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().oracle_bf16_to_f32(_p(h), _p(out), h.size)
    return out


# ------------------------------------------------------------- routing ----
def route_topk(logits, k: int, renorm: int = 1):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _check(lib().oracle_route_topk(_p(logits), T, E, k, renorm, _p(ids), _p(w)), "route_topk")
    return ids, w


def permute(ids, E: int, slot_of):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    slot_of = np.ascontiguousarray(slot_of, dtype=np.int32)
    assert slot_of.shape == (E,)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_route = np.empty(T * k, dtype=np.int32)
    route_pos = np.empty(T * k, dtype=np.int32)
    nd = np.zeros(1, dtype=np.int32)
    _check(lib().oracle_permute(_p(ids), T, k, E, _p(slot_of), _p(offsets), _p(sorted_route),
                                _p(route_pos), _p(nd)), "permute")
    return offsets, sorted_route, route_pos, int(nd[0])


# -------------------------------------------------------- quantisation ----
def quantize_int8(w_bf16):
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.int8)
    s = np.empty(N, dtype=np.float32)
    lib().oracle_quantize_int8(_p(w), N, K, _p(q), _p(s))
    return q, s


def quantize_int4(w_bf16):
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    N, K = w.shape
    assert K % 64 == 0
    q = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N, K // 64), dtype=np.uint16)
    lib().oracle_quantize_int4(_p(w), N, K, _p(q), _p(s))
    return q, s


def int4_candidates(group_bf16):
    """All ten clip candidates of one 64-element group: (bf16 scale bits [10], squared errors [10])."""
    g = np.ascontiguousarray(group_bf16, dtype=np.uint16).reshape(64)
    sc = np.zeros(10, np.uint16)
    er = np.zeros(10, np.float64)
    lib().oracle_int4_candidates(_p(g), _p(sc), _p(er))
    return sc, er


def blob_layout(fmt: int, H: int, FF: int):
    off = np.zeros(5, dtype=np.uint64)
    _check(lib().oracle_blob_layout(fmt, H, FF, _p(off)), "blob_layout")
    return [int(v) for v in off]


def expert_bytes(fmt: int, H: int, FF: int) -> int:
    return blob_layout(fmt, H, FF)[4]


def pack_expert(fmt: int, w13_bf16, w2_bf16, H: int, FF: int) -> np.ndarray:
    w13 = np.ascontiguousarray(w13_bf16, dtype=np.uint16)
    w2 = np.ascontiguousarray(w2_bf16, dtype=np.uint16)
    assert w13.shape == (2 * FF, H) and w2.shape == (H, FF)
    blob = np.empty(expert_bytes(fmt, H, FF), dtype=np.uint8)
    _check(lib().oracle_pack_expert(fmt, _p(w13), _p(w2), H, FF, _p(blob)), "pack_expert")
    return blob


def pack_expert_canonical(fmt: int, w13_bf16, w2_bf16, H: int, FF: int) -> np.ndarray:
    """The expert's canonical form: the blob layout with int4 codes row-major."""
    w13 = np.ascontiguousarray(w13_bf16, dtype=np.uint16)
    w2 = np.ascontiguousarray(w2_bf16, dtype=np.uint16)
    assert w13.shape == (2 * FF, H) and w2.shape == (H, FF)
    blob = np.empty(expert_bytes(fmt, H, FF), dtype=np.uint8)
    _check(lib().oracle_pack_expert_canonical(fmt, _p(w13), _p(w2), H, FF, _p(blob)), "pack_expert_canonical")
    return blob


def fill_slot(fmt: int, canonical, H: int, FF: int) -> np.ndarray:
    """Canonical form -> the slot form the kernels read."""
    src = np.ascontiguousarray(canonical, dtype=np.uint8)
    assert src.size == expert_bytes(fmt, H, FF)
    slot = np.empty_like(src)
    _check(lib().oracle_fill_slot(fmt, _p(src), H, FF, _p(slot)), "fill_slot")
    return slot


def router_logits(x_f32, w_router) -> np.ndarray:
    """fp64 router logits x [T, H] . Wr [E, H]^T."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    wr = np.ascontiguousarray(w_router, dtype=np.float32)
    T, H = x.shape
    E = wr.shape[0]
    assert wr.shape == (E, H)
    out = np.empty((T, E), dtype=np.float64)
    _check(lib().oracle_router_logits(_p(x), _p(wr), T, H, E, _p(out)), "router_logits")
    return out


def residency_refresh(ids, E: int, budget: int, S: int, slot_of):
    """[rlx_runtime expert_pool.rs] hit counts, target, paired promote/demote
    and the new slot table; returns a dict of numpy arrays."""
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    slot_of = np.ascontiguousarray(slot_of, dtype=np.int32)
    assert slot_of.shape == (E,)
    out = dict(hits=np.empty(E, np.int32), target=np.empty(max(budget, 1), np.int32),
               promote=np.empty(E, np.int32), promote_slot=np.empty(E, np.int32), demote=np.empty(E, np.int32),
               counts=np.empty(3, np.int32), slot_of=np.empty(E, np.int32))
    _check(lib().oracle_residency_refresh(_p(ids), ids.size, E, budget, S, _p(slot_of), _p(out["hits"]),
                                          _p(out["target"]), _p(out["promote"]), _p(out["promote_slot"]),
                                          _p(out["demote"]), _p(out["counts"]), _p(out["slot_of"])),
           "residency_refresh")
    nt, np_, nd = (int(v) for v in out["counts"])
    out["target"] = out["target"][:budget]
    out["promote"], out["promote_slot"] = out["promote"][:np_], out["promote_slot"][:np_]
    out["demote"] = out["demote"][:nd]
    return out


def min_weight(ids, w, E: int, slot_of, share: float):
    """[prain] "Trading quality for speed": (ids_out, w_out, miss_count) for
    routes ids/w [T, k] at min_weight = share (fp32)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    slot_of = np.ascontiguousarray(slot_of, dtype=np.int32)
    T, k = ids.shape
    assert w.shape == (T, k) and slot_of.shape == (E,)
    ids_out = np.empty_like(ids)
    w_out = np.empty_like(w)
    miss = np.empty(E, dtype=np.int32)
    _check(lib().oracle_min_weight(_p(ids), _p(w), T, k, E, _p(slot_of), float(np.float32(share)), _p(ids_out),
                                   _p(w_out), _p(miss)), "min_weight")
    return ids_out, w_out, miss


def dequant(blob, fmt: int, H: int, FF: int, which: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    rows, K = (H, FF) if which else (2 * FF, H)
    out = np.empty((rows, K), dtype=np.float64)
    _check(lib().oracle_dequant(_p(blob), fmt, H, FF, which, _p(out)), "dequant")
    return out


def act(kind: int, g) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    out = np.empty_like(g)
    lib().oracle_act(kind, _p(g), _p(out), g.size)
    return out


# ---------------------------------------------------------- expert FFN ----
def expert_ffn(pool, slot_bytes: int, slot_of, E: int, H: int, FF: int, fmt: int, act_kind: int,
               x_f32, ids, routes):
    """fp64 outputs o[len(routes), H] of the listed routes, and a kept flag per route."""
    pool = np.ascontiguousarray(pool, dtype=np.uint8)
    slot_of = np.ascontiguousarray(slot_of, dtype=np.int32)
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    assert x.shape == (T, H)
    routes = np.ascontiguousarray(routes, dtype=np.int32)
    o = np.empty((routes.size, H), dtype=np.float64)
    ok = np.empty(routes.size, dtype=np.int32)
    _check(lib().oracle_expert_ffn(_p(pool), slot_bytes, _p(slot_of), E, H, FF, fmt, act_kind, _p(x),
                                   T, k, _p(ids), _p(routes), routes.size, _p(o), _p(ok)),
           "expert_ffn")
    return o, ok


def combine(o_rows, route_row, w, tokens):
    """y[len(tokens), H] = sum_j w[t, j] * o_rows[route_row[q, j]] (row -1 = dropped)."""
    o_rows = np.ascontiguousarray(o_rows, dtype=np.float64)
    route_row = np.ascontiguousarray(route_row, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    k = w.shape[1]
    H = o_rows.shape[1]
    assert route_row.shape == (tokens.size, k)
    y = np.empty((tokens.size, H), dtype=np.float64)
    _check(lib().oracle_combine(_p(o_rows), _p(route_row), _p(w), k, H, _p(tokens), tokens.size,
                                _p(y)), "combine")
    return y


def set_threads(n: int) -> int:
    """Threads of the oracle's parallel loops (n <= 0 leaves them); returns the count in use."""
    return int(lib().oracle_set_threads(n))


def moe_layer(logits, x_f32, pool, slot_bytes: int, slot_of, H: int, FF: int, fmt: int,
              act_kind: int, k: int, renorm: int = 1, tokens=None):
    """The whole layer for the listed tokens (all by default): route, permute,
    expert FFN of those tokens' routes, combine.  Returns a dict of every step."""
    T, E = logits.shape
    ids, w = route_topk(logits, k, renorm)
    offsets, sorted_route, route_pos, n_dropped = permute(ids, E, slot_of)
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.asarray(tokens, dtype=np.int32)
    routes = (tokens[:, None] * k + np.arange(k, dtype=np.int32)[None, :]).reshape(-1)
    o, ok = expert_ffn(pool, slot_bytes, slot_of, E, H, FF, fmt, act_kind, x_f32, ids, routes)
    route_row = np.where(ok.reshape(tokens.size, k) > 0,
                         np.arange(routes.size, dtype=np.int32).reshape(tokens.size, k), -1)
    y = combine(o, route_row, w, tokens)
    return dict(ids=ids, w=w, offsets=offsets, sorted_route=sorted_route, route_pos=route_pos,
                n_dropped=n_dropped, routes=routes, o=o, kept=ok, tokens=tokens, y=y)
