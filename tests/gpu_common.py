"""Helpers of the GPU parity tests: build a layer's slot pool on the device with
the library's packer, evaluate the same layer with the oracle on sampled
tokens, and compare.  The oracle packs its own blobs from the same bf16
weights; nothing it computes comes from the device."""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle as ora
import synth

FMT = {"bf16": 0, "int8": 1, "int4": 2}
TOL = {0: 2e-2, 1: 3e-2, 2: 3e-2}      # max row-relative error (bf16 / quantised weights)


def log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=4)
def host_weights(seed, layer, E, H, FF):
    """bf16 bit patterns of every expert of a layer (numpy)."""
    return [synth.expert_weights(seed, layer, e, H, FF) for e in range(E)]


def build_pool(seed, layer, E, H, FF, fmt, slot_of, n_slots=None, device="cuda"):
    """Device pool with expert e packed (by the library) at slot slot_of[e]."""
    import expert_ffn_amd as lib
    sb = lib.expert_bytes(fmt, H, FF)
    n_slots = int(slot_of.max()) + 1 if n_slots is None else n_slots
    pool = torch.zeros(max(n_slots, 1) * sb, dtype=torch.uint8, device=device)
    W = host_weights(seed, layer, E, H, FF)
    for e in range(E):
        if slot_of[e] < 0:
            continue
        w13 = torch.from_numpy(W[e][0].view(np.int16)).to(device)
        w2 = torch.from_numpy(W[e][1].view(np.int16)).to(device)
        lib.pack_expert(fmt, w13, w2, pool[slot_of[e] * sb:(slot_of[e] + 1) * sb])
    return pool, sb


def oracle_layer(seed, layer, E, k, H, FF, fmt, act, logits, x_f32, slot_of, tokens, routes_in=None,
                 weights=None):
    """Oracle route + permute for all tokens, FFN and combine for the sampled
    tokens, with blobs the oracle packs itself (only the experts those tokens
    need).  routes_in = (ids, w) replaces the oracle's own top-k; weights (a
    function e -> (w13, w2) bf16 bit patterns) replaces the host generator."""
    T = logits.shape[0]
    ids, w = ora.route_topk(logits, k) if routes_in is None else routes_in
    offsets, sorted_route, route_pos, nd = ora.permute(ids, E, slot_of)
    tokens = np.asarray(tokens, dtype=np.int32)
    need = sorted({int(e) for e in ids[tokens].reshape(-1) if slot_of[e] >= 0})
    sb = ora.expert_bytes(fmt, H, FF)
    if weights is None:
        W = host_weights(seed, layer, E, H, FF)
        weights = lambda e: W[e]
    cpool = np.zeros(max(len(need), 1) * sb, np.uint8)
    cslot = np.full(E, -1, np.int32)
    blobs = {}
    for j, e in enumerate(need):
        w13, w2 = weights(e)
        blobs[e] = ora.pack_expert(fmt, w13, w2, H, FF)
        cpool[j * sb:(j + 1) * sb] = blobs[e]
        cslot[e] = j
    routes = (tokens[:, None] * k + np.arange(k, dtype=np.int32)[None, :]).reshape(-1)
    o, ok = ora.expert_ffn(cpool, sb, cslot, E, H, FF, fmt, act, x_f32, ids, routes)
    route_row = np.where(ok.reshape(tokens.size, k) > 0,
                         np.arange(routes.size, dtype=np.int32).reshape(tokens.size, k), -1)
    y = ora.combine(o, route_row, w, tokens)
    return dict(ids=ids, w=w, offsets=offsets, sorted_route=sorted_route, route_pos=route_pos,
                n_dropped=nd, y=y, o=o, routes=routes, kept=ok, blobs=blobs, tokens=tokens)


def row_rel_err(y, ref):
    """Per token row: max |y - ref| / max |ref|; returns (max, median)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    err = np.abs(y - ref).max(axis=1) / den
    return float(err.max()), float(np.median(err))


def to_np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T, dtype=np.int32)
    r = np.random.default_rng(seed)
    s = np.sort(r.choice(T, n, replace=False)).astype(np.int32)
    s[0], s[-1] = 0, T - 1
    return np.unique(s)
