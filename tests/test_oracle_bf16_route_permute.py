"""Pins of the oracle's bf16 rounding, router top-k and permutation (CPU only).

Each check compares the oracle with something other than itself: torch's
conversion routine, numpy's stable sort, the values printed in the unit tests
of rlx_runtime/expert_pool.rs, or identities that any correct result obeys.
"""
import numpy as np
import pytest
import torch

import synth
from conftest import read_golden


# ------------------------------------------------------------------ bf16 ----
def test_bf16_exhaustive_roundtrip(ora):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = ora.bf16_to_f32(bits)
    # widening is placement of the bits in the upper half
    assert np.array_equal(f.view(np.uint32), bits.astype(np.uint32) << 16)
    back = ora.f32_to_bf16(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(back[nan] == 0x7FC0)


def test_bf16_rounding_matches_torch(ora):
    r = np.random.default_rng(1)
    # random bit patterns cover every exponent, subnormals included
    x = r.integers(0, 1 << 32, 400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    # exact ties (lower half 0x8000) with odd and even upper halves
    ties = (r.integers(0, 1 << 15, 20_000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    special = np.array([np.inf, -np.inf, 0.0, -0.0, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45],
                       dtype=np.float32)
    x = np.concatenate([x, ties, special])
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ora.f32_to_bf16(x), ref)
    # NaN (torch's scalar and vector paths disagree on the payload): quiet NaN 0x7FC0
    nans = np.array([np.nan, -np.nan], np.float32)
    assert np.all(ora.f32_to_bf16(nans) == 0x7FC0)


# ------------------------------------------------------------- routing ----
def test_route_topk_rlx_printed_vector(ora):
    for row in read_golden("rlx_expert_pool_vectors.txt"):
        if row[0] != "top_by_count":
            continue
        _, inp, par, exp = row
        counts = np.array([[float(v) for v in inp.split()]], dtype=np.float32)
        ids, _ = ora.route_topk(counts, int(par))
        assert ids[0].tolist() == [int(v) for v in exp.split()]


def _stable_topk(l, k):
    # numpy's stable sort of the negated logits: larger first, equal -> lower id first
    return np.argsort(-l, axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(8, 4, 2), (16, 128, 8), (64, 128, 8), (5, 7, 7), (3, 300, 32)])
def test_route_topk_ids_brute_force(ora, T, E, k):
    l = synth.logits(0, 0, T, E)
    ids, _ = ora.route_topk(l, k)
    assert np.array_equal(ids, _stable_topk(l, k))


def test_route_topk_ties_and_specials(ora):
    r = np.random.default_rng(7)
    l = r.integers(-3, 3, size=(200, 16)).astype(np.float32)   # many equal logits
    ids, _ = ora.route_topk(l, 5)
    assert np.array_equal(ids, _stable_topk(l, 5))
    # -0 equals +0, NaN ranks below -inf
    l = np.array([[0.0, -0.0, np.nan, -np.inf, 1.0, np.nan]], dtype=np.float32)
    ids, _ = ora.route_topk(l, 6)
    assert ids[0].tolist() == [4, 0, 1, 3, 2, 5]


@pytest.mark.parametrize("zipf", [None, 1.1])
def test_route_topk_weights(ora, zipf):
    l = synth.logits(3, 1, 64, 128, zipf)
    ids, w = ora.route_topk(l, 8, renorm=1)
    sel = torch.from_numpy(np.take_along_axis(l, ids, 1).astype(np.float64))
    ref = torch.softmax(sel, dim=1).numpy()
    assert np.max(np.abs(w - ref)) < 1e-7
    assert np.max(np.abs(w.astype(np.float64).sum(1) - 1.0)) < 1e-6
    assert np.all(np.diff(w, axis=1) <= 0)
    _, w0 = ora.route_topk(l, 8, renorm=0)
    full = torch.softmax(torch.from_numpy(l.astype(np.float64)), dim=1).numpy()
    assert np.max(np.abs(w0 - np.take_along_axis(full, ids, 1))) < 1e-7
    # k = E with renormalisation is the plain softmax in rank order
    ids_all, w_all = ora.route_topk(l[:, :16], 16, renorm=1)
    full16 = torch.softmax(torch.from_numpy(l[:, :16].astype(np.float64)), 1).numpy()
    assert np.max(np.abs(w_all - np.take_along_axis(full16, ids_all, 1))) < 1e-7


# ----------------------------------------------------------- permutation --
def test_permute_rlx_count_hits(ora):
    for row in read_golden("rlx_expert_pool_vectors.txt"):
        if row[0] != "count_hits":
            continue
        _, inp, par, exp = row
        ids = np.array([[int(v)] for v in inp.split()], dtype=np.int32)
        E = int(par)
        offsets, _, _, nd = ora.permute(ids, E, np.zeros(E, dtype=np.int32))
        assert np.diff(offsets).tolist() == [int(v) for v in exp.split()]
        assert nd == 0


def _brute_permute(ids, E, slot_of):
    flat = ids.reshape(-1)
    kept = [(0 <= e < E) and slot_of[e] >= 0 for e in flat]
    order = sorted((i for i in range(flat.size) if kept[i]), key=lambda i: (flat[i], i))
    counts = np.zeros(E, dtype=np.int64)
    for i in order:
        counts[flat[i]] += 1
    return order, counts, flat.size - len(order)


@pytest.mark.parametrize("T,k,E,drop", [(8, 2, 4, 0), (16, 8, 128, 0), (64, 8, 128, 17),
                                        (1024, 8, 128, 40), (3, 3, 3, 1)])
def test_permute_brute_force(ora, T, k, E, drop):
    r = np.random.default_rng(T + E)
    ids = r.integers(0, E, size=(T, k)).astype(np.int32)
    slot_of = r.permutation(E).astype(np.int32)
    slot_of[r.choice(E, drop, replace=False)] = -1
    offsets, sorted_route, route_pos, nd = ora.permute(ids, E, slot_of)
    order, counts, ndrop = _brute_permute(ids, E, slot_of)
    n = len(order)
    assert nd == ndrop
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert offsets[E] == T * k - nd
    assert sorted_route[:n].tolist() == order
    assert np.all(sorted_route[n:] == -1)
    # route_pos inverts sorted_route; dropped routes have -1
    assert np.array_equal(route_pos[sorted_route[:n]], np.arange(n))
    flat = ids.reshape(-1)
    dropped = slot_of[flat] < 0
    assert np.all(route_pos[dropped] == -1) and np.all(route_pos[~dropped] >= 0)
    # numpy's stable argsort gives the same order
    key = np.where(dropped, E, flat)
    assert np.array_equal(np.argsort(key, kind="stable")[:n], sorted_route[:n])


# ---------------------------------------------------------- router GEMV ----
def test_router_logits_is_the_matrix_product(ora):
    # the fp64 sum equals numpy's fp64 product (another implementation of the
    # same definition) to rounding; one-hot hidden states pick router columns
    x = synth.x_f32(4, 0, 9, 320)
    wr = synth.router_weight(4, 0, 12, 320)
    got = ora.router_logits(x, wr)
    want = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    eye = np.eye(320, dtype=np.float32)[[0, 7, 319]]
    assert np.array_equal(ora.router_logits(eye, wr), wr[:, [0, 7, 319]].T.astype(np.float64))
    assert ora.router_logits(np.zeros((2, 320), np.float32), wr).max() == 0.0
