"""Pins of the oracle's min_weight routing (prain README, "Trading quality for
speed"), CPU only: the reductions the page fixes (min_weight 1 is the full
routing; with every expert resident nothing changes), a worked example, and a
brute-force search over every subset of the non-resident routes on tiny
inputs, which must find the same number of copies as the greedy rule."""
import itertools

import numpy as np
import pytest


def _routes(seed, T, k, E):
    r = np.random.default_rng(seed)
    ids = np.stack([r.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    z = r.normal(0, 1.5, (T, k))
    w = np.exp(z) / np.exp(z).sum(1, keepdims=True)
    return ids, w.astype(np.float32)


@pytest.mark.parametrize("share", [1.0, 1.5])
def test_share_one_is_the_full_routing(ora, share):
    E = 16
    ids, w = _routes(1, 50, 4, E)
    slot_of = np.where(np.arange(E) % 3 == 0, -1, np.arange(E)).astype(np.int32)
    io, wo, miss = ora.min_weight(ids, w, E, slot_of, share)
    assert np.array_equal(io, ids) and np.array_equal(wo, w)
    assert np.array_equal(miss, np.bincount(ids[slot_of[ids] < 0], minlength=E))


@pytest.mark.parametrize("share", [0.0, 0.4, 0.6, 0.99])
def test_all_resident_changes_nothing(ora, share):
    E = 12
    ids, w = _routes(2, 40, 3, E)
    io, wo, miss = ora.min_weight(ids, w, E, np.arange(E, dtype=np.int32), share)
    assert np.array_equal(io, ids) and np.array_equal(wo, w) and not miss.any()


def test_worked_example(ora):
    # weights 0.4 / 0.3 / 0.2 / 0.1 on experts 0..3, only expert 1 resident:
    #   share 0.75: 0.3 -> + 0.4 = 0.7 -> + 0.2 = 0.9 >= 0.75, skip 0.1; scale by 1 / 0.9
    #   share 0.6:  0.3 -> + 0.4 = 0.7 >= 0.6, skip 0.2 and 0.1; scale by 1 / 0.7
    #   share 0.25: 0.3 >= 0.25 already: every copy skipped; expert 1 alone, weight 1
    ids = np.array([[0, 1, 2, 3]], np.int32)
    w = np.array([[0.4, 0.3, 0.2, 0.1]], np.float32)
    slot_of = np.array([-1, 0, -1, -1], np.int32)
    for share, kept, miss_want in ((0.75, [1, 1, 1, 0], [1, 0, 1, 0]), (0.6, [1, 1, 0, 0], [1, 0, 0, 0]),
                                   (0.25, [0, 1, 0, 0], [0, 0, 0, 0]), (0.0, [0, 1, 0, 0], [0, 0, 0, 0])):
        io, wo, miss = ora.min_weight(ids, w, 4, slot_of, share)
        kept = np.array(kept, bool)
        assert np.array_equal(io[0], np.where(kept, ids[0], -1))
        want = np.where(kept, w[0].astype(np.float64) / w[0][kept].astype(np.float64).sum(), 0.0)
        assert np.allclose(wo[0], want, rtol=1e-6, atol=0)
        assert miss.tolist() == miss_want


def test_ties_take_the_lower_route_first(ora):
    ids = np.array([[5, 2, 7, 1]], np.int32)
    w = np.array([[0.25, 0.25, 0.25, 0.25]], np.float32)
    slot_of = np.full(8, -1, np.int32)
    io, wo, _ = ora.min_weight(ids, w, 8, slot_of, 0.5)
    assert io[0].tolist() == [5, 2, -1, -1]
    assert wo[0].tolist() == [0.5, 0.5, 0.0, 0.0]


def test_invalid_ids_are_skipped(ora):
    ids = np.array([[0, -1, 3, 9]], np.int32)
    w = np.array([[0.5, 0.2, 0.2, 0.1]], np.float32)
    slot_of = np.array([0, 1, 2, -1], np.int32)
    io, wo, miss = ora.min_weight(ids, w, 4, slot_of, 1.0)
    assert io[0].tolist() == [0, -1, 3, -1]
    assert np.array_equal(wo[0], np.float32([0.5, 0.0, 0.2, 0.0]))   # min_weight 1: no rescaling
    assert miss.tolist() == [0, 0, 0, 1]
    io, wo, miss = ora.min_weight(ids, w, 4, slot_of, 0.5)   # W = 0.7, resident 0.5 >= 0.35
    assert io[0].tolist() == [0, -1, -1, -1]
    assert abs(wo[0, 0] - 0.7) < 1e-6 and not miss.any()


def test_brute_force_fewest_copies(ora):
    # the greedy rule keeps the fewest non-resident routes that reach the
    # share: an enumeration of every subset finds the same count, the kept
    # ones are the heaviest, and the kept weights sum to the token's weight
    r = np.random.default_rng(7)
    E, checked = 10, 0
    for trial in range(400):
        k = int(r.integers(2, 7))
        ids, w = _routes(100 + trial, 1, k, E)
        slot_of = np.where(r.random(E) < 0.35, np.arange(E), -1).astype(np.int32)
        share = float(np.float32(r.choice([0.0, 0.2, 0.4, 0.6, 0.8, 0.95])))
        wd = w[0].astype(np.float64)
        res = slot_of[ids[0]] >= 0
        nr = np.flatnonzero(~res)
        W, cR = wd.sum(), wd[res].sum()
        sums = [cR + wd[list(S)].sum() for m in range(len(nr) + 1) for S in itertools.combinations(nr, m)]
        if min(abs(x - share * W) for x in sums) < 1e-5:
            continue            # too close to the threshold for rounding not to decide
        need = min(m for m in range(len(nr) + 1)
                   if any(cR + wd[list(S)].sum() >= share * W for S in itertools.combinations(nr, m)))
        io, wo, miss = ora.min_weight(ids, w, E, slot_of, share)
        kept = io[0] >= 0
        assert kept[res].all()
        assert int(kept[nr].sum()) == need
        if need and need < len(nr):
            assert wd[nr][kept[nr]].min() >= wd[nr][~kept[nr]].max()
        if not kept.all():
            assert abs(wo[0][kept].astype(np.float64).sum() - W) < 1e-5
            assert wd[kept].sum() >= share * W
        assert np.array_equal(miss, np.bincount(ids[0][kept & ~res], minlength=E))
        checked += 1
    assert checked > 300
