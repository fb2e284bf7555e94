"""Pins of the oracle's residency refresh (rlx_runtime expert_pool.rs,
TIDE-style placement), CPU only: the values the crate's unit tests print
(tests/golden/rlx_expert_pool_vectors.txt), and, on random cases, the target
against numpy's stable sort and the promote/demote/slot rules checked as set
identities."""
import numpy as np
import pytest

from conftest import read_golden


def _ids_for_counts(counts):
    return np.repeat(np.arange(len(counts), dtype=np.int32), counts)


def _table(E, resident):
    t = np.full(E, -1, np.int32)
    for j, e in enumerate(resident):
        t[e] = j
    return t


def test_printed_vectors(ora):
    rows = read_golden("rlx_expert_pool_vectors.txt")
    seen = set()
    for name, *f in rows:
        if name == "count_hits":
            ids, E, want = f
            r = ora.residency_refresh([int(v) for v in ids.split()], int(E), 0, 0, np.full(int(E), -1, np.int32))
            assert r["hits"].tolist() == [int(v) for v in want.split()]
        elif name == "top_by_count":
            counts, budget, want = f
            c = [int(v) for v in counts.split()]
            r = ora.residency_refresh(_ids_for_counts(c), len(c), int(budget), int(budget),
                                      np.full(len(c), -1, np.int32))
            assert r["target"].tolist() == [int(v) for v in want.split()]
        elif name == "placement":
            before, target, pd, after = ([int(v) for v in x.split()] for x in f)
            E = 8
            # hits that make `target` the top-|target| in that order (equal counts, ascending ids)
            ids = np.array(target, np.int32)
            assert sorted(target) == target
            r = ora.residency_refresh(ids, E, len(target), len(before), _table(E, before))
            assert [int(r["counts"][1]), int(r["counts"][2])] == pd
            assert sorted(np.flatnonzero(r["slot_of"] >= 0).tolist()) == after
        elif name == "refresh_mask":
            ids, mask = ([int(v) for v in x.split()] for x in f)
            r = ora.residency_refresh(ids, 4, 2, 2, _table(4, [0, 1]))   # a new pool: resident 0 .. budget-1
            assert (r["slot_of"] >= 0).astype(int).tolist() == mask
        else:
            continue   # host schedule rows: the library's helpers (test_abi.py)
        seen.add(name)
    assert seen == {"count_hits", "top_by_count", "placement", "refresh_mask"}


@pytest.mark.parametrize("seed", range(40))
def test_rules_on_random_cases(ora, seed):
    r = np.random.default_rng(seed)
    E = int(r.integers(4, 200))
    budget = int(r.integers(0, E + 1))
    S = budget + int(r.integers(0, 8))
    n_res = int(r.integers(0, min(S, E) + 1))
    slot_of = np.full(E, -1, np.int32)
    slot_of[r.choice(E, n_res, replace=False)] = r.choice(S, n_res, replace=False)
    ids = r.integers(-2, E + 2, int(r.integers(0, 400))).astype(np.int32)   # a few invalid ids
    out = ora.residency_refresh(ids, E, budget, S, slot_of)
    valid = ids[(ids >= 0) & (ids < E)]
    hits = np.bincount(valid, minlength=E)
    assert np.array_equal(out["hits"], hits)
    order = [e for e in np.lexsort((np.arange(E), -hits)) if hits[e] > 0][:budget]
    nt = len(order)
    assert out["target"][:nt].tolist() == order and (out["target"][nt:] == -1).all()
    res = slot_of >= 0
    tset = set(order)
    promote = [e for e in order if not res[e]]
    can = [e for e in range(E) if res[e] and e not in tset]
    demote = can[:len(promote)]
    assert out["promote"].tolist() == promote and out["demote"].tolist() == demote
    new = out["slot_of"]
    assert set(np.flatnonzero(new >= 0).tolist()) == tset | set(can[len(promote):])
    held = new[new >= 0]
    assert len(set(held.tolist())) == held.size and (held < S).all()   # distinct slots
    free = [s for s in range(S) if s not in set(slot_of[res].tolist())]
    for j, e in enumerate(promote):
        want = slot_of[demote[j]] if j < len(demote) else free[j - len(demote)]
        assert out["promote_slot"][j] == want and new[e] == want
    for e in range(E):
        if e not in promote and e not in demote:
            assert new[e] == slot_of[e]
