"""The C ABI without a GPU: the library loads, exports every function the
public header declares, reports the pack layout, and rejects invalid
arguments on the host before launching anything (these calls never reach the
HIP runtime)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "expert_ffn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import expert_ffn_amd as lib
    if not os.path.exists(lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return lib


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    cdll = L.lib()
    for n in names:
        assert hasattr(cdll, n), f"{n} declared in include/expert_ffn.h but not exported"


def test_layout_matches_oracle(L, ora):
    for fmt in (0, 1, 2):
        for H, FF in ((2816, 704), (64, 64), (128, 64), (192, 128)):
            assert L.blob_layout(fmt, H, FF) == ora.blob_layout(fmt, H, FF)
            assert L.expert_bytes(fmt, H, FF) == ora.expert_bytes(fmt, H, FF)
    assert L.expert_bytes(2, 2816, 700) == 0          # int4 needs FF % 64 == 0


def _call(L, name, *args):
    rc = getattr(L.lib(), name)(*args)
    return rc, L.lib().moe_last_error().decode()


def test_host_validation_errors(L):
    P = ctypes.c_void_p
    fake = P(1 << 20)   # never dereferenced: every call below fails its checks first
    rc, msg = _call(L, "moe_route_topk", None, 4, 8, 2, 1, fake, fake, None)
    assert rc == 1 and msg.startswith("moe_route_topk")
    rc, msg = _call(L, "moe_route_topk", fake, 4, 8, 9, 1, fake, fake, None)
    assert rc == 2 and "k=9" in msg
    rc, msg = _call(L, "moe_route_topk", fake, 4, 600, 8, 1, fake, fake, None)
    assert rc == 2 and "E=600" in msg
    rc, msg = _call(L, "moe_permute", fake, 4, 33, 64, fake, fake, fake, fake, fake, None)
    assert rc == 2 and "k=33" in msg
    ffn = lambda **kw: _call(L, "moe_expert_ffn", *[kw.get(n, d) for n, d in (
        ("pool", P(1 << 20)), ("sb", 3159552), ("slot", fake), ("E", 128), ("H", 2816), ("FF", 704),
        ("fmt", 2), ("act", 0), ("x", fake), ("xdt", 1), ("T", 16), ("k", 8), ("off", fake),
        ("sr", fake), ("out", fake), ("odt", 0), ("ws", P(1 << 20)), ("wsb", 0), ("s", None))])
    rc, msg = ffn(FF=700)
    assert rc == 2 and "FF=700" in msg
    rc, msg = ffn(H=2800)
    assert rc == 2 and "H=2800" in msg
    rc, msg = ffn(sb=3159552 - 256)
    assert rc == 1 and "slot_bytes" in msg
    rc, msg = ffn(fmt=7)
    assert rc == 1
    rc, msg = ffn(act=5)
    assert rc == 1 and "activation" in msg
    rc, msg = ffn(wsb=1024)
    assert rc == 4 and "ws_bytes" in msg
    rc, msg = ffn(pool=None)
    assert rc == 1
    rc, msg = _call(L, "moe_quantize", 0, fake, 4, 64, fake, fake, None)
    assert rc == 1 and "not a quantised format" in msg
    rc, msg = _call(L, "moe_quantize", 2, fake, 4, 96, fake, fake, None)
    assert rc == 2
    rc, msg = _call(L, "moe_combine", fake, 0, fake, fake, 4, 2, 60, fake, 0, None)
    assert rc == 2 and "H=60" in msg
    # no-alloc FFN: a workspace larger than the static scratch array is refused on the host
    rc, msg = _call(L, "moe_expert_ffn_noalloc", fake, ctypes.c_uint64(3159552), fake, 128, 2816, 704, 2, 0, fake, 1,
                    4096, 8, fake, fake, fake, 0, None)
    assert rc == 4 and "scratch" in msg
    rc, msg = _call(L, "moe_expert_ffn_noalloc", fake, ctypes.c_uint64(3159552), fake, 128, 2816, 700, 2, 0, fake, 1,
                    16, 8, fake, fake, fake, 0, None)
    assert rc == 2 and "FF=700" in msg
    rc, msg = _call(L, "moe_fill_slot", 2, fake, 1, 2816, 704, None, fake, None)
    assert rc == 1 and "staging" in msg
    rc, msg = _call(L, "moe_fill_slot", 2, fake, 0, 2816, 704, None, fake, None)
    assert rc == 1 and "overlaps" in msg
    rc, msg = _call(L, "moe_fill_slot", 2, fake, 0, 2816, 700, None, P(1 << 30), None)
    assert rc == 2 and "FF=700" in msg
    rc, msg = _call(L, "moe_fill_slot", 1, P((1 << 20) + 8), 0, 2816, 704, None, P(1 << 30), None)
    assert rc == 1 and "aligned" in msg
    rc, msg = _call(L, "moe_verify_slot", 2, fake, 2816, 704, fake, None, None)
    assert rc == 1
    rc, msg = _call(L, "moe_fill_slots", 2, 65, fake, 2816, 704, fake, fake, None)
    assert rc == 2 and "n=65" in msg
    rc, msg = _call(L, "moe_fill_slots", 2, 0, None, 2816, 704, None, None, None)
    assert rc == 0                                       # nothing to do, nothing enqueued
    rc, msg = _call(L, "moe_fill_slots", 2, 2, None, 2816, 704, fake, fake, None)
    assert rc == 1 and "null" in msg
    rc, msg = _call(L, "moe_min_weight", fake, fake, 4, 8, 128, fake, ctypes.c_float(float("nan")), fake, fake,
                    fake, None)
    assert rc == 1 and "NaN" in msg
    rc, msg = _call(L, "moe_min_weight", fake, fake, 4, 33, 128, fake, ctypes.c_float(0.5), fake, fake, fake, None)
    assert rc == 2 and "k=33" in msg


def test_slot_admit_claims_the_lowest_free_slot(L):
    import torch
    E, S = 6, 3
    slot_of = torch.full((E,), -1, dtype=torch.int32)
    owner = torch.full((S,), -1, dtype=torch.int32)
    assert L.slot_admit(slot_of, owner, 4) == 0
    assert L.slot_admit(slot_of, owner, 1) == 1
    assert L.slot_admit(slot_of, owner, 4) == 0          # already resident
    owner[0] = -1                                        # evict expert 4
    slot_of[4] = -1
    assert L.slot_admit(slot_of, owner, 5) == 0
    assert L.slot_admit(slot_of, owner, 2) == 2
    with pytest.raises(L.MoeError, match="no free slot"):
        L.slot_admit(slot_of, owner, 3)
    assert slot_of.tolist() == [-1, 1, 2, -1, -1, 0] and owner.tolist() == [5, 1, 2]
    with pytest.raises(L.MoeError):
        L.slot_admit(slot_of, owner, 6)


def test_workspace_grows_with_tokens(L):
    a = L.workspace_bytes(16, 8, 128, 2816, 704, 2)
    b = L.workspace_bytes(1024, 8, 128, 2816, 704, 2)
    assert 0 < a < b
    assert b >= 1024 * 8 * 704 * 2 + 1024 * 2816 * 2


def test_refresh_schedule_and_budget_printed_vectors(L):
    from conftest import read_golden
    n = 0
    for row in read_golden("rlx_expert_pool_vectors.txt"):
        if row[0] == "refresh_due":
            step, prefill, want = (int(v) for v in row[1:])
            assert L.refresh_due(3, step, bool(prefill), True) == bool(want)
            n += 1
        elif row[0] == "budget":
            args = [int(v) for v in row[1].split()]
            b = L.budget_from_memory(*args)
            assert b == int(row[2]) and 0 < b <= 128
            n += 1
    assert n == 6
    assert not L.refresh_due(1, 0, True, False)          # no offload: never
    assert L.refresh_due(1, 7, False, True)              # every forward
    assert L.budget_from_memory(0, 0, 0, 20, 64, 32) == 32
