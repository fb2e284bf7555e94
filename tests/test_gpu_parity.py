"""GPU parity of the whole path against the oracle, through the C ABI.

Bit-exact: expert ids, group offsets, sorted routes, route positions, dropped
count and every packed byte of the experts the oracle packs itself.  Within
tolerance: router weights (1e-5 absolute) and the layer output y (max
row-relative error 2e-2 for bf16 weights, 3e-2 for int8/int4, against the
fp64 oracle on the same dequantised weights).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import (FMT, TOL, build_pool, log, oracle_layer, row_rel_err, sample_tokens,
                        to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import expert_ffn_amd as lib
    lib.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


def _x(seed, layer, T, H, kind):
    """Device x and its fp32 values: "f32" (N(0,1) kept fp32), "bf16" (N(0,1)
    rounded), "heavy" (Student-t(2) with 100x outliers, rounded)."""
    import oracle as ora
    if kind == "f32":
        xh = synth.x_f32(seed, layer, T, H)
        return torch.from_numpy(xh).cuda(), xh
    bits = synth.x_heavy_bf16(seed, layer, T, H) if kind == "heavy" else synth.x_bf16(seed, layer, T, H)
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16), ora.bf16_to_f32(bits)


def run_case(L, name, *, E, k, H, FF, fmt, T, act=0, x_kind="bf16", y_dtype=torch.bfloat16,
             zipf=None, slot_of=None, n_sample=None, seed=0, layer=0, out_dtype=torch.float32, gemm=None,
             logits=None):
    from expert_ffn_amd.layer import MoeLayer
    log(f"[case] {name}: E={E} k={k} H={H} FF={FF} fmt={fmt} T={T} act={act} zipf={zipf}")
    f = FMT[fmt]
    if slot_of is None:
        slot_of = np.arange(E, dtype=np.int32)
    slot_of = np.asarray(slot_of, np.int32)
    if logits is None:
        logits = synth.logits(seed, layer, T, E, zipf)
    x_d, x_f32 = _x(seed, layer, T, H, x_kind)
    pool, sb = build_pool(seed, layer, E, H, FF, f, slot_of)
    slot_d = torch.from_numpy(slot_of).cuda()
    ml = MoeLayer(E, k, H, FF, f, max(T, 1), act=act, y_dtype=y_dtype, out_dtype=out_dtype)
    ml.bind(pool, sb, slot_d)
    y = ml.run(torch.from_numpy(logits).cuda(), x_d)
    torch.cuda.synchronize()
    v = ml.views(T)
    tokens = sample_tokens(T, T if n_sample is None else n_sample)
    ref = oracle_layer(seed, layer, E, k, H, FF, f, act, logits, x_f32, slot_of, tokens)
    assert np.array_equal(to_np(v["topk_ids"]), ref["ids"]), "topk ids differ"
    assert np.max(np.abs(to_np(v["topk_w"]) - ref["w"])) <= 1e-5, "router weights differ"
    assert np.array_equal(to_np(v["offsets"]), ref["offsets"]), "expert offsets differ"
    assert np.array_equal(to_np(v["sorted_route"]), ref["sorted_route"]), "sorted routes differ"
    assert np.array_equal(to_np(v["route_pos"]), ref["route_pos"]), "route positions differ"
    assert int(to_np(v["n_dropped"])[0]) == ref["n_dropped"]
    # int4 kernel family per expert group: more than GEMM_GROUP_MIN routes (when
    # T > GEMM_T_MIN) -> grouped GEMM, else streaming; gemm = (some GEMM groups,
    # some streaming groups) the case is meant to cover
    m = np.diff(ref["offsets"])
    n_gemm = int(((m > GEMM_GROUP_MIN) & (T > GEMM_T_MIN)).sum()) if f == 2 else 0
    n_stream = int((m > 0).sum()) - n_gemm
    log(f"    groups: {n_gemm} grouped-GEMM, {n_stream} streaming, largest {int(m.max()) if m.size else 0}")
    if gemm is not None:
        assert (n_gemm > 0, n_stream > 0) == gemm, f"{name}: families used {(n_gemm > 0, n_stream > 0)}"
    for e, blob in ref["blobs"].items():
        got = to_np(pool[slot_of[e] * sb:slot_of[e] * sb + blob.size])
        assert np.array_equal(got, blob), f"packed bytes of expert {e} differ"
    err, med = row_rel_err(to_np(y)[tokens], ref["y"])
    log(f"    y: max row-rel err {err:.3e}, median {med:.3e} over {tokens.size} tokens "
        f"(tolerance {TOL[f]:.0e})")
    assert err <= TOL[f], f"{name}: y error {err} > {TOL[f]}"
    return ml, pool, sb, y


# ------------------------------------------------------------ tiny layer ----
@pytest.mark.parametrize("act", [0, 1])
def test_tiny_bf16(L, act):
    c = synth.CONFIGS["tiny"]
    run_case(L, "tiny", E=c["E"], k=c["k"], H=c["H"], FF=c["FF"], fmt="bf16", T=c["T"], act=act,
             x_kind="f32", y_dtype=torch.float32, slot_of=[2, 0, 3, 1])


def test_tiny_dropped_expert(L):
    c = synth.CONFIGS["tiny"]
    run_case(L, "tiny-dropped", E=c["E"], k=c["k"], H=c["H"], FF=c["FF"], fmt="bf16", T=c["T"],
             x_kind="f32", y_dtype=torch.float32, slot_of=[1, -1, 0, 2])


@pytest.mark.parametrize("fmt", ["int8", "int4"])
@pytest.mark.parametrize("act", [0, 1])
def test_tiny_quantised(L, fmt, act):
    run_case(L, f"tiny-{fmt}", E=4, k=2, H=128, FF=64, fmt=fmt, T=8, act=act, x_kind="f32",
             y_dtype=torch.float32, slot_of=[3, 1, 0, 2])


def test_ragged_shapes(L):
    # E, T not multiples of anything; two experts not resident; several groups of 17+ routes
    slot_of = np.array([4, -1, 0, 6, 2, -1, 1], np.int32)
    for fmt in ("bf16", "int8", "int4"):
        run_case(L, f"ragged-{fmt}", E=7, k=3, H=192, FF=128, fmt=fmt, T=37, slot_of=slot_of,
                 n_sample=37, seed=3)


def test_all_dropped(L):
    ml, _, _, y = run_case(L, "all-dropped", E=4, k=2, H=64, FF=32, fmt="bf16", T=5,
                           slot_of=[-1, -1, -1, -1], x_kind="f32", y_dtype=torch.float32)
    assert int(to_np(ml.n_dropped)[0]) == 10
    assert not to_np(y).any()


# -------------------------------------------------- Gemma-shaped layers ----
G = synth.GEMMA
GEMM_GROUP_MIN, GEMM_T_MIN = 8, 32      # the library's dispatch thresholds (csrc/kernels.h)


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_gemma_bf16_decode(L, T):
    run_case(L, f"gemma-bf16-T{T}", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="bf16", T=T)


def test_gemma_bf16_silu(L):
    run_case(L, "gemma-bf16-silu", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="bf16", T=16, act=1)


def test_gemma_int8_decode_zipf(L):
    run_case(L, "gemma-int8-zipf-T16", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="int8", T=16,
             zipf=1.1)


def test_gemma_int4_decode(L):
    slot_of = synth.slot_table(0, 1, G["E"])[0]
    run_case(L, "gemma-int4-T16", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="int4", T=16,
             slot_of=slot_of)


def _logits_for_group_sizes(T, E, k, sizes, seed):
    """Logits whose top-k gives expert e exactly sizes[e] routes (the rest of
    each token's k picks spread evenly over the remaining experts): expert e goes to
    the sizes[e] tokens with the fewest picks so far, a token's picks get
    distinct logits 10 - 0.01 rank, all other logits are N(0,1) - 5."""
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((T, E)) - 5.0).astype(np.float32)
    picks = [[] for _ in range(T)]
    sizes = list(sizes)
    e = 0
    while sum(len(p) for p in picks) < T * k:
        left = T * k - sum(len(p) for p in picks)
        n = sizes[e] if e < len(sizes) else -(-left // (E - e))
        order = sorted((t for t in range(T) if len(picks[t]) < k), key=lambda t: (len(picks[t]), t))
        for t in order[:n]:
            picks[t].append(e)
        e += 1
    for t in range(T):
        for rank, ex in enumerate(picks[t]):
            lg[t, ex] = 10.0 - 0.01 * rank
    return lg


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
@pytest.mark.parametrize("T,sizes,x_kind", [
    (16, (16, 5, 4, 3, 2, 1, 8, 6), "bf16"),
    (40, (40, 17, 5, 4, 4, 1, 33), "f32"),
])
def test_streaming_tile_sizes(L, fmt, T, sizes, x_kind):
    """The bf16 / int8 streaming kernels at the Gemma shape on groups of chosen
    sizes: 4 routes (the last size whose gate/up tile takes x from LDS), 5
    (the first that reads it per lane from L2), 16 and more (down's full
    16-route tile, and more than one route tile per group)."""
    lg = _logits_for_group_sizes(T, G["E"], G["k"], sizes, seed=7)
    ml, *_ = run_case(L, f"gemma-{fmt}-T{T}-sizes", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt=fmt, T=T,
                      x_kind=x_kind, logits=lg)
    m = np.diff(to_np(ml.views(T)["offsets"]))
    for n in sizes:
        assert n in m, f"no group of {n} routes"


@pytest.mark.parametrize("T,zipf", [(1, None), (5, None), (16, 1.1), (37, None)])
def test_gemma_int4_decode_sizes(L, T, zipf):
    slot_of = synth.slot_table(1, 1, G["E"])[0]
    run_case(L, f"gemma-int4-T{T}-zipf{zipf}", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="int4", T=T,
             zipf=zipf, slot_of=slot_of, seed=2)


def test_gemma_int4_decode_f32_x(L):
    run_case(L, "gemma-int4-T8-f32x", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="int4", T=8,
             x_kind="f32", y_dtype=torch.float32, act=1)


@pytest.mark.parametrize("zipf", [None, 1.1])
def test_gemma_int4_prefill(L, zipf):
    run_case(L, f"gemma-int4-T1024-zipf{zipf}", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="int4",
             T=1024, zipf=zipf)


# The int4 grouped-GEMM path (groups of more than 8 routes) on small shapes:
# partial and multiple 128-route tiles, wide 64-route tiles, odd group counts,
# ragged N tiles, and calls where both kernel families take groups.
GEMM_CASES = [
    dict(name="gemm-E8-H256-FF128-T100", E=8, k=2, H=256, FF=128, T=100),
    dict(name="gemm-E2-H384-FF384-T300-zipf", E=2, k=1, H=384, FF=384, T=300, zipf=1.1),
    dict(name="gemm-E4-H640-FF640-T150-silu-f32x", E=4, k=2, H=640, FF=640, T=150, act=1, x_kind="f32",
         out_dtype=torch.bfloat16),
    dict(name="gemm-E4-H192-FF192-T90", E=4, k=2, H=192, FF=192, T=90),
    dict(name="gemm-E16-H128-FF256-T100-dropped", E=16, k=4, H=128, FF=256, T=100,
         slot_of=np.array([0, -1, 2, 3, -1, 5, 6, 7, 8, 9, -1, 11, 12, 13, 14, 15], np.int32)),
    dict(name="mixed-E32-H256-FF192-T80-zipf", E=32, k=2, H=256, FF=192, T=80, zipf=1.1, gemm=(True, True)),
    dict(name="mixed-E24-H384-FF128-T70-zipf-f32x", E=24, k=3, H=384, FF=128, T=70, zipf=1.1, x_kind="f32",
         gemm=(True, True)),
    # H = 3328 (52 groups), FF = 1152 (18): the item set-up's scale tile takes more than one batch
    # in both halves and the bias more than three 16-group steps; wide tiles of 49-70 routes,
    # then 128-route tiles
    dict(name="gemm-E4-H3328-FF1152-T120", E=4, k=2, H=3328, FF=1152, T=120, out_dtype=torch.bfloat16),
    dict(name="gemm-E2-H3328-FF1152-T250-narrow", E=2, k=1, H=3328, FF=1152, T=250),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c["name"] for c in GEMM_CASES])
def test_int4_gemm_path(L, case):
    c = dict(case)
    c.setdefault("gemm", (True, False) if c["name"].startswith("gemm") else None)
    if c["name"].startswith("gemm-E16"):
        c["gemm"] = None      # a few small groups may remain with the streaming kernels
    run_case(L, c.pop("name"), fmt="int4", seed=3, **c)


def test_gemma_int4_gemm_T256(L):
    run_case(L, "gemma-int4-T256", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt="int4", T=256)


# Mid-sized batches, where one expert's group can be large while the others
# stay small (the kernel family is chosen per expert group): every format at
# T = 128 with Zipf(1.1) routing and T = 256 with uniform routing.
@pytest.mark.parametrize("fmt", ["bf16", "int8", "int4"])
@pytest.mark.parametrize("T,zipf", [(128, 1.1), (256, None)])
def test_gemma_mid_batches(L, fmt, T, zipf):
    run_case(L, f"gemma-{fmt}-T{T}-zipf{zipf}", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt=fmt, T=T,
             zipf=zipf, seed=4)


# Heavy-tailed activations (Student-t(2), 4 elements per row at 100x): the
# int4 kernels remove the code offset through per-group activation sums kept
# as bf16 hi + lo, whose cancellation is worst with such inputs.
@pytest.mark.parametrize("fmt,T,zipf", [("int4", 16, None), ("int4", 256, None), ("int4", 128, 1.1),
                                        ("int8", 16, None), ("bf16", 16, None)])
def test_gemma_heavy_tailed_x(L, fmt, T, zipf):
    run_case(L, f"gemma-{fmt}-T{T}-heavy-zipf{zipf}", E=G["E"], k=G["k"], H=G["H"], FF=G["FF"], fmt=fmt, T=T,
             zipf=zipf, x_kind="heavy", seed=5)


# ------------------------------------------------------------ invariants ----
def test_determinism_and_slot_shuffle(L):
    from expert_ffn_amd.layer import MoeLayer
    E, k, H, FF, T = 16, 4, 256, 128, 64
    log("[case] determinism + slot shuffle int4")
    logits = torch.from_numpy(synth.logits(5, 0, T, E, 1.1)).cuda()
    x_d, _ = _x(5, 0, T, H, "bf16")
    s1 = np.arange(E, dtype=np.int32)
    s2 = np.random.default_rng(1).permutation(E).astype(np.int32) + 3
    outs = []
    for so in (s1, s1, s2):
        pool, sb = build_pool(5, 0, E, H, FF, 2, so)
        ml = MoeLayer(E, k, H, FF, 2, T).bind(pool, sb, torch.from_numpy(so).cuda())
        outs.append(to_np(ml.run(logits, x_d).clone()))
    assert np.array_equal(outs[0], outs[1]), "repeat run differs"
    assert np.array_equal(outs[0], outs[2]), "slot shuffle changes y"


def test_split_halves_equal_whole(L):
    from expert_ffn_amd.layer import MoeLayer
    E, k, H, FF, T = 8, 2, 128, 64, 24
    log("[case] gate_up + down == expert_ffn")
    for f in (0, 1, 2):
        logits = torch.from_numpy(synth.logits(6, 0, T, E)).cuda()
        x_d, _ = _x(6, 0, T, H, "bf16")
        so = np.arange(E, dtype=np.int32)
        pool, sb = build_pool(6, 0, E, H, FF, f, so)
        ml = MoeLayer(E, k, H, FF, f, T).bind(pool, sb, torch.from_numpy(so).cuda())
        whole = to_np(ml.run(logits, x_d).clone())
        ml.out_routes.zero_()
        ml.gate_up(x_d)
        ml.down(T)
        ml.combine(T)
        assert np.array_equal(to_np(ml.y[:T]), whole)


def test_bf16_out_routes_and_renorm0(L):
    import expert_ffn_amd as lib
    import oracle as ora
    run_case(L, "out-bf16", E=8, k=2, H=128, FF=64, fmt="int4", T=20, out_dtype=torch.bfloat16)
    T, E, k = 33, 128, 8
    logits = synth.logits(9, 0, T, E)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lib.route_topk(torch.from_numpy(logits).cuda(), k, ids, w, renorm=0)
    torch.cuda.synchronize()
    rid, rw = ora.route_topk(logits, k, renorm=0)
    assert np.array_equal(to_np(ids), rid)
    assert np.max(np.abs(to_np(w) - rw)) <= 1e-6


def test_route_ties_and_nan(L):
    import expert_ffn_amd as lib
    import oracle as ora
    r = np.random.default_rng(2)
    for E, k in ((4, 2), (100, 7), (300, 32)):
        l = r.integers(-3, 3, size=(50, E)).astype(np.float32)
        l[3, :] = 0.0
        l[4, ::2] = -0.0
        l[5, 1] = np.nan
        l[6, :] = -np.inf
        ids = torch.empty((50, k), dtype=torch.int32, device="cuda")
        w = torch.empty((50, k), dtype=torch.float32, device="cuda")
        lib.route_topk(torch.from_numpy(l).cuda(), k, ids, w)
        torch.cuda.synchronize()
        rid, _ = ora.route_topk(l, k)
        assert np.array_equal(to_np(ids), rid)


def test_permute_large_and_empty(L):
    import expert_ffn_amd as lib
    import oracle as ora
    r = np.random.default_rng(4)
    for T, k, E in ((4096, 8, 128), (1000, 3, 512), (0, 8, 128)):
        ids = r.integers(0, E, size=(T, k)).astype(np.int32)
        so = r.permutation(E).astype(np.int32)
        so[r.choice(E, E // 10, replace=False)] = -1
        d = lambda a: torch.from_numpy(a).cuda()
        off = torch.full((E + 1,), 7, dtype=torch.int32, device="cuda")
        sr = torch.empty(max(T * k, 1), dtype=torch.int32, device="cuda")
        rp = torch.empty(max(T * k, 1), dtype=torch.int32, device="cuda")
        nd = torch.empty(1, dtype=torch.int32, device="cuda")
        lib.permute(d(ids), E, d(so), off, sr[:T * k], rp[:T * k], nd)
        torch.cuda.synchronize()
        ro, rs, rr, rn = ora.permute(ids, E, so)
        assert np.array_equal(to_np(off), ro)
        assert np.array_equal(to_np(sr[:T * k]), rs) and np.array_equal(to_np(rp[:T * k]), rr)
        assert int(to_np(nd)[0]) == rn


@pytest.mark.parametrize("T,E,k,zipf,case", [
    (16, 128, 8, None, "decode"),          # one launch
    (1, 128, 8, None, "one-token"),
    (64, 128, 16, 1.2, "full-block"),     # T k = 1024: still one launch
    (65, 128, 8, None, "fallback"),       # T > 64: two launches
    (200, 512, 8, None, "fallback-large"),
    (37, 7, 3, None, "ragged"),
    (40, 300, 25, None, "ties-nan"),
    (0, 16, 4, None, "empty"),
])
def test_route_permute_fused(L, T, E, k, zipf, case):
    """moe_route_permute against the oracle's route_topk + permute (ids, order,
    offsets bit-exact; weights within 1e-5), with experts not resident."""
    import expert_ffn_amd as lib
    import oracle as ora
    log(f"[case] route_permute {case}: T={T} E={E} k={k} zipf={zipf}")
    r = np.random.default_rng(T * 1000 + E)
    logits = synth.logits(5, 0, T, E, zipf) if T else np.zeros((0, E), np.float32)
    if case == "ties-nan":
        logits = r.integers(-3, 3, size=(T, E)).astype(np.float32)
        logits[3, :] = 0.0
        logits[4, ::2] = -0.0
        logits[5, 1] = np.nan
        logits[6, :] = -np.inf
    so = r.permutation(E).astype(np.int32)
    so[r.choice(E, max(E // 10, 1), replace=False)] = -1
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    R = max(T * k, 1)
    ids = torch.full((max(T, 1), k), -5, dtype=torch.int32, device="cuda")
    w = torch.empty((max(T, 1), k), dtype=torch.float32, device="cuda")
    off = torch.full((E + 1,), 7, dtype=torch.int32, device="cuda")
    sr = torch.empty(R, dtype=torch.int32, device="cuda")
    rp = torch.empty(R, dtype=torch.int32, device="cuda")
    nd = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    lib.route_permute(d(logits).reshape(T, E), k, d(so), ids[:T], w[:T], off, sr[:T * k], rp[:T * k], nd)
    torch.cuda.synchronize()
    rid, rw = ora.route_topk(logits, k)
    ro, rs, rr, rn = ora.permute(rid, E, so)
    assert np.array_equal(to_np(ids[:T]), rid), "topk ids differ"
    if T:
        assert np.nanmax(np.abs(to_np(w[:T]) - rw)) <= 1e-5, "router weights differ"
    assert np.array_equal(to_np(off), ro), "expert offsets differ"
    assert np.array_equal(to_np(sr[:T * k]), rs) and np.array_equal(to_np(rp[:T * k]), rr), "order differs"
    assert int(to_np(nd)[0]) == rn


def test_quantize_bit_exact_specials(L):
    import expert_ffn_amd as lib
    import oracle as ora
    r = np.random.default_rng(8)
    w = (r.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[0] = 0.0                                  # zero row / zero groups
    w[1, :64] = 1e-39                           # subnormal group
    w[2] *= 1e4                                 # large values
    w[3, 5] = 7.0                               # one outlier
    from test_oracle_quant_ffn import CLIP_065_GROUP
    w[4, :64] = ora.bf16_to_f32(CLIP_065_GROUP)   # a group whose best clip is alpha = 0.65
    bits = synth.to_bf16_bits(w)
    wd = torch.from_numpy(bits.view(np.int16)).cuda()
    for fmt in (1, 2):
        N, K = bits.shape
        if fmt == 1:
            q = torch.empty((N, K), dtype=torch.int8, device="cuda")
            s = torch.empty(N, dtype=torch.float32, device="cuda")
            rq, rs = ora.quantize_int8(bits)
        else:
            q = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
            s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
            rq, rs = ora.quantize_int4(bits)
        lib.quantize(fmt, wd, q, s)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(q).view(rq.dtype), rq)
        assert np.array_equal(to_np(s).view(rs.dtype), rs)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("H,FF", [(128, 192), (2816, 704)])
def test_fill_slot_bit_exact(L, fmt, H, FF):
    # canonical blob (the oracle's) -> slot, from pinned host memory through a
    # staging buffer and from device memory: every byte equals the oracle's
    # packed blob; verify_slot counts 0, then 1 after one corrupted byte
    import oracle as ora
    log(f"fill_slot fmt={fmt} H={H} FF={FF}")
    w13, w2 = synth.expert_weights(21, 0, 3, H, FF)
    canon = ora.pack_expert_canonical(fmt, w13, w2, H, FF)
    want = ora.pack_expert(fmt, w13, w2, H, FF)
    sb = L.expert_bytes(fmt, H, FF)
    pool = torch.full((3 * sb,), 0xAB, dtype=torch.uint8, device="cuda")
    src_h = torch.from_numpy(canon).pin_memory()
    staging = torch.empty(sb, dtype=torch.uint8, device="cuda")
    L.fill_slot(fmt, src_h, H, FF, pool[sb:2 * sb], staging=staging)
    src_d = torch.from_numpy(canon).cuda()
    L.fill_slot(fmt, src_d, H, FF, pool[2 * sb:])
    torch.cuda.synchronize()
    got = to_np(pool)
    assert np.array_equal(got[sb:2 * sb], want)
    assert np.array_equal(got[2 * sb:], want)
    assert (got[:sb] == 0xAB).all()                     # nothing written outside the slots
    L.fill_slot(fmt, src_h, H, FF, pool[:sb], direct=True)   # the kernel reads the pinned blob
    torch.cuda.synchronize()
    assert np.array_equal(to_np(pool[:sb]), want)
    with pytest.raises(L.MoeError, match="pinned"):
        L.fill_slot(fmt, torch.from_numpy(canon), H, FF, pool[:sb], direct=True)
    bad = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    L.verify_slot(fmt, src_d, H, FF, pool[sb:2 * sb], bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    off = L.blob_layout(fmt, H, FF)
    pool[sb + off[2] + 5] ^= 1                          # one byte of the w2 block
    L.verify_slot(fmt, src_d, H, FF, pool[sb:2 * sb], bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1


# ------------------------------------------------------------ min_weight ----
@pytest.mark.parametrize("T,E,k,n_res", [(1, 128, 8, 15), (16, 128, 8, 15), (1000, 128, 8, 64), (300, 64, 32, 20),
                                         (0, 128, 8, 15)])
def test_min_weight_bit_exact(L, T, E, k, n_res):
    # routes from the oracle's top-k on seeded logits (plus planted ties and
    # invalid ids); every share: ids, weights (fp32 bits) and miss counts exact
    import oracle as ora
    log(f"min_weight T={T} E={E} k={k} resident={n_res}")
    r = np.random.default_rng(T + E + k)
    ids, w = ora.route_topk(synth.logits(3, 0, T, E, None), k) if T else (np.zeros((0, k), np.int32),
                                                                            np.zeros((0, k), np.float32))
    if T >= 4:
        w[1, :] = np.float32(1.0 / k)                  # all weights tied
        ids[2, 0] = -1                                 # invalid ids
        ids[3, k - 1] = E
    slot_of = np.full(E, -1, np.int32)
    slot_of[r.choice(E, n_res, replace=False)] = np.arange(n_res, dtype=np.int32)
    slot_d = torch.from_numpy(slot_of).cuda()
    for share in (0.0, 0.4, 0.6, 0.95, 1.0):
        ids_d = torch.from_numpy(ids).cuda()
        w_d = torch.from_numpy(w).cuda()
        io = torch.full_like(ids_d, 77)
        wo = torch.full_like(w_d, 77.0)
        miss = torch.full((E,), 55, dtype=torch.int32, device="cuda")
        L.min_weight(ids_d, w_d, E, slot_d, share, io, wo, miss)
        rio, rwo, rmiss = ora.min_weight(ids, w, E, slot_of, share)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(io), rio), share
        assert np.array_equal(to_np(wo).view(np.uint32), rwo.view(np.uint32)), share
        assert np.array_equal(to_np(miss), rmiss), share
        L.min_weight(ids_d, w_d, E, slot_d, share, ids_d, w_d, miss)     # in place
        torch.cuda.synchronize()
        assert np.array_equal(to_np(ids_d), rio) and np.array_equal(to_np(w_d).view(np.uint32), rwo.view(np.uint32))


@pytest.mark.parametrize("share", [0.6, 0.4])
def test_min_weight_miss_step(L, share):
    # the serving step with a small resident set (15 of 128 experts, as with
    # 450 slots over 30 layers): select, copy the missed experts into free
    # slots, then group, FFN and combine; y against the oracle run on the
    # oracle's own selection with the same residency
    from expert_ffn_amd.layer import MoeLayer
    import oracle as ora
    from gpu_common import host_weights
    c = synth.CONFIGS["int4_stack"]
    E, k, H, FF, T, f = c["E"], c["k"], c["H"], c["FF"], 16, L.W_INT4_G64
    log(f"min_weight miss step share={share}")
    slot_of = np.full(E, -1, np.int32)
    slot_of[np.arange(0, E, 9)[:15]] = np.arange(15, dtype=np.int32)
    pool, sb = build_pool(5, 0, E, H, FF, f, slot_of, n_slots=E)
    logits = synth.logits(5, 0, T, E, None)
    x_d, x_f32 = _x(5, 0, T, H, "bf16")
    ml = MoeLayer(E, k, H, FF, f, T, out_dtype=torch.float32)
    slot_d = torch.from_numpy(slot_of).cuda()
    ml.bind(pool, sb, slot_d)
    ml.select(torch.from_numpy(logits).cuda(), share)
    miss = to_np(ml.miss_count)
    W = host_weights(5, 0, E, H, FF)
    filled = slot_of.copy()
    nxt = 15
    for e in np.flatnonzero(miss):
        L.pack_expert(f, torch.from_numpy(W[e][0].view(np.int16)).cuda(),
                      torch.from_numpy(W[e][1].view(np.int16)).cuda(), pool[nxt * sb:(nxt + 1) * sb])
        filled[e] = nxt
        nxt += 1
    slot_d.copy_(torch.from_numpy(filled))
    ml.group(T)
    ml.ffn(x_d)
    ml.combine(T)
    torch.cuda.synchronize()
    ids, w = ora.route_topk(logits, k)
    sid, sw, smiss = ora.min_weight(ids, w, E, slot_of, share)
    assert np.array_equal(to_np(ml.topk_ids[:T]), sid)
    assert np.max(np.abs(to_np(ml.topk_w[:T]) - sw)) <= 2e-5
    assert np.array_equal(miss, smiss)
    full = int((slot_of[ids] < 0).sum())
    log(f"    copies: {int(smiss.sum())} routes to {int((smiss > 0).sum())} experts (full routing: {full} routes)")
    assert smiss.sum() < full
    tokens = np.arange(T, dtype=np.int32)
    ref = oracle_layer(5, 0, E, k, H, FF, f, 0, logits, x_f32, filled, tokens, routes_in=(sid, sw))
    err, med = row_rel_err(to_np(ml.y[:T])[tokens], ref["y"])
    log(f"    y: max row-rel err {err:.3e}, median {med:.3e}")
    assert err <= TOL[f]


# ------------------------------------------------------- router GEMV + top-k ----
@pytest.mark.parametrize("T,E,k,H,xdt", [(1, 128, 8, 2816, "bf16"), (16, 128, 8, 2816, "bf16"),
                                         (1024, 128, 8, 2816, "bf16"), (37, 64, 4, 320, "f32"),
                                         (5, 300, 8, 128, "bf16"), (3, 16, 2, 8192, "f32"), (0, 128, 8, 2816, "bf16"),
                                         (100, 64, 4, 320, "f32"), (130, 300, 8, 192, "bf16")])
def test_router_topk(L, T, E, k, H, xdt):
    # logits against the fp64 product within an fp32 bound per element; ids
    # exact wherever the oracle's logits separate the ranks by more than
    # that bound (else the chosen logit must match the rank's within it);
    # weights within 1e-5; a second call (over the first's workspace) identical
    import oracle as ora
    log(f"router_topk T={T} E={E} k={k} H={H} x={xdt}")
    wr = synth.router_weight(9, 0, E, H)
    if xdt == "bf16":
        bits = synth.x_bf16(9, 0, T, H)
        x_d = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        x_h = ora.bf16_to_f32(bits).reshape(T, H)
    else:
        x_h = synth.x_f32(9, 0, T, H)
        x_d = torch.from_numpy(x_h).cuda()
    wr_d = torch.from_numpy(wr).cuda()
    ws = torch.full((L.router_ws_bytes(T, H, E),), 0x7F, dtype=torch.uint8, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.router_topk(x_d, wr_d, k, logits, ws, ids, w)
    torch.cuda.synchronize()
    got_l, got_i, got_w = to_np(logits), to_np(ids), to_np(w)
    L.router_topk(x_d, wr_d, k, logits, ws, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(logits).view(np.uint32), got_l.view(np.uint32))
    assert np.array_equal(to_np(ids), got_i) and np.array_equal(to_np(w), got_w)
    if T == 0:
        return
    ref = ora.router_logits(x_h, wr)
    bound = 64 * 2.0 ** -24 * (np.abs(x_h).astype(np.float64) @ np.abs(wr).astype(np.float64).T)
    assert np.all(np.abs(got_l - ref) <= bound)
    rid, rw = ora.route_topk(ref.astype(np.float32), k)
    exact = 0
    for t in range(T):
        order = np.lexsort((np.arange(E), -ref[t]))
        if np.array_equal(got_i[t], rid[t]):
            exact += 1
        else:
            assert len(set(got_i[t].tolist())) == k
            for j in range(k):   # a near tie: the chosen logit is the rank's within the bound
                assert abs(ref[t, got_i[t, j]] - ref[t, order[j]]) <= 2 * bound[t].max()
    log(f"    ids identical for {exact} of {T} tokens; max logit err {np.max(np.abs(got_l - ref)):.2e}")
    same = np.all(got_i == rid, axis=1)
    assert np.max(np.abs(got_w[same] - rw[same])) <= 1e-5
    assert exact >= T - max(1, T // 100)


def test_router_topk_softmax_over_all_and_k_equals_E(L):
    # renorm = 0 (softmax over all E) and k = E (every expert, in rank order)
    import oracle as ora
    T, H = 24, 192
    for E, k, renorm in ((16, 16, 1), (40, 5, 0), (3, 3, 0)):
        wr = synth.router_weight(11, 0, E, H)
        x_h = synth.x_f32(11, 0, T, H)
        ws = torch.empty(L.router_ws_bytes(T, H, E), dtype=torch.uint8, device="cuda")
        logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        L.router_topk(torch.from_numpy(x_h).cuda(), torch.from_numpy(wr).cuda(), k, logits, ws, ids, w, renorm=renorm)
        torch.cuda.synchronize()
        ref = ora.router_logits(x_h, wr)
        rid, rw = ora.route_topk(ref.astype(np.float32), k, renorm)
        assert np.array_equal(to_np(ids), rid), (E, k, renorm)
        assert np.max(np.abs(to_np(w) - rw)) <= 1e-5
        if renorm or k == E:
            assert np.allclose(to_np(w).sum(1), 1.0, atol=1e-5)


def test_min_weight_share_zero_without_residents_empties_the_layer(L):
    # share 0 and no resident expert: every route skipped, nothing to copy,
    # and the layer's output is zero
    from expert_ffn_amd.layer import MoeLayer
    E, k, H, FF, T = 8, 2, 64, 64, 5
    slot_of = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    pool = torch.zeros(L.expert_bytes(L.W_BF16, H, FF), dtype=torch.uint8, device="cuda")
    ml = MoeLayer(E, k, H, FF, L.W_BF16, T, out_dtype=torch.float32)
    ml.bind(pool, L.expert_bytes(L.W_BF16, H, FF), slot_of)
    ml.select(torch.from_numpy(synth.logits(2, 0, T, E, None)).cuda(), 0.0)
    ml.group(T)
    x = torch.from_numpy(synth.x_bf16(2, 0, T, H).view(np.int16)).cuda().view(torch.bfloat16)
    ml.ffn(x)
    ml.combine(T)
    torch.cuda.synchronize()
    assert (to_np(ml.topk_ids[:T]) == -1).all() and not to_np(ml.topk_w[:T]).any()
    assert not to_np(ml.miss_count).any()
    assert int(to_np(ml.n_dropped)[0]) == T * k
    assert not to_np(ml.y[:T]).any()


@pytest.mark.parametrize("fmt", [1, 2])
def test_fill_slots_batch_bit_exact(L, fmt):
    # five experts' canonical blobs from pinned host memory in one call, into
    # scattered slots of a pool: each slot equals the oracle's packed blob,
    # the slots in between stay untouched; a slot inside staging is refused
    import oracle as ora
    H, FF = 256, 128
    sb = L.expert_bytes(fmt, H, FF)
    pool = torch.full((12 * sb,), 0x5A, dtype=torch.uint8, device="cuda")
    targets = [7, 1, 10, 4, 2]
    canon, want = [], []
    for e in range(5):
        w13, w2 = synth.expert_weights(41, 0, e, H, FF)
        canon.append(torch.from_numpy(ora.pack_expert_canonical(fmt, w13, w2, H, FF)).pin_memory())
        want.append(ora.pack_expert(fmt, w13, w2, H, FF))
    staging = torch.empty(5 * sb, dtype=torch.uint8, device="cuda")
    L.fill_slots(fmt, canon, H, FF, [pool[t * sb:(t + 1) * sb] for t in targets], staging)
    torch.cuda.synchronize()
    got = to_np(pool).reshape(12, sb)
    for e, t in enumerate(targets):
        assert np.array_equal(got[t], want[e]), (e, t)
    for t in set(range(12)) - set(targets):
        assert (got[t] == 0x5A).all()
    with pytest.raises(L.MoeError, match="overlaps"):
        L.fill_slots(fmt, canon[:2], H, FF, [pool[:sb], staging[sb:2 * sb]], staging)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_fill_slot_smallest_expert_and_errors(L, fmt):
    # H = FF = 64 (one 64-group per row, one 32-row tile per w2 block), then
    # the host-side rejections: staging overlapping the slot, a misaligned slot
    import oracle as ora
    H = FF = 64
    w13, w2 = synth.expert_weights(31, 0, 0, H, FF)
    canon = ora.pack_expert_canonical(fmt, w13, w2, H, FF)
    sb = L.expert_bytes(fmt, H, FF)
    buf = torch.zeros(3 * sb + 256, dtype=torch.uint8, device="cuda")
    src_h = torch.from_numpy(canon).pin_memory()
    L.fill_slot(fmt, src_h, H, FF, buf[:sb], staging=buf[sb:2 * sb])
    torch.cuda.synchronize()
    assert np.array_equal(to_np(buf[:sb]), ora.pack_expert(fmt, w13, w2, H, FF))
    with pytest.raises(L.MoeError, match="overlaps"):
        L.fill_slot(fmt, src_h, H, FF, buf[:sb], staging=buf[sb // 2:sb // 2 + sb])
    with pytest.raises(L.MoeError, match="aligned"):
        L.fill_slot(fmt, src_h, H, FF, buf[8:8 + sb], staging=buf[2 * sb + 256:])


# ------------------------------------------------------ residency refresh ----
def _refresh_gpu(L, ids, E, budget, S, slot_of):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    ids_d, slot_d = d(np.asarray(ids, np.int32).reshape(-1)), d(slot_of)
    outs = {n: torch.full((m,), -9, dtype=torch.int32, device="cuda")
            for n, m in (("hits", E), ("target", max(budget, 1)), ("promote", E), ("promote_slot", E),
                         ("demote", E), ("counts", 3))}
    L.residency_refresh(ids_d, E, budget, S, slot_d, outs["hits"], outs["target"], outs["promote"],
                        outs["promote_slot"], outs["demote"], outs["counts"])
    torch.cuda.synchronize()
    o = {n: to_np(t) for n, t in outs.items()}
    o["slot_of"] = to_np(slot_d)
    return o


@pytest.mark.parametrize("case", range(12))
def test_residency_refresh_bit_exact(L, case):
    # hit counts, target, promotions (with slots), demotions and the new table
    # equal the oracle's; cases include Gemma decode (16 tokens x top-8) and
    # prefill (1024 x 8) routing, empty routing, budget 0 and budget = E
    import oracle as ora
    r = np.random.default_rng(100 + case)
    if case == 0:
        E, budget, S, R = 128, 15, 15, 128
    elif case == 1:
        E, budget, S, R = 128, 15, 20, 8192
    elif case == 2:
        E, budget, S, R = 512, 200, 512, 3000
    elif case == 3:
        E, budget, S, R = 64, 0, 8, 100
    elif case == 4:
        E, budget, S, R = 32, 32, 32, 0
    else:
        E = int(r.integers(2, 513))
        budget = int(r.integers(0, E + 1))
        S = int(r.integers(max(budget, 1), 513))
        R = int(r.integers(0, 5000))
    n_res = int(r.integers(0, min(S, E) + 1))
    slot_of = np.full(E, -1, np.int32)
    slot_of[r.choice(E, n_res, replace=False)] = r.choice(S, n_res, replace=False)
    ids = r.integers(-1, E + 1, R).astype(np.int32)
    log(f"residency refresh case {case}: E={E} budget={budget} slots={S} routes={R} resident={n_res}")
    got = _refresh_gpu(L, ids, E, budget, S, slot_of)
    want = ora.residency_refresh(ids, E, budget, S, slot_of)
    nt, np_, nd = (int(v) for v in want["counts"])
    assert got["counts"].tolist() == [nt, np_, nd]
    assert np.array_equal(got["hits"], want["hits"])
    assert np.array_equal(got["target"][:budget], want["target"])
    assert np.array_equal(got["promote"][:np_], want["promote"])
    assert np.array_equal(got["promote_slot"][:np_], want["promote_slot"])
    assert np.array_equal(got["demote"][:nd], want["demote"])
    assert np.array_equal(got["slot_of"], want["slot_of"])


def test_slot_cache_admit_fill_verify_then_layer(L):
    # the slot-cache sequence (admit on the host, fill from pinned memory,
    # verify) builds a pool for a layer whose table starts empty; the layer
    # then matches the oracle, and a corrupted slot is caught by verify
    from expert_ffn_amd.layer import MoeLayer
    import oracle as ora
    E, k, H, FF, T, S = 8, 2, 128, 64, 12, 5
    f = L.W_INT4_G64
    sb = L.expert_bytes(f, H, FF)
    pool = torch.zeros(S * sb, dtype=torch.uint8, device="cuda")
    slot_of = torch.full((E,), -1, dtype=torch.int32)
    owner = torch.full((S,), -1, dtype=torch.int32)
    staging = torch.empty(sb, dtype=torch.uint8, device="cuda")
    bad = torch.empty(1, dtype=torch.int32, device="cuda")
    W = {}
    for e in (6, 1, 3, 0, 4):                               # admitted in this order: slots 0..4
        j = L.slot_admit(slot_of, owner, e)
        W[e] = synth.expert_weights(51, 0, e, H, FF)
        canon = torch.from_numpy(ora.pack_expert_canonical(f, W[e][0], W[e][1], H, FF)).pin_memory()
        L.fill_slot(f, canon, H, FF, pool[j * sb:(j + 1) * sb], staging=staging)
        L.verify_slot(f, canon.cuda(), H, FF, pool[j * sb:(j + 1) * sb], bad)
        torch.cuda.synchronize()
        assert int(bad.item()) == 0
    assert slot_of.tolist() == [3, 1, -1, 2, 4, -1, 0, -1]
    with pytest.raises(L.MoeError, match="no free slot"):
        L.slot_admit(slot_of, owner, 7)
    logits = synth.logits(51, 0, T, E, None)
    x_d, x_f32 = _x(51, 0, T, H, "bf16")
    ml = MoeLayer(E, k, H, FF, f, T, out_dtype=torch.float32)
    ml.bind(pool, sb, slot_of.cuda())
    y = ml.run(torch.from_numpy(logits).cuda(), x_d)
    torch.cuda.synchronize()
    tokens = np.arange(T, dtype=np.int32)
    ref = oracle_layer(51, 0, E, k, H, FF, f, 0, logits, x_f32, slot_of.numpy(), tokens)
    err, _ = row_rel_err(to_np(y), ref["y"])
    assert err <= TOL[f]
    assert int(to_np(ml.n_dropped)[0]) == ref["n_dropped"] > 0
    pool[2 * sb + 100] ^= 0x10                              # one code byte of expert 3's slot
    canon3 = torch.from_numpy(ora.pack_expert_canonical(f, W[3][0], W[3][1], H, FF)).cuda()
    L.verify_slot(f, canon3, H, FF, pool[2 * sb:3 * sb], bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1
