"""Pins of the oracle's pack formats, quantisers, expert FFN and combine (CPU).

The pins: the byte counts printed by prain/README.md ("Expert formats" and
"Trading quality for speed"), hand-worked quantisation examples, error bounds
that follow from the format definitions, the dense gated MLP written with
torch's matmuls and activations in fp64, and invariances of the layer.
"""
import numpy as np
import pytest
import torch

import synth
from conftest import read_golden

FMT = {"bf16": 0, "int8": 1, "int4": 2}
MiB, GiB = float(1 << 20), float(1 << 30)


# ---------------------------------------------------------- byte counts ----
def test_pack_sizes_match_printed_table(ora):
    H, FF = synth.GEMMA["H"], synth.GEMMA["FF"]
    rows = read_golden("prain_expert_formats.txt")
    sizes = {}
    for r in rows:
        if r[0] in FMT:
            b = ora.expert_bytes(FMT[r[0]], H, FF)
            sizes[r[0]] = b
            assert round(b / MiB, 2) == float(r[1]), (r, b / MiB)
            assert round(30 * 128 * b / GiB, 1) == float(r[2]), (r, 30 * 128 * b / GiB)
    for r in rows:
        if r[0] == "slots":
            assert round(int(r[1]) * sizes[r[2]] / GiB, 2) == float(r[3])
        if r[0] == "resident":
            assert int(r[2]) * sizes[r[1]] <= float(r[3]) * GiB
    # the exact sub-block offsets of the int8 and int4 blobs (all 256-aligned)
    assert ora.blob_layout(1, H, FF) == [0, 3964928, 3970560, 5953024, 5964288]
    assert ora.blob_layout(2, H, FF) == [0, 1982464, 2106368, 3097600, 3159552]
    assert ora.blob_layout(0, H, FF) == [0, 7929856, 7929856, 11894784, 11894784]


# ------------------------------------------------------------------ int8 ----
def test_int8_hand_example(ora):
    g = {r[0]: r[1] for r in read_golden("quant_hand_examples.txt")}
    w = np.array([float(v) / 128 for v in g["int8_w_times128"].split()], dtype=np.float32)
    q, s = ora.quantize_int8(synth.to_bf16_bits(w)[None, :])
    assert q[0].tolist() == [int(v) for v in g["int8_q"].split()]
    assert s[0] == np.float32(float(g["int8_s_times128"]) / 128)


def test_int8_bounds_and_roundtrip(ora):
    _, w2 = synth.expert_weights(0, 0, 0, 256, 128)
    wf = ora.bf16_to_f32(w2).astype(np.float64)
    q, s = ora.quantize_int8(w2)
    # absmax scale: nothing is clipped, every element within half a step
    assert np.all(np.abs(wf - s[:, None].astype(np.float64) * q) <= s[:, None] / 2 * (1 + 1e-4))  # fp32 quotient rounding
    assert np.all(np.abs(q) <= 127) and np.all(np.abs(q).max(1) == 127)
    # rows that are exactly s*q with a power-of-two s come back exactly
    r = np.random.default_rng(0)
    qq = r.integers(-127, 128, size=(16, 64)).astype(np.float32)
    qq[:, 5] = 127
    ss = np.float32(2.0) ** r.integers(-12, -3, size=16).astype(np.float32)
    q2, s2 = ora.quantize_int8(synth.to_bf16_bits(qq * ss[:, None]))
    assert np.array_equal(q2, qq.astype(np.int8)) and np.array_equal(s2, ss)
    # an all-zero row has scale 0 and codes 0
    q3, s3 = ora.quantize_int8(np.zeros((1, 64), np.uint16))
    assert s3[0] == 0 and not q3.any()


# ------------------------------------------------------------------ int4 ----
def test_int4_hand_example(ora):
    g = {r[0]: r[1] for r in read_golden("quant_hand_examples.txt")}
    qv = np.array([int(v) for v in g["int4_q"].split()], dtype=np.float32)
    q, s = ora.quantize_int4(synth.to_bf16_bits(qv / 64)[None, :])
    assert s[0, 0] == int(g["int4_s_bits"], 16)
    assert q[0].tolist() == [int(v, 16) for v in g["int4_bytes"].split()]
    # an all-zero group: scale 0, every code 0 (stored nibble 8)
    qz, sz = ora.quantize_int4(np.zeros((1, 64), np.uint16))
    assert sz[0, 0] == 0 and np.all(qz == 0x88)


def _unpack_nibbles(q):
    lo = (q & 0xF).astype(np.int32) - 8
    hi = (q >> 4).astype(np.int32) - 8
    out = np.empty((q.shape[0], q.shape[1] * 2), np.int32)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


def test_int4_mse_clip_invariants(ora):
    w13, _ = synth.expert_weights(0, 0, 3, 512, 64)
    wf = ora.bf16_to_f32(w13).astype(np.float64)
    q, s = ora.quantize_int4(w13)
    codes = _unpack_nibbles(q)
    sf = ora.bf16_to_f32(s).astype(np.float64)
    N, K = wf.shape
    G = K // 64
    wg = wf.reshape(N, G, 64)
    cg = codes.reshape(N, G, 64)
    err = ((wg - sf[:, :, None] * cg) ** 2).sum(-1)
    # the error of the alpha = 1 candidate (s = bf16(absmax / 7), no clipping)
    a = np.abs(wg).max(-1)
    s1 = ora.bf16_to_f32(ora.f32_to_bf16((a / 7).astype(np.float32))).astype(np.float64)
    c1 = np.clip(np.rint(wg / s1[:, :, None]), -8, 7)
    err1 = ((wg - s1[:, :, None] * c1) ** 2).sum(-1)
    assert np.all(err <= err1 * (1 + 1e-12))
    # each kept scale is one of the ten candidates alpha*absmax/7, alpha >= 0.55
    ratio = sf * 7 / a
    assert np.all((ratio > 0.55 - 0.01) & (ratio < 1.0 + 0.01))
    # unclipped elements reconstruct within half a step
    inside = (wg / sf[:, :, None] <= 7.5) & (wg / sf[:, :, None] >= -8.5)
    assert np.all(np.abs(wg - sf[:, :, None] * cg)[inside] <= (sf[:, :, None] / 2 * (1 + 1e-5)).repeat(64, -1)[inside])


def _exact(r, fmt, rows, K):
    """Weights the format represents exactly: s * q with a power-of-two s and
    the largest code present in every row (int8) or every group of 64 (int4)."""
    top = 127 if fmt == 1 else 7
    qv = r.integers(-top, top + 1, size=(rows, K)).astype(np.float32)
    qv[:, ::64] = top
    sc = np.float32(2.0) ** -r.integers(6, 9, size=(rows, 1)).astype(np.float32)
    return synth.to_bf16_bits(qv * sc)


def test_dequant_reads_the_format(ora):
    # weights that are exactly representable come back exactly from every format
    H, FF = 128, 64
    r = np.random.default_rng(5)
    for fmt in (0, 1, 2):
        w13, w2 = _exact(r, fmt, 2 * FF, H), _exact(r, fmt, H, FF)
        blob = ora.pack_expert(fmt, w13, w2, H, FF)
        assert np.array_equal(ora.dequant(blob, fmt, H, FF, 0), ora.bf16_to_f32(w13))
        assert np.array_equal(ora.dequant(blob, fmt, H, FF, 1), ora.bf16_to_f32(w2))


def test_int4_blob_tiles_the_row_major_codes(ora):
    # the blob's int4 code blocks are the quantiser's row-major codes in tiles
    # of 32 rows: [N/32][K/64][32 rows][32 bytes]; the scales stay row-major
    H, FF = 192, 128
    r = np.random.default_rng(11)
    w13 = synth.to_bf16_bits(r.normal(0, 0.02, (2 * FF, H)).astype(np.float32))
    w2 = synth.to_bf16_bits(r.normal(0, 0.02, (H, FF)).astype(np.float32))
    blob = ora.pack_expert(2, w13, w2, H, FF)
    off = ora.blob_layout(2, H, FF)
    for w, o_codes, o_scales in ((w13, off[0], off[1]), (w2, off[2], off[3])):
        N, K = w.shape
        q, sc = ora.quantize_int4(w)
        tiles = blob[o_codes:o_codes + N * K // 2].reshape(N // 32, K // 64, 32, 32)
        assert np.array_equal(tiles.transpose(0, 2, 1, 3).reshape(N, K // 2), q)
        assert np.array_equal(blob[o_scales:o_scales + N * K // 32].view(np.uint16).reshape(N, K // 64), sc)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_slot_fill_of_the_canonical_form_is_the_packed_blob(ora, fmt):
    # canonical form: the blob layout with the int4 codes as the quantiser
    # writes them (row-major); filling a slot from it gives the packed blob
    H, FF = 128, 192
    r = np.random.default_rng(12 + fmt)
    w13 = synth.to_bf16_bits(r.normal(0, 0.02, (2 * FF, H)).astype(np.float32))
    w2 = synth.to_bf16_bits(r.normal(0, 0.02, (H, FF)).astype(np.float32))
    canon = ora.pack_expert_canonical(fmt, w13, w2, H, FF)
    off = ora.blob_layout(fmt, H, FF)
    assert canon.size == off[4] == ora.expert_bytes(fmt, H, FF)
    if fmt == 2:
        for w, o_codes, o_scales in ((w13, off[0], off[1]), (w2, off[2], off[3])):
            N, K = w.shape
            q, sc = ora.quantize_int4(w)
            assert np.array_equal(canon[o_codes:o_codes + N * K // 2].reshape(N, K // 2), q)
            assert np.array_equal(canon[o_scales:o_scales + N * K // 32].view(np.uint16).reshape(N, K // 64), sc)
        # padding between the blocks is zero
        used = np.zeros(off[4], bool)
        for o, n in ((off[0], 2 * FF * H // 2), (off[1], 2 * FF * H // 32), (off[2], H * FF // 2), (off[3], H * FF // 32)):
            used[o:o + n] = True
        assert not canon[~used].any()
    else:
        assert np.array_equal(canon, ora.pack_expert(fmt, w13, w2, H, FF))
    assert np.array_equal(ora.fill_slot(fmt, canon, H, FF), ora.pack_expert(fmt, w13, w2, H, FF))


def test_slot_fill_moves_each_int4_code_byte_once(ora):
    # a position-dependent byte pattern: each code byte lands where the tile
    # formula says; scales and padding are copied as they are
    H, FF = 128, 64
    off = ora.blob_layout(2, H, FF)
    canon = (np.arange(off[4], dtype=np.int64) * 7 % 251).astype(np.uint8)
    slot = ora.fill_slot(2, canon, H, FF)
    for o, N, K in ((off[0], 2 * FF, H), (off[2], H, FF)):
        rm = canon[o:o + N * K // 2].reshape(N, K // 2)
        t = slot[o:o + N * K // 2].reshape(N // 32, K // 64, 32, 32).transpose(0, 2, 1, 3).reshape(N, K // 2)
        assert np.array_equal(t, rm)
    assert np.array_equal(slot[off[1]:off[2]], canon[off[1]:off[2]])
    assert np.array_equal(slot[off[3]:], canon[off[3]:])


# ----------------------------------------------------------- activation ----
def test_activations_match_torch(ora):
    g = np.linspace(-12, 12, 4001)
    gt = torch.from_numpy(g)
    assert np.max(np.abs(ora.act(0, g) - torch.nn.functional.gelu(gt, approximate="tanh").numpy())) < 1e-14
    assert np.max(np.abs(ora.act(1, g) - torch.nn.functional.silu(gt).numpy())) < 1e-14


# ------------------------------------------------------------- the layer ----
def _pool(ora, fmt, seed, E, H, FF, slot_of, layer=0):
    sb = ora.expert_bytes(fmt, H, FF)
    pool = np.zeros((int(slot_of.max()) + 1) * sb, np.uint8)
    W = {}
    for e in range(E):
        w13, w2 = synth.expert_weights(seed, layer, e, H, FF)
        W[e] = (w13, w2)
        if slot_of[e] >= 0:
            pool[slot_of[e] * sb:(slot_of[e] + 1) * sb] = ora.pack_expert(fmt, w13, w2, H, FF)
    return pool, sb, W


def _dense_mlp_torch(w13, w2, x, FF, act):
    W13 = torch.from_numpy(w13.view(np.int16)).view(torch.bfloat16).double()
    W2 = torch.from_numpy(w2.view(np.int16)).view(torch.bfloat16).double()
    X = torch.from_numpy(x.astype(np.float64))
    g, u = X @ W13[:FF].T, X @ W13[FF:].T
    a = torch.nn.functional.gelu(g, approximate="tanh") if act == 0 else torch.nn.functional.silu(g)
    return ((a * u) @ W2.T).numpy()


@pytest.mark.parametrize("act", [0, 1])
def test_single_expert_is_dense_gated_mlp(ora, act):
    H, FF, T = 64, 32, 8
    slot_of = np.array([0], np.int32)
    pool, sb, W = _pool(ora, 0, 0, 1, H, FF, slot_of)
    x = synth.x_f32(0, 0, T, H)
    out = ora.moe_layer(np.zeros((T, 1), np.float32), x, pool, sb, slot_of, H, FF, 0, act, k=1)
    ref = _dense_mlp_torch(*W[0], x, FF, act)
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())
    assert np.all(out["w"] == 1.0)


@pytest.mark.parametrize("act", [0, 1])
def test_tiny_layer_end_to_end_brute_force(ora, act):
    c = synth.CONFIGS["tiny"]
    E, k, H, FF, T = c["E"], c["k"], c["H"], c["FF"], c["T"]
    slot_of = np.array([2, 0, 3, 1], np.int32)
    pool, sb, W = _pool(ora, 0, 0, E, H, FF, slot_of)
    l = synth.logits(0, 0, T, E)
    x = synth.x_f32(0, 0, T, H)
    out = ora.moe_layer(l, x, pool, sb, slot_of, H, FF, 0, act, k=k)
    ids = np.argsort(-l, axis=1, kind="stable")[:, :k]
    w = torch.softmax(torch.from_numpy(np.take_along_axis(l, ids, 1).astype(np.float64)), 1).numpy()
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            ref[t] += w[t, j] * _dense_mlp_torch(*W[ids[t, j]], x[t:t + 1], FF, act)[0]
    assert np.max(np.abs(out["y"] - ref)) <= 1e-6 * np.abs(ref).max()


@pytest.mark.parametrize("fmt", [1, 2])
def test_quantised_ffn_equals_bf16_on_exact_weights(ora, fmt):
    # weights representable in the format: the quantised layer is the bf16 layer
    E, k, H, FF, T = 4, 2, 128, 64, 6
    slot_of = np.arange(E, dtype=np.int32)
    pools = {}
    for f in (0, fmt):
        sb = ora.expert_bytes(f, H, FF)
        pool = np.zeros(E * sb, np.uint8)
        r = np.random.default_rng(99)          # the same weights for both formats
        for e in range(E):
            pool[e * sb:(e + 1) * sb] = ora.pack_expert(f, _exact(r, fmt, 2 * FF, H),
                                                        _exact(r, fmt, H, FF), H, FF)
        pools[f] = (pool, sb)
    l = synth.logits(1, 0, T, E)
    x = synth.x_f32(1, 0, T, H)
    y0 = ora.moe_layer(l, x, *pools[0], slot_of, H, FF, 0, 0, k=k)["y"]
    y1 = ora.moe_layer(l, x, *pools[fmt], slot_of, H, FF, fmt, 0, k=k)["y"]
    assert np.array_equal(y0, y1)


def test_layer_invariances(ora):
    E, k, H, FF, T = 6, 2, 64, 32, 10
    slot_of = np.arange(E, dtype=np.int32)
    pool, sb, W = _pool(ora, 0, 4, E, H, FF, slot_of)
    l = synth.logits(4, 0, T, E)
    x = synth.x_f32(4, 0, T, H)
    y = ora.moe_layer(l, x, pool, sb, slot_of, H, FF, 0, 0, k=k)["y"]
    # token order: permuting tokens permutes the output rows
    p = np.random.default_rng(1).permutation(T)
    yp = ora.moe_layer(l[p], x[p], pool, sb, slot_of, H, FF, 0, 0, k=k)["y"]
    assert np.array_equal(yp, y[p])
    # slot table: moving experts to other slots changes nothing
    perm = np.random.default_rng(2).permutation(E).astype(np.int32)
    pool2 = np.zeros_like(pool)
    for e in range(E):
        pool2[perm[e] * sb:(perm[e] + 1) * sb] = pool[e * sb:(e + 1) * sb]
    assert np.array_equal(ora.moe_layer(l, x, pool2, sb, perm, H, FF, 0, 0, k=k)["y"], y)
    # expert labels: relabelling logit columns and slots together changes nothing
    lab = np.random.default_rng(3).permutation(E)
    l2 = np.empty_like(l)
    l2[:, lab] = l
    slot2 = np.empty(E, np.int32)
    slot2[lab] = slot_of
    assert np.array_equal(ora.moe_layer(l2, x, pool, sb, slot2, H, FF, 0, 0, k=k)["y"], y)


def test_combine_drops_and_one_hot(ora):
    E, k, H, FF, T = 4, 2, 64, 32, 8
    slot_of = np.array([0, -1, 1, 2], np.int32)      # expert 1 not resident
    pool, sb, W = _pool(ora, 0, 5, E, H, FF, slot_of)
    l = synth.logits(5, 0, T, E)
    x = synth.x_f32(5, 0, T, H)
    out = ora.moe_layer(l, x, pool, sb, slot_of, H, FF, 0, 0, k=k)
    ids, w = out["ids"], out["w"]
    assert out["n_dropped"] == int((ids == 1).sum())
    for t in range(T):
        ref = np.zeros(H)
        for j in range(k):
            if ids[t, j] != 1:
                ref += w[t, j] * _dense_mlp_torch(*W[ids[t, j]], x[t:t + 1], FF, 0)[0]
        assert np.max(np.abs(out["y"][t] - ref)) <= 1e-9 * max(1e-30, np.abs(ref).max()) + 1e-300
    # one-hot weights pick one route's output exactly
    o = np.random.default_rng(0).standard_normal((4, H))
    y = ora.combine(o, np.array([[2, 0]], np.int32), np.array([[1.0, 0.0]], np.float32),
                    np.array([0], np.int32))
    assert np.array_equal(y[0], o[2])


def test_int4_clip_choice_brute_force(ora):
    """Brute force over the ten clip candidates, evaluated independently in
    numpy (IEEE fp32 division, half-even rounding, sequential fp64 sum), on
    groups from light- and heavy-tailed distributions.  Candidates with alpha
    <= 0.65 are never the best for these (or any searched) groups; every other
    candidate is selected here and must match."""
    r = np.random.default_rng(11)
    groups = np.concatenate([r.standard_normal((6000, 64)), r.laplace(size=(6000, 64)),
                             r.standard_t(2, size=(6000, 64))]).astype(np.float32) * np.float32(0.02)
    wb = synth.to_bf16_bits(groups)
    w = ora.bf16_to_f32(wb)
    q, s = ora.quantize_int4(wb)
    a = np.abs(w).max(1)
    errs, scales = [], []
    for i in range(10):
        si = (a * np.float32(20 - i) / np.float32(140)).astype(np.float32)
        si = ora.bf16_to_f32(synth.to_bf16_bits(si))
        qi = np.clip(np.rint(w / si[:, None]), -8, 7)
        d = w.astype(np.float64) - si[:, None].astype(np.float64) * qi
        e = np.zeros(w.shape[0])
        for c in range(64):
            e = e + d[:, c] * d[:, c]
        errs.append(e)
        scales.append(si)
    best = np.argmin(np.array(errs), 0)           # first minimum = the larger alpha
    assert set(range(7)) <= set(best.tolist())
    chosen = np.array(scales)[best, np.arange(w.shape[0])]
    assert np.array_equal(ora.bf16_to_f32(s[:, 0]), chosen)
    qb = np.clip(np.rint(w / chosen[:, None]), -8, 7).astype(np.int32)
    assert np.array_equal(_unpack_nibbles(q), qb)


# A 64-element group where the clip candidate alpha = 0.65 (i = 7) has the
# smallest squared error: one element at +1.0 (the absmax) and 63 elements at
# integer multiples of that candidate's scale, chosen by a search over such
# groups.  (No group of this kind was found where alpha = 0.60 or 0.55 wins:
# clipping the absmax element costs more than the rounding errors they save.)
CLIP_065_GROUP = np.array([16256, 15934, 48958, 16014, 48934, 16166, 48702, 48702, 48830, 48878, 48574, 16014, 48830, 48702, 16142, 48702, 48782, 16110, 15934, 48574, 16166, 48702, 15934, 15934, 48702, 48831, 16062, 48878, 48878, 15806, 48934, 15934, 48958, 48702, 15934, 15934, 15934, 48958, 15934, 16062, 15934, 48782, 15934, 16110, 16166, 48574, 48574, 15806, 48934, 48878, 48878, 48782, 48702, 15724, 15806, 48574, 48782, 48702, 48702, 16110, 48830, 15934, 48702, 15806], dtype=np.uint16)


def _numpy_candidates(wb):
    """All ten clip candidates of 64-element groups (rows of bf16 bits), in
    numpy: scales bf16(fp32(a * (20 - i)) / 140) (IEEE fp32 ops, RNE), codes
    clamp(rint(w / s), -8, 7) (0 when s = 0), error summed in fp64 in order."""
    import oracle as ora_m
    w = ora_m.bf16_to_f32(wb)
    a = np.abs(w).max(1)
    scales, errs = [], []
    for i in range(10):
        si_bits = synth.to_bf16_bits((a * np.float32(20 - i) / np.float32(140)).astype(np.float32))
        si = ora_m.bf16_to_f32(si_bits)
        with np.errstate(divide="ignore", invalid="ignore"):
            qi = np.where(si[:, None] == 0, 0.0, np.clip(np.rint(w / si[:, None]), -8, 7))
        d = w.astype(np.float64) - si[:, None].astype(np.float64) * qi
        e = np.zeros(w.shape[0])
        for c in range(64):
            e = e + d[:, c] * d[:, c]
        scales.append(si_bits)
        errs.append(e)
    return np.array(scales).T, np.array(errs).T


def test_int4_every_clip_candidate(ora):
    """Scale and error of all ten candidates (alpha = 1.00 ... 0.55), including
    those that never win, against the numpy enumeration, on normal, heavy-tailed,
    zero and constructed groups; and the constructed group where alpha = 0.65 wins
    is quantised with that candidate's scale."""
    r = np.random.default_rng(12)
    groups = np.concatenate([r.standard_normal((40, 64)), r.standard_t(2, size=(40, 64)),
                             np.zeros((1, 64))]).astype(np.float32) * np.float32(0.02)
    wb = np.concatenate([synth.to_bf16_bits(groups), CLIP_065_GROUP[None, :]])
    ns, ne = _numpy_candidates(wb)
    for j in range(wb.shape[0]):
        sc, er = ora.int4_candidates(wb[j])
        assert np.array_equal(sc, ns[j]), j
        assert np.array_equal(er, ne[j]), j
    assert int(np.argmin(ne[-1])) == 7
    q, s = ora.quantize_int4(CLIP_065_GROUP[None, :])
    assert int(s[0, 0]) == int(ns[-1, 7])
