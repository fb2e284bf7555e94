"""Parity of the 30-layer int4 stack against the oracle, run exactly as the
benchmark runs it.

The stack is the Gemma-4-26B-A4B shape (30 layers x 128 experts, H = 2816,
FF = 704, top-8) with int4 experts (prain README, "Expert formats": 3.01 MiB
per expert, 11.3 GiB for all of them) packed into one pool of 3,840 slots, each
layer's experts found through its own shuffled expert -> slot table, so that
most experts sit more than 4 GiB into the pool.  The benchmark's step is
captured in one HIP graph -- per layer moe_route_permute, moe_ffn_gate_up,
moe_ffn_down (bf16 per-route outputs) and moe_combine (bf16 y) -- and
replayed; the test checks the replayed results:

  - ids, expert offsets, sorted routes, route positions and dropped counts
    bit-exact, router weights within 1e-5, for the layers checked;
  - every slot the checked routes read holds, byte for byte, the blob the
    oracle packs from the same bf16 weights (the slot table's addressing);
  - y on every token within 3e-2 (max row-relative error) of the fp64 oracle.

The layers' weights are drawn on the device by torch's generator (the input
recipe of the stack); the oracle packs its own blobs from a host copy of them.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import TOL, log, oracle_layer, row_rel_err, to_np

pytestmark = pytest.mark.gpu

G = synth.GEMMA
E, K, H, FF = G["E"], G["k"], G["H"], G["FF"]
L_STACK = 30
INT4 = 2
SEED = 0


@pytest.fixture(scope="module")
def lib():
    import expert_ffn_amd as lib
    lib.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return lib


@pytest.fixture(scope="module")
def stack(lib):
    import bench
    log("[stack] building the 30-layer int4 stack (11.3 GiB)")
    pool, sb, slots = bench.build_stack(lib, SEED, L_STACK, E, H, FF, INT4, torch.device("cuda"))
    assert pool.numel() == L_STACK * E * sb
    yield pool, sb, slots
    del pool
    torch.cuda.empty_cache()


def layer_weights_host(layer):
    """Host copy of a stack layer's bf16 weights (bit patterns) as e -> (w13, w2)."""
    w13, w2 = synth.layer_weights_cuda(SEED, layer, E, H, FF, "cuda")
    a = w13.view(torch.int16).cpu().numpy().view(np.uint16)
    b = w2.view(torch.int16).cpu().numpy().view(np.uint16)
    del w13, w2
    return lambda e: (a[e], b[e])


def check_layer(name, run, l, slot_of, logits_h, x_f32, pool, sb):
    T = logits_h.shape[0]
    ref = oracle_layer(SEED, l, E, K, H, FF, INT4, 0, logits_h, x_f32, slot_of, np.arange(T),
                       weights=layer_weights_host(l))
    r = run.rt[l]
    assert np.array_equal(to_np(r["ids"]), ref["ids"]), f"{name}: topk ids differ"
    assert np.max(np.abs(to_np(r["w"]) - ref["w"])) <= 1e-5, f"{name}: router weights differ"
    assert np.array_equal(to_np(r["offsets"]), ref["offsets"]), f"{name}: expert offsets differ"
    assert np.array_equal(to_np(r["sorted_route"]), ref["sorted_route"]), f"{name}: sorted routes differ"
    assert np.array_equal(to_np(r["route_pos"]), ref["route_pos"]), f"{name}: route positions differ"
    assert int(to_np(r["n_dropped"])[0]) == ref["n_dropped"] == 0
    far = 0
    for e, blob in ref["blobs"].items():
        off = int(slot_of[e]) * sb
        far += off >= (1 << 32)
        got = to_np(pool[off:off + blob.size])
        assert np.array_equal(got, blob), f"{name}: slot {slot_of[e]} (expert {e}) differs from the oracle's blob"
    err, med = row_rel_err(to_np(r["y"]), ref["y"])
    log(f"    {name}: {len(ref['blobs'])} experts ({far} beyond 4 GiB), y max row-rel err {err:.3e}, "
        f"median {med:.3e} over {T} tokens")
    assert far > 0, "no checked expert sits beyond 4 GiB: the shuffled table should put most there"
    assert err <= TOL[INT4], f"{name}: y error {err} > {TOL[INT4]}"


def run_stack(lib, pool, sb, slots, T, seed, zipf=None, layers=None):
    """The benchmark's runner over the given layers (all by default): one
    eager step, then a captured graph replayed 3 times; returns the runner
    after checking that the replays reproduce the eager y bit for bit."""
    import bench
    layers = list(range(L_STACK)) if layers is None else layers
    dev = torch.device("cuda")
    logits = [torch.from_numpy(synth.logits(seed, l, T, E, zipf)).to(dev) for l in layers]
    xs = [torch.from_numpy(synth.x_bf16(seed, l, T, H).view(np.int16)).to(dev).view(torch.bfloat16)
          for l in layers]
    # the runner's layer index i is stack layer layers[i]; give it those layers' tables
    sl = np.stack([slots[l] for l in layers])
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run = bench.StackRunner(lib, pool, sb, sl, T, E, K, H, FF, INT4, logits, xs, stream)
        run.step()
        torch.cuda.synchronize()
        eager = [r["y"].clone() for r in run.rt]
        graph = run.capture(stream)
        for r in run.rt:
            r["y"].fill_(0)
        torch.cuda.synchronize()
        for rep in range(3):
            graph.replay()
            torch.cuda.synchronize()
            for i, r in enumerate(run.rt):
                assert torch.equal(r["y"], eager[i]), f"replay {rep}: layer {layers[i]} y differs from eager"
    return run


def test_stack_decode_T16_graph(lib, stack):
    pool, sb, slots = stack
    T = 16
    log("[case] stack decode T=16: graph of 30 layers, layers 0, 14, 29 against the oracle")
    run = run_stack(lib, pool, sb, slots, T, SEED)
    import oracle as ora
    for l in (0, 14, 29):
        check_layer(f"decode layer {l}", run, l, slots[l], synth.logits(SEED, l, T, E),
                    ora.bf16_to_f32(synth.x_bf16(SEED, l, T, H)), pool, sb)


@pytest.mark.parametrize("zipf", [None, 1.1])
def test_stack_prefill_T1024(lib, stack, zipf):
    """One 1024-token chunk (the grouped-GEMM regime) through a stack layer,
    every token compared."""
    import oracle as ora
    pool, sb, slots = stack
    T, seed = 1024, SEED + 1
    l = 7 if zipf is None else 22
    log(f"[case] stack prefill T=1024 zipf={zipf}: layer {l}, all tokens")
    run = run_stack(lib, pool, sb, slots, T, seed, zipf=zipf, layers=[l])

    class One:   # the runner's index 0 is stack layer l
        rt = {l: run.rt[0]}
    check_layer(f"prefill layer {l} zipf={zipf}", One, l, slots[l], synth.logits(seed, l, T, E, zipf),
                ora.bf16_to_f32(synth.x_bf16(seed, l, T, H)), pool, sb)
