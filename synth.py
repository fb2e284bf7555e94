"""Seeded synthetic inputs for the routed expert FFN, shared by the oracle's
tests, the GPU parity tests, the smoke check and the benchmark.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no routing, no quantisation, no matmul).  bf16 inputs are
produced by torch's own fp32 -> bf16 conversion.

Recipe (one numpy PCG64 stream per tensor, keyed by SeedSequence([seed,
tensor id, layer, expert])):
  router logits   fp32 N(0, 1), optionally plus ln p_e for a Zipf(s) expert
                  popularity p_e = rank_e^-s / sum, ranks a seeded permutation
                  of 1..E
  activations x   fp32 N(0, 1); bf16 by rounding.  A heavy-tailed variant
                  for edge cases: Student-t with 2 degrees of freedom, and in
                  each row 4 elements at random positions multiplied by 100
  expert weights  fp32 N(0, 0.02) -> bf16, w13 [2FF, H] and w2 [H, FF]
  slot table      a seeded permutation of the L*E slots of a pool, [L, E]
  router weight   fp32 N(0, 1/H) [E, H], so that x . Wr has unit spread like
                  the synthetic logits
The shapes are those of a Gemma-4-26B-A4B MoE layer (E = 128, top-8, H = 2816,
FF = 704) and of a tiny layer (E = 4, top-2, H = 64, FF = 32).  The GPU stack
generator draws the same distributions with torch's device generator, for
stacks too large to draw on the host.
"""
from __future__ import annotations

import numpy as np

T_LOGITS, T_X, T_W13, T_W2, T_SLOTS, T_ZIPF, T_ROUTER, T_XHEAVY = 1, 2, 3, 4, 5, 6, 7, 8
WEIGHT_STD = 0.02

GEMMA = dict(E=128, k=8, H=2816, FF=704)
TINY = dict(E=4, k=2, H=64, FF=32)


def rng(seed: int, tensor: int, layer: int = 0, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, layer, expert])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns (torch's round-to-nearest-even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def zipf_bias(seed: int, layer: int, E: int, s: float) -> np.ndarray:
    ranks = rng(seed, T_ZIPF, layer).permutation(E).astype(np.float64) + 1.0
    p = ranks ** (-s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def logits(seed: int, layer: int, T: int, E: int, zipf_s: float | None = None) -> np.ndarray:
    l = rng(seed, T_LOGITS, layer).standard_normal((T, E), dtype=np.float32)
    if zipf_s is not None:
        l = (l + zipf_bias(seed, layer, E, zipf_s)[None, :]).astype(np.float32)
    return l


def x_f32(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    return rng(seed, T_X, layer).standard_normal((T, H), dtype=np.float32)


def x_bf16(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    return to_bf16_bits(x_f32(seed, layer, T, H))


def x_heavy_f32(seed: int, layer: int, T: int, H: int, outliers: int = 4, gain: float = 100.0) -> np.ndarray:
    """Heavy-tailed activations: Student-t(2) draws, with `outliers` elements
    per row (at seeded positions) multiplied by `gain`."""
    r = rng(seed, T_XHEAVY, layer)
    x = r.standard_t(2.0, size=(T, H)).astype(np.float32)
    for t in range(T):
        pos = r.choice(H, size=min(outliers, H), replace=False)
        x[t, pos] *= np.float32(gain)
    return x


def x_heavy_bf16(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    return to_bf16_bits(x_heavy_f32(seed, layer, T, H))


def router_weight(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    """fp32 [E, H] router weight."""
    return (rng(seed, T_ROUTER, layer).standard_normal((E, H), dtype=np.float32)
            * np.float32(1.0 / np.sqrt(H))).astype(np.float32)


def expert_weights(seed: int, layer: int, e: int, H: int, FF: int, std: float = WEIGHT_STD):
    """(w13 [2FF, H], w2 [H, FF]) as bf16 bit patterns."""
    w13 = rng(seed, T_W13, layer, e).standard_normal((2 * FF, H), dtype=np.float32) * np.float32(std)
    w2 = rng(seed, T_W2, layer, e).standard_normal((H, FF), dtype=np.float32) * np.float32(std)
    return to_bf16_bits(w13), to_bf16_bits(w2)


def slot_table(seed: int, L: int, E: int, shuffled: bool = True) -> np.ndarray:
    if not shuffled:
        return np.arange(L * E, dtype=np.int32).reshape(L, E)
    return rng(seed, T_SLOTS).permutation(L * E).astype(np.int32).reshape(L, E)


def layer_weights_cuda(seed: int, layer: int, E: int, H: int, FF: int, device,
                       std: float = WEIGHT_STD):
    """All E experts of one layer drawn on the device: bf16 tensors
    w13 [E, 2FF, H] and w2 [E, H, FF] (torch's Philox generator, seeded per
    layer)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(layer) * 7919 + 17)
    w13 = (torch.randn((E, 2 * FF, H), generator=g, device=device, dtype=torch.float32) * std
           ).to(torch.bfloat16)
    w2 = (torch.randn((E, H, FF), generator=g, device=device, dtype=torch.float32) * std
          ).to(torch.bfloat16)
    return w13, w2


# The five workloads (sizes and distributions of the pages' Gemma 4 26B-A4B
# serving setup; the tiny one is for parity at a size the oracle finishes at
# once).
CONFIGS = {
    "tiny": dict(TINY, T=8, fmt="bf16", x="f32", y="f32", zipf=None),
    "bf16_decode": dict(GEMMA, Ts=(1, 4, 16, 64), fmt="bf16", x="bf16", y="bf16", zipf=None),
    "int8_decode_zipf": dict(GEMMA, T=16, fmt="int8", x="bf16", y="bf16", zipf=1.1),
    "int4_prefill": dict(GEMMA, T=1024, fmt="int4", x="bf16", y="bf16", zipf=(None, 1.1)),
    "int4_stack": dict(GEMMA, L=30, Ts=(16, 1024), fmt="int4", x="bf16", y="bf16", zipf=None),
}
