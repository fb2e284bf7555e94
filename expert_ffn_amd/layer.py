"""One MoE layer's routed expert FFN on the device: route -> permute -> expert
FFN -> combine, through the C ABI, over buffers torch allocates once.

Buffers are sized for up to T_max tokens; run() works on the first T rows.
"""
from __future__ import annotations

import torch

from . import (ACT_GELU_TANH, F32, combine, expert_ffn, ffn_down, ffn_gate_up, min_weight, permute,
               route_topk, workspace_bytes)


class MoeLayer:
    def __init__(self, E, k, H, FF, fmt, T_max, device="cuda", act=ACT_GELU_TANH, renorm=1,
                 out_dtype=torch.float32, y_dtype=torch.bfloat16):
        self.E, self.k, self.H, self.FF, self.fmt, self.T_max = E, k, H, FF, fmt, T_max
        self.act, self.renorm = act, renorm
        d = torch.device(device)
        i32 = torch.int32
        self.topk_ids = torch.empty((T_max, k), dtype=i32, device=d)
        self.topk_w = torch.empty((T_max, k), dtype=torch.float32, device=d)
        self.offsets = torch.empty(E + 1, dtype=i32, device=d)
        self.sorted_route = torch.empty(T_max * k, dtype=i32, device=d)
        self.route_pos = torch.empty(T_max * k, dtype=i32, device=d)
        self.n_dropped = torch.empty(1, dtype=i32, device=d)
        self.miss_count = torch.zeros(E, dtype=i32, device=d)
        self.out_routes = torch.empty((T_max * k, H), dtype=out_dtype, device=d)
        nbytes = workspace_bytes(T_max, k, E, H, FF, fmt)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=d)
        self.y = torch.empty((T_max, H), dtype=y_dtype, device=d)

    def views(self, T):
        k = self.k
        return dict(topk_ids=self.topk_ids[:T], topk_w=self.topk_w[:T], offsets=self.offsets,
                    sorted_route=self.sorted_route[:T * k], route_pos=self.route_pos[:T * k],
                    n_dropped=self.n_dropped, out_routes=self.out_routes[:T * k], y=self.y[:T])

    def route(self, logits, stream=None):
        T = logits.shape[0]
        route_topk(logits, self.k, self.topk_ids[:T], self.topk_w[:T], self.renorm, stream)
        self.group(T, stream)

    def select(self, logits, share, stream=None):
        """Top-k, then min_weight partial routing at `share` in place; leaves
        in miss_count the kept routes per non-resident expert (the experts to
        fill before group())."""
        T = logits.shape[0]
        route_topk(logits, self.k, self.topk_ids[:T], self.topk_w[:T], self.renorm, stream)
        min_weight(self.topk_ids[:T], self.topk_w[:T], self.E, self._slot_of, share, self.topk_ids[:T],
                   self.topk_w[:T], self.miss_count, stream)

    def group(self, T, stream=None):
        """Permute the current top-k routes against the bound slot table."""
        permute(self.topk_ids[:T], self.E, self._slot_of, self.offsets, self.sorted_route[:T * self.k],
                self.route_pos[:T * self.k], self.n_dropped, stream)

    def ffn(self, x, stream=None):
        T = x.shape[0]
        expert_ffn(self._pool, self._slot_bytes, self._slot_of, self.E, self.H, self.FF, self.fmt,
                   self.act, x, self.k, self.offsets, self.sorted_route[:T * self.k],
                   self.out_routes[:T * self.k], self.ws, stream)

    def gate_up(self, x, stream=None):
        ffn_gate_up(self._pool, self._slot_bytes, self._slot_of, self.E, self.H, self.FF, self.fmt,
                    self.act, x, self.k, self.offsets, self.sorted_route[:x.shape[0] * self.k], self.ws,
                    stream)

    def down(self, T, stream=None):
        ffn_down(self._pool, self._slot_bytes, self._slot_of, self.E, self.H, self.FF, self.fmt, T,
                 self.k, self.offsets, self.sorted_route[:T * self.k], self.out_routes[:T * self.k],
                 self.ws, stream)

    def combine(self, T, stream=None):
        combine(self.out_routes[:T * self.k], self.topk_w[:T], self.route_pos[:T * self.k],
                self.y[:T], stream)

    def bind(self, pool, slot_bytes, slot_of):
        """Select the layer's experts: a slot pool, its slot size and expert -> slot table."""
        self._pool, self._slot_bytes, self._slot_of = pool, int(slot_bytes), slot_of
        return self

    def run(self, logits, x, stream=None):
        """The whole layer for T = logits.shape[0] tokens; returns the y view."""
        T = logits.shape[0]
        self.route(logits, stream)
        self.ffn(x, stream)
        self.combine(T, stream)
        return self.y[:T]


__all__ = ["MoeLayer", "F32"]
