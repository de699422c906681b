"""A stack of MoE layers whose experts live in pinned host memory and are
brought to the GPU through the LRU slot cache (ft_slot_cache_*).

Host control flow only: every computation runs in libftmoe's kernels and every
copy through the library's copy engine.  The host reads each layer's expert
histogram back (the one device->host step the slot cache needs) and turns it
into the list of experts to map or prefetch.

Per layer l the order is: route + align layer l+1 (its inputs do not depend
on layer l in this synthetic stack), FFN + combine of layer l, release of
layer l, then -- once layer l+1's histogram is on the host -- prefetch of
layer l+1's missing experts on the copy stream while layer l computes, and
the map of layer l+1.  For prefill every expert of the next layer is
prefetched: a prefill batch routes to nearly all experts, so the whole next
layer streams in while the current one computes (FreeToken hub article,
paragraph on prefill overlap).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

from . import ftmoe as ft
from . import synth


@dataclasses.dataclass
class StackStats:
    steps: int = 0
    demand: int = 0
    hits: int = 0
    prefetch_hits: int = 0
    misses: int = 0
    bytes_h2d: int = 0
    prefetch_warnings: int = 0

    @property
    def hit_rate(self) -> float:
        return self.hits / self.demand if self.demand else 0.0

    @property
    def hit_rate_incl_prefetch(self) -> float:
        return (self.hits + self.prefetch_hits) / self.demand if self.demand else 0.0


class SlotStack:
    def __init__(self, shape: synth.LayerShape, n_layers: int, n_slots: int,
                 scope: int = ft.SCOPE_GLOBAL, dev: str = "cuda", gen_device: str = "cuda"):
        self.sh, self.L, self.dev = shape, n_layers, dev
        self.n_exp = synth.n_experts_total(shape)
        self.stride = ft.slot_stride(shape.wdtype, shape.H, shape.I)
        self.expert_bytes = ft.expert_layout(shape.wdtype, shape.H, shape.I)[0]
        # pinned host pool [L][E][stride], filled from the seeded generator
        self.host = torch.empty((n_layers, self.n_exp, self.stride), dtype=torch.uint8,
                                pin_memory=True)
        stage = torch.empty((self.n_exp, self.stride), dtype=torch.uint8, device=dev)
        for l in range(n_layers):
            for e in range(self.n_exp):
                ex = synth.gen_expert(shape, e, l, device=gen_device)
                ft.pack_expert({k: v.to(dev) for k, v in ex.items()}, shape.wdtype, shape.H,
                               shape.I, stage[e])
            self.host[l].copy_(stage)
        del stage
        self.slots = torch.empty((n_slots, self.stride), dtype=torch.uint8, device=dev)
        self.cache = ft.SlotCache(n_layers, self.n_exp, self.expert_bytes, self.host,
                                  self.slots, scope)
        self.wts = ft.make_weights(shape.wdtype, shape.E, shape.H, shape.I, self.slots,
                                   n_shared=shape.n_shared, shared_slot=0)
        self.routers = [synth.gen_router(shape, l, device=dev) for l in range(n_layers)]
        self.biases = [synth.gen_bias(shape, l, device=dev) for l in range(n_layers)]
        # slot table per layer: one entry per expert of the layer (routed + shared)
        self.tables = [torch.full((self.n_exp,), -1, dtype=torch.int32, device=dev)
                       for _ in range(n_layers)]
        self.copy_stream = torch.cuda.Stream(device=dev)
        self.stats = StackStats()

    # ------------------------------------------------------------------
    def _route(self, l: int, x: torch.Tensor, logits: Optional[torch.Tensor] = None):
        sh = self.sh
        T = x.shape[0]
        if logits is None:
            ids, w, _ = ft.route(T, sh.E, sh.k, x=x, w_router=self.routers[l],
                                 bias=self.biases[l])
        else:
            ids, w, _ = ft.route(T, sh.E, sh.k, logits=logits, bias=self.biases[l])
        counts, offsets, perm, inv = ft.align(ids, sh.E)
        counts_h = torch.empty(sh.E, dtype=torch.int32, pin_memory=True)
        counts_h.copy_(counts, non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        return dict(ids=ids, w=w, offsets=offsets, perm=perm, inv=inv, counts_h=counts_h, ev=ev)

    def _experts_of(self, r) -> List[int]:
        r["ev"].synchronize()
        need = torch.nonzero(r["counts_h"]).flatten().tolist()
        return need + ([self.sh.E] if self.sh.n_shared else [])  # the shared expert rides along

    def _map(self, l: int, experts: List[int]):
        st = self.cache.map(l, experts, self.tables[l], copy=self.copy_stream)
        self.stats.demand += st.n_demand
        self.stats.hits += st.n_hit
        self.stats.prefetch_hits += st.n_prefetch_hit
        self.stats.misses += st.n_miss
        self.stats.bytes_h2d += st.bytes_h2d

    def _prefetch(self, l: int, experts: List[int]):
        before = self.cache.stats().bytes_h2d
        status, _ = self.cache.prefetch(l, experts, copy=self.copy_stream)
        self.stats.bytes_h2d += self.cache.stats().bytes_h2d - before
        if status == ft.WARN_OVERLAP_DISABLED:
            self.stats.prefetch_warnings += 1

    def forward(self, xs: List[torch.Tensor], prefill: bool = False,
                out_dtype=torch.bfloat16,
                logits: Optional[List[torch.Tensor]] = None) -> List[torch.Tensor]:
        """One pass through all layers; xs[l] is layer l's input batch [T, H]
        (independent per layer).  `logits` optionally supplies each layer's
        router logits instead of the router GEMM.  Returns the per-layer outputs."""
        sh = self.sh
        lg = logits if logits is not None else [None] * self.L
        outs = []
        r = self._route(0, xs[0], lg[0])
        self._map(0, self._experts_of(r))
        for l in range(self.L):
            nxt = self._route(l + 1, xs[l + 1], lg[l + 1]) if l + 1 < self.L else None
            if sh.n_shared:
                self.wts.shared_slot = self.cache.lookup(l, sh.E)
            y = ft.ffn(self.wts, xs[l], sh.k, r["perm"], r["offsets"],
                       slot_of_expert=self.tables[l])
            outs.append(ft.combine(y, r["inv"], r["w"], n_shared=sh.n_shared,
                                   out_dtype=out_dtype))
            self.cache.release(l)
            if nxt is not None:
                if prefill:
                    self._prefetch(l + 1, list(range(self.n_exp)))
                need = self._experts_of(nxt)
                if not prefill:
                    self._prefetch(l + 1, need)
                self._map(l + 1, need)
                r = nxt
        self.stats.steps += 1
        return outs

    def resize(self, n_slots: int, new_array: bool = False):
        """Grow or shrink the device slot budget between steps
        (ft_slot_cache_resize): resident experts that fit stay resident.  A
        budget beyond the current array, or new_array, moves the slots into a
        fresh array of n_slots (the old one is released once the copies are done)."""
        dev_slots = None
        if new_array or n_slots > self.slots.shape[0]:
            dev_slots = torch.empty((n_slots, self.stride), dtype=torch.uint8, device=self.dev)
        self.cache.resize(n_slots, dev_slots, copy=self.copy_stream)
        if dev_slots is not None:
            self.copy_stream.synchronize()
            self.slots = dev_slots
            self.wts = ft.make_weights(self.sh.wdtype, self.sh.E, self.sh.H, self.sh.I,
                                       self.slots, n_shared=self.sh.n_shared, shared_slot=0)

    def close(self):
        self.cache.close()
