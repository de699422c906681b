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

Hybrid decode (``hybrid=True``): the pages' bandwidth-adaptive split of cache
misses.  Of the m experts of layer l+1 that are neither resident nor in
flight, n = ft_split_misses(m, Bp, Bh) are copied to the GPU as before and the
rest are computed on host cores straight from the pinned pool, as one job
queued on the library's host threads (ft_host_moe_ffn_submit) that overlaps
the GPU's work on layer l and the copies of layer l+1; their rows are copied
to the device and placed into layer l+1's y_perm by ft_moe_scatter_rows before
its combine.

Device-table decode (``device_table=True``): the pass runs without the host
waiting for any layer's histogram.  The library keeps a device slot table that
sends each expert either to its slot (once its copy has landed) or to the
pinned pool, read over the host link; the histograms come back in one copy
after the pass and the LRU takes them one or two passes later (``flush()``
settles the rest), copying missed experts into slots for the passes after.

Each layer's device buffers (logits, routing, alignment, workspaces, y_perm,
output) are allocated once per batch size and reused from step to step: the
outputs forward() returns stay valid until the next call.  Without hybrid
decode the whole pass is one library call (ft_slot_stack_forward), which does
the per-layer host work in C++; hybrid decode keeps the loop here.
Bp (pinned host-to-device GB/s) and Bh (host FFN GB/s of expert weights) come
from ``calibrate()`` (chenxutan.com article, "瓶颈为什么是带宽而不是容量", the
q* strategy; freelamp.com article, section 2.1).
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
import time
from typing import List, Optional

import torch

from . import ftmoe as ft
from . import synth


# How many of m missed experts to copy to the GPU (the rest run on host
# cores): the library's ft_split_misses.
split_misses = ft.split_misses


@dataclasses.dataclass
class StackStats:
    steps: int = 0
    demand: int = 0
    hits: int = 0
    prefetch_hits: int = 0
    misses: int = 0
    bytes_h2d: int = 0
    prefetch_warnings: int = 0
    cpu_experts: int = 0       # hybrid decode: missed experts computed on the host

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
        torch.cuda.synchronize()
        # one CPU read per 4 KB page of the pool: the first CPU pass over pinned
        # pages written by DMA ran at 6 GB/s, later passes at 85-95 GB/s (host
        # FFN of cold experts), so hybrid decode would pay it on its first misses
        int(self.host.view(-1)[::4096].sum())
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
        self._hbufs = [dict() for _ in range(n_layers)]
        self._dbufs = [dict() for _ in range(n_layers)]
        # host FFN outputs, two sets used by alternate layers: a set is refilled
        # only after the copy that read it two layers earlier has finished
        self._rows = [None, None]
        self._rows_dev = [None, None]
        self._rows_ev = [torch.cuda.Event(), torch.cuda.Event()]
        self.bp = self.bh = 0.0   # GB/s, from calibrate()
        self._steps = {}          # (T, out dtype) -> ctypes array of per-layer step descriptors
        self._counts_host = torch.empty((n_layers, shape.E), dtype=torch.int32, pin_memory=True)
        # host FFN threads: 8 measured fastest on a 16-core share (84-96 GB/s)
        self.host_threads = max(1, min(8, len(os.sched_getaffinity(0))))

    # ------------------------------------------------------------------
    def _dev_bufs(self, l: int, T: int, out_dtype) -> dict:
        """Layer l's device buffers for a batch of T tokens (allocated on the
        first use of this T, then reused)."""
        db = self._dbufs[l]
        if db.get("T") != T:
            sh, dev, k = self.sh, self.dev, self.sh.k
            i32, f32 = torch.int32, torch.float32
            self._steps.clear()  # descriptors name the buffers freed here
            db.clear()
            db.update(T=T, logits=torch.empty((T, sh.E), dtype=f32, device=dev),
                      ids=torch.empty((T, k), dtype=i32, device=dev),
                      w=torch.empty((T, k), dtype=f32, device=dev),
                      align=(torch.empty(sh.E, dtype=i32, device=dev),
                             torch.empty(sh.E + 1, dtype=i32, device=dev),
                             torch.empty(T * k, dtype=i32, device=dev),
                             torch.empty(T * k, dtype=i32, device=dev)),
                      aws=torch.empty(max(1, ft.align_workspace(T, k, sh.E)), dtype=torch.uint8,
                                      device=dev),
                      fws=torch.empty(max(256, ft.ffn_workspace(self.wts, T, k)),
                                      dtype=torch.uint8, device=dev),
                      y=torch.empty((T * k + sh.n_shared * T, sh.H), dtype=torch.bfloat16,
                                    device=dev))
        if db.get("out") is None or db["out"].dtype != out_dtype:
            self._steps.clear()
            db["out"] = torch.empty((T, self.sh.H), dtype=out_dtype, device=self.dev)
        return db

    def _route(self, l: int, x: torch.Tensor, logits: Optional[torch.Tensor] = None,
               want_x: bool = False, out_dtype=torch.bfloat16, stream=None):
        sh = self.sh
        T = x.shape[0]
        db = self._dev_bufs(l, T, out_dtype)
        if logits is None:
            ids, w, _ = ft.route(T, sh.E, sh.k, x=x, w_router=self.routers[l],
                                 bias=self.biases[l], logits_out=db["logits"], ids=db["ids"],
                                 w=db["w"], stream=stream)
        else:
            ids, w, _ = ft.route(T, sh.E, sh.k, logits=logits, bias=self.biases[l],
                                 ids=db["ids"], w=db["w"], stream=stream)
        counts, offsets, perm, inv = ft.align(ids, sh.E, ws=db["aws"], out=db["align"],
                                              stream=stream)
        hb = self._host_bufs(l, T)
        hb["counts"].copy_(counts, non_blocking=True)
        if want_x:  # the host FFN's inputs, ready with the routing (no wait on later work)
            hb["offsets"].copy_(offsets, non_blocking=True)
            hb["perm"].copy_(perm, non_blocking=True)
            hb["x"].copy_(x, non_blocking=True)
        ev = hb["ev"]
        ev.record()
        return dict(ids=ids, w=w, offsets=offsets, perm=perm, inv=inv, counts_h=hb["counts"],
                    hb=hb, ev=ev, db=db)

    def _host_bufs(self, l: int, T: int) -> dict:
        """Layer l's pinned read-back buffers for a batch of T tokens, reused
        from step to step (each is read on the host before the next step
        writes it again)."""
        hb = self._hbufs[l]
        if hb.get("T") != T:
            sh = self.sh
            pin = dict(pin_memory=True)
            hb.update(T=T, counts=torch.empty(sh.E, dtype=torch.int32, **pin),
                      offsets=torch.empty(sh.E + 1, dtype=torch.int32, **pin),
                      perm=torch.empty(T * sh.k, dtype=torch.int32, **pin),
                      x=torch.empty((T, sh.H), dtype=torch.bfloat16, **pin),
                      ev=torch.cuda.Event())
        return hb

    def _experts_of(self, r) -> List[int]:
        r["ev"].synchronize()
        need = torch.nonzero(r["counts_h"]).flatten().tolist()
        return need + ([self.sh.E] if self.sh.n_shared else [])  # the shared expert rides along

    def _map(self, l: int, experts: List[int], stream=None):
        st = self.cache.map(l, experts, self.tables[l], compute=stream, copy=self.copy_stream)
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

    # ---- hybrid decode: the CPU share of a layer's misses -----------------
    def calibrate(self, reps: int = 5):
        """Measure Bp (pinned host-to-device copy of one expert slot) and Bh
        (host FFN of one expert at T = 1, bytes of weights per second), GB/s."""
        sh = self.sh
        src = self.host[0][0]
        dst = torch.empty_like(src, device=self.dev)
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        self.bp = reps * self.expert_bytes / (time.perf_counter() - t) / 1e9
        x = torch.zeros((1, sh.H), dtype=torch.bfloat16)
        ft.host_expert_ffn(self.host[0][0], x, sh.H, sh.I, self.host_threads)
        n = min(4 * reps, sh.E - 1)  # distinct experts: weights come from DRAM, not cache
        t = time.perf_counter()
        for e in range(1, n + 1):
            ft.host_expert_ffn(self.host[self.L - 1][e], x, sh.H, sh.I, self.host_threads)
        self.bh = n * self.expert_bytes / (time.perf_counter() - t) / 1e9
        return self.bp, self.bh

    def _cpu_share(self, l: int, need: List[int]) -> List[int]:
        """Routed experts of layer l's demand to compute on the host: the
        misses beyond split_misses(m, Bp, Bh)."""
        miss = [e for e in need if e < self.sh.E and self.cache.lookup(l, e) < 0]
        return miss[split_misses(len(miss), self.bp, self.bh):]

    def _start_cpu(self, l: int, r: dict, experts: List[int]):
        """Queue the host FFN of `experts` on their rows of layer l
        (ft_host_moe_ffn_submit: the library's host threads run it while this
        thread goes on enqueueing GPU work).  r must come from _route with
        want_x (its event already waited on).  Returns (job, set) where
        set = (rows [n, H] fp32, pos [n] int64, event) pinned buffers."""
        sh, hb = self.sh, r["hb"]
        p = l & 1
        need = hb["T"] * sh.k
        if self._rows[p] is None or self._rows[p][0].shape[0] < need:
            self._rows[p] = (torch.empty((need, sh.H), dtype=torch.float32, pin_memory=True),
                             torch.empty(need, dtype=torch.int64, pin_memory=True))
            self._rows_dev[p] = (torch.empty((need, sh.H), dtype=torch.float32, device=self.dev),
                                 torch.empty(need, dtype=torch.int64, device=self.dev))
        else:
            self._rows_ev[p].synchronize()  # the copy out of this set two layers ago
        rows, pos = self._rows[p]
        job = ft.host_moe_ffn_submit(self.host[l], sh.E, sh.H, sh.I, sh.k, experts,
                                     hb["offsets"], hb["perm"], hb["x"], rows, pos,
                                     self.host_threads)
        self.stats.cpu_experts += len(experts)
        return job, (rows, pos, self._rows_dev[p], self._rows_ev[p])

    def _native_steps(self, T: int, out_dtype):
        """The per-layer ft_moe_step descriptors of the native pass for T tokens
        (buffers from _dev_bufs; x is set per call)."""
        key = (T, out_dtype)
        if key not in self._steps:
            sh = self.sh
            arr = (ft.MoeStep * self.L)()
            for l in range(self.L):
                db = self._dev_bufs(l, T, out_dtype)
                c, off, perm, inv = db["align"]
                b = self.biases[l]
                arr[l] = ft.MoeStep(self.wts, 0, ft.BF16, self.routers[l].data_ptr(),
                                    None if b is None else b.data_ptr(), T, sh.k,
                                    self.tables[l].data_ptr(), db["logits"].data_ptr(),
                                    db["ids"].data_ptr(), db["w"].data_ptr(), c.data_ptr(),
                                    off.data_ptr(), perm.data_ptr(), inv.data_ptr(),
                                    db["aws"].data_ptr(), db["aws"].numel(), db["y"].data_ptr(),
                                    ft.BF16, db["fws"].data_ptr(), db["fws"].numel(),
                                    db["out"].data_ptr(), ft._dt(db["out"]))
            self._steps[key] = arr
        return self._steps[key]

    def _add_stats(self, st):
        self.stats.demand += st.demand
        self.stats.hits += st.hits
        self.stats.prefetch_hits += st.prefetch_hits
        self.stats.misses += st.misses
        self.stats.bytes_h2d += st.bytes_h2d
        self.stats.prefetch_warnings += st.prefetch_warnings

    def flush(self):
        """Take every pending device-table pass through the LRU (its stats
        are then in self.stats)."""
        st = self.cache.forward_stack(None, 0, None, device_table=True,
                                      compute=torch.cuda.current_stream(), copy=self.copy_stream)
        self._add_stats(st)

    def _forward_native(self, xs, prefill, out_dtype, logits, device_table=False):
        T = xs[0].shape[0]
        arr = self._native_steps(T, out_dtype)
        for l in range(self.L):
            if xs[l].shape[0] != T or not xs[l].is_cuda or not xs[l].is_contiguous():
                raise ValueError("every layer's input must be a contiguous device [T, H] tensor")
            arr[l].x = xs[l].data_ptr()
        lin = None
        if logits is not None:
            lin = (C.c_void_p * self.L)(*[None if a is None else a.data_ptr() for a in logits])
        st = self.cache.forward_stack(arr, self.L, self._counts_host, lin, prefill,
                                      compute=torch.cuda.current_stream(), copy=self.copy_stream,
                                      device_table=device_table)
        self._add_stats(st)
        self.stats.steps += 1
        return [self._dbufs[l]["out"] for l in range(self.L)]

    def forward(self, xs: List[torch.Tensor], prefill: bool = False,
                out_dtype=torch.bfloat16,
                logits: Optional[List[torch.Tensor]] = None,
                hybrid: bool = False, device_table: bool = False) -> List[torch.Tensor]:
        """One pass through all layers; xs[l] is layer l's input batch [T, H]
        (independent per layer).  `logits` optionally supplies each layer's
        router logits instead of the router GEMM.  `hybrid` splits each layer's
        misses between PCIe copies and host cores (decode; needs calibrate()).
        `device_table` runs a decode pass without host waits: experts not in
        a slot are read from the pinned pool over the host link, and the LRU
        takes the pass's routing one or two passes later (flush() settles it).
        Returns the per-layer outputs."""
        sh = self.sh
        if hybrid and sh.wdtype != "bf16":
            raise ValueError("hybrid decode computes missed experts on the host in bf16 only")
        if hybrid and device_table:
            raise ValueError("hybrid and device_table decode are separate modes")
        if not (hybrid and not prefill):
            return self._forward_native(xs, prefill, out_dtype, logits, device_table)
        lg = logits if logits is not None else [None] * self.L
        outs = []
        want_x = hybrid and not prefill
        cs = torch.cuda.current_stream()  # the compute stream (looked up once)
        r = self._route(0, xs[0], lg[0], out_dtype=out_dtype, stream=cs)
        self._map(0, self._experts_of(r), cs)
        for l in range(self.L):
            nxt = (self._route(l + 1, xs[l + 1], lg[l + 1], want_x=want_x, out_dtype=out_dtype,
                               stream=cs)
                   if l + 1 < self.L else None)
            if sh.n_shared:
                self.wts.shared_slot = self.cache.lookup(l, sh.E)
            db = r["db"]
            y = ft.ffn(self.wts, xs[l], sh.k, r["perm"], r["offsets"],
                       slot_of_expert=self.tables[l], y=db["y"], ws=db["fws"], stream=cs)
            if "cpu" in r:  # the host's rows of this layer (its experts were skipped above)
                job, (rows, pos, (rows_d, pos_d), ev) = r["cpu"]
                n = job.wait()
                if n:
                    rows_d[:n].copy_(rows[:n], non_blocking=True)
                    pos_d[:n].copy_(pos[:n], non_blocking=True)
                    ft.scatter_rows(rows_d, pos_d, y, n, stream=cs)
                ev.record()
            outs.append(ft.combine(y, r["inv"], r["w"], n_shared=sh.n_shared, out=db["out"],
                                   stream=cs))
            self.cache.release(l, compute=cs)
            if nxt is not None:
                if prefill:
                    self._prefetch(l + 1, list(range(self.n_exp)))
                need = self._experts_of(nxt)
                if want_x:
                    cpu = self._cpu_share(l + 1, need)
                    if cpu:
                        need = [e for e in need if e not in cpu]
                        nxt["cpu"] = self._start_cpu(l + 1, nxt, cpu)
                if not prefill:
                    self._prefetch(l + 1, need)
                self._map(l + 1, need, cs)
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
            self._steps.clear()  # their weights name the old array

    def close(self):
        self.cache.close()
