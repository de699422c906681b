"""GPU tests of the expert-slot cache: layers whose experts stream from pinned
host memory through LRU device slots must give bitwise the same outputs as the
same layers with every expert resident, and match the oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from expert_ffn_execution_amd import ftmoe as ft  # noqa: E402
from expert_ffn_execution_amd import synth  # noqa: E402
from expert_ffn_execution_amd.stack import SlotStack  # noqa: E402
from tests.layer_harness import DEV, check_close, unpack_slot  # noqa: E402
from oracle import oracle as orc  # noqa: E402

SMALL = synth.LayerShape("gpu_stack_small", H=512, E=32, k=4, I=256, bias="zipf", bias_param=1.1)


def _say(*a):
    print("[gpu-test]", *a, flush=True)


def _resident_layer(stack: SlotStack, l: int, x: torch.Tensor):
    """Layer l with all its experts resident (same kernels, identity slots)."""
    sh = stack.sh
    pool = stack.host[l].to(DEV)
    wts = ft.make_weights(sh.wdtype, sh.E, sh.H, sh.I, pool, n_shared=sh.n_shared,
                          shared_slot=sh.E)
    ids, w, _ = ft.route(x.shape[0], sh.E, sh.k, x=x, w_router=stack.routers[l],
                         bias=stack.biases[l])
    c, off, perm, inv = ft.align(ids, sh.E)
    y = ft.ffn(wts, x, sh.k, perm, off)
    return ft.combine(y, inv, w, n_shared=sh.n_shared), ids, w


def _inputs(sh, L, T, step):
    return [synth.gen_x(sh, T, step=step, device=DEV, layer=l) for l in range(L)]


@pytest.mark.parametrize("scope", [ft.SCOPE_GLOBAL, ft.SCOPE_PER_LAYER])
def test_decode_steps_match_resident(scope):
    _say("slot stack decode scope", scope)
    L = 4
    st = SlotStack(SMALL, L, n_slots=24, scope=scope)
    try:
        for step in range(6):
            xs = _inputs(SMALL, L, 2, step)
            outs = st.forward(xs)
            for l in range(L):
                ref, _, _ = _resident_layer(st, l, xs[l])
                assert torch.equal(outs[l], ref), (step, l)
        assert st.stats.demand > 0 and st.stats.misses > 0
        assert st.stats.hits + st.stats.prefetch_hits + st.stats.misses == st.stats.demand
        cs = st.cache.stats()
        assert cs.held == 0 and cs.resident <= 24
    finally:
        st.close()


def test_prefill_overlap_and_warning():
    _say("slot stack prefill")
    L = 3
    # two whole layers fit: whole-layer prefetch succeeds
    st = SlotStack(SMALL, L, n_slots=2 * SMALL.E)
    try:
        xs = _inputs(SMALL, L, 300, 0)
        outs = st.forward(xs, prefill=True)
        for l in range(L):
            ref, _, _ = _resident_layer(st, l, xs[l])
            assert torch.equal(outs[l], ref), l
        assert st.stats.prefetch_warnings == 0
        assert st.stats.prefetch_hits > 0
    finally:
        st.close()
    # fewer than two layers of slots: the prefetch reports overlap disabled, results unchanged
    st = SlotStack(SMALL, L, n_slots=SMALL.E + 8)
    try:
        outs = st.forward(xs, prefill=True)
        for l in range(L):
            ref, _, _ = _resident_layer(st, l, xs[l])
            assert torch.equal(outs[l], ref), l
        assert st.stats.prefetch_warnings > 0
    finally:
        st.close()


def test_stack_layer_matches_oracle():
    _say("slot stack vs oracle")
    L = 2
    st = SlotStack(SMALL, L, n_slots=20)
    try:
        xs = _inputs(SMALL, L, 16, 3)
        # oracle router logits, supplied to both sides so routing is identical by construction
        lgs = [orc.router_logits(xs[l].cpu(), st.routers[l].cpu()) for l in range(L)]
        outs = st.forward(xs, logits=[torch.from_numpy(a).to(DEV) for a in lgs])
        for l in range(L):
            ids, w = orc.route(lgs[l], SMALL.k, st.biases[l].cpu().numpy())
            experts = [unpack_slot(st.host[l, e], SMALL) for e in range(SMALL.E)]
            ref = orc.moe_layer(xs[l].cpu(), ids, w, experts, "bf16", SMALL.I, out_fmt="f32")
            check_close(outs[l], ref, "bf16", f"stack layer {l}")
    finally:
        st.close()


def test_pageable_pool_is_refused():
    _say("pageable pool")
    host = torch.empty((2, 4, 4096), dtype=torch.uint8)          # not pinned
    slots = torch.empty((4, 4096), dtype=torch.uint8, device=DEV)
    with pytest.raises(ft.FtError) as ei:
        ft.SlotCache(2, 4, 4096, host, slots)
    assert ei.value.status == ft.ERR_NOT_PINNED


def test_full_size_slot_stack_sampled():
    """8 layers of the 35B-A3B layer shape, 64 slots per layer under one global
    LRU, Zipf(1.1)-biased routers: a few decode steps and one prefill, each
    layer's output compared with the resident computation; then decode steps
    and a prefill with every layer compared with the oracle."""
    sh = synth.SLOT_STACK
    L = synth.SLOT_STACK_LAYERS
    _say("full-size slot stack")
    st = SlotStack(sh, L, n_slots=L * synth.SLOT_STACK_SLOTS_PER_LAYER)
    try:
        for step in range(3):
            xs = _inputs(sh, L, 1, step)
            outs = st.forward(xs)
            l = step % L
            ref, _, _ = _resident_layer(st, l, xs[l])
            assert torch.equal(outs[l], ref)
        xs = _inputs(sh, L, 2048, 100)
        outs = st.forward(xs, prefill=True)
        for l in (0, L - 1):
            ref, _, _ = _resident_layer(st, l, xs[l])
            assert torch.equal(outs[l], ref)
        assert st.stats.prefetch_warnings == 0
        _say("  hit rate", st.stats.hit_rate, "demand", st.stats.demand)
        # every layer against the oracle, routed from the oracle's logits on both
        # sides: two decode steps (all tokens) and one prefill (64 seeded tokens
        # of each layer)
        experts = [[unpack_slot(st.host[l, e], sh) for e in range(sh.E)] for l in range(L)]
        rng = np.random.default_rng(5)
        for step, T in ((200, 1), (201, 1), (202, 2048)):
            xs = _inputs(sh, L, T, step)
            lgs = [orc.router_logits(xs[l].cpu(), st.routers[l].cpu()) for l in range(L)]
            outs = st.forward(xs, logits=[torch.from_numpy(a).to(DEV) for a in lgs],
                              prefill=T > 1)
            tok = (np.arange(T, dtype=np.int32) if T <= 64
                   else np.sort(rng.choice(T, size=64, replace=False)).astype(np.int32))
            for l in range(L):
                ids, w = orc.route(lgs[l], sh.k, st.biases[l].cpu().numpy())
                ref = orc.moe_layer(xs[l].cpu(), ids, w, experts[l], "bf16", sh.I, out_fmt="f32",
                                    tokens=tok)
                got = outs[l].cpu()[torch.from_numpy(tok).long()]
                e, m = check_close(got, ref, "bf16", f"full-size stack T{T} layer {l}")
            _say(f"  oracle T={T}: {L} layers, last rel_l2 {e:.3e} max/amax {m:.3e}")
        assert st.stats.prefetch_warnings == 0
    finally:
        st.close()


def _slots_hold_their_experts(st):
    """Every resident (layer, expert) slot holds that expert's bytes."""
    torch.cuda.synchronize()
    st.copy_stream.synchronize()
    n = 0
    for l in range(st.L):
        for e in range(st.n_exp):
            s = st.cache.lookup(l, e)
            if s < 0:
                continue
            got = st.slots[s, :st.expert_bytes].cpu()
            assert torch.equal(got, st.host[l, e, :st.expert_bytes]), (l, e, s)
            n += 1
    return n


def test_resize_between_steps_matches_resident():
    """ft_slot_cache_resize: shrink in place, grow into a new array, shrink into
    a new array; after each, the resident slots hold their experts' bytes and
    decode steps stay bitwise equal to the all-resident layers."""
    _say("slot stack resize")
    L = 4
    st = SlotStack(SMALL, L, n_slots=24)
    try:
        step = 0
        for n_slots, new_array in ((24, False), (12, False), (40, False), (20, True)):
            if step:
                st.resize(n_slots, new_array)
                cs = st.cache.stats()
                assert cs.n_slots == n_slots and cs.resident <= n_slots
                assert _slots_hold_their_experts(st) == cs.resident
            for _ in range(2):
                xs = _inputs(SMALL, L, 2, step)
                outs = st.forward(xs)
                for l in range(L):
                    ref, _, _ = _resident_layer(st, l, xs[l])
                    assert torch.equal(outs[l], ref), (n_slots, step, l)
                step += 1
        assert st.cache.stats().held == 0
    finally:
        st.close()


@pytest.mark.parametrize("bp,bh", [(1.0, 1.0), (1.0, 1e6), (1e-6, 1.0)])
def test_hybrid_decode_matches_oracle(bp, bh):
    """Misses split between PCIe copies and host cores (bp:bh sets the share:
    half, nearly all on the host, all on the host): every layer still matches
    the oracle, the host rows being the CPU FFN's."""
    _say("slot stack hybrid decode", bp, bh)
    L = 3
    st = SlotStack(SMALL, L, n_slots=12)
    st.bp, st.bh = bp, bh
    try:
        experts = [[unpack_slot(st.host[l, e], SMALL) for e in range(SMALL.E)] for l in range(L)]
        for step, T in enumerate((2, 5, 1, 3)):  # T changes: read-back buffers are re-sized
            xs = _inputs(SMALL, L, T, 40 + step)
            lgs = [orc.router_logits(xs[l].cpu(), st.routers[l].cpu()) for l in range(L)]
            outs = st.forward(xs, logits=[torch.from_numpy(a).to(DEV) for a in lgs], hybrid=True)
            for l in range(L):
                ids, w = orc.route(lgs[l], SMALL.k, st.biases[l].cpu().numpy())
                ref = orc.moe_layer(xs[l].cpu(), ids, w, experts[l], "bf16", SMALL.I, out_fmt="f32")
                check_close(outs[l], ref, "bf16", f"hybrid step {step} layer {l}")
        assert st.stats.cpu_experts > 0
        cs = st.cache.stats()
        assert cs.held == 0
    finally:
        st.close()


def test_full_size_hybrid_decode_matches_oracle():
    """Two layers of the 35B-A3B layer shape behind 24 slots, with the
    calibrated bandwidths: misses go both ways, and each layer's output of a
    few 4-token decode steps matches the oracle."""
    sh = synth.SLOT_STACK
    L = 2
    _say("full-size hybrid decode")
    st = SlotStack(sh, L, n_slots=24)
    try:
        bp, bh = st.calibrate()
        _say("  calibrated Bp", bp, "Bh", bh)
        experts = [[unpack_slot(st.host[l, e], sh) for e in range(sh.E)] for l in range(L)]
        for step in range(3):
            xs = _inputs(sh, L, 4, 300 + step)
            lgs = [orc.router_logits(xs[l].cpu(), st.routers[l].cpu()) for l in range(L)]
            outs = st.forward(xs, logits=[torch.from_numpy(a).to(DEV) for a in lgs], hybrid=True)
            for l in range(L):
                ids, w = orc.route(lgs[l], sh.k, st.biases[l].cpu().numpy())
                ref = orc.moe_layer(xs[l].cpu(), ids, w, experts[l], "bf16", sh.I, out_fmt="f32")
                check_close(outs[l], ref, "bf16", f"full-size hybrid step {step} layer {l}")
        _say("  host experts", st.stats.cpu_experts, "misses", st.stats.misses)
        assert st.stats.cpu_experts > 0 and st.stats.bytes_h2d > 0
    finally:
        st.close()


def test_calibrate_measures_both_bandwidths():
    st = SlotStack(SMALL, 1, n_slots=8)
    try:
        bp, bh = st.calibrate()
        assert bp > 0.1 and bh > 0.01, (bp, bh)
    finally:
        st.close()


# ---------------------------------------------------------------------------
# device-table decode passes (FT_STACK_DEVICE_TABLE)

@pytest.mark.parametrize("n_slots", [12, 40])
def test_device_table_decode_matches_resident(n_slots):
    """Passes enqueued without host waits: experts in slots are read there,
    the others from the pinned pool; every layer bitwise equal to the
    all-resident layer, and after a flush the LRU has counted every pass."""
    _say("device-table decode, slots", n_slots)
    L = 4
    st = SlotStack(SMALL, L, n_slots=n_slots)
    try:
        for step in range(10):
            xs = _inputs(SMALL, L, 2, 500 + step)
            outs = st.forward(xs, device_table=True)
            for l in range(L):
                ref, _, _ = _resident_layer(st, l, xs[l])
                assert torch.equal(outs[l], ref), (n_slots, step, l)
        st.flush()
        s = st.stats
        assert s.demand > 0 and s.misses > 0
        # 12 slots are fewer than one pass's distinct experts (about 20 over
        # the 4 layers), so the LRU thrashes; 40 hold them
        if n_slots >= 40:
            assert s.hits > 0
        assert s.hits + s.prefetch_hits + s.misses == s.demand
        cs = st.cache.stats()
        assert cs.held == 0 and 0 < cs.resident <= n_slots
        # after the flush every copy it issued lands, and the slots hold their experts
        assert _slots_hold_their_experts(st) == cs.resident
    finally:
        st.close()


def test_device_table_decode_between_other_modes():
    """Device-table passes, a prefill through the per-layer path (which first
    settles the pending passes), per-layer decode, a resize, and device-table
    passes again: every layer of every pass bitwise equal to the resident one."""
    _say("device-table decode between other modes")
    L = 3
    st = SlotStack(SMALL, L, n_slots=2 * SMALL.E)
    try:
        def check(outs, xs, what):
            for l in range(L):
                ref, _, _ = _resident_layer(st, l, xs[l])
                assert torch.equal(outs[l], ref), (what, l)

        for step in range(3):
            xs = _inputs(SMALL, L, 1, 600 + step)
            check(st.forward(xs, device_table=True), xs, f"dt {step}")
        xs = _inputs(SMALL, L, 300, 610)
        check(st.forward(xs, prefill=True, device_table=True), xs, "prefill")
        assert st.stats.prefetch_warnings == 0
        for step in range(2):
            xs = _inputs(SMALL, L, 2, 620 + step)
            check(st.forward(xs), xs, f"per-layer {step}")
        st.resize(20, new_array=True)
        for step in range(4):
            xs = _inputs(SMALL, L, 3, 630 + step)
            check(st.forward(xs, device_table=True), xs, f"dt after resize {step}")
        st.flush()
        s = st.stats
        assert s.hits + s.prefetch_hits + s.misses == s.demand
        cs = st.cache.stats()
        assert cs.held == 0 and cs.resident <= 20
        assert _slots_hold_their_experts(st) == cs.resident
    finally:
        st.close()


def test_full_size_device_table_decode_matches_oracle():
    """8 layers of the 35B-A3B layer shape, 512 slots under one global LRU,
    Zipf(1.1)-biased routers: device-table decode steps, each layer compared
    with the resident computation, the last two with the oracle."""
    sh = synth.SLOT_STACK
    L = synth.SLOT_STACK_LAYERS
    _say("full-size device-table decode")
    st = SlotStack(sh, L, n_slots=L * synth.SLOT_STACK_SLOTS_PER_LAYER)
    try:
        for step in range(6):
            xs = _inputs(sh, L, 1, 700 + step)
            outs = st.forward(xs, device_table=True)
            for l in range(L):
                ref, _, _ = _resident_layer(st, l, xs[l])
                assert torch.equal(outs[l], ref), (step, l)
        experts = [[unpack_slot(st.host[l, e], sh) for e in range(sh.E)] for l in range(L)]
        for step in (710, 711):
            xs = _inputs(sh, L, 1, step)
            lgs = [orc.router_logits(xs[l].cpu(), st.routers[l].cpu()) for l in range(L)]
            outs = st.forward(xs, logits=[torch.from_numpy(a).to(DEV) for a in lgs],
                              device_table=True)
            for l in range(L):
                ids, w = orc.route(lgs[l], sh.k, st.biases[l].cpu().numpy())
                ref = orc.moe_layer(xs[l].cpu(), ids, w, experts[l], "bf16", sh.I, out_fmt="f32")
                check_close(outs[l], ref, "bf16", f"device-table step {step} layer {l}")
        st.flush()
        s = st.stats
        _say("  demand", s.demand, "hits", s.hits, "misses", s.misses)
        assert s.hits + s.prefetch_hits + s.misses == s.demand and s.misses > 0
        assert st.cache.stats().held == 0
    finally:
        st.close()


def test_device_table_decode_beyond_layer_capacity():
    """Per-layer scope with 3 slots per layer and up to 16 distinct experts per
    layer: the LRU cannot take a layer's experts (the bookkeeping counts them
    and moves on), and every pass still matches the resident layers."""
    _say("device-table decode beyond a layer's slots")
    L = 2
    st = SlotStack(SMALL, L, n_slots=3 * L, scope=ft.SCOPE_PER_LAYER)
    try:
        for step in range(4):
            xs = _inputs(SMALL, L, 4, 800 + step)
            outs = st.forward(xs, device_table=True)
            for l in range(L):
                ref, _, _ = _resident_layer(st, l, xs[l])
                assert torch.equal(outs[l], ref), (step, l)
        st.flush()
        s = st.stats
        assert s.demand > 0 and s.hits + s.prefetch_hits + s.misses == s.demand
        assert st.cache.stats().held == 0
    finally:
        st.close()


def test_mixed_operations_random_walk():
    """A seeded random walk over the cache's operations: device-table and
    per-layer decode passes, prefills, explicit evictions of one expert or a
    whole layer, and resizes (in place and into a new array).  After every
    pass each layer equals the resident layer bitwise; at the end the LRU's
    counts add up and every resident slot holds its expert.  The per-layer
    passes map a layer's experts before it runs, so they run only where the
    slots can take them (a prefill routes to all 32 experts, T = 4 decode to
    up to 16); device-table passes run at any budget."""
    _say("slot cache random walk")
    L = 3
    n_slots = 24
    st = SlotStack(SMALL, L, n_slots=n_slots)
    rng = np.random.default_rng(2034)  # a walk that visits every kind of operation
    try:
        step = 0
        for it in range(32):
            op = rng.choice(["dt", "dt", "dt", "layer", "prefill", "evict", "resize"])
            if op == "prefill" and n_slots < SMALL.E:
                op = "dt"
            if op in ("dt", "layer", "prefill"):
                T = 300 if op == "prefill" else int(rng.integers(1, 5))
                if op == "layer":
                    T = min(T, n_slots // SMALL.k)
                xs = _inputs(SMALL, L, T, 900 + step)
                step += 1
                outs = st.forward(xs, prefill=op == "prefill", device_table=op != "layer")
                for l in range(L):
                    ref, _, _ = _resident_layer(st, l, xs[l])
                    assert torch.equal(outs[l], ref), (it, op, l)
            elif op == "evict":
                st.flush()  # nothing of this cache may be held or in flight for an eviction
                torch.cuda.synchronize()
                st.copy_stream.synchronize()
                l = int(rng.integers(0, L))
                st.cache.evict(l, int(rng.integers(-1, SMALL.E)))
            else:
                st.flush()
                n_slots = int(rng.choice([8, 20, 2 * SMALL.E]))
                st.resize(n_slots, new_array=bool(rng.integers(0, 2)))
        st.flush()
        s = st.stats
        assert s.demand > 0 and s.hits + s.prefetch_hits + s.misses == s.demand
        cs = st.cache.stats()
        assert cs.held == 0
        assert _slots_hold_their_experts(st) == cs.resident
    finally:
        st.close()
