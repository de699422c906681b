"""GPU checks of the whole-layer step (ft_moe_step_run) and of the same step
captured into a HIP graph (ft_moe_graph_*).

The eager step is checked against the oracle (picks bit-exact on the step's
own fp32 logits, outputs within the layer tolerance).  Each graph is then
replayed several times, with new activations copied into x in place and an
eager step plus synchronisations between the replays; every replay must give
the same bits (logits, picks, gates, output) as an eager step on the same x.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from expert_ffn_execution_amd import ftmoe as ft  # noqa: E402
from expert_ffn_execution_amd import synth  # noqa: E402
from oracle import oracle as orc  # noqa: E402
from tests.layer_harness import DEV, Layer, check_close, oracle_out  # noqa: E402

SHAPES = {
    "tiny_f32": synth.TINY_F32,
    "small_bf16": synth.LayerShape("graph_small_bf16", H=512, E=16, k=4, I=384, bias="zipf"),
    "small_mx": synth.LayerShape("graph_small_mx", H=512, E=16, k=6, I=256, n_shared=1,
                                 wdtype="mxfp4"),
    "35b_a3b_bf16": synth.A3B_BF16,
    "284b_a13b_mxfp4": synth.A13B_MXFP4,
    "35b_a3b_fp8": synth.A3B_FP8,
    "35b_a3b_nvfp4": synth.A3B_NVFP4,
}
# (shape, T, permuted slots): decode sizes take the streaming kernels, T = 300
# on the small shapes the MFMA tiles (tile list built on the device)
CASES = [("tiny_f32", 64, False), ("small_bf16", 3, True), ("small_bf16", 300, False),
         ("small_mx", 5, False), ("small_mx", 300, True), ("35b_a3b_bf16", 1, False),
         ("35b_a3b_bf16", 16, False), ("35b_a3b_bf16", 8, False), ("35b_a3b_bf16", 9, False),
         ("284b_a13b_mxfp4", 1, False), ("284b_a13b_mxfp4", 8, False), ("35b_a3b_fp8", 1, False),
         ("35b_a3b_fp8", 8, False), ("35b_a3b_fp8", 64, False), ("35b_a3b_nvfp4", 1, False),
         ("35b_a3b_nvfp4", 8, False)]
_LAYERS = {}


def _say(*a):
    print("[gpu-test]", *a, flush=True)


def _layer(name, permuted):
    key = (name, permuted)
    if key not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        sh = SHAPES[name]
        perm = None
        if permuted:
            n = synth.n_experts_total(sh)
            perm = list(np.random.default_rng(5).permutation(n))
        big = sh.E >= 128
        _LAYERS[key] = Layer(sh, gen_device=DEV if big else "cpu", keep_host=not big,
                             slot_perm=perm)
    return _LAYERS[key]


def _snapshot(step):
    return [t.clone() for t in (step.logits, step.ids, step.w, step.out)]


@pytest.mark.parametrize("name,T,permuted", CASES)
def test_step_and_graph(name, T, permuted):
    _say("step/graph", name, "T", T, "permuted slots" if permuted else "identity slots")
    L = _layer(name, permuted)
    sh = L.shape
    act = torch.float32 if sh.adtype == "f32" else torch.bfloat16
    y_dt = torch.float32 if sh.wdtype == "f32" else torch.bfloat16
    wr = synth.gen_router(sh, device=DEV)
    bias = synth.gen_bias(sh, device=DEV)
    x = synth.gen_x(sh, T, step=3, device=DEV).contiguous()
    step = ft.LayerStep(L.wts, x, sh.k, wr, bias=bias, slot_of_expert=L.slot_table,
                        y_dtype=y_dt, out_dtype=act)

    # eager step against the oracle
    step.run()
    torch.cuda.synchronize()
    lg = step.logits.cpu().numpy()
    ref_ids, ref_w = orc.route(lg, sh.k, None if bias is None else bias.cpu().numpy())
    assert np.array_equal(step.ids.cpu().numpy(), ref_ids)
    assert np.max(np.abs(step.w.cpu().numpy() - ref_w)) <= 1e-6
    check_close(step.out, oracle_out(L, x.cpu(), ref_ids, ref_w), sh.wdtype,
                f"step {name} T{T}")
    # the step (top-k and alignment fused for decode-sized batches) gives the
    # same bits as the four entry points called one by one
    ids, w, lg = ft.route(T, sh.E, sh.k, x=x, w_router=wr, bias=bias)
    counts, offsets, perm, inv = ft.align(ids, sh.E)
    y = ft.ffn(L.wts, x, sh.k, perm, offsets, slot_of_expert=L.slot_table, y_dtype=y_dt)
    out = ft.combine(y, inv, w, n_shared=sh.n_shared, out_dtype=act)
    torch.cuda.synchronize()
    for a, b, what in ((step.logits, lg, "logits"), (step.ids, ids, "ids"), (step.w, w, "w"),
                       (step.counts, counts, "counts"), (step.offsets, offsets, "offsets"),
                       (step.perm[:T * sh.k], perm, "perm"), (step.inv[:T * sh.k], inv, "inv"),
                       (step.out, out, "out")):
        assert torch.equal(a, b), f"step vs separate calls: {what}"

    # graph replays, each against an eager step on the same activations
    g = step.capture()
    try:
        for r in range(3):
            x.copy_(synth.gen_x(sh, T, step=10 + r, device=DEV))
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            got = _snapshot(step)
            step.run()
            torch.cuda.synchronize()
            want = _snapshot(step)
            for a, b, what in zip(got, want, ("logits", "ids", "w", "out")):
                assert torch.equal(a, b), f"replay {r}: {what} differs from the eager step"
    finally:
        g.close()


@pytest.mark.parametrize("T", [4, 600])
def test_profile_events_time_the_expert_kernels(T):
    """ft_set_profile_events on the gate/up and down stages: the events ride on
    the kernels' own dispatch; both read a positive time that fits inside the
    whole call, on the streaming (T = 4) and the MFMA (T = 600) path."""
    sh = synth.SHAPES["35b_a3b_bf16"]
    x = synth.gen_x(sh, T, device=DEV)
    pool = torch.empty((sh.E, ft.slot_stride(sh.wdtype, sh.H, sh.I)), dtype=torch.uint8, device=DEV)
    for e in range(sh.E):
        ft.pack_expert(synth.gen_expert(sh, e, device=DEV), sh.wdtype,
                       sh.H, sh.I, pool[e])
    wts = ft.make_weights(sh.wdtype, sh.E, sh.H, sh.I, pool)
    ids, w, _ = ft.route(T, sh.E, sh.k, x=x, w_router=synth.gen_router(sh, device=DEV))
    _, off, perm, _ = ft.align(ids, sh.E)
    ev = ft.HipEvents()
    pairs = {which: (ev.create(), ev.create()) for which in (ft.PROF_GEMM1, ft.PROF_GEMM2)}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        for which, (e0, e1) in pairs.items():
            ft.set_profile_events(which, e0, e1)
        a.record()
        ft.ffn(wts, x, sh.k, perm, off)
        b.record()
        torch.cuda.synchronize()
    finally:
        for which in pairs:
            ft.set_profile_events(which, None, None)
    total = a.elapsed_time(b)
    t1 = ev.elapsed_ms(*pairs[ft.PROF_GEMM1])
    t2 = ev.elapsed_ms(*pairs[ft.PROF_GEMM2])
    ev.close()
    assert 0 < t1 and 0 < t2 and t1 + t2 <= total * 1.05 + 0.01, (t1, t2, total)
