"""GPU tests of the host tier of the expert weights: a slot-table entry -2 - j
reads expert j of a pinned host array over the host link (zero-copy) instead
of a device slot.  The FFN must give bitwise the outputs of the same experts
held in device slots, on both kernel families and in every weight format."""
import pytest
import torch

pytestmark = pytest.mark.gpu

from expert_ffn_execution_amd import ftmoe as ft  # noqa: E402
from expert_ffn_execution_amd import synth  # noqa: E402
from tests.layer_harness import DEV, Layer  # noqa: E402

FORMATS = ("bf16", "mxfp4", "fp8", "nvfp4")


def _shape(fmt):
    return synth.LayerShape(f"host_tier_{fmt}", H=512, E=32, k=4, I=256, wdtype=fmt)


def _say(*a):
    print("[gpu-test]", *a, flush=True)


@pytest.mark.parametrize("fmt", FORMATS)
def test_host_tier_matches_device_slots(fmt):
    sh = _shape(fmt)
    _say("host tier", fmt)
    lay = Layer(sh, keep_host=False)
    g = torch.Generator().manual_seed(17)
    # host index j holds expert order[j] (not expert j), so an index mix-up shows
    order = torch.randperm(sh.E, generator=g)
    host = torch.empty((sh.E, lay.stride), dtype=torch.uint8, pin_memory=True)
    host.copy_(lay.pool[:sh.E][order.to(DEV)].cpu())
    where = torch.empty(sh.E, dtype=torch.int64)
    where[order] = torch.arange(sh.E)
    mixed = torch.tensor([e if e % 2 == 0 else -2 - int(where[e]) for e in range(sh.E)],
                         dtype=torch.int32, device=DEV)
    all_host = torch.tensor([-2 - int(where[e]) for e in range(sh.E)], dtype=torch.int32,
                            device=DEV)
    # without a host pool an entry -2 - j skips the expert, as -1 does
    wts_h = ft.make_weights(fmt, sh.E, sh.H, sh.I, lay.pool, host_pool=host)
    router = synth.gen_router(sh).to(DEV)
    for T in (1, 3, 64, 400):
        x = synth.gen_x(sh, T, step=T, device=DEV)
        ids, w, _ = ft.route(T, sh.E, sh.k, x=x, w_router=router)
        c, off, perm, inv = ft.align(ids, sh.E)
        for path in (1, 2):  # weight streaming, MFMA tiles
            old = ft.set_ffn_path(path)
            try:
                ref = ft.ffn(lay.wts, x, sh.k, perm, off, y_dtype=torch.float32)
                for name, table in (("mixed", mixed), ("all host", all_host)):
                    got = ft.ffn(wts_h, x, sh.k, perm, off, slot_of_expert=table,
                                 y_dtype=torch.float32)
                    assert torch.equal(got, ref), (fmt, T, path, name)
            finally:
                ft.set_ffn_path(old)
    torch.cuda.synchronize()


def test_host_entry_without_host_pool_skips_the_expert():
    sh = _shape("bf16")
    _say("host entry without a host pool")
    lay = Layer(sh, keep_host=False)
    router = synth.gen_router(sh).to(DEV)
    T = 5
    x = synth.gen_x(sh, T, device=DEV)
    ids, w, _ = ft.route(T, sh.E, sh.k, x=x, w_router=router)
    c, off, perm, inv = ft.align(ids, sh.E)
    skip = torch.full((sh.E,), -1, dtype=torch.int32, device=DEV)
    skip[0::2] = torch.arange(0, sh.E, 2, dtype=torch.int32, device=DEV)
    host_like = skip.clone()
    host_like[1::2] = -2 - torch.arange(1, sh.E, 2, dtype=torch.int32, device=DEV)
    sentinel = 7.0
    a = torch.full((T * sh.k, sh.H), sentinel, dtype=torch.float32, device=DEV)
    b = a.clone()
    ft.ffn(lay.wts, x, sh.k, perm, off, slot_of_expert=skip, y=a)
    ft.ffn(lay.wts, x, sh.k, perm, off, slot_of_expert=host_like, y=b)
    assert torch.equal(a, b)
    assert (a == sentinel).any()  # the odd experts' rows were left alone
