"""GPU test of ft_moe_ffn_noalloc (the FFN with its workspace in the
library's static scratch array) against ft_moe_ffn with a caller workspace.

Same kernels on the same inputs: the outputs must be bitwise equal, on both
kernel families, for two calls in a row whose second is smaller (the scratch
keeps the first call's contents), and at the largest 35B-A3B prefill whose
workspace fits the array.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from expert_ffn_execution_amd import ftmoe as ft  # noqa: E402
from expert_ffn_execution_amd import synth  # noqa: E402
from tests.layer_harness import DEV, Layer  # noqa: E402


def _say(*a):
    print("[gpu-test]", *a, flush=True)


@pytest.fixture(autouse=True)
def _reset_path():
    ft.set_ffn_path(0)
    yield
    ft.set_ffn_path(0)
    torch.cuda.synchronize()


def _routed(sh, T, step):
    x = synth.gen_x(sh, T, step=step, device=DEV)
    lg = synth.gen_logits(sh, T, step=step, device=DEV, scale=0.02 * np.sqrt(sh.H))
    ids, w, _ = ft.route(T, sh.E, sh.k, logits=lg)
    counts, offsets, perm, inv = ft.align(ids, sh.E)
    return x, perm, offsets


SHAPES = {
    "bf16": synth.LayerShape("noalloc_bf16", H=512, E=16, k=4, I=384, n_shared=1),
    "mxfp4": synth.LayerShape("noalloc_mx", H=512, E=16, k=6, I=256, n_shared=1, wdtype="mxfp4"),
}


@pytest.mark.parametrize("kind", list(SHAPES))
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("y_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_ffn_two_calls(kind, path, y_dtype):
    sh = SHAPES[kind]
    _say("ffn_noalloc", kind, "path", path, y_dtype)
    L = Layer(sh, keep_host=False)
    ft.set_ffn_path(path)
    for T, step in ((300, 0), (37, 1)):          # the second call is smaller
        x, perm, offsets = _routed(sh, T, step)
        ref = ft.ffn(L.wts, x, sh.k, perm, offsets, y_dtype=y_dtype)
        got = ft.ffn_noalloc(L.wts, x, sh.k, perm, offsets, y_dtype=y_dtype)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (kind, path, T)


def test_noalloc_full_size_prefill_and_decode():
    """The 35B-A3B layer at prefill T = 4096 (about 50 MB of workspace, most of
    the array), then a decode call at T = 16 in the same array."""
    sh = synth.A3B_BF16
    _say("ffn_noalloc 35b-a3b")
    L = Layer(sh, gen_device=DEV, keep_host=False)
    for T, step in ((4096, 0), (16, 1)):
        assert ft.ffn_workspace(L.wts, T, sh.k) <= ft.NOALLOC_SCRATCH_BYTES
        x, perm, offsets = _routed(sh, T, step)
        ref = ft.ffn(L.wts, x, sh.k, perm, offsets)
        got = ft.ffn_noalloc(L.wts, x, sh.k, perm, offsets)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), T


def test_noalloc_refuses_oversize_without_device_work():
    sh = synth.A3B_BF16
    _say("ffn_noalloc oversize")
    L = Layer(SHAPES["bf16"], keep_host=False)
    T = 8192
    wts = ft.make_weights(sh.wdtype, sh.E, sh.H, sh.I, L.pool)  # the array is never read
    x = torch.zeros((T, sh.H), dtype=torch.bfloat16, device=DEV)
    perm = torch.zeros(T * sh.k, dtype=torch.int32, device=DEV)
    offsets = torch.zeros(sh.E + 1, dtype=torch.int32, device=DEV)
    y = torch.full((T * sh.k, sh.H), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ft.FtError) as ei:
        ft.ffn_noalloc(wts, x, sh.k, perm, offsets, y=y)
    assert ei.value.status == ft.ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
