"""CPU checks of the host expert FFN (ft_host_expert_ffn), the CPU share of the
bandwidth-adaptive split of cache misses, and of the split's arithmetic.

The host FFN runs on the CPU, so these tests need no GPU: it is checked
against the oracle's expert FFN (fp64 sums, h rounded to bf16 as on the GPU),
for identical bits across thread counts, and for its argument checks.
"""
import ctypes as C

import numpy as np
import pytest
import torch

from expert_ffn_execution_amd import ftmoe as ft
from expert_ffn_execution_amd import synth
from expert_ffn_execution_amd.stack import split_misses
from oracle import oracle as orc


def _slot(sh, e=0):
    ex = synth.gen_expert(sh, e)
    raw = torch.zeros(ft.slot_stride(sh.wdtype, sh.H, sh.I), dtype=torch.uint8)
    ft.pack_expert(ex, sh.wdtype, sh.H, sh.I, raw)
    return ex, raw


@pytest.mark.parametrize("H,I,T", [(256, 192, 3), (2048, 768, 1), (128, 64, 5)])
def test_host_ffn_matches_oracle(H, I, T):
    sh = synth.LayerShape(f"host_ffn_{H}_{I}", H=H, E=1, k=1, I=I)
    ex, raw = _slot(sh)
    x = synth.gen_x(sh, T)
    y = ft.host_expert_ffn(raw, x, H, I, n_threads=4).numpy().astype(np.float64)
    ref = np.stack([orc.expert_ffn(ex, "bf16", x[r].to(torch.float64).numpy(), H, I, True)
                    for r in range(T)])
    # fp32 sums against fp64 ones; h is rounded to bf16 on both sides, so a few
    # elements of h may land one bf16 step apart where the sum sits on a tie
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel <= 1e-4, rel
    assert np.max(np.abs(y - ref)) <= 2e-3 * np.max(np.abs(ref))


def test_host_ffn_same_bits_for_any_thread_count():
    sh = synth.LayerShape("host_ffn_threads", H=512, E=1, k=1, I=256)
    _, raw = _slot(sh)
    x = synth.gen_x(sh, 4)
    ys = [ft.host_expert_ffn(raw, x, sh.H, sh.I, n_threads=n) for n in (1, 3, 8, 16)]
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


def test_host_ffn_rejects_bad_arguments():
    lib = ft.load()
    p = C.c_void_p(4096)
    assert lib.ft_host_expert_ffn(ft.FP8, 256, 128, p, p, ft.BF16, 1, p, 4) == ft.ERR_INVALID_ARG
    assert lib.ft_host_expert_ffn(ft.BF16, 100, 128, p, p, ft.BF16, 1, p, 4) == ft.ERR_INVALID_ARG
    assert lib.ft_host_expert_ffn(ft.BF16, 256, 128, p, p, ft.BF16, 1, p, 0) == ft.ERR_INVALID_ARG
    assert lib.ft_host_expert_ffn(ft.BF16, 256, 128, None, p, ft.BF16, 1, p, 4) == ft.ERR_INVALID_ARG
    assert lib.ft_host_expert_ffn(ft.BF16, 256, 128, None, None, ft.BF16, 0, None, 4) == ft.OK


def test_split_balances_the_two_sides():
    # n_gpu misses cross PCIe (Bp), the rest are read by the CPU (Bh): both
    # sides take about the same time, n_gpu / Bp ~ (m - n_gpu) / Bh
    assert split_misses(0, 52.7, 77.3) == 0
    assert split_misses(10, 52.7, 77.3) == 4          # 10 * 52.7 / 130 = 4.05
    assert split_misses(10, 1.0, 0.0) == 10            # no CPU: all to the GPU
    assert split_misses(10, 0.0, 1.0) == 0
    for m in range(1, 40):
        for bp, bh in ((52.7, 77.3), (57.3, 20.0), (10.0, 90.0)):
            n = split_misses(m, bp, bh)
            best = min(range(m + 1), key=lambda q: max(q / bp, (m - q) / bh))
            assert max(n / bp, (m - n) / bh) == pytest.approx(max(best / bp, (m - best) / bh))
