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


def _layer(E=6, H=256, I=128, k=2, T=5, seed=3):
    """E bf16 experts packed into one host pool, T tokens routed top-k at random,
    aligned by the oracle."""
    sh = synth.LayerShape(f"host_moe_{E}_{H}_{I}", H=H, E=E, k=k, I=I)
    stride = ft.slot_stride(sh.wdtype, H, I)
    pool = torch.zeros((E, stride), dtype=torch.uint8)
    exs = []
    for e in range(E):
        ex = synth.gen_expert(sh, e)
        ft.pack_expert(ex, sh.wdtype, H, I, pool[e])
        exs.append(ex)
    g = torch.Generator().manual_seed(seed)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    _, offsets, perm, _ = orc.align(ids.numpy(), E)
    x = synth.gen_x(sh, T)
    return sh, pool, exs, torch.from_numpy(offsets), torch.from_numpy(perm), x


def _job(sh, pool, offsets, perm, x, experts, max_rows=None, n_threads=4):
    T = x.shape[0]
    max_rows = T * sh.k if max_rows is None else max_rows
    rows = torch.full((max_rows, sh.H), float("nan"))
    pos = torch.full((max_rows,), -1, dtype=torch.int64)
    job = ft.host_moe_ffn_submit(pool, sh.E, sh.H, sh.I, sh.k, experts, offsets, perm, x,
                                 rows, pos, n_threads)
    return job, rows, pos


def test_moe_job_matches_per_expert_calls_and_oracle():
    sh, pool, exs, offsets, perm, x = _layer()
    experts = [4, 1, 3]
    job, rows, pos = _job(sh, pool, offsets, perm, x, experts)
    n = job.wait()
    want_n = sum(int(offsets[e + 1] - offsets[e]) for e in experts)
    assert n == want_n
    b = 0
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        tok = perm[lo:hi].long() // sh.k
        assert pos[b:b + hi - lo].tolist() == list(range(lo, hi))
        # the same bits as one expert at a time
        one = ft.host_expert_ffn(pool[e], x[tok], sh.H, sh.I, n_threads=3)
        assert torch.equal(rows[b:b + hi - lo], one)
        ref = np.stack([orc.expert_ffn(exs[e], "bf16", x[t].to(torch.float64).numpy(), sh.H, sh.I,
                                       True) for t in tok.tolist()])
        got = rows[b:b + hi - lo].numpy().astype(np.float64)
        assert np.linalg.norm(got - ref) <= 1e-4 * np.linalg.norm(ref)
        b += hi - lo
    assert pos[n:].eq(-1).all() and torch.isnan(rows[n:]).all()  # nothing beyond n_rows


def test_moe_jobs_queue_in_order():
    sh, pool, _, offsets, perm, x = _layer(E=8, T=9, seed=5)
    lists = [[0, 2], [7], [5, 6, 1], []]
    jobs = [_job(sh, pool, offsets, perm, x, ex) for ex in lists]
    for (job, rows, pos), ex in zip(jobs, lists):
        n = job.wait()
        ref, rpos, _ = _job(sh, pool, offsets, perm, x, ex, n_threads=1)
        assert ref.wait() == n
        assert torch.equal(rows[:n], rpos[:n]) and torch.equal(pos[:n], _[:n])


def test_moe_job_rejects_bad_descriptors():
    sh, pool, _, offsets, perm, x = _layer()
    with pytest.raises(ft.FtError) as ei:
        _job(sh, pool, offsets, perm, x, [1, 1])
    assert ei.value.status == ft.ERR_INVALID_ARG
    with pytest.raises(ft.FtError) as ei:
        _job(sh, pool, offsets, perm, x, [sh.E])
    assert ei.value.status == ft.ERR_INVALID_ARG
    big = [e for e in range(sh.E) if offsets[e + 1] > offsets[e]]
    with pytest.raises(ft.FtError) as ei:
        _job(sh, pool, offsets, perm, x, big, max_rows=1)
    assert ei.value.status == ft.ERR_CAPACITY
    bad = perm.clone()
    bad[int(offsets[big[0]])] = x.shape[0] * sh.k
    with pytest.raises(ft.FtError) as ei:
        _job(sh, pool, offsets, bad, x, big[:1])
    assert ei.value.status == ft.ERR_INVALID_ARG
    boff = offsets.clone()
    boff[big[0] + 1] = x.shape[0] * sh.k + 1
    with pytest.raises(ft.FtError):
        _job(sh, pool, boff, perm, x, big[:1])
    lib = ft.load()
    h, n = C.c_void_p(), C.c_int()
    assert lib.ft_host_moe_ffn_submit(None, C.byref(h), C.byref(n)) == ft.ERR_INVALID_ARG
    assert lib.ft_host_job_wait(None) == ft.ERR_INVALID_ARG
    job, _, _ = _job(sh, pool, offsets, perm, x, [])
    assert job.wait() == 0


def test_moe_jobs_from_several_threads():
    """Jobs submitted from four threads at once run one at a time and each
    gives the same bits as the same job alone."""
    import threading
    sh, pool, _, offsets, perm, x = _layer(E=8, T=12, seed=9)
    lists = [[0, 3], [7, 1], [2], [4, 5, 6]]
    want = []
    for ex in lists:
        job, rows, pos = _job(sh, pool, offsets, perm, x, ex, n_threads=2)
        n = job.wait()
        want.append((rows[:n].clone(), pos[:n].clone()))
    errors = []

    def worker(i):
        try:
            for _ in range(5):
                job, rows, pos = _job(sh, pool, offsets, perm, x, lists[i], n_threads=3)
                n = job.wait()
                assert torch.equal(rows[:n], want[i][0]) and torch.equal(pos[:n], want[i][1])
        except Exception as e:  # surfaced below
            errors.append(e)

    ths = [threading.Thread(target=worker, args=(i,)) for i in range(len(lists))]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    assert not errors, errors
