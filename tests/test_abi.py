"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching a GPU."""
import ctypes as C
import os
import re

import pytest

from expert_ffn_execution_amd import ftmoe as ft

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ftmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ft_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_what_binding_lists():
    assert sorted(ft.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    lib = ft.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.ft_version().startswith(b"ftmoe")


def test_expert_layout():
    n, offs = ft.expert_layout("bf16", 2048, 768)
    assert n == 3 * 2048 * 768 * 2 and offs[:3] == [0, 2048 * 768 * 2, 2 * 2048 * 768 * 2]
    n, offs = ft.expert_layout("mxfp4", 4096, 2048)
    HI = 4096 * 2048
    assert n == 3 * HI // 2 + 3 * HI // 32
    assert offs == [0, HI // 2, HI, 3 * HI // 2, 3 * HI // 2 + HI // 32, 3 * HI // 2 + HI // 16]
    n, offs = ft.expert_layout("fp8", 2048, 768)
    HI = 2048 * 768
    assert n == 3 * HI + 16 and offs == [0, HI, 2 * HI, 3 * HI, 3 * HI + 4, 3 * HI + 8]
    n, offs = ft.expert_layout("nvfp4", 2048, 768)
    assert n == 3 * HI // 2 + 3 * HI // 16 + 16
    assert offs == [0, HI // 2, HI, 3 * HI // 2, 3 * HI // 2 + HI // 16, 3 * HI // 2 + HI // 8]
    with pytest.raises(ft.FtError):
        ft.expert_layout("bf16", 100, 64)


def _route(**kw):
    lib = ft.load()
    a = dict(x=None, x_dt=ft.BF16, w_router=None, logits_in=C.c_void_p(16), bias=None, T=4, H=0,
             E=8, k=2, logits_out=None, ids=C.c_void_p(16), w=C.c_void_p(16), s=None)
    a.update(kw)
    return lib.ft_moe_route(a["x"], a["x_dt"], a["w_router"], a["logits_in"], a["bias"], a["T"],
                            a["H"], a["E"], a["k"], a["logits_out"], a["ids"], a["w"], a["s"])


def test_route_rejects_bad_arguments():
    assert _route(k=0) == ft.ERR_INVALID_ARG
    assert _route(k=9) == ft.ERR_INVALID_ARG
    assert _route(E=1025, k=2) == ft.ERR_INVALID_ARG
    assert _route(T=-1) == ft.ERR_INVALID_ARG
    assert _route(T=1 << 30, k=2) == ft.ERR_INVALID_ARG          # T*k >= 2^31
    assert _route(ids=None) == ft.ERR_INVALID_ARG
    assert _route(x=C.c_void_p(16)) == ft.ERR_INVALID_ARG         # both logits and x
    assert _route(logits_in=None) == ft.ERR_INVALID_ARG          # neither
    assert _route(logits_in=None, x=C.c_void_p(16), w_router=C.c_void_p(16),
                  logits_out=C.c_void_p(16), H=100) == ft.ERR_INVALID_ARG
    assert _route(T=0) == ft.OK                                  # empty batch: no-op
    assert "k must be" in ft.last_error() or ft.last_error() == ""


def test_align_rejects_bad_arguments():
    lib = ft.load()
    p = C.c_void_p(16)
    assert lib.ft_moe_align(p, 4, 0, 8, p, p, p, p, None, 0, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_align(p, 4, 2, 2000, p, p, p, p, None, 0, None) == ft.ERR_INVALID_ARG
    # large problems need the workspace
    need = lib.ft_moe_align_workspace(10000, 8, 256)
    assert need > 0
    assert lib.ft_moe_align(p, 10000, 8, 256, p, p, p, p, None, 0, None) == ft.ERR_INVALID_ARG
    assert "workspace" in ft.last_error()


def _w(**kw):
    a = dict(w_dt=ft.BF16, E=8, H=256, I=128, n_shared=0, pool=4096,
             slot_stride=ft.slot_stride("bf16", 256, 128), shared_slot=0, host_pool=None,
             host_stride=0)
    a.update(kw)
    return ft.MoeWeights(a["w_dt"], a["E"], a["H"], a["I"], a["n_shared"], a["pool"],
                         a["slot_stride"], a["shared_slot"], a["host_pool"], a["host_stride"])


def test_ffn_rejects_bad_arguments():
    lib = ft.load()
    p = C.c_void_p(4096)

    def call(w, act=ft.BF16, ydt=ft.BF16, ws_bytes=1 << 30, T=4, k=2):
        return lib.ft_moe_ffn(C.byref(w), p, act, T, k, p, p, None, p, ydt, p, ws_bytes, None)

    assert call(_w(H=100)) == ft.ERR_INVALID_ARG                 # H not a multiple of 64
    assert call(_w(I=96)) == ft.ERR_INVALID_ARG
    assert call(_w(slot_stride=1000)) == ft.ERR_INVALID_ARG      # too small / unaligned
    assert call(_w(pool=4097)) == ft.ERR_INVALID_ARG             # unaligned pool
    assert call(_w(n_shared=2)) == ft.ERR_INVALID_ARG
    assert call(_w(), act=ft.F32) == ft.ERR_INVALID_ARG          # bf16 weights, fp32 x
    assert call(_w(w_dt=ft.F32, slot_stride=ft.slot_stride("f32", 256, 128)),
                ydt=ft.BF16, act=ft.F32) == ft.ERR_INVALID_ARG
    assert call(_w(), ws_bytes=16) == ft.ERR_INVALID_ARG         # workspace too small
    assert call(_w(), k=9) == ft.ERR_INVALID_ARG
    assert call(_w(), T=0) == ft.OK
    w = _w()
    assert lib.ft_moe_ffn_workspace(C.byref(w), 4, 2) > 4 * 2 * 128 * 2


def test_ffn_refuses_shapes_past_32bit_offsets():
    """The kernels address activation rows with 32-bit element offsets: T*k rows
    of h at I = 2048 reach 2^32 elements at T*k = 2^21, so the boundary refuses
    it (and anything larger) instead of wrapping; just below it is accepted up
    to the workspace check."""
    lib = ft.load()
    p = C.c_void_p(4096)

    def call(w, T, k, ws_bytes=1 << 62):
        return lib.ft_moe_ffn(C.byref(w), p, ft.BF16, T, k, p, p, None, p, ft.BF16, p, ws_bytes, None)

    w = _w(E=256, H=256, I=2048, slot_stride=ft.slot_stride("bf16", 256, 2048))
    assert call(w, T=1 << 18, k=8) == ft.ERR_UNSUPPORTED          # (T*k)*I = 2^32
    assert "32-bit" in ft.last_error()
    # one token fewer passes this check and stops at the next one (a workspace
    # too small), so no kernel is launched
    assert call(w, T=(1 << 18) - 1, k=8, ws_bytes=16) == ft.ERR_INVALID_ARG
    assert "workspace" in ft.last_error()
    # one shared-expert row per token tips it over: (T*k + T)*I >= 2^32
    ws = _w(E=256, H=256, I=2048, n_shared=1, slot_stride=ft.slot_stride("bf16", 256, 2048))
    T = (1 << 32) // (9 * 2048) + 1
    assert call(ws, T=T, k=8) == ft.ERR_UNSUPPORTED
    # T*H at the gate/up input
    wh = _w(E=8, H=1 << 16, I=64, slot_stride=ft.slot_stride("bf16", 1 << 16, 64))
    assert call(wh, T=1 << 16, k=1) == ft.ERR_UNSUPPORTED
    # an expert slot of 2^32 bytes or more
    big = ft.slot_stride("bf16", 1 << 16, 1 << 14)
    assert call(_w(E=8, H=1 << 16, I=1 << 14, slot_stride=big), T=1, k=1) == ft.ERR_UNSUPPORTED


def test_ffn_noalloc_refuses_what_its_scratch_cannot_hold():
    """ft_moe_ffn_noalloc takes its workspace from a 64 MiB static array: a
    call needing more returns FT_ERR_CAPACITY before any device work."""
    lib = ft.load()
    p = C.c_void_p(4096)
    w = _w(E=128, H=2048, I=768, slot_stride=ft.slot_stride("bf16", 2048, 768))
    T = 8192                                   # h alone: 8192 * 8 * 768 * 2 B = 96 MiB
    assert lib.ft_moe_ffn_workspace(C.byref(w), T, 8) > ft.NOALLOC_SCRATCH_BYTES
    assert lib.ft_moe_ffn_noalloc(C.byref(w), p, ft.BF16, T, 8, p, p, None, p, ft.BF16,
                                  None) == ft.ERR_CAPACITY
    assert "static scratch" in ft.last_error()
    assert lib.ft_moe_ffn_noalloc(None, p, ft.BF16, 4, 2, p, p, None, p, ft.BF16,
                                  None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_ffn_noalloc(C.byref(w), p, ft.BF16, 0, 8, p, p, None, p, ft.BF16,
                                  None) == ft.OK          # empty batch: no-op


def test_scatter_rows_rejects_bad_arguments():
    lib = ft.load()
    p = C.c_void_p(4096)
    assert lib.ft_moe_scatter_rows(p, p, 4, 100, p, ft.BF16, None) == ft.ERR_INVALID_ARG  # H % 8
    assert lib.ft_moe_scatter_rows(p, p, 4, 64, p, ft.MXFP4, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_scatter_rows(p, p, -1, 64, p, ft.BF16, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_scatter_rows(None, None, 0, 64, None, ft.BF16, None) == ft.OK  # empty
    assert lib.ft_moe_scatter_rows(C.c_void_p(4100), p, 4, 64, p, ft.BF16, None) == ft.ERR_INVALID_ARG


def test_combine_rejects_bad_arguments():
    lib = ft.load()
    p = C.c_void_p(4096)
    assert lib.ft_moe_combine(p, ft.BF16, p, p, 4, 2, 100, 0, p, ft.BF16, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_combine(p, ft.MXFP4, p, p, 4, 2, 64, 0, p, ft.BF16, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_combine(p, ft.BF16, p, p, 4, 2, 64, 3, p, ft.BF16, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_combine(p, ft.BF16, p, p, 0, 2, 64, 0, p, ft.BF16, None) == ft.OK


def test_slot_cache_rejects_bad_descriptors():
    lib = ft.load()
    h = C.c_void_p()
    d = ft.SlotCacheDesc(0, 8, 1024, 4096, 1024, 4096, 1024, 16, 0)
    assert lib.ft_slot_cache_create(C.byref(d), C.byref(h)) == ft.ERR_INVALID_ARG
    d = ft.SlotCacheDesc(2, 8, 1024, 4096, 512, 4096, 1024, 16, 0)      # host stride too small
    assert lib.ft_slot_cache_create(C.byref(d), C.byref(h)) == ft.ERR_INVALID_ARG
    d = ft.SlotCacheDesc(3, 8, 1024, 4096, 1024, 4096, 1024, 16, 1)     # 16 % 3 per-layer
    assert lib.ft_slot_cache_create(C.byref(d), C.byref(h)) == ft.ERR_INVALID_ARG


def _step(k=2, T=4):
    w = ft.MoeWeights(ft.BF16, 8, 128, 128, 0, 4096, 3 * 128 * 128 * 2, 0)
    p = 4096
    return ft.MoeStep(w, p, ft.BF16, p, None, T, k, None, p, p, p, p, p, p, p, p, 1 << 20, p,
                      ft.BF16, p, 1 << 20, p, ft.BF16)


def test_step_and_graph_reject_bad_arguments():
    lib = ft.load()
    h = C.c_void_p()
    assert lib.ft_moe_step_run(None, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_graph_create(None, None, C.byref(h)) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_graph_launch(None, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_graph_destroy(None) == ft.OK
    # the step's own checks run before anything is enqueued or captured
    bad = _step(k=0)
    assert lib.ft_moe_step_run(C.byref(bad), None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_graph_create(C.byref(bad), None, C.byref(h)) == ft.ERR_INVALID_ARG
    assert not h.value
    assert lib.ft_moe_step_run(C.byref(_step(k=9)), None) == ft.ERR_INVALID_ARG


def test_fused_step_refuses_what_it_cannot_take():
    """The fused step's checks run on the host before any device call: bad
    arguments and shapes past its limits come back without a GPU."""
    lib = ft.load()
    h = C.c_void_p()
    assert lib.ft_moe_step_fused(None, None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_graph_create_fused(None, None, C.byref(h)) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_fused_timeouts(None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_step_fused(C.byref(_step(k=0)), None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_step_fused(C.byref(_step(k=9)), None) == ft.ERR_INVALID_ARG
    assert lib.ft_moe_step_fused(C.byref(_step(T=0)), None) == ft.OK        # nothing enqueued

    def step(w_dt=ft.BF16, act=ft.BF16, E=8, H=128, I=128, n_shared=0, T=4, k=2):
        w = ft.MoeWeights(w_dt, E, H, I, n_shared, 4096,
                          ft.slot_stride({ft.BF16: "bf16", ft.F32: "f32", ft.MXFP4: "mxfp4"}[w_dt], H, I), 0)
        p = 4096
        return ft.MoeStep(w, p, act, p, None, T, k, None, p, p, p, p, p, p, p, p, 1 << 20, p,
                          ft.BF16, p, 1 << 20, p, ft.BF16)

    for bad in (step(T=5), step(w_dt=ft.F32, act=ft.F32), step(w_dt=ft.MXFP4), step(E=600),
                step(H=32768, T=3), step(I=4096, T=4, k=8, E=64),
                step(T=4, k=16, n_shared=1, E=64)):
        assert lib.ft_moe_step_fused(C.byref(bad), None) == ft.ERR_UNSUPPORTED
        assert lib.ft_moe_graph_create_fused(C.byref(bad), None, C.byref(h)) == ft.ERR_UNSUPPORTED
        assert not h.value
    assert "fused step" in ft.last_error()


def test_struct_layouts_match_the_header(tmp_path):
    """ctypes mirrors of the header's structs: same size and field offsets as
    the C compiler gives them."""
    structs = {"ft_moe_weights": ft.MoeWeights, "ft_moe_step": ft.MoeStep,
               "ft_slot_cache_desc": ft.SlotCacheDesc, "ft_map_stats": ft.MapStats,
               "ft_cache_stats": ft.CacheStats, "ft_host_moe_job_desc": ft.HostMoeJobDesc,
               "ft_stack_pass": ft.StackPass, "ft_stack_stats": ft.StackStats}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ftmoe.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f in py._fields_:
            lines.append(f'printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines += ['return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    r = subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    want = []
    for cname, py in structs.items():
        want.append(f"{cname} size {C.sizeof(py)}")
        for f in py._fields_:
            want.append(f"{cname} {f[0]} {getattr(py, f[0]).offset}")
    assert [l for l in got if l] == want


def test_ffn_rejects_a_bad_host_pool():
    """The host tier of ft_moe_weights is checked before any device work:
    256-byte aligned, stride a multiple of 256 covering one expert."""
    lib = ft.load()
    p = C.c_void_p(4096)
    st = ft.slot_stride("bf16", 256, 128)

    def call(w):
        return lib.ft_moe_ffn(C.byref(w), p, ft.BF16, 4, 2, p, p, None, p, ft.BF16, p, 1 << 30, None)

    assert call(_w(host_pool=4096 + 64, host_stride=st)) == ft.ERR_INVALID_ARG   # misaligned
    assert call(_w(host_pool=8192, host_stride=st + 16)) == ft.ERR_INVALID_ARG   # stride % 256
    assert call(_w(host_pool=8192, host_stride=256)) == ft.ERR_INVALID_ARG       # below one expert
    assert "host_pool" in ft.last_error()
    assert lib.ft_host_device_pointer(None, C.byref(C.c_void_p())) == ft.ERR_INVALID_ARG
    assert lib.ft_host_device_pointer(p, None) == ft.ERR_INVALID_ARG


def test_stack_forward_rejects_bad_arguments():
    lib = ft.load()
    # unknown flags are refused before the cache is looked at
    bad = ft.StackPass(0, None, None, None, 0, 2)
    assert lib.ft_slot_stack_forward(C.c_void_p(4096), C.byref(bad), None, None, None) == ft.ERR_INVALID_ARG
    assert "flags" in ft.last_error()
    p = ft.StackPass(0, None, None, None, 0)
    assert lib.ft_slot_stack_forward(None, C.byref(p), None, None, None) == ft.ERR_INVALID_ARG
    assert lib.ft_slot_stack_forward(C.c_void_p(4096), None, None, None, None) == ft.ERR_INVALID_ARG
    assert lib.ft_slot_stack_forward(C.c_void_p(4096), C.byref(p), None, None, None) == ft.ERR_INVALID_ARG


def test_slot_cache_resize_rejects_bad_arguments():
    lib = ft.load()
    assert lib.ft_slot_cache_resize(None, 8, None, None) == ft.ERR_INVALID_ARG
