"""Thin ctypes binding of libftmoe.so (the C ABI in include/ftmoe.h).

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and a non-OK status raises FtError with
the library's message.  Every step of the MoE layer runs in the library's HIP
kernels; nothing here computes.  The library must have been built
(``python -m expert_ffn_execution_amd.build``); loading fails loudly if not.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libftmoe.so")

F32, BF16, MXFP4, FP8, NVFP4 = 0, 1, 2, 3, 4
DT = {"f32": F32, "bf16": BF16, "mxfp4": MXFP4, "fp8": FP8, "nvfp4": NVFP4}
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_NOT_PINNED, ERR_BUSY, ERR_HIP = range(7)
WARN_OVERLAP_DISABLED = 100
SCOPE_GLOBAL, SCOPE_PER_LAYER = 0, 1
PROF_GEMM1, PROF_GEMM2, PROF_FFN, PROF_ROUTE, PROF_ALIGN, PROF_COMBINE = range(6)

# symbols declared in include/ftmoe.h
EXPORTS = [
    "ft_last_error", "ft_version", "ft_moe_route", "ft_moe_align_workspace", "ft_moe_align",
    "ft_expert_layout", "ft_moe_ffn_workspace", "ft_moe_ffn", "ft_moe_ffn_set_path",
    "ft_set_profile_events", "ft_moe_combine", "ft_slot_cache_create", "ft_slot_cache_destroy",
    "ft_slot_cache_map", "ft_slot_cache_release", "ft_slot_cache_prefetch", "ft_slot_cache_evict",
    "ft_slot_cache_stats", "ft_slot_cache_lookup", "ft_slot_cache_resize", "ft_moe_step_run",
    "ft_moe_graph_create", "ft_moe_graph_launch", "ft_moe_graph_destroy", "ft_host_expert_ffn",
    "ft_host_moe_ffn_submit", "ft_host_job_wait", "ft_moe_ffn_noalloc", "ft_split_misses",
    "ft_moe_scatter_rows", "ft_slot_stack_forward", "ft_host_device_pointer", "ft_moe_step_fused",
    "ft_moe_graph_create_fused", "ft_moe_fused_timeouts",
]
STACK_DEVICE_TABLE = 1   # FT_STACK_DEVICE_TABLE
NOALLOC_SCRATCH_BYTES = 64 << 20   # FT_NOALLOC_SCRATCH_BYTES


class FtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ftmoe status {status}: {msg}")
        self.status = status


class MoeWeights(C.Structure):
    _fields_ = [("w_dt", C.c_int), ("E", C.c_int), ("H", C.c_int), ("I", C.c_int),
                ("n_shared", C.c_int), ("pool", C.c_void_p), ("slot_stride", C.c_size_t),
                ("shared_slot", C.c_int), ("host_pool", C.c_void_p), ("host_stride", C.c_size_t)]


class MoeStep(C.Structure):
    _fields_ = [("weights", MoeWeights), ("x", C.c_void_p), ("act_dt", C.c_int),
                ("w_router", C.c_void_p), ("bias", C.c_void_p), ("T", C.c_int), ("k", C.c_int),
                ("slot_of_expert", C.c_void_p), ("logits", C.c_void_p), ("topk_ids", C.c_void_p),
                ("topk_w", C.c_void_p), ("counts", C.c_void_p), ("offsets", C.c_void_p),
                ("perm", C.c_void_p), ("inv_perm", C.c_void_p), ("align_ws", C.c_void_p),
                ("align_ws_bytes", C.c_size_t), ("y_perm", C.c_void_p), ("y_dt", C.c_int),
                ("ffn_ws", C.c_void_p), ("ffn_ws_bytes", C.c_size_t), ("out", C.c_void_p),
                ("out_dt", C.c_int)]


class SlotCacheDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("n_experts", C.c_int), ("expert_bytes", C.c_size_t),
                ("host_pool", C.c_void_p), ("host_stride", C.c_size_t),
                ("dev_slots", C.c_void_p), ("slot_stride", C.c_size_t), ("n_slots", C.c_int),
                ("scope", C.c_int)]


class StackPass(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("layers", C.c_void_p), ("logits_in", C.c_void_p),
                ("counts_host", C.c_void_p), ("prefill", C.c_int), ("flags", C.c_int)]


class StackStats(C.Structure):
    _fields_ = [("demand", C.c_longlong), ("hits", C.c_longlong), ("prefetch_hits", C.c_longlong),
                ("misses", C.c_longlong), ("bytes_h2d", C.c_longlong), ("prefetch_warnings", C.c_int)]


class MapStats(C.Structure):
    _fields_ = [("n_demand", C.c_int), ("n_hit", C.c_int), ("n_prefetch_hit", C.c_int),
                ("n_miss", C.c_int), ("bytes_h2d", C.c_size_t)]


class CacheStats(C.Structure):
    _fields_ = [("maps", C.c_longlong), ("demand", C.c_longlong), ("hits", C.c_longlong),
                ("prefetch_hits", C.c_longlong), ("misses", C.c_longlong),
                ("prefetch_issued", C.c_longlong), ("evictions", C.c_longlong),
                ("bytes_h2d", C.c_longlong), ("resident", C.c_int), ("held", C.c_int),
                ("in_flight", C.c_int), ("n_slots", C.c_int)]


class HostMoeJobDesc(C.Structure):
    _fields_ = [("w_dt", C.c_int), ("E", C.c_int), ("H", C.c_int), ("I", C.c_int), ("k", C.c_int),
                ("pool", C.c_void_p), ("slot_stride", C.c_size_t), ("experts", C.c_void_p),
                ("n_experts", C.c_int), ("offsets", C.c_void_p), ("perm", C.c_void_p),
                ("x", C.c_void_p), ("x_dt", C.c_int), ("T", C.c_int), ("rows", C.c_void_p),
                ("pos", C.c_void_p), ("max_rows", C.c_int), ("n_threads", C.c_int)]


_lib = None


def load() -> C.CDLL:
    """Load libftmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m expert_ffn_execution_amd.build` (there is no fallback)")
    lib = C.CDLL(LIB_PATH)
    P, I32, SZ = C.c_void_p, C.c_int, C.c_size_t
    lib.ft_last_error.restype = C.c_char_p
    lib.ft_version.restype = C.c_char_p
    sig = {
        "ft_moe_route": [P, I32, P, P, P, I32, I32, I32, I32, P, P, P, P],
        "ft_moe_align_workspace": [I32, I32, I32],
        "ft_moe_align": [P, I32, I32, I32, P, P, P, P, P, SZ, P],
        "ft_expert_layout": [I32, I32, I32, P],
        "ft_moe_ffn_workspace": [C.POINTER(MoeWeights), I32, I32],
        "ft_moe_ffn": [C.POINTER(MoeWeights), P, I32, I32, I32, P, P, P, P, I32, P, SZ, P],
        "ft_moe_ffn_noalloc": [C.POINTER(MoeWeights), P, I32, I32, I32, P, P, P, P, I32, P],
        "ft_moe_scatter_rows": [P, P, I32, I32, P, I32, P],
        "ft_slot_stack_forward": [P, C.POINTER(StackPass), P, P, C.POINTER(StackStats)],
        "ft_moe_ffn_set_path": [I32],
        "ft_set_profile_events": [I32, P, P],
        "ft_moe_combine": [P, I32, P, P, I32, I32, I32, I32, P, I32, P],
        "ft_slot_cache_create": [C.POINTER(SlotCacheDesc), C.POINTER(P)],
        "ft_slot_cache_destroy": [P],
        "ft_slot_cache_map": [P, I32, P, I32, P, P, P, C.POINTER(MapStats)],
        "ft_slot_cache_release": [P, I32, P],
        "ft_slot_cache_prefetch": [P, I32, P, I32, P, C.POINTER(C.c_int)],
        "ft_slot_cache_evict": [P, I32, I32],
        "ft_slot_cache_stats": [P, C.POINTER(CacheStats)],
        "ft_slot_cache_lookup": [P, I32, I32],
        "ft_host_expert_ffn": [I32, I32, I32, P, P, I32, I32, P, I32],
        "ft_host_moe_ffn_submit": [C.POINTER(HostMoeJobDesc), C.POINTER(P), C.POINTER(C.c_int)],
        "ft_host_job_wait": [P],
        "ft_slot_cache_resize": [P, I32, P, P],
        "ft_moe_step_run": [C.POINTER(MoeStep), P],
        "ft_moe_graph_create": [C.POINTER(MoeStep), P, C.POINTER(P)],
        "ft_moe_graph_launch": [P, P],
        "ft_moe_graph_destroy": [P],
        "ft_host_device_pointer": [P, C.POINTER(P)],
        "ft_moe_step_fused": [C.POINTER(MoeStep), P],
        "ft_moe_graph_create_fused": [C.POINTER(MoeStep), P, C.POINTER(P)],
        "ft_moe_fused_timeouts": [C.POINTER(C.c_int)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int
    lib.ft_split_misses.argtypes = [I32, C.c_double, C.c_double]
    lib.ft_split_misses.restype = C.c_int
    lib.ft_moe_align_workspace.restype = C.c_size_t
    lib.ft_expert_layout.restype = C.c_size_t
    lib.ft_moe_ffn_workspace.restype = C.c_size_t
    _lib = lib
    return lib


def last_error() -> str:
    return load().ft_last_error().decode()


def _check(st: int, allow=(OK,)) -> int:
    if st not in allow:
        raise FtError(st, last_error())
    return st


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    return F32 if t.dtype == torch.float32 else BF16


def _dev(*ts):
    for t in ts:
        if t is not None:
            assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA tensors"


# ---------------------------------------------------------------------------
# layer steps
# ---------------------------------------------------------------------------
def route(T: int, E: int, k: int, *, logits: Optional[torch.Tensor] = None,
          x: Optional[torch.Tensor] = None, w_router: Optional[torch.Tensor] = None,
          bias: Optional[torch.Tensor] = None, logits_out: Optional[torch.Tensor] = None,
          ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None, stream=None):
    """ft_moe_route.  Returns (ids [T,k] int32, w [T,k] fp32, logits_out or None)."""
    dev = (logits if logits is not None else x).device
    ids = ids if ids is not None else torch.empty((T, k), dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty((T, k), dtype=torch.float32, device=dev)
    H = 0
    xdt = BF16
    if logits is None:
        H = x.shape[1]
        xdt = _dt(x)
        if logits_out is None:
            logits_out = torch.empty((T, E), dtype=torch.float32, device=dev)
    _dev(logits, x, w_router, bias, logits_out, ids, w)
    _check(load().ft_moe_route(_p(x), xdt, _p(w_router), _p(logits), _p(bias), T, H, E, k,
                               _p(logits_out), _p(ids), _p(w), _stream(stream)))
    return ids, w, logits_out


def align_workspace(T: int, k: int, E: int) -> int:
    return load().ft_moe_align_workspace(T, k, E)


def align(ids: torch.Tensor, E: int, ws: Optional[torch.Tensor] = None, out=None, stream=None):
    """ft_moe_align.  Returns (counts [E], offsets [E+1], perm [T*k], inv_perm [T*k])."""
    T, k = ids.shape
    dev = ids.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev))
    counts, offsets, perm, inv = out
    need = align_workspace(T, k, E)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(ids, counts, offsets, perm, inv)
    _check(load().ft_moe_align(_p(ids), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv),
                               _p(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return counts, offsets, perm, inv


def expert_layout(wdtype: str, H: int, I: int):
    """(slot bytes, [offsets of gate, up, down, gate_sc, up_sc, down_sc])."""
    offs = (C.c_size_t * 6)()
    n = load().ft_expert_layout(DT[wdtype], H, I, offs)
    if n == 0:
        raise FtError(ERR_INVALID_ARG, f"unsupported layout {wdtype} H={H} I={I}")
    return n, list(offs)


def slot_stride(wdtype: str, H: int, I: int) -> int:
    n, _ = expert_layout(wdtype, H, I)
    return (n + 255) // 256 * 256


def pack_expert(ex: dict, wdtype: str, H: int, I: int, out: torch.Tensor):
    """Write one expert's logical tensors into a slot (uint8 view of slot_stride bytes)."""
    n, offs = expert_layout(wdtype, H, I)
    names = ["gate", "up", "down"] + (["gate_sc", "up_sc", "down_sc"]
                                      if wdtype in ("mxfp4", "fp8", "nvfp4") else [])
    offs = list(offs)
    if wdtype == "nvfp4":  # the fp32 tensor scales follow the down block scales
        names += ["gate_ts", "up_ts", "down_ts"]
        offs += [offs[5] + H * I // 16 + 4 * m for m in range(3)]
    for name, off in zip(names, offs):
        t = ex[name].contiguous()
        b = t.view(torch.uint8).reshape(-1)
        out[off:off + b.numel()].copy_(b)


def host_device_pointer(t: torch.Tensor) -> int:
    """ft_host_device_pointer: the device-visible address of a pinned host tensor."""
    if t.is_cuda or not t.is_pinned():
        raise FtError(ERR_INVALID_ARG, "host_device_pointer needs a pinned host tensor")
    out = C.c_void_p()
    _check(load().ft_host_device_pointer(C.c_void_p(t.data_ptr()), C.byref(out)))
    return out.value


def make_weights(wdtype: str, E: int, H: int, I: int, pool: torch.Tensor, n_shared: int = 0,
                 shared_slot: int = 0, host_pool: Optional[torch.Tensor] = None) -> MoeWeights:
    """Describe a device slot array pool [n_slots, slot_stride] (uint8), and
    optionally a pinned host array host_pool [n, stride] (uint8) whose expert
    j a slot-table entry -2 - j reads over the host link."""
    _dev(pool)
    hp, hs = None, 0
    if host_pool is not None:
        hp, hs = host_device_pointer(host_pool), host_pool.shape[-1]
    return MoeWeights(DT[wdtype], E, H, I, n_shared, pool.data_ptr(), pool.shape[1], shared_slot,
                      hp, hs)


def ffn_workspace(wts: MoeWeights, T: int, k: int) -> int:
    return load().ft_moe_ffn_workspace(C.byref(wts), T, k)


def set_ffn_path(path: int) -> int:
    return load().ft_moe_ffn_set_path(path)


def ffn(wts: MoeWeights, x: torch.Tensor, k: int, perm: torch.Tensor, offsets: torch.Tensor,
        slot_of_expert: Optional[torch.Tensor] = None, y_dtype=torch.bfloat16,
        y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """ft_moe_ffn.  Returns y_perm [T*k + n_shared*T, H]."""
    T = x.shape[0]
    dev = x.device
    rows = T * k + wts.n_shared * T
    if y is None:
        y = torch.empty((rows, wts.H), dtype=y_dtype, device=dev)
    if ws is None:
        ws = torch.empty(ffn_workspace(wts, T, k), dtype=torch.uint8, device=dev)
    _dev(x, perm, offsets, slot_of_expert, y, ws)
    _check(load().ft_moe_ffn(C.byref(wts), _p(x), _dt(x), T, k, _p(perm), _p(offsets),
                             _p(slot_of_expert), _p(y), _dt(y), _p(ws), ws.numel(),
                             _stream(stream)))
    return y


def ffn_noalloc(wts: MoeWeights, x: torch.Tensor, k: int, perm: torch.Tensor,
                offsets: torch.Tensor, slot_of_expert: Optional[torch.Tensor] = None,
                y_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None, stream=None):
    """ft_moe_ffn_noalloc (workspace in the library's static scratch array).
    Returns y_perm [T*k + n_shared*T, H]; y is allocated here unless given."""
    T = x.shape[0]
    rows = T * k + wts.n_shared * T
    if y is None:
        y = torch.empty((rows, wts.H), dtype=y_dtype, device=x.device)
    _dev(x, perm, offsets, slot_of_expert, y)
    _check(load().ft_moe_ffn_noalloc(C.byref(wts), _p(x), _dt(x), T, k, _p(perm), _p(offsets),
                                     _p(slot_of_expert), _p(y), _dt(y), _stream(stream)))
    return y


def host_expert_ffn(slot: torch.Tensor, x: torch.Tensor, H: int, I: int, n_threads: int = 8,
                    y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ft_host_expert_ffn: one bf16 expert's FFN on host cores.  slot: host
    uint8 view of the expert's slot; x [T, H] bf16 host.  Returns y [T, H] fp32."""
    if slot.is_cuda or x.is_cuda:
        raise FtError(ERR_INVALID_ARG, "host_expert_ffn takes host tensors")
    x = x.contiguous()
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32)
    if (y.is_cuda or y.dtype != torch.float32 or tuple(y.shape) != (T, H)
            or not y.is_contiguous()):
        raise FtError(ERR_INVALID_ARG, "y must be a contiguous host fp32 tensor [T, H]")
    _check(load().ft_host_expert_ffn(BF16, H, I, slot.data_ptr(), x.data_ptr(), BF16, T,
                                     y.data_ptr(), n_threads))
    return y


class HostJob:
    """A queued ft_host_moe_ffn_submit job: holds the buffers it reads and
    writes until wait()."""

    def __init__(self, handle, n_rows: int, keep):
        self.handle, self.n_rows, self._keep = handle, n_rows, keep

    def wait(self):
        """ft_host_job_wait; idempotent on the Python side."""
        if self.handle is not None:
            h, self.handle = self.handle, None
            _check(load().ft_host_job_wait(h))
        return self.n_rows


def host_moe_ffn_submit(pool: torch.Tensor, E: int, H: int, I: int, k: int,
                        experts: Sequence[int], offsets: torch.Tensor, perm: torch.Tensor,
                        x: torch.Tensor, rows: torch.Tensor, pos: torch.Tensor,
                        n_threads: int = 8) -> HostJob:
    """ft_host_moe_ffn_submit: the host FFN of `experts` on their rows of one
    layer, queued on the library's host threads.  pool [E(+shared)][stride]
    uint8 host (one layer's slots); offsets [E+1] / perm [T*k] int32 host as
    ft_moe_align wrote them; x [T, H] bf16 host; rows [max_rows, H] fp32 and
    pos [max_rows] int64 host outputs.  Returns the job (its n_rows is known
    at once); call .wait() before reading rows / pos."""
    for t in (pool, offsets, perm, x, rows, pos):
        if t.is_cuda or not t.is_contiguous():
            raise FtError(ERR_INVALID_ARG, "host_moe_ffn_submit takes contiguous host tensors")
    if (offsets.dtype != torch.int32 or perm.dtype != torch.int32 or x.dtype != torch.bfloat16
            or rows.dtype != torch.float32 or pos.dtype != torch.int64 or rows.dim() != 2
            or rows.shape[1] != H or pos.shape[0] < rows.shape[0]):
        raise FtError(ERR_INVALID_ARG, "host_moe_ffn_submit: tensor dtypes / shapes")
    ex = (C.c_int32 * len(experts))(*experts)
    d = HostMoeJobDesc(BF16, E, H, I, k, pool.data_ptr(), pool.stride(0) * pool.element_size(),
                       C.cast(ex, C.c_void_p), len(experts), offsets.data_ptr(), perm.data_ptr(),
                       x.data_ptr(), BF16, x.shape[0], rows.data_ptr(), pos.data_ptr(),
                       rows.shape[0], n_threads)
    h = C.c_void_p()
    n = C.c_int()
    _check(load().ft_host_moe_ffn_submit(C.byref(d), C.byref(h), C.byref(n)))
    return HostJob(h, n.value, (pool, offsets, perm, x, rows, pos))


def split_misses(m: int, bp: float, bh: float) -> int:
    """ft_split_misses: how many of m missed experts to copy to the GPU (the
    rest run on host cores), from the measured Bp and Bh in GB/s."""
    return load().ft_split_misses(int(m), float(bp), float(bh))


def scatter_rows(rows: torch.Tensor, pos: torch.Tensor, y_perm: torch.Tensor, n: Optional[int] = None,
                 stream=None) -> torch.Tensor:
    """ft_moe_scatter_rows: y_perm[pos[i]] = rows[i] (rounded to y_perm's dtype)
    for the first n rows (all by default); rows [>=n, H] fp32, pos [>=n] int64,
    both on y_perm's device."""
    n = rows.shape[0] if n is None else n
    H = y_perm.shape[1]
    if (rows.dtype != torch.float32 or pos.dtype != torch.int64 or rows.shape[1] != H
            or not rows.is_contiguous() or not pos.is_contiguous() or not y_perm.is_contiguous()):
        raise FtError(ERR_INVALID_ARG, "scatter_rows: rows fp32 [n, H], pos int64 [n], contiguous")
    _dev(rows, pos, y_perm)
    _check(load().ft_moe_scatter_rows(_p(rows), _p(pos), n, H, _p(y_perm), _dt(y_perm),
                                      _stream(stream)))
    return y_perm


def combine(y_perm: torch.Tensor, inv_perm: torch.Tensor, w: torch.Tensor, n_shared: int = 0,
            out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None, stream=None):
    """ft_moe_combine.  Returns out [T, H]."""
    T, k = w.shape
    H = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y_perm.device)
    _dev(y_perm, inv_perm, w, out)
    _check(load().ft_moe_combine(_p(y_perm), _dt(y_perm), _p(inv_perm), _p(w), T, k, H,
                                 n_shared, _p(out), _dt(out), _stream(stream)))
    return out


class LayerStep:
    """The buffers of one whole MoE-layer step and its ft_moe_step descriptor.

    x, w_router, bias and slot_of_expert are the caller's tensors (refill x in
    place between runs); everything else is allocated here, once.
    """

    def __init__(self, wts: MoeWeights, x: torch.Tensor, k: int, w_router: torch.Tensor,
                 bias: Optional[torch.Tensor] = None,
                 slot_of_expert: Optional[torch.Tensor] = None, y_dtype=torch.bfloat16,
                 out_dtype=torch.bfloat16):
        T, H = x.shape
        E = wts.E
        dev = x.device
        _dev(x, w_router, bias, slot_of_expert)
        i32, f32 = torch.int32, torch.float32
        self.x, self.w_router, self.bias, self.slot_of_expert = x, w_router, bias, slot_of_expert
        self.logits = torch.empty((T, E), dtype=f32, device=dev)
        self.ids = torch.empty((T, k), dtype=i32, device=dev)
        self.w = torch.empty((T, k), dtype=f32, device=dev)
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.perm = torch.empty(max(1, T * k), dtype=i32, device=dev)
        self.inv = torch.empty(max(1, T * k), dtype=i32, device=dev)
        self.aws = torch.empty(max(1, align_workspace(T, k, E)), dtype=torch.uint8, device=dev)
        self.y = torch.empty((T * k + wts.n_shared * T, H), dtype=y_dtype, device=dev)
        self.fws = torch.empty(max(256, ffn_workspace(wts, T, k)), dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, H), dtype=out_dtype, device=dev)
        self.desc = MoeStep(wts, x.data_ptr(), _dt(x), w_router.data_ptr(),
                            None if bias is None else bias.data_ptr(), T, k,
                            None if slot_of_expert is None else slot_of_expert.data_ptr(),
                            self.logits.data_ptr(), self.ids.data_ptr(), self.w.data_ptr(),
                            self.counts.data_ptr(), self.offsets.data_ptr(), self.perm.data_ptr(),
                            self.inv.data_ptr(), self.aws.data_ptr(), self.aws.numel(),
                            self.y.data_ptr(), _dt(self.y), self.fws.data_ptr(),
                            self.fws.numel(), self.out.data_ptr(), _dt(self.out))

    def run(self, stream=None) -> torch.Tensor:
        """ft_moe_step_run: route -> align -> ffn -> combine; returns out."""
        _check(load().ft_moe_step_run(C.byref(self.desc), _stream(stream)))
        return self.out

    def capture(self, stream=None) -> "Graph":
        """ft_moe_graph_create (runs the step once, then captures it)."""
        return Graph(self, stream)

    def run_fused(self, stream=None) -> torch.Tensor:
        """ft_moe_step_fused: the step as one kernel; writes logits, ids, w and out."""
        _check(load().ft_moe_step_fused(C.byref(self.desc), _stream(stream)))
        return self.out

    def capture_fused(self, stream=None) -> "Graph":
        """ft_moe_graph_create_fused (one fused step, then its one-node graph)."""
        return Graph(self, stream, fused=True)


class Graph:
    """A captured LayerStep (ft_moe_graph_*); keeps the step's buffers alive."""

    def __init__(self, step: LayerStep, stream=None, fused: bool = False):
        self.step = step
        h = C.c_void_p()
        create = load().ft_moe_graph_create_fused if fused else load().ft_moe_graph_create
        _check(create(C.byref(step.desc), _stream(stream), C.byref(h)))
        self.h = h

    def launch(self, stream=None) -> torch.Tensor:
        _check(load().ft_moe_graph_launch(self.h, _stream(stream)))
        return self.step.out

    def close(self):
        if self.h:
            _check(load().ft_moe_graph_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fused_timeouts() -> int:
    """ft_moe_fused_timeouts: fused-step waits that gave up since the last call."""
    n = C.c_int(0)
    _check(load().ft_moe_fused_timeouts(C.byref(n)))
    return n.value


def set_profile_events(which: int, start, stop):
    """start/stop: hipEvent_t handles (int or c_void_p, see HipEvents) or None."""
    _check(load().ft_set_profile_events(which, start, stop))


class HipEvents:
    """hipEvent_t handles from the HIP runtime the process already uses (for
    ft_set_profile_events, which records them inside the library)."""

    def __init__(self):
        self.rt = C.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [C.c_void_p]
        self.made = []

    def create(self) -> C.c_void_p:
        e = C.c_void_p()
        rc = self.rt.hipEventCreate(C.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.made.append(e)
        return e

    def elapsed_ms(self, a, b) -> float:
        self.rt.hipEventSynchronize(b)
        f = C.c_float()
        rc = self.rt.hipEventElapsedTime(C.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def close(self):
        for e in self.made:
            self.rt.hipEventDestroy(e)
        self.made = []


# ---------------------------------------------------------------------------
# slot cache
# ---------------------------------------------------------------------------
class SlotCache:
    """ft_slot_cache_* over a pinned host pool and a device slot array."""

    def __init__(self, n_layers: int, n_experts: int, expert_bytes: int,
                 host_pool: torch.Tensor, dev_slots: torch.Tensor, scope: int = SCOPE_GLOBAL):
        self.desc = SlotCacheDesc(n_layers, n_experts, expert_bytes, host_pool.data_ptr(),
                                  host_pool.shape[-1], dev_slots.data_ptr(), dev_slots.shape[1],
                                  dev_slots.shape[0], scope)
        self._keep = (host_pool, dev_slots)
        h = C.c_void_p()
        _check(load().ft_slot_cache_create(C.byref(self.desc), C.byref(h)))
        self.h = h
        self.n_experts = n_experts

    def close(self):
        if self.h:
            load().ft_slot_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _list(experts: Sequence[int]):
        arr = (C.c_int32 * max(1, len(experts)))(*experts)
        return arr, len(experts)

    def map(self, layer: int, experts: Sequence[int], slot_table: torch.Tensor, compute=None,
            copy=None) -> MapStats:
        arr, n = self._list(experts)
        st = MapStats()
        _check(load().ft_slot_cache_map(self.h, layer, arr, n, _p(slot_table), _stream(compute),
                                        _stream(copy), C.byref(st)))
        return st

    def release(self, layer: int, compute=None):
        _check(load().ft_slot_cache_release(self.h, layer, _stream(compute)))

    def prefetch(self, layer: int, experts: Sequence[int], copy=None):
        arr, n = self._list(experts)
        got = C.c_int(0)
        st = _check(load().ft_slot_cache_prefetch(self.h, layer, arr, n, _stream(copy),
                                                  C.byref(got)),
                    allow=(OK, WARN_OVERLAP_DISABLED))
        return st, got.value

    def forward_stack(self, steps, n_layers: int, counts_host: Optional[torch.Tensor], logits_in=None,
                      prefill: bool = False, compute=None, copy=None,
                      device_table: bool = False) -> StackStats:
        """ft_slot_stack_forward over n_layers: steps is a ctypes array of
        MoeStep (one per layer, with its buffers), counts_host a pinned int32
        host tensor [n_layers, E] (unused by device-table decode passes),
        logits_in None or a ctypes array of n_layers device pointers (None
        entries: router GEMM).  device_table: FT_STACK_DEVICE_TABLE (with
        n_layers == 0: flush the pending passes)."""
        if counts_host is not None and (counts_host.is_cuda or not counts_host.is_pinned()
                                        or counts_host.dtype != torch.int32):
            raise FtError(ERR_INVALID_ARG, "counts_host must be pinned host int32")
        p = StackPass(n_layers, None if steps is None else C.cast(steps, C.c_void_p),
                      None if logits_in is None else C.cast(logits_in, C.c_void_p),
                      None if counts_host is None else counts_host.data_ptr(), int(prefill),
                      STACK_DEVICE_TABLE if device_table else 0)
        st = StackStats()
        _check(load().ft_slot_stack_forward(self.h, C.byref(p), _stream(compute), _stream(copy),
                                            C.byref(st)))
        return st

    def evict(self, layer: int, expert: int = -1):
        _check(load().ft_slot_cache_evict(self.h, layer, expert))

    def resize(self, n_slots: int, dev_slots: Optional[torch.Tensor] = None, copy=None):
        """ft_slot_cache_resize; dev_slots (a new [n_slots, slot_stride] array) is
        kept alive here in place of the old one."""
        _check(load().ft_slot_cache_resize(self.h, n_slots, _p(dev_slots), _stream(copy)))
        if dev_slots is not None:
            self._keep = (self._keep[0], dev_slots)

    def stats(self) -> CacheStats:
        s = CacheStats()
        _check(load().ft_slot_cache_stats(self.h, C.byref(s)))
        return s

    def lookup(self, layer: int, expert: int) -> int:
        return load().ft_slot_cache_lookup(self.h, layer, expert)
