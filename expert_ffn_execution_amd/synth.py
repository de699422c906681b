"""Seeded synthetic inputs for the MoE-layer FFN workloads.

This module is the one place where inputs are made; both the HIP path's tests
and benchmark and the CPU oracle's tests draw from it.  It holds no step of the
MoE layer itself (no routing, no expert FFN, no combine): only random draws,
rounding of the draws to the storage format (bf16 round-to-nearest-even, and
the MXFP4 quantiser that turns fp32 draws into e2m1 codes with e8m0 block
scales), and the workload shapes.

The pages describe an engine for MoE models whose experts are streamed through
an LRU slot cache (FreeToken hub article, two-level expert memory hierarchy;
chenxutan.com article, "瓶颈为什么是带宽而不是容量").  They print no data,
so every tensor here is synthetic: activations N(0,1), router weight
N(0, 0.02), expert weights N(0, 1/sqrt(fan_in)) (sigma is the standard
deviation; fan_in is H for gate/up and I for down).

Random draws use ``torch.Generator`` seeded per (workload, layer, tensor,
expert, step), so any single expert can be regenerated on its own.  Draws on
the CPU and on a GPU give different numbers for the same seed; a test always
generates a tensor once, on one device, and hands the same bytes to both the
oracle and the HIP path.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

# tensor ids used in seeds
_T_X, _T_ROUTER, _T_BIAS, _T_GATE, _T_UP, _T_DOWN, _T_LOGITS = range(7)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape and storage formats of one MoE layer."""
    name: str
    H: int              # hidden size
    E: int              # routed experts
    k: int              # experts per token
    I: int              # expert intermediate size
    n_shared: int = 0   # always-on shared experts (0 or 1)
    wdtype: str = "bf16"    # expert weight storage: "f32" | "bf16" | "mxfp4" | "fp8" | "nvfp4"
    adtype: str = "bf16"    # activation / router storage: "f32" | "bf16"
    bias: str = "none"      # router logit bias: "none" | "zipf" | "normal"
    bias_param: float = 0.0  # zipf exponent s, or normal std
    router_std: float = 0.02

    @property
    def cfg_id(self) -> int:
        return int(hashlib.sha256(self.name.encode()).hexdigest()[:8], 16)


# The five workloads.  Shapes follow the model families the pages name
# (a 35B-A3B model, a 284B-A13B model with 6 routed experts, a 753B-A40B model:
# freelamp.com article section 1.3; chenxutan.com article, "官方口径").
TINY_F32 = LayerShape("tiny_f32", H=256, E=8, k=2, I=512, wdtype="f32", adtype="f32")
A3B_BF16 = LayerShape("35b_a3b_bf16", H=2048, E=128, k=8, I=768)
A13B_MXFP4 = LayerShape("284b_a13b_mxfp4", H=4096, E=256, k=6, I=2048, n_shared=1,
                        wdtype="mxfp4")
SLOT_STACK = LayerShape("slot_stack_bf16", H=2048, E=128, k=8, I=768, bias="zipf",
                        bias_param=1.1)
A40B_BF16 = LayerShape("753b_a40b_bf16", H=6144, E=256, k=8, I=2048, bias="normal",
                       bias_param=1.0)
A40B_MXFP4 = LayerShape("753b_a40b_mxfp4", H=6144, E=256, k=8, I=2048, wdtype="mxfp4",
                        bias="normal", bias_param=1.0)

# The 35B-A3B layer with FP8 (e4m3) weights: a weight format the pages list,
# on the shape of the bf16 configuration (not one of the five configurations).
A3B_FP8 = LayerShape("35b_a3b_fp8", H=2048, E=128, k=8, I=768, wdtype="fp8")
# ... and with NVFP4 weights (e2m1 codes, an e4m3 scale per 16, an fp32 scale
# per matrix), another format the pages list.
A3B_NVFP4 = LayerShape("35b_a3b_nvfp4", H=2048, E=128, k=8, I=768, wdtype="nvfp4")

SHAPES = {s.name: s for s in (TINY_F32, A3B_BF16, A13B_MXFP4, SLOT_STACK, A40B_BF16,
                              A40B_MXFP4, A3B_FP8, A3B_NVFP4)}

# Token counts each workload is run at (decode points, then prefill).
POINTS = {
    "tiny_f32": [64],
    "35b_a3b_bf16": [1, 16, 64, 4096],
    "284b_a13b_mxfp4": [1, 8, 64, 8192],
    "slot_stack_bf16": [1, 2048],
    "753b_a40b_bf16": [1, 32, 16384],
    "753b_a40b_mxfp4": [1, 32, 16384],
    "35b_a3b_fp8": [1, 16, 64, 4096],
    "35b_a3b_nvfp4": [1, 16, 64, 4096],
}
SLOT_STACK_LAYERS = 8
SLOT_STACK_SLOTS_PER_LAYER = 64
SLOT_STACK_DECODE_STEPS = 256


def seed_of(shape: LayerShape, tensor: int, layer: int = 0, expert: int = 0,
            step: int = 0, extra: int = 0) -> int:
    h = hashlib.sha256(f"{shape.cfg_id}/{tensor}/{layer}/{expert}/{step}/{extra}".encode())
    return int(h.hexdigest()[:15], 16)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std: float, seed: int, device) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def to_storage(t: torch.Tensor, dtype: str) -> torch.Tensor:
    """fp32 draw -> storage dtype (bf16 by round-to-nearest-even)."""
    if dtype == "f32":
        return t.contiguous()
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# MXFP4 quantiser (input recipe).  OCP Microscaling Formats v1.0: blocks of 32
# values along the contraction dim share an e8m0 scale 2^(X-127); elements are
# e2m1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).  Shared exponent
# floor(log2(amax)) - 2 (2 = largest e2m1 exponent), round-to-nearest-even on
# the e2m1 grid, saturating at 6; an all-zero block gets X = 127.  Codes: bit 3
# sign, bits 2..1 exponent, bit 0 mantissa; element 2j in the low nibble of
# byte j, 2j+1 in the high nibble.
# ---------------------------------------------------------------------------
def quantize_mxfp4(w: torch.Tensor):
    """w [N, K] fp32, K % 32 == 0 -> (codes uint8 [N, K/2], scales uint8 [N, K/32])."""
    N, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(N, K // 32, 32)
    amax = blk.abs().amax(dim=2)
    _, e = torch.frexp(amax)                        # amax = m * 2^e, m in [0.5, 1)
    shared = (e.to(torch.int32) - 1) - 2             # floor(log2 amax) - emax(e2m1)
    shared = torch.where(amax > 0, shared, torch.zeros_like(shared))
    X = (shared + 127).clamp(0, 254)
    shared = X - 127
    a = torch.ldexp(blk.abs(), (-shared).unsqueeze(2).to(blk.dtype))
    # RNE onto {0,.5,1,1.5,2,3,4,6}: a tie goes to the code with even mantissa bit
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).to(torch.uint8)
    neg = (blk < 0) & (code > 0)
    code = code | (neg.to(torch.uint8) << 3)
    code = code.reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, X.to(torch.uint8).contiguous()


# ---------------------------------------------------------------------------
# FP8 quantiser (input recipe).  OCP 8-bit floating point, E4M3 encoding (bias
# 7, largest finite magnitude 448, no infinities).  One fp32 scale per matrix,
# s = amax / 448 (1 for an all-zero matrix); codes = round-to-nearest-even of
# w / s on the e4m3 grid (torch's float8_e4m3fn cast).  Weight = value(code) * s.
# ---------------------------------------------------------------------------
def quantize_fp8(w: torch.Tensor):
    """w [N, K] fp32 -> (codes uint8 [N, K], scale fp32 [1])."""
    amax = w.abs().amax()
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    codes = (w / s).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, s.reshape(1).contiguous()


# ---------------------------------------------------------------------------
# NVFP4 quantiser (input recipe).  Blocks of 16 values along the contraction
# dim share an e4m3 scale; the matrix has one fp32 tensor scale
# ts = amax / (6 * 448) (1 for an all-zero matrix), so every block scale
# bmax / 6 / ts fits e4m3; block scales are rounded to nearest even on the
# e4m3 grid (torch's float8_e4m3fn cast), elements w / (scale * ts) to nearest
# even on the e2m1 grid, saturating at 6 (code 0 where the block scale is 0).
# Codes and nibble order as for MXFP4.  Weight = e2m1 * e4m3(scale) * ts.
# ---------------------------------------------------------------------------
def quantize_nvfp4(w: torch.Tensor):
    """w [N, K] fp32, K % 16 == 0 -> (codes uint8 [N, K/2], block scales uint8 [N, K/16],
    tensor scale fp32 [1])."""
    N, K = w.shape
    assert K % 16 == 0
    amax = w.abs().amax()
    ts = torch.where(amax > 0, amax / (6.0 * 448.0), torch.ones_like(amax)).to(torch.float32)
    blk = w.reshape(N, K // 16, 16)
    bs = (blk.abs().amax(dim=2) / 6.0 / ts).to(torch.float8_e4m3fn)
    den = (bs.to(torch.float32) * ts).unsqueeze(2)
    a = torch.where(den > 0, blk.abs() / torch.where(den > 0, den, torch.ones_like(den)),
                    torch.zeros_like(blk))
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).to(torch.uint8)
    neg = (blk < 0) & (code > 0)
    code = (code | (neg.to(torch.uint8) << 3)).reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, bs.view(torch.uint8).contiguous(), ts.reshape(1).contiguous()


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------
def gen_x(shape: LayerShape, T: int, step: int = 0, device="cpu", layer: int = 0) -> torch.Tensor:
    """Activations [T, H], N(0,1), in the activation storage dtype."""
    return to_storage(_randn((T, shape.H), 1.0, seed_of(shape, _T_X, layer, 0, step, T), device),
                      shape.adtype)


def gen_router(shape: LayerShape, layer: int = 0, device="cpu") -> torch.Tensor:
    """Router weight [E, H], N(0, 0.02), in the activation storage dtype."""
    return to_storage(_randn((shape.E, shape.H), shape.router_std,
                             seed_of(shape, _T_ROUTER, layer), device), shape.adtype)


def gen_bias(shape: LayerShape, layer: int = 0, device="cpu") -> Optional[torch.Tensor]:
    """Per-expert router logit bias [E] fp32, or None.

    zipf(s): b_e = -s * ln(r_e) with r a seeded permutation of 1..E, i.e. the
    log of a Zipf pmf over a random expert ranking (constant term dropped: it
    cancels in top-k and in the softmax).  normal(sd): b_e ~ N(0, sd).
    """
    if shape.bias == "none":
        return None
    g = _gen(seed_of(shape, _T_BIAS, layer), "cpu")
    if shape.bias == "zipf":
        r = torch.randperm(shape.E, generator=g).to(torch.float64) + 1.0
        b = (-shape.bias_param * torch.log(r)).to(torch.float32)
    elif shape.bias == "normal":
        b = torch.randn(shape.E, generator=g, dtype=torch.float32) * shape.bias_param
    else:
        raise ValueError(shape.bias)
    return b.to(device)


def gen_logits(shape: LayerShape, T: int, step: int = 0, device="cpu", scale: float = 1.0):
    """Free-standing fp32 router logits [T, E] ~ N(0, scale) (routing-only tests)."""
    return _randn((T, shape.E), scale, seed_of(shape, _T_LOGITS, 0, 0, step, T), device)


def gen_expert(shape: LayerShape, e: int, layer: int = 0, device="cpu") -> dict:
    """One expert's weights in logical layout.

    f32/bf16: {"gate": [I,H], "up": [I,H], "down": [H,I]}.
    mxfp4:    {"gate": codes [I,H/2], "gate_sc": [I,H/32], "up", "up_sc",
               "down": codes [H,I/2], "down_sc": [H,I/32]}.
    fp8:      {"gate": e4m3 codes [I,H], "gate_sc": fp32 [1], "up", "up_sc",
               "down": codes [H,I], "down_sc": fp32 [1]}.
    nvfp4:    {"gate": codes [I,H/2], "gate_sc": e4m3 [I,H/16], "gate_ts": fp32 [1],
               "up", "up_sc", "up_ts", "down": codes [H,I/2], "down_sc": [H,I/16],
               "down_ts"}.
    Expert index ``e == shape.E`` is the shared expert (when n_shared == 1).
    """
    H, I = shape.H, shape.I
    sg, sd = 1.0 / math.sqrt(H), 1.0 / math.sqrt(I)
    g = _randn((I, H), sg, seed_of(shape, _T_GATE, layer, e), device)
    u = _randn((I, H), sg, seed_of(shape, _T_UP, layer, e), device)
    d = _randn((H, I), sd, seed_of(shape, _T_DOWN, layer, e), device)
    if shape.wdtype in ("f32", "bf16"):
        return {"gate": to_storage(g, shape.wdtype), "up": to_storage(u, shape.wdtype),
                "down": to_storage(d, shape.wdtype)}
    out = {}
    for name, t in (("gate", g), ("up", u), ("down", d)):
        if shape.wdtype == "nvfp4":
            out[name], out[name + "_sc"], out[name + "_ts"] = quantize_nvfp4(t)
        else:
            quant = quantize_mxfp4 if shape.wdtype == "mxfp4" else quantize_fp8
            out[name], out[name + "_sc"] = quant(t)
    return out


def n_experts_total(shape: LayerShape) -> int:
    return shape.E + shape.n_shared
