"""Seeded synthetic inputs for the Beam MoE block.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds the layer shapes and the input recipe only: it draws random numbers
and converts them to the stored dtypes with torch's own conversions.  None of
the block's arithmetic (routing, expert MLPs, combine, activation
quantisation) lives here.

Shapes come from the pages:
  * "Hugging Face releases Beam, a 501B-parameter open Mixture-of-Experts model
    with 1M-token context" (the architecture paragraphs): hidden size 5,120,
    256 experts per MoE layer, SwiGLU intermediate size 2,560, top-8 experts
    from the top-4 of 8 groups of 32.
  * "Reflection Releases Beam ..." section "Where Beam Saves and Where the
    Memory Bill Comes In": no shared expert, DeepSeek-V3 group-limited sigmoid
    router, routed weights normalised and scaled by 2.5.

The init notation N(0, 1/H) for the router is read as a variance (logit std
1) and N(0, 0.02) for expert weights as a standard deviation.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

F32, BF16, FP8, MXFP4 = "f32", "bf16", "fp8", "mxfp4"


@dataclasses.dataclass(frozen=True)
class Shape:
    hidden: int
    intermediate: int
    n_experts: int
    n_groups: int
    topk_groups: int
    top_k: int
    group_score_topn: int = 2
    routed_scale: float = 2.5

    @property
    def group_size(self) -> int:
        return self.n_experts // self.n_groups


BEAM = Shape(hidden=5120, intermediate=2560, n_experts=256, n_groups=8,
             topk_groups=4, top_k=8)
# One GPU's share under expert parallelism over 8 GPUs: one group of 32
# experts at the Beam widths; 16K tokens x top-8 over 32 experts gives about
# 4K rows per expert.
EP8_SHARE = Shape(hidden=5120, intermediate=2560, n_experts=32, n_groups=1,
                  topk_groups=1, top_k=8)
TINY = Shape(hidden=256, intermediate=128, n_experts=16, n_groups=4,
             topk_groups=2, top_k=4)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    shape: Shape
    act_dtype: str          # dtype of x and out: f32 or bf16
    weight_dtype: str       # f32, bf16, fp8 (e4m3 + 128x128 fp32 scales) or
                            # mxfp4 (E2M1 pairs + one E8M0 byte per 32 of a row)
    bias: str               # "zero", "uniform:<a>", "skew:<v>:<e0,e1,...>"
    seed: int
    expert_std: float = 0.02


# The five workloads, in the order the layer is specified for measurement.
WORKLOADS = {
    "tiny": Workload("tiny", 16, TINY, F32, F32, "uniform:0.01", 0),
    "decode64": Workload("decode64", 64, BEAM, BF16, BF16, "zero", 1),
    "prefill4k": Workload("prefill4k", 4096, BEAM, BF16, BF16, "uniform:0.02", 2),
    "prefill16k_skew": Workload("prefill16k_skew", 16384, BEAM, BF16, BF16,
                                "skew:0.5:0,1,2,3,32,33,34,35", 3),
    "fp8_8k": Workload("fp8_8k", 8192, BEAM, BF16, FP8, "zero", 4),
    # decode batch on the FP8 weights (the 128-row tiles with a copy ring)
    "fp8_decode64": Workload("fp8_decode64", 64, BEAM, BF16, FP8, "zero", 8),
    # the per-GPU share of an expert-parallel layer (32 local experts)
    "ep8_share16k": Workload("ep8_share16k", 16384, EP8_SHARE, BF16, BF16, "zero", 7),
    # the 4-bit checkpoint form (MXFP4 stands in for the pages' NVFP4)
    "mxfp4_decode64": Workload("mxfp4_decode64", 64, BEAM, BF16, MXFP4, "zero", 5),
    "mxfp4_8k": Workload("mxfp4_8k", 8192, BEAM, BF16, MXFP4, "zero", 6),
}


def _bias(spec: str, E: int, g: torch.Generator, device) -> torch.Tensor:
    if spec == "zero":
        return torch.zeros(E, dtype=torch.float32, device=device)
    if spec.startswith("uniform:"):
        a = float(spec.split(":")[1])
        u = torch.rand(E, generator=g, device=device, dtype=torch.float32)
        return (u * (2 * a) - a).contiguous()
    if spec.startswith("skew:"):
        _, v, idx = spec.split(":")
        b = torch.zeros(E, dtype=torch.float32, device=device)
        for e in idx.split(","):
            b[int(e)] = float(v)
        return b
    raise ValueError(f"unknown bias spec {spec!r}")


def _store(t: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == F32:
        return t.contiguous()
    if dtype == BF16:
        return t.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def _fp8_blocks(w: torch.Tensor, block: int = 128):
    """Offline weight preparation for the FP8 checkpoint form: torch's own
    e4m3fn conversion of w / (block amax / 448), per block x block tile."""
    R, C = w.shape
    wb = w.reshape(R // block, block, C // block, block)
    amax = wb.abs().amax(dim=(1, 3))                      # [R/b, C/b]
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wb / scale[:, None, :, None]).clamp(-448.0, 448.0)
    q = q.to(torch.float8_e4m3fn).reshape(R, C)
    return q.view(torch.uint8).contiguous(), scale.to(torch.float32).contiguous()


_E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _mxfp4_rows(w: torch.Tensor):
    """Offline weight preparation for the 4-bit checkpoint form, OCP MX FP4:
    per 32 consecutive values of a row the shared exponent is floor(log2 of
    the block's largest magnitude) - 2 (E8M0 byte, exponent + 127, -127 for a
    zero block); each value scaled by 2^-exponent goes to the nearest E2M1
    value (ties to the even code, saturating at 6).  Codes are packed two per
    byte, the even column in the low nibble."""
    R, C = w.shape
    wb = w.reshape(R, C // 32, 32)
    amax = wb.abs().amax(dim=-1)
    _, e = torch.frexp(amax)
    x = torch.where(amax > 0, e - 3, torch.full_like(e, -127)).clamp(-127, 127)
    u = torch.ldexp(wb, (-x)[..., None].to(wb.dtype))
    a = u.abs().contiguous()
    grid = torch.tensor(_E2M1_MAGNITUDES, dtype=a.dtype, device=a.device)
    lo = (torch.searchsorted(grid, a, right=True) - 1).clamp(0, 7)
    hi = (lo + 1).clamp(max=7)
    dlo, dhi = a - grid[lo], grid[hi] - a
    code = torch.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    code = (code + 8 * torch.signbit(u).to(code.dtype)).reshape(R, C).to(torch.uint8)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, (x + 127).to(torch.uint8).contiguous()


@dataclasses.dataclass
class Inputs:
    workload: Workload
    x: torch.Tensor            # [T, H] f32 or bf16
    w_router: torch.Tensor     # [E, H] f32
    bias: torch.Tensor         # [E] f32
    w_gate_up: torch.Tensor    # [E, 2I, H] f32/bf16, uint8 e4m3 codes, or
                               # [E, 2I, H/2] uint8 E2M1 pairs (mxfp4)
    w_down: torch.Tensor       # [E, H, I] likewise ([E, H, I/2] for mxfp4)
    s_gate_up: Optional[torch.Tensor] = None   # [E, 2I/128, H/128] f32 (fp8);
                                               # [E, 2I, H/32] uint8 E8M0 (mxfp4)
    s_down: Optional[torch.Tensor] = None      # [E, H/128, I/128] f32 (fp8);
                                               # [E, H, I/32] uint8 E8M0 (mxfp4)


def make_inputs(w: Workload, device="cpu", tokens: Optional[int] = None,
                shape: Optional[Shape] = None, seed: Optional[int] = None,
                bias: Optional[str] = None) -> Inputs:
    """Draw the inputs of one workload, in a fixed order: x, router weights,
    bias, then per expert its gate/up and down weights.  The same seed and
    device give the same bytes."""
    T = w.tokens if tokens is None else tokens
    S = w.shape if shape is None else shape
    sd = w.seed if seed is None else seed
    bspec = w.bias if bias is None else bias
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(sd)
    H, I, E = S.hidden, S.intermediate, S.n_experts

    x = torch.randn(T, H, generator=g, device=dev, dtype=torch.float32)
    x = _store(x, w.act_dtype)
    wr = torch.randn(E, H, generator=g, device=dev, dtype=torch.float32)
    wr = (wr * (1.0 / math.sqrt(H))).contiguous()
    b = _bias(bspec, E, g, dev)

    fp8 = w.weight_dtype == FP8
    mx4 = w.weight_dtype == MXFP4
    st = torch.uint8 if (fp8 or mx4) else (torch.float32 if w.weight_dtype == F32
                                           else torch.bfloat16)
    div = 2 if mx4 else 1
    wgu = torch.empty(E, 2 * I, H // div, dtype=st, device=dev)
    wd = torch.empty(E, H, I // div, dtype=st, device=dev)
    sgu = sdn = None
    if fp8:
        sgu = torch.empty(E, 2 * I // 128, H // 128, device=dev)
        sdn = torch.empty(E, H // 128, I // 128, device=dev)
    if mx4:
        sgu = torch.empty(E, 2 * I, H // 32, dtype=torch.uint8, device=dev)
        sdn = torch.empty(E, H, I // 32, dtype=torch.uint8, device=dev)
    for e in range(E):
        a = torch.randn(2 * I, H, generator=g, device=dev) * w.expert_std
        c = torch.randn(H, I, generator=g, device=dev) * w.expert_std
        if fp8:
            wgu[e], sgu[e] = _fp8_blocks(a)
            wd[e], sdn[e] = _fp8_blocks(c)
        elif mx4:
            wgu[e], sgu[e] = _mxfp4_rows(a)
            wd[e], sdn[e] = _mxfp4_rows(c)
        else:
            wgu[e] = a.to(st)
            wd[e] = c.to(st)
    return Inputs(w, x, wr, b, wgu, wd, sgu, sdn)


def small_shape(hidden=512, intermediate=256, n_experts=64, n_groups=8,
                topk_groups=4, top_k=8) -> Shape:
    """A reduced Beam-like layer for parity runs the oracle finishes fast."""
    return Shape(hidden=hidden, intermediate=intermediate, n_experts=n_experts,
                 n_groups=n_groups, topk_groups=topk_groups, top_k=top_k)
