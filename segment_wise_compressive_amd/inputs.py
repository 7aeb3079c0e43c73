"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws i.i.d. normal
q, k, v tensors from a seeded torch generator, scales them and rounds them to
the input dtype.  Both the HIP path and the oracle are fed the very tensors
produced here.

Recipe (same for every workload):
  * one ``torch.Generator`` on the requested device, seeded with the workload's
    seed; q, then k, then v are drawn with ``torch.randn`` in float32;
  * each is multiplied (in float32) by the workload's scale (1 for the fp32
    workload, 1/sqrt(d) for the bf16 workloads);
  * bf16 workloads round the float32 values to bfloat16 (round to nearest even).
  * The decode workload draws the prefix q, k, v [B, H, P, d] first and then
    the per-step q, k, v [T, B, H, d].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "causal" | "segmented" | "decode" | "noncausal" | "memory"
    dtype: torch.dtype   # input dtype of q, k, v
    B: int
    H: int
    N: int               # tokens per head (whole sequence; decode: steps)
    d: int
    seed: int
    scale: float
    eps: float = 1e-6
    chunk: int = 0       # 0 = library default
    segment: int = 0     # segmented: tokens per segment
    prefix: int = 0      # decode: prefix length that initialises the state

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.N


def _isqrt(d: int) -> float:
    return 1.0 / math.sqrt(d)


# The five synthetic workloads (shapes, dtypes and distributions of the
# causal / segment-carried / decode / non-causal uses of linear attention).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("causal_f32_b1h1n256d32", "causal", torch.float32,
                 1, 1, 256, 32, seed=1001, scale=1.0),
        Workload("causal_bf16_b4h8n4096d64", "causal", torch.bfloat16,
                 4, 8, 4096, 64, seed=1002, scale=_isqrt(64), chunk=64),
        Workload("segmented_bf16_b1h16n65536d128_seg2048", "segmented", torch.bfloat16,
                 1, 16, 65536, 128, seed=1003, scale=_isqrt(128), segment=2048),
        Workload("decode_bf16_b64h32d128_prefix1024_steps1024", "decode", torch.bfloat16,
                 64, 32, 1024, 128, seed=1004, scale=_isqrt(128), prefix=1024),
        Workload("noncausal_bf16_b8h16n16384d64", "noncausal", torch.bfloat16,
                 8, 16, 16384, 64, seed=1005, scale=_isqrt(64)),
        # compressive memory (retrieval, then update) over the segment stream
        # of the segment-carried workload's shape
        Workload("memory_bf16_b1h16n65536d128_seg2048", "memory", torch.bfloat16,
                 1, 16, 65536, 128, seed=1006, scale=_isqrt(128), segment=2048),
    ]
}
SMALL = "causal_f32_b1h1n256d32"
HEADLINE = "causal_bf16_b4h8n4096d64"
SEGMENTED = "segmented_bf16_b1h16n65536d128_seg2048"
DECODE = "decode_bf16_b64h32d128_prefix1024_steps1024"
NONCAUSAL = "noncausal_bf16_b8h16n16384d64"
MEMORY = "memory_bf16_b1h16n65536d128_seg2048"


def draw(shape, gen: torch.Generator, dtype: torch.dtype, scale: float,
         device: Optional[str] = None) -> torch.Tensor:
    """One tensor: float32 N(0,1) * scale, rounded to ``dtype``."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device or gen.device)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype) if dtype != torch.float32 else x


def make_generator(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def qkv(shape, seed: int, dtype: torch.dtype, scale: float, device: str = "cpu"):
    """q, k, v of ``shape`` drawn in that order from one generator."""
    g = make_generator(seed, device)
    return tuple(draw(shape, g, dtype, scale) for _ in range(3))


def workload_inputs(w: Workload, device: str = "cpu"):
    """Inputs of a workload.

    causal / segmented / noncausal / memory: (q, k, v) each [B, H, N, d].
    decode: (prefix (q, k, v) each [B, H, P, d], steps (q, k, v) each [T, B, H, d]).
    """
    g = make_generator(w.seed, device)
    if w.kind == "decode":
        pre = tuple(draw((w.B, w.H, w.prefix, w.d), g, w.dtype, w.scale) for _ in range(3))
        steps = tuple(draw((w.N, w.B, w.H, w.d), g, w.dtype, w.scale) for _ in range(3))
        return pre, steps
    return tuple(draw((w.B, w.H, w.N, w.d), g, w.dtype, w.scale) for _ in range(3))
