"""Seeded synthetic inputs for the causal Based forward.

This module holds no arithmetic of the method. It only draws i.i.d. N(0, 1) numbers and rounds them to
bfloat16, so that the GPU path and the CPU oracle can be fed the same bytes.

The page that specifies the operation ("Write a fast Based (Taylor linear attention) forward kernel",
field make_inputs_src) draws q, then k, then v with torch.randn in bfloat16 from a CUDA generator. That
stream cannot be reproduced off the GPU, so the recipe here is: numpy.random.default_rng(seed) (PCG64),
standard_normal in float32 for q, then k, then v, each in C order over (B, T, H, K) or (B, T, H, V), then
float32 -> bfloat16 with round-to-nearest-even. Same distribution, different stream.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic Based forward problem: shapes, seed, scale (None = K**-0.5) and output dtype."""
    name: str
    B: int
    T: int
    H: int
    K: int
    V: int
    seed: int
    scale: float | None
    out_dtype: str  # "bf16" or "f32"

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H


# The five problem sizes this implementation is measured and checked on. The first is small enough for the
# oracle's direct O(T^2) form in well under a second; the third is the headline shape.
WORKLOADS = (
    Workload("b1_t512_h2_k8_v64", 1, 512, 2, 8, 64, 0, None, "f32"),
    Workload("b2_t2048_h8_k16_v64", 2, 2048, 8, 16, 64, 1, None, "bf16"),
    Workload("b4_t8192_h16_k16_v64", 4, 8192, 16, 16, 64, 2, None, "bf16"),
    Workload("b8_t4096_h16_k16_v128", 8, 4096, 16, 16, 128, 3, 0.2, "bf16"),
    Workload("b1_t65000_h16_k16_v64", 1, 65000, 16, 16, 64, 4, None, "bf16"),
)
HEADLINE = WORKLOADS[2]

# The shape lists the page gives for this task (field shapes of the task spec): (B, T, H, K, V) for its
# correctness, quick-measure, measure and grader runs. Scale K**-0.5, bfloat16 output.
_PAGE = (
    ("correct", [(1, 256, 4, 16, 128), (2, 512, 8, 16, 64), (1, 512, 6, 8, 128), (2, 128, 4, 16, 128)]),
    ("quick", [(1, 2048, 16, 16, 128), (2, 2048, 8, 16, 128), (1, 4096, 16, 8, 128)]),
    ("measure", [(4, 12288, 32, 16, 128), (8, 8192, 16, 16, 128), (4, 16384, 32, 16, 64), (2, 16384, 32, 16, 128),
                 (4, 16384, 32, 8, 128)]),
    ("grader", [(4, 16384, 32, 16, 128), (8, 8192, 32, 16, 128), (8, 16384, 16, 16, 128), (8, 16384, 32, 16, 64),
                (8, 16384, 32, 8, 128)]),
)
PAGE_SHAPES = tuple(
    Workload(f"page_{role}_b{B}_t{T}_h{H}_k{K}_v{V}", B, T, H, K, V, 100 + 10 * r + i, None, "bf16")
    for r, (role, shapes) in enumerate(_PAGE) for i, (B, T, H, K, V) in enumerate(shapes))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_qkv(B: int, T: int, H: int, K: int, V: int, seed: int):
    """Return (q, k, v) as uint16 bfloat16 bit patterns of shapes (B,T,H,K), (B,T,H,K), (B,T,H,V)."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, T, H, K), dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((B, T, H, K), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, T, H, V), dtype=np.float32))
    return q, k, v


def make_workload(w: Workload):
    return make_qkv(w.B, w.T, w.H, w.K, w.V, w.seed)


def make_qkv_device(B: int, T: int, H: int, K: int, V: int, seed: int, device):
    """Seeded N(0, 1) inputs drawn directly on the GPU (torch's generator for that device), rounded to
    bfloat16: q, then k, then v. For timing runs at sizes where host-side generation would dominate; the
    values are not reproducible off the GPU and are never compared with the oracle."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for shape in ((B, T, H, K), (B, T, H, K), (B, T, H, V)):
        out.append(torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16))
    return tuple(out)
