"""Seeded synthetic inputs for the LAGA per-rank attention path.

This module only draws random numbers and rounds them to the storage dtype of a
workload. It holds none of the method's arithmetic, so both the fp64 oracle and
the HIP path can take their inputs from it without sharing any computation.

Workloads follow the paper "A Training-Memory Regression in MLA Sequence
Parallelism: Why Megatron-Core Forbids Absorption, and LAGA -- a
Communication-Efficient Fix" (arXiv 2607.17644v1): DeepSeek-V3 dimensions from
§4.1 (n_h=128, d_nope=d_v=128, d_rope=64, d_kv=512), sequence lengths 4K and 16K
from §4.2-§4.4, and the head shard n_h/P of one rank from §3.3.

Draw order (fp64 standard normals from numpy's PCG64, one generator per call):
  1. q       [B, S, h, d_nope + d_rope]   (nope part first)
  2. latent  [B, S, d_kv]
  3. k_pe    [B, S, d_rope]
  4. w_kv_b  [n_h, d_nope + d_v, d_kv] scaled by 1/sqrt(d_kv)
  5. gamma   [d_kv] = 1 + 0.1 * z
  6. d_o     [B, S, h, d_v]               (only when a backward is requested)
Every tensor is then rounded once to the workload's dtype; the rounded values
are what both sides consume.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Dims:
    """Shape of one rank's share: h = n_h / sp_size local heads, H_r = [r*h, (r+1)*h)."""

    B: int
    S: int
    n_h: int
    sp_size: int
    sp_rank: int
    d_kv: int
    d_nope: int
    d_rope: int
    d_v: int
    dtype: str
    eps: float = 1e-6

    @property
    def h(self) -> int:
        return self.n_h // self.sp_size

    @property
    def d_qk(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def head_lo(self) -> int:
        return self.sp_rank * self.h


# The five workloads: the first is the small fp32 case, the others use
# DeepSeek-V3 head dimensions at one rank's share (SP=8) or at SP=1.
WORKLOADS = {
    "tiny_f32_s256_h2": dict(
        dims=Dims(B=1, S=256, n_h=2, sp_size=1, sp_rank=0, d_kv=64, d_nope=32,
                  d_rope=16, d_v=32, dtype=F32), backward=False),
    "v3_sp8_s4096_h16": dict(
        dims=Dims(B=1, S=4096, n_h=128, sp_size=8, sp_rank=0, d_kv=512, d_nope=128,
                  d_rope=64, d_v=128, dtype=BF16), backward=False),
    "v3_sp8_s16384_h16": dict(
        dims=Dims(B=1, S=16384, n_h=128, sp_size=8, sp_rank=0, d_kv=512, d_nope=128,
                  d_rope=64, d_v=128, dtype=BF16), backward=False),
    "v3_sp1_s4096_h128": dict(
        dims=Dims(B=1, S=4096, n_h=128, sp_size=1, sp_rank=0, d_kv=512, d_nope=128,
                  d_rope=64, d_v=128, dtype=BF16), backward=False),
    "v3_sp8_s16384_h16_train": dict(
        dims=Dims(B=1, S=16384, n_h=128, sp_size=8, sp_rank=0, d_kv=512, d_nope=128,
                  d_rope=64, d_v=128, dtype=BF16), backward=True),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even, via float32) and return the raw 16-bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """One input: `value` is the rounded tensor in fp64, `raw` its storage (uint16 bf16 bits or float32)."""

    value: np.ndarray
    raw: np.ndarray
    dtype: str


def _round(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == F32:
        raw = np.ascontiguousarray(x, dtype=np.float32)
        return Tensor(raw.astype(np.float64), raw, dtype)
    if dtype == BF16:
        raw = bf16_bits(x)
        return Tensor(bf16_bits_to_f64(raw), raw, dtype)
    raise ValueError(f"unknown dtype {dtype}")


def make_inputs(dims: Dims, seed: int = 0, backward: bool = False) -> dict[str, Tensor]:
    """Draw the inputs of one rank's share in the fixed order documented above."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, S, h = dims.B, dims.S, dims.h
    out = {}
    out["q"] = _round(rng.standard_normal((B, S, h, dims.d_qk)), dims.dtype)
    out["latent"] = _round(rng.standard_normal((B, S, dims.d_kv)), dims.dtype)
    out["k_pe"] = _round(rng.standard_normal((B, S, dims.d_rope)), dims.dtype)
    w = rng.standard_normal((dims.n_h, dims.d_nope + dims.d_v, dims.d_kv)) / np.sqrt(dims.d_kv)
    out["w_kv_b"] = _round(w, dims.dtype)
    out["gamma"] = _round(1.0 + 0.1 * rng.standard_normal(dims.d_kv), dims.dtype)
    if backward:
        out["d_o"] = _round(rng.standard_normal((B, S, h, dims.d_v)), dims.dtype)
    return out


def workload(name: str) -> tuple[Dims, bool]:
    w = WORKLOADS[name]
    return w["dims"], w["backward"]


def to_torch(t: Tensor, device="cuda"):
    """Copy one input to a torch tensor on `device` in its storage dtype (bf16 or float32)."""
    import torch
    if t.dtype == BF16:
        host = torch.from_numpy(t.raw.view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(t.raw)
    return host.to(device).contiguous()
