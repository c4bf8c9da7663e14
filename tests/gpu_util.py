"""Helpers of the GPU parity tests: run the HIP path through the C ABI on seeded
inputs and measure its error against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import laga_inputs as li
from head_latent_attention_laga_amd import LagaPath

# Bars of the path: fp32 inputs max-abs 1e-4; bf16 inputs max-abs 1e-2 and mean-abs 1e-3.
F32_MAX = 1e-4
BF16_MAX, BF16_MEAN = 1e-2, 1e-3

FP16, SPLIT = 0, 1


def announce(msg: str):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def device_inputs(inp: dict) -> dict:
    return {k: li.to_torch(v) for k, v in inp.items()}


def make_path(d: li.Dims, precision: int) -> LagaPath:
    return LagaPath(d.B, d.S, d.n_h, d.sp_size, d.sp_rank, d.d_kv, d.d_nope, d.d_rope, d.d_v,
                    d.dtype, precision, d.eps)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def kv_host(path, t: torch.Tensor, width: int) -> np.ndarray:
    """Value of a k_nope / v buffer (the storage laga.h documents) in fp64."""
    return path.kv_value(t, width).numpy()


def err(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    e = np.abs(got - ref)
    return float(e.max()), float(e.mean())


def check(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, report: dict | None = None):
    mx, mn = err(got, ref)
    if report is not None:
        report[name] = (mx, mn)
    print(f"  {name:10s} max-abs {mx:.3e} mean-abs {mn:.3e}", flush=True)
    if dtype == li.F32:
        assert mx <= F32_MAX, f"{name}: max-abs {mx:.3e} > {F32_MAX}"
    else:
        assert mx <= BF16_MAX, f"{name}: max-abs {mx:.3e} > {BF16_MAX}"
        assert mn <= BF16_MEAN, f"{name}: mean-abs {mn:.3e} > {BF16_MEAN}"


def sample_rows(S: int, n: int = 40, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, S // 2, S - 2, S - 1]
    rows = set(t for t in fixed if 0 <= t < S)
    rows.update(int(t) for t in rng.integers(0, S, size=n))
    return np.array(sorted(rows))
