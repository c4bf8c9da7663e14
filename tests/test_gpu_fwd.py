"""Forward parity of the HIP path against the fp64 oracle (needs an MI355X).

Small shapes are compared element by element on every output (L, rstd, k_nope,
v, o, lse); the DeepSeek-V3 workloads at their full sizes are compared on
sampled query rows, which the oracle computes one by one, plus the full
intermediate tensors.
"""
import numpy as np
import pytest
import torch

import laga_inputs as li
import oracle
from gpu_util import FP16, SPLIT, announce, check, device_inputs, host, kv_host, make_path, sample_rows

pytestmark = pytest.mark.gpu


def _dims(B, S, n_h, sp_size, sp_rank, dtype):
    if dtype == li.F32:
        return li.Dims(B=B, S=S, n_h=n_h, sp_size=sp_size, sp_rank=sp_rank, d_kv=64, d_nope=32,
                       d_rope=16, d_v=32, dtype=li.F32)
    return li.Dims(B=B, S=S, n_h=n_h, sp_size=sp_size, sp_rank=sp_rank, d_kv=512, d_nope=128,
                   d_rope=64, d_v=128, dtype=li.BF16)


# Split K/V storage (fp16 + e4m3 low plane) holds the up-projection to ~2^-15
# relative: |x| stays below ~8 on these inputs, so the stored value is within
# 2^-12 * 2^-4 * 8 = 2^-13 of the exact one plus the fp32 GEMM's error.
# Single fp16 storage would miss this bound (its error reaches 2^-9 at |x| = 4).
SPLIT_KV_MAX = 2.0 ** -12


def check_kv(path, name, buf, ref, d, precision):
    width = d.d_nope if name == "k_nope" else d.d_v
    got = kv_host(path, buf, width)
    check(name, got, ref, d.dtype)
    if d.dtype == li.BF16 and precision == SPLIT:
        mx = float(np.abs(got - ref).max())
        assert mx <= SPLIT_KV_MAX, f"{name}: split storage max-abs {mx:.3e} > {SPLIT_KV_MAX:.3e}"


def _full_forward_check(d: li.Dims, precision: int, seed: int = 0):
    announce(f"forward full compare dims={d} precision={precision} seed={seed}")
    inp = li.make_inputs(d, seed)
    x = device_inputs(inp)
    path = make_path(d, precision)
    out = path.alloc_forward()
    for k in ("latent_n", "rstd", "o", "lse"):
        out[k].fill_(float("nan"))
    path.forward(x, out)
    torch.cuda.synchronize()
    v = {k: t.value for k, t in inp.items()}
    ref = oracle.forward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], n_h=d.n_h,
                         sp_size=d.sp_size, sp_rank=d.sp_rank, d_nope=d.d_nope, eps=d.eps)
    check("L", host(out["latent_n"]), ref["L"], d.dtype)
    check("rstd", host(out["rstd"]), ref["rstd"], li.F32 if d.dtype == li.F32 else d.dtype)
    check_kv(path, "k_nope", out["k_nope"], ref["k_nope"], d, precision)
    check_kv(path, "v", out["v"], ref["v"], d, precision)
    check("o", host(out["o"]), ref["O"], d.dtype)
    check("lse", host(out["lse"]), ref["lse"], d.dtype)
    return out


def test_tiny_f32_workload():
    d, _ = li.workload("tiny_f32_s256_h2")
    _full_forward_check(d, FP16)


@pytest.mark.parametrize("B,S,n_h,P,r", [(1, 200, 2, 1, 0), (1, 1, 2, 1, 0), (2, 77, 4, 2, 1),
                                         (1, 129, 16, 2, 0), (3, 64, 8, 8, 5)])
def test_f32_shapes(B, S, n_h, P, r):
    _full_forward_check(_dims(B, S, n_h, P, r, li.F32), FP16, seed=B * 1000 + S)


@pytest.mark.parametrize("precision", [FP16, SPLIT])
@pytest.mark.parametrize("B,S,n_h,P,r", [(1, 300, 16, 8, 3), (2, 130, 64, 8, 7), (1, 1, 16, 8, 0),
                                         (1, 64, 128, 16, 2), (1, 1000, 16, 8, 2), (1, 150, 15, 5, 2),
                                         (2, 97, 5, 1, 0)])
def test_bf16_shapes(precision, B, S, n_h, P, r):
    _full_forward_check(_dims(B, S, n_h, P, r, li.BF16), precision, seed=S + P)


@pytest.mark.parametrize("name,precision", [("v3_sp8_s4096_h16", FP16), ("v3_sp8_s16384_h16", FP16),
                                            ("v3_sp1_s4096_h128", FP16),
                                            ("v3_sp8_s16384_h16", SPLIT)])
def test_full_size_workloads(name, precision):
    d, _ = li.workload(name)
    announce(f"forward full-size {name} precision={precision}")
    inp = li.make_inputs(d, 0)
    x = device_inputs(inp)
    path = make_path(d, precision)
    out = path.forward(x)
    torch.cuda.synchronize()
    v = {k: t.value for k, t in inp.items()}
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    L, rstd = oracle.latent_rmsnorm(v["latent"], v["gamma"], d.eps)
    check("L", host(out["latent_n"]), L, d.dtype)
    check("rstd", host(out["rstd"]), rstd, d.dtype)
    kn, vv = oracle.kv_up(L, v["w_kv_b"], heads, d.d_nope)
    del L
    check_kv(path, "k_nope", out["k_nope"], kn, d, precision)
    check_kv(path, "v", out["v"], vv, d, precision)
    rows = sample_rows(d.S)
    O, lse = oracle.attention_fwd_rows(v["q"], kn, v["k_pe"], vv, rows)
    check("o[rows]", host(out["o"])[:, rows], O, d.dtype)
    check("lse[rows]", host(out["lse"])[..., rows], lse, d.dtype)


def test_long_sequence_sampled_rows():
    """Twice the longest workload's sequence (16 local heads, fp16 operands):
    index arithmetic of every kernel beyond the workload sizes, checked on
    sampled query rows."""
    d = _dims(1, 32768, 128, 8, 0, li.BF16)
    announce(f"forward long sequence dims={d}")
    inp = li.make_inputs(d, 11)
    x = device_inputs(inp)
    out = make_path(d, FP16).forward(x)
    torch.cuda.synchronize()
    v = {k: t.value for k, t in inp.items()}
    del inp, x
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    L, _ = oracle.latent_rmsnorm(v["latent"], v["gamma"], d.eps)
    kn, vv = oracle.kv_up(L, v["w_kv_b"], heads, d.d_nope)
    del L
    rows = sample_rows(d.S, n=24, seed=3)
    O, lse = oracle.attention_fwd_rows(v["q"], kn, v["k_pe"], vv, rows)
    check("o[rows]", host(out["o"])[:, rows], O, d.dtype)
    check("lse[rows]", host(out["lse"])[..., rows], lse, d.dtype)


def test_determinism_and_causality():
    d = _dims(1, 700, 16, 8, 1, li.BF16)
    announce(f"determinism/causality dims={d}")
    inp = li.make_inputs(d, 5)
    x = device_inputs(inp)
    path = make_path(d, SPLIT)
    a = {k: t.clone() for k, t in path.forward(x).items()}
    b = path.forward(x)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    t0 = 333
    x2 = {k: t.clone() for k, t in x.items()}
    x2["q"][:, t0 + 1:] = -x2["q"][:, t0 + 1:]
    x2["latent"][:, t0 + 1:] = x2["latent"][:, t0 + 1:] * 3
    x2["k_pe"][:, t0 + 1:] = 0
    c = path.forward(x2)
    torch.cuda.synchronize()
    assert torch.equal(c["o"][:, :t0 + 1], a["o"][:, :t0 + 1])
    assert torch.equal(c["lse"][..., :t0 + 1], a["lse"][..., :t0 + 1])
    assert not torch.equal(c["o"][:, t0 + 1:], a["o"][:, t0 + 1:])
