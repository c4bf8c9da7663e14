"""Parity of the fused forward (laga_attn_fwd_fused: RMSNorm, head-shard
up-projection and attention with K/V kept in the library's workspace) against
the fp64 oracle (needs an MI355X).

Small shapes compare o and lse element by element; the full-size workloads
compare sampled query rows, which the oracle computes one by one.  The shapes
cover ragged sequence tails (S not a multiple of the 256-key producer tile or
the 256-query attention tile), batches, and head counts whose batch x heads
product is not a multiple of 8 (one ticket queue instead of eight).
"""
import numpy as np
import pytest
import torch

import laga_inputs as li
import oracle
from gpu_util import FP16, announce, check, device_inputs, host, make_path, sample_rows

pytestmark = pytest.mark.gpu


def _dims(B, S, n_h, P, r):
    return li.Dims(B=B, S=S, n_h=n_h, sp_size=P, sp_rank=r, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                   dtype=li.BF16)


def _err_word(out) -> int:
    """The fused kernel's error word (set only if a consumer gave up waiting)."""
    return int(out["workspace"][32:36].view(torch.int32).item())


def _oracle_full(inp, d):
    v = {k: t.value for k, t in inp.items()}
    return oracle.forward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], n_h=d.n_h, sp_size=d.sp_size,
                          sp_rank=d.sp_rank, d_nope=d.d_nope, eps=d.eps)


@pytest.mark.parametrize("B,S,n_h,P,r", [
    (1, 300, 16, 8, 3), (2, 130, 64, 8, 7), (1, 1, 16, 8, 0), (1, 64, 128, 16, 2), (1, 1000, 16, 8, 2),
    (1, 256, 16, 8, 1), (1, 257, 16, 8, 4), (3, 77, 24, 8, 1), (1, 513, 40, 8, 5), (2, 600, 128, 16, 9),
    (2, 2048, 16, 8, 6)])
def test_fused_full_compare(B, S, n_h, P, r):
    d = _dims(B, S, n_h, P, r)
    announce(f"fused forward full compare dims={d}")
    inp = li.make_inputs(d, seed=7 * S + r)
    x = device_inputs(inp)
    path = make_path(d, FP16)
    out = path.alloc_fused()
    out["o"].fill_(float("nan"))
    out["lse"].fill_(float("nan"))
    path.forward_fused(x, out)
    torch.cuda.synchronize()
    assert _err_word(out) == 0
    ref = _oracle_full(inp, d)
    check("o", host(out["o"]), ref["O"], d.dtype)
    check("lse", host(out["lse"]), ref["lse"], d.dtype)


def test_fused_reuses_workspace_and_is_deterministic():
    """Two problems in a row on one workspace: the second sees nothing of the
    first (images, counters); a repeat of a call is bitwise equal."""
    d = _dims(1, 1500, 16, 8, 6)
    announce(f"fused forward workspace reuse dims={d}")
    path = make_path(d, FP16)
    out = path.alloc_fused()
    first = li.make_inputs(d, seed=101)
    path.forward_fused(device_inputs(first), out)
    second = li.make_inputs(d, seed=202)
    x2 = device_inputs(second)
    path.forward_fused(x2, out)
    torch.cuda.synchronize()
    o1, l1 = out["o"].clone(), out["lse"].clone()
    assert _err_word(out) == 0
    ref = _oracle_full(second, d)
    check("o", host(o1), ref["O"], d.dtype)
    check("lse", host(l1), ref["lse"], d.dtype)
    for _ in range(3):
        path.forward_fused(x2, out)
        torch.cuda.synchronize()
        assert torch.equal(out["o"], o1) and torch.equal(out["lse"], l1)


def test_fused_matches_unfused_and_is_causal():
    d = _dims(1, 700, 16, 8, 1)
    announce(f"fused vs unfused, causality dims={d}")
    inp = li.make_inputs(d, 5)
    x = device_inputs(inp)
    path = make_path(d, FP16)
    a = path.forward_fused(x)
    a = {k: a[k].clone() for k in ("o", "lse")}
    u = path.forward(x)
    torch.cuda.synchronize()
    # Both paths round K/V to fp16; the fused one also rounds L and W to fp16
    # before the product, so they agree to well inside the oracle bars.
    check("o fused-unfused", host(a["o"]), host(u["o"]), d.dtype)
    check("lse fused-unfused", host(a["lse"]), host(u["lse"]), d.dtype)
    t0 = 333
    x2 = {k: t.clone() for k, t in x.items()}
    x2["q"][:, t0 + 1:] = -x2["q"][:, t0 + 1:]
    x2["latent"][:, t0 + 1:] = x2["latent"][:, t0 + 1:] * 3
    x2["k_pe"][:, t0 + 1:] = 0
    c = path.forward_fused(x2)
    torch.cuda.synchronize()
    assert torch.equal(c["o"][:, :t0 + 1], a["o"][:, :t0 + 1])
    assert torch.equal(c["lse"][..., :t0 + 1], a["lse"][..., :t0 + 1])
    assert not torch.equal(c["o"][:, t0 + 1:], a["o"][:, t0 + 1:])


@pytest.mark.parametrize("name", ["v3_sp8_s4096_h16", "v3_sp8_s16384_h16", "v3_sp1_s4096_h128"])
def test_fused_full_size_workloads(name):
    d, _ = li.workload(name)
    announce(f"fused forward full-size {name}")
    inp = li.make_inputs(d, 0)
    x = device_inputs(inp)
    path = make_path(d, FP16)
    out = path.forward_fused(x)
    torch.cuda.synchronize()
    assert _err_word(out) == 0
    v = {k: t.value for k, t in inp.items()}
    del inp, x
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    L, _ = oracle.latent_rmsnorm(v["latent"], v["gamma"], d.eps)
    kn, vv = oracle.kv_up(L, v["w_kv_b"], heads, d.d_nope)
    del L
    rows = sample_rows(d.S)
    O, lse = oracle.attention_fwd_rows(v["q"], kn, v["k_pe"], vv, rows)
    check("o[rows]", host(out["o"])[:, rows], O, d.dtype)
    check("lse[rows]", host(out["lse"])[..., rows], lse, d.dtype)


def test_fused_rejects_other_modes():
    from head_latent_attention_laga_amd import _lib
    from gpu_util import SPLIT
    d = _dims(1, 128, 16, 8, 0)
    assert _lib.attn_fwd_fused_workspace_bytes(make_path(d, SPLIT).dims) == 0
    assert np.isfinite(_lib.attn_fwd_fused_workspace_bytes(make_path(d, FP16).dims))
