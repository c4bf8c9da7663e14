"""laga_attn_bwd_noalloc (static per-device scratch, no allocation) against
laga_attn_bwd (caller workspace) on the same inputs (needs an MI355X).

Both run the same kernels, which are deterministic, so every gradient must be
bitwise equal.  Two calls in a row, the second on a smaller problem, show that
what the first call left in the shared scratch does not leak into the second;
the second is also checked against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import laga_inputs as li
import oracle
from gpu_util import SPLIT, announce, check, device_inputs, host, make_path
from head_latent_attention_laga_amd import _lib

pytestmark = pytest.mark.gpu

GRADS = ("dq", "d_latent", "d_k_pe", "d_w_kv_b", "d_gamma")


def _fresh(path):
    g = path.alloc_backward()
    for k in ("dq", "d_latent", "d_k_pe", "d_gamma"):
        g[k].fill_(float("nan"))
    g["d_w_kv_b"].fill_(-7.0)
    return g


def _both(d: li.Dims, seed: int):
    inp = li.make_inputs(d, seed, backward=True)
    x = device_inputs(inp)
    path = make_path(d, SPLIT)
    assert _lib.attn_bwd_workspace_bytes(path.dims) <= _lib.LAGA_NOALLOC_SCRATCH_BYTES
    fwd = path.forward(x)
    ref = path.backward(x, fwd, x["d_o"], _fresh(path))
    got = _fresh(path)
    del got["workspace"]
    _lib.attn_bwd_noalloc(path.dims, x["q"], x["latent"], x["gamma"], fwd["rstd"], fwd["k_nope"], x["k_pe"],
                          fwd["v"], x["w_kv_b"], fwd["o"], fwd["lse"], x["d_o"], got["dq"], got["d_latent"],
                          got["d_k_pe"], got["d_w_kv_b"], got["d_gamma"])
    torch.cuda.synchronize()
    for k in GRADS:
        a, b = got[k], ref[k]
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{k}: noalloc differs from laga_attn_bwd"
    return inp, got


def test_noalloc_matches_workspace_backward_on_two_calls():
    big = li.Dims(B=1, S=4096, n_h=128, sp_size=8, sp_rank=3, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                  dtype=li.BF16)
    announce(f"noalloc backward, first call dims={big}")
    _both(big, seed=11)
    small = li.Dims(B=2, S=301, n_h=128, sp_size=8, sp_rank=6, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                    dtype=li.BF16)
    announce(f"noalloc backward, second (smaller) call dims={small}")
    inp, got = _both(small, seed=12)
    v = {k: t.value for k, t in inp.items()}
    ref = oracle.backward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], v["d_o"], n_h=small.n_h,
                          sp_size=small.sp_size, sp_rank=small.sp_rank, d_nope=small.d_nope, eps=small.eps)
    check("dq", host(got["dq"]), ref["dq"], small.dtype)
    check("d_latent", host(got["d_latent"]), ref["d_latent"], small.dtype)
    check("dk_pe", host(got["d_k_pe"]), ref["dk_pe"], small.dtype)
    check("d_gamma", host(got["d_gamma"]), ref["d_gamma"], small.dtype)
    heads = oracle.head_shard(small.n_h, small.sp_size, small.sp_rank)
    dW = host(got["d_w_kv_b"])
    check("d_w_kv_b", dW[heads], ref["d_w_kv_b"][heads], small.dtype)
    others = np.ones(small.n_h, dtype=bool)
    others[heads] = False
    assert np.all(dW[others] == -7.0), "rows outside the head shard were written"


def test_noalloc_rejects_oversize_before_launch():
    d = li.Dims(B=1, S=16384, n_h=128, sp_size=8, sp_rank=0, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                dtype=li.BF16)
    path = make_path(d, SPLIT)
    assert _lib.attn_bwd_workspace_bytes(path.dims) > _lib.LAGA_NOALLOC_SCRATCH_BYTES
    t = torch.empty(64, device="cuda")
    with pytest.raises(_lib.LagaError, match="WORKSPACE"):
        _lib.attn_bwd_noalloc(path.dims, *([t] * 16))
