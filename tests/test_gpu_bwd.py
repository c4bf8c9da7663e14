"""Backward parity of the HIP path against the fp64 oracle (needs an MI355X).

Small shapes compare every gradient element by element with the oracle run in
the test; the full-size training workload (S=16384, 16 local heads, V3 dims)
compares sampled entries with values the oracle wrote once
(tests/golden/make_train_golden.py), since its fp64 backward takes minutes.
"""
import os

import numpy as np
import pytest
import torch

import laga_inputs as li
import oracle
from gpu_util import FP16, SPLIT, announce, check, device_inputs, host, make_path

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "train_v3_sp8_s16384_h16.npz")


def _dims(B, S, n_h, P, r, dtype):
    if dtype == li.F32:
        return li.Dims(B=B, S=S, n_h=n_h, sp_size=P, sp_rank=r, d_kv=64, d_nope=32, d_rope=16, d_v=32,
                       dtype=li.F32)
    return li.Dims(B=B, S=S, n_h=n_h, sp_size=P, sp_rank=r, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                   dtype=li.BF16)


def _run(d: li.Dims, seed: int):
    inp = li.make_inputs(d, seed, backward=True)
    x = device_inputs(inp)
    path = make_path(d, FP16 if d.dtype == li.F32 else SPLIT)
    fwd = path.forward(x)
    g = path.alloc_backward()
    for k in ("dq", "d_latent", "d_k_pe", "d_gamma"):
        g[k].fill_(float("nan"))
    g["d_w_kv_b"].fill_(-7.0)  # rows outside this rank's shard must stay untouched
    path.backward(x, fwd, x["d_o"], g)
    torch.cuda.synchronize()
    return inp, fwd, g


@pytest.mark.parametrize("B,S,n_h,P,r,dtype", [
    (1, 256, 2, 1, 0, li.F32), (2, 77, 4, 2, 1, li.F32), (1, 1, 2, 1, 0, li.F32), (1, 200, 16, 8, 7, li.F32),
    (1, 300, 16, 8, 3, li.BF16), (2, 130, 64, 8, 7, li.BF16), (1, 1, 16, 8, 0, li.BF16),
    (1, 257, 128, 32, 5, li.BF16), (1, 1000, 16, 8, 2, li.BF16), (1, 150, 15, 5, 2, li.BF16),
    (2, 97, 5, 1, 0, li.BF16)])
def test_backward_full_compare(B, S, n_h, P, r, dtype):
    d = _dims(B, S, n_h, P, r, dtype)
    announce(f"backward full compare dims={d}")
    inp, fwd, g = _run(d, seed=S + 17 * r)
    v = {k: t.value for k, t in inp.items()}
    ref = oracle.backward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], v["d_o"], n_h=d.n_h,
                          sp_size=d.sp_size, sp_rank=d.sp_rank, d_nope=d.d_nope, eps=d.eps)
    check("dq", host(g["dq"]), ref["dq"], d.dtype)
    check("d_latent", host(g["d_latent"]), ref["d_latent"], d.dtype)
    check("dk_pe", host(g["d_k_pe"]), ref["dk_pe"], d.dtype)
    check("d_gamma", host(g["d_gamma"]), ref["d_gamma"], d.dtype)
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    dW = host(g["d_w_kv_b"])
    check("d_w_kv_b", dW[heads], ref["d_w_kv_b"][heads], d.dtype)
    others = np.ones(d.n_h, dtype=bool)
    others[heads] = False
    assert np.all(dW[others] == -7.0), "rows outside the head shard were written"


def test_training_workload_against_golden():
    assert os.path.exists(GOLDEN), "golden file missing: run tests/golden/make_train_golden.py"
    gold = np.load(GOLDEN, allow_pickle=False)
    d, _ = li.workload("v3_sp8_s16384_h16_train")
    announce(f"training workload fwd+bwd dims={d}")
    inp, fwd, g = _run(d, seed=0)
    rows = gold["rows"]
    rep = {}
    check("o[rows]", host(fwd["o"])[:, rows], gold["O"], d.dtype, rep)
    check("lse[rows]", host(fwd["lse"])[..., rows], gold["lse"], d.dtype, rep)
    check("dq[rows]", host(g["dq"])[:, rows], gold["dq"], d.dtype, rep)
    check("d_latent", host(g["d_latent"])[:, rows], gold["d_latent"], d.dtype, rep)
    check("dk_pe", host(g["d_k_pe"])[:, rows], gold["dk_pe"], d.dtype, rep)
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    dW = host(g["d_w_kv_b"])[heads].reshape(-1, d.d_kv)
    check("d_w_kv_b", dW[gold["w_rows"]], gold["d_w"], d.dtype, rep)
    check("d_gamma", host(g["d_gamma"]), gold["d_gamma"], d.dtype, rep)


def test_backward_is_deterministic():
    d = _dims(1, 500, 16, 8, 2, li.BF16)
    announce(f"backward determinism dims={d}")
    inp = li.make_inputs(d, 3, backward=True)
    x = device_inputs(inp)
    path = make_path(d, SPLIT)
    fwd = path.forward(x)
    g1 = {k: t.clone() for k, t in path.backward(x, fwd, x["d_o"]).items() if k != "workspace"}
    g2 = path.backward(x, fwd, x["d_o"])
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


@pytest.mark.parametrize("scale_exp", [-20, 12])
def test_backward_gradient_magnitude(scale_exp):
    """dO scaled by 2^scale_exp (exact in bf16): at 2^-20 its values sit deep in
    fp16's subnormal range, at 2^12 the score gradients would overflow fp16.
    The gradients are linear in dO, so both sides are divided by the scale and
    held to the usual bars, i.e. the same relative accuracy as at unit scale."""
    d = _dims(1, 300, 16, 8, 3, li.BF16)
    announce(f"backward with dO * 2^{scale_exp} dims={d}")
    inp = li.make_inputs(d, 29, backward=True)
    x = device_inputs(inp)
    sc = 2.0 ** scale_exp
    x["d_o"] = (x["d_o"].float() * sc).to(torch.bfloat16)
    path = make_path(d, SPLIT)
    fwd = path.forward(x)
    g = path.backward(x, fwd, x["d_o"])
    torch.cuda.synchronize()
    v = {k: t.value for k, t in inp.items()}
    assert np.array_equal(host(x["d_o"]), v["d_o"] * sc), "scaling dO by a power of two must be exact"
    ref = oracle.backward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], v["d_o"] * sc, n_h=d.n_h,
                          sp_size=d.sp_size, sp_rank=d.sp_rank, d_nope=d.d_nope, eps=d.eps)
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    check("dq/s", host(g["dq"]) / sc, ref["dq"] / sc, d.dtype)
    check("d_latent/s", host(g["d_latent"]) / sc, ref["d_latent"] / sc, d.dtype)
    check("dk_pe/s", host(g["d_k_pe"]) / sc, ref["dk_pe"] / sc, d.dtype)
    check("d_gamma/s", host(g["d_gamma"]) / sc, ref["d_gamma"] / sc, d.dtype)
    check("d_w/s", host(g["d_w_kv_b"])[heads] / sc, ref["d_w_kv_b"][heads] / sc, d.dtype)


def test_backward_row_varying_gradient_magnitude():
    """dO of every odd token scaled by 2^-16 (exact in bf16), the even tokens
    at unit scale: the global dO scale is set by the large rows, so without a
    per-row scale the small rows' score gradients would sit in fp16's
    subnormal range and their dq would lose most of its relative precision.
    dq of a token is linear in that token's dO row, so each dq row is divided
    by its own factor and held to the usual bars (relative accuracy per row);
    the gradients that sum over queries are held to the bars as they are."""
    d = _dims(1, 300, 16, 8, 3, li.BF16)
    announce(f"backward with row-varying dO magnitudes dims={d}")
    inp = li.make_inputs(d, 31, backward=True)
    x = device_inputs(inp)
    rs = np.ones(d.S)
    rs[1::2] = 2.0 ** -16
    rst = torch.tensor(rs, dtype=torch.float32, device=x["d_o"].device)[None, :, None, None]
    x["d_o"] = (x["d_o"].float() * rst).to(torch.bfloat16)
    path = make_path(d, SPLIT)
    fwd = path.forward(x)
    g = path.backward(x, fwd, x["d_o"])
    torch.cuda.synchronize()
    v = {k: t.value for k, t in inp.items()}
    d_o = v["d_o"] * rs[None, :, None, None]
    assert np.array_equal(host(x["d_o"]), d_o), "scaling dO rows by powers of two must be exact"
    ref = oracle.backward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], d_o, n_h=d.n_h,
                          sp_size=d.sp_size, sp_rank=d.sp_rank, d_nope=d.d_nope, eps=d.eps)
    per_row = rs[None, :, None, None]
    check("dq/s_t", host(g["dq"]) / per_row, ref["dq"] / per_row, d.dtype)
    check("d_latent", host(g["d_latent"]), ref["d_latent"], d.dtype)
    check("dk_pe", host(g["d_k_pe"]), ref["dk_pe"], d.dtype)
    check("d_gamma", host(g["d_gamma"]), ref["d_gamma"], d.dtype)
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    check("d_w_kv_b", host(g["d_w_kv_b"])[heads], ref["d_w_kv_b"][heads], d.dtype)
