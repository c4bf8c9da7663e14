"""Absorbed-form (B2) forward and backward against the fp64 oracle (needs an MI355X).

B2 is the pages' inference-side reformulation ported to training [LAGA §3.2
(B2)]: the outputs (o, lse) equal the explicit form's, and the two
n_h*d_kv-wide intermediates (the absorbed query q_abs and the latent
accumulator acc) are checked against their definitions in the oracle.  Small
shapes compare every row; the full-size workload compares sampled query rows.
"""
import numpy as np
import pytest
import torch

import laga_inputs as li
import oracle
from gpu_util import FP16, announce, check, device_inputs, host, make_path, sample_rows
from head_latent_attention_laga_amd import _lib

pytestmark = pytest.mark.gpu


def _run(d: li.Dims, seed: int):
    inp = li.make_inputs(d, seed)
    x = device_inputs(inp)
    path = make_path(d, FP16)
    out = path.alloc_absorbed()
    for k in ("q_abs", "acc", "o", "lse"):
        out[k].fill_(float("nan"))
    path.absorbed_forward(x, out)
    torch.cuda.synchronize()
    return inp, out


def _compare(d: li.Dims, inp, out, rows):
    v = {k: t.value for k, t in inp.items()}
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    L, _ = oracle.latent_rmsnorm(v["latent"], v["gamma"], d.eps)
    q_abs, acc, O, lse = oracle.absorbed_forward_rows(v["q"], L, v["k_pe"], v["w_kv_b"], heads, d.d_nope, rows)
    check("q_abs", host(out["q_abs"])[:, rows], q_abs, d.dtype)
    check("acc", host(out["acc"])[:, rows], acc, d.dtype)
    check("o", host(out["o"])[:, rows], O, d.dtype)
    check("lse", host(out["lse"])[..., rows], lse, d.dtype)


@pytest.mark.parametrize("B,S,n_h,P,r", [(1, 300, 16, 8, 3), (2, 130, 64, 8, 7), (1, 1, 16, 8, 0),
                                         (1, 64, 128, 16, 2), (1, 97, 128, 1, 0), (1, 1000, 16, 8, 2),
                                         (1, 150, 15, 5, 2), (2, 97, 5, 1, 0)])
def test_absorbed_forward_shapes(B, S, n_h, P, r):
    d = li.Dims(B=B, S=S, n_h=n_h, sp_size=P, sp_rank=r, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                dtype=li.BF16)
    announce(f"absorbed forward dims={d}")
    inp, out = _run(d, seed=S + 3 * P)
    _compare(d, inp, out, np.arange(S))


def test_absorbed_forward_full_size():
    d, _ = li.workload("v3_sp8_s16384_h16")
    announce(f"absorbed forward full size dims={d}")
    inp, out = _run(d, seed=0)
    _compare(d, inp, out, sample_rows(d.S))


def test_absorbed_matches_laga_forward():
    """Both forms compute the same o from the same inputs [LAGA §3.2]: the
    absorbed path against LAGA's fp16-operand path on one workload."""
    d = li.Dims(B=1, S=700, n_h=128, sp_size=8, sp_rank=5, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                dtype=li.BF16)
    announce(f"absorbed vs LAGA dims={d}")
    inp, out = _run(d, seed=41)
    x = device_inputs(inp)
    lg = make_path(d, FP16).forward(x)
    torch.cuda.synchronize()
    check("o B2-LAGA", host(out["o"]), host(lg["o"]), d.dtype)
    check("lse B2-LAGA", host(out["lse"]), host(lg["lse"]), d.dtype)


def test_absorbed_forward_is_deterministic():
    """Two runs on the same inputs give bit-identical q_abs, kx, acc, o and lse
    (no atomics, fixed reduction orders).  A race between the key-block loads
    and the LDS reads of the latent-attention kernel would show up here as a
    run-to-run difference, even where it stays within the parity bars."""
    d = li.Dims(B=1, S=1000, n_h=128, sp_size=8, sp_rank=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                dtype=li.BF16)
    announce(f"absorbed forward determinism dims={d}")
    inp = li.make_inputs(d, 5)
    x = device_inputs(inp)
    path = make_path(d, FP16)
    a = path.absorbed_forward(x)
    first = {k: t.clone() for k, t in a.items()}
    for _ in range(3):
        b = path.absorbed_forward(x)
        torch.cuda.synchronize()
        for k in first:
            assert torch.equal(first[k], b[k]), k


# ------------------------------------------------------------------ backward
def _b2_step(d: li.Dims, seed: int, workspace: str = "default"):
    inp = li.make_inputs(d, seed, backward=True)
    x = device_inputs(inp)
    path = make_path(d, FP16)
    absf = path.absorbed_forward(x)
    full = _lib.absorbed_bwd_workspace_bytes(path.dims)
    least = _lib.absorbed_bwd_min_workspace_bytes(path.dims)
    ws = {"default": full, "min": least, "mid": (full + least) // 2}[workspace]
    g = path.alloc_backward(workspace_bytes=ws)
    for k in ("dq", "d_latent", "d_k_pe", "d_gamma"):
        g[k].fill_(float("nan"))
    g["d_w_kv_b"].fill_(-7.0)  # rows outside this rank's shard must stay untouched
    path.absorbed_backward(x, absf, x["d_o"], g)
    torch.cuda.synchronize()
    return inp, path, x, absf, g


@pytest.mark.parametrize("B,S,n_h,P,r,ws", [(1, 300, 16, 8, 3, "default"), (2, 130, 64, 8, 7, "default"),
                                            (1, 1, 16, 8, 0, "default"), (1, 257, 128, 32, 5, "default"),
                                            (1, 1000, 16, 8, 2, "default"), (1, 1000, 16, 8, 2, "min"),
                                            (2, 300, 16, 8, 5, "min"), (1, 1000, 16, 8, 4, "mid"),
                                            (1, 150, 15, 5, 2, "default"), (2, 97, 5, 1, 0, "min")])
def test_absorbed_backward_shapes(B, S, n_h, P, r, ws):
    """Every gradient against the oracle's B2 backward (itself equal to the explicit
    backward).  ws: the workspace passed; "min" runs 32-token chunks of query rows
    (32 chunks at S=1000, 10 per sequence at S=300), "mid" a size in between."""
    d = li.Dims(B=B, S=S, n_h=n_h, sp_size=P, sp_rank=r, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                dtype=li.BF16)
    announce(f"absorbed backward dims={d} workspace={ws}")
    inp, _, _, _, g = _b2_step(d, seed=S + 11 * r, workspace=ws)
    v = {k: t.value for k, t in inp.items()}
    ref = oracle.absorbed_backward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], v["d_o"], n_h=d.n_h,
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


def test_absorbed_backward_training_workload_against_golden():
    """S=16384, 16 local heads: the query rows run in many chunks; sampled rows of
    dq, d_latent, dk_pe and sampled rows of dW, and all of dgamma, against the
    fp64 oracle's values for this workload (tests/golden)."""
    import os
    gold = np.load(os.path.join(os.path.dirname(__file__), "golden", "train_v3_sp8_s16384_h16.npz"),
                   allow_pickle=False)
    d, _ = li.workload("v3_sp8_s16384_h16_train")
    announce(f"absorbed backward, training workload dims={d}")
    _, path, _, _, g = _b2_step(d, seed=0)
    rows = gold["rows"]
    check("dq[rows]", host(g["dq"])[:, rows], gold["dq"], d.dtype)
    check("d_latent", host(g["d_latent"])[:, rows], gold["d_latent"], d.dtype)
    check("dk_pe", host(g["d_k_pe"])[:, rows], gold["dk_pe"], d.dtype)
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    dW = host(g["d_w_kv_b"])[heads].reshape(-1, d.d_kv)
    check("d_w_kv_b", dW[gold["w_rows"]], gold["d_w"], d.dtype)
    check("d_gamma", host(g["d_gamma"]), gold["d_gamma"], d.dtype)


def test_absorbed_backward_is_deterministic():
    d = li.Dims(B=1, S=700, n_h=16, sp_size=8, sp_rank=1, d_kv=512, d_nope=128, d_rope=64, d_v=128, dtype=li.BF16)
    announce(f"absorbed backward determinism dims={d}")
    _, path, x, absf, g = _b2_step(d, seed=9)
    first = {k: t.clone() for k, t in g.items() if k != "workspace"}
    for _ in range(2):
        path.absorbed_backward(x, absf, x["d_o"], g)
        torch.cuda.synchronize()
        for k in first:
            assert torch.equal(first[k], g[k]), k
