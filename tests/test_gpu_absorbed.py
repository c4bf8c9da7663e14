"""Absorbed-form (B2) forward against the fp64 oracle (needs an MI355X).

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
                                         (1, 64, 128, 16, 2), (1, 97, 128, 1, 0), (1, 1000, 16, 8, 2)])
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
