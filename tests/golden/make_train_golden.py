"""Write the sampled fp64 oracle values of the full-size training workload.

Workload: B=1, S=16384, h=16 local heads (n_h=128, SP=8, rank 0), DeepSeek-V3
dims (d_kv=512, d_nope=d_v=128, d_rope=64), bf16 inputs, seed 0, forward and
backward of sum(d_o * o).  The oracle runs the whole computation in fp64 (a
few minutes on 8 cores); only sampled entries are stored:
  rows            sampled query / token positions
  O, lse          forward output and log-sum-exp at `rows`
  dq, d_latent, dk_pe   gradients at `rows`
  w_rows, d_w     every 16th row of this shard's [h*(d_nope+d_v), d_kv] W_kv_b gradient
  d_gamma         the whole gamma gradient
Calls only oracle/ and laga_inputs.  Usage: python tests/golden/make_train_golden.py
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import laga_inputs as li  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(HERE, "train_v3_sp8_s16384_h16.npz")


def sample_rows(S, n=40, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, S // 2, S - 2, S - 1]
    rows = set(t for t in fixed if 0 <= t < S)
    rows.update(int(t) for t in rng.integers(0, S, size=n))
    return np.array(sorted(rows))


def main():
    d, _ = li.workload("v3_sp8_s16384_h16_train")
    inp = li.make_inputs(d, 0, backward=True)
    v = {k: t.value for k, t in inp.items()}
    kw = dict(n_h=d.n_h, sp_size=d.sp_size, sp_rank=d.sp_rank, d_nope=d.d_nope, eps=d.eps)
    t0 = time.time()
    f = oracle.forward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], **kw)
    print(f"forward {time.time() - t0:.1f}s", flush=True)
    g = oracle.backward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], v["d_o"], fwd=f, **kw)
    print(f"backward {time.time() - t0:.1f}s", flush=True)
    rows = sample_rows(d.S)
    heads = oracle.head_shard(d.n_h, d.sp_size, d.sp_rank)
    dW = g["d_w_kv_b"][heads].reshape(-1, d.d_kv)
    w_rows = np.arange(0, dW.shape[0], 16)
    np.savez_compressed(
        OUT, rows=rows, O=f["O"][:, rows], lse=f["lse"][..., rows], dq=g["dq"][:, rows],
        d_latent=g["d_latent"][:, rows], dk_pe=g["dk_pe"][:, rows], w_rows=w_rows, d_w=dW[w_rows],
        d_gamma=g["d_gamma"])
    print(f"wrote {OUT} ({os.path.getsize(OUT) / 1e6:.2f} MB)")


if __name__ == "__main__":
    main()
