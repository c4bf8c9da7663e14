"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties one oracle function to an independent fact: a pure-Python brute
force on tiny inputs, torch's fp64 library routines (rms_norm, linear,
scaled_dot_product_attention, autograd), central finite differences, the
absorbed-form identity of the LAGA paper (§2.3, §3.2), closed forms, softmax
normalisation, causality and the head-shard equivalence of §5.1.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(1234)


def tiny(S=5, n_h=4, sp_size=2, sp_rank=1, d_kv=5, d_nope=4, d_rope=2, d_v=3, B=1,
         seed=0, d_o=True):
    rng = np.random.default_rng(seed)
    h = n_h // sp_size
    d = dict(
        q=rng.standard_normal((B, S, h, d_nope + d_rope)),
        latent=rng.standard_normal((B, S, d_kv)),
        k_pe=rng.standard_normal((B, S, d_rope)),
        w_kv_b=rng.standard_normal((n_h, d_nope + d_v, d_kv)) / math.sqrt(d_kv),
        gamma=1.0 + 0.1 * rng.standard_normal(d_kv),
    )
    if d_o:
        d["d_o"] = rng.standard_normal((B, S, h, d_v))
    kw = dict(n_h=n_h, sp_size=sp_size, sp_rank=sp_rank, d_nope=d_nope)
    return d, kw


def fwd(d, kw):
    return oracle.forward(d["q"], d["latent"], d["k_pe"], d["w_kv_b"], d["gamma"], **kw)


def bwd(d, kw):
    return oracle.backward(d["q"], d["latent"], d["k_pe"], d["w_kv_b"], d["gamma"], d["d_o"], **kw)


# ---------------------------------------------------------------- brute force
def brute_forward(d, kw, eps=1e-6):
    """Loop-only forward in plain Python floats."""
    q, x, kpe, W, g = d["q"], d["latent"], d["k_pe"], d["w_kv_b"], d["gamma"]
    B, S, h, dqk = q.shape
    d_kv = x.shape[-1]
    dn = kw["d_nope"]
    dv = W.shape[1] - dn
    r0 = kw["sp_rank"] * h
    L = [[[0.0] * d_kv for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for t in range(S):
            ms = sum(float(x[b, t, j]) ** 2 for j in range(d_kv)) / d_kv
            r = 1.0 / math.sqrt(ms + eps)
            for j in range(d_kv):
                L[b][t][j] = float(g[j]) * float(x[b, t, j]) * r
    kn = np.zeros((B, S, h, dn))
    vv = np.zeros((B, S, h, dv))
    for b in range(B):
        for t in range(S):
            for i in range(h):
                for c in range(dn + dv):
                    acc = 0.0
                    for j in range(d_kv):
                        acc += float(W[r0 + i, c, j]) * L[b][t][j]
                    if c < dn:
                        kn[b, t, i, c] = acc
                    else:
                        vv[b, t, i, c - dn] = acc
    O = np.zeros((B, S, h, dv))
    lse = np.zeros((B, h, S))
    for b in range(B):
        for i in range(h):
            for t in range(S):
                sc = []
                for u in range(t + 1):
                    acc = 0.0
                    for c in range(dqk):
                        kc = kn[b, u, i, c] if c < dn else float(kpe[b, u, c - dn])
                        acc += float(q[b, t, i, c]) * kc
                    sc.append(acc / math.sqrt(dqk))
                m = max(sc)
                ex = [math.exp(s - m) for s in sc]
                tot = sum(ex)
                lse[b, i, t] = m + math.log(tot)
                for c in range(dv):
                    O[b, t, i, c] = sum(ex[u] / tot * vv[b, u, i, c] for u in range(t + 1))
    return dict(L=np.array(L), k_nope=kn, v=vv, O=O, lse=lse)


@pytest.mark.parametrize("seed,B", [(0, 1), (1, 2)])
def test_brute_force_forward(seed, B):
    d, kw = tiny(S=6, B=B, seed=seed)
    got = fwd(d, kw)
    ref = brute_forward(d, kw)
    for k in ("L", "k_nope", "v", "O", "lse"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-12, err_msg=k)


# --------------------------------------------------------- library routines
def torch_forward(d, kw, requires_grad=False):
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=requires_grad) for k, v in d.items()}
    h = d["q"].shape[2]
    dn = kw["d_nope"]
    r0 = kw["sp_rank"] * h
    L = torch.nn.functional.rms_norm(t["latent"], (t["latent"].shape[-1],), t["gamma"], eps=1e-6)
    W = t["w_kv_b"][r0:r0 + h]                                   # [h, dn+dv, d_kv]
    kv = torch.nn.functional.linear(L, W.reshape(-1, W.shape[-1]))  # [B,S,h*(dn+dv)]
    kv = kv.reshape(*L.shape[:2], h, W.shape[1])
    k_nope, v = kv[..., :dn], kv[..., dn:]
    k = torch.cat([k_nope, t["k_pe"][:, :, None, :].expand(-1, -1, h, -1)], dim=-1)
    qq = t["q"].transpose(1, 2)
    O = torch.nn.functional.scaled_dot_product_attention(
        qq, k.transpose(1, 2), v.transpose(1, 2), is_causal=True,
        scale=1.0 / math.sqrt(d["q"].shape[-1]))
    return t, L, k_nope, v, O.transpose(1, 2)


def test_library_forward():
    d, kw = tiny(S=9, n_h=6, sp_size=3, sp_rank=2, d_kv=7, d_nope=5, d_rope=3, d_v=4, B=2)
    got = fwd(d, kw)
    _, L, kn, v, O = torch_forward(d, kw)
    np.testing.assert_allclose(got["L"], L.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["k_nope"], kn.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["v"], v.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["O"], O.numpy(), rtol=1e-11, atol=1e-13)


def test_library_backward():
    d, kw = tiny(S=8, n_h=6, sp_size=3, sp_rank=1, d_kv=7, d_nope=5, d_rope=3, d_v=4, B=2)
    got = bwd(d, kw)
    t, _, _, _, O = torch_forward({k: v for k, v in d.items() if k != "d_o"}, kw,
                                  requires_grad=True)
    (O * torch.tensor(d["d_o"])).sum().backward()
    np.testing.assert_allclose(got["dq"], t["q"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_latent"], t["latent"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dk_pe"], t["k_pe"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_w_kv_b"], t["w_kv_b"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["d_gamma"], t["gamma"].grad.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------- finite differences
def loss(d, kw):
    return float(np.sum(fwd(d, kw)["O"] * d["d_o"]))


@pytest.mark.parametrize("name,key", [("q", "dq"), ("latent", "d_latent"), ("k_pe", "dk_pe"),
                                      ("w_kv_b", "d_w_kv_b"), ("gamma", "d_gamma")])
def test_finite_differences(name, key):
    d, kw = tiny(S=5, seed=3)
    g = bwd(d, kw)[key]
    hstep = 1e-5
    fd = np.zeros_like(d[name])
    it = np.nditer(d[name], flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        dp = {k: v.copy() for k, v in d.items()}
        dm = {k: v.copy() for k, v in d.items()}
        dp[name][idx] += hstep
        dm[name][idx] -= hstep
        fd[idx] = (loss(dp, kw) - loss(dm, kw)) / (2 * hstep)
    scale = max(1.0, np.max(np.abs(fd)))
    assert np.max(np.abs(fd - g)) <= 1e-7 * scale, (name, np.max(np.abs(fd - g)))


def test_dw_outside_shard_is_zero():
    d, kw = tiny(S=4)
    dW = bwd(d, kw)["d_w_kv_b"]
    h = d["q"].shape[2]
    r0 = kw["sp_rank"] * h
    mask = np.ones(dW.shape[0], dtype=bool)
    mask[r0:r0 + h] = False
    assert np.all(dW[mask] == 0.0)
    assert np.all(np.any(dW[~mask] != 0.0, axis=(1, 2)))


# ------------------------------------------------------- absorbed-form identity
def test_absorbed_identity():
    d, kw = tiny(S=7, n_h=4, sp_size=2, sp_rank=0, d_kv=6, d_nope=5, d_rope=3, d_v=4, B=2)
    f = fwd(d, kw)
    heads = oracle.head_shard(kw["n_h"], kw["sp_size"], kw["sp_rank"])
    s_abs, O_abs = oracle.absorbed_scores_and_out(d["q"], f["L"], d["k_pe"], d["w_kv_b"],
                                                  heads, kw["d_nope"])
    s_exp = oracle.explicit_scores(d["q"], f["k_nope"], d["k_pe"])
    fin = np.isfinite(s_exp)
    assert np.array_equal(fin, np.isfinite(s_abs))
    np.testing.assert_allclose(s_abs[fin], s_exp[fin], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(O_abs, f["O"], rtol=1e-10, atol=1e-12)


def test_absorbed_forward_matches_explicit_and_definitions():
    """B2's forward (with its intermediates) against the explicit forward, which
    the absorbed identity equates, and against the intermediates' definitions."""
    d, kw = tiny(S=9, n_h=6, sp_size=3, sp_rank=2, d_kv=7, d_nope=4, d_rope=3, d_v=5, B=2, seed=3)
    f = fwd(d, kw)
    heads = oracle.head_shard(kw["n_h"], kw["sp_size"], kw["sp_rank"])
    rows = np.arange(9)
    q_abs, acc, O, lse = oracle.absorbed_forward_rows(d["q"], f["L"], d["k_pe"], d["w_kv_b"], heads,
                                                      kw["d_nope"], rows)
    np.testing.assert_allclose(O, f["O"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, f["lse"], rtol=1e-12, atol=1e-12)
    # q_abs against its contraction written as plain loops, and the un-absorb
    # O[t,i,j] = sum_c W[h_i, d_nope + j, c] acc[t,i,c] likewise.
    W = d["w_kv_b"]
    for b in range(2):
        for t in (0, 4, 8):
            for i, hg in enumerate(heads):
                for c in range(7):
                    ref = sum(d["q"][b, t, i, n] * W[hg, n, c] for n in range(4))
                    assert abs(q_abs[b, t, i, c] - ref) < 1e-12
                for j in range(5):
                    ref = sum(W[hg, 4 + j, c] * acc[b, t, i, c] for c in range(7))
                    assert abs(O[b, t, i, j] - ref) < 1e-12
    # the first query attends only to key 0: acc = L[0]
    np.testing.assert_allclose(acc[:, 0], np.broadcast_to(f["L"][:, 0, None, :], acc[:, 0].shape), rtol=0,
                               atol=1e-13)


@pytest.mark.parametrize("shape", [
    dict(S=7, n_h=4, sp_size=2, sp_rank=0, d_kv=6, d_nope=5, d_rope=3, d_v=4, B=2, seed=1),
    dict(S=1, n_h=2, sp_size=1, sp_rank=0, d_kv=5, d_nope=4, d_rope=2, d_v=3, B=1, seed=2),
    dict(S=10, n_h=6, sp_size=3, sp_rank=2, d_kv=7, d_nope=4, d_rope=3, d_v=5, B=1, seed=4)])
def test_absorbed_backward_matches_explicit(shape):
    """B2's backward, taken through its own steps, equals the explicit backward
    (pinned by finite differences and autograd above): the two forms are one
    function, so every gradient agrees to rounding."""
    d, kw = tiny(**shape)
    ref = bwd(d, kw)
    got = oracle.absorbed_backward(d["q"], d["latent"], d["k_pe"], d["w_kv_b"], d["gamma"], d["d_o"], **kw)
    for key in ("dq", "dk_pe", "dL", "d_latent", "d_w_kv_b", "d_gamma"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-10, atol=1e-12, err_msg=key)


def test_absorbed_backward_intermediates():
    """d_acc against its contraction written as loops; d_q_abs against central
    differences of the loss with q_abs as a free input of the latent attention."""
    d, kw = tiny(S=4, n_h=2, sp_size=1, sp_rank=0, d_kv=3, d_nope=2, d_rope=2, d_v=2, B=1, seed=5)
    g = oracle.absorbed_backward(d["q"], d["latent"], d["k_pe"], d["w_kv_b"], d["gamma"], d["d_o"], **kw)
    W = d["w_kv_b"]
    for t in range(4):
        for i in range(2):
            for c in range(3):
                ref = sum(d["d_o"][0, t, i, j] * W[i, 2 + j, c] for j in range(2))
                assert abs(g["d_acc"][0, t, i, c] - ref) < 1e-12
    L, _ = oracle.latent_rmsnorm(d["latent"], d["gamma"])

    def loss_from_q_abs(qa, i):
        s = (qa @ L[0].T + d["q"][0, :, i, 2:] @ d["k_pe"][0].T) / math.sqrt(4)
        s = np.where(np.tril(np.ones((4, 4), dtype=bool)), s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return float(np.sum(d["d_o"][0, :, i] * ((p @ L[0]) @ W[i, 2:].T)))

    for i in range(2):
        qa = d["q"][0, :, i, :2] @ W[i, :2]
        for t in range(4):
            for c in range(3):
                qp, qm = qa.copy(), qa.copy()
                qp[t, c] += 1e-6
                qm[t, c] -= 1e-6
                fd = (loss_from_q_abs(qp, i) - loss_from_q_abs(qm, i)) / 2e-6
                assert abs(fd - g["d_q_abs"][0, t, i, c]) < 1e-7


# ------------------------------------------------------------ softmax and lse
def test_softmax_rows_sum_to_one():
    d, kw = tiny(S=11, d_kv=6)
    f = fwd(d, kw)
    s = oracle.explicit_scores(d["q"], f["k_nope"], d["k_pe"])
    p = np.exp(s - f["lse"][..., None])
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    # strictly-upper entries carry no probability
    assert np.all(p[..., np.triu_indices(11, 1)[0], np.triu_indices(11, 1)[1]] == 0.0)


# ------------------------------------------------------------------ causality
def test_causality_forward_and_backward():
    d, kw = tiny(S=9, seed=5)
    t = 4
    base = fwd(d, kw)
    pert = {k: v.copy() for k, v in d.items()}
    pert["q"][:, t + 1:] += 3.0
    pert["latent"][:, t + 1:] *= -2.0
    pert["k_pe"][:, t + 1:] += 1.5
    p = fwd(pert, kw)
    np.testing.assert_array_equal(p["O"][:, :t + 1], base["O"][:, :t + 1])
    np.testing.assert_array_equal(p["lse"][..., :t + 1], base["lse"][..., :t + 1])
    # <dO[<=t], O[<=t]>: zero upstream gradient after t -> the truncated problem
    dz = {k: v.copy() for k, v in d.items()}
    dz["d_o"][:, t + 1:] = 0.0
    g = bwd(dz, kw)
    tr = {k: (v[:, :t + 1] if k in ("q", "latent", "k_pe", "d_o") else v) for k, v in d.items()}
    gt = bwd(tr, kw)
    for k in ("dq", "d_latent", "dk_pe"):
        assert np.all(g[k][:, t + 1:] == 0.0), k
        np.testing.assert_allclose(g[k][:, :t + 1], gt[k], rtol=1e-12, atol=1e-14)
    for k in ("d_w_kv_b", "d_gamma"):
        np.testing.assert_allclose(g[k], gt[k], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------- closed forms
def test_single_token_closed_form():
    d, kw = tiny(S=1, seed=7)
    f = fwd(d, kw)
    g = bwd(d, kw)
    np.testing.assert_array_equal(f["O"], f["v"])            # one key: p = 1
    np.testing.assert_allclose(f["lse"], oracle.explicit_scores(d["q"], f["k_nope"], d["k_pe"])[..., 0])
    assert np.all(np.abs(g["dq"]) < 1e-15)
    assert np.all(np.abs(g["dk_nope"]) < 1e-15)
    assert np.all(np.abs(g["dk_pe"]) < 1e-15)
    np.testing.assert_allclose(g["dv"], d["d_o"], rtol=0, atol=1e-15)


def test_zero_query_is_prefix_mean():
    d, kw = tiny(S=8, seed=8)
    d["q"][:] = 0.0
    f = fwd(d, kw)
    S = d["q"].shape[1]
    cum = np.cumsum(f["v"], axis=1) / np.arange(1, S + 1)[None, :, None, None]
    np.testing.assert_allclose(f["O"], cum, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(f["lse"], np.broadcast_to(np.log(np.arange(1, S + 1)), f["lse"].shape),
                               rtol=1e-14, atol=1e-15)


def test_rmsnorm_closed_forms():
    d_kv = 16
    gamma = 1.0 + 0.1 * RNG.standard_normal(d_kv)
    c = 0.37
    L, r = oracle.latent_rmsnorm(np.full((1, 1, d_kv), c), gamma)
    np.testing.assert_allclose(L[0, 0], gamma * c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    np.testing.assert_allclose(r[0, 0], 1.0 / math.sqrt(c * c + 1e-6), rtol=1e-15)
    # scale invariance up to the eps term
    x = RNG.standard_normal((2, 3, d_kv))
    L1, _ = oracle.latent_rmsnorm(x, gamma, eps=0.0)
    L2, _ = oracle.latent_rmsnorm(x * 123.0, gamma, eps=0.0)
    np.testing.assert_allclose(L1, L2, rtol=1e-13)
    # sum_j x_j dx_j = r (g.x) eps / (ms + eps) with g = gamma * dL
    dL = RNG.standard_normal(x.shape)
    eps = 1e-2
    _, rstd = oracle.latent_rmsnorm(x, gamma, eps)
    dx, dgamma = oracle.latent_rmsnorm_bwd(dL, x, gamma, rstd)
    ms = np.mean(x * x, -1)
    want = rstd * np.sum(gamma * dL * x, -1) * eps / (ms + eps)
    np.testing.assert_allclose(np.sum(x * dx, -1), want, rtol=1e-10, atol=1e-13)
    # dgamma is the sum over tokens of dL * x_hat
    np.testing.assert_allclose(dgamma, np.einsum("bsj,bsj->j", dL, x * rstd[..., None]), rtol=1e-13)


# ------------------------------------------- head-shard equivalence (§5.1)
@pytest.mark.parametrize("P", [2, 4])
def test_shard_consistency(P):
    n_h = 4
    d1, kw1 = tiny(S=6, n_h=n_h, sp_size=1, sp_rank=0, seed=11)
    full = bwd(d1, kw1)
    ffwd = fwd(d1, kw1)
    h = n_h // P
    Os, dqs, dws = [], [], np.zeros_like(full["d_w_kv_b"])
    dlat, dkpe, dgam = 0.0, 0.0, 0.0
    for r in range(P):
        dr = dict(d1)
        dr["q"] = d1["q"][:, :, r * h:(r + 1) * h]
        dr["d_o"] = d1["d_o"][:, :, r * h:(r + 1) * h]
        kw = dict(kw1, sp_size=P, sp_rank=r)
        Os.append(fwd(dr, kw)["O"])
        g = bwd(dr, kw)
        dqs.append(g["dq"])
        dws += g["d_w_kv_b"]
        dlat = dlat + g["d_latent"]
        dkpe = dkpe + g["dk_pe"]
        dgam = dgam + g["d_gamma"]
    np.testing.assert_allclose(np.concatenate(Os, axis=2), ffwd["O"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(np.concatenate(dqs, axis=2), full["dq"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dws, full["d_w_kv_b"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dlat, full["d_latent"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dkpe, full["dk_pe"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dgam, full["d_gamma"], rtol=1e-12, atol=1e-14)


def test_row_sampled_forward_matches_full():
    d, kw = tiny(S=13, seed=9)
    f = fwd(d, kw)
    rows = [0, 5, 12]
    O, lse = oracle.attention_fwd_rows(d["q"], f["k_nope"], d["k_pe"], f["v"], rows)
    np.testing.assert_allclose(O, f["O"][:, rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, f["lse"][..., rows], rtol=1e-12, atol=1e-14)


def test_head_shard_rejects_bad_split():
    with pytest.raises(ValueError):
        oracle.head_shard(6, 4, 0)
    with pytest.raises(ValueError):
        oracle.head_shard(8, 4, 4)
