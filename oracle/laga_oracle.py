"""fp64 CPU oracle of the LAGA per-rank attention path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the product path never does.

Source: "A Training-Memory Regression in MLA Sequence Parallelism: Why
Megatron-Core Forbids Absorption, and LAGA -- a Communication-Efficient Fix"
(arXiv 2607.17644v1), cited as [LAGA §...].  The rank-local computation of LAGA
is the explicit MLA attention of §2.1 restricted to the rank's head shard H_r
(§3.3, Algorithm 1; §5.1 per-head form).  §5.1 Propositions 1 and 2 state that
this equals the explicit form, so the oracle is the plain definition written
out in NumPy float64, one head at a time, with no blocking or fusion.

Readings where the paper is silent or garbled:
  * Score formula: §2.1 prints q_nope on the key side; §3.3 Algorithm 1 and
    §5.3 use (k_nope || k_pe).  The key side is (k_nope || k_pe).
  * Scale 1/sqrt(d): d is the per-head q.k width d_nope + d_rope (192 at V3
    dims, matching "D_q = D_k = 192" in §4.6), not d_model.
  * "LN"/"LayerNorm" of the latent: RMS form over d_kv, eps 1e-6 inside the
    square root, learned gamma, no bias and no mean subtraction.
  * Mask: causal over global positions, key u <= query t, square S x S.
  * RoPE itself is upstream: q_rope and k_pe arrive already rotated.
  * w_kv_b layout: [n_h, d_nope + d_v, d_kv], per head the d_nope K rows then
    the d_v V rows ("(k_nope, v) = split(kv)" in §2.1).
  * No dropout, bias, softcap or window.
  * Backward (§5.2): gradients of this rank's share; dk_pe is the sum over the
    local heads of the broadcast band's gradient, dLatent is with respect to
    the pre-norm gathered latent, dW_kv_b covers the rows of H_r only.  The
    cross-rank sums (reduce-scatter, all-reduce) are outside this path.

Pins (tests/test_oracle_pins.py): pure-Python brute force on tiny inputs,
torch's fp64 rms_norm / linear / scaled_dot_product_attention and autograd as
independent library routines, central finite differences for every gradient,
the absorbed-form identity of §2.3/§3.2, softmax rows summing to one,
causality, closed forms at S=1 and q=0, and head-shard consistency (§5.1).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# O1: latent RMSNorm  [LAGA §2.1 kv = W_kv_b LN(latent); §3.3 Algorithm 1 norm]
# ----------------------------------------------------------------------------
def latent_rmsnorm(latent: np.ndarray, gamma: np.ndarray, eps: float = 1e-6):
    """L = gamma * x / sqrt(mean_j x_j^2 + eps), per token over d_kv.

    Returns (L [..., d_kv], rstd [...]) with rstd = 1/sqrt(mean x^2 + eps).
    """
    x = np.asarray(latent, dtype=np.float64)
    ms = np.mean(x * x, axis=-1)
    rstd = 1.0 / np.sqrt(ms + eps)
    L = np.asarray(gamma, dtype=np.float64) * (x * rstd[..., None])
    return L, rstd


def head_shard(n_h: int, sp_size: int, sp_rank: int) -> np.ndarray:
    """H_r = {r n_h/P, ..., (r+1) n_h/P - 1}  [LAGA §3.3 Algorithm 1 input]."""
    if n_h % sp_size != 0 or not 0 <= sp_rank < sp_size:
        raise ValueError("head shard needs n_h % P == 0 and 0 <= r < P")
    h = n_h // sp_size
    return np.arange(sp_rank * h, (sp_rank + 1) * h)


# ----------------------------------------------------------------------------
# O2: head-shard up-projection  [LAGA §3.3 Algorithm 1 local up-projection;
#     §5.1 k_nope[i,t] = W^k[i] L[t], v[i,t] = W^v[i] L[t]]
# ----------------------------------------------------------------------------
def kv_up(L: np.ndarray, w_kv_b: np.ndarray, heads: np.ndarray, d_nope: int):
    """k_nope[b,t,i,:] = W^k[H_r[i]] L[b,t];  v[b,t,i,:] = W^v[H_r[i]] L[b,t].

    L [B,S,d_kv], w_kv_b [n_h, d_nope+d_v, d_kv] -> k_nope [B,S,h,d_nope], v [B,S,h,d_v].
    """
    W = np.asarray(w_kv_b, dtype=np.float64)[heads]          # [h, d_nope+d_v, d_kv]
    B, S, _ = L.shape
    h = len(heads)
    kv = np.empty((B, S, h, W.shape[1]))
    for i in range(h):
        kv[:, :, i, :] = L @ W[i].T                           # per head: W[i] L[t]
    return kv[..., :d_nope].copy(), kv[..., d_nope:].copy()


# ----------------------------------------------------------------------------
# O3-O6: causal attention forward  [LAGA §3.3 Algorithm 1 scores/softmax/out;
#        §5.3 the k_pe band is shared by every head]
# ----------------------------------------------------------------------------
def _keys(k_nope_bi: np.ndarray, k_pe_b: np.ndarray) -> np.ndarray:
    """K[u] = k_nope[u] || k_pe[u] for one (batch, head)."""
    return np.concatenate([k_nope_bi, k_pe_b], axis=-1)


def _causal_probs(q_bi: np.ndarray, K: np.ndarray):
    """Exact softmax of scores q.K^T / sqrt(d_qk) over keys u <= t; also returns ln-sum-exp."""
    S, d_qk = q_bi.shape
    s = (q_bi @ K.T) / np.sqrt(d_qk)
    allowed = np.tril(np.ones((S, S), dtype=bool))
    s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def attention_fwd(q, k_nope, k_pe, v):
    """O[b,t,i] = sum_{u<=t} softmax_u(s[b,i,t,u]) v[b,u,i], s = (q||.)(k_nope||k_pe)^T/sqrt(d_qk).

    q [B,S,h,d_nope+d_rope] (nope first), k_nope [B,S,h,d_nope], k_pe [B,S,d_rope],
    v [B,S,h,d_v] -> O [B,S,h,d_v], lse [B,h,S] (natural log of sum_u exp(s)).
    """
    B, S, h, _ = q.shape
    O = np.empty((B, S, h, v.shape[-1]))
    lse = np.empty((B, h, S))
    for b in range(B):
        for i in range(h):
            P, lse[b, i] = _causal_probs(q[b, :, i], _keys(k_nope[b, :, i], k_pe[b]))
            O[b, :, i] = P @ v[b, :, i]
    return O, lse


# ----------------------------------------------------------------------------
# O7-O9: attention backward (chain rule of the forward above) [LAGA §5.2]
# ----------------------------------------------------------------------------
def attention_bwd(q, k_nope, k_pe, v, d_o):
    """Gradients of sum(d_o * O) with respect to q, k_nope, k_pe and v.

    dv = P^T dO; dP = dO v^T; dS = P * (dP - rowsum(P * dP)); dq = dS K / sqrt(d_qk);
    dK = dS^T q / sqrt(d_qk); dk_nope = dK[:, :d_nope]; dk_pe = sum over local heads
    of dK[:, d_nope:] (the broadcast band's gradient).
    """
    B, S, h, d_qk = q.shape
    d_nope = k_nope.shape[-1]
    dq = np.empty_like(q, dtype=np.float64)
    dk_nope = np.empty(k_nope.shape)
    dv = np.empty(v.shape)
    dk_pe = np.zeros(k_pe.shape)
    for b in range(B):
        for i in range(h):
            K = _keys(k_nope[b, :, i], k_pe[b])
            P, _ = _causal_probs(q[b, :, i], K)
            dO = d_o[b, :, i]
            dv[b, :, i] = P.T @ dO
            dP = dO @ v[b, :, i].T
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[b, :, i] = (dS @ K) / np.sqrt(d_qk)
            dK = (dS.T @ q[b, :, i]) / np.sqrt(d_qk)
            dk_nope[b, :, i] = dK[:, :d_nope]
            dk_pe[b] += dK[:, d_nope:]
    return dq, dk_nope, dk_pe, dv


# ----------------------------------------------------------------------------
# O10-O11: fold of dk_nope / dv through W_kv_b  [LAGA §5.2: the W_kv_b gradient
#          of a rank is its (full_seq, H_r) shard]
# ----------------------------------------------------------------------------
def kv_up_bwd(dk_nope, dv, L, w_kv_b, heads):
    """dL[b,t] = sum_i W^k[i]^T dk_nope[b,t,i] + W^v[i]^T dv[b,t,i];
    dW[H_r[i]] = sum_{b,t} (dk_nope || dv)[b,t,i] outer L[b,t].

    Returns dL [B,S,d_kv] and dW_shard [h, d_nope+d_v, d_kv].
    """
    W = np.asarray(w_kv_b, dtype=np.float64)[heads]
    dkv = np.concatenate([dk_nope, dv], axis=-1)              # [B,S,h,d_nope+d_v]
    B, S, h, C = dkv.shape
    dL = np.zeros(L.shape)
    dW = np.zeros((h, C, L.shape[-1]))
    Lf = L.reshape(B * S, -1)
    for i in range(h):
        g = dkv[:, :, i, :]
        dL += g @ W[i]
        dW[i] = g.reshape(B * S, C).T @ Lf
    return dL, dW


# ----------------------------------------------------------------------------
# O12: RMSNorm backward (chain rule of O1)
# ----------------------------------------------------------------------------
def latent_rmsnorm_bwd(dL, latent, gamma, rstd):
    """x_hat = x r; dgamma = sum_{b,t} dL * x_hat; dx = r (g - x_hat * mean_j(g_j x_hat_j)), g = gamma dL."""
    x = np.asarray(latent, dtype=np.float64)
    xhat = x * rstd[..., None]
    dgamma = np.sum(dL * xhat, axis=tuple(range(dL.ndim - 1)))
    g = np.asarray(gamma, dtype=np.float64) * dL
    dx = rstd[..., None] * (g - xhat * np.mean(g * xhat, axis=-1, keepdims=True))
    return dx, dgamma


# ----------------------------------------------------------------------------
# Whole rank-local path
# ----------------------------------------------------------------------------
def forward(q, latent, k_pe, w_kv_b, gamma, *, n_h, sp_size, sp_rank, d_nope, eps=1e-6):
    """Norm -> head-shard up-projection -> causal attention for rank r of P."""
    heads = head_shard(n_h, sp_size, sp_rank)
    L, rstd = latent_rmsnorm(latent, gamma, eps)
    k_nope, v = kv_up(L, w_kv_b, heads, d_nope)
    O, lse = attention_fwd(q, k_nope, k_pe, v)
    return dict(L=L, rstd=rstd, k_nope=k_nope, v=v, O=O, lse=lse)


def backward(q, latent, k_pe, w_kv_b, gamma, d_o, *, n_h, sp_size, sp_rank, d_nope,
             eps=1e-6, fwd=None):
    """Gradients of sum(d_o * O) for rank r: dq, d_latent, dk_pe, dW rows of H_r, dgamma."""
    heads = head_shard(n_h, sp_size, sp_rank)
    if fwd is None:
        fwd = forward(q, latent, k_pe, w_kv_b, gamma, n_h=n_h, sp_size=sp_size,
                      sp_rank=sp_rank, d_nope=d_nope, eps=eps)
    dq, dk_nope, dk_pe, dv = attention_bwd(q, fwd["k_nope"], k_pe, fwd["v"], d_o)
    dL, dW_shard = kv_up_bwd(dk_nope, dv, fwd["L"], w_kv_b, heads)
    d_latent, d_gamma = latent_rmsnorm_bwd(dL, latent, gamma, fwd["rstd"])
    dW = np.zeros(np.shape(w_kv_b))
    dW[heads] = dW_shard
    return dict(dq=dq, dk_nope=dk_nope, dv=dv, dk_pe=dk_pe, dL=dL, d_latent=d_latent,
                d_w_kv_b=dW, d_gamma=d_gamma)


# ----------------------------------------------------------------------------
# Row-sampled forward for large inputs (same definition, only selected queries)
# ----------------------------------------------------------------------------
def attention_fwd_rows(q, k_nope, k_pe, v, rows):
    """O and lse of the definition above for the query positions `rows` only.

    Each output row of causal attention depends on q[t] and keys/values u <= t,
    so a selected row is computed exactly as in attention_fwd.
    """
    B, S, h, d_qk = q.shape
    rows = np.asarray(rows)
    O = np.empty((B, len(rows), h, v.shape[-1]))
    lse = np.empty((B, h, len(rows)))
    for b in range(B):
        for i in range(h):
            K = _keys(k_nope[b, :, i], k_pe[b])
            for j, t in enumerate(rows):
                s = (K[: t + 1] @ q[b, t, i]) / np.sqrt(d_qk)
                m = np.max(s)
                e = np.exp(s - m)
                l = np.sum(e)
                O[b, j, i] = (e / l) @ v[b, : t + 1, i]
                lse[b, i, j] = m + np.log(l)
    return O, lse


# ----------------------------------------------------------------------------
# Absorbed form (B2 of §3.2), used only as an independent identity check
# ----------------------------------------------------------------------------
def absorbed_scores_and_out(q, L, k_pe, w_kv_b, heads, d_nope):
    """Scores and output through the absorbed reformulation [LAGA §2.3, §3.2 (B2)].

    q_abs[t,i] = W^k[i]^T q_nope[t,i] (an n_h*d_kv-wide intermediate), scores
    (q_abs . L[u] + q_rope . k_pe[u]) / sqrt(d_qk), latent-space accumulator
    acc[t,i] = sum_u p L[u], output W^v[i] acc.  Returns (scores [B,h,S,S] with
    -inf above the diagonal, O [B,S,h,d_v]).
    """
    W = np.asarray(w_kv_b, dtype=np.float64)[heads]
    B, S, h, d_qk = q.shape
    scores = np.empty((B, h, S, S))
    O = np.empty((B, S, h, W.shape[1] - d_nope))
    allowed = np.tril(np.ones((S, S), dtype=bool))
    for b in range(B):
        for i in range(h):
            Wk, Wv = W[i, :d_nope], W[i, d_nope:]
            q_abs = q[b, :, i, :d_nope] @ Wk                      # [S, d_kv]
            s = (q_abs @ L[b].T + q[b, :, i, d_nope:] @ k_pe[b].T) / np.sqrt(d_qk)
            s = np.where(allowed, s, -np.inf)
            scores[b, i] = s
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            acc = p @ L[b]                                         # [S, d_kv]
            O[b, :, i] = acc @ Wv.T
    return scores, O


def explicit_scores(q, k_nope, k_pe):
    """s[b,i,t,u] = q[b,t,i].(k_nope[b,u,i] || k_pe[b,u]) / sqrt(d_qk), -inf for u > t."""
    B, S, h, d_qk = q.shape
    out = np.empty((B, h, S, S))
    allowed = np.tril(np.ones((S, S), dtype=bool))
    for b in range(B):
        for i in range(h):
            s = (q[b, :, i] @ _keys(k_nope[b, :, i], k_pe[b]).T) / np.sqrt(d_qk)
            out[b, i] = np.where(allowed, s, -np.inf)
    return out


# ----------------------------------------------------------------------------
# Absorbed form (B2 of §3.2) as a forward path of its own, with the two
# n_h * d_kv-wide intermediates whose memory §3.2 / §4.3 measure
# ----------------------------------------------------------------------------
def absorbed_forward_rows(q, L, k_pe, w_kv_b, heads, d_nope, rows):
    """B2's per-rank forward for the query positions `rows` [LAGA §3.2 (B2), Fig. 2].

    Absorb: q_abs[t,i] = W^k[i]^T q_nope[t,i] (d_kv wide).  Latent attention
    over the shared latent L (keys L || k_pe, values L): scores
    (q_abs . L[u] + q_rope . k_pe[u]) / sqrt(d_nope + d_rope), causal softmax,
    acc[t,i] = sum_u p L[u] (d_kv wide).  Un-absorb: O[t,i] = W^v[i] acc.
    The softmax scale is that of the explicit scores, which these equal.
    Returns q_abs, acc [B,len(rows),h,d_kv], O [B,len(rows),h,d_v], lse [B,h,len(rows)].
    """
    W = np.asarray(w_kv_b, dtype=np.float64)[heads]
    B, S, h, d_qk = q.shape
    d_kv = L.shape[-1]
    rows = np.asarray(rows)
    q_abs = np.empty((B, len(rows), h, d_kv))
    acc = np.empty((B, len(rows), h, d_kv))
    O = np.empty((B, len(rows), h, W.shape[1] - d_nope))
    lse = np.empty((B, h, len(rows)))
    for b in range(B):
        for i in range(h):
            Wk, Wv = W[i, :d_nope], W[i, d_nope:]
            for j, t in enumerate(rows):
                qa = q[b, t, i, :d_nope] @ Wk
                s = (L[b, : t + 1] @ qa + k_pe[b, : t + 1] @ q[b, t, i, d_nope:]) / np.sqrt(d_qk)
                m = np.max(s)
                e = np.exp(s - m)
                l = np.sum(e)
                a = (e / l) @ L[b, : t + 1]
                q_abs[b, j, i], acc[b, j, i] = qa, a
                O[b, j, i] = Wv @ a
                lse[b, i, j] = m + np.log(l)
    return q_abs, acc, O, lse


def absorbed_backward(q, latent, k_pe, w_kv_b, gamma, d_o, *, n_h, sp_size, sp_rank, d_nope, eps=1e-6):
    """Gradients of sum(d_o * O) for B2's forward [LAGA §3.2 (B2), Fig. 2], by the
    chain rule through B2's own steps (absorb, latent attention, un-absorb), one
    head at a time.  With P the causal softmax of the latent-space scores:

      d_acc   = dO W^v                    (the un-absorb's input gradient, d_kv wide)
      dW^v    = dO^T acc
      dP      = d_acc L^T,  dS = P * (dP - rowsum(P * dP))
      d_q_abs = dS L / sqrt(d_qk),  dq_rope = dS k_pe / sqrt(d_qk)
      dL     += P^T d_acc + dS^T q_abs / sqrt(d_qk)   (L is both the values and the keys)
      dk_pe  += dS^T q_rope / sqrt(d_qk)
      dq_nope = d_q_abs W^k^T,  dW^k = q_nope^T d_q_abs

    then the norm's backward.  Same outputs as backward() (the two forms are the
    same function), plus the two n_h * d_kv-wide gradients d_acc and d_q_abs.
    """
    heads = head_shard(n_h, sp_size, sp_rank)
    W = np.asarray(w_kv_b, dtype=np.float64)[heads]
    L, rstd = latent_rmsnorm(latent, gamma, eps)
    B, S, h, d_qk = q.shape
    d_kv = L.shape[-1]
    allowed = np.tril(np.ones((S, S), dtype=bool))
    scale = 1.0 / np.sqrt(d_qk)
    dq = np.empty((B, S, h, d_qk))
    dL = np.zeros(L.shape)
    dk_pe = np.zeros(np.shape(k_pe))
    dW_shard = np.zeros(W.shape)
    d_acc_all = np.empty((B, S, h, d_kv))
    d_q_abs_all = np.empty((B, S, h, d_kv))
    for b in range(B):
        for i in range(h):
            Wk, Wv = W[i, :d_nope], W[i, d_nope:]
            q_nope, q_rope = q[b, :, i, :d_nope], q[b, :, i, d_nope:]
            q_abs = q_nope @ Wk                                        # absorb
            s = np.where(allowed, (q_abs @ L[b].T + q_rope @ k_pe[b].T) * scale, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            acc = P @ L[b]                                             # latent accumulator
            dO = d_o[b, :, i]
            d_acc = dO @ Wv                                            # through the un-absorb
            dW_shard[i, d_nope:] += dO.T @ acc
            dP = d_acc @ L[b].T
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            d_q_abs = (dS @ L[b]) * scale
            dq[b, :, i, d_nope:] = (dS @ k_pe[b]) * scale
            dL[b] += P.T @ d_acc + (dS.T @ q_abs) * scale
            dk_pe[b] += (dS.T @ q_rope) * scale
            dq[b, :, i, :d_nope] = d_q_abs @ Wk.T                      # through the absorb
            dW_shard[i, :d_nope] += q_nope.T @ d_q_abs
            d_acc_all[b, :, i], d_q_abs_all[b, :, i] = d_acc, d_q_abs
    d_latent, d_gamma = latent_rmsnorm_bwd(dL, latent, gamma, rstd)
    dW = np.zeros(np.shape(w_kv_b))
    dW[heads] = dW_shard
    return dict(dq=dq, dk_pe=dk_pe, dL=dL, d_latent=d_latent, d_w_kv_b=dW, d_gamma=d_gamma,
                d_acc=d_acc_all, d_q_abs=d_q_abs_all)
