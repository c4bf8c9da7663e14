"""Allocation and sequencing of the four C-ABI calls for one rank's share.

LagaPath owns no arithmetic: it allocates the output and workspace tensors with
torch on the current device and calls laga_latent_norm, laga_kv_up,
laga_attn_fwd and laga_attn_bwd in the order of the paper's per-rank forward
(norm of the gathered latent, head-shard up-projection, attention) and its
backward.
"""
from __future__ import annotations

import torch

from . import _lib


class LagaPath:
    def __init__(self, B, S, n_h, sp_size, sp_rank, d_kv, d_nope, d_rope, d_v, dtype, precision,
                 eps=1e-6, device="cuda"):
        self.dims = _lib.make_dims(B, S, n_h, sp_size, sp_rank, d_kv, d_nope, d_rope, d_v,
                                   _lib.LAGA_BF16 if dtype == "bf16" else _lib.LAGA_F32,
                                   precision, eps)
        self.B, self.S, self.h = B, S, n_h // sp_size
        self.n_h, self.d_kv, self.d_nope, self.d_rope, self.d_v = n_h, d_kv, d_nope, d_rope, d_v
        self.device = torch.device(device)
        kvb = _lib.kv_elem_bytes(self.dims)
        if kvb == 0:
            raise _lib.LagaError("laga_kv_elem_bytes", 2, "dims rejected")
        # k_nope / v storage: [planes, B, S, h, d]; bf16 inputs store fp16 (two
        # planes hi, lo with split operands), float32 inputs one float32 plane.
        bf16 = dtype == "bf16"
        self.kv_dtype = torch.float16 if bf16 else torch.float32
        self.kv_planes = kvb // 2 if bf16 else 1

    def _empty(self, shape, dtype=torch.float32):
        return torch.empty(shape, dtype=dtype, device=self.device)

    def alloc_forward(self):
        B, S, h = self.B, self.S, self.h
        return dict(
            latent_n=self._empty((B, S, self.d_kv)), rstd=self._empty((B, S)),
            k_nope=self._empty((self.kv_planes, B, S, h, self.d_nope), self.kv_dtype),
            v=self._empty((self.kv_planes, B, S, h, self.d_v), self.kv_dtype),
            o=self._empty((B, S, h, self.d_v)), lse=self._empty((B, h, S)))

    def forward(self, x, out=None, stream=None):
        """x: dict of device tensors q, latent, k_pe, w_kv_b, gamma."""
        out = out or self.alloc_forward()
        _lib.latent_norm(self.dims, x["latent"], x["gamma"], out["latent_n"], out["rstd"], stream)
        _lib.kv_up(self.dims, out["latent_n"], x["w_kv_b"], out["k_nope"], out["v"], stream)
        _lib.attn_fwd(self.dims, x["q"], out["k_nope"], x["k_pe"], out["v"], out["o"], out["lse"], stream)
        return out

    @staticmethod
    def kv_value(t):
        """The value a k_nope / v buffer holds: the sum of its planes, as float32."""
        return t.float().sum(0)

    def alloc_backward(self):
        B, S, h = self.B, self.S, self.h
        ws = _lib.attn_bwd_workspace_bytes(self.dims)
        return dict(
            dq=self._empty((B, S, h, self.d_nope + self.d_rope)), d_latent=self._empty((B, S, self.d_kv)),
            d_k_pe=self._empty((B, S, self.d_rope)),
            d_w_kv_b=torch.zeros((self.n_h, self.d_nope + self.d_v, self.d_kv), dtype=torch.float32,
                                 device=self.device),
            d_gamma=self._empty((self.d_kv,)),
            workspace=torch.empty((ws,), dtype=torch.uint8, device=self.device))

    def backward(self, x, fwd, d_o, grads=None, stream=None):
        g = grads or self.alloc_backward()
        _lib.attn_bwd(self.dims, x["q"], x["latent"], x["gamma"], fwd["rstd"], fwd["k_nope"], x["k_pe"],
                      fwd["v"], x["w_kv_b"], fwd["o"], fwd["lse"], d_o, g["dq"], g["d_latent"],
                      g["d_k_pe"], g["d_w_kv_b"], g["d_gamma"], g["workspace"], stream)
        return g
