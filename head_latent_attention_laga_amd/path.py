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
        # k_nope / v storage (laga.h): float32, fp16, or an fp16 plane followed
        # by an e4m3 low plane (kvb == 3); held here as flat byte tensors.
        self.kv_bytes = kvb

    def _kv_empty(self, width):
        return torch.empty((self.B * self.S * self.h * width * self.kv_bytes,), dtype=torch.uint8,
                           device=self.device)

    def kv_value(self, t, width):
        """The value a k_nope / v buffer of row width `width` holds, as a float64
        [B, S, h, width] CPU tensor (decoding only; for checks and inspection)."""
        shape = (self.B, self.S, self.h, width)
        n = self.B * self.S * self.h * width
        t = t.detach().cpu()
        if self.kv_bytes == 4:
            return t.view(torch.float32).double().view(shape)
        hi = t[:2 * n].view(torch.float16).double().view(shape)
        if self.kv_bytes == 2:
            return hi
        lo = t[2 * n:].view(torch.float8_e4m3fn).double().view(shape)
        return hi + lo * 2.0 ** -_lib.LAGA_KV_LO_SHIFT

    def _empty(self, shape, dtype=torch.float32):
        return torch.empty(shape, dtype=dtype, device=self.device)

    def alloc_forward(self):
        B, S, h = self.B, self.S, self.h
        return dict(
            latent_n=self._empty((B, S, self.d_kv)), rstd=self._empty((B, S)),
            k_nope=self._kv_empty(self.d_nope), v=self._kv_empty(self.d_v),
            o=self._empty((B, S, h, self.d_v)), lse=self._empty((B, h, S)))

    def forward(self, x, out=None, stream=None):
        """x: dict of device tensors q, latent, k_pe, w_kv_b, gamma."""
        out = out or self.alloc_forward()
        _lib.latent_norm(self.dims, x["latent"], x["gamma"], out["latent_n"], out["rstd"], stream)
        _lib.kv_up(self.dims, out["latent_n"], x["w_kv_b"], out["k_nope"], out["v"], stream)
        _lib.attn_fwd(self.dims, x["q"], out["k_nope"], x["k_pe"], out["v"], out["o"], out["lse"], stream)
        return out

    def alloc_fused(self):
        """Outputs and workspace of the fused forward (fp16 operands, bf16 V3 dims only)."""
        B, S, h = self.B, self.S, self.h
        ws = _lib.attn_fwd_fused_workspace_bytes(self.dims)
        if ws == 0:
            raise _lib.LagaError("laga_attn_fwd_fused_workspace_bytes", 2, "dims rejected by the fused forward")
        return dict(o=self._empty((B, S, h, self.d_v)), lse=self._empty((B, h, S)),
                    workspace=torch.empty((ws,), dtype=torch.uint8, device=self.device))

    def forward_fused(self, x, out=None, stream=None):
        """o and lse from one laga_attn_fwd_fused call (norm, up-projection and
        attention fused; K/V never leave the library's workspace)."""
        out = out or self.alloc_fused()
        _lib.attn_fwd_fused(self.dims, x["q"], x["latent"], x["gamma"], x["k_pe"], x["w_kv_b"], out["o"],
                            out["lse"], out["workspace"], stream)
        return out

    def alloc_absorbed(self):
        """Buffers of the absorbed-form (B2) forward: its n_h*d_kv-wide intermediates
        q_abs (fp16) and acc (float32), the fp16 key rows kx, and o, lse."""
        B, S, h = self.B, self.S, self.h
        return dict(
            latent_n=self._empty((B, S, self.d_kv)), rstd=self._empty((B, S)),
            q_abs=self._empty((B, S, h, self.d_kv), torch.float16),
            kx=self._empty((B, S, self.d_kv + self.d_rope), torch.float16),
            acc=self._empty((B, S, h, self.d_kv)),
            o=self._empty((B, S, h, self.d_v)), lse=self._empty((B, h, S)))

    def absorbed_forward(self, x, out=None, stream=None):
        """The absorbed form's forward on the same inputs: norm, then laga_absorbed_fwd."""
        out = out or self.alloc_absorbed()
        _lib.latent_norm(self.dims, x["latent"], x["gamma"], out["latent_n"], out["rstd"], stream)
        _lib.absorbed_fwd(self.dims, x["q"], out["latent_n"], x["k_pe"], x["w_kv_b"], out["q_abs"], out["kx"],
                          out["acc"], out["o"], out["lse"], stream)
        return out

    def absorbed_backward(self, x, absf, d_o, grads=None, stream=None):
        """The absorbed form's backward for the output of absorbed_forward(x) (absf: its rstd is used;
        the backward recomputes q_abs, lse and acc itself)."""
        g = grads or self.alloc_backward(workspace_bytes=_lib.absorbed_bwd_workspace_bytes(self.dims))
        _lib.absorbed_bwd(self.dims, x["q"], x["latent"], x["gamma"], absf["rstd"], x["k_pe"], x["w_kv_b"], d_o,
                          g["dq"], g["d_latent"], g["d_k_pe"], g["d_w_kv_b"], g["d_gamma"], g["workspace"], stream)
        return g

    def alloc_backward(self, workspace_bytes=None):
        B, S, h = self.B, self.S, self.h
        ws = _lib.attn_bwd_workspace_bytes(self.dims) if workspace_bytes is None else workspace_bytes
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
