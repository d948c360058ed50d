"""An ordinary pre-norm causal transformer block built from PyTorch library
routines (CPU, float64), written independently of ``oracle/``.

It serves as the textbook special case the oracle must reduce to: with one
expert, one depth and one window spanning the document, the routed core is a
single block (its gate is the softmax of one logit, i.e. 1).  Library
routines used: ``torch.nn.functional.rms_norm``,
``scaled_dot_product_attention`` (causal flag or an explicit boolean mask),
``silu``, ``gelu`` (exact), and complex multiplication for the rotary
embedding (pairs (j, j + d_h/2) as the real and imaginary parts).
"""
from __future__ import annotations

import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(a, dtype=torch.float64)


def rotary(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    # x: [H][T][dh]
    if theta == 0.0:
        return x
    dh = x.shape[-1]
    half = dh // 2
    freqs = 1.0 / (theta ** (torch.arange(0, dh, 2, dtype=torch.float64) / dh))
    rot = torch.polar(torch.ones(len(pos), half, dtype=torch.float64),
                      pos.to(torch.float64)[:, None] * freqs[None, :])
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def block(x, wqkv, wo, w_gu, w_down, g_attn, g_ffn, n_heads, mlp, eps=1e-6,
          theta=10000.0, film=None, mask=None, positions=None):
    """y = h + MLP(norm(h)), h = x + Attn(norm(x)) over the whole sequence.

    x [T][d]; weights in [out][in] layout; film = (gamma[2][d], beta[2][d]) or
    None; mask: None for plain causal attention, else a boolean [T][T] of
    allowed (query, key) pairs.
    """
    x = _t(x)
    T, d = x.shape
    dh = d // n_heads
    pos = torch.arange(T) if positions is None else torch.as_tensor(positions)
    u = F.rms_norm(x, (d,), weight=_t(g_attn), eps=eps)
    if film is not None:
        u = _t(film[0][0]) * u + _t(film[1][0])
    qkv = u @ _t(wqkv).T
    q, k, v = (qkv[:, i * d:(i + 1) * d].reshape(T, n_heads, dh).transpose(0, 1)
               for i in range(3))
    q, k = rotary(q, pos, theta), rotary(k, pos, theta)
    if mask is None:
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    else:
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.as_tensor(mask))
    h = x + o.transpose(0, 1).reshape(T, d) @ _t(wo).T
    u2 = F.rms_norm(h, (d,), weight=_t(g_ffn), eps=eps)
    if film is not None:
        u2 = _t(film[0][1]) * u2 + _t(film[1][1])
    w_gu = _t(w_gu)
    if mlp == "swiglu":
        f = w_gu.shape[0] // 2
        mid = F.silu(u2 @ w_gu[:f].T) * (u2 @ w_gu[f:].T)
    else:
        mid = F.gelu(u2 @ w_gu.T, approximate="none")
    return (h + mid @ _t(w_down).T).numpy()
