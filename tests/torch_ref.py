"""Independent token-parallel formulations built from torch CPU library routines.

Used only to pin the oracle: attention comes from
torch.nn.functional.scaled_dot_product_attention (with causal, sliding-window
or prefix masks), RMSNorm from torch.nn.functional.rms_norm, SiLU from
torch.nn.functional.silu, and the rotary encoding is written as a complex
exponential (z_i * exp(i * p * theta_i) with z_i = x_i + i x_{i+dh/2}) instead
of the oracle's rotate-half real form. Everything runs in float64.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def T(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def rms(x, g, eps):
    return F.rms_norm(x, (x.shape[-1],), weight=g, eps=eps)


def rope_complex(x, pos, H, dh, base):
    """x [..., n, H*dh], pos [n] -> rotated, via complex multiplication."""
    half = dh // 2
    xs = x.reshape(*x.shape[:-1], H, dh)
    z = torch.complex(xs[..., :half], xs[..., half:])
    theta = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / dh)
    ang = torch.as_tensor(np.asarray(pos, dtype=np.float64))[:, None] * theta[None, :]   # [n, half]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]                             # [n, 1, half]
    zr = z * rot
    return torch.cat([zr.real, zr.imag], dim=-1).reshape(x.shape)


def heads(x, H, dh):
    """[B, n, H*dh] -> [B, H, n, dh]"""
    B, n, _ = x.shape
    return x.reshape(B, n, H, dh).transpose(1, 2)


def unheads(x):
    B, H, n, dh = x.shape
    return x.transpose(1, 2).reshape(B, n, H * dh)


def swiglu(x, w1, w3, w2):
    return (F.silu(x @ w1.T) * (x @ w3.T)) @ w2.T


def encoder(cfg, P, tokens):
    """Causal pre-norm encoder over a whole prefix; returns e [B, T, d]."""
    H, dh = cfg.n_heads, cfg.d_head
    B, n = tokens.shape
    pos = np.arange(1, n + 1)
    h = T(P["emb"])[torch.as_tensor(tokens, dtype=torch.long)]
    for l in range(cfg.L_E):
        a = rms(h, T(P[f"enc.{l}.n1"]), cfg.rms_eps)
        q = rope_complex(a @ T(P[f"enc.{l}.wq"]).T, pos, H, dh, cfg.rope_base)
        k = rope_complex(a @ T(P[f"enc.{l}.wk"]).T, pos, H, dh, cfg.rope_base)
        v = a @ T(P[f"enc.{l}.wv"]).T
        o = F.scaled_dot_product_attention(heads(q, H, dh), heads(k, H, dh), heads(v, H, dh), is_causal=True)
        h = h + unheads(o) @ T(P[f"enc.{l}.wo"]).T
        h = h + swiglu(rms(h, T(P[f"enc.{l}.n2"]), cfg.rms_eps), T(P[f"enc.{l}.w1"]),
                       T(P[f"enc.{l}.w3"]), T(P[f"enc.{l}.w2"]))
    return h


def memory(cfg, P, e):
    H, dh = cfg.n_heads, cfg.d_head
    n = e.shape[1]
    pos = np.arange(1, n + 1)
    en = rms(e, T(P["mem.nE"]), cfg.rms_eps)
    ks, vs = [], []
    for g in range(cfg.groups):
        ks.append(rope_complex(en @ T(P[f"mem.{g}.wk"]).T, pos, H, dh, cfg.rope_base))
        vs.append(en @ T(P[f"mem.{g}.wv"]).T)
    return ks, vs


def merge(cfg, P, e, s_prev):
    r = rms(s_prev, T(P["merge.ns"]), cfg.rms_eps)
    g = torch.sigmoid(torch.cat([e, r], dim=-1) @ T(P["merge.wg"]).T + T(P["merge.bg"]))
    return e + cfg.alpha * g * (r @ T(P["merge.ws"]).T)


def parallel_decoder(cfg, P, u):
    """Decoder blocks over all positions at once, valid when u_t does not depend on s_{t-1}.

    SWA: query t sees keys max(1, t-W+1)..t (band mask). Cross: query t sees
    memory 1..t (prefix mask). Returns s [B, T, d].
    """
    H, dh, W = cfg.n_heads, cfg.d_head, cfg.window
    B, n, d = u.shape
    pos = np.arange(1, n + 1)
    e = None
    i = torch.arange(n)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    prefix = i[None, :] <= i[:, None]
    return _decode_with_masks(cfg, P, u, pos, band, prefix)


def _dec(P, cfg, l, short):
    return T(P[f"enc.{l}.{short}"]) if cfg.share else T(P[f"dec.{l}.{short}"])


def _decode_with_masks(cfg, P, u, pos, band, prefix):
    H, dh = cfg.n_heads, cfg.d_head
    mk, mv = P["_mem_k"], P["_mem_v"]
    z = u
    for l in range(cfg.L_D):
        a = rms(z, T(P[f"dec.{l}.m1"]), cfg.rms_eps)
        q = rope_complex(a @ _dec(P, cfg, l, "wq").T, pos, H, dh, cfg.rope_base)
        k = rope_complex(a @ _dec(P, cfg, l, "wk").T, pos, H, dh, cfg.rope_base)
        v = a @ _dec(P, cfg, l, "wv").T
        o = F.scaled_dot_product_attention(heads(q, H, dh), heads(k, H, dh), heads(v, H, dh), attn_mask=band)
        z = z + unheads(o) @ _dec(P, cfg, l, "wo").T
        b = rms(z, T(P[f"dec.{l}.m2"]), cfg.rms_eps)
        qx = rope_complex(b @ T(P[f"dec.{l}.xq"]).T, pos, H, dh, cfg.rope_base)
        g = 0 if cfg.groups == 1 else l
        o = F.scaled_dot_product_attention(heads(qx, H, dh), heads(mk[g], H, dh), heads(mv[g], H, dh),
                                           attn_mask=prefix)
        z = z + unheads(o) @ T(P[f"dec.{l}.xo"]).T
        z = z + swiglu(rms(z, T(P[f"dec.{l}.m3"]), cfg.rms_eps), _dec(P, cfg, l, "w1"),
                       _dec(P, cfg, l, "w3"), _dec(P, cfg, l, "w2"))
    return z


def readout(cfg, P, s):
    return rms(s, T(P["out.nO"]), cfg.rms_eps) @ T(P["out.w"]).T


def feedforward_model(cfg, P, tokens, s_fixed=None):
    """Whole model when the decoder input does not depend on earlier outputs.

    RLT-0: u_t = e_t. With s_fixed given (RLT-2 with one chunk covering every
    position): u_t = Merge(e_t, s_fixed). Returns (logits [B, T, V], s [B, T, d]).
    """
    e = encoder(cfg, P, tokens)
    ks, vs = memory(cfg, P, e)
    P = dict(P)
    P["_mem_k"], P["_mem_v"] = ks, vs
    if s_fixed is None:
        u = e
    else:
        u = merge(cfg, P, e, T(s_fixed).expand(e.shape[0], e.shape[1], -1))
    s = parallel_decoder(cfg, P, u)
    return readout(cfg, P, s), s
