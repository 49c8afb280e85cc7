"""Oracle of the full-BPTT gradient of the current-policy replay.

TEST INFRASTRUCTURE ONLY, under the same rule as rlt_oracle: only the tests may import it.
It shares no code with the HIP library or its binding.

What is differentiated ([R] = jiphyeonjeon.kr/blog/rlt, "Recurrent Looped Transformer",
review of the technical report; [S] = greeksharifa.github.io, "Recurrent Looped
Transformer 요약 설명"): the replay of [R] §6.2 (eq 5.5) -- from H_0 with the current
parameters, the causal encoder over the whole history, the memory, and the sequential
transitions -- giving log p(x_{t+1} | x_<=t) for t = 1..T-1. The loss is
L = sum_{b,t} w[b, t] * logprob[b, t] for given weights w (the gradient of any loss built
from the replay's log-probabilities, e.g. an importance-weighted policy loss, enters this
way). [R] Appendix B eq B.4 and §6.4: the reference training computation is full BPTT --
the gradient flows through s_t, through every decoder key/value (including entries the
window later drops) and through the encoder memory; nothing is detached.

The gradient's plain definition is the derivative of L; the oracle writes the forward pass
once more with torch float64 tensors (the same steps, in the same order and notation, as
rlt_oracle: pre-norm RMSNorm, rotate-half RoPE with float64 angles, SwiGLU, sigmoid merge
over [e ; r], window max(1, t-W+1)..t, memory prefix 1..t) and lets torch's reverse-mode
differentiation (a library routine) produce dL/dtheta. Pins: the forward equals
rlt_oracle's replay, and the gradient equals central finite differences of L
(tests/test_oracle_grad.py).
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

V0, V1, V2 = 0, 1, 2


class GradOracle:
    def __init__(self, cfg, params: Dict[str, np.ndarray]):
        self.cfg = cfg
        self.P = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True) for k, v in params.items()}

    def p(self, name):
        return self.P[name]

    def dec_w(self, l, short):
        return self.p(f"enc.{l}.{short}") if self.cfg.share else self.p(f"dec.{l}.{short}")

    def rms(self, x, g):
        return x / torch.sqrt((x * x).mean(-1, keepdim=True) + self.cfg.rms_eps) * g

    def rope(self, v, pos):
        """v [..., H*dh]; pos broadcast against the leading dims (float64 angles)."""
        H, dh = self.cfg.n_heads, self.cfg.d_head
        half = dh // 2
        x = v.reshape(v.shape[:-1] + (H, dh))
        theta = self.cfg.rope_base ** (-2.0 * torch.arange(half, dtype=torch.float64) / dh)
        ang = torch.as_tensor(pos, dtype=torch.float64)[..., None, None] * theta
        c, s = torch.cos(ang), torch.sin(ang)
        x1, x2 = x[..., :half], x[..., half:]
        return torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], dim=-1).reshape(v.shape)

    def swiglu(self, x, w1, w3, w2):
        a = x @ w1.T
        return (a * torch.sigmoid(a) * (x @ w3.T)) @ w2.T

    def attend(self, q, keys, vals):
        """q [B, H*dh]; keys, vals [B, n, H*dh]."""
        H, dh = self.cfg.n_heads, self.cfg.d_head
        B, n = keys.shape[0], keys.shape[1]
        sc = torch.einsum("bhd,bnhd->bhn", q.reshape(B, H, dh), keys.reshape(B, n, H, dh)) / np.sqrt(dh)
        w = torch.softmax(sc, dim=-1)
        return torch.einsum("bhn,bnhd->bhd", w, vals.reshape(B, n, H, dh)).reshape(B, H * dh)

    def replay(self, tokens: np.ndarray):
        """Returns logprob [B, T-1] (torch float64, differentiable)."""
        cfg = self.cfg
        H, dh = cfg.n_heads, cfg.d_head
        x = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
        B, T = x.shape
        pos = torch.arange(1, T + 1, dtype=torch.float64)
        # encoder: token-parallel, causal
        h = self.p("emb")[x]
        causal = torch.arange(T)[None, :] <= torch.arange(T)[:, None]
        for l in range(cfg.L_E):
            a = self.rms(h, self.p(f"enc.{l}.n1"))
            q = self.rope(a @ self.p(f"enc.{l}.wq").T, pos).reshape(B, T, H, dh)
            k = self.rope(a @ self.p(f"enc.{l}.wk").T, pos).reshape(B, T, H, dh)
            v = (a @ self.p(f"enc.{l}.wv").T).reshape(B, T, H, dh)
            sc = torch.einsum("bihd,bjhd->bhij", q, k) / np.sqrt(dh)
            sc = sc.masked_fill(~causal[None, None], float("-inf"))
            o = torch.einsum("bhij,bjhd->bihd", torch.softmax(sc, -1), v).reshape(B, T, H * dh)
            h = h + o @ self.p(f"enc.{l}.wo").T
            h = h + self.swiglu(self.rms(h, self.p(f"enc.{l}.n2")), self.p(f"enc.{l}.w1"), self.p(f"enc.{l}.w3"),
                                self.p(f"enc.{l}.w2"))
        e = h
        mem_k, mem_v = [], []
        if cfg.L_D > 0:
            en = self.rms(e, self.p("mem.nE"))
            for g in range(cfg.groups):
                mem_k.append(self.rope(en @ self.p(f"mem.{g}.wk").T, pos))
                mem_v.append(en @ self.p(f"mem.{g}.wv").T)
        # decoder: sequential transitions
        s = self.p("merge.s0").expand(B, cfg.d) if cfg.variant != V0 else None
        rho = s
        ks = [[] for _ in range(cfg.L_D)]
        vs = [[] for _ in range(cfg.L_D)]
        outs = []
        for t in range(1, T + 1):
            et = e[:, t - 1]
            if cfg.variant == V0:
                u = et
            else:
                src = s if cfg.variant == V1 else rho
                r = self.rms(src, self.p("merge.ns"))
                gt = torch.sigmoid(torch.cat([et, r], -1) @ self.p("merge.wg").T + self.p("merge.bg"))
                u = et + cfg.alpha * gt * (r @ self.p("merge.ws").T)
            z = u
            for l in range(cfg.L_D):
                a = self.rms(z, self.p(f"dec.{l}.m1"))
                q = self.rope(a @ self.dec_w(l, "wq").T, float(t))
                ks[l].append(self.rope(a @ self.dec_w(l, "wk").T, float(t)))
                vs[l].append(a @ self.dec_w(l, "wv").T)
                lo = max(1, t - cfg.window + 1)
                keys = torch.stack(ks[l][lo - 1:t], 1)
                vals = torch.stack(vs[l][lo - 1:t], 1)
                z = z + self.attend(q, keys, vals) @ self.dec_w(l, "wo").T
                b = self.rms(z, self.p(f"dec.{l}.m2"))
                qx = self.rope(b @ self.p(f"dec.{l}.xq").T, float(t))
                gi = 0 if cfg.groups == 1 else l
                z = z + self.attend(qx, mem_k[gi][:, :t], mem_v[gi][:, :t]) @ self.p(f"dec.{l}.xo").T
                z = z + self.swiglu(self.rms(z, self.p(f"dec.{l}.m3")), self.dec_w(l, "w1"), self.dec_w(l, "w3"),
                                    self.dec_w(l, "w2"))
            s = z
            if cfg.variant == V2 and t % cfg.chunk == 0:
                rho = s
            outs.append(s)
        S = torch.stack(outs, 1)                                          # [B, T, d]
        logits = self.rms(S, self.p("out.nO")) @ self.p("out.w").T
        lp = torch.log_softmax(logits[:, :-1], -1)
        return torch.gather(lp, -1, x[:, 1:, None])[..., 0]

    def grad(self, tokens: np.ndarray, w: np.ndarray):
        """(logprob [B, T-1] numpy, {name: dL/dname numpy}) for L = sum(w * logprob)."""
        for v in self.P.values():
            v.grad = None
        lp = self.replay(tokens)
        loss = (lp * torch.as_tensor(np.asarray(w, dtype=np.float64))).sum()
        loss.backward()
        return lp.detach().numpy(), {k: (v.grad.numpy() if v.grad is not None else np.zeros(v.shape))
                                     for k, v in self.P.items()}

    def loss(self, tokens: np.ndarray, w: np.ndarray) -> float:
        with torch.no_grad():
            return float((self.replay(tokens) * torch.as_tensor(np.asarray(w, dtype=np.float64))).sum())
