"""Oracle: a plain, slow CPU definition of the Recurrent Looped Transformer forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library or its binding; it reads the
parameter dictionary and token arrays that the seeded generators produce.

Sources (the pages are web pages about the method; citations name the page and
the section / equation on it):
  [S] greeksharifa.github.io, "Recurrent Looped Transformer 요약 설명"
      (summary of the arXiv version): §2.1 sequence and state, §2.2 encoder and
      memory, §2.3 one transition per token, §2.4 prefill / incremental
      decoding, §2.5 merge and decoder blocks (merge equation), §2.7 RLT-0/1/2,
      appendix A.1 (weight sharing), appendix I (RLT-2 chunks).
  [R] jiphyeonjeon.kr/blog/rlt, "Recurrent Looped Transformer" (review of the
      technical report): §2 eq 2.1-2.2 (memory), §3.1 eq 2.7 (composition),
      §3.2 (E^step), §3.3 eq 2.9-2.16 (merge, blocks, retained window),
      §3.4 (sharing), §6.2 eq 5.5 (replay log-probabilities).

Readings taken where the pages leave a form open (each is listed in the design
notes): RoPE (rotate-half, base 10000) on every query/key; pre-norm RMSNorm with
a learned gain on every sublayer, eps 1e-6; SwiGLU FFN without biases; full gate
matrix W_g over [e_t ; r] with bias b_g, W_s without bias, alpha fixed at 0.1;
memory K and V both from RMSNorm_E(e); no final encoder norm; s_t is the
decoder residual stream before the readout norm; untied readout; BOS = V-1.

Parity pins: see tests/test_oracle_*.py. Absolute logit values of a whole model
are "parity unpinned" by the pages (no printed model outputs exist for this
parameterisation); every component is pinned by closed forms, special cases,
library routines and the pages' propositions.

All arithmetic runs in the dtype given to Oracle (float64 by default). The
batch dimension B holds independent sequences at the same position; nothing
mixes rows.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

V0, V1, V2 = 0, 1, 2


class Oracle:
    """Parameters + configuration; every step of the method is a method here."""

    def __init__(self, cfg, params: Dict[str, np.ndarray], dtype=np.float64):
        self.cfg = cfg
        self.dt = np.dtype(dtype)
        # A mapping that decodes entries on read (16-bit storage of the largest
        # shapes) stays lazy: each read yields that entry in the working dtype.
        self._lazy = bool(getattr(params, "upcast_on_read", False))
        self._P = params if self._lazy else {k: np.asarray(v, dtype=self.dt) for k, v in params.items()}
        self.used = set()          # names read so far (parameter-count pins)
        self.block_steps = 0       # dependent decoder block steps (schedule-depth pin)

    # ------------------------------------------------------------------ params
    def p(self, name: str) -> np.ndarray:
        self.used.add(name)
        if self._lazy:
            return np.asarray(self._P[name], dtype=self.dt)
        return self._P[name]

    def dec_w(self, l: int, short: str) -> np.ndarray:
        """Decoder SWA / FFN weight; aliases the encoder layer's when shared ([S] appendix A.1, [R] §3.4)."""
        if self.cfg.share:
            return self.p(f"enc.{l}.{short}")
        return self.p(f"dec.{l}.{short}")

    def group_of(self, l: int) -> int:
        """g(l): one shared group when G = 1, one group per decoder layer when G = L_D ([S] §2.2)."""
        if self.cfg.groups == 1:
            return 0
        assert self.cfg.groups == self.cfg.L_D, "only G = 1 and G = L_D are defined"
        return l

    # -------------------------------------------------------------- primitives
    def rms(self, x: np.ndarray, gain: np.ndarray) -> np.ndarray:
        """RMSNorm with learned gain: x / sqrt(mean(x^2) + eps) * gain."""
        ms = np.mean(x * x, axis=-1, keepdims=True)
        return x / np.sqrt(ms + self.dt.type(self.cfg.rms_eps)) * gain

    def rope(self, v: np.ndarray, pos) -> np.ndarray:
        """Rotary position encoding (rotate-half pairs (i, i + dh/2)), angle pos * base^(-2i/dh).

        v has trailing size H*dh; pos is a scalar or an array broadcast against
        the leading dimensions (one position per row). Angles in float64.
        """
        H, dh = self.cfg.n_heads, self.cfg.d_head
        half = dh // 2
        shp = v.shape
        x = v.reshape(shp[:-1] + (H, dh))
        i = np.arange(half, dtype=np.float64)
        theta = self.cfg.rope_base ** (-2.0 * i / dh)
        p = np.asarray(pos, dtype=np.float64)
        ang = p[..., None, None] * theta            # [..., 1, half]
        c = np.cos(ang).astype(self.dt)
        s = np.sin(ang).astype(self.dt)
        x1, x2 = x[..., :half], x[..., half:]
        out = np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)
        return out.reshape(shp)

    @staticmethod
    def sigmoid(x):
        return 1.0 / (1.0 + np.exp(-x))

    def swiglu(self, x: np.ndarray, w1, w3, w2) -> np.ndarray:
        """SwiGLU FFN: W2 (silu(W1 x) * (W3 x)), silu(z) = z * sigmoid(z)."""
        a = x @ w1.T
        b = x @ w3.T
        return (a * self.sigmoid(a) * b) @ w2.T

    def attend(self, q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
        """One query per row and head over n keys: softmax(q.k / sqrt(dh)) weighted sum of values.

        q [B, H*dh]; keys, vals [B, n, H*dh] (already position-encoded). Returns [B, H*dh].
        """
        H, dh = self.cfg.n_heads, self.cfg.d_head
        B, n = keys.shape[0], keys.shape[1]
        qh = q.reshape(B, H, dh)
        kh = keys.reshape(B, n, H, dh)
        vh = vals.reshape(B, n, H, dh)
        scores = np.einsum("bhd,bnhd->bhn", qh, kh) / np.sqrt(self.dt.type(dh))
        scores = scores - scores.max(axis=-1, keepdims=True)
        w = np.exp(scores)
        w = w / w.sum(axis=-1, keepdims=True)
        out = np.einsum("bhn,bnhd->bhd", w, vh)
        return out.reshape(B, H * dh)

    # ------------------------------------------------------------------ state
    def new_state(self, B: int) -> "OracleState":
        """H_0 = (s*, empty caches); the RLT-2 register starts at s* ([S] §2.1, [R] §3.1)."""
        st = OracleState(self.cfg, B, self.dt)
        if self.cfg.variant != V0:
            s0 = self.p("merge.s0")
            st.s = np.broadcast_to(s0, (B, self.cfg.d)).astype(self.dt).copy()
            st.rho = st.s.copy()
        return st

    # --------------------------------------------------------------- encoder
    def encoder_step(self, st: "OracleState", x: np.ndarray) -> np.ndarray:
        """Incremental encoder E^step: (e_t, C^E_t) from x_t and C^E_{t-1} ([R] §3.2, [S] §2.4).

        x int [B]. Appends this position's keys/values to every layer's encoder
        cache and returns e_t [B, d] (the raw residual output, no final norm).
        """
        cfg = self.cfg
        t = st.n_enc + 1
        h = self.p("emb")[x].astype(self.dt)
        for l in range(cfg.L_E):
            a = self.rms(h, self.p(f"enc.{l}.n1"))
            q = self.rope(a @ self.p(f"enc.{l}.wq").T, t)
            k = self.rope(a @ self.p(f"enc.{l}.wk").T, t)
            v = a @ self.p(f"enc.{l}.wv").T
            st.enc_k[l].append(k)
            st.enc_v[l].append(v)
            keys = np.stack(st.enc_k[l], axis=1)
            vals = np.stack(st.enc_v[l], axis=1)
            h = h + self.attend(q, keys, vals) @ self.p(f"enc.{l}.wo").T
            h = h + self.swiglu(self.rms(h, self.p(f"enc.{l}.n2")), self.p(f"enc.{l}.w1"),
                                self.p(f"enc.{l}.w3"), self.p(f"enc.{l}.w2"))
        st.n_enc = t
        self._append_memory(st, h, t)
        st.e.append(h)
        return h

    def encoder_chunk(self, st: "OracleState", xs: np.ndarray) -> np.ndarray:
        """Token-parallel causal encoding of the next n positions ([S] §2.2, §2.4; [R] §3.2).

        xs int [B, n]. Position p attends to encoder keys 1..p (earlier chunks
        come from the encoder cache). Returns e [B, n, d] and appends memory.
        """
        cfg = self.cfg
        H, dh = cfg.n_heads, cfg.d_head
        B, n = xs.shape
        t0 = st.n_enc
        pos = np.arange(t0 + 1, t0 + n + 1, dtype=np.float64)
        h = self.p("emb")[xs].astype(self.dt)                       # [B, n, d]
        for l in range(cfg.L_E):
            a = self.rms(h, self.p(f"enc.{l}.n1"))
            q = self.rope(a @ self.p(f"enc.{l}.wq").T, pos)            # [B, n, H*dh]
            k = self.rope(a @ self.p(f"enc.{l}.wk").T, pos)
            v = a @ self.p(f"enc.{l}.wv").T
            for i in range(n):
                st.enc_k[l].append(k[:, i])
                st.enc_v[l].append(v[:, i])
            keys = np.stack(st.enc_k[l], axis=1)                      # [B, t0+n, H*dh]
            vals = np.stack(st.enc_v[l], axis=1)
            N = keys.shape[1]
            qh = q.reshape(B, n, H, dh)
            kh = keys.reshape(B, N, H, dh)
            vh = vals.reshape(B, N, H, dh)
            scores = np.einsum("bihd,bjhd->bhij", qh, kh) / np.sqrt(self.dt.type(dh))
            allowed = np.arange(N)[None, :] <= (t0 + np.arange(n))[:, None]   # key j+1 <= query position
            scores = np.where(allowed[None, None], scores, -np.inf)
            scores = scores - scores.max(axis=-1, keepdims=True)
            w = np.exp(scores)
            w = w / w.sum(axis=-1, keepdims=True)
            o = np.einsum("bhij,bjhd->bihd", w, vh).reshape(B, n, H * dh)
            h = h + o @ self.p(f"enc.{l}.wo").T
            h = h + self.swiglu(self.rms(h, self.p(f"enc.{l}.n2")), self.p(f"enc.{l}.w1"),
                                self.p(f"enc.{l}.w3"), self.p(f"enc.{l}.w2"))
        for i in range(n):
            self._append_memory(st, h[:, i], t0 + 1 + i)
            st.e.append(h[:, i])
        st.n_enc = t0 + n
        return h

    def _append_memory(self, st: "OracleState", e: np.ndarray, t: int) -> None:
        """Memory entry at t: k^g_t = RoPE_t(W^g_K RMSNorm_E(e_t)), v^g_t = W^g_V RMSNorm_E(e_t) ([R] §2, eq 2.1-2.2)."""
        if self.cfg.L_D == 0:
            return
        en = self.rms(e, self.p("mem.nE"))
        for g in range(self.cfg.groups):
            st.mem_k[g].append(self.rope(en @ self.p(f"mem.{g}.wk").T, t))
            st.mem_v[g].append(en @ self.p(f"mem.{g}.wv").T)

    # ------------------------------------------------------------- transition
    def merge(self, e: np.ndarray, s_prev: np.ndarray) -> np.ndarray:
        """u_t = e_t + alpha * g_t * (W_s r), r = RMSNorm_s(s_prev), g_t = sigmoid(W_g [e_t ; r] + b_g) ([S] §2.5; [R] §3.3 eq 2.9-2.11)."""
        r = self.rms(s_prev, self.p("merge.ns"))
        g = self.sigmoid(np.concatenate([e, r], axis=-1) @ self.p("merge.wg").T + self.p("merge.bg"))
        return e + self.dt.type(self.cfg.alpha) * g * (r @ self.p("merge.ws").T)

    def transition(self, st: "OracleState", u: np.ndarray, t: int) -> np.ndarray:
        """H_t = D_phi(u_t; M_<=t, C^D_{t-1}, t): L_D blocks of SWA -> cross -> FFN ([S] §2.3, §2.5; [R] §3.3 eq 2.12-2.16).

        The current key/value comes from the layer input before attention; the
        window holds positions max(1, t-W+1)..t; after the update layer l keeps
        positions max(1, t-W+2)..t (empty when W = 1).
        """
        cfg = self.cfg
        W = cfg.window
        z = u
        for l in range(cfg.L_D):
            a = self.rms(z, self.p(f"dec.{l}.m1"))
            q = self.rope(a @ self.dec_w(l, "wq").T, t)
            k = self.rope(a @ self.dec_w(l, "wk").T, t)
            v = a @ self.dec_w(l, "wv").T
            ring = st.rings[l]
            ring[t] = (k, v)
            win = [p for p in sorted(ring) if max(1, t - W + 1) <= p <= t]
            keys = np.stack([ring[p][0] for p in win], axis=1)
            vals = np.stack([ring[p][1] for p in win], axis=1)
            z = z + self.attend(q, keys, vals) @ self.dec_w(l, "wo").T
            for p in list(ring):
                if p < t - W + 2:
                    del ring[p]
            assert sorted(ring) == list(range(max(1, t - W + 2), t + 1))
            b = self.rms(z, self.p(f"dec.{l}.m2"))
            qx = self.rope(b @ self.p(f"dec.{l}.xq").T, t)
            g = self.group_of(l)
            mk = np.stack(st.mem_k[g][:t], axis=1)          # prefix M_<=t only
            mv = np.stack(st.mem_v[g][:t], axis=1)
            z = z + self.attend(qx, mk, mv) @ self.p(f"dec.{l}.xo").T
            z = z + self.swiglu(self.rms(z, self.p(f"dec.{l}.m3")), self.dec_w(l, "w1"),
                                self.dec_w(l, "w3"), self.dec_w(l, "w2"))
            self.block_steps += 1
        return z

    def readout(self, s: np.ndarray) -> np.ndarray:
        """logits = W_out RMSNorm_out(s_t) ([S] §2.3)."""
        return self.rms(s, self.p("out.nO")) @ self.p("out.w").T

    def decode(self, st: "OracleState", n: int) -> tuple:
        """Consume the next n encoded positions in order, one transition each ([S] §2.4, §2.7; [R] §3.1 eq 2.7).

        RLT-1 merges with s_{t-1}; RLT-2 merges with the chunk register rho,
        replaced by s_t only when t closes a complete chunk (chunks anchored at
        BOS = position 1); RLT-0 passes u_t = e_t. Returns logits [B, n, V] and
        s [B, n, d].
        """
        cfg = self.cfg
        logits, states = [], []
        for _ in range(n):
            t = st.n_dec + 1
            assert t <= st.n_enc, "decoder position ahead of the encoder"
            e = st.e[t - 1]
            if cfg.variant == V0:
                u = e
            elif cfg.variant == V1:
                u = self.merge(e, st.s)
            else:
                u = self.merge(e, st.rho)
            s = self.transition(st, u, t) if cfg.L_D > 0 else u
            st.s = s
            if cfg.variant == V2 and t % cfg.chunk == 0:
                st.rho = s
            st.n_dec = t
            logits.append(self.readout(s))
            states.append(s)
        return np.stack(logits, axis=1), np.stack(states, axis=1)

    # ------------------------------------------------------------- procedures
    def prefill(self, st: "OracleState", tokens: np.ndarray) -> tuple:
        """Recurrent prompt prefill: parallel causal encode, then sequential transitions ([S] §2.4, appendix F.1)."""
        self.encoder_chunk(st, tokens)
        return self.decode(st, tokens.shape[1])

    def consume(self, st: "OracleState", x: np.ndarray) -> tuple:
        """Generation: encoder step, memory append, one transition; logits predict the next token ([S] §2.4, appendix F.2)."""
        self.encoder_step(st, x)
        logits, s = self.decode(st, 1)
        return logits[:, 0], s[:, 0]

    def replay(self, tokens: np.ndarray) -> tuple:
        """Current-policy replay from H_0: log p(x_{t+1} | x_<=t) for t = 1..T-1 ([R] §6.2 eq 5.5; [S] §2.8).

        Returns (logprob [B, T-1], logits [B, T, V], s [B, T, d]); the
        log-sum-exp runs in float64.
        """
        B, T = tokens.shape
        st = self.new_state(B)
        logits, s = self.prefill(st, tokens)
        lp = log_softmax64(logits[:, :T - 1])
        nxt = tokens[:, 1:]
        logprob = np.take_along_axis(lp, nxt[..., None].astype(np.int64), axis=-1)[..., 0]
        return logprob, logits, s


def log_softmax64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    return x - m - np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True))


class OracleState:
    """Per-batch state: s, rho, decoder rings C^D, encoder cache C^E, memory M, and encoded e_t."""

    def __init__(self, cfg, B: int, dt):
        self.B = B
        self.s: Optional[np.ndarray] = None
        self.rho: Optional[np.ndarray] = None
        self.n_enc = 0
        self.n_dec = 0
        self.e: List[np.ndarray] = []
        self.enc_k: List[List[np.ndarray]] = [[] for _ in range(cfg.L_E)]
        self.enc_v: List[List[np.ndarray]] = [[] for _ in range(cfg.L_E)]
        self.mem_k: List[List[np.ndarray]] = [[] for _ in range(cfg.groups)]
        self.mem_v: List[List[np.ndarray]] = [[] for _ in range(cfg.groups)]
        self.rings: List[dict] = [dict() for _ in range(cfg.L_D)]

    def ring_positions(self, l: int) -> List[int]:
        return sorted(self.rings[l])
