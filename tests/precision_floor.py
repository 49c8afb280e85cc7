"""How far 16-bit attention operands alone move the oracle's logits (precision study).

Runs the CPU oracle (float32) with chosen intermediates rounded as the GPU path stores
them, and reports the largest logit change against the unrounded oracle. It answers
"which operand has to carry more than 16 bits at this shape for the logits to stay
within a tolerance", independently of the GPU: nothing here calls the HIP library.

Rounding points (each "fp16", "bf16", "fp16x2" = two fp16 terms hi + lo, or absent):
  enc_qk   encoder self-attention queries and keys (after the rotary map)
  enc_v    encoder self-attention values
  enc_p    encoder attention probabilities exp(s - max) before they weight the values
  mem_kv   memory keys and values (what cross-attention reads)
  swa_qkv  decoder window query, keys and values
  cross_q  decoder cross-attention query
  act      inputs of the projections: every RMSNorm output
  enc_act  the encoder's projection inputs: its RMSNorm outputs (blocks and memory norm), its
           attention outputs and SwiGLU hidden rows
  dec_act  the decoder's projection inputs: its RMSNorm outputs (merge, blocks, readout), its
           attention outputs and SwiGLU hidden rows

The encoder runs token by token here (the oracle's incremental encoder, pinned equal to
its parallel form), so every attention goes through Oracle.attend.

    python -m tests.precision_floor paper_shared --positions 16 --param-cache DIR
"""
from __future__ import annotations

import argparse
import json
import time

import numpy as np

from oracle import Oracle
from recurrent_looped_transformer_amd.synth import CONFIGS, file_params, make_params, make_tokens, round_bf16

POINTS = ("enc_qk", "enc_v", "enc_p", "mem_kv", "swa_qkv", "cross_q", "act", "enc_act", "dec_act")


def rounder(kind):
    if kind is None:
        return None
    if kind == "fp16":
        return lambda x: np.asarray(x, np.float32).astype(np.float16).astype(np.float32)
    if kind == "bf16":
        return lambda x: round_bf16(np.asarray(x, np.float32))
    if kind == "fp16x2":
        def two(x):
            x = np.asarray(x, np.float32)
            hi = x.astype(np.float16).astype(np.float32)
            lo = (x - hi).astype(np.float16).astype(np.float32)
            return hi + lo
        return two
    raise ValueError(kind)


class RoundingOracle(Oracle):
    """The oracle with 16-bit storage emulated at the chosen points (float32 otherwise)."""

    def __init__(self, cfg, params, spec, dtype=np.float32):
        super().__init__(cfg, params, dtype)
        self.r = {k: rounder(spec.get(k)) for k in POINTS}
        self._ctx = ""
        self._calls = 0

    def _rd(self, point, x):
        f = self.r[point]
        return x if f is None else f(x).astype(self.dt)

    def rms(self, x, gain):
        y = super().rms(x, gain)
        if gain is None:
            return y
        y = self._rd("act", y)
        return self._rd("enc_act" if self._ctx == "enc" else "dec_act", y)

    def swiglu(self, x, w1, w3, w2):
        point = "enc_act" if self._ctx == "enc" else "dec_act"
        if self.r[point] is None:
            return super().swiglu(x, w1, w3, w2)
        a = x @ w1.T
        b = x @ w3.T
        return self._rd(point, a * self.sigmoid(a) * b) @ w2.T

    def attend(self, q, keys, vals):
        if self._ctx == "enc":
            q, keys, vals = self._rd("enc_qk", q), self._rd("enc_qk", keys), self._rd("enc_v", vals)
            pr = self.r["enc_p"]
        else:
            cross = self._calls % 2 == 1
            self._calls += 1
            if cross:
                q = self._rd("cross_q", q)
                keys, vals = self._rd("mem_kv", keys), self._rd("mem_kv", vals)
            else:
                q, keys, vals = (self._rd("swa_qkv", a) for a in (q, keys, vals))
            pr = None
        if pr is None:
            out = super().attend(q, keys, vals)
            return self._rd("enc_act" if self._ctx == "enc" else "dec_act", out)
        H, dh = self.cfg.n_heads, self.cfg.d_head
        B, n = keys.shape[0], keys.shape[1]
        s = np.einsum("bhd,bnhd->bhn", q.reshape(B, H, dh), keys.reshape(B, n, H, dh)) / np.sqrt(self.dt.type(dh))
        e = np.exp(s - s.max(axis=-1, keepdims=True))
        out = np.einsum("bhn,bnhd->bhd", pr(e).astype(self.dt), vals.reshape(B, n, H, dh))
        return self._rd("enc_act", (out / e.sum(axis=-1)[..., None]).reshape(B, H * dh))

    def encoder_step(self, st, x):
        self._ctx = "enc"
        try:
            return super().encoder_step(st, x)
        finally:
            self._ctx = ""

    def _append_memory(self, st, e, t):
        super()._append_memory(st, e, t)
        if self.cfg.L_D > 0 and self.r["mem_kv"] is not None:
            for g in range(self.cfg.groups):
                st.mem_k[g][-1] = self._rd("mem_kv", st.mem_k[g][-1])
                st.mem_v[g][-1] = self._rd("mem_kv", st.mem_v[g][-1])

    def logits(self, tokens):
        st = self.new_state(tokens.shape[0])
        for i in range(tokens.shape[1]):
            self.encoder_step(st, tokens[:, i])
        lg, _ = self.decode(st, tokens.shape[1])
        return lg


def logit_shift(cfg, P, tokens, spec):
    """max |logits(spec) - logits(float32 oracle)| over every position and id."""
    ref = RoundingOracle(cfg, P, {}).logits(tokens)
    got = RoundingOracle(cfg, P, spec).logits(tokens)
    return float(np.max(np.abs(got - ref)))


# What the GPU path stores with two-term GEMM inputs: the encoder's attention operands two-term,
# the decoder's (memory, window, queries) one fp16 term.
GPU_FP16X2 = {"enc_qk": "fp16x2", "enc_v": "fp16x2", "enc_p": "fp16x2", "mem_kv": "fp16", "swa_qkv": "fp16",
              "cross_q": "fp16"}

STUDY = [
    {"enc_qk": "fp16"}, {"enc_v": "fp16"}, {"enc_p": "fp16"}, {"mem_kv": "fp16"},
    {"swa_qkv": "fp16"}, {"cross_q": "fp16"}, {"act": "fp16"},
    {"enc_qk": "fp16", "enc_v": "fp16", "enc_p": "fp16", "mem_kv": "fp16", "swa_qkv": "fp16", "cross_q": "fp16"},
    {"enc_qk": "fp16x2", "enc_v": "fp16", "enc_p": "fp16", "mem_kv": "fp16", "swa_qkv": "fp16", "cross_q": "fp16"},
    {"enc_qk": "fp16x2", "enc_v": "fp16", "enc_p": "fp16", "swa_qkv": "fp16", "cross_q": "fp16"},
    {"enc_qk": "fp16x2", "enc_v": "fp16x2", "enc_p": "fp16x2", "mem_kv": "fp16x2", "swa_qkv": "fp16x2",
     "cross_q": "fp16x2"},
    GPU_FP16X2,
]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("shape")
    ap.add_argument("--positions", type=int, default=16)
    ap.add_argument("--rows", type=int, default=1)
    ap.add_argument("--param-cache", default="")
    ap.add_argument("--only-gpu-spec", action="store_true")
    ap.add_argument("--specs", default="", help="JSON list of specs to run instead of the study")
    args = ap.parse_args()
    cfg = CONFIGS[args.shape]
    P = file_params(cfg, args.param_cache) if args.param_cache else make_params(cfg, bf16_storage=cfg.d >= 4096)
    tokens = make_tokens(cfg, length=cfg.seq_len + cfg.gen_len)[:args.rows, :args.positions]
    ref = RoundingOracle(cfg, P, {}).logits(tokens)
    specs = json.loads(args.specs) if args.specs else ([GPU_FP16X2] if args.only_gpu_spec else STUDY)
    for spec in specs:
        t0 = time.time()
        got = RoundingOracle(cfg, P, spec).logits(tokens)
        print(f"{args.shape} rows {args.rows} x {args.positions} positions {spec}: max logit shift "
              f"{float(np.max(np.abs(got - ref))):.3e} ({time.time() - t0:.0f} s)", flush=True)


if __name__ == "__main__":
    main()
