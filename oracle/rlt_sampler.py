"""Oracle of behaviour sampling, its recorded log-probabilities and the importance ratio.

TEST INFRASTRUCTURE ONLY, under the same rule as rlt_oracle: only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it. It shares no code
with the HIP library or its binding.

Sources (web pages about the method; citations name the page and the section):
  [R] jiphyeonjeon.kr/blog/rlt, "Recurrent Looped Transformer" (review of the
      technical report): §6.2 and its Figure 4 -- the sampler draws each response
      token from the behaviour policy mu and records log mu(y_i | c, y_<i) under
      the sampling law actually used, temperature included; the trainer replays
      with the current parameters and forms r_i = exp(log p_Theta - log mu)
      (eq 5.5). The same section notes that truncated behaviour sampling (top-k,
      top-p) breaks the support condition p_Theta << mu that exact importance
      sampling needs, so only the full softmax at a temperature is offered.
  [S] greeksharifa.github.io, "Recurrent Looped Transformer 요약 설명", appendix F.2
      (generation: the last emitted token is consumed once before continuing).

Readings taken here (listed in the design notes):
  - mu = softmax(logits / tau) over the whole vocabulary. A draw is the Gumbel-max
    form of it: token = argmax_j (logits_j / tau + G_j), G_j = -log(-log U_j), which
    is distributed exactly as mu (a textbook property of the Gumbel distribution).
    tau = 0 is greedy decoding: argmax of the logits, lowest index on ties, and
    log mu = 0 (a point mass).
  - U_j comes from Philox4x64-10, the counter-based generator of Salmon, Moraes,
    Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011),
    written here from that definition: ten rounds of the two 64-bit
    multiply-high/low S-boxes with the key advanced by the Weyl constants between
    rounds. Row b, vocabulary entry j, draw index `step`: key (seed, 0), counter
    (j // 4, b, step, 0), output word j % 4, U = ((x >> 11) + 0.5) * 2^-53.
  - Scores, the log-sum-exp and the ratio are evaluated in float64 from the fp32
    logits; the recorded log-probability and the ratio are rounded to fp32.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
# S-box multipliers and Weyl key increments of Philox4x64 (Salmon et al., SC 2011)
PHILOX_M0, PHILOX_M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
PHILOX_W0, PHILOX_W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B


def philox4x64_10(ctr, key):
    """One Philox4x64-10 block: four 64-bit words from a 256-bit counter and a 128-bit key."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in ctr)
    k0, k1 = (int(x) & MASK64 for x in key)
    for r in range(10):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = (p1 >> 64) ^ c1 ^ k0, p1 & MASK64, (p0 >> 64) ^ c3 ^ k1, p0 & MASK64
    return c0, c1, c2, c3


def uniforms(b: int, V: int, seed: int, step: int) -> np.ndarray:
    """U[j] in (0, 1) for row b, j = 0..V-1 (float64)."""
    u = np.empty(V, dtype=np.float64)
    for jb in range((V + 3) // 4):
        words = philox4x64_10((jb, b, step, 0), (seed, 0))
        for w in range(4):
            j = 4 * jb + w
            if j < V:
                u[j] = ((words[w] >> 11) + 0.5) * 2.0 ** -53
    return u


def sample(logits: np.ndarray, temperature: float, seed: int, step: int):
    """Draw one token per row from softmax(logits / temperature) and record log mu of it ([R] §6.2).

    logits: fp32 [B, V]. Returns (tokens int32 [B], logprob fp32 [B], scores float64 [B, V])
    where scores are the Gumbel-perturbed values whose argmax is the token (the
    plain logits when temperature is 0).
    """
    logits = np.asarray(logits, dtype=np.float32)
    B, V = logits.shape
    tokens = np.empty(B, dtype=np.int32)
    logprob = np.empty(B, dtype=np.float32)
    scores = np.empty((B, V), dtype=np.float64)
    tau = float(np.float32(temperature))
    for b in range(B):
        if tau == 0.0:
            scores[b] = logits[b].astype(np.float64)
            tokens[b] = int(np.argmax(logits[b]))          # first maximum: lowest index on ties
            logprob[b] = 0.0
            continue
        z = logits[b].astype(np.float64) / tau
        g = -np.log(-np.log(uniforms(b, V, seed, step)))
        y = z + g
        scores[b] = y
        tok = int(np.argmax(y))
        m = z.max()
        lse = m + np.log(np.sum(np.exp(z - m)))
        tokens[b] = tok
        logprob[b] = np.float32(z[tok] - lse)
    return tokens, logprob, scores


def importance_ratio(logp_current: np.ndarray, logp_behaviour: np.ndarray) -> np.ndarray:
    """r_i = exp(log p_Theta - log mu) ([R] §6.2 eq 5.5), float64 inside, fp32 out."""
    d = np.asarray(logp_current, dtype=np.float64) - np.asarray(logp_behaviour, dtype=np.float64)
    return np.exp(d).astype(np.float32)


def generate(oracle, st, first: np.ndarray, n: int, temperature: float, seed: int, step0: int):
    """Generation with behaviour sampling ([S] appendix F.2; [R] §6.2 Figure 4).

    Consumes `first` (the last emitted token of every row), then n times: logits of
    the next position, draw x ~ mu with draw index step0 + i, record it and its
    log mu, and consume it before the next draw -- except after the last draw, whose
    token is returned unconsumed. Returns (tokens [B, n], logprob [B, n],
    logits [B, n, V], scores [B, n, V]).
    """
    x = np.asarray(first, dtype=np.int32)
    toks, lps, lgs, scs = [], [], [], []
    for i in range(n):
        logits, _ = oracle.consume(st, x)
        x, lp, sc = sample(np.asarray(logits, dtype=np.float32), temperature, seed, step0 + i)
        toks.append(x)
        lps.append(lp)
        lgs.append(np.asarray(logits, dtype=np.float32))
        scs.append(sc)
    return (np.stack(toks, axis=1), np.stack(lps, axis=1), np.stack(lgs, axis=1), np.stack(scs, axis=1))
