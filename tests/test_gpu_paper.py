"""Full-size GPU parity at the paper's reference shape against stored oracle outputs.

Workload: 48 + 48 blocks with the attention / FFN weights shared between the encoder
and decoder stacks, d 4096, 32 x 128 heads, SwiGLU 11008, vocab 32000, W 1024, G 1,
RLT-1, batch 64, Zipf prompt (11.7 B parameters; every input from the seeded
generators).

- Replay of the first 16 positions at the full batch of 64, rows 0-1 against the
  oracle (tests/golden/paper_shared.npz, written by tests/golden/make_golden.py from
  the oracle alone).
- Generation: prefill of 8 positions with the encoder cache kept, then 8 rlt_step
  calls consuming the stream's next tokens; rows 0-1 at positions 9-16 against the
  oracle on every id.
- The full 8192-token prompt encoded at batch 64, then the decoder scan of its
  first 16 positions: the same logits as the 16-position run, bit for bit (encoder
  causality and memory prefix restriction hold at any length, and every kernel's
  per-row arithmetic is independent of the row count).
"""
import os

import numpy as np
import pytest
import torch

from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CFG = CONFIGS["paper_shared"]
# Logit bar at this shape. The 2e-2 used for the smaller 16-bit shapes is below what 16-bit
# attention operands allow at 48 + 48 blocks of width 4096: the oracle itself, with nothing
# but the encoder's queries and keys rounded to fp16, moves its logits by 1.8e-2 over these
# 16 positions, and the fp16x2 path (two-term GEMM inputs, fp16 caches) measures 2.5e-2.
# The bar here is 3e-2 on logits, 2e-2 on log-probabilities, plus the argmax rule.
TOL = 3e-2
TOL_LP = 2e-2
T_SHORT = 16


def argmax_check(gpu_argmax, top_idx, top_val, err):
    raw = gpu_argmax == top_idx[..., 0]
    hit = top_idx == gpu_argmax[..., None]
    near = np.any(hit & (top_val >= top_val[..., :1] - 2 * err), axis=-1)
    return float(np.mean(raw | near)), float(np.mean(raw))


@pytest.fixture(scope="module")
def paper():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    path = os.path.join(GOLDEN, "paper_shared.npz")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run tests/golden/make_golden.py paper_shared --rows 2 --len 16")
    g = dict(np.load(path))
    tokens = make_tokens(CFG)                          # [64, 8704]
    assert np.array_equal(tokens[:2, :T_SHORT], g["tokens"]), "seeded token stream changed"
    print("[case] paper_shared: drawing 11.7 B parameters", flush=True)
    P = make_params(CFG, bf16_storage=True)
    keys = [k for k in ("emb", "out.w", "merge.s0") if k in P]
    probe = np.concatenate([np.asarray(P[k]).ravel()[:8] for k in keys]).astype(np.float32)
    assert np.array_equal(probe, g["param_probe"]), "seeded parameter draw changed"
    print("[case] paper_shared: creating model", flush=True)
    m = rlt.Model(CFG, P)
    del P
    torch.cuda.synchronize()
    yield m, tokens, g
    m.close()


def short_replay(m, tokens):
    B = tokens.shape[0]
    st = m.state(B, T_SHORT, keep_encoder_cache=False)
    x = torch.as_tensor(np.ascontiguousarray(tokens[:, :T_SHORT])).cuda()
    lg = torch.empty((B, T_SHORT, CFG.vocab), dtype=torch.float32, device="cuda")
    s = torch.empty((B, T_SHORT, CFG.d), dtype=torch.float32, device="cuda")
    rlt.rlt_encode(m.h, st, x)
    rlt.rlt_decode_scan(m.h, st, T_SHORT, logits=lg, s_out=s)
    lp, _ = m.replay(st, x)
    torch.cuda.synchronize()
    return lg, lp, s


def test_paper_replay_vs_oracle(paper):
    m, tokens, g = paper
    print(f"[case] paper_shared replay B={tokens.shape[0]} T={T_SHORT}", flush=True)
    lg, lp, s = short_replay(m, tokens)
    r = lg[:2].cpu().numpy()
    err_h = float(np.max(np.abs(r[:, :, :64] - g["logits_head"])))
    err_t = float(np.max(np.abs(r[:, -8:, :] - g["logits_tail"])))
    err = max(err_h, err_t)
    agree, raw = argmax_check(lg[:2].argmax(-1).cpu().numpy(), g["top8_idx"], g["top8_val"], err)
    lp_err = float(np.max(np.abs(lp[:2].cpu().numpy() - g["logprob"])))
    s_err = float(np.max(np.abs(s[:2, -1].cpu().numpy() - g["s_last"])))
    print(f"[parity] paper_shared replay rows 0-1 x positions 1-16: logits err first-64 ids {err_h:.3e}, "
          f"positions 9-16 all ids {err_t:.3e}; argmax agreement {agree:.5f} (raw {raw:.5f}); "
          f"log-prob err {lp_err:.3e}; s_T err {s_err:.3e}", flush=True)
    assert err <= TOL
    assert agree >= 0.999
    assert lp_err <= TOL_LP


def test_paper_generation_steps_vs_oracle(paper):
    m, tokens, g = paper
    B, p = tokens.shape[0], 8
    print(f"[case] paper_shared generation: prefill {p} then {T_SHORT - p} rlt_step at B={B}", flush=True)
    st = m.state(B, T_SHORT, keep_encoder_cache=True)
    x = torch.as_tensor(np.ascontiguousarray(tokens[:, :T_SHORT])).cuda()
    rlt.rlt_encode(m.h, st, x[:, :p].contiguous())
    rlt.rlt_decode_scan(m.h, st, p)
    steps = [m.step(st, x[:, i].contiguous()) for i in range(p, T_SHORT)]
    torch.cuda.synchronize()
    lg = torch.stack(steps, dim=1)[:2].cpu().numpy()            # positions 9..16, rows 0-1
    err = float(np.max(np.abs(lg - g["logits_tail"])))
    print(f"[parity] paper_shared rlt_step rows 0-1 positions 9-16 vs oracle, every id: max abs err {err:.3e}",
          flush=True)
    assert err <= TOL


def test_paper_full_prompt_encode_prefix_invariance(paper):
    m, tokens, _ = paper
    B, T = tokens.shape[0], CFG.seq_len
    lg_short, _, _ = short_replay(m, tokens)
    free, total = torch.cuda.mem_get_info()
    print(f"[case] paper_shared full encode B={B} T={T}, then scan of {T_SHORT} positions "
          f"(device memory free {free / 2**30:.1f} of {total / 2**30:.1f} GiB)", flush=True)
    st = m.state(B, T, keep_encoder_cache=False)
    x = torch.as_tensor(np.ascontiguousarray(tokens[:, :T])).cuda()
    rlt.rlt_encode(m.h, st, x)
    lg = torch.empty((B, T_SHORT, CFG.vocab), dtype=torch.float32, device="cuda")
    rlt.rlt_decode_scan(m.h, st, T_SHORT, logits=lg)
    torch.cuda.synchronize()
    d = float((lg - lg_short).abs().max())
    print(f"[parity] paper_shared first {T_SHORT} positions after the {T}-token encode vs the "
          f"{T_SHORT}-token run: max abs diff {d:.3e}", flush=True)
    assert d == 0.0
