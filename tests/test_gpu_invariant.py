"""Batch-invariant mode (rlt_set_batch_invariant): step == replay bit for bit.

In this mode a row's arithmetic does not depend on the batch, the positions per call or
the serving split, so for every variant and 16-bit type:
- a full prefill (token-parallel encode + scan), BOS then one rlt_step per token, and a
  7-token prefill then steps give identical logits, bit for bit;
- the first rows of a batch equal the same rows run as a smaller batch, bit for bit;
- the logits still meet the oracle bar (1e-4 fp32, 2e-2 16-bit);
- generation then replay at temperature 1: the importance ratio is exactly 1 (the replay's
  log-probabilities equal the recorded behaviour log-probabilities bit for bit), the
  pages' sampler / trainer agreement with equal kernels (review §6.2-§6.3).
"""
import numpy as np
import pytest
import torch

from oracle import Oracle, V0, V2
from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens

pytestmark = pytest.mark.gpu
TINY = CONFIGS["tiny_fp32"]
ALGO = CONFIGS["algo_bf16"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load()
    yield


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda()


def run(m, cfg, x, p):
    """prefill x[:, :p] (logits), then rlt_step over the rest; logits [B, T, V] on the host."""
    B, T = x.shape
    st = m.state(B, T, keep_encoder_cache=True)
    xt = dev(x)
    lg, _ = m.prefill(st, xt[:, :p].contiguous())
    out = [lg] + [m.step(st, xt[:, i].contiguous())[:, None] for i in range(p, T)]
    torch.cuda.synchronize()
    return torch.cat(out, 1).cpu().numpy()


CASES = {
    "tiny_fp32_rlt1": (TINY, {}),
    "algo_bf16_rlt1": (ALGO, dict(batch=16, seq_len=40, compute="bf16")),
    "algo_bf16_rlt0": (ALGO, dict(batch=16, seq_len=40, variant=V0, compute="bf16")),
    "rlt2_bf16_k4_GLD": (CONFIGS["rlt2_bf16"], dict(batch=16, seq_len=40, compute="bf16")),
    "algo_fp16_rlt1": (ALGO, dict(batch=16, seq_len=40, compute="fp16")),
    "algo_fp16x2_rlt1": (ALGO, dict(batch=16, seq_len=40, compute="fp16x2")),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_step_equals_replay_bitwise(case):
    base, kw = CASES[case]
    cfg = base.replace(**kw)
    P = make_params(cfg)
    x = make_tokens(cfg)[:, :cfg.seq_len]
    print(f"[case] batch-invariant {case} B={x.shape[0]} T={x.shape[1]}", flush=True)
    m = rlt.Model(cfg, P)
    try:
        rlt.rlt_set_batch_invariant(m.h, True)
        full = run(m, cfg, x, x.shape[1])
        steps = run(m, cfg, x, 1)
        mixed = run(m, cfg, x, 7)
        small = run(m, cfg, x[:4], 7)
        rlt.rlt_set_batch_invariant(m.h, False)
        default_steps = run(m, cfg, x, 1)
        default_full = run(m, cfg, x, x.shape[1])
    finally:
        m.close()
    assert np.array_equal(full, steps)
    assert np.array_equal(full, mixed)
    assert np.array_equal(full[:4], small)
    d = float(np.max(np.abs(default_full - default_steps)))
    _, ref, _ = Oracle(cfg, P, np.float32).replay(x[:4])
    err = float(np.max(np.abs(full[:4] - ref)))
    bar = 1e-4 if cfg.dtype == "fp32" else 2e-2
    print(f"[parity] {case}: invariant replay == steps == 7+steps == batch-4 rows, bit for bit; "
          f"vs oracle (rows 0-3) {err:.3e}; default mode step-vs-replay diff {d:.3e}", flush=True)
    assert err <= bar


def test_generation_replay_ratio_exactly_one():
    cfg = ALGO.replace(batch=16, seq_len=40)
    P = make_params(cfg)
    x = make_tokens(cfg)
    p, n = 10, 20
    m = rlt.Model(cfg, P)
    try:
        rlt.rlt_set_batch_invariant(m.h, True)
        st = m.state(cfg.batch, p + n + 1, keep_encoder_cache=True)
        xt = dev(x)
        m.prefill(st, xt[:, :p].contiguous(), want_logits=False)
        tok = torch.empty((cfg.batch, n), dtype=torch.int32, device="cuda")
        lp_mu = torch.empty((cfg.batch, n), dtype=torch.float32, device="cuda")
        rlt.rlt_generate(m.h, st, xt[:, p].contiguous(), n, 1.0, 5, 0, tok, lp_mu)
        hist = torch.cat([xt[:, :p + 1], tok], 1).contiguous()
        rs = m.state(cfg.batch, hist.shape[1], keep_encoder_cache=False)
        lp_cur, _ = m.replay(rs, hist)
        cur = lp_cur[:, p:].contiguous()
        ratio = torch.empty_like(cur)
        rlt.rlt_importance_ratio(cur, lp_mu, ratio)
        torch.cuda.synchronize()
        r = ratio.cpu().numpy()
        same = bool(torch.equal(cur, lp_mu))
    finally:
        m.close()
    print(f"[parity] batch-invariant generation -> replay: log-probs identical {same}; "
          f"ratio min {r.min():.9f} max {r.max():.9f} over {r.size} draws", flush=True)
    assert same
    assert np.all(r == 1.0)
