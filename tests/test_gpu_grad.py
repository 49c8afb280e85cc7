"""GPU parity of the full-BPTT replay gradient (rlt_replay_grad) against the gradient oracle.

The oracle differentiates the replay in float64 (torch reverse mode over the definition,
pinned to the numpy oracle's forward and to finite differences). The GPU path runs fp32
throughout. Bars (derivation: every gradient entry is a sum of fp32 products over up to
T*B rows and through L_E + L_D blocks of T dependent steps; fp32 rounding u = 6e-8 grows
like sqrt(terms) per sum and roughly linearly along the chain, which stays below 1e-5
relative at these sizes; the bars leave a margin of about 5 and 10 above the measured worst):
  - logprob: max |gpu - oracle| <= 2e-5;
  - every parameter gradient: ||gpu - oracle||_2 <= 5e-5 ||oracle||_2 + 1e-7 sqrt(n)
    (measured worst with the MFMA products: 4.2e-6 on logprob (the ragged shape), 4.6e-6
    relative on a gradient (the 512-wide shape)).
Cases: the tiny fp32 configuration and its variants (RLT-0, RLT-2 with K_c = 3, one memory
group per layer, shared encoder/decoder weights, window 1, no decoder), and a ragged shape
(d 128, f 320, B 3, T 37: GEMM tiles with a tail in every dimension, windows that slide).
At the 512-wide shape (4 + 4 blocks, W 32, T 257) the oracle runs on 2 sequences; the full
batch of 64 is then checked on the GPU by additivity: the gradient of a loss summed over
sequences equals the sum of the per-slice gradients.
"""
import numpy as np
import pytest
import torch

from oracle.rlt_grad import GradOracle
from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens, manifest

pytestmark = pytest.mark.gpu
TINY = CONFIGS["tiny_fp32"]
ALGO = CONFIGS["algo_bf16"]

LP_TOL = 2e-5
G_REL, G_ABS = 5e-5, 1e-7

CASES = {
    "rlt1": dict(),
    "rlt0": dict(variant=0),
    "rlt2_k3": dict(variant=2, chunk=3),
    "groups_per_layer": dict(groups=2),
    "shared": dict(share=True),
    "window1": dict(window=1),
    "no_decoder": dict(L_D=0),
    "ragged": dict(d=128, ffn=320, n_heads=4, d_head=32, batch=3, seq_len=37, window=5),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load()
    yield


def to_dev(P):
    return {k: torch.as_tensor(np.ascontiguousarray(v, dtype=np.float32)).cuda() for k, v in P.items()}


def weights_for(cfg, B, T, seed=5):
    return np.random.default_rng(seed).standard_normal((B, T - 1)).astype(np.float32)


def run_gpu(cfg, P, x, w, ck=False):
    lp, G = rlt.rlt_replay_grad(cfg, to_dev(P), torch.as_tensor(x, dtype=torch.int32).cuda(),
                                torch.as_tensor(w).cuda(), checkpoint=ck)
    torch.cuda.synchronize()
    return lp.cpu().numpy().astype(np.float64), {k: v.cpu().numpy().astype(np.float64) for k, v in G.items()}


def compare(cfg, lp, G, lp_ref, G_ref, tag):
    err_lp = float(np.max(np.abs(lp - lp_ref)))
    worst = (0.0, "")
    for name, _ in manifest(cfg):
        a, b = G[name].reshape(-1), G_ref[name].reshape(-1)
        num = float(np.linalg.norm(a - b))
        den = float(np.linalg.norm(b))
        rel = num / max(den, 1e-30)
        assert num <= G_REL * den + G_ABS * np.sqrt(a.size), (tag, name, num, den)
        if den > 1e-12:   # gradients that vanish identically (window 1: dL/dk = 0) have no relative error
            worst = max(worst, (rel, name))
    print(f"[grad] {tag}: logprob max err {err_lp:.2e}; worst gradient rel err {worst[0]:.2e} ({worst[1]})",
          flush=True)
    assert err_lp <= LP_TOL, (tag, err_lp)


@pytest.mark.parametrize("ck", [False, True], ids=["kept", "checkpointed"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_gradient_matches_oracle(case, ck):
    cfg = TINY.replace(**CASES[case])
    P = make_params(cfg, std=0.1)
    x = make_tokens(cfg)
    w = weights_for(cfg, cfg.batch, cfg.seq_len)
    print(f"[grad] case {case} B={cfg.batch} T={cfg.seq_len} checkpoint={ck}", flush=True)
    lp, G = run_gpu(cfg, P, x, w, ck)
    lp_ref, G_ref = GradOracle(cfg, P).grad(x, w.astype(np.float64))
    compare(cfg, lp, G, lp_ref, G_ref, case + (" checkpointed" if ck else ""))


@pytest.mark.parametrize("ck", [False, True], ids=["kept", "checkpointed"])
def test_gradient_is_deterministic(ck):
    """Two calls give the same bits: every reduction (split-K slices of the weight gradients,
    gain / bias column sums, the embedding gradient's per-token sums) adds in a fixed order.
    The 512-wide shape at 4 x 64 positions (weight-gradient products split over k there) and
    the tiny shape."""
    for cfg, B, T in ((TINY, TINY.batch, TINY.seq_len), (ALGO.replace(dtype="fp32", compute="fp32"), 4, 64)):
        P = make_params(cfg, std=0.1 if cfg is TINY else 0.02)
        x = make_tokens(cfg, batch=B, length=T)
        w = weights_for(cfg, B, T)
        lp1, G1 = run_gpu(cfg, P, x, w, ck)
        lp2, G2 = run_gpu(cfg, P, x, w, ck)
        assert np.array_equal(lp1, lp2)
        for k in G1:
            assert np.array_equal(G1[k], G2[k]), k     # float32 values, compared exactly


def test_zero_loss_weights_give_zero_gradient():
    cfg = TINY
    P = make_params(cfg, std=0.1)
    x = make_tokens(cfg)
    _, G = run_gpu(cfg, P, x, np.zeros((cfg.batch, cfg.seq_len - 1), np.float32))
    assert all(np.all(g == 0) for g in G.values())


def algo_fp32():
    return ALGO.replace(dtype="fp32", compute="fp32")


def test_algo_shape_two_sequences_match_oracle():
    """The 512-wide 4 + 4 shape at its full length T = 257 (window 32 slides 225 times),
    2 sequences, against the float64 oracle, with and without checkpointing."""
    cfg = algo_fp32().replace(batch=2)
    P = make_params(cfg)
    x = make_tokens(cfg)
    w = weights_for(cfg, 2, cfg.seq_len)
    print("[grad] algo shape B=2 T=257", flush=True)
    lp_ref, G_ref = GradOracle(cfg, P).grad(x, w.astype(np.float64))
    for ck in (False, True):
        lp, G = run_gpu(cfg, P, x, w, ck)
        compare(cfg, lp, G, lp_ref, G_ref, "algo B=2" + (" checkpointed" if ck else ""))


def test_checkpointed_equals_kept_at_full_batch():
    """B = 64 at T = 257: the checkpointed gradient equals the kept-intermediates one within
    fp32 reassociation (weight gradients summed position by position instead of at once);
    the log-probabilities are identical (the same forward kernels)."""
    cfg = algo_fp32()
    P = make_params(cfg)
    x = make_tokens(cfg)
    w = weights_for(cfg, cfg.batch, cfg.seq_len)
    lp0, G0 = run_gpu(cfg, P, x, w, False)
    lp1, G1 = run_gpu(cfg, P, x, w, True)
    assert np.array_equal(lp0, lp1)
    for name, _ in manifest(cfg):
        a, b = G1[name].reshape(-1), G0[name].reshape(-1)
        assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(b) + 1e-7 * np.sqrt(a.size), name


def test_algo_shape_full_batch_is_sum_of_slices():
    """B = 64 at T = 257: the gradient equals the sum of the gradients of 4 slices of 16
    sequences (each sequence's loss depends on its own tokens only), within fp32
    reassociation; the log-probabilities are equal row for row."""
    cfg = algo_fp32()
    P = make_params(cfg)
    x = make_tokens(cfg)
    w = weights_for(cfg, cfg.batch, cfg.seq_len)
    print("[grad] algo shape B=64 T=257 vs 4 slices of 16", flush=True)
    lp, G = run_gpu(cfg, P, x, w)
    acc = {k: np.zeros_like(v) for k, v in G.items()}
    for s in range(4):
        sl = slice(16 * s, 16 * (s + 1))
        lps, Gs = run_gpu(cfg.replace(batch=16), P, x[sl], w[sl])
        assert np.max(np.abs(lps - lp[sl])) <= 1e-5
        for k in acc:
            acc[k] += Gs[k]
    for name, _ in manifest(cfg):
        a, b = G[name].reshape(-1), acc[name].reshape(-1)
        assert np.linalg.norm(a - b) <= 1e-4 * np.linalg.norm(b) + 1e-7 * np.sqrt(a.size), name
