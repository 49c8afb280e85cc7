"""Pins of the gradient oracle (CPU only).

The gradient oracle re-expresses the replay with torch float64 tensors and differentiates
it. Two facts pin it from outside itself:
  1. its forward equals the numpy oracle's replay (an independent implementation of the
     same definition: per-position loops with caches, ring eviction, separate parallel and
     incremental encoders), on every variant and option the gradient supports;
  2. its gradient equals central finite differences of the loss (the definition of a
     derivative), on random coordinates of every parameter tensor; a dropped path (state,
     evicted window entries, memory) or a wrong sign shows up as a mismatch there.
"""
import numpy as np
import pytest

from oracle import Oracle
from oracle.rlt_grad import GradOracle
from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens, manifest

TINY = CONFIGS["tiny_fp32"]

CASES = {
    "rlt1": dict(),
    "rlt0": dict(variant=0),
    "rlt2_k3": dict(variant=2, chunk=3),
    "groups_per_layer": dict(groups=2),
    "shared": dict(share=True),
    "window1": dict(window=1),
    "no_decoder": dict(L_D=0),
}


def small(**kw):
    # d 16, 2 heads of 8, f 32, T 9: finite differences of every coordinate stay cheap
    base = dict(d=16, n_heads=2, d_head=8, ffn=32, vocab=8, seq_len=9, batch=2, window=3)
    base.update(kw)
    return TINY.replace(**base)


def loss_weights(cfg, seed=7):
    return np.random.default_rng(seed).standard_normal((cfg.batch, cfg.seq_len - 1))


@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_equals_numpy_oracle(case):
    cfg = TINY.replace(**CASES[case])
    P = make_params(cfg)
    x = make_tokens(cfg)
    ref, _, _ = Oracle(cfg, P).replay(x)
    with __import__("torch").no_grad():
        got = GradOracle(cfg, P).replay(x).numpy()
    assert np.max(np.abs(got - ref)) < 1e-11


@pytest.mark.parametrize("case", sorted(CASES))
def test_gradient_equals_finite_differences(case):
    cfg = small(**CASES[case])
    P = make_params(cfg, std=0.3)
    x = make_tokens(cfg)
    w = loss_weights(cfg)
    go = GradOracle(cfg, P)
    _, G = go.grad(x, w)
    rng = np.random.default_rng(11)
    h = 1e-5
    for name, shape in manifest(cfg):
        flat = np.asarray(P[name], dtype=np.float64).reshape(-1)
        for idx in rng.choice(flat.size, size=min(3, flat.size), replace=False):
            Pp = {k: np.array(v, dtype=np.float64) for k, v in P.items()}
            Pm = {k: np.array(v, dtype=np.float64) for k, v in P.items()}
            Pp[name].reshape(-1)[idx] += h
            Pm[name].reshape(-1)[idx] -= h
            fd = (GradOracle(cfg, Pp).loss(x, w) - GradOracle(cfg, Pm).loss(x, w)) / (2 * h)
            an = G[name].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-6 + 1e-5 * abs(fd), (name, idx, fd, an)


def test_zero_weights_give_zero_gradient():
    cfg = small()
    P = make_params(cfg, std=0.3)
    x = make_tokens(cfg)
    _, G = GradOracle(cfg, P).grad(x, np.zeros((cfg.batch, cfg.seq_len - 1)))
    assert all(np.all(g == 0) for g in G.values())
