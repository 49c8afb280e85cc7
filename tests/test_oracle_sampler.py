"""Pins of the sampling oracle (oracle/rlt_sampler.py), CPU only.

- Philox4x64-10 equals numpy's Philox bit generator (a library implementation of the
  same published generator), block by block, including carries of the counter.
- Gumbel-max draws follow softmax(logits / tau): empirical frequencies over 16,000
  draws within 4.5 sigma of the softmax probabilities at two temperatures.
- The recorded behaviour log-probability is scipy's log_softmax(logits / tau) at the
  drawn token; at tau = 1 it is the replay's log-probability definition.
- tau = 0 is greedy decoding with the lowest index on ties and log mu = 0.
- Importance ratio: exp of the difference (closed forms).
- Generation: one call of n draws equals k draws then n - k draws with the draw index
  carried on (the state and the counter are the whole history).
"""
import numpy as np
import scipy.special

from oracle import Oracle, log_softmax64
from oracle.rlt_sampler import generate, importance_ratio, philox4x64_10, sample, uniforms
from recurrent_looped_transformer_amd.synth import CONFIGS, make_logits, make_params, make_tokens

M64 = (1 << 64) - 1


def _numpy_block(ctr, key, blocks=1):
    """numpy's Philox increments the 256-bit counter before each block: start one below."""
    v = (sum(int(x) << (64 * i) for i, x in enumerate(ctr)) - 1) % (1 << 256)
    c = np.array([(v >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(counter=c, key=np.array(key, dtype=np.uint64))
    return [int(x) for x in g.random_raw(4 * blocks)]


def test_philox_equals_numpy_bit_generator():
    cases = [((0, 0, 0, 0), (0, 0)), ((1, 0, 0, 0), (0, 0)), ((7, 3, 11, 0), (12345, 0)),
             ((M64, 0, 5, 0), (2**63 + 1, 9)), ((M64, M64, M64, M64), (M64, M64)),
             ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
              (0x452821E638D01377, 0xBE5466CF34E90C6C))]
    for ctr, key in cases:
        two = _numpy_block(ctr, key, blocks=2)
        assert list(philox4x64_10(ctr, key)) == two[:4]
        nxt = (sum(int(x) << (64 * i) for i, x in enumerate(ctr)) + 1) % (1 << 256)
        nctr = [(nxt >> (64 * i)) & M64 for i in range(4)]
        assert list(philox4x64_10(nctr, key)) == two[4:]


def test_uniforms_open_interval_and_distinct_streams():
    u = uniforms(0, 1000, seed=5, step=0)
    assert np.all(u > 0) and np.all(u < 1)
    assert not np.array_equal(u, uniforms(1, 1000, seed=5, step=0))
    assert not np.array_equal(u, uniforms(0, 1000, seed=5, step=1))
    assert not np.array_equal(u, uniforms(0, 1000, seed=6, step=0))
    assert abs(u.mean() - 0.5) < 0.05


def test_gumbel_max_follows_softmax_at_temperature():
    logits = np.array([[1.5, -0.3, 0.0, 2.2, 0.7]] * 8, dtype=np.float32)
    for tau in (1.0, 0.6):
        p = scipy.special.softmax(logits[0].astype(np.float64) / np.float64(np.float32(tau)))
        counts = np.zeros(5)
        n = 0
        for step in range(2000):
            tok, _, _ = sample(logits, tau, seed=99, step=step)
            np.add.at(counts, tok, 1)
            n += len(tok)
        freq = counts / n
        sigma = np.sqrt(p * (1 - p) / n)
        assert np.all(np.abs(freq - p) <= 4.5 * sigma), (tau, freq, p)


def test_behaviour_logprob_is_log_softmax_at_token():
    logits = make_logits(6, 300, seed=11)
    for tau in (1.0, 0.5, 1.7):
        tok, lp, sc = sample(logits, tau, seed=3, step=4)
        ref = scipy.special.log_softmax(logits.astype(np.float64) / np.float64(np.float32(tau)), axis=-1)
        assert np.allclose(lp, ref[np.arange(6), tok], rtol=0, atol=1e-6)
        assert np.array_equal(tok, np.argmax(sc, axis=-1))
    tok, lp, _ = sample(logits, 1.0, seed=3, step=4)
    assert np.allclose(lp, log_softmax64(logits)[np.arange(6), tok], atol=1e-6)


def test_zero_temperature_is_greedy_lowest_index():
    logits = make_logits(4, 50, seed=12)
    logits[2, 7] = logits[2, 31] = logits[2].max() + 1.0       # exact tie
    tok, lp, _ = sample(logits, 0.0, seed=1, step=0)
    assert np.array_equal(tok, np.argmax(logits, axis=-1))
    assert tok[2] == 7
    assert np.all(lp == 0.0)


def test_importance_ratio_closed_forms():
    a = np.array([-1.25, -3.0, -0.5, 0.0], dtype=np.float32)
    assert np.array_equal(importance_ratio(a, a), np.ones(4, dtype=np.float32))
    r = importance_ratio(np.float32([0.0, -np.log(2)]), np.float32([np.log(2), 0.0]))
    assert np.allclose(r, [0.5, 0.5], rtol=1e-7)
    assert importance_ratio(np.float32([-2.0]), np.float32([-3.0]))[0] == np.float32(np.e)


def test_generation_split_equals_one_call():
    cfg = CONFIGS["tiny_fp32"]
    P = make_params(cfg)
    x = make_tokens(cfg)
    o = Oracle(cfg, P, np.float32)
    a = o.new_state(cfg.batch)
    o.prefill(a, x[:, :5])
    ta, la, _, _ = generate(o, a, x[:, 5], 6, 1.0, seed=42, step0=10)
    b = o.new_state(cfg.batch)
    o.prefill(b, x[:, :5])
    t1, l1, _, _ = generate(o, b, x[:, 5], 2, 1.0, seed=42, step0=10)
    t2, l2, _, _ = generate(o, b, t1[:, -1], 4, 1.0, seed=42, step0=12)
    assert np.array_equal(ta, np.concatenate([t1, t2], axis=1))
    assert np.array_equal(la, np.concatenate([l1, l2], axis=1))
    assert a.n_dec == b.n_dec == 5 + 6
