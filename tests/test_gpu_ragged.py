"""GPU parity of rows at their own positions (continuous batching: rlt_step_rows,
rlt_state_reset_rows, rlt_state_row_positions).

Every row is an independent sequence (the state H_t is per sequence, greeksharifa summary
§2.1), so the oracle runs each row alone, one consume per token, and the GPU's batched rows
at unequal positions must match it: fp32 logits within 1e-4; the 16-bit algorithmic shape
within the 2e-2 logit bar (raw argmax agreement printed). Schedules are seeded: each row moves with
probability 0.6 per call, rows start late, rows fill max_len and stay idle while the others
move (their discarded step lands in the slack position), rows are reset mid-stream and take
a new sequence, RLT-2 rows close chunks at different calls (partial chunks inside a mixed
batch). GPU-only identities: with every row moving, a per-row call equals rlt_step bit for
bit; in batch-invariant mode a mixed batch equals single-row runs of each row bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import Oracle
from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import CONFIGS, make_params

pytestmark = pytest.mark.gpu
TINY = CONFIGS["tiny_fp32"]
ALGO = CONFIGS["algo_bf16"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rlt.load()
    yield


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def run_ragged(cfg, P, B, max_len, calls, seed, resets=None, p_move=0.6, invariant=False):
    """Returns (per-row list of (tokens, logits) in order of consumption, per-row segment starts,
    final positions). Row b's token at its position 1 is BOS, later tokens are drawn uniformly."""
    rng = np.random.default_rng(seed)
    m = rlt.Model(cfg, P)
    if invariant:
        rlt.rlt_set_batch_invariant(m.h, True)
    try:
        st = m.state(B, max_len, keep_encoder_cache=True)
        pos = np.zeros(B, np.int64)
        hist = [[] for _ in range(B)]      # (segment id, token, logits)
        seg = np.zeros(B, np.int64)
        lg = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
        for k in range(calls):
            if resets and k in resets:
                rows = np.zeros(B, np.int32)
                rows[resets[k]] = 1
                rlt.rlt_state_reset_rows(m.h, st, rows)
                pos[resets[k]] = 0
                seg[resets[k]] += 1
            act = (rng.random(B) < p_move) & (pos < max_len)
            toks = np.where(pos == 0, cfg.bos, rng.integers(0, cfg.vocab - 1, size=B)).astype(np.int32)
            rlt.rlt_step_rows(m.h, st, dev(toks), act.astype(np.int32), lg)
            g = lg.cpu().numpy()
            for b in np.nonzero(act)[0]:
                hist[b].append((int(seg[b]), int(toks[b]), g[b].copy()))
                pos[b] += 1
        assert rlt.rlt_state_row_positions(st, B) == [int(p) for p in pos]
        return hist, pos
    finally:
        m.close()


def oracle_rows(cfg, P, hist):
    """Oracle logits for every consumed token of every row, each row (segment) alone."""
    o = Oracle(cfg, P)
    out = []
    for h in hist:
        ref, st, cur = [], None, None
        for sg, tok, _ in h:
            if sg != cur:
                st, cur = o.new_state(1), sg
            lg, _ = o.consume(st, np.array([tok], dtype=np.int64))
            ref.append(lg[0])
        out.append(ref)
    return out


def compare(cfg, hist, ref, bar, tag):
    worst, n, agree = 0.0, 0, 0
    for h, r in zip(hist, ref):
        for (_, _, g), rr in zip(h, r):
            e = float(np.max(np.abs(g - rr)))
            worst = max(worst, e)
            n += 1
            agree += int(np.argmax(g) == np.argmax(rr))
    print(f"[ragged] {tag}: {n} row-steps, max abs logit err {worst:.2e}, raw argmax agreement {agree / n:.4f}",
          flush=True)
    assert worst <= bar, (tag, worst)


CASES = {
    "rlt1": dict(),
    "rlt0": dict(variant=0),
    "rlt2_k3": dict(variant=2, chunk=3),
    "groups_per_layer": dict(groups=2),
    "window1": dict(window=1),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_rows_at_own_positions_match_oracle(case):
    cfg = TINY.replace(**CASES[case])
    P = make_params(cfg)
    B, max_len = 5, 20
    print(f"[ragged] case {case} B={B} max_len={max_len}", flush=True)
    # 60 calls: rows reach max_len and idle; rows 1 and 3 restart at call 38
    hist, pos = run_ragged(cfg, P, B, max_len, 60, seed=17, resets={38: [1, 3]})
    assert max(len(h) for h in hist) > max_len        # some row consumed two sequences
    compare(cfg, hist, oracle_rows(cfg, P, hist), 1e-4, case)


def test_algo_shape_rows_at_own_positions():
    """The 512-wide bf16 shape, 8 rows at staggered positions, against the oracle."""
    cfg = ALGO
    P = make_params(cfg)
    print("[ragged] algo bf16 B=8", flush=True)
    hist, _ = run_ragged(cfg, P, 8, 48, 40, seed=5, resets={30: [0]})
    compare(cfg, hist, oracle_rows(cfg, P, hist), 2e-2, "algo bf16")


def test_all_rows_moving_equals_batch_step():
    """With every row active at every call the per-row path runs the batch-wide step's kernels
    on the same rows: logits bit for bit equal to rlt_step."""
    cfg = ALGO
    P = make_params(cfg)
    B, T = 16, 12
    rng = np.random.default_rng(3)
    x = rng.integers(0, cfg.vocab - 1, size=(B, T)).astype(np.int32)
    x[:, 0] = cfg.bos
    m = rlt.Model(cfg, P)
    try:
        a = m.state(B, T, keep_encoder_cache=True)
        b = m.state(B, T, keep_encoder_cache=True)
        lg = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
        for t in range(T):
            ref = m.step(a, dev(x[:, t]))
            rlt.rlt_step_rows(m.h, b, dev(x[:, t]), np.ones(B, np.int32), lg)
            assert torch.equal(ref, lg), t
        assert rlt.rlt_state_positions(b) == (T, T)   # rows level again: batch-wide view
    finally:
        m.close()


def test_invariant_mode_mixed_batch_equals_single_rows():
    """Batch-invariant arithmetic: each row of a mixed batch equals that row run alone
    (B = 1, rlt_step), bit for bit, at every one of its positions."""
    cfg = ALGO
    P = make_params(cfg)
    B = 6
    hist, _ = run_ragged(cfg, P, B, 24, 30, seed=9, invariant=True)
    m = rlt.Model(cfg, P)
    rlt.rlt_set_batch_invariant(m.h, True)
    try:
        for b in range(B):
            st = m.state(1, 24, keep_encoder_cache=True)
            for _, tok, g in hist[b]:
                one = m.step(st, dev([tok])).cpu().numpy()[0]
                assert np.array_equal(one, g), b
    finally:
        m.close()


def test_order_capacity_and_reset():
    cfg = TINY
    P = make_params(cfg)
    B, L = 3, 4
    m = rlt.Model(cfg, P)
    try:
        st = m.state(B, L, keep_encoder_cache=True)
        lg = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
        tok = dev([cfg.bos] * B)
        rlt.rlt_step_rows(m.h, st, tok, [1, 0, 1], lg)
        assert rlt.rlt_state_row_positions(st, B) == [1, 0, 1]
        with pytest.raises(rlt.RltError) as e:
            m.step(st, tok)
        assert e.value.code == -7                      # ORDER: rows at different positions
        with pytest.raises(rlt.RltError):
            rlt.rlt_state_positions(st)
        for _ in range(3):
            rlt.rlt_step_rows(m.h, st, dev([1, 1, 1]), [1, 0, 0], lg)
        assert rlt.rlt_state_row_positions(st, B) == [4, 0, 1]
        with pytest.raises(rlt.RltError) as e:
            rlt.rlt_step_rows(m.h, st, dev([1, 1, 1]), [1, 1, 1], lg)
        assert e.value.code == -4                      # CAPACITY: row 0 is full
        rlt.rlt_step_rows(m.h, st, dev([cfg.bos, 1, 1]), [0, 1, 1], lg)   # the full row idles
        assert rlt.rlt_state_row_positions(st, B) == [4, 1, 2]
        rlt.rlt_state_reset_rows(m.h, st, [1, 0, 0])
        assert rlt.rlt_state_row_positions(st, B) == [0, 1, 2]
        rlt.rlt_state_reset(m.h, st)                  # back to the batch-wide form
        assert rlt.rlt_state_positions(st) == (0, 0)
        m.step(st, tok)
    finally:
        m.close()


def test_long_rows_split_attention():
    """Tiny fp32, 2 rows prefilled to 1030 positions, then 150 per-row calls (rows end up ~90
    positions apart): 8 attention blocks per launch, so memory ranges of 1024 keys or more are
    cut into pieces; every row's logits against the oracle (prefill of the same prefix, then
    one consume per token). Also a single-row replay of 1200 positions against the oracle."""
    cfg = TINY
    P = make_params(cfg)
    B, L, p0 = 2, 1200, 1030
    rng = np.random.default_rng(23)
    prefix = rng.integers(0, cfg.vocab - 1, size=(B, p0)).astype(np.int32)
    prefix[:, 0] = cfg.bos
    m = rlt.Model(cfg, P)
    hist = [[] for _ in range(B)]
    try:
        st = m.state(B, L, keep_encoder_cache=True)
        rlt.rlt_encode(m.h, st, dev(prefix))
        rlt.rlt_decode_scan(m.h, st, p0)
        lg = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
        for _ in range(150):
            act = (rng.random(B) < np.array([0.9, 0.3])).astype(np.int32)
            toks = rng.integers(0, cfg.vocab - 1, size=B).astype(np.int32)
            rlt.rlt_step_rows(m.h, st, dev(toks), act, lg)
            g = lg.cpu().numpy()
            for b in np.nonzero(act)[0]:
                hist[b].append((int(toks[b]), g[b].copy()))
        x1 = rng.integers(0, cfg.vocab - 1, size=(1, L)).astype(np.int32)
        x1[:, 0] = cfg.bos
        st1 = m.state(1, L, keep_encoder_cache=False)
        lp1, _ = m.replay(st1, dev(x1))
        lp1 = lp1.cpu().numpy()
    finally:
        m.close()
    o = Oracle(cfg, P)
    worst = 0.0
    for b in range(B):
        ost = o.new_state(1)
        o.prefill(ost, prefix[b:b + 1].astype(np.int64))
        for tok, g in hist[b]:
            ref, _ = o.consume(ost, np.array([tok], dtype=np.int64))
            worst = max(worst, float(np.max(np.abs(g - ref[0]))))
    ref_lp, _, _ = o.replay(x1.astype(np.int64))
    lp_err = float(np.max(np.abs(lp1 - ref_lp)))
    print(f"[ragged] long rows (positions {p0}..{p0 + max(len(h) for h in hist)}): max abs logit err "
          f"{worst:.2e}; replay of {L} positions log-prob err {lp_err:.2e}", flush=True)
    assert worst <= 1e-4
    assert lp_err <= 1e-4
