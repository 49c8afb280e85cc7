"""GPU parity of behaviour sampling, generation with on-device draws, and the importance ratio.

- rlt_sample against the sampling oracle on seeded synthetic logits (vocabulary 32000,
  8 and ragged sizes, temperatures 1, 0.7, 1.6 and 0): identical tokens (both sides take
  the decision in float64; a differing token is accepted only as a float64 near-tie of
  the oracle's scores, 1e-9), recorded log-probabilities within 1e-6.
- rlt_generate on the tiny fp32 configuration against the oracle's own generation loop
  (the oracle draws from its own logits with the same generator): identical tokens up to
  the first draw whose oracle score gap is within the logit bar (then the histories part
  and the rest is not comparable), logits within 1e-4, log mu within 2e-4.
- GPU-only identities: one rlt_generate call of n draws equals k + (n - k) draws, and
  equals rlt_step + rlt_sample per token, bit for bit.
- Replay contract (review §6.2 eq 5.5): at temperature 1 with unchanged weights, the
  current-policy replay log-probabilities of the generated tokens give an importance
  ratio of 1 within the step-vs-replay difference of the arithmetic (fp32: 1e-3;
  bf16: |log r| <= 4e-2).
- rlt_importance_ratio against the oracle on synthetic inputs: within 1 fp32 ulp.
"""
import numpy as np
import pytest
import torch

from oracle import Oracle
from oracle.rlt_sampler import generate as oracle_generate
from oracle.rlt_sampler import importance_ratio as oracle_ratio
from oracle.rlt_sampler import sample as oracle_sample
from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import CONFIGS, make_logits, make_params, make_tokens

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


def gpu_sample(logits, tau, seed, step):
    B = logits.shape[0]
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    rlt.rlt_sample(dev(logits), tau, seed, step, tok, lp)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lp.cpu().numpy()


def check_tokens(name, tok, ref_tok, ref_scores, gap):
    diff = np.nonzero(tok != ref_tok)[0]
    for b in diff:
        g = ref_scores[b, ref_tok[b]] - ref_scores[b, tok[b]]
        assert g <= gap, f"{name}: row {b} drew {tok[b]}, oracle {ref_tok[b]} (score gap {g:.3e})"
    print(f"[parity] {name}: tokens identical on {len(tok) - len(diff)}/{len(tok)} rows", flush=True)


@pytest.mark.parametrize("B,V", [(8, 32000), (64, 8), (5, 37), (3, 1)])
@pytest.mark.parametrize("tau", [1.0, 0.7, 1.6, 0.0])
def test_sample_kernel_vs_oracle(B, V, tau):
    logits = make_logits(B, V, seed=500 + V)
    if V >= 8:
        logits[0, 3] = logits[0, V - 1] = logits[0].max() + 0.5      # exact tie for greedy
    for step in (0, 7, 2**40 + 3):
        seed = 0x1234_5678_9ABC_DEF0 + B
        print(f"[case] rlt_sample B={B} V={V} tau={tau} step={step}", flush=True)
        tok, lp = gpu_sample(logits, tau, seed, step)
        ref_tok, ref_lp, ref_sc = oracle_sample(logits, tau, seed, step)
        check_tokens(f"sample B={B} V={V} tau={tau} step={step}", tok, ref_tok, ref_sc, 1e-9)
        same = tok == ref_tok
        err = float(np.max(np.abs(lp[same] - ref_lp[same]))) if same.any() else 0.0
        assert err <= 1e-6, err
        assert np.all((tok >= 0) & (tok < V))


def test_sample_row_stride_and_rows_zero():
    logits = make_logits(4, 40, seed=9)
    wide = np.zeros((4, 64), dtype=np.float32)
    wide[:, :40] = logits
    tok = torch.empty(4, dtype=torch.int32, device="cuda")
    lp = torch.empty(4, dtype=torch.float32, device="cuda")
    lib = rlt.load()
    w = dev(wide)
    rc = lib.rlt_sample(rlt._ptr(w), 4, 40, 64, 1.0, 77, 5, rlt._ptr(tok), rlt._ptr(lp), None, 0,
                        rlt.ctypes.c_void_p(rlt._stream()))
    assert rc == 0
    torch.cuda.synchronize()
    ref_tok, ref_lp, _ = oracle_sample(logits, 1.0, 77, 5)
    assert np.array_equal(tok.cpu().numpy(), ref_tok)
    assert np.max(np.abs(lp.cpu().numpy() - ref_lp)) <= 1e-6
    assert lib.rlt_sample(rlt._ptr(w), 0, 40, 64, 1.0, 77, 5, rlt._ptr(tok), None, None, 0,
                          rlt.ctypes.c_void_p(rlt._stream())) == 0
    assert lib.rlt_sample(rlt._ptr(w), 4, 40, 39, 1.0, 77, 5, rlt._ptr(tok), None, None, 0,
                          rlt.ctypes.c_void_p(rlt._stream())) == -1
    assert lib.rlt_sample(rlt._ptr(w), 4, 40, 64, -1.0, 77, 5, rlt._ptr(tok), None, None, 0,
                          rlt.ctypes.c_void_p(rlt._stream())) == -1


@pytest.mark.parametrize("tau", [1.0, 0.7, 0.0])
def test_sample_chunks_side_by_side_equal_one_workgroup(tau):
    """With a workspace the 4096-id chunks of each row run in separate workgroups: tokens and
    log mu equal the one-workgroup-per-row path bit for bit (vocabulary 32000: 8 chunks; 37
    rows), and both equal the oracle's draws."""
    logits = make_logits(37, 32000, seed=21)
    lg = dev(logits)
    t1 = torch.empty(37, dtype=torch.int32, device="cuda")
    l1 = torch.empty(37, dtype=torch.float32, device="cuda")
    t2, l2 = torch.empty_like(t1), torch.empty_like(l1)
    ws = torch.empty(rlt.rlt_sample_workspace(37, 32000), dtype=torch.uint8, device="cuda")
    rlt.rlt_sample(lg, tau, 5, 11, t1, l1)
    rlt.rlt_sample(lg, tau, 5, 11, t2, l2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2) and torch.equal(l1, l2)
    ref_tok, ref_lp, _ = oracle_sample(logits, tau, 5, 11)
    assert np.array_equal(t1.cpu().numpy(), ref_tok)
    assert np.max(np.abs(l1.cpu().numpy() - ref_lp)) <= 1e-6
    with pytest.raises(rlt.RltError):
        rlt.rlt_sample(lg, tau, 5, 11, t2, l2, workspace=ws[:8])


def gpu_generate(cfg, P, x, p, n, tau, seed, step0, splits=None):
    """Prefill x[:, :p], then rlt_generate n draws starting from x[:, p] (in pieces of `splits`)."""
    B = x.shape[0]
    m = rlt.Model(cfg, P)
    try:
        st = m.state(B, p + n + 1, keep_encoder_cache=True)
        xt = dev(x)
        m.prefill(st, xt[:, :p].contiguous(), want_logits=False)
        toks, lps, lgs = [], [], []
        first = xt[:, p].contiguous()
        done = 0
        for k in (splits or [n]):
            tok = torch.empty((B, k), dtype=torch.int32, device="cuda")
            lp = torch.empty((B, k), dtype=torch.float32, device="cuda")
            lg = torch.empty((B, k, cfg.vocab), dtype=torch.float32, device="cuda")
            rlt.rlt_generate(m.h, st, first, k, tau, seed, step0 + done, tok, lp, lg)
            first = tok[:, -1].contiguous()
            done += k
            toks.append(tok)
            lps.append(lp)
            lgs.append(lg)
        torch.cuda.synchronize()
        assert rlt.rlt_state_positions(st) == (p + n, p + n)
        return (torch.cat(toks, 1).cpu().numpy(), torch.cat(lps, 1).cpu().numpy(),
                torch.cat(lgs, 1).cpu().numpy())
    finally:
        m.close()


@pytest.mark.parametrize("tau", [1.0, 0.7, 0.0])
def test_generate_tiny_fp32_vs_oracle(tau):
    cfg = TINY
    P = make_params(cfg)
    x = make_tokens(cfg)
    p, n, seed, step0 = 5, 10, 2024, 100
    print(f"[case] rlt_generate tiny fp32 tau={tau} prefill {p} + {n} draws", flush=True)
    tok, lp, lg = gpu_generate(cfg, P, x, p, n, tau, seed, step0)
    o = Oracle(cfg, P, np.float32)
    st = o.new_state(cfg.batch)
    o.prefill(st, x[:, :p])
    r_tok, r_lp, r_lg, r_sc = oracle_generate(o, st, x[:, p], n, tau, seed, step0)
    for b in range(cfg.batch):
        for i in range(n):
            e = float(np.max(np.abs(lg[b, i] - r_lg[b, i])))
            assert e <= 1e-4, (b, i, e)
            if tok[b, i] != r_tok[b, i]:
                gap = r_sc[b, i, r_tok[b, i]] - r_sc[b, i, tok[b, i]]
                bar = 2e-4 / max(tau, 1e-30) if tau > 0 else 2e-4
                assert gap <= bar, f"row {b} draw {i}: GPU {tok[b, i]} vs oracle {r_tok[b, i]}, gap {gap:.3e}"
                print(f"[parity] row {b} parts at draw {i} on a near-tie (gap {gap:.2e})", flush=True)
                break
            assert abs(float(lp[b, i]) - float(r_lp[b, i])) <= 2e-4
    print(f"[parity] rlt_generate tiny fp32 tau={tau}: tokens {tok.tolist()} match the oracle's", flush=True)


def test_generate_split_and_step_sample_identity():
    cfg = ALGO.replace(batch=16, seq_len=40)
    P = make_params(cfg)
    x = make_tokens(cfg)
    p, n, seed, step0 = 20, 12, 7, 0
    a = gpu_generate(cfg, P, x, p, n, 1.0, seed, step0)
    b = gpu_generate(cfg, P, x, p, n, 1.0, seed, step0, splits=[5, 1, 6])
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    # the same draws from rlt_step + rlt_sample per token
    m = rlt.Model(cfg, P)
    try:
        st = m.state(cfg.batch, p + n + 1, keep_encoder_cache=True)
        xt = dev(x)
        m.prefill(st, xt[:, :p].contiguous(), want_logits=False)
        cur = xt[:, p].contiguous()
        toks, lps = [], []
        for i in range(n):
            lg = m.step(st, cur)
            tok = torch.empty(cfg.batch, dtype=torch.int32, device="cuda")
            lp = torch.empty(cfg.batch, dtype=torch.float32, device="cuda")
            rlt.rlt_sample(lg, 1.0, seed, step0 + i, tok, lp)
            toks.append(tok)
            lps.append(lp)
            cur = tok
        torch.cuda.synchronize()
        assert np.array_equal(torch.stack(toks, 1).cpu().numpy(), a[0])
        assert np.array_equal(torch.stack(lps, 1).cpu().numpy(), a[1])
    finally:
        m.close()
    print(f"[parity] rlt_generate bf16 B=16: one call == 5+1+6 calls == rlt_step+rlt_sample, bit for bit", flush=True)


@pytest.mark.parametrize("name,bar", [("tiny_fp32", 1e-3), ("algo_bf16", 4e-2)])
def test_replay_contract_ratio_is_one(name, bar):
    cfg = CONFIGS[name].replace(batch=min(CONFIGS[name].batch, 16), seq_len=24)
    P = make_params(cfg)
    x = make_tokens(cfg)
    p, n = 8, 12
    tok, lp_mu, _ = gpu_generate(cfg, P, x, p, n, 1.0, 31, 0)
    # full history: prompt x_1..x_p, the consumed first token x_{p+1}, then the draws
    hist = np.concatenate([x[:, :p + 1], tok], axis=1).astype(np.int32)
    m = rlt.Model(cfg, P)
    try:
        st = m.state(cfg.batch, hist.shape[1], keep_encoder_cache=False)
        lp_cur, _ = m.replay(st, dev(hist))
        cur = lp_cur[:, p:].contiguous()                    # log p(y_i | history) of the n draws
        ratio = torch.empty_like(cur)
        rlt.rlt_importance_ratio(cur, dev(lp_mu), ratio)
        torch.cuda.synchronize()
        lr = np.log(ratio.cpu().numpy().astype(np.float64))
    finally:
        m.close()
    err = float(np.max(np.abs(lr)))
    print(f"[parity] replay contract {name}: max |log r| = {err:.3e} over {lr.size} draws", flush=True)
    assert err <= bar


def test_importance_ratio_kernel_vs_oracle():
    a = make_logits(1, 100003, seed=41, scale=2.0)[0]
    b = make_logits(1, 100003, seed=42, scale=2.0)[0]
    r = torch.empty(a.size, dtype=torch.float32, device="cuda")
    rlt.rlt_importance_ratio(dev(a), dev(b), r)
    torch.cuda.synchronize()
    ref = oracle_ratio(a, b)
    rel = np.abs(r.cpu().numpy().astype(np.float64) - ref) / ref
    print(f"[parity] importance ratio: max rel err {rel.max():.3e}", flush=True)
    assert rel.max() <= 2 ** -23
