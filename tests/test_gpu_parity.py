"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Tolerances: fp32 configuration <= 1e-4 max abs logit error; 16-bit configurations
<= 2e-2 max abs logit error. The argmax bar (identical argmax on >= 99.9% of positions) is
asserted on the raw agreement of the full-size workloads (test_gpu_fullsize, test_gpu_lm,
test_gpu_paper), where thousands of positions make a 0.1% rate measurable; the reduced
cases here hold a few hundred positions each and print their raw agreement.
"""
import numpy as np
import pytest
import torch

from oracle import Oracle, V0, V1, V2
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


_ORACLE_CACHE = {}


def oracle_replay(cfg, P, x, dtype=np.float32):
    key = (cfg, x.tobytes(), np.dtype(dtype).str)
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = Oracle(cfg, P, dtype).replay(x)
    return _ORACLE_CACHE[key]


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda()


def tol_of(cfg):
    return 1e-4 if cfg.dtype == "fp32" else 2e-2


def report(name, gpu, ref):
    err = float(np.max(np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))))
    print(f"[parity] {name}: max abs err {err:.3e}", flush=True)
    return err


def raw_argmax_agreement(gpu_logits, ref_logits):
    return float(np.mean(np.argmax(gpu_logits, axis=-1) == np.argmax(ref_logits, axis=-1)))


def check_logits(cfg, name, gpu, ref):
    err = report(name, gpu, ref)
    assert err <= tol_of(cfg), f"{name}: {err}"
    if cfg.dtype != "fp32":
        raw = raw_argmax_agreement(np.asarray(gpu), np.asarray(ref))
        n = int(np.prod(np.asarray(gpu).shape[:-1]))
        print(f"[parity] {name}: raw argmax agreement {raw:.5f} over {n} positions", flush=True)


def gpu_prefill(cfg, P, x, steps_from=None, keep_enc=True, scan_mode=0):
    """Prefill x[:, :p] then consume the rest one token at a time (p = steps_from or all)."""
    B, T = x.shape
    p = T if steps_from is None else steps_from
    m = rlt.Model(cfg, P)
    rlt.rlt_set_scan_mode(m.h, scan_mode)
    try:
        st = m.state(B, T, keep_encoder_cache=keep_enc)
        xt = dev(x)
        lg, s = m.prefill(st, xt[:, :p].contiguous(), want_logits=True, want_s=True)
        lgs, ss = [lg], [s]
        for i in range(p, T):
            lgs.append(m.step(st, xt[:, i].contiguous())[:, None])
        torch.cuda.synchronize()
        logits = torch.cat(lgs, dim=1).cpu().numpy()
        return logits, s.cpu().numpy(), rlt.rlt_state_block_steps(st)
    finally:
        m.close()


def gpu_replay(cfg, P, x, scan_mode=0):
    B, T = x.shape
    m = rlt.Model(cfg, P)
    rlt.rlt_set_scan_mode(m.h, scan_mode)
    try:
        st = m.state(B, T, keep_encoder_cache=False)
        lp, s = m.replay(st, dev(x), want_s=True)
        torch.cuda.synchronize()
        return lp.cpu().numpy(), s.cpu().numpy()
    finally:
        m.close()


TINY_CASES = {
    "rlt1": {},
    "rlt0": dict(variant=V0),
    "rlt2_k3": dict(variant=V2, chunk=3),
    "rlt2_k4": dict(variant=V2, chunk=4),
    "groups_LD": dict(groups=2),
    "shared": dict(share=True),
    "window1": dict(window=1),
    "window_ge_T": dict(window=32),
    "no_decoder": dict(L_D=0),
    "batch3_L3": dict(batch=3, L_E=3, L_D=3, groups=3),
}


@pytest.mark.parametrize("case", sorted(TINY_CASES))
def test_tiny_fp32_prefill_matches_oracle(case):
    cfg = TINY.replace(**TINY_CASES[case])
    P = make_params(cfg)
    x = make_tokens(cfg)
    print(f"[case] tiny_fp32 {case} B={x.shape[0]} T={x.shape[1]}", flush=True)
    _, ref_logits, ref_s = Oracle(cfg, P).replay(x)
    logits, s, _ = gpu_prefill(cfg, P, x)
    check_logits(cfg, f"tiny {case} logits", logits, ref_logits)
    assert report(f"tiny {case} s", s, ref_s) <= 1e-4


@pytest.mark.parametrize("case", ["rlt1", "rlt2_k3", "rlt0"])
def test_tiny_fp32_replay_logprob(case):
    cfg = TINY.replace(**TINY_CASES[case])
    P = make_params(cfg)
    x = make_tokens(cfg)
    ref_lp, _, ref_s = Oracle(cfg, P).replay(x)
    lp, s = gpu_replay(cfg, P, x)
    assert report(f"tiny {case} replay logprob", lp, ref_lp) <= 1e-4
    assert report(f"tiny {case} replay s", s, ref_s) <= 1e-4


@pytest.mark.parametrize("split", [1, 5, 12, 16])
def test_tiny_fp32_serving_split_on_gpu(split):
    """Prefill of x_1..p then single-token steps equals the oracle's replay for every split p
    (jiphyeonjeon review §4.1, Proposition 3.1)."""
    cfg = TINY
    P = make_params(cfg)
    x = make_tokens(cfg)
    _, ref_logits, _ = Oracle(cfg, P).replay(x)
    logits, _, _ = gpu_prefill(cfg, P, x, steps_from=split)
    check_logits(cfg, f"tiny split {split}", logits, ref_logits)


def test_rlt2_generation_partial_chunks():
    """RLT-2 generation is token by token; a partial chunk keeps the previous register
    (greeksharifa summary appendix I.3). Prefill ends mid-chunk."""
    cfg = TINY.replace(variant=V2, chunk=4)
    P = make_params(cfg)
    x = make_tokens(cfg)
    _, ref_logits, _ = Oracle(cfg, P).replay(x)
    logits, _, _ = gpu_prefill(cfg, P, x, steps_from=6)
    check_logits(cfg, "rlt2 split 6", logits, ref_logits)


def test_block_step_counts():
    """Dependent decoder block passes: T*L_D (RLT-1), ceil(T/K_c)*L_D (RLT-2), per pass for RLT-0
    (greeksharifa summary §2.7, Table 1)."""
    for kw, expect in ((dict(), 16 * 2), (dict(variant=V2, chunk=4), 4 * 2), (dict(variant=V2, chunk=3), 6 * 2),
                       (dict(variant=V0), 1 * 2)):
        cfg = TINY.replace(**kw)
        P = make_params(cfg)
        _, _, steps = gpu_prefill(cfg, P, make_tokens(cfg))
        assert steps == expect, (kw, steps)


# per-position launches; persistent grid-wide; persistent per-XCD groups with 1, 2, 4 blocks per CU;
# per-position launches on 2 and 4 batch slices with a stream each; graph replay per position
SCAN_MODES = [1, 3, 4, 5, 6, 7, 8, 9]


def test_graph_replay_matches_launches():
    """Mode 9 (one position's launch sequence captured as a HIP graph and replayed per position)
    equals mode 1 bit for bit: a 60-position prefill, then 10 rlt_step calls (each a replay and
    an eager readout between replays), and a 70-position rlt_replay whose readout flushes after
    64 replays."""
    cfg = ALGO.replace(batch=8, seq_len=70)
    P = make_params(cfg)
    x = make_tokens(cfg)
    outs = {}
    for mode in (1, 9):
        logits, s, _ = gpu_prefill(cfg, P, x, steps_from=60, scan_mode=mode)
        lp, _ = gpu_replay(cfg, P, x, scan_mode=mode)
        outs[mode] = (logits, s, lp)
    for a, b in zip(outs[1], outs[9]):
        assert np.array_equal(a, b)
    ref_lp, ref_logits, _ = oracle_replay(cfg, P, x)
    check_logits(cfg, "graph replay logits", outs[9][0], ref_logits)


@pytest.mark.parametrize("scan_mode", SCAN_MODES)
@pytest.mark.parametrize("variant", [V1, V0])
def test_algo_bf16_reduced(variant, scan_mode):
    cfg = ALGO.replace(variant=variant, batch=32, seq_len=40)
    P = make_params(cfg)
    x = make_tokens(cfg)
    print(f"[case] algo_bf16 variant={variant} B=32 T=40 scan_mode={scan_mode}", flush=True)
    ref_lp, ref_logits, ref_s = oracle_replay(cfg, P, x)
    logits, s, _ = gpu_prefill(cfg, P, x, steps_from=30, scan_mode=scan_mode)
    check_logits(cfg, f"algo v{variant} m{scan_mode} logits", logits, ref_logits)
    lp, _ = gpu_replay(cfg, P, x, scan_mode=scan_mode)
    assert report(f"algo v{variant} m{scan_mode} logprob", lp, ref_lp) <= 2e-2


@pytest.mark.parametrize("scan_mode", SCAN_MODES)
@pytest.mark.parametrize("kw", [dict(variant=V2, chunk=4), dict(variant=V2, chunk=3), dict(L_D=0),
                                dict(groups=4), dict(share=True, L_E=4), dict(window=1), dict(batch=3),
                                dict(variant=V2, chunk=3, batch=32), dict(compute="bf16"),
                                dict(compute="fp16x2"), dict(compute="fp16x2", variant=V2, chunk=3, batch=5)],
                         ids=["rlt2_k4", "rlt2_k3", "no_decoder", "groups_LD", "shared", "window1", "batch3",
                              "rlt2_k3_b32", "bf16", "fp16x2", "fp16x2_rlt2_b5"])
def test_bf16_variants_small(kw, scan_mode):
    cfg = ALGO.replace(**{"batch": 8, "seq_len": 21, **kw})
    P = make_params(cfg)
    x = make_tokens(cfg)
    print(f"[case] algo_bf16 {kw} B={x.shape[0]} T=21 scan_mode={scan_mode}", flush=True)
    _, ref_logits, ref_s = oracle_replay(cfg, P, x)
    logits, s, steps = gpu_prefill(cfg, P, x, steps_from=13, scan_mode=scan_mode)
    check_logits(cfg, f"bf16 {kw} m{scan_mode} logits", logits, ref_logits)
    assert report(f"bf16 {kw} m{scan_mode} s", s, ref_s[:, :13]) <= 5e-2


def test_rlt2_bf16_reduced():
    cfg = CONFIGS["rlt2_bf16"].replace(batch=16, seq_len=24)
    P = make_params(cfg)
    x = make_tokens(cfg)
    print("[case] rlt2_bf16 B=16 T=24", flush=True)
    _, ref_logits, _ = oracle_replay(cfg, P, x)
    for mode in SCAN_MODES:
        logits, _, _ = gpu_prefill(cfg, P, x, scan_mode=mode)
        check_logits(cfg, f"rlt2 bf16 m{mode} logits", logits, ref_logits)


# ------------------------------------------------------------------ error paths
def test_errors_capacity_order_stale():
    cfg = TINY
    P = make_params(cfg)
    x = dev(make_tokens(cfg))
    m = rlt.Model(cfg, P)
    try:
        st = m.state(2, 16, keep_encoder_cache=True)
        with pytest.raises(rlt.RltError) as e:
            rlt.rlt_decode_scan(m.h, st, 1)
        assert e.value.code == -7
        rlt.rlt_encode(m.h, st, x[:, :10].contiguous())
        with pytest.raises(rlt.RltError) as e:
            rlt.rlt_encode(m.h, st, x)                       # 10 + 16 > 16
        assert e.value.code == -4
        assert rlt.rlt_state_positions(st) == (10, 0)
        rlt.rlt_update_weights(m.h, P)
        with pytest.raises(rlt.RltError) as e:
            rlt.rlt_decode_scan(m.h, st, 1)
        assert e.value.code == -5
        rlt.rlt_state_reset(m.h, st)
        rlt.rlt_encode(m.h, st, x[:, :4].contiguous())
        rlt.rlt_decode_scan(m.h, st, 4)
        st2 = m.state(2, 16, keep_encoder_cache=False)
        rlt.rlt_encode(m.h, st2, x[:, :4].contiguous())
        with pytest.raises(rlt.RltError) as e:
            rlt.rlt_encode(m.h, st2, x[:, 4:8].contiguous())  # continuation needs the encoder cache
        assert e.value.code == -2
        torch.cuda.synchronize()
    finally:
        m.close()


def test_state_storage_terms():
    """Allocated state bytes follow the storage terms of jiphyeonjeon review §4.2 eq 3.3:
    encoder cache (L_E t d_KV), memory (G t d_KV), rings (L_D W d_KV), recurrent output (d)."""
    cfg = TINY
    m = rlt.Model(cfg, make_params(cfg))
    try:
        B, Tm = 2, 16
        st = m.state(B, Tm, keep_encoder_cache=True)
        by = rlt.rlt_state_bytes(st)
        e = 4
        hd = cfg.hd
        assert by[0] == 2 * cfg.L_E * B * Tm * hd * e
        assert by[1] == 2 * cfg.groups * B * Tm * hd * e
        assert by[2] == 2 * cfg.L_D * B * cfg.window * hd * e       # RLT-1: ring of W slots
        assert by[3] == 2 * B * cfg.d * 4
        st2 = m.state(B, Tm, keep_encoder_cache=False)
        assert rlt.rlt_state_bytes(st2)[0] == 0
    finally:
        m.close()
