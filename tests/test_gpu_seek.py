"""rlt_state_seek (decoder sought to a later position) and the kernel timers, on the GPU.

After a seek to n, the state's decoder has consumed positions 1..n without running them:
s (and the RLT-2 register) keep their values and every window entry at positions
max(1, n-W+2)..n holds zero keys and values, while the memory of every encoded position is
real. Both sides run a few real transitions first (so the GPU's window holds entries to
clear), then the oracle builds the sought state from its own parts (its encoder's memory
and outputs, its s and register, zero window entries) and runs the transitions after n;
the GPU must match it at the usual bars. The timers must count every launch of their kind.
"""
import numpy as np
import pytest
import torch

from oracle import Oracle, V2
from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens

pytestmark = pytest.mark.gpu


def oracle_after_seek(cfg, P, x, n, dtype=np.float64):
    """Logits of positions n+1..T of the oracle started from the sought state: the first
    min(3, n) transitions run (as on the GPU), then s and the register are kept and the
    window holds zero entries at positions max(1, n-W+2)..n."""
    o = Oracle(cfg, P, dtype)
    st = o.new_state(x.shape[0])
    o.encoder_chunk(st, x)
    if n > 0:
        o.decode(st, min(3, n))
    zero = np.zeros((x.shape[0], cfg.hd), dtype=o.dt)
    for l in range(cfg.L_D):
        st.rings[l] = {p: (zero, zero) for p in range(max(1, n - cfg.window + 2), n + 1)}
    st.n_dec = n
    lg, _ = o.decode(st, x.shape[1] - n)
    return lg


def gpu_after_seek(cfg, P, x, n, timers=False):
    B, T = x.shape
    m = rlt.Model(cfg, P)
    try:
        st = m.state(B, T, keep_encoder_cache=False)
        xt = torch.as_tensor(x).cuda()
        rlt.rlt_encode(m.h, st, xt)
        if n > 0:
            # run a few real transitions first, so the seek has stale window entries to clear
            k = min(3, n)
            rlt.rlt_decode_scan(m.h, st, k)
            rlt.rlt_state_seek(m.h, st, n)
        assert rlt.rlt_state_positions(st) == (T, n)
        lg = torch.empty((B, T - n, cfg.vocab), dtype=torch.float32, device="cuda")
        if timers:
            rlt.rlt_kernel_timing(m.h, True)
        rlt.rlt_decode_scan(m.h, st, T - n, logits=lg)
        counts = {}
        if timers:
            for kind in range(5):
                counts[kind] = rlt.rlt_kernel_time(m.h, kind)
            rlt.rlt_kernel_timing(m.h, False)
        torch.cuda.synchronize()
        return lg.cpu().numpy(), counts
    finally:
        m.close()


@pytest.mark.parametrize("kw", [dict(), dict(variant=V2, chunk=3), dict(window=1), dict(groups=2)],
                         ids=["rlt1", "rlt2_k3", "window1", "groups_LD"])
def test_seek_matches_oracle_tiny(kw):
    cfg = CONFIGS["tiny_fp32"].replace(**kw)
    P = make_params(cfg)
    x = make_tokens(cfg)
    for n in (5, 11):
        ref = oracle_after_seek(cfg, P, x, n)
        got, _ = gpu_after_seek(cfg, P, x, n)
        err = float(np.max(np.abs(got - ref)))
        print(f"[parity] seek tiny {kw} to {n}: max abs logit err {err:.3e}", flush=True)
        assert err <= 1e-4


def test_seek_matches_oracle_algo_shape():
    cfg = CONFIGS["algo_bf16"].replace(batch=8, seq_len=72)
    P = make_params(cfg)
    x = make_tokens(cfg)
    n = 50
    ref = oracle_after_seek(cfg, P, x, n, np.float32)
    got, counts = gpu_after_seek(cfg, P, x, n, timers=True)
    err = float(np.max(np.abs(got - ref)))
    print(f"[parity] seek algo shape B=8 to {n}: max abs logit err {err:.3e}", flush=True)
    assert err <= 2e-2
    steps = x.shape[1] - n
    assert counts[rlt.TIME_MEMORY_ATTN][1] == steps * cfg.L_D
    assert counts[rlt.TIME_WINDOW_ATTN][1] == steps * cfg.L_D
    assert counts[rlt.TIME_ENCODER_ATTN][1] == 0 and counts[rlt.TIME_ENCODER_GEMM][1] == 0
    assert counts[rlt.TIME_DECODER_GEMM][1] == steps * (1 + 6 * cfg.L_D) + 1     # merge, 6 per block, readout
    assert all(counts[k][0] > 0 for k in (rlt.TIME_MEMORY_ATTN, rlt.TIME_WINDOW_ATTN, rlt.TIME_DECODER_GEMM))


def test_seek_order_errors():
    cfg = CONFIGS["tiny_fp32"]
    P = make_params(cfg)
    x = torch.as_tensor(make_tokens(cfg)).cuda()
    m = rlt.Model(cfg, P)
    try:
        st = m.state(2, 16, keep_encoder_cache=False)
        rlt.rlt_encode(m.h, st, x[:, :8].contiguous())
        with pytest.raises(rlt.RltError) as e:
            rlt.rlt_state_seek(m.h, st, 9)             # past the encoded positions
        assert e.value.code == -7
        rlt.rlt_decode_scan(m.h, st, 4)
        with pytest.raises(rlt.RltError) as e:
            rlt.rlt_state_seek(m.h, st, 3)             # behind the decoded positions
        assert e.value.code == -7
        rlt.rlt_state_seek(m.h, st, 8)
        assert rlt.rlt_state_positions(st) == (8, 8)
        torch.cuda.synchronize()
    finally:
        m.close()
