"""Throughput of the RLT hot path on one MI355X.

Default: the paper's reference shape (48 + 48 blocks with attention / FFN weights shared
between encoder and decoder, d 4096, 32 x 128 heads, SwiGLU 11008, vocab 32000, W 1024,
G 1, RLT-1) at batch 64. The token-parallel causal encode of the 8192-token Zipf prompt
(plus the positions the decoder then consumes) is timed once (encoder tok/s); the decoder
is sought to position 8192 (memory of every encoded position real, window entries zero)
and --steps batched transitions at positions 8193.. are timed with HIP events (decoder
transitions/s = batch x steps / time). The roofline object is that of the step's dominant
kernel, the cross-attention over the memory prefix, timed live per launch with HIP events
on its stream; step_roofline is the whole transition against the same HBM peak. The CPU
oracle is timed on a bounded sample (cpu_baseline).

--config NAME picks another workload (same measurement at its prompt length); --replay
times whole replays (encode + scan of every position + log-probabilities) as before;
--grad, --generate, --ragged, --snapshot and --sweep decode time the other paths.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "decoder transitions/sec at batch B + encoder tok/s; % of HBM/MFMA roofline"


def scan_bytes(cfg, B: int, T: int, t_start: int = 0) -> float:
    """Algorithmic HBM bytes of decoder transitions t_start+1 .. t_start+T for B sequences.

    Per transition at position t (batched): the decoder weights once per step
    (e * P_dec with P_dec = L_D(6 d hd-sized blocks + 3 d f + 3 d) + 3 d^2 + 3 d + V d + d),
    each layer's SWA window reads (min(t, W) - 1 past positions), each layer's
    read of the memory prefix 1..t of its group, ring writes, e_t in, s in/out
    and the fp32 logits out.
    """
    e = 2 if cfg.dtype == "bf16" else 4
    d, f, V, L, W, hd = cfg.d, cfg.ffn, cfg.vocab, cfg.L_D, cfg.window, cfg.hd
    P_dec = L * (4 * d * hd + 2 * d * hd + 3 * d * f + 3 * d) + 3 * d * d + 3 * d + V * d + d
    total = 0.0
    for t in range(t_start + 1, t_start + T + 1):
        total += e * P_dec
        total += B * L * (min(t, W) - 1) * 2 * hd * e
        total += B * L * t * 2 * hd * e
        total += B * (L * 2 * hd * e + d * 4 + 2 * d * 4 + V * 4)
    return total


def encoder_flops(cfg, B: int, T: int) -> float:
    d, f, hd, L = cfg.d, cfg.ffn, cfg.hd, cfg.L_E
    G = cfg.groups if cfg.L_D > 0 else 0
    per_tok = 2 * (L * (4 * d * hd + 3 * d * f) + G * 2 * d * hd + (d * d if cfg.variant != 0 else 0))
    attn = B * L * 4 * hd * T * (T + 1) / 2
    return B * T * per_tok + attn


def step_flops(cfg, B: int, t: int) -> float:
    """Algorithmic flops of one batched decoder transition at position t (weights as GEMMs + attention)."""
    d, f, V, L, W, hd = cfg.d, cfg.ffn, cfg.vocab, cfg.L_D, cfg.window, cfg.hd
    P_dec = L * (4 * d * hd + 2 * d * hd + 3 * d * f + 3 * d) + 3 * d * d + 3 * d + V * d + d
    return 2.0 * P_dec * B + B * L * 4 * hd * (min(t, W) + t)


def decode_sweep(shapes, batches, positions, steps: int = 8):
    """Decoder transitions at batch B and position t: one JSON line per point.

    For each point: encode t + steps tokens, seek the decoder to position t-1 (rlt_state_seek:
    window entries zero, memory real), then time the scan of positions t..t+steps-1 with HIP
    events. Reports us per transition step (the
    whole batch), the algorithmic bytes / flops of those steps, and their fractions of the
    8 TB/s HBM and 2.5 PFLOP/s 16-bit MFMA peaks.
    """
    import torch
    from recurrent_looped_transformer_amd import rlt
    from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens
    for name in shapes:
        cfg = CONFIGS[name]
        P = make_params(cfg, bf16_storage=cfg.d >= 4096)
        model = rlt.Model(cfg, P)
        del P
        toks_all = make_tokens(cfg, batch=max(batches), length=max(positions[name]) + steps)
        for B in batches:
            for t in positions[name]:
                st = model.state(B, t + steps, keep_encoder_cache=False)
                x = torch.as_tensor(np.ascontiguousarray(toks_all[:B, :t + steps])).cuda()
                rlt.rlt_encode(model.h, st, x)
                rlt.rlt_state_seek(model.h, st, t - 1)
                stream = torch.cuda.current_stream()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                rlt.rlt_decode_scan(model.h, st, steps)
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                rlt.rlt_state_destroy(st)
                model.states.remove(st)
                by = scan_bytes(cfg, B, steps, t_start=t - 1)
                fl = sum(step_flops(cfg, B, tt) for tt in range(t, t + steps))
                sec = ms / 1e3
                print(json.dumps({"sweep": "decode", "config": name, "dtype": cfg.path_dtype, "batch": B,
                                  "position": t, "steps": steps, "us_per_step": ms * 1e3 / steps,
                                  "transitions_s": B * steps / sec,
                                  "hbm_GBs": by / sec / 1e9, "hbm_frac": by / sec / 1e9 / HBM_PEAK_GBS,
                                  "mfma_TFs": fl / sec / 1e12,
                                  "mfma_frac": fl / sec / 1e12 / BF16_PEAK_TFLOPS}), flush=True)
        model.close()


FP32_PEAK_TFLOPS = 157.3
GRAD_METRIC = "replay gradient (full BPTT) transitions/sec at batch B; % of fp32 MFMA roofline"


def grad_flops(cfg, B: int, T: int) -> float:
    """Algorithmic flops of one full-BPTT gradient pass (forward kept for the backward).

    Every matrix product appears three times (forward, input gradient, weight gradient):
    3 * 2 * (B*T rows) * (matrix parameters: encoder, memory, decoder, merge, readout). The
    attention terms (scores and weighted sums: 4*hd per query-key pair; encoder causal,
    decoder window min(t, W) and memory prefix t) also count three times (forward; and
    the backward's four products over the same pairs, two of which repeat forward ones).
    """
    d, f, hd, V, LE, LD, W = cfg.d, cfg.ffn, cfg.hd, cfg.vocab, cfg.L_E, cfg.L_D, cfg.window
    G = cfg.groups if LD > 0 else 0
    mats = LE * (4 * d * hd + 3 * d * f) + G * 2 * d * hd + LD * (6 * d * hd + 3 * d * f) \
        + (3 * d * d if cfg.variant != 0 else 0) + V * d
    gemm = 2.0 * B * T * mats
    attn = B * LE * 4 * hd * T * (T + 1) / 2 + B * LD * 4 * hd * sum(min(t, W) + t for t in range(1, T + 1))
    return 3.0 * (gemm + attn)


def grad_bench(args, cfg):
    import torch
    from recurrent_looped_transformer_amd import rlt
    from recurrent_looped_transformer_amd.synth import make_params, make_tokens
    B, T = cfg.batch, cfg.seq_len
    P = make_params(cfg)
    tokens = make_tokens(cfg, length=T)
    w = np.random.default_rng(3).standard_normal((B, T - 1)).astype(np.float32)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    W = {k: torch.as_tensor(np.ascontiguousarray(v, dtype=np.float32)).to(dev) for k, v in P.items()}
    G = {k: torch.empty_like(v) for k, v in W.items()}
    x = torch.as_tensor(tokens).to(dev)
    wt = torch.as_tensor(w).to(dev)
    lp = torch.empty((B, T - 1), dtype=torch.float32, device=dev)
    ck = bool(args.checkpoint)
    ws = torch.empty(rlt.rlt_replay_grad_workspace(cfg, B, T, ck), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        rlt.rlt_replay_grad(cfg, W, x, wt, workspace=ws, grads=G, logprob=lp, checkpoint=ck)
        if ev: ev[1].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] gradient warm-up {i + 1}/{args.warmup} done", flush=True)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pass_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    ms_per_step = wall * 1e3 / args.steps
    fl = grad_flops(cfg, B, T)
    achieved = fl / (pass_ms / 1e3) / 1e12
    out = {
        "metric": GRAD_METRIC, "value": B * T / (ms_per_step / 1e3), "unit": "transitions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} shape, full-BPTT gradient of the replay loss "
                               f"(fp32 arithmetic{', activation checkpointing' if ck else ''}), "
                               f"RLT-{cfg.variant} B={B} T={T}",
                   "batch": B, "seq_len": T, "d": cfg.d, "L_E": cfg.L_E, "L_D": cfg.L_D, "window": cfg.window,
                   "groups": cfg.groups, "vocab": cfg.vocab, "variant": f"RLT-{cfg.variant}",
                   "workspace_bytes": ws.numel(), "checkpoint": ck},
        "gradient_pass_ms": pass_ms,
        "roofline": {"bound": "mfma", "kernel": "gradient pass (saved forward + reverse scan + weight gradients)",
                     "achieved": achieved, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_PEAK_TFLOPS, "traffic": None, "algorithmic_flops_per_launch": fl},
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_info
        from oracle.rlt_grad import GradOracle
        sb = min(args.cpu_sample, B, 4)
        t1 = time.perf_counter()
        GradOracle(cfg, P).grad(tokens[:sb], w[:sb].astype(np.float64))
        dt = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": sb * T / dt, "unit": "transitions/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"{sb} of {B} sequences x {T} positions, full-BPTT gradient, "
                                         f"float64 torch reverse mode, {dt:.1f} s"}
    print(json.dumps(out), flush=True)


RAGGED_METRIC = "continuous-batching generation tokens/sec (every row at its own position); % of HBM roofline"


def gen_step_bytes(cfg, positions) -> float:
    """Algorithmic HBM bytes of one generation step of rows at the given positions (1-based
    position of the token each row consumes): encoder, memory, merge and decoder weights once
    per step (e * P_dec as in scan_bytes, plus the encoder's e * P_enc), and per row the
    encoder-cache reads (L_E * t keys and values), the window and memory-prefix reads of
    every decoder layer, the cache / memory / ring writes and the state and logits I/O."""
    e = 2 if cfg.dtype == "bf16" else 4
    d, f, V, LE, LD, W, hd = cfg.d, cfg.ffn, cfg.vocab, cfg.L_E, cfg.L_D, cfg.window, cfg.hd
    G = cfg.groups if LD > 0 else 0
    P_enc = LE * (4 * d * hd + 3 * d * f + 2 * d) + G * 2 * d * hd + (d if LD > 0 else 0) \
        + (d * d if cfg.variant != 0 else 0)
    P_dec = LD * (4 * d * hd + 2 * d * hd + 3 * d * f + 3 * d) + 3 * d * d + 3 * d + V * d + d
    total = float(e * (P_enc + P_dec))
    for t in positions:
        total += LE * t * 2 * hd * e + LD * (min(t, W) - 1) * 2 * hd * e + LD * t * 2 * hd * e
        total += (LE + LD + G) * 2 * hd * e + 3 * d * 4 + V * 4
    return total


def ragged_bench(args, cfg):
    """Rows at unequal positions: prefill every row to `base`, move row b alone for
    b * spread / (B - 1) more positions (rows spread linearly over base..base+spread), then
    time steps in which every row consumes one token at its own position. The same batch
    stepping at one common position (the mean) is timed beside it."""
    import torch
    from recurrent_looped_transformer_amd import rlt
    from recurrent_looped_transformer_amd.synth import make_params, make_tokens
    B = cfg.batch
    base = args.ragged_base or cfg.seq_len // 2
    spread = args.ragged_spread
    K, Wm = args.steps, args.warmup
    max_len = base + spread + Wm + K + 1
    P = make_params(cfg, bf16_storage=cfg.d >= 4096)
    torch.cuda.set_device(0)
    model = rlt.Model(cfg, P)
    del P
    toks = make_tokens(cfg, batch=B, length=max_len)
    x = torch.as_tensor(np.ascontiguousarray(toks)).cuda()
    rows = torch.arange(B, device="cuda")
    stream = torch.cuda.current_stream()
    lg = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")

    st = model.state(B, max_len, keep_encoder_cache=True)
    rlt.rlt_encode(model.h, st, x[:, :base].contiguous())
    rlt.rlt_decode_scan(model.h, st, base)
    pos = np.full(B, base, np.int64)
    target = base + (np.arange(B) * spread) // max(1, B - 1)
    for c in range(spread):
        act = (pos < target).astype(np.int32)
        tk = x[rows, torch.as_tensor(np.minimum(pos, max_len - 1)).cuda()].contiguous()
        rlt.rlt_step_rows(model.h, st, tk, act, lg)
        pos += act
        if (c + 1) % 128 == 0 or c + 1 == spread:
            torch.cuda.synchronize()
            print(f"[bench] rows spread: {c + 1}/{spread} calls", flush=True)
    ones = np.ones(B, np.int32)

    def timed(fn):
        for _ in range(Wm):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(K):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / K

    pos_start = pos.copy()

    def ragged_step():
        tk = x[rows, torch.as_tensor(pos).cuda()].contiguous()
        rlt.rlt_step_rows(model.h, st, tk, ones, lg)
        pos[:] += 1

    ms_r = timed(ragged_step)
    by = np.mean([gen_step_bytes(cfg, pos_start + Wm + k + 1) for k in range(K)])
    print("[bench] ragged steps timed", flush=True)
    rlt.rlt_state_destroy(st)
    model.states.remove(st)

    mean_p = int(round(float(np.mean(pos_start))))
    su = model.state(B, max_len, keep_encoder_cache=True)
    rlt.rlt_encode(model.h, su, x[:, :mean_p].contiguous())
    rlt.rlt_decode_scan(model.h, su, mean_p)
    col = [mean_p]

    def uniform_step():
        rlt.rlt_step(model.h, su, x[:, col[0]].contiguous(), lg)
        col[0] += 1

    ms_u = timed(uniform_step)
    by_u = np.mean([gen_step_bytes(cfg, [mean_p + Wm + k + 1] * B) for k in range(K)])
    model.close()
    ach = by / (ms_r / 1e3) / 1e9
    out = {
        "metric": RAGGED_METRIC, "value": B / (ms_r / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": Wm, "ms_per_step": ms_r, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp16": "f16", "fp16x2": "f16x2"}[cfg.path_dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} generation, B={B} rows at positions {int(pos_start.min())}.."
                               f"{int(pos_start.max())} (linear spread), every row consuming one token per step",
                   "batch": B, "positions_min": int(pos_start.min()), "positions_max": int(pos_start.max()),
                   "d": cfg.d, "L_E": cfg.L_E, "L_D": cfg.L_D, "window": cfg.window, "vocab": cfg.vocab},
        "uniform_same_mean": {"position": mean_p, "ms_per_step": ms_u, "tokens_s": B / (ms_u / 1e3),
                              "hbm_GBs": by_u / (ms_u / 1e3) / 1e9},
        "roofline": {"bound": "hbm", "kernel": "generation step (encoder step + transition + logits)",
                     "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": by},
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_info
        from oracle import Oracle
        from recurrent_looped_transformer_amd.synth import make_params as mp
        n = min(256, max_len)
        o = Oracle(cfg, mp(cfg, bf16_storage=cfg.d >= 4096), np.float32)
        ost = o.new_state(1)
        t1 = time.perf_counter()
        for i in range(n):
            o.consume(ost, toks[:1, i])
        dt = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"1 row x {n} generation steps from BOS (positions 1-{n}; the "
                                         f"oracle's per-position cost is dominated by streaming the weights), "
                                         f"float32 numpy, {dt:.1f} s"}
    print(json.dumps(out), flush=True)


GEN_METRIC = "generation tokens/sec with on-device behaviour sampling and recorded log-probabilities; % of HBM roofline"
SNAP_METRIC = "prefix snapshot + restore bandwidth (device and pinned-host copies); % of HBM roofline"


def _events(torch, stream, fn, reps):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(reps):
        fn()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def generate_bench(args, cfg):
    """rlt_generate after a prefill of `base` positions: n draws per call (temperature 1), each
    consumed before the next; plus the sampler kernel alone on the same logits shape."""
    import torch
    from recurrent_looped_transformer_amd import rlt
    from recurrent_looped_transformer_amd.synth import make_logits, make_params, make_tokens
    B = cfg.batch
    base = args.ragged_base or cfg.seq_len
    n = 32
    K, Wm = args.steps, args.warmup
    max_len = base + (K + Wm) * n + 1
    P = make_params(cfg, bf16_storage=cfg.d >= 4096)
    torch.cuda.set_device(0)
    model = rlt.Model(cfg, P)
    del P
    toks = make_tokens(cfg, batch=B, length=base)
    x = torch.as_tensor(np.ascontiguousarray(toks)).cuda()
    st = model.state(B, max_len, keep_encoder_cache=True)
    rlt.rlt_encode(model.h, st, x[:, :base - 1].contiguous())
    rlt.rlt_decode_scan(model.h, st, base - 1)
    torch.cuda.synchronize()
    print(f"[bench] prefill of {base - 1} positions done", flush=True)
    stream = torch.cuda.current_stream()
    first = x[:, base - 1].contiguous()
    out_t = torch.empty((B, n), dtype=torch.int32, device="cuda")
    out_lp = torch.empty((B, n), dtype=torch.float32, device="cuda")
    calls = [0]
    start_pos = base

    def gen():
        rlt.rlt_generate(model.h, st, first, n, 1.0, 1234, calls[0] * n, out_t, out_lp)
        first.copy_(out_t[:, n - 1])
        calls[0] += 1

    for _ in range(Wm):
        gen()
    p0 = start_pos + Wm * n
    ms = _events(torch, stream, gen, K) / n          # per generated token of the batch
    positions = [p0 + i for i in range(K * n)]
    by = float(np.mean([gen_step_bytes(cfg, [p] * B) for p in positions])) + B * cfg.vocab * 4 * 2
    model.close()
    # the sampler alone: B rows of V logits
    lg = torch.as_tensor(make_logits(B, cfg.vocab, seed=7)).cuda()
    tk = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    step = [0]

    def samp():
        rlt.rlt_sample(lg, 1.0, 99, step[0], tk, lp)
        step[0] += 1

    for _ in range(3):
        samp()
    us_s1 = _events(torch, stream, samp, 200) * 1e3
    ws = torch.empty(rlt.rlt_sample_workspace(B, cfg.vocab), dtype=torch.uint8, device="cuda")

    def samp_ws():
        rlt.rlt_sample(lg, 1.0, 99, step[0], tk, lp, workspace=ws)
        step[0] += 1

    for _ in range(3):
        samp_ws()
    us_s = _events(torch, stream, samp_ws, 200) * 1e3
    sb = B * cfg.vocab * 4
    ach = by / (ms / 1e3) / 1e9
    out = {
        "metric": GEN_METRIC, "value": B / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp16": "f16", "fp16x2": "f16x2"}[cfg.path_dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} generation (rlt_generate, {n} draws per call, temperature 1) after a "
                               f"{base - 1}-position prefill, B={B}", "batch": B, "prefill": base - 1,
                   "draws_per_call": n, "vocab": cfg.vocab},
        "sampler": {"us_per_call": us_s, "us_per_call_one_workgroup_per_row": us_s1, "rows": B,
                    "vocab": cfg.vocab, "logit_bytes": sb, "GBs": sb / (us_s / 1e6) / 1e9},
        "roofline": {"bound": "hbm", "kernel": "generation step (encoder step + transition + logits + draw)",
                     "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": by},
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_info
        from oracle.rlt_sampler import sample as oracle_sample
        lgh = make_logits(B, cfg.vocab, seed=7)
        reps = 0
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < 10.0:
            oracle_sample(lgh, 1.0, 99, reps)
            reps += 1
        dt = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": reps * B / dt, "unit": "draws/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"{reps} sampler calls of {B} rows x {cfg.vocab} logits (Philox4x64-10 "
                                         f"uniforms, Gumbel-max, float64 log mu), {dt:.1f} s; the GPU's sampler "
                                         f"alone: {B / (us_s / 1e6):.0f} draws/s"}
    print(json.dumps(out), flush=True)


def snapshot_bench(args, cfg):
    """Snapshot and restore of a state after a prefill of `base` positions (encoder cache kept):
    to / from a device buffer and a pinned host buffer. Algorithmic bytes: the payload read
    and written once per copy."""
    import torch
    from recurrent_looped_transformer_amd import rlt
    from recurrent_looped_transformer_amd.synth import make_params, make_tokens
    B = cfg.batch
    base = args.ragged_base or 512
    P = make_params(cfg, bf16_storage=cfg.d >= 4096)
    torch.cuda.set_device(0)
    model = rlt.Model(cfg, P)
    del P
    x = torch.as_tensor(np.ascontiguousarray(make_tokens(cfg, batch=B, length=base))).cuda()
    st = model.state(B, base, keep_encoder_cache=True)
    rlt.rlt_encode(model.h, st, x)
    rlt.rlt_decode_scan(model.h, st, base)
    nbytes = rlt.rlt_snapshot_size(model.h, st)
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    hbuf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    stream = torch.cuda.current_stream()
    info = [None]

    def snap_d():
        info[0] = rlt.rlt_snapshot(model.h, st, dbuf)

    def rest_d():
        rlt.rlt_restore(model.h, st, info[0], dbuf)

    def snap_h():
        info[0] = rlt.rlt_snapshot(model.h, st, hbuf)

    def rest_h():
        rlt.rlt_restore(model.h, st, info[0], hbuf)

    res = {}
    for name, fn in (("snapshot_device", snap_d), ("restore_device", rest_d), ("snapshot_host", snap_h),
                     ("restore_host", rest_h)):
        fn()
        ms = _events(torch, stream, fn, args.steps)
        res[name] = {"ms": ms, "GBs": nbytes / (ms / 1e3) / 1e9}
        print(f"[bench] {name}: {ms:.3f} ms", flush=True)
    model.close()
    ms = res["snapshot_device"]["ms"]
    ach = 2 * nbytes / (ms / 1e3) / 1e9
    out = {
        "metric": SNAP_METRIC, "value": nbytes / (ms / 1e3) / 1e9, "unit": "GB/s (payload, device snapshot)",
        "n_gpus": 1, "steps": args.steps, "warmup": 1, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp16": "f16", "fp16x2": "f16x2"}[cfg.path_dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} state after a {base}-position prefill, B={B}, encoder cache kept",
                   "batch": B, "positions": base, "payload_bytes": nbytes},
        "copies": res,
        "roofline": {"bound": "hbm", "kernel": "device snapshot (payload read + written once)",
                     "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": 2 * nbytes},
    }
    if not args.no_cpu:
        import copy
        from oracle import Oracle
        cs = cfg.replace(batch=1)
        o = Oracle(cs, make_params(cs, bf16_storage=cs.d >= 4096), np.float32)
        ost = o.new_state(1)
        o.encoder_chunk(ost, make_tokens(cs, batch=1, length=min(base, 64)))
        t1 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t1 < 5.0:
            copy.deepcopy(ost)
            reps += 1
        dt = time.perf_counter() - t1
        cache = sum(a.nbytes for l in ost.enc_k + ost.enc_v for a in l) + \
            sum(a.nbytes for g in ost.mem_k + ost.mem_v for a in g)
        out["cpu_baseline"] = {"value": cache * reps / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"deep copies of the oracle's state of 1 row after {min(base, 64)} "
                                         f"encoded positions ({cache / 1e6:.1f} MB of caches and memory), "
                                         f"{reps} copies in {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def mem_attn_bytes(cfg, B: int, t: int) -> float:
    """Algorithmic bytes of one decoder cross-attention launch at position t: every row reads the
    keys and values of memory positions 1..t of its group once (16-bit), reads its query and
    writes its output (two-term output rows when GEMM inputs are two-term)."""
    e = 2 if cfg.dtype == "bf16" else 4
    act = 2 if cfg.path_dtype == "fp16x2" else 1
    return B * (t * 2 * cfg.hd * e + cfg.hd * e + act * cfg.hd * e)


def decode_bench(args, cfg, prompt: int):
    """Decoder transitions at position ~prompt for the whole batch, plus the encoder prefill.

    Encodes prompt + warmup + 2 steps tokens per row (timed: encoder tok/s), seeks the
    decoder to position `prompt` (the window rings cleared, the memory of every encoded
    position real: rlt_state_seek), runs `warmup` transitions, then times `steps` transitions
    with HIP events around the whole run (the value). A second run of `steps` transitions with
    the per-kernel event timers on gives the step breakdown and the cross-attention's
    per-launch duration (the timers' own events would slow the first run). A step is one
    batched transition (merge, L_D blocks, readout with fp32 logits) of every row."""
    import torch
    from recurrent_looped_transformer_amd import rlt
    from recurrent_looped_transformer_amd.synth import make_params, make_tokens
    B, K, Wm = cfg.batch, args.steps, args.warmup
    T = prompt + Wm + 2 * K
    t0 = time.perf_counter()
    P = make_params(cfg, bf16_storage=cfg.d >= 4096)
    torch.cuda.set_device(0)
    model = rlt.Model(cfg, P)
    print(f"[bench] {cfg.name}: parameters drawn and packed in {time.perf_counter() - t0:.0f} s", flush=True)
    tokens = make_tokens(cfg, length=T)
    x = torch.as_tensor(tokens).cuda()
    st = model.state(B, T, keep_encoder_cache=False)
    stream = torch.cuda.current_stream()
    lg = torch.empty((B, K, cfg.vocab), dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    rlt.rlt_encode(model.h, st, x)
    ev[1].record(stream)
    torch.cuda.synchronize()
    enc_ms = ev[0].elapsed_time(ev[1])
    print(f"[bench] encode of {B} x {T} tokens: {enc_ms:.0f} ms", flush=True)
    rlt.rlt_state_seek(model.h, st, prompt)
    if Wm:
        rlt.rlt_decode_scan(model.h, st, Wm)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev[2].record(stream)
    rlt.rlt_decode_scan(model.h, st, K, logits=lg)
    ev[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    scan_ms = ev[2].elapsed_time(ev[3])
    # second run with the per-kernel timers (breakdown, dominant kernel's launch duration)
    rlt.rlt_kernel_timing(model.h, True)
    rlt.rlt_decode_scan(model.h, st, K, logits=lg)
    torch.cuda.synchronize()
    att_ms, att_n = rlt.rlt_kernel_time(model.h, rlt.TIME_MEMORY_ATTN)
    win_ms, win_n = rlt.rlt_kernel_time(model.h, rlt.TIME_WINDOW_ATTN)
    gem_ms, gem_n = rlt.rlt_kernel_time(model.h, rlt.TIME_DECODER_GEMM)
    rlt.rlt_kernel_timing(model.h, False)
    assert att_n == K * cfg.L_D, (att_n, K * cfg.L_D)
    pos = list(range(prompt + Wm + 1, prompt + Wm + K + 1))
    pos2 = list(range(prompt + Wm + K + 1, prompt + Wm + 2 * K + 1))
    ms_step = scan_ms / K
    sb = scan_bytes(cfg, B, K, t_start=prompt + Wm)
    att_bytes = float(np.mean([mem_attn_bytes(cfg, B, t) for t in pos2]))
    att_avg = att_ms / att_n
    ach = att_bytes / (att_avg / 1e3) / 1e9
    ef = encoder_flops(cfg, B, T)
    act = 2 if cfg.path_dtype == "fp16x2" else 1
    traffic = None
    tf = os.path.join(ROOT, "profiles", f"traffic_memattn_{cfg.name}.json")
    if os.path.exists(tf):
        try:
            rec = json.load(open(tf))
            if rec.get("lib_sha") == rlt_lib_sha() and rec.get("B") == B and rec.get("position") == prompt:
                traffic = rec.get("bytes_per_launch")
        except Exception:
            traffic = None
    kern = f"attn_decode_k<{'f16' if cfg.path_dtype != 'bf16' else 'bf16'},{cfg.d_head},false,1> " \
           f"(decoder cross-attention over the memory prefix)"
    out = {
        "metric": METRIC, "value": B * K / (scan_ms / 1e3), "unit": "transitions/s", "n_gpus": 1,
        "steps": K, "warmup": Wm, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp16": "f16", "fp16x2": "f16x2"}[cfg.path_dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: decoder transitions of B={B} rows at positions {pos[0]}-{pos[-1]} "
                               f"(RLT-{cfg.variant}, L_E+L_D={cfg.L_E}+{cfg.L_D}{' shared' if cfg.share else ''}, "
                               f"d {cfg.d}, {cfg.n_heads}x{cfg.d_head} heads, SwiGLU {cfg.ffn}, W {cfg.window}, "
                               f"vocab {cfg.vocab}) after the {T}-token encode of the Zipf prompt; the decoder is "
                               f"sought to position {prompt} (memory real, window entries zero), a step is one "
                               f"batched transition with fp32 logits",
                   "batch": B, "prompt": prompt, "positions": [pos[0], pos[-1]], "d": cfg.d, "L_E": cfg.L_E,
                   "L_D": cfg.L_D, "window": cfg.window, "groups": cfg.groups, "vocab": cfg.vocab,
                   "shared": bool(cfg.share), "variant": f"RLT-{cfg.variant}", "gemm_inputs": "two-term" if act == 2
                   else "one-term"},
        "decode_transitions_s": B * K / (scan_ms / 1e3),
        "decode_step_ms": ms_step,
        "step_roofline": {"bound": "hbm", "achieved": sb / (scan_ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": sb / (scan_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                          "algorithmic_bytes_per_step": sb / K},
        "step_breakdown_ms": {"memory_attention": att_ms / K, "window_attention": win_ms / K,
                              "gemms": gem_ms / K, "launches_per_step": (att_n + win_n + gem_n) / K,
                              "positions": [pos2[0], pos2[-1]],
                              "note": "a second run of the same number of steps with per-kernel event timers"},
        "encoder_tok_s": B * T / (enc_ms / 1e3), "encoder_ms": enc_ms, "encoder_tokens": B * T,
        "encoder_tflops": ef / (enc_ms / 1e3) / 1e12,
        "encoder_mfma_frac": ef / (enc_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": att_bytes,
                     "avg_launch_ms": att_avg, "launches": att_n},
        "wall_s_timed": wall,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_steps(cfg, P, tokens, args.cpu_seconds)
    model.close()
    print(json.dumps(out), flush=True)


def cpu_baseline_steps(cfg, P, tokens, budget_s: float):
    """The oracle (float32 numpy, as it stands) on one row: encode 2 tokens, then decoder
    transitions until the time budget is spent (at least one). Its per-transition cost is the
    decoder's weights streamed once per position and row, nearly independent of the position."""
    from threadpoolctl import threadpool_info
    from oracle import Oracle
    o = Oracle(cfg, P, np.float32)
    st = o.new_state(1)
    n_enc = 8
    t0 = time.perf_counter()
    o.encoder_chunk(st, tokens[:1, :n_enc])
    enc_s = time.perf_counter() - t0
    t1 = time.perf_counter()
    n = 0
    while n < n_enc and (n == 0 or time.perf_counter() - t1 < budget_s):
        o.decode(st, 1)
        n += 1
    dt = time.perf_counter() - t1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": n / dt, "unit": "transitions/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 row: encode of {n_enc} tokens ({enc_s:.1f} s, {n_enc / enc_s:.2f} tok/s), then {n} "
                      f"decoder transitions at positions 1-{n} ({dt:.1f} s), float32 numpy"}


def cpu_baseline(cfg, P, tokens, sample_B: int):
    from threadpoolctl import threadpool_info
    from oracle import Oracle
    x = tokens[:sample_B]
    o = Oracle(cfg, P)
    t0 = time.perf_counter()
    o.replay(x)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": x.shape[0] * x.shape[1] / dt, "unit": "transitions/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{x.shape[0]} of {tokens.shape[0]} sequences x {x.shape[1]} positions, full replay "
                      f"(encode + scan + log-probs), float64 numpy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default=None,
                    help="workload (default: paper_shared for the decoder-transition line; algo_bf16 for "
                         "--replay, --grad, --ragged, --generate and --snapshot)")
    ap.add_argument("--replay", action="store_true",
                    help="time whole replays (encode + scan over every position + log-probs) instead of "
                         "decoder transitions at the prompt's end")
    ap.add_argument("--prompt", type=int, default=0, help="decoder position of the timed transitions "
                                                           "(default: the configuration's prompt length)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--batch", type=int, default=0)
    ap.add_argument("--seq-len", type=int, default=0)
    ap.add_argument("--variant", type=int, default=-1)
    ap.add_argument("--scan-mode", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=32)
    ap.add_argument("--progress-every", type=int, default=0,
                    help="issue the scan as calls of this many positions, each followed by a sync and a "
                         "progress line (slow profiler passes; adds one norm kernel per call)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (counter calibration)")
    ap.add_argument("--sweep", default="",
                    help="decode: decoder transitions at batch 1-8 (and the given --sweep-batches) at "
                         "t = 32 and the prompt length of each shape; prints one JSON line per point")
    ap.add_argument("--sweep-shapes", default="algo_bf16,medium_lm,paper_shared")
    ap.add_argument("--sweep-batches", default="1,2,4,8")
    ap.add_argument("--sweep-positions", default="32,prompt",
                    help="decoder positions of the sweep points (\"prompt\": the shape's prompt length)")
    ap.add_argument("--generate", action="store_true",
                    help="time rlt_generate (on-device sampling with recorded log-probabilities) and the sampler")
    ap.add_argument("--snapshot", action="store_true",
                    help="time prefix snapshot / restore to device and pinned-host buffers")
    ap.add_argument("--ragged", action="store_true",
                    help="time generation steps of rows at unequal positions (continuous batching)")
    ap.add_argument("--ragged-base", type=int, default=0)
    ap.add_argument("--ragged-spread", type=int, default=512)
    ap.add_argument("--checkpoint", action="store_true",
                    help="with --grad: activation checkpointing (recompute block intermediates per position)")
    ap.add_argument("--grad", action="store_true",
                    help="time the full-BPTT gradient of the replay (fp32 arithmetic) instead of the replay")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the RLT scan shards over independent sequences with no "
              "exchange during the scan, and this build runs on a single MI355X (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.sweep == "decode":
        from recurrent_looped_transformer_amd.synth import CONFIGS
        shapes = [x for x in args.sweep_shapes.split(",") if x]
        pos = {n: [CONFIGS[n].seq_len if p == "prompt" else int(p) for p in args.sweep_positions.split(",") if p]
               for n in shapes}
        decode_sweep(shapes, [int(b) for b in args.sweep_batches.split(",")], pos)
        return
    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}))
        return
    from recurrent_looped_transformer_amd import rlt
    from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens

    if args.config is None:
        side = args.replay or args.grad or args.ragged or args.generate or args.snapshot
        args.config = "algo_bf16" if side else "paper_shared"
    cfg = CONFIGS[args.config]
    if args.batch:
        cfg = cfg.replace(batch=args.batch)
    if args.seq_len:
        cfg = cfg.replace(seq_len=args.seq_len)
    if args.variant >= 0:
        cfg = cfg.replace(variant=args.variant, chunk=cfg.chunk if args.variant == 2 else 1)
    if args.grad:
        grad_bench(args, cfg)
        return
    if args.ragged:
        ragged_bench(args, cfg)
        return
    if args.generate:
        generate_bench(args, cfg)
        return
    if args.snapshot:
        snapshot_bench(args, cfg)
        return
    if not args.replay:
        decode_bench(args, cfg, args.prompt or cfg.seq_len)
        return
    B, T = cfg.batch, cfg.seq_len
    P = make_params(cfg)
    tokens = make_tokens(cfg, length=T)
    nxt = np.concatenate([tokens[:, 1:], np.full((B, 1), -1, np.int32)], axis=1)

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    x = torch.as_tensor(tokens).to(dev)
    nx = torch.as_tensor(np.ascontiguousarray(nxt)).to(dev)
    lp = torch.empty((B, T), dtype=torch.float32, device=dev)
    model = rlt.Model(cfg, P)
    if args.scan_mode:
        rlt.rlt_set_scan_mode(model.h, args.scan_mode)
    st = model.state(B, T, keep_encoder_cache=False)
    stream = torch.cuda.current_stream()
    pieces = []   # (first column, positions, log-prob buffer, next tokens) of each progress call
    for c0 in range(0, T, args.progress_every if args.progress_every > 0 else T):
        n = min(args.progress_every, T - c0) if args.progress_every > 0 else T
        pieces.append((c0, n, torch.empty((B, n), dtype=torch.float32, device=dev), nx[:, c0:c0 + n].contiguous()))

    def step(evs=None):
        rlt.rlt_state_reset(model.h, st)
        if evs: evs[0].record(stream)
        rlt.rlt_encode(model.h, st, x)
        if evs: evs[1].record(stream)
        if args.progress_every > 0:
            for c0, n, lpc, nxc in pieces:
                rlt.rlt_decode_scan(model.h, st, n, next_logprob=lpc, next_tokens=nxc)
                torch.cuda.synchronize()
                print(f"[bench] scan positions {c0 + n}/{T} done", flush=True)
        else:
            rlt.rlt_decode_scan(model.h, st, T, next_logprob=lp, next_tokens=nx)
        if evs: evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    ms_per_step = wall * 1e3 / args.steps
    value = B * T / (ms_per_step / 1e3)

    sb = scan_bytes(cfg, B, T)
    achieved = sb / (scan_ms / 1e3) / 1e9
    ef = encoder_flops(cfg, B, T)
    traffic = None
    tf = os.path.join(ROOT, "profiles", f"traffic_scan_{cfg.name}.json")
    if os.path.exists(tf):
        try:
            rec = json.load(open(tf))
            if rec.get("scan_mode") == args.scan_mode and rec.get("B") == B and rec.get("T") == T and \
                    rec.get("lib_sha") == rlt_lib_sha():
                traffic = rec.get("bytes_per_launch")
        except Exception:
            traffic = None

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "transitions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp16": "f16", "fp16x2": "f16x2"}[cfg.path_dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} replay (encode + decoder scan + log-probs), "
                               f"RLT-{cfg.variant} B={B} T={T}",
                   "batch": B, "seq_len": T, "d": cfg.d, "L_E": cfg.L_E, "L_D": cfg.L_D,
                   "window": cfg.window, "groups": cfg.groups, "vocab": cfg.vocab,
                   "variant": f"RLT-{cfg.variant}", "chunk": cfg.chunk, "scan_mode": args.scan_mode},
        "encoder_tok_s": B * T / (enc_ms / 1e3),
        "encoder_ms": enc_ms,
        "encoder_tflops": ef / (enc_ms / 1e3) / 1e12,
        "decode_transitions_s": B * T / (scan_ms / 1e3),
        "decode_scan_ms": scan_ms,
        "roofline": {"bound": "hbm", "kernel": "decoder scan (all T transitions, one launch sequence)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": sb},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, P, tokens, min(args.cpu_sample, B))
    model.close()
    print(json.dumps(out), flush=True)


def rlt_lib_sha() -> str:
    import hashlib
    p = os.path.join(ROOT, "recurrent_looped_transformer_amd", "librlt.so")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16] if os.path.exists(p) else ""


if __name__ == "__main__":
    main()
