"""The precision study (tests/precision_floor.py) on the CPU.

Small shape, always: with nothing rounded the emulating oracle is the oracle, bit for bit;
two-term (hi + lo fp16) operands everywhere move the logits far less than one fp16 term.

Paper shape (48 + 48 shared blocks, d 4096), when RLT_PARAM_CACHE names a directory for the
float32 parameter files (written on first use, 47 GB; a few minutes per case): rounding only
the encoder's attention queries and keys, or only its values, to one fp16 term moves the
logits of 16 positions by more than 1e-2; the storage the GPU path uses with two-term GEMM
inputs (encoder attention operands two-term, the decoder's one fp16 term) stays below 2e-3.
"""
import os

import numpy as np
import pytest

from oracle import Oracle
from recurrent_looped_transformer_amd.synth import CONFIGS, file_params, make_params, make_tokens
from tests.precision_floor import GPU_FP16X2, RoundingOracle, logit_shift


def test_no_rounding_is_the_oracle():
    cfg = CONFIGS["algo_bf16"].replace(batch=2, seq_len=10)
    P = make_params(cfg)
    x = make_tokens(cfg)
    _, ref, _ = Oracle(cfg, P, np.float32).replay(x)
    got = RoundingOracle(cfg, P, {}).logits(x)
    assert np.max(np.abs(got - ref)) < 1e-5      # token-by-token encoder vs the parallel one


def test_two_terms_are_finer_than_one():
    cfg = CONFIGS["algo_bf16"].replace(batch=2, seq_len=10)
    P = make_params(cfg)
    x = make_tokens(cfg)
    one = {k: "fp16" for k in ("enc_qk", "enc_v", "enc_p", "mem_kv", "swa_qkv", "cross_q")}
    two = {k: "fp16x2" for k in one}
    s1, s2 = logit_shift(cfg, P, x, one), logit_shift(cfg, P, x, two)
    assert 0 < s2 < s1 / 20


@pytest.mark.skipif(not os.environ.get("RLT_PARAM_CACHE"), reason="needs RLT_PARAM_CACHE (47 GB of float32 "
                                                                   "parameter files for the paper shape)")
def test_paper_shape_encoder_attention_needs_two_terms():
    cfg = CONFIGS["paper_shared"]
    P = file_params(cfg, os.environ["RLT_PARAM_CACHE"])
    x = make_tokens(cfg, length=cfg.seq_len + cfg.gen_len)[:1, :16]
    assert logit_shift(cfg, P, x, {"enc_qk": "fp16"}) > 1e-2
    assert logit_shift(cfg, P, x, {"enc_v": "fp16"}) > 1e-2
    assert logit_shift(cfg, P, x, GPU_FP16X2) < 2e-3
