"""Decode GEMMs cut along K (split-K: partial tiles, then a reduce-and-epilogue kernel), on the GPU.

Shape: the language-model widths (d 2048, 16 x 128 heads, SwiGLU 5632, vocab 32000) with
2 + 2 blocks, two-term fp16 GEMM inputs, RLT-1, 12 positions. Every decode GEMM whose K is
at least 2048 can be cut into 2 or 4 runs of K here. RLT_SKINNY_TILE, read when a model is
created, forces one tile shape and split count on every decode launch of that model that
admits it (tiles of TPW x 16 features and NMB x 16 rows, S splits); for each forced shape:
- the prefill logits (decoder GEMMs at B rows) and the logits of rlt_step calls after an
  8-position prefill (encoder-step and decoder GEMMs at B rows) meet the oracle bar on rows
  0-1 and agree with the cost model's own choice on every row;
- two runs give identical logits, bit for bit (the partial tiles are added in split order).
Batches of 40 and 80 rows: a ragged row block, and two row blocks.
In batch-invariant mode a forced split is ignored (a row's sums keep one order), so the
first rows of the 80-row batch equal the same rows run alone, bit for bit.
"""
import os

import numpy as np
import pytest
import torch

from oracle import Oracle
from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import CONFIGS, make_params, make_tokens

pytestmark = pytest.mark.gpu
CFG = CONFIGS["medium_lm"].replace(L_E=2, L_D=2, batch=80, seq_len=12, gen_len=0)
T = 12
P_PRE = 8
TOL = 2e-2
TILES = ["4x2x4", "4x2x2", "2x2x4", "1x1x2", "4x1x4"]


@pytest.fixture(scope="module")
def lm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    P = make_params(CFG)
    x = make_tokens(CFG)[:, :T]
    ref = Oracle(CFG, P, np.float32).replay(x[:2])[1]          # logits [2, T, V]
    models = {}
    yield P, x, ref, models
    for m in models.values():
        m.close()


def model(lm, tile):
    """The model created with RLT_SKINNY_TILE = tile (None: unset), one per tile."""
    P, _, _, models = lm
    if tile not in models:
        if tile is None:
            os.environ.pop("RLT_SKINNY_TILE", None)
        else:
            os.environ["RLT_SKINNY_TILE"] = tile
        try:
            models[tile] = rlt.Model(CFG, P)
        finally:
            os.environ.pop("RLT_SKINNY_TILE", None)
    return models[tile]


def run(m, x):
    """(prefill logits of every position, logits of rlt_step at positions P_PRE+1..T after a
    P_PRE-position prefill), on the host."""
    B = x.shape[0]
    xt = torch.as_tensor(np.ascontiguousarray(x)).cuda()
    st = m.state(B, T, keep_encoder_cache=True)
    full, _ = m.prefill(st, xt)
    st2 = m.state(B, T, keep_encoder_cache=True)
    m.prefill(st2, xt[:, :P_PRE].contiguous(), want_logits=False)
    steps = torch.stack([m.step(st2, xt[:, i].contiguous()) for i in range(P_PRE, T)], dim=1)
    torch.cuda.synchronize()
    out = full.cpu().numpy(), steps.cpu().numpy()
    for s in (st, st2):
        rlt.rlt_state_destroy(s)
        m.states.remove(s)
    return out


@pytest.mark.parametrize("B", [40, 80])
def test_forced_splits_match_oracle_and_unsplit(lm, B):
    _, x, ref, _ = lm
    xb = x[:B]
    base_full, base_steps = run(model(lm, None), xb)
    e0 = float(np.max(np.abs(base_full[:2] - ref)))
    print(f"[parity] split-K B={B} cost-model tiles: prefill vs oracle {e0:.3e}", flush=True)
    assert e0 <= TOL
    for tile in TILES:
        print(f"[case] split-K B={B} tile {tile}", flush=True)
        m = model(lm, tile)
        full, steps = run(m, xb)
        again, again_steps = run(m, xb)
        e_full = float(np.max(np.abs(full[:2] - ref)))
        e_steps = float(np.max(np.abs(steps[:2] - ref[:, P_PRE:])))
        d_full = float(np.max(np.abs(full - base_full)))
        d_steps = float(np.max(np.abs(steps - base_steps)))
        print(f"[parity] split-K B={B} tile {tile}: prefill vs oracle {e_full:.3e}, steps vs oracle {e_steps:.3e}; "
              f"vs cost-model tiles (all rows) prefill {d_full:.3e}, steps {d_steps:.3e}", flush=True)
        assert e_full <= TOL and e_steps <= TOL
        assert d_full <= TOL and d_steps <= TOL
        assert np.array_equal(full, again) and np.array_equal(steps, again_steps)


def test_batch_invariant_mode_ignores_splits(lm):
    _, x, _, _ = lm
    split, plain = model(lm, "4x2x4"), model(lm, None)
    for m in (split, plain):
        rlt.rlt_set_batch_invariant(m.h, True)
    try:
        split_full, split_steps = run(split, x)
        plain_full, plain_steps = run(plain, x)
        small_full, small_steps = run(split, x[:2])
    finally:
        for m in (split, plain):
            rlt.rlt_set_batch_invariant(m.h, False)
    print("[parity] split-K batch-invariant: forced split == no override == rows alone "
          f"{np.array_equal(split_full, plain_full) and np.array_equal(split_full[:2], small_full)}", flush=True)
    assert np.array_equal(split_full, plain_full) and np.array_equal(split_steps, plain_steps)
    assert np.array_equal(split_full[:2], small_full) and np.array_equal(split_steps[:2], small_steps)
