"""rlt_sample_noalloc (static scratch, no allocation) against rlt_sample with a workspace.

Both run the same kernels on the same logits; the tokens and log-probabilities must be
identical bit for bit. Two calls in a row, the second on a smaller input, check that the
shared scratch array serves consecutive calls; a call beyond the array's capacity is
rejected on the host before any launch.
"""
import numpy as np
import pytest
import torch

from recurrent_looped_transformer_amd import rlt
from recurrent_looped_transformer_amd.synth import make_logits

pytestmark = pytest.mark.gpu


def draw_both(rows, vocab, temperature, seed, step):
    lg = torch.as_tensor(make_logits(rows, vocab, seed=11 + rows)).cuda()
    tk_ws = torch.empty(rows, dtype=torch.int32, device="cuda")
    lp_ws = torch.empty(rows, dtype=torch.float32, device="cuda")
    ws = torch.empty(rlt.rlt_sample_workspace(rows, vocab), dtype=torch.uint8, device="cuda")
    rlt.rlt_sample(lg, temperature, seed, step, tk_ws, lp_ws, workspace=ws)
    tk = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    lp = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    rlt.rlt_sample_noalloc(lg, temperature, seed, step, tk, lp)
    torch.cuda.synchronize()
    return tk_ws.cpu().numpy(), lp_ws.cpu().numpy(), tk.cpu().numpy(), lp.cpu().numpy()


def test_noalloc_equals_workspace_two_calls():
    for rows, vocab, temp in ((64, 32000, 1.0), (16, 8000, 0.7)):      # the second call is smaller
        a_t, a_l, b_t, b_l = draw_both(rows, vocab, temp, seed=1234, step=rows)
        print(f"[no-alloc] rows {rows} vocab {vocab}: tokens equal {np.array_equal(a_t, b_t)}, "
              f"log mu equal {np.array_equal(a_l, b_l)}", flush=True)
        assert np.array_equal(a_t, b_t)
        assert np.array_equal(a_l.view(np.uint32), b_l.view(np.uint32))


def test_noalloc_rejects_beyond_capacity():
    rows, vocab = 5000, 32000                 # 5000 * 8 * 32 bytes > 1 MiB
    lg = torch.zeros((rows, vocab), dtype=torch.float32, device="cuda")
    tk = torch.empty(rows, dtype=torch.int32, device="cuda")
    with pytest.raises(rlt.RltError) as e:
        rlt.rlt_sample_noalloc(lg, 1.0, 1, 0, tk)
    assert e.value.code == -4
