"""The C-ABI library loads, exports every function include/rlt.h declares, and
rejects invalid arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

from recurrent_looped_transformer_amd import rlt, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlt.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rlt_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rlt.LIB_PATH):
        pytest.fail("librlt.so is not built (run python -m recurrent_looped_transformer_amd.build)")
    return rlt.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["rlt_create", "rlt_destroy", "rlt_state_create", "rlt_state_reset", "rlt_state_destroy",
              "rlt_encode", "rlt_decode_scan", "rlt_step", "rlt_replay", "rlt_status_string"]:
        assert n in names
    assert sorted(rlt.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", rlt.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (rlt_[a-z_]+)\b", out))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert lib.rlt_status_string(0) == b"ok"
    assert lib.rlt_status_string(-5) == b"stale state"
    assert lib.rlt_status_string(-4) == b"capacity exceeded"


def _create(lib, cfg, tensors=None, n=0):
    c = rlt.config_struct(cfg)
    out = ctypes.c_void_p()
    return lib.rlt_create(ctypes.byref(c), tensors, n, None, ctypes.byref(out)), out


def test_config_validation_on_host(lib):
    base = synth.CONFIGS["tiny_fp32"]
    assert _create(lib, base.replace(groups=3))[0] == -2          # G not in {1, L_D}
    assert _create(lib, base.replace(d_head=15, n_heads=4))[0] in (-1, -2)
    assert _create(lib, base.replace(window=0))[0] == -1
    assert _create(lib, base.replace(chunk=2))[0] == -1           # chunk only for RLT-2
    assert _create(lib, base.replace(share=True, L_E=3))[0] == -2
    code, out = _create(lib, base)                                 # valid config, no weights
    assert code == -1 and b"missing weight" in lib.rlt_last_error()
    assert out.value is None


def test_weight_validation_on_host(lib):
    cfg = synth.CONFIGS["tiny_fp32"]
    names = synth.manifest(cfg)
    arr = (rlt.rlt_tensor * len(names))()
    for i, (nm, shp) in enumerate(names):
        arr[i] = rlt.rlt_tensor(nm.encode(), 16, 1)                  # wrong sizes (fake pointer, never read)
    code, _ = _create(lib, cfg, arr, len(names))
    assert code == -1 and b"wrong size" in lib.rlt_last_error()
    arr[0] = rlt.rlt_tensor(b"no.such.weight", 16, 1)
    code, _ = _create(lib, cfg, arr, len(names))
    assert code == -1 and b"unknown weight" in lib.rlt_last_error()


def test_null_arguments(lib):
    assert lib.rlt_encode(None, None, None, 1, None) == -1
    assert lib.rlt_decode_scan(None, None, 1, None, None, None, None, None) == -1
    assert lib.rlt_step(None, None, None, None, None) == -1
    assert lib.rlt_replay(None, None, None, 4, None, None, None) == -1
    assert lib.rlt_state_destroy(None) == -1
    assert lib.rlt_destroy(None) == -1
    assert lib.rlt_set_scan_mode(None, 0) == -1


def test_replay_grad_workspace_and_host_checks(lib):
    """Workspace bytes: positive, 256-byte multiple, growing with T and B; invalid
    arguments are rejected on the host before any launch."""
    cfg = synth.CONFIGS["tiny_fp32"]
    a = rlt.rlt_replay_grad_workspace(cfg, 2, 16)
    b = rlt.rlt_replay_grad_workspace(cfg, 2, 32)
    c = rlt.rlt_replay_grad_workspace(cfg, 4, 16)
    assert 0 < a < b and a < c and a % 256 == 0
    n = ctypes.c_int64(0)
    cs = rlt.config_struct(cfg)
    assert lib.rlt_replay_grad_workspace(ctypes.byref(cs), 2, 1, 0, ctypes.byref(n)) == -1    # T < 2
    assert lib.rlt_replay_grad_workspace(ctypes.byref(cs), 0, 16, 0, ctypes.byref(n)) == -1   # B < 1
    bad = rlt.config_struct(cfg.replace(groups=3))
    assert lib.rlt_replay_grad_workspace(ctypes.byref(bad), 2, 16, 0, ctypes.byref(n)) == -2  # G not in {1, L_D}
    # checkpointing keeps a fraction of the intermediates
    big = synth.CONFIGS["algo_bf16"]
    full = rlt.rlt_replay_grad_workspace(big, 64, 257)
    ck = rlt.rlt_replay_grad_workspace(big, 64, 257, checkpoint=True)
    assert ck < 0.5 * full
    # null tokens / workspace: rejected before touching the device
    assert lib.rlt_replay_grad(ctypes.byref(cs), None, 0, None, 0, None, 2, 16, None, None, 0, None, 0, None) == -1


def test_binding_rejects_tensors_with_other_row_counts():
    """A buffer passed with a state must hold the state's rows: the library accesses [rows, ...]
    through plain pointers, so the binding refuses a shorter (or longer) tensor on the host."""
    import ctypes

    import torch

    from recurrent_looped_transformer_amd import rlt
    h = ctypes.c_void_p(0x1000)                    # a registered handle; nothing is called
    rlt._STATE_ROWS[h.value] = 4
    try:
        rlt._rows(h, torch.zeros(4, 7), None, torch.zeros(4))
        with pytest.raises(ValueError):
            rlt._rows(h, torch.zeros(3, 1100, dtype=torch.int32))
        with pytest.raises(ValueError):
            rlt._rows(h, torch.zeros(4, 7), torch.zeros(5, 7))
        with pytest.raises(ValueError):
            rlt.rlt_replay(None, h, torch.zeros(3, 9, dtype=torch.int32), torch.zeros(3, 8))
    finally:
        rlt._STATE_ROWS.pop(h.value, None)
