"""Python binding of librlt (ctypes). Argument marshalling only: every step of the
forward pass runs in the library's HIP kernels. torch supplies device memory and
the stream; no torch type crosses the C ABI.

The functions mirror include/rlt.h one to one (same names); device arguments are
torch tensors on the GPU, passed as raw pointers.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np
import torch

from . import synth

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librlt.so")

RLT_OK = 0
STATUS = {0: "RLT_OK", -1: "RLT_ERR_INVALID_ARG", -2: "RLT_ERR_UNSUPPORTED", -3: "RLT_ERR_OOM",
          -4: "RLT_ERR_CAPACITY", -5: "RLT_ERR_STALE_STATE", -6: "RLT_ERR_HIP", -7: "RLT_ERR_ORDER"}

EXPORTS = ["rlt_create", "rlt_update_weights", "rlt_destroy", "rlt_state_create", "rlt_state_reset",
           "rlt_state_destroy", "rlt_state_bytes", "rlt_state_positions", "rlt_encode", "rlt_decode_scan",
           "rlt_step", "rlt_replay", "rlt_set_scan_mode", "rlt_state_block_steps", "rlt_status_string",
           "rlt_last_error", "rlt_sample", "rlt_generate", "rlt_importance_ratio", "rlt_snapshot_size",
           "rlt_snapshot", "rlt_restore", "rlt_set_batch_invariant", "rlt_replay_grad_workspace",
           "rlt_replay_grad", "rlt_step_rows", "rlt_state_reset_rows", "rlt_state_row_positions",
           "rlt_sample_workspace", "rlt_state_seek", "rlt_kernel_timing", "rlt_kernel_time", "rlt_sample_noalloc"]

# kernel kinds of rlt_kernel_time (rlt_time_kind)
TIME_MEMORY_ATTN, TIME_WINDOW_ATTN, TIME_ENCODER_ATTN, TIME_ENCODER_GEMM, TIME_DECODER_GEMM = range(5)


class RltError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class rlt_config(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int), ("d", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("d_head", ctypes.c_int), ("L_E", ctypes.c_int), ("L_D", ctypes.c_int),
                ("ffn", ctypes.c_int), ("window", ctypes.c_int), ("groups", ctypes.c_int),
                ("variant", ctypes.c_int), ("chunk", ctypes.c_int), ("share_enc_dec", ctypes.c_int),
                ("dtype", ctypes.c_int), ("alpha", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("rope_base", ctypes.c_float)]


class rlt_snapshot_info(ctypes.Structure):
    _fields_ = [("config_digest", ctypes.c_uint64), ("weights_digest", ctypes.c_uint64), ("batch", ctypes.c_int32),
                ("n_encoded", ctypes.c_int32), ("n_decoded", ctypes.c_int32), ("window", ctypes.c_int32),
                ("ring_slots", ctypes.c_int32), ("has_encoder_cache", ctypes.c_int32),
                ("block_steps", ctypes.c_int64), ("bytes", ctypes.c_int64)]


class rlt_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class rlt_grad_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("numel", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librlt.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m recurrent_looped_transformer_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)
    sig = {
        "rlt_create": [ctypes.POINTER(rlt_config), ctypes.POINTER(rlt_tensor), i32, vp, ctypes.POINTER(vp)],
        "rlt_update_weights": [vp, ctypes.POINTER(rlt_tensor), i32, vp],
        "rlt_destroy": [vp],
        "rlt_state_create": [vp, i32, i32, i32, vp, ctypes.POINTER(vp)],
        "rlt_state_reset": [vp, vp, vp],
        "rlt_state_destroy": [vp],
        "rlt_state_bytes": [vp, i64p],
        "rlt_state_positions": [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)],
        "rlt_encode": [vp, vp, vp, i32, vp],
        "rlt_decode_scan": [vp, vp, i32, vp, vp, vp, vp, vp],
        "rlt_step": [vp, vp, vp, vp, vp],
        "rlt_replay": [vp, vp, vp, i32, vp, vp, vp],
        "rlt_set_scan_mode": [vp, i32],
        "rlt_state_seek": [vp, vp, i32, vp],
        "rlt_kernel_timing": [vp, i32],
        "rlt_kernel_time": [vp, i32, ctypes.POINTER(ctypes.c_double), i64p],
        "rlt_set_batch_invariant": [vp, i32],
        "rlt_state_block_steps": [vp, i64p],
        "rlt_sample": [vp, i32, i32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp,
                       ctypes.c_int64, vp],
        "rlt_sample_workspace": [i32, i32, i64p],
        "rlt_sample_noalloc": [vp, i32, i32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, vp,
                               vp, vp],
        "rlt_generate": [vp, vp, vp, i32, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp, vp],
        "rlt_importance_ratio": [vp, vp, ctypes.c_int64, vp, vp],
        "rlt_snapshot_size": [vp, vp, i64p],
        "rlt_snapshot": [vp, vp, vp, ctypes.c_int64, ctypes.POINTER(rlt_snapshot_info), vp],
        "rlt_restore": [vp, vp, ctypes.POINTER(rlt_snapshot_info), vp, vp],
        "rlt_replay_grad_workspace": [ctypes.POINTER(rlt_config), i32, i32, i32, i64p],
        "rlt_step_rows": [vp, vp, vp, ctypes.POINTER(ctypes.c_int32), vp, vp],
        "rlt_state_reset_rows": [vp, vp, ctypes.POINTER(ctypes.c_int32), vp],
        "rlt_state_row_positions": [vp, ctypes.POINTER(ctypes.c_int32)],
        "rlt_replay_grad": [ctypes.POINTER(rlt_config), ctypes.POINTER(rlt_tensor), i32,
                            ctypes.POINTER(rlt_grad_tensor), i32, vp, i32, i32, vp, vp, i32, vp, ctypes.c_int64,
                            vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.rlt_status_string.argtypes = [ctypes.c_int]
    L.rlt_status_string.restype = ctypes.c_char_p
    L.rlt_last_error.argtypes = []
    L.rlt_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(code: int) -> None:
    if code != RLT_OK:
        raise RltError(code, load().rlt_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("device tensors must be contiguous CUDA tensors")
    return ctypes.c_void_p(t.data_ptr())


def config_struct(cfg: synth.Config) -> rlt_config:
    return rlt_config(cfg.vocab, cfg.d, cfg.n_heads, cfg.d_head, cfg.L_E, cfg.L_D, cfg.ffn, cfg.window,
                      cfg.groups, cfg.variant, cfg.chunk, 1 if cfg.share else 0,
                      {"fp32": 0, "bf16": 1, "fp16": 2, "fp16x2": 3}[cfg.path_dtype], cfg.alpha, cfg.rms_eps, cfg.rope_base)


def _tensors(params: Dict[str, np.ndarray], device) -> tuple:
    keep, arr = [], (rlt_tensor * len(params))()
    for i, (name, a) in enumerate(params.items()):
        t = torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        keep.append(t)
        arr[i] = rlt_tensor(name.encode(), t.data_ptr(), t.numel())
    return arr, keep


# ----------------------------------------------------------------- C ABI mirror
def rlt_create(cfg: synth.Config, params: Dict[str, np.ndarray], device="cuda") -> ctypes.c_void_p:
    L = load()
    arr, keep = _tensors(params, device)
    out = ctypes.c_void_p()
    c = config_struct(cfg)
    _check(L.rlt_create(ctypes.byref(c), arr, len(params), ctypes.c_void_p(_stream()), ctypes.byref(out)))
    del keep
    torch.cuda.empty_cache()   # the fp32 staging copies (46.7 GB at the paper shape) go back to the device
    return out


def rlt_update_weights(model, params: Dict[str, np.ndarray], device="cuda") -> None:
    arr, keep = _tensors(params, device)
    _check(load().rlt_update_weights(model, arr, len(params), ctypes.c_void_p(_stream())))
    del keep


def rlt_destroy(model) -> None:
    _check(load().rlt_destroy(model))


# Rows of every live state: a buffer passed with a state must hold exactly that many rows (the
# library reads and writes [rows, ...] through plain pointers, so a shorter tensor would be
# accessed out of bounds on the device).
_STATE_ROWS: Dict[int, int] = {}


def _rows(state, *tensors) -> None:
    rows = _STATE_ROWS.get(state.value if isinstance(state, ctypes.c_void_p) else int(state))
    if rows is None:
        return
    for t in tensors:
        if t is not None and (t.dim() == 0 or t.shape[0] != rows):
            raise ValueError(f"a tensor of shape {tuple(t.shape)} passed with a state of {rows} rows")


def rlt_state_create(model, batch: int, max_len: int, keep_encoder_cache: bool = True) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    _check(load().rlt_state_create(model, batch, max_len, 1 if keep_encoder_cache else 0,
                                   ctypes.c_void_p(_stream()), ctypes.byref(out)))
    _STATE_ROWS[out.value] = batch
    return out


def rlt_state_reset(model, state) -> None:
    _check(load().rlt_state_reset(model, state, ctypes.c_void_p(_stream())))


def rlt_state_destroy(state) -> None:
    _check(load().rlt_state_destroy(state))
    _STATE_ROWS.pop(state.value if isinstance(state, ctypes.c_void_p) else int(state), None)


def rlt_state_bytes(state) -> list:
    out = (ctypes.c_int64 * 6)()
    _check(load().rlt_state_bytes(state, out))
    return list(out)


def rlt_state_positions(state) -> tuple:
    a, b = ctypes.c_int(), ctypes.c_int()
    _check(load().rlt_state_positions(state, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def rlt_state_block_steps(state) -> int:
    out = ctypes.c_int64()
    _check(load().rlt_state_block_steps(state, ctypes.byref(out)))
    return out.value


def rlt_set_scan_mode(model, mode: int) -> None:
    _check(load().rlt_set_scan_mode(model, mode))


def rlt_state_seek(model, state, n: int) -> None:
    _check(load().rlt_state_seek(model, state, n, ctypes.c_void_p(_stream())))


def rlt_kernel_timing(model, on: bool) -> None:
    _check(load().rlt_kernel_timing(model, 1 if on else 0))


def rlt_kernel_time(model, kind: int) -> tuple:
    """(total ms, launches) of one kernel kind since the last read."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(load().rlt_kernel_time(model, kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def rlt_set_batch_invariant(model, on: bool) -> None:
    _check(load().rlt_set_batch_invariant(model, 1 if on else 0))


def rlt_encode(model, state, tokens: torch.Tensor) -> None:
    assert tokens.dtype == torch.int32 and tokens.dim() == 2
    _rows(state, tokens)
    _check(load().rlt_encode(model, state, _ptr(tokens), tokens.shape[1], ctypes.c_void_p(_stream())))


def rlt_decode_scan(model, state, T: int, logits=None, next_logprob=None, next_tokens=None, s_out=None) -> None:
    _rows(state, logits, next_logprob, next_tokens, s_out)
    _check(load().rlt_decode_scan(model, state, T, _ptr(logits), _ptr(next_logprob), _ptr(next_tokens),
                                  _ptr(s_out), ctypes.c_void_p(_stream())))


def rlt_step(model, state, tokens: torch.Tensor, logits: torch.Tensor) -> None:
    assert tokens.dtype == torch.int32 and tokens.dim() == 1
    _rows(state, tokens, logits)
    _check(load().rlt_step(model, state, _ptr(tokens), _ptr(logits), ctypes.c_void_p(_stream())))


def rlt_replay(model, state, tokens: torch.Tensor, logprob: torch.Tensor, s_out=None) -> None:
    assert tokens.dtype == torch.int32 and tokens.dim() == 2
    _rows(state, tokens, logprob, s_out)
    _check(load().rlt_replay(model, state, _ptr(tokens), tokens.shape[1], _ptr(logprob), _ptr(s_out),
                             ctypes.c_void_p(_stream())))


def rlt_sample_workspace(rows: int, vocab: int) -> int:
    n = ctypes.c_int64(0)
    _check(load().rlt_sample_workspace(rows, vocab, ctypes.byref(n)))
    return n.value


def rlt_sample(logits: torch.Tensor, temperature: float, seed: int, step: int, tokens: torch.Tensor,
               logprob: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> None:
    assert logits.dtype == torch.float32 and logits.dim() == 2 and tokens.dtype == torch.int32
    rows, V = logits.shape
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    wn = workspace.numel() if workspace is not None else 0
    _check(load().rlt_sample(_ptr(logits), rows, V, V, temperature, seed, step, _ptr(tokens), _ptr(logprob),
                             ws, wn, ctypes.c_void_p(_stream())))


def rlt_sample_noalloc(logits: torch.Tensor, temperature: float, seed: int, step: int, tokens: torch.Tensor,
                       logprob: Optional[torch.Tensor] = None) -> None:
    """rlt_sample with the library's static scratch (no allocation here or in the library)."""
    assert logits.dtype == torch.float32 and logits.dim() == 2 and tokens.dtype == torch.int32
    rows, V = logits.shape
    _check(load().rlt_sample_noalloc(_ptr(logits), rows, V, V, temperature, seed, step, _ptr(tokens), _ptr(logprob),
                                     ctypes.c_void_p(_stream())))


def rlt_generate(model, state, first: torch.Tensor, n: int, temperature: float, seed: int, step0: int,
                 tokens: torch.Tensor, logprob: torch.Tensor, logits: Optional[torch.Tensor] = None) -> None:
    assert first.dtype == torch.int32 and first.dim() == 1 and tokens.dtype == torch.int32
    _rows(state, first, tokens, logprob, logits)
    _check(load().rlt_generate(model, state, _ptr(first), n, temperature, seed, step0, _ptr(tokens), _ptr(logprob),
                               _ptr(logits), ctypes.c_void_p(_stream())))


def rlt_importance_ratio(logprob_current: torch.Tensor, logprob_behaviour: torch.Tensor, ratio: torch.Tensor) -> None:
    n = logprob_current.numel()
    assert logprob_behaviour.numel() == n and ratio.numel() == n
    _check(load().rlt_importance_ratio(_ptr(logprob_current), _ptr(logprob_behaviour), n, _ptr(ratio),
                                       ctypes.c_void_p(_stream())))


def rlt_snapshot_size(model, state) -> int:
    n = ctypes.c_int64(0)
    _check(load().rlt_snapshot_size(model, state, ctypes.byref(n)))
    return n.value


def rlt_snapshot(model, state, dst: torch.Tensor) -> rlt_snapshot_info:
    """Snapshot into dst (a contiguous uint8 tensor on the GPU, or pinned on the host)."""
    assert dst.dtype == torch.uint8 and dst.is_contiguous()
    info = rlt_snapshot_info()
    _check(load().rlt_snapshot(model, state, ctypes.c_void_p(dst.data_ptr()), dst.numel(), ctypes.byref(info),
                               ctypes.c_void_p(_stream())))
    return info


def rlt_restore(model, state, info: rlt_snapshot_info, src: torch.Tensor) -> None:
    assert src.dtype == torch.uint8 and src.is_contiguous() and src.numel() >= info.bytes
    _check(load().rlt_restore(model, state, ctypes.byref(info), ctypes.c_void_p(src.data_ptr()),
                              ctypes.c_void_p(_stream())))


def _host_i32(vals) -> ctypes.Array:
    vals = [int(v) for v in vals]
    return (ctypes.c_int32 * len(vals))(*vals)


def rlt_step_rows(model, state, tokens: torch.Tensor, active, logits: torch.Tensor) -> None:
    """One position for the rows with active[b] (host sequence of B flags), each at its own position."""
    assert tokens.dtype == torch.int32 and tokens.dim() == 1 and logits.dtype == torch.float32
    _rows(state, tokens, logits)
    _check(load().rlt_step_rows(model, state, _ptr(tokens), _host_i32(active), _ptr(logits),
                                ctypes.c_void_p(_stream())))


def rlt_state_reset_rows(model, state, rows) -> None:
    _check(load().rlt_state_reset_rows(model, state, _host_i32(rows), ctypes.c_void_p(_stream())))


def rlt_state_row_positions(state, batch: int) -> list:
    out = (ctypes.c_int32 * batch)()
    _check(load().rlt_state_row_positions(state, out))
    return list(out)


def rlt_replay_grad_workspace(cfg: synth.Config, B: int, T: int, checkpoint: bool = False) -> int:
    n = ctypes.c_int64(0)
    c = config_struct(cfg)
    _check(load().rlt_replay_grad_workspace(ctypes.byref(c), B, T, 1 if checkpoint else 0, ctypes.byref(n)))
    return n.value


def rlt_replay_grad(cfg: synth.Config, weights: Dict[str, torch.Tensor], tokens: torch.Tensor,
                    dlogprob: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                    grads: Optional[Dict[str, torch.Tensor]] = None, logprob: Optional[torch.Tensor] = None,
                    checkpoint: bool = False):
    """Full-BPTT gradient of sum(dlogprob * logprob) over the replay of tokens [B, T].

    weights: manifest name -> contiguous fp32 device tensor. Returns (logprob [B, T-1],
    {name: gradient tensor}). The workspace (uint8 device tensor), the gradient tensors and
    the log-probability buffer are allocated here unless given."""
    assert tokens.dtype == torch.int32 and tokens.dim() == 2 and dlogprob.dtype == torch.float32
    B, T = tokens.shape
    dev = tokens.device
    need = rlt_replay_grad_workspace(cfg, B, T, checkpoint)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    assert workspace.dtype == torch.uint8 and workspace.numel() >= need
    names = list(weights)
    warr = (rlt_tensor * len(names))()
    garr = (rlt_grad_tensor * len(names))()
    if grads is None:
        grads = {n: torch.empty_like(weights[n]) for n in names}
    for i, n in enumerate(names):
        t, gt = weights[n], grads[n]
        assert t.dtype == torch.float32 and t.is_contiguous() and t.is_cuda
        assert gt.dtype == torch.float32 and gt.is_contiguous() and gt.numel() == t.numel()
        warr[i] = rlt_tensor(n.encode(), t.data_ptr(), t.numel())
        garr[i] = rlt_grad_tensor(n.encode(), gt.data_ptr(), t.numel())
    if logprob is None:
        logprob = torch.empty(B, T - 1, dtype=torch.float32, device=dev)
    dlp = dlogprob.contiguous()
    c = config_struct(cfg)
    _check(load().rlt_replay_grad(ctypes.byref(c), warr, len(names), garr, len(names), _ptr(tokens), B, T,
                                  _ptr(dlp), _ptr(logprob), 1 if checkpoint else 0, ctypes.c_void_p(workspace.data_ptr()),
                                  workspace.numel(), ctypes.c_void_p(_stream())))
    return logprob, grads


# ----------------------------------------------------------------- convenience
class Model:
    """Owns one rlt_model and frees it on close()."""

    def __init__(self, cfg: synth.Config, params: Dict[str, np.ndarray], device="cuda"):
        self.cfg = cfg
        self.device = device
        self.h = rlt_create(cfg, params, device)
        self.states = []

    def state(self, batch: int, max_len: int, keep_encoder_cache: bool = True):
        s = rlt_state_create(self.h, batch, max_len, keep_encoder_cache)
        self.states.append(s)
        return s

    def replay(self, state, tokens: torch.Tensor, want_s: bool = False):
        B, T = tokens.shape
        lp = torch.empty((B, T - 1), dtype=torch.float32, device=self.device)
        s = torch.empty((B, T, self.cfg.d), dtype=torch.float32, device=self.device) if want_s else None
        rlt_replay(self.h, state, tokens, lp, s)
        return lp, s

    def prefill(self, state, tokens: torch.Tensor, want_logits=True, want_s=False):
        B, T = tokens.shape
        rlt_encode(self.h, state, tokens)
        lg = torch.empty((B, T, self.cfg.vocab), dtype=torch.float32, device=self.device) if want_logits else None
        s = torch.empty((B, T, self.cfg.d), dtype=torch.float32, device=self.device) if want_s else None
        rlt_decode_scan(self.h, state, T, logits=lg, s_out=s)
        return lg, s

    def step(self, state, tok: torch.Tensor):
        lg = torch.empty((tok.shape[0], self.cfg.vocab), dtype=torch.float32, device=self.device)
        rlt_step(self.h, state, tok, lg)
        return lg

    def close(self):
        for s in self.states:
            rlt_state_destroy(s)
        self.states = []
        if self.h is not None:
            rlt_destroy(self.h)
            self.h = None
