"""Python binding of the C ABI in ``include/dpo_head.h`` (argument marshalling only).

Each function has the name of the C entry point it calls.  Arguments are
torch tensors on the GPU (device memory and streams come from torch); sizes
are read from tensor shapes, checked, and passed with raw pointers.  Every
step of the path runs in the HIP library; if the library is not built this
module raises instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

from . import build as _build

DPO_OK = 0
DPO_ERR_NULL = -1
DPO_ERR_SHAPE = -2
DPO_ERR_ALIGN = -3
DPO_ERR_BETA = -4
DPO_ERR_LAYOUT = -5
DPO_ERR_WORKSPACE = -6
DPO_ERR_TARGET_RANGE = -7
DPO_ERR_HIP = -8
DPO_ERR_ALPHA = -9
DPO_ERR_SCRATCH = -10

DPO_PAIRS_ADJACENT = 0
DPO_PAIRS_HALVES = 1

DPO_OP_SEQ_LOGPS = 0
DPO_OP_REF_SCORE = 1
DPO_OP_HEAD_BACKWARD = 2
DPO_OP_LOGITS_SEQ_LOGPS = 3
DPO_OP_LOGITS_BACKWARD = 4
DPO_OP_SHARD_COMBINE = 5
DPO_OP_SEQ_LOGPS_METRICS = 6

DPO_LOSS_LENGTH_NORM = 1
DPO_LOSS_REFERENCE_FREE = 2

HEADER = os.path.join(_build.ROOT, "include", "dpo_head.h")

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_SIGS = {
    "dpo_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "dpo_seq_logps": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "dpo_ref_score": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "dpo_loss": (_I, [_P, _P, _I, ctypes.c_double, _I, _P, _P, _P, _P, _P, _P]),
    "dpo_head_backward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "dpo_logits_seq_logps": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "dpo_logits_backward": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "dpo_loss_ex": (_I, [_P, _P, _P, _I, ctypes.c_double, _I, _I, ctypes.c_double, _P, _P, _P, _P, _P, _P,
                         _P]),
    "dpo_logits_f32_seq_logps": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "dpo_logits_f32_backward": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "dpo_seq_logps_shard": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "dpo_shard_combine": (_I, [_P, _P, _P, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "dpo_head_backward_shard": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _Z,
                                     _P]),
    "dpo_seq_logps_metrics": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dpo_logits_mean": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "dpo_logits_seq_logps_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "dpo_device_status": (_I, [_P, _P]),
    "dpo_strerror": (ctypes.c_char_p, [_I]),
    "dpo_profile_enable": (_I, [_I]),
    "dpo_profile_select": (_I, [ctypes.c_char_p]),
    "dpo_profile_count": (_I, []),
    "dpo_profile_entry": (_I, [_I, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                               ctypes.POINTER(ctypes.c_int)]),
}

_lib = None


class DpoError(RuntimeError):
    """A device-side or HIP failure reported by the library."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def library_path() -> str:
    return _build.LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library {path} is not built: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def declared_functions(header: str = HEADER):
    """Names of the functions the public header declares."""
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dpo_\w+)\s*\(", txt)))


def _check(status: int) -> None:
    if status == DPO_OK:
        return
    msg = lib().dpo_strerror(status).decode()
    if status in (DPO_ERR_NULL, DPO_ERR_SHAPE, DPO_ERR_ALIGN, DPO_ERR_BETA, DPO_ERR_LAYOUT,
                  DPO_ERR_WORKSPACE, DPO_ERR_ALPHA, DPO_ERR_SCRATCH):
        raise ValueError(f"{msg} (status {status})")
    raise DpoError(status, msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class _Dev:
    """Pointers of the call's tensors, all on one GPU; the call runs with that
    GPU current (the library launches on the current device)."""

    def __init__(self, anchor):
        self.dev = anchor.device

    def p(self, t) -> Optional[int]:
        if t is None:
            return None
        if t.device != self.dev:
            raise ValueError(f"tensors on {t.device} and {self.dev}: all arguments must be on one GPU")
        return t.data_ptr()


def _stream(stream, like=None):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    dev = like.device if like is not None else torch.device("cuda")
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, dtype, name, shape=None):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def dpo_workspace_bytes(op: int, rows: int, T: int, H: int, V: int) -> int:
    return int(lib().dpo_workspace_bytes(op, rows, T, H, V))


def alloc_workspace(op: int, rows: int, T: int, H: int, V: int, device="cuda"):
    """A uint8 device tensor of dpo_workspace_bytes() bytes."""
    import torch
    n = dpo_workspace_bytes(op, rows, T, H, V)
    if n == 0:
        raise ValueError("sizes break the shape rules")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dpo_seq_logps(hidden, w_vocab, targets, mask, logp_sum, logp_sum64=None, lse=None, n_tokens=None,
                  workspace=None, stream=None) -> None:
    import torch
    rows, T, H = hidden.shape
    V = w_vocab.shape[0]
    _need(hidden, torch.bfloat16, "hidden")
    _need(w_vocab, torch.bfloat16, "w_vocab", (V, H))
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(logp_sum, torch.float32, "logp_sum", (rows,))
    if logp_sum64 is not None:
        _need(logp_sum64, torch.float64, "logp_sum64", (rows,))
    if lse is not None:
        _need(lse, torch.float32, "lse", (rows, T))
    if n_tokens is not None:
        _need(n_tokens, torch.int32, "n_tokens", (rows,))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(hidden)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_seq_logps(_d.p(hidden), _d.p(w_vocab), _d.p(targets), _d.p(mask), rows, T, H, V,
                                   _d.p(logp_sum), _d.p(logp_sum64), _d.p(lse), _d.p(n_tokens),
                                   _d.p(workspace), workspace.numel(), _stream(stream, hidden)))


def dpo_ref_score(hidden, w_vocab, targets, mask, ref_sum, workspace=None, stream=None) -> None:
    import torch
    rows, T, H = hidden.shape
    V = w_vocab.shape[0]
    _need(hidden, torch.bfloat16, "hidden")
    _need(w_vocab, torch.bfloat16, "w_vocab", (V, H))
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(ref_sum, torch.float32, "ref_sum", (rows,))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(hidden)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_ref_score(_d.p(hidden), _d.p(w_vocab), _d.p(targets), _d.p(mask), rows, T, H, V,
                                   _d.p(ref_sum), _d.p(workspace), workspace.numel(), _stream(stream, hidden)))


def dpo_loss(policy_sum64, ref_sum, beta: float, layout: int, loss, weight, reward=None, margin=None,
             accuracy=None, stream=None) -> None:
    import torch
    R = policy_sum64.shape[0]
    _need(policy_sum64, torch.float64, "policy_sum64")
    _need(ref_sum, torch.float32, "ref_sum", (R,))
    _need(loss, torch.float32, "loss", (1,))
    _need(weight, torch.float32, "weight", (R,))
    if reward is not None:
        _need(reward, torch.float32, "reward", (R,))
    if margin is not None:
        _need(margin, torch.float32, "margin", (R // 2,))
    if accuracy is not None:
        _need(accuracy, torch.float32, "accuracy", (1,))
    if R % 2:
        raise ValueError("rows must be even")
    _d = _Dev(policy_sum64)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_loss(_d.p(policy_sum64), _d.p(ref_sum), R // 2, float(beta), int(layout), _d.p(loss),
                              _d.p(weight), _d.p(reward), _d.p(margin), _d.p(accuracy),
                              _stream(stream, policy_sum64)))


def dpo_head_backward(hidden, w_vocab, targets, mask, lse, weight, d_hidden, d_w_vocab,
                      accumulate_dw: int = 0, workspace=None, stream=None) -> None:
    import torch
    rows, T, H = hidden.shape
    V = w_vocab.shape[0]
    _need(hidden, torch.bfloat16, "hidden")
    _need(w_vocab, torch.bfloat16, "w_vocab", (V, H))
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(lse, torch.float32, "lse", (rows, T))
    _need(weight, torch.float32, "weight", (rows,))
    _need(d_hidden, torch.float32, "d_hidden", (rows, T, H))
    _need(d_w_vocab, torch.float32, "d_w_vocab", (V, H))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(hidden)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_head_backward(_d.p(hidden), _d.p(w_vocab), _d.p(targets), _d.p(mask), rows, T, H, V,
                                       _d.p(lse), _d.p(weight), _d.p(d_hidden), _d.p(d_w_vocab), int(accumulate_dw),
                                       _d.p(workspace), workspace.numel(), _stream(stream, hidden)))


def dpo_logits_seq_logps(logits, targets, mask, logp_sum, logp_sum64=None, lse=None, n_tokens=None,
                         workspace=None, stream=None) -> None:
    import torch
    rows, T, V = logits.shape
    _need(logits, torch.bfloat16, "logits")
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(logp_sum, torch.float32, "logp_sum", (rows,))
    if logp_sum64 is not None:
        _need(logp_sum64, torch.float64, "logp_sum64", (rows,))
    if lse is not None:
        _need(lse, torch.float32, "lse", (rows, T))
    if n_tokens is not None:
        _need(n_tokens, torch.int32, "n_tokens", (rows,))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(logits)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_logits_seq_logps(_d.p(logits), _d.p(targets), _d.p(mask), rows, T, V, _d.p(logp_sum),
                                          _d.p(logp_sum64), _d.p(lse), _d.p(n_tokens), _d.p(workspace),
                                          workspace.numel(), _stream(stream, logits)))


def dpo_logits_seq_logps_noalloc(logits, targets, mask, logp_sum, status, logp_sum64=None, lse=None,
                                 n_tokens=None, stream=None) -> None:
    """The logits forward on the library's static scratch (no workspace, no
    allocation); ``status`` is a one-element int32 device tensor that receives
    DPO_OK or DPO_ERR_TARGET_RANGE on the stream."""
    import torch
    rows, T, V = logits.shape
    _need(logits, torch.bfloat16, "logits")
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(logp_sum, torch.float32, "logp_sum", (rows,))
    _need(status, torch.int32, "status", (1,))
    if logp_sum64 is not None:
        _need(logp_sum64, torch.float64, "logp_sum64", (rows,))
    if lse is not None:
        _need(lse, torch.float32, "lse", (rows, T))
    if n_tokens is not None:
        _need(n_tokens, torch.int32, "n_tokens", (rows,))
    _d = _Dev(logits)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_logits_seq_logps_noalloc(_d.p(logits), _d.p(targets), _d.p(mask), rows, T, V,
                                                  _d.p(logp_sum), _d.p(logp_sum64), _d.p(lse), _d.p(n_tokens),
                                                  _d.p(status), _stream(stream, logits)))


def dpo_logits_backward(logits, targets, mask, lse, weight, d_logits, workspace=None, stream=None) -> None:
    import torch
    rows, T, V = logits.shape
    _need(logits, torch.bfloat16, "logits")
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(lse, torch.float32, "lse", (rows, T))
    _need(weight, torch.float32, "weight", (rows,))
    _need(d_logits, torch.bfloat16, "d_logits", (rows, T, V))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(logits)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_logits_backward(_d.p(logits), _d.p(targets), _d.p(mask), rows, T, V, _d.p(lse),
                                         _d.p(weight), _d.p(d_logits), _d.p(workspace), workspace.numel(),
                                         _stream(stream, logits)))


def dpo_loss_ex(policy_sum64, ref_sum, n_tokens, beta: float, layout: int, flags: int, sft_alpha: float,
                loss, weight, reward=None, margin=None, accuracy=None, nll=None, stream=None) -> None:
    import torch
    R = policy_sum64.shape[0]
    _need(policy_sum64, torch.float64, "policy_sum64")
    if ref_sum is not None:
        _need(ref_sum, torch.float32, "ref_sum", (R,))
    if n_tokens is not None:
        _need(n_tokens, torch.int32, "n_tokens", (R,))
    _need(loss, torch.float32, "loss", (1,))
    _need(weight, torch.float32, "weight", (R,))
    for t, name, shape in ((reward, "reward", (R,)), (margin, "margin", (R // 2,)),
                           (accuracy, "accuracy", (1,)), (nll, "nll", (1,))):
        if t is not None:
            _need(t, torch.float32, name, shape)
    if R % 2:
        raise ValueError("rows must be even")
    _d = _Dev(policy_sum64)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_loss_ex(_d.p(policy_sum64), _d.p(ref_sum), _d.p(n_tokens), R // 2, float(beta),
                                 int(layout), int(flags), float(sft_alpha), _d.p(loss), _d.p(weight),
                                 _d.p(reward), _d.p(margin), _d.p(accuracy), _d.p(nll),
                                 _stream(stream, policy_sum64)))


def dpo_logits_f32_seq_logps(logits, targets, mask, logp_sum, logp_sum64=None, lse=None, n_tokens=None,
                             workspace=None, stream=None) -> None:
    import torch
    rows, T, V = logits.shape
    _need(logits, torch.float32, "logits")
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(logp_sum, torch.float32, "logp_sum", (rows,))
    if logp_sum64 is not None:
        _need(logp_sum64, torch.float64, "logp_sum64", (rows,))
    if lse is not None:
        _need(lse, torch.float32, "lse", (rows, T))
    if n_tokens is not None:
        _need(n_tokens, torch.int32, "n_tokens", (rows,))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(logits)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_logits_f32_seq_logps(_d.p(logits), _d.p(targets), _d.p(mask), rows, T, V,
                                              _d.p(logp_sum), _d.p(logp_sum64), _d.p(lse), _d.p(n_tokens),
                                              _d.p(workspace), workspace.numel(), _stream(stream, logits)))


def dpo_logits_f32_backward(logits, targets, mask, lse, weight, d_logits, workspace=None,
                            stream=None) -> None:
    import torch
    rows, T, V = logits.shape
    _need(logits, torch.float32, "logits")
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(lse, torch.float32, "lse", (rows, T))
    _need(weight, torch.float32, "weight", (rows,))
    _need(d_logits, torch.float32, "d_logits", (rows, T, V))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(logits)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_logits_f32_backward(_d.p(logits), _d.p(targets), _d.p(mask), rows, T, V, _d.p(lse),
                                             _d.p(weight), _d.p(d_logits), _d.p(workspace), workspace.numel(),
                                             _stream(stream, logits)))


def dpo_seq_logps_shard(hidden, w_shard, targets, mask, v_begin: int, V_total: int, part_max, part_sumexp,
                        part_tgt, workspace=None, stream=None) -> None:
    import torch
    rows, T, H = hidden.shape
    Vs = w_shard.shape[0]
    _need(hidden, torch.bfloat16, "hidden")
    _need(w_shard, torch.bfloat16, "w_shard", (Vs, H))
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    for t, name in ((part_max, "part_max"), (part_sumexp, "part_sumexp"), (part_tgt, "part_tgt")):
        _need(t, torch.float32, name, (rows, T))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(hidden)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_seq_logps_shard(_d.p(hidden), _d.p(w_shard), _d.p(targets), _d.p(mask), rows, T, H, Vs,
                                         int(v_begin), int(V_total), _d.p(part_max), _d.p(part_sumexp),
                                         _d.p(part_tgt), _d.p(workspace), workspace.numel(),
                                         _stream(stream, hidden)))


def dpo_shard_combine(part_max, part_sumexp, part_tgt, targets, mask, V_total: int, logp_sum, logp_sum64=None,
                      lse=None, n_tokens=None, workspace=None, stream=None) -> None:
    import torch
    S, rows, T = part_max.shape
    for t, name in ((part_max, "part_max"), (part_sumexp, "part_sumexp"), (part_tgt, "part_tgt")):
        _need(t, torch.float32, name, (S, rows, T))
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(logp_sum, torch.float32, "logp_sum", (rows,))
    if logp_sum64 is not None:
        _need(logp_sum64, torch.float64, "logp_sum64", (rows,))
    if lse is not None:
        _need(lse, torch.float32, "lse", (rows, T))
    if n_tokens is not None:
        _need(n_tokens, torch.int32, "n_tokens", (rows,))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(part_max)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_shard_combine(_d.p(part_max), _d.p(part_sumexp), _d.p(part_tgt), S, _d.p(targets),
                                       _d.p(mask), rows, T, int(V_total), _d.p(logp_sum), _d.p(logp_sum64),
                                       _d.p(lse), _d.p(n_tokens), _d.p(workspace), workspace.numel(),
                                       _stream(stream, part_max)))


def dpo_head_backward_shard(hidden, w_shard, targets, mask, v_begin: int, V_total: int, lse, weight,
                            d_hidden, d_w_shard, accumulate_dw: int = 0, workspace=None, stream=None) -> None:
    import torch
    rows, T, H = hidden.shape
    Vs = w_shard.shape[0]
    _need(hidden, torch.bfloat16, "hidden")
    _need(w_shard, torch.bfloat16, "w_shard", (Vs, H))
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(lse, torch.float32, "lse", (rows, T))
    _need(weight, torch.float32, "weight", (rows,))
    _need(d_hidden, torch.float32, "d_hidden", (rows, T, H))
    _need(d_w_shard, torch.float32, "d_w_shard", (Vs, H))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(hidden)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_head_backward_shard(_d.p(hidden), _d.p(w_shard), _d.p(targets), _d.p(mask), rows, T, H,
                                             Vs, int(v_begin), int(V_total), _d.p(lse), _d.p(weight),
                                             _d.p(d_hidden), _d.p(d_w_shard), int(accumulate_dw),
                                             _d.p(workspace), workspace.numel(), _stream(stream, hidden)))


def dpo_seq_logps_metrics(hidden, w_vocab, targets, mask, logp_sum, logit_sum, logp_sum64=None, lse=None,
                          n_tokens=None, workspace=None, stream=None) -> None:
    import torch
    rows, T, H = hidden.shape
    V = w_vocab.shape[0]
    _need(hidden, torch.bfloat16, "hidden")
    _need(w_vocab, torch.bfloat16, "w_vocab", (V, H))
    _need(targets, torch.int32, "targets", (rows, T))
    _need(mask, torch.uint8, "mask", (rows, T))
    _need(logp_sum, torch.float32, "logp_sum", (rows,))
    _need(logit_sum, torch.float64, "logit_sum", (rows,))
    if logp_sum64 is not None:
        _need(logp_sum64, torch.float64, "logp_sum64", (rows,))
    if lse is not None:
        _need(lse, torch.float32, "lse", (rows, T))
    if n_tokens is not None:
        _need(n_tokens, torch.int32, "n_tokens", (rows,))
    _need(workspace, torch.uint8, "workspace")
    _d = _Dev(hidden)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_seq_logps_metrics(_d.p(hidden), _d.p(w_vocab), _d.p(targets), _d.p(mask), rows, T, H, V,
                                           _d.p(logp_sum), _d.p(logp_sum64), _d.p(lse), _d.p(n_tokens),
                                           _d.p(logit_sum), _d.p(workspace), workspace.numel(),
                                           _stream(stream, hidden)))


def dpo_logits_mean(logit_sum, n_tokens, V: int, layout: int, means, stream=None) -> None:
    import torch
    R = logit_sum.shape[0]
    _need(logit_sum, torch.float64, "logit_sum")
    _need(n_tokens, torch.int32, "n_tokens", (R,))
    _need(means, torch.float32, "means", (2,))
    if R % 2:
        raise ValueError("rows must be even")
    _d = _Dev(logit_sum)
    with torch.cuda.device(_d.dev):
        _check(lib().dpo_logits_mean(_d.p(logit_sum), _d.p(n_tokens), R // 2, int(V), int(layout), _d.p(means),
                                     _stream(stream, logit_sum)))


def dpo_device_status(workspace, stream=None) -> int:
    """Waits for the stream; raises DpoError on a device-detected error."""
    import torch
    with torch.cuda.device(workspace.device):
        st = lib().dpo_device_status(_ptr(workspace), _stream(stream, workspace))
    _check(st)
    return st


def dpo_strerror(status: int) -> str:
    return lib().dpo_strerror(int(status)).decode()


def dpo_profile_enable(on: bool) -> None:
    _check(lib().dpo_profile_enable(1 if on else 0))


def dpo_profile_select(name: str | None) -> None:
    """Time only the kernels called `name` while timing is on (None: all)."""
    _check(lib().dpo_profile_select(None if not name else name.encode()))


def dpo_profile_read() -> dict:
    """{kernel name: (total ms, launches)} of what was timed since enabling."""
    L = lib()
    out = {}
    for i in range(L.dpo_profile_count()):
        name = ctypes.c_char_p()
        ms = ctypes.c_double()
        n = ctypes.c_int()
        _check(L.dpo_profile_entry(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)))
        out[name.value.decode()] = (ms.value, n.value)
    return out
