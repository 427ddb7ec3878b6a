"""ctypes binding of libgdr.so (argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI declared in
include/gdr.h.  PyTorch supplies device memory and the current stream.  There
is no fallback: if the library is missing or the GPU is unavailable, calls
raise.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_ALIGNMENT, GDR_ERR_WORKSPACE, GDR_ERR_HIP = range(6)
GDR_F32, GDR_BF16 = 0, 1
GATES = {"none": 0, "scalar": 1, "channel": 2}
FORMS = {"page": 0, "literal": 1}

EXPORTED = ("gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd", "gdr_chunk_fwd_varlen_workspace_size",
            "gdr_chunk_fwd_varlen", "gdr_recurrent_step", "gdr_chunk_fwd_wkey", "gdr_recurrent_step_wkey",
            "gdr_precond_scan", "gdr_status_string", "gdr_last_error", "gdr_version",
            "gdr_chunk_bwd_workspace_size", "gdr_chunk_bwd", "gdr_chunk_bwd_wkey", "gdr_chunk_bwd_varlen_workspace_size",
            "gdr_chunk_bwd_varlen", "gdr_chunk_fwd_noalloc", "gdr_precond_scan_bwd_workspace_size",
            "gdr_precond_scan_bwd", "gdr_chunk_fwd_varlen_wkey", "gdr_chunk_bwd_varlen_wkey", "gdr_chunk_fwd_save",
            "gdr_chunk_bwd_saved")


class GdrDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("d_k", ctypes.c_int64), ("d_v", ctypes.c_int64), ("chunk", ctypes.c_int32),
                ("io", ctypes.c_int32), ("gate", ctypes.c_int32), ("form", ctypes.c_int32)]


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


_lock = threading.Lock()
_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libgdr.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m gated_delta_rule_21_amd.build`")
        lib = ctypes.CDLL(p)
        vp = ctypes.c_void_p
        lib.gdr_chunk_fwd_workspace_size.restype = ctypes.c_int
        lib.gdr_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(GdrDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.gdr_chunk_fwd.restype = ctypes.c_int
        lib.gdr_chunk_fwd.argtypes = [ctypes.POINTER(GdrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.gdr_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(GdrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdr_chunk_fwd_varlen_workspace_size.restype = ctypes.c_int
        lib.gdr_chunk_fwd_varlen_workspace_size.argtypes = [ctypes.POINTER(GdrDesc), ctypes.c_int64,
                                                            ctypes.POINTER(ctypes.c_size_t)]
        lib.gdr_chunk_fwd_varlen.restype = ctypes.c_int
        lib.gdr_chunk_fwd_varlen.argtypes = [ctypes.POINTER(GdrDesc), vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_fwd_wkey.restype = ctypes.c_int
        lib.gdr_chunk_fwd_wkey.argtypes = [ctypes.POINTER(GdrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_size_t, vp]
        lib.gdr_recurrent_step_wkey.restype = ctypes.c_int
        lib.gdr_recurrent_step_wkey.argtypes = [ctypes.POINTER(GdrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdr_recurrent_step.restype = ctypes.c_int
        lib.gdr_recurrent_step.argtypes = [ctypes.POINTER(GdrDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdr_precond_scan.restype = ctypes.c_int
        lib.gdr_precond_scan.argtypes = [ctypes.POINTER(GdrDesc), vp, vp, vp, ctypes.c_float, vp, vp, vp, vp]
        lib.gdr_precond_scan_bwd_workspace_size.restype = ctypes.c_int
        lib.gdr_precond_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(GdrDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.gdr_precond_scan_bwd.restype = ctypes.c_int
        lib.gdr_precond_scan_bwd.argtypes = ([ctypes.POINTER(GdrDesc), vp, vp, vp, ctypes.c_float] + [vp] * 7 +
                                             [vp, ctypes.c_size_t, vp])
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_chunk_bwd_workspace_size.restype = ctypes.c_int
        lib.gdr_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(GdrDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.gdr_chunk_bwd.restype = ctypes.c_int
        lib.gdr_chunk_bwd.argtypes = [ctypes.POINTER(GdrDesc)] + [vp] * 15 + [ctypes.c_size_t, vp]
        lib.gdr_chunk_bwd_wkey.restype = ctypes.c_int
        lib.gdr_chunk_bwd_wkey.argtypes = [ctypes.POINTER(GdrDesc)] + [vp] * 17 + [ctypes.c_size_t, vp]
        lib.gdr_chunk_bwd_varlen_wkey.restype = ctypes.c_int
        lib.gdr_chunk_bwd_varlen_wkey.argtypes = ([ctypes.POINTER(GdrDesc), vp, ctypes.c_int64] + [vp] * 17 +
                                                  [ctypes.c_size_t, vp])
        lib.gdr_chunk_fwd_varlen_wkey.restype = ctypes.c_int
        lib.gdr_chunk_fwd_varlen_wkey.argtypes = ([ctypes.POINTER(GdrDesc), vp, ctypes.c_int64] + [vp] * 10 +
                                                  [ctypes.c_size_t, vp])
        lib.gdr_chunk_bwd_varlen_workspace_size.restype = ctypes.c_int
        lib.gdr_chunk_bwd_varlen_workspace_size.argtypes = [ctypes.POINTER(GdrDesc), ctypes.c_int64,
                                                            ctypes.POINTER(ctypes.c_size_t)]
        lib.gdr_chunk_bwd_varlen.restype = ctypes.c_int
        lib.gdr_chunk_bwd_varlen.argtypes = ([ctypes.POINTER(GdrDesc), vp, ctypes.c_int64] + [vp] * 15 +
                                             [ctypes.c_size_t, vp])
        lib.gdr_chunk_fwd_save.restype = ctypes.c_int
        lib.gdr_chunk_fwd_save.argtypes = ([ctypes.POINTER(GdrDesc), vp, ctypes.c_int64] + [vp] * 10 +
                                           [ctypes.c_size_t, vp])
        lib.gdr_chunk_bwd_saved.restype = ctypes.c_int
        lib.gdr_chunk_bwd_saved.argtypes = ([ctypes.POINTER(GdrDesc), vp, ctypes.c_int64] + [vp] * 17 +
                                            [ctypes.c_size_t, vp])
        lib.gdr_status_string.argtypes = [ctypes.c_int]
        lib.gdr_last_error.restype = ctypes.c_char_p
        lib.gdr_last_error.argtypes = []
        lib.gdr_version.restype = ctypes.c_int
        lib.gdr_version.argtypes = []
        if path is None:
            _lib = lib
        return lib


def _check(lib, status: int) -> None:
    if status != GDR_OK:
        msg = lib.gdr_last_error().decode() or lib.gdr_status_string(status).decode()
        raise GdrError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _io_of(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"unsupported I/O dtype {t.dtype}; use bfloat16 or float32")


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gate_of(log_a, beta_shape, k_shape) -> int:
    if log_a is None:
        return GATES["none"]
    if tuple(log_a.shape) == tuple(beta_shape):
        return GATES["scalar"]
    if tuple(log_a.shape) == tuple(k_shape):
        return GATES["channel"]
    raise ValueError(f"log_a shape {tuple(log_a.shape)} fits neither {tuple(beta_shape)} nor {tuple(k_shape)}")


def _stream_handle(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def chunk_workspace_size(B: int, T: int, H: int, d_k: int, d_v: int, dtype=torch.bfloat16,
                         gate: str = "scalar") -> int:
    """Bytes of scratch gdr_chunk_fwd needs for these sizes (gdr_chunk_fwd_workspace_size)."""
    lib = load()
    io = 1 if dtype == torch.bfloat16 else 0
    desc = GdrDesc(B, T, H, d_k, d_v, 64, io, GATES[gate], 0)
    n = ctypes.c_size_t(0)
    _check(lib, lib.gdr_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def chunk_fwd(q, k, v, beta, log_a=None, S0=None, *, form: str = "page", o=None, S_T=None,
              want_state: bool = True, workspace=None, stream=None, kw=None):
    """gdr_chunk_fwd on torch tensors.  q, k [B, T, H, d_k]; v [B, T, H, d_v];
    beta [B, T, H]; log_a None, [B, T, H] or [B, T, H, d_k] (all one I/O dtype);
    S0 None or [B, H, d_k, d_v] float32.  `workspace` is an optional uint8 device
    tensor of at least chunk_workspace_size() bytes (allocated per call when
    None).  `kw` (optional, [B, T, H, d_k], bf16) is a separate write key
    (gdr_chunk_fwd_wkey).  Returns (o, S_T) (S_T None when want_state is False).
    Asynchronous on the current (or given) stream."""
    lib = load()
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dt = q.dtype
    _require(q, "q", dt, (B, T, H, dk))
    _require(k, "k", dt, (B, T, H, dk))
    _require(v, "v", dt, (B, T, H, dv))
    _require(beta, "beta", dt, (B, T, H))
    gate = _gate_of(log_a, beta.shape, k.shape)
    if log_a is not None:
        _require(log_a, "log_a", dt, tuple(log_a.shape))
    if S0 is not None:
        _require(S0, "S0", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    _require(o, "o", dt, (B, T, H, dv))
    if want_state and S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if S_T is not None:
        _require(S_T, "S_T", torch.float32, (B, H, dk, dv))
    desc = GdrDesc(B, T, H, dk, dv, 64, _io_of(q), gate, FORMS[form])
    need = ctypes.c_size_t(0)
    _check(lib, lib.gdr_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    if kw is not None:
        _require(kw, "kw", dt, (B, T, H, dk))
        st = lib.gdr_chunk_fwd_wkey(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(kw), _ptr(v), _ptr(beta), _ptr(log_a),
                                    _ptr(S0), _ptr(o), _ptr(S_T), _ptr(workspace), workspace.numel(),
                                    _stream_handle(stream))
        _check(lib, st)
        return o, S_T
    st = lib.gdr_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0),
                           _ptr(o), _ptr(S_T), _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _check(lib, st)
    return o, S_T


def chunk_fwd_noalloc(q, k, v, beta, log_a=None, S0=None, *, form: str = "page", o=None, S_T=None,
                      want_state: bool = True, stream=None):
    """gdr_chunk_fwd_noalloc on torch tensors: chunk_fwd with its scratch in the
    library's static device array (no workspace, no device allocation by the call
    beyond o and S_T when they are not given).  Calls that overlap in time on one
    GPU share that array and race.  Returns (o, S_T)."""
    lib = load()
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dt = q.dtype
    _require(q, "q", dt, (B, T, H, dk))
    _require(k, "k", dt, (B, T, H, dk))
    _require(v, "v", dt, (B, T, H, dv))
    _require(beta, "beta", dt, (B, T, H))
    gate = _gate_of(log_a, beta.shape, k.shape)
    if log_a is not None:
        _require(log_a, "log_a", dt, tuple(log_a.shape))
    if S0 is not None:
        _require(S0, "S0", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    _require(o, "o", dt, (B, T, H, dv))
    if want_state and S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if S_T is not None:
        _require(S_T, "S_T", torch.float32, (B, H, dk, dv))
    desc = GdrDesc(B, T, H, dk, dv, 64, _io_of(q), gate, FORMS[form])
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0),
                                   _ptr(o), _ptr(S_T), _stream_handle(stream))
    _check(lib, st)
    return o, S_T


def chunk_bwd_workspace_size(B: int, T: int, H: int, d_k: int, d_v: int, dtype=torch.bfloat16,
                             gate: str = "scalar") -> int:
    """Bytes of scratch gdr_chunk_bwd needs for these sizes (gdr_chunk_bwd_workspace_size)."""
    lib = load()
    io = 1 if dtype == torch.bfloat16 else 0
    desc = GdrDesc(B, T, H, d_k, d_v, 64, io, GATES[gate], 0)
    n = ctypes.c_size_t(0)
    _check(lib, lib.gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def chunk_fwd_save(q, k, v, beta, log_a=None, S0=None, *, cu_seqlens=None, form: str = "page", kw=None, o=None,
                   S_T=None, want_state: bool = True, workspace=None, stream=None):
    """gdr_chunk_fwd_save on torch tensors: the forward of a training step.  The
    arguments are those of chunk_fwd (with `cu_seqlens`: of chunk_fwd_varlen); bf16
    and the backward's configurations.  Returns (o, S_T, workspace): o and S_T as
    chunk_fwd's, and the workspace (uint8, the backward's size; given or allocated)
    holding the transform's records and the chunk-start states, for
    chunk_bwd(..., saved=workspace) over the same inputs."""
    lib = load()
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dt = q.dtype
    packed = cu_seqlens is not None
    if packed:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
                or cu_seqlens.device != q.device:
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on the inputs' device")
        if B != 1:
            raise ValueError("packed sequences take [1, T, H, d] tensors")
        nstate = cu_seqlens.numel() - 1
    else:
        nstate = B
    _require(q, "q", dt, (B, T, H, dk))
    _require(k, "k", dt, (B, T, H, dk))
    _require(v, "v", dt, (B, T, H, dv))
    _require(beta, "beta", dt, (B, T, H))
    gate = _gate_of(log_a, beta.shape, k.shape)
    if log_a is not None:
        _require(log_a, "log_a", dt, tuple(log_a.shape))
    if S0 is not None:
        _require(S0, "S0", torch.float32, (nstate, H, dk, dv))
    if kw is not None:
        _require(kw, "kw", dt, (B, T, H, dk))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    _require(o, "o", dt, (B, T, H, dv))
    if want_state and S_T is None:
        S_T = torch.empty((nstate, H, dk, dv), dtype=torch.float32, device=q.device)
    if S_T is not None:
        _require(S_T, "S_T", torch.float32, (nstate, H, dk, dv))
    desc = GdrDesc(B, T, H, dk, dv, 64, _io_of(q), gate, FORMS[form])
    need = ctypes.c_size_t(0)
    if packed:
        _check(lib, lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(desc), nstate, ctypes.byref(need)))
    else:
        _check(lib, lib.gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    st = lib.gdr_chunk_fwd_save(ctypes.byref(desc), _ptr(cu_seqlens), nstate if packed else 0, _ptr(q), _ptr(k),
                                _ptr(kw), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0), _ptr(o), _ptr(S_T),
                                _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _check(lib, st)
    return o, S_T, workspace


def chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T=None, *, cu_seqlens=None, form: str = "page", want_dS0: bool = True,
              workspace=None, stream=None, kw=None, saved=None):
    """gdr_chunk_bwd on torch tensors: the gradients of L = <dO, o> + <dS_T, S_T> for
    the forward chunk_fwd(q, k, v, beta, log_a, S0, form=form) (bf16 I/O; no gate, a
    scalar gate, or a per-channel gate with d_k = 128).  dO [B, T, H, d_v] bf16; dS_T None or
    [B, H, d_k, d_v] float32.  With `cu_seqlens` (int32 device tensor [n_seq + 1])
    the sequences are packed along T of [1, T, H, .] tensors (gdr_chunk_bwd_varlen)
    and S0, dS_T, dS0 are [n_seq, H, d_k, d_v].  Returns dict(dq, dk, dv, dbeta,
    dlog_a, dS0) (dlog_a None without a gate, dS0 None when want_dS0 is False).
    `kw` ([B, T, H, d_k] bf16, no gate or a scalar gate) is the forward's write key
    (gdr_chunk_bwd_wkey, gdr_chunk_bwd_varlen_wkey): then dk is the read side's
    gradient and the dict also holds dkw.  `saved` is the workspace returned by
    chunk_fwd_save over the same inputs (gdr_chunk_bwd_saved: the transform and the
    chunk-start states are taken from it, and S0 is not read); it is overwritten.
    Asynchronous on the current (or given) stream."""
    lib = load()
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    packed = cu_seqlens is not None
    if packed:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
                or cu_seqlens.device != q.device:
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on the inputs' device")
        if B != 1:
            raise ValueError("packed sequences take [1, T, H, d] tensors")
        nstate = cu_seqlens.numel() - 1
    else:
        nstate = B
    dt = q.dtype
    _require(q, "q", dt, (B, T, H, dk))
    _require(k, "k", dt, (B, T, H, dk))
    _require(v, "v", dt, (B, T, H, dv))
    _require(beta, "beta", dt, (B, T, H))
    _require(dO, "dO", dt, (B, T, H, dv))
    gate = _gate_of(log_a, beta.shape, k.shape)
    if log_a is not None:
        _require(log_a, "log_a", dt, tuple(log_a.shape))
    if S0 is not None:
        _require(S0, "S0", torch.float32, (nstate, H, dk, dv))
    if dS_T is not None:
        _require(dS_T, "dS_T", torch.float32, (nstate, H, dk, dv))
    if kw is not None:
        _require(kw, "kw", dt, (B, T, H, dk))
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dbeta=torch.empty_like(beta),
               dlog_a=torch.empty_like(log_a) if log_a is not None else None,
               dS0=torch.empty((nstate, H, dk, dv), dtype=torch.float32, device=q.device) if want_dS0 else None)
    desc = GdrDesc(B, T, H, dk, dv, 64, _io_of(q), gate, FORMS[form])
    need = ctypes.c_size_t(0)
    if packed:
        _check(lib, lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(desc), nstate, ctypes.byref(need)))
    else:
        _check(lib, lib.gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)))
    if saved is not None:
        workspace = saved
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    if saved is not None:
        if kw is not None:
            out["dkw"] = torch.empty_like(k)
        st = lib.gdr_chunk_bwd_saved(ctypes.byref(desc), _ptr(cu_seqlens), nstate if packed else 0, _ptr(q), _ptr(k),
                                     _ptr(kw), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0), _ptr(dO), _ptr(dS_T),
                                     _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out.get("dkw")), _ptr(out["dv"]),
                                     _ptr(out["dbeta"]), _ptr(out["dlog_a"]), _ptr(out["dS0"]), _ptr(workspace),
                                     workspace.numel(), _stream_handle(stream))
        _check(lib, st)
        return out
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(out["dq"]),
            _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dlog_a"]), _ptr(out["dS0"]),
            _ptr(workspace), workspace.numel(), _stream_handle(stream))
    if kw is not None:
        out["dkw"] = torch.empty_like(k)
        wargs = (_ptr(q), _ptr(k), _ptr(kw), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0), _ptr(dO), _ptr(dS_T),
                 _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dkw"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
                 _ptr(out["dlog_a"]), _ptr(out["dS0"]), _ptr(workspace), workspace.numel(), _stream_handle(stream))
        if packed:
            st = lib.gdr_chunk_bwd_varlen_wkey(ctypes.byref(desc), _ptr(cu_seqlens), nstate, *wargs)
        else:
            st = lib.gdr_chunk_bwd_wkey(ctypes.byref(desc), *wargs)
    elif packed:
        st = lib.gdr_chunk_bwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), nstate, *args)
    else:
        st = lib.gdr_chunk_bwd(ctypes.byref(desc), *args)
    _check(lib, st)
    return out


def chunk_varlen_workspace_size(T: int, n_seq: int, H: int, d_k: int, d_v: int, dtype=torch.bfloat16,
                                gate: str = "scalar") -> int:
    """Bytes of scratch gdr_chunk_fwd_varlen needs (gdr_chunk_fwd_varlen_workspace_size)."""
    lib = load()
    desc = GdrDesc(1, T, H, d_k, d_v, 64, 1 if dtype == torch.bfloat16 else 0, GATES[gate], 0)
    n = ctypes.c_size_t(0)
    _check(lib, lib.gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(desc), int(n_seq), ctypes.byref(n)))
    return int(n.value)


def chunk_fwd_varlen(q, k, v, beta, log_a, cu_seqlens, S0=None, *, form: str = "page", o=None, S_T=None,
                     want_state: bool = True, workspace=None, stream=None, kw=None):
    """gdr_chunk_fwd_varlen on torch tensors: sequences packed along T.
    q, k [1, T, H, d_k]; v [1, T, H, d_v]; beta [1, T, H]; log_a None, [1, T, H] or
    [1, T, H, d_k] (bf16); cu_seqlens int32 device tensor [N + 1] of offsets;
    S0 None or [N, H, d_k, d_v] float32.  `kw` (optional, [1, T, H, d_k]) is a separate
    write key (gdr_chunk_fwd_varlen_wkey).  Returns (o [1, T, H, d_v], S_T [N, H, d_k, d_v])."""
    lib = load()
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dt = q.dtype
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
            or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on the inputs' device")
    N = cu_seqlens.numel() - 1
    _require(q, "q", dt, (1, T, H, dk))
    _require(k, "k", dt, (1, T, H, dk))
    _require(v, "v", dt, (1, T, H, dv))
    _require(beta, "beta", dt, (1, T, H))
    gate = _gate_of(log_a, beta.shape, k.shape)
    if log_a is not None:
        _require(log_a, "log_a", dt, tuple(log_a.shape))
    if S0 is not None:
        _require(S0, "S0", torch.float32, (N, H, dk, dv))
    if o is None:
        o = torch.empty((1, T, H, dv), dtype=dt, device=q.device)
    _require(o, "o", dt, (1, T, H, dv))
    if want_state and S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if S_T is not None:
        _require(S_T, "S_T", torch.float32, (N, H, dk, dv))
    desc = GdrDesc(1, T, H, dk, dv, 64, _io_of(q), gate, FORMS[form])
    need = ctypes.c_size_t(0)
    _check(lib, lib.gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(desc), N, ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    if kw is not None:
        _require(kw, "kw", dt, (1, T, H, dk))
        st = lib.gdr_chunk_fwd_varlen_wkey(ctypes.byref(desc), _ptr(cu_seqlens), N, _ptr(q), _ptr(k), _ptr(kw),
                                           _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0), _ptr(o), _ptr(S_T),
                                           _ptr(workspace), workspace.numel(), _stream_handle(stream))
    else:
        st = lib.gdr_chunk_fwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), N, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                      _ptr(log_a), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(workspace), workspace.numel(),
                                      _stream_handle(stream))
    _check(lib, st)
    return o, S_T


def recurrent_step(q, k, v, beta, log_a, S, *, S_new=None, o=None, form: str = "page", stream=None, kw=None):
    """gdr_recurrent_step on torch tensors.  q, k [B, H, d_k]; v [B, H, d_v];
    beta [B, H]; log_a None, [B, H] or [B, H, d_k]; S [B, H, d_k, d_v] float32.
    S_new defaults to S (update in place).  `kw` (optional, [B, H, d_k]) is a
    separate write key (gdr_recurrent_step_wkey).  Returns (o, S_new)."""
    lib = load()
    B, H, dk = k.shape
    dv = v.shape[-1]
    dt = q.dtype
    _require(q, "q", dt, (B, H, dk))
    _require(k, "k", dt, (B, H, dk))
    _require(v, "v", dt, (B, H, dv))
    _require(beta, "beta", dt, (B, H))
    gate = _gate_of(log_a, beta.shape, k.shape)
    if log_a is not None:
        _require(log_a, "log_a", dt, tuple(log_a.shape))
    _require(S, "S", torch.float32, (B, H, dk, dv))
    if S_new is None:
        S_new = S
    _require(S_new, "S_new", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=q.device)
    _require(o, "o", dt, (B, H, dv))
    desc = GdrDesc(B, 1, H, dk, dv, 0, _io_of(q), gate, FORMS[form])
    if kw is not None:
        _require(kw, "kw", dt, (B, H, dk))
        st = lib.gdr_recurrent_step_wkey(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(kw), _ptr(v), _ptr(beta),
                                         _ptr(log_a), _ptr(S), _ptr(S_new), _ptr(o), _stream_handle(stream))
        _check(lib, st)
        return o, S_new
    st = lib.gdr_recurrent_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S),
                                _ptr(S_new), _ptr(o), _stream_handle(stream))
    _check(lib, st)
    return o, S_new


def precond_scan(k, beta, eta: float, r=None, d0=None, *, kw=None, d_T=None, want_state: bool = True,
                 stream=None):
    """gdr_precond_scan on torch tensors: the preconditioner scan that produces
    the write keys kw_t = d_t * k_t.  k [B, T, H, d_k]; beta [B, T, H]; r None
    (no forgetting) or [B, T, H] retention (same I/O dtype); eta step size;
    d0 None (ones) or [B, H, d_k] float32.  Returns (kw [B, T, H, d_k] in the
    I/O dtype, d_T [B, H, d_k] float32, None when want_state is False).
    d_T may be d0 (updated in place)."""
    lib = load()
    B, T, H, dk = k.shape
    dt = k.dtype
    _require(k, "k", dt, (B, T, H, dk))
    _require(beta, "beta", dt, (B, T, H))
    if r is not None:
        _require(r, "r", dt, (B, T, H))
    if d0 is not None:
        _require(d0, "d0", torch.float32, (B, H, dk))
    if kw is None:
        kw = torch.empty((B, T, H, dk), dtype=dt, device=k.device)
    _require(kw, "kw", dt, (B, T, H, dk))
    if want_state and d_T is None:
        d_T = torch.empty((B, H, dk), dtype=torch.float32, device=k.device)
    if d_T is not None:
        _require(d_T, "d_T", torch.float32, (B, H, dk))
    desc = GdrDesc(B, T, H, dk, dk, 64, _io_of(k), 0, 0)
    st = lib.gdr_precond_scan(ctypes.byref(desc), _ptr(k), _ptr(beta), _ptr(r), float(eta), _ptr(d0), _ptr(kw),
                              _ptr(d_T), _stream_handle(stream))
    _check(lib, st)
    return kw, d_T


def precond_scan_bwd_workspace_size(B: int, T: int, H: int, d_k: int) -> int:
    """Bytes of scratch gdr_precond_scan_bwd needs (gdr_precond_scan_bwd_workspace_size)."""
    lib = load()
    desc = GdrDesc(B, T, H, d_k, d_k, 64, 1, 0, 0)
    n = ctypes.c_size_t(0)
    _check(lib, lib.gdr_precond_scan_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def precond_scan_bwd(k, beta, eta: float, r=None, d0=None, dkw=None, dd_T=None, *, want_dd0: bool = True,
                     workspace=None, stream=None):
    """gdr_precond_scan_bwd on torch tensors: the gradients of <dkw, kw> + <dd_T, d_T>
    for the scan precond_scan(k, beta, eta, r, d0).  dkw None (zero) or
    [B, T, H, d_k] in the I/O dtype; dd_T None (zero) or [B, H, d_k] float32.
    Returns dict(dk, dbeta, dr, dd0) (dr None without r, dd0 None when want_dd0 is
    False).  Asynchronous on the current (or given) stream."""
    lib = load()
    B, T, H, dk = k.shape
    dt = k.dtype
    _require(k, "k", dt, (B, T, H, dk))
    _require(beta, "beta", dt, (B, T, H))
    if r is not None:
        _require(r, "r", dt, (B, T, H))
    if d0 is not None:
        _require(d0, "d0", torch.float32, (B, H, dk))
    if dkw is not None:
        _require(dkw, "dkw", dt, (B, T, H, dk))
    if dd_T is not None:
        _require(dd_T, "dd_T", torch.float32, (B, H, dk))
    desc = GdrDesc(B, T, H, dk, dk, 64, _io_of(k), 0, 0)
    need = ctypes.c_size_t(0)
    _check(lib, lib.gdr_precond_scan_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=k.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != k.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    out = dict(dk=torch.empty_like(k), dbeta=torch.empty_like(beta),
               dr=torch.empty_like(r) if r is not None else None,
               dd0=torch.empty((B, H, dk), dtype=torch.float32, device=k.device) if want_dd0 else None)
    st = lib.gdr_precond_scan_bwd(ctypes.byref(desc), _ptr(k), _ptr(beta), _ptr(r), float(eta), _ptr(d0), _ptr(dkw),
                                  _ptr(dd_T), _ptr(out["dk"]), _ptr(out["dbeta"]), _ptr(out["dr"]), _ptr(out["dd0"]),
                                  _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _check(lib, st)
    return out


class _PrecondScan(torch.autograd.Function):
    """precond_scan with precond_scan_bwd as its backward (marshalling only)."""

    @staticmethod
    def forward(ctx, k, beta, eta, r, d0):
        kw, d_T = precond_scan(k, beta, eta, r, d0)
        ctx.save_for_backward(k, beta, r, d0)
        ctx.eta = eta
        return kw, d_T

    @staticmethod
    def backward(ctx, dkw, dd_T):
        k, beta, r, d0 = ctx.saved_tensors
        dkw = None if dkw is None else dkw.to(k.dtype).contiguous()
        dd_T = None if dd_T is None else dd_T.float().contiguous()
        g = precond_scan_bwd(k, beta, ctx.eta, r, d0, dkw, dd_T, want_dd0=d0 is not None)
        return g["dk"], g["dbeta"], None, g["dr"], g["dd0"]


def precond_attn(k, beta, eta: float, r=None, d0=None):
    """(kw, d_T) of precond_scan as a torch autograd function whose backward is
    precond_scan_bwd: gradients flow to k, beta, r and d0.  Composed with
    chunk_attn(..., kw=kw) it gives the gradients of both phases of the
    preconditioned delta rule."""
    return _PrecondScan.apply(k, beta, float(eta), r, d0)


class _ChunkAttn(torch.autograd.Function):
    """chunk_fwd with chunk_bwd as its backward (marshalling only)."""

    @staticmethod
    def forward(ctx, q, k, v, beta, log_a, S0, cu_seqlens, form, kw):
        # the training forward: its workspace keeps the transform and the chunk-start
        # states for the backward, which then only runs the reverse pass and the
        # per-chunk gradients
        if any(ctx.needs_input_grad):
            o, S_T, ctx.ws = chunk_fwd_save(q, k, v, beta, log_a, S0, cu_seqlens=cu_seqlens, form=form, kw=kw)
        elif cu_seqlens is not None:
            o, S_T = chunk_fwd_varlen(q, k, v, beta, log_a, cu_seqlens, S0, form=form, kw=kw)
        else:
            o, S_T = chunk_fwd(q, k, v, beta, log_a, S0, form=form, kw=kw)
        ctx.save_for_backward(q, k, v, beta, log_a, S0, cu_seqlens, kw)
        ctx.form = form
        ctx.gated = log_a is not None
        ctx.has_S0 = S0 is not None
        return o, S_T

    @staticmethod
    def backward(ctx, dO, dS_T):
        q, k, v, beta, log_a, S0, cu_seqlens, kw = ctx.saved_tensors
        dO = torch.zeros_like(v) if dO is None else dO.to(v.dtype).contiguous()
        dS_T = None if dS_T is None else dS_T.float().contiguous()
        # the backward leaves the records and the states in place, so the graph may be
        # walked more than once (retain_graph)
        g = chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, cu_seqlens=cu_seqlens, form=ctx.form, want_dS0=ctx.has_S0,
                      kw=kw, saved=ctx.ws)
        return (g["dq"], g["dk"], g["dv"], g["dbeta"], g["dlog_a"] if ctx.gated else None,
                g["dS0"] if ctx.has_S0 else None, None, None, g.get("dkw"))


def chunk_attn(q, k, v, beta, log_a=None, S0=None, cu_seqlens=None, form: str = "page", kw=None):
    """(o, S_T) of chunk_fwd (or chunk_fwd_varlen with cu_seqlens) as a torch autograd
    function whose backward is chunk_bwd: bf16, any gate (per-channel with d_k = 128),
    either form.  The forward is chunk_fwd_save and the backward takes what it kept
    (the backward's workspace stays allocated between the two).  Gradients flow to q, k, v, beta, log_a and S0, and to the write key
    `kw` when one is given (no gate or a scalar gate)."""
    if kw is not None and log_a is not None and log_a.dim() == 4:
        raise ValueError("chunk_attn with a write key: no gate or a scalar gate (the backward's scope)")
    return _ChunkAttn.apply(q, k, v, beta, log_a, S0, cu_seqlens, form, kw)
