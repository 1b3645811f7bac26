"""ctypes binding over libkda.so (the C ABI declared in include/kda.h).

Argument marshalling only: torch supplies device memory and the stream; every
step of the computation runs in the library's HIP kernels. Importing this
module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_EINVAL, KDA_ENOTSUP, KDA_EALIGN, KDA_EHIP = 0, -1, -2, -3, -4
KDA_F32, KDA_BF16 = 0, 1
GATE_CHANNEL, GATE_SCALAR = 0, 1

STAGE_PREP, STAGE_STATE, STAGE_ALL = 1, 2, 3

EXPORTS = ("kda_chunk_fwd", "kda_chunk_fwd_stage", "kda_chunk_fwd_workspace_bytes", "kda_chunk_bwd",
           "kda_chunk_bwd_workspace_bytes", "kda_gauge_fold", "kda_gauge_fold_workspace_bytes", "kda_chunk_fwd_gauge",
           "kda_chunk_fwd_gauge_workspace_bytes", "kda_decode_step", "kda_strerror", "kda_last_hip_error",
           "kda_version")


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s failed: %s (%d)" % (where, strerror(status), status)
        if status == KDA_EHIP:
            msg += ", hipError %d" % _lib().kda_last_hip_error()
        super().__init__(msg)


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkda.so is not built (%s); run python -m gated_delta_rule_46_amd.build"
                              % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.kda_chunk_fwd.restype = i
        lib.kda_chunk_fwd.argtypes = [vp] * 8 + [i] * 6 + [vp, i, i, i, vp, sz, vp]
        lib.kda_chunk_fwd_stage.restype = i
        lib.kda_chunk_fwd_stage.argtypes = [i] + [vp] * 8 + [i] * 6 + [vp, i, i, i, vp, sz, vp]
        lib.kda_chunk_fwd_workspace_bytes.restype = sz
        lib.kda_chunk_fwd_workspace_bytes.argtypes = [i] * 9
        lib.kda_chunk_bwd.restype = i
        lib.kda_chunk_bwd.argtypes = [vp] * 14 + [i] * 5 + [vp, i, i, i, vp, sz, vp]
        lib.kda_chunk_bwd_workspace_bytes.restype = sz
        lib.kda_chunk_bwd_workspace_bytes.argtypes = [i] * 7
        lib.kda_gauge_fold.restype = i
        lib.kda_gauge_fold.argtypes = [vp] * 7 + [i] * 4 + [vp, i, i, i, vp, sz, vp]
        lib.kda_gauge_fold_workspace_bytes.restype = sz
        lib.kda_gauge_fold_workspace_bytes.argtypes = [i] * 7
        lib.kda_chunk_fwd_gauge.restype = i
        lib.kda_chunk_fwd_gauge.argtypes = [vp] * 8 + [i] * 6 + [vp, i, i, i, vp, sz, vp]
        lib.kda_chunk_fwd_gauge_workspace_bytes.restype = sz
        lib.kda_chunk_fwd_gauge_workspace_bytes.argtypes = [i] * 10
        lib.kda_decode_step.restype = i
        lib.kda_decode_step.argtypes = [vp] * 7 + [i] * 6 + [vp]
        lib.kda_strerror.restype = ctypes.c_char_p
        lib.kda_strerror.argtypes = [i]
        lib.kda_last_hip_error.restype = i
        lib.kda_last_hip_error.argtypes = []
        lib.kda_version.restype = i
        lib.kda_version.argtypes = []
        _L = lib
    return _L


def library():
    """The loaded ctypes library (raises ImportError if not built)."""
    return _lib()


def strerror(status: int) -> str:
    return _lib().kda_strerror(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("inputs must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check_dev(name: str, t: torch.Tensor, device):
    if not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int, N: int = 0,
                    varlen: bool = False, dtype: torch.dtype = torch.bfloat16) -> int:
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(_lib().kda_chunk_fwd_workspace_bytes(B, H, T, dk, dv, chunk, N, int(varlen), code))


def chunk_fwd(q, k, v, gate, beta, S0=None, cu_seqlens=None, chunk: int = 64, gate_kind: Optional[int] = None,
              out: Optional[torch.Tensor] = None, state_out: bool = True, S_T: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None,
              stage: int = STAGE_ALL) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise forward. q, k [B,T,H,dk]; v [B,T,H,dv]; gate [B,T,H,dk] or
    [B,T,H]; beta [B,T,H]; S0 [N,H,dk,dv] fp32 or None; cu_seqlens int32 [N+1]
    on the device (B must be 1) or None. Returns (o fp32 [B,T,H,dv], S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        _check_dev(name, t, device)
    if gate_kind is None:
        gate_kind = GATE_SCALAR if gate.dim() == 3 else GATE_CHANNEL
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    varlen = cu_seqlens is not None
    N = int(cu_seqlens.numel() - 1) if varlen else B
    if varlen:
        _check_dev("cu_seqlens", cu_seqlens, device)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
    if S0 is not None:
        _check_dev("S0", S0, device)
        if S0.dtype != torch.float32 or tuple(S0.shape) != (N, H, dk, dv):
            raise ValueError("S0 must be fp32 [%d,%d,%d,%d]" % (N, H, dk, dv))
    if out is None:
        out = torch.empty((B, T, H, dv), device=device, dtype=torch.float32)
    if S_T is None and state_out:
        S_T = torch.empty((N, H, dk, dv), device=device, dtype=torch.float32)
    need = workspace_bytes(B, H, T, dk, dv, chunk, N, varlen, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    st = _stream_handle(stream, device)
    rc = _lib().kda_chunk_fwd_stage(int(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0), _ptr(out),
                              _ptr(S_T), B, H, T, dk, dv, chunk, _ptr(cu_seqlens), N if varlen else 0, dt,
                              int(gate_kind), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_stage")
    return out, S_T


def bwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, N: int = 0, varlen: bool = False) -> int:
    return int(_lib().kda_chunk_bwd_workspace_bytes(B, H, T, dk, dv, N, int(varlen)))


def chunk_bwd(q, k, v, gate, beta, dO, S0=None, dS_T=None, cu_seqlens=None, gate_kind: Optional[int] = None,
              want_dS0: bool = True, out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
              stream=None) -> dict:
    """Gradient of chunk_fwd for L = sum(o * dO) + sum(S_T * dS_T). Inputs as
    for chunk_fwd; dO fp32 [B,T,H,dv]; dS_T fp32 [N,H,dk,dv] or None. Returns
    a dict of fp32 tensors dq, dk, dv, dgate, dbeta (input layouts) and dS0
    ([N,H,dk,dv], or None when not wanted). ``out`` may supply that dict's
    tensors to write into."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta), ("dO", dO)):
        _check_dev(name, t, device)
    if gate_kind is None:
        gate_kind = GATE_SCALAR if gate.dim() == 3 else GATE_CHANNEL
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    if dO.dtype != torch.float32 or tuple(dO.shape) != (B, T, H, dv):
        raise ValueError("dO must be fp32 [%d,%d,%d,%d]" % (B, T, H, dv))
    varlen = cu_seqlens is not None
    N = int(cu_seqlens.numel() - 1) if varlen else B
    if varlen:
        _check_dev("cu_seqlens", cu_seqlens, device)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _check_dev(name, t, device)
            if t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv):
                raise ValueError("%s must be fp32 [%d,%d,%d,%d]" % (name, N, H, dk, dv))
    f32 = dict(device=device, dtype=torch.float32)
    if out is None:
        out = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
               "dv": torch.empty((B, T, H, dv), **f32), "dgate": torch.empty(tuple(gate.shape), **f32),
               "dbeta": torch.empty((B, T, H), **f32),
               "dS0": torch.empty((N, H, dk, dv), **f32) if want_dS0 else None}
    need = bwd_workspace_bytes(B, H, T, dk, dv, N, varlen)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    st = _stream_handle(stream, device)
    rc = _lib().kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_T),
                              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dgate"]),
                              _ptr(out["dbeta"]), _ptr(out.get("dS0")), B, H, T, dk, dv, _ptr(cu_seqlens),
                              N if varlen else 0, dt, int(gate_kind), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_bwd")
    return out


def gauge_fold(q, k, gate, cu_seqlens=None, gate_kind: Optional[int] = None, stream=None):
    """Gauge fold: returns (q~, k~, gate~, c_T) with c_T int8 [N,H,dk] or
    [N,H]. Inputs as for chunk_fwd."""
    B, T, H, dk = q.shape
    device = q.device
    for name, t in (("q", q), ("k", k), ("gate", gate)):
        _check_dev(name, t, device)
    if gate_kind is None:
        gate_kind = GATE_SCALAR if gate.dim() == 3 else GATE_CHANNEL
    dt = _dtype_code(q)
    varlen = cu_seqlens is not None
    N = int(cu_seqlens.numel() - 1) if varlen else B
    qo, ko, go = torch.empty_like(q), torch.empty_like(k), torch.empty_like(gate)
    sign = torch.empty((N, H, dk) if gate_kind == GATE_CHANNEL else (N, H), device=device, dtype=torch.int8)
    need = int(_lib().kda_gauge_fold_workspace_bytes(B, H, T, dk, N, int(varlen), int(gate_kind)))
    ws = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    st = _stream_handle(stream, device)
    rc = _lib().kda_gauge_fold(_ptr(q), _ptr(k), _ptr(gate), _ptr(qo), _ptr(ko), _ptr(go), _ptr(sign), B, H, T, dk,
                               _ptr(cu_seqlens), N if varlen else 0, dt, int(gate_kind), _ptr(ws), need,
                               ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_gauge_fold")
    return qo, ko, go, sign


def fwd_gauge_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int, N: int = 0, varlen: bool = False,
                              dtype: torch.dtype = torch.bfloat16, gate_kind: int = GATE_CHANNEL) -> int:
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(_lib().kda_chunk_fwd_gauge_workspace_bytes(B, H, T, dk, dv, chunk, N if varlen else B, int(varlen), code,
                                                          int(gate_kind)))


def chunk_fwd_gauge(q, k, v, gate, beta, S0=None, cu_seqlens=None, chunk: int = 64, gate_kind: Optional[int] = None,
                    out: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """chunk_fwd through the gauge transform (kda_chunk_fwd_gauge). Same
    arguments and results as chunk_fwd."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        _check_dev(name, t, device)
    if gate_kind is None:
        gate_kind = GATE_SCALAR if gate.dim() == 3 else GATE_CHANNEL
    dt = _dtype_code(q)
    varlen = cu_seqlens is not None
    N = int(cu_seqlens.numel() - 1) if varlen else B
    if out is None:
        out = torch.empty((B, T, H, dv), device=device, dtype=torch.float32)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), device=device, dtype=torch.float32)
    need = fwd_gauge_workspace_bytes(B, H, T, dk, dv, chunk, N, varlen, q.dtype, gate_kind)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    st = _stream_handle(stream, device)
    rc = _lib().kda_chunk_fwd_gauge(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_T),
                                    B, H, T, dk, dv, chunk, _ptr(cu_seqlens), N if varlen else 0, dt, int(gate_kind),
                                    _ptr(workspace), workspace.numel(), ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_gauge")
    return out, S_T


def decode_step(q, k, v, gate, beta, S, out: Optional[torch.Tensor] = None, gate_kind: Optional[int] = None,
                stream=None) -> torch.Tensor:
    """One decode step, S [N,H,dk,dv] fp32 updated in place. q, k [N,H,dk];
    v [N,H,dv]; gate [N,H,dk] or [N,H]; beta [N,H]. Returns o fp32 [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta), ("S", S)):
        _check_dev(name, t, device)
    if S.dtype != torch.float32 or tuple(S.shape) != (N, H, dk, dv):
        raise ValueError("S must be fp32 [%d,%d,%d,%d]" % (N, H, dk, dv))
    if gate_kind is None:
        gate_kind = GATE_SCALAR if gate.dim() == 2 else GATE_CHANNEL
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((N, H, dv), device=device, dtype=torch.float32)
    st = _stream_handle(stream, device)
    rc = _lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S), _ptr(out),
                                N, H, dk, dv, dt, int(gate_kind), ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_decode_step")
    return out
