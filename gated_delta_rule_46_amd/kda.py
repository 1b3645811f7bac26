"""ctypes binding over libkda.so (the C ABI declared in include/kda.h).

Argument marshalling only: torch supplies device memory and the stream; every
step of the computation runs in the library's HIP kernels. Importing this
module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import contextlib
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIB names another build of the same library (the sanitizer build of the
# host-side validation code loads that way); default: the in-tree libkda.so.
LIB_PATH = os.environ.get("KDA_LIB") or os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_EINVAL, KDA_ENOTSUP, KDA_EALIGN, KDA_EHIP, KDA_EWAIT, KDA_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 128 << 20
KDA_F32, KDA_BF16 = 0, 1
GATE_CHANNEL, GATE_SCALAR = 0, 1

STAGE_PREP, STAGE_STATE, STAGE_ALL = 1, 2, 3

EXPORTS = ("kda_chunk_fwd", "kda_chunk_fwd_stage", "kda_chunk_fwd_workspace_bytes", "kda_chunk_bwd",
           "kda_chunk_bwd_workspace_bytes", "kda_gauge_fold", "kda_gauge_fold_workspace_bytes", "kda_chunk_fwd_gauge",
           "kda_chunk_fwd_gauge_workspace_bytes", "kda_decode_step", "kda_strerror", "kda_last_hip_error",
           "kda_version", "kda_chunk_fwd_status", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_ew",
           "kda_decode_step_ew", "kda_chunk_bwd_cw", "kda_chunk_bwd_cw_workspace_bytes", "kda_chunk_bwd_ew",
           "kda_chunk_bwd_ew_workspace_bytes")


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s failed: %s (%d)" % (where, strerror(status), status)
        if status == KDA_EHIP:
            msg += ", hipError %d" % _lib().kda_last_hip_error()
        super().__init__(msg)


_L = None


def load(path: str):
    """A ctypes handle on the build of the library at `path`, with the
    argument and result types of every export set."""
    if not os.path.exists(path):
        raise ImportError("%s is not built; run python -m gated_delta_rule_46_amd.build" % path)
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_chunk_fwd.restype = i
    lib.kda_chunk_fwd.argtypes = [vp] * 8 + [i] * 6 + [vp, i, i, i, vp, sz, vp]
    lib.kda_chunk_fwd_stage.restype = i
    lib.kda_chunk_fwd_stage.argtypes = [i] + [vp] * 8 + [i] * 6 + [vp, i, i, i, vp, sz, vp]
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i] * 9
    lib.kda_chunk_bwd.restype = i
    lib.kda_chunk_bwd.argtypes = [vp] * 14 + [i] * 5 + [vp, i, i, i, vp, sz, vp]
    lib.kda_chunk_bwd_cw.restype = i
    lib.kda_chunk_bwd_cw.argtypes = [vp] * 14 + [i] * 5 + [vp, i, i, i, vp, sz, vp]
    lib.kda_chunk_bwd_cw_workspace_bytes.restype = sz
    lib.kda_chunk_bwd_cw_workspace_bytes.argtypes = [i] * 7
    lib.kda_chunk_bwd_ew.restype = i
    lib.kda_chunk_bwd_ew.argtypes = [vp] * 16 + [i] * 5 + [vp, i, i, i, vp, sz, vp]
    lib.kda_chunk_bwd_ew_workspace_bytes.restype = sz
    lib.kda_chunk_bwd_ew_workspace_bytes.argtypes = [i] * 7
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
    lib.kda_chunk_fwd_status.restype = i
    lib.kda_chunk_fwd_status.argtypes = [ctypes.c_uint32]
    lib.kda_chunk_fwd_ew.restype = i
    lib.kda_chunk_fwd_ew.argtypes = [vp] * 9 + [i] * 6 + [vp, i, i, i, vp, sz, vp]
    lib.kda_decode_step_ew.restype = i
    lib.kda_decode_step_ew.argtypes = [vp] * 8 + [i] * 6 + [vp]
    lib.kda_chunk_fwd_noalloc.restype = i
    lib.kda_chunk_fwd_noalloc.argtypes = [vp] * 8 + [i] * 6 + [vp, i, i, i, vp]
    return lib


def _lib():
    global _L
    if _L is None:
        _L = load(LIB_PATH)
    return _L


@contextlib.contextmanager
def using_library(path: str):
    """Route this module's calls through another build of the library (for
    instance the LDS-poisoning debug build) inside a with-block."""
    global _L
    prev = _lib()
    _L = load(path)
    try:
        yield _L
    finally:
        _L = prev


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


def _check_shape(name: str, t: torch.Tensor, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _gate_kind(gate: torch.Tensor, lead: int, gate_kind: Optional[int]) -> int:
    """Gate kind from the gate's rank (lead = number of leading dims before
    dk), checked against an explicit gate_kind."""
    by_rank = {lead + 1: GATE_CHANNEL, lead: GATE_SCALAR}
    if gate.dim() not in by_rank:
        raise ValueError("gate has %d dims, expected %d (channel) or %d (scalar)" % (gate.dim(), lead + 1, lead))
    kind = by_rank[gate.dim()]
    if gate_kind is not None and int(gate_kind) != kind:
        raise ValueError("gate of rank %d does not match gate_kind %d" % (gate.dim(), gate_kind))
    return kind


def _check_seq_inputs(q, k, v, gate, beta, gate_kind):
    """Shapes of a whole-sequence call: q, k [B,T,H,dk], v [B,T,H,dv], gate
    [B,T,H,dk] or [B,T,H], beta [B,T,H]; one dtype. Returns (B, T, H, dk, dv,
    gate_kind)."""
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk], got %s" % (tuple(q.shape),))
    B, T, H, dk = q.shape
    if v.dim() != 4:
        raise ValueError("v must be [B,T,H,dv], got %s" % (tuple(v.shape),))
    dv = v.shape[-1]
    _check_shape("k", k, (B, T, H, dk))
    _check_shape("v", v, (B, T, H, dv))
    gate_kind = _gate_kind(gate, 3, gate_kind)
    _check_shape("gate", gate, (B, T, H, dk) if gate_kind == GATE_CHANNEL else (B, T, H))
    _check_shape("beta", beta, (B, T, H))
    for name, t in (("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    return B, T, H, dk, dv, gate_kind


def _check_varlen(cu_seqlens, B, device):
    if cu_seqlens is None:
        return False, B
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise TypeError("cu_seqlens must be a 1-D int32 tensor of N+1 offsets")
    if B != 1:
        raise ValueError("packed sequences (cu_seqlens) need B = 1, got %d" % B)
    _check_dev("cu_seqlens", cu_seqlens, device)
    return True, int(cu_seqlens.numel() - 1)


def _check_state(name, t, N, H, dk, dv, device):
    if t is None:
        return
    if t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv):
        raise ValueError("%s must be fp32 [%d,%d,%d,%d]" % (name, N, H, dk, dv))
    _check_dev(name, t, device)


def status_from_word(word: int) -> int:
    """KDA_OK or KDA_EWAIT for the status word a forward left in its workspace."""
    return int(_lib().kda_chunk_fwd_status(ctypes.c_uint32(int(word) & 0xFFFFFFFF)))


def fwd_status(workspace: torch.Tensor) -> int:
    """Read the status word of the last forward that used ``workspace`` (waits
    for the device) and map it; KDA_OK means every state-pass wait completed."""
    torch.cuda.synchronize(workspace.device)
    word = int(workspace[:4].cpu().view(torch.int32).item())
    return status_from_word(word)


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
    B, T, H, dk, dv, gate_kind = _check_seq_inputs(q, k, v, gate, beta, gate_kind)
    N = B if cu_seqlens is None else int(cu_seqlens.numel() - 1)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences (cu_seqlens) need B = 1, got %d" % B)
    if S0 is not None and (S0.dtype != torch.float32 or tuple(S0.shape) != (N, H, dk, dv)):
        raise ValueError("S0 must be fp32 [%d,%d,%d,%d]" % (N, H, dk, dv))
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    varlen, N = _check_varlen(cu_seqlens, B, device)
    _check_state("S0", S0, N, H, dk, dv, device)
    if out is None:
        out = torch.empty((B, T, H, dv), device=device, dtype=torch.float32)
    else:
        _check_dev("out", out, device)
        if out.dtype != torch.float32:
            raise TypeError("out must be fp32")
        _check_shape("out", out, (B, T, H, dv))
    if S_T is None and state_out:
        S_T = torch.empty((N, H, dk, dv), device=device, dtype=torch.float32)
    _check_state("S_T", S_T, N, H, dk, dv, device)
    need = workspace_bytes(B, H, T, dk, dv, chunk, N, varlen, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    st = _stream_handle(stream, device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_T), B, H, T, dk, dv, chunk,
            _ptr(cu_seqlens), N if varlen else 0, dt, int(gate_kind), _ptr(workspace),
            workspace.numel() * workspace.element_size(), ctypes.c_void_p(st) if st else None)
    if stage == STAGE_ALL:
        rc, where = _lib().kda_chunk_fwd(*args), "kda_chunk_fwd"
    else:
        rc, where = _lib().kda_chunk_fwd_stage(int(stage), *args), "kda_chunk_fwd_stage"
    if rc != KDA_OK:
        raise KDAError(rc, where)
    return out, S_T


def bwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, N: int = 0, varlen: bool = False) -> int:
    return int(_lib().kda_chunk_bwd_workspace_bytes(B, H, T, dk, dv, N, int(varlen)))


def bwd_cw_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, N: int = 0, varlen: bool = False) -> int:
    return int(_lib().kda_chunk_bwd_cw_workspace_bytes(B, H, T, dk, dv, N, int(varlen)))


def chunk_bwd(q, k, v, gate, beta, dO, S0=None, dS_T=None, cu_seqlens=None, gate_kind: Optional[int] = None,
              want_dS0: bool = True, out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
              stream=None, chunked: Optional[bool] = None) -> dict:
    """Gradient of chunk_fwd for L = sum(o * dO) + sum(S_T * dS_T). Inputs as
    for chunk_fwd; dO fp32 [B,T,H,dv]; dS_T fp32 [N,H,dk,dv] or None. Returns
    a dict of fp32 tensors dq, dk, dv, dgate, dbeta (input layouts) and dS0
    ([N,H,dk,dv], or None when not wanted). ``out`` may supply that dict's
    tensors to write into. ``chunked`` picks kda_chunk_bwd_cw (True) or the
    token-form kda_chunk_bwd (False); None takes the chunkwise form where it
    applies (dk = 64 or 128) and the token form elsewhere."""
    B, T, H, dk, dv, gate_kind = _check_seq_inputs(q, k, v, gate, beta, gate_kind)
    if chunked is None:
        chunked = dk in (64, 128)
    if dO.dtype != torch.float32 or tuple(dO.shape) != (B, T, H, dv):
        raise ValueError("dO must be fp32 [%d,%d,%d,%d]" % (B, T, H, dv))
    N = B if cu_seqlens is None else int(cu_seqlens.numel() - 1)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences (cu_seqlens) need B = 1, got %d" % B)
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv)):
            raise ValueError("%s must be fp32 [%d,%d,%d,%d]" % (name, N, H, dk, dv))
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta), ("dO", dO)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    varlen, N = _check_varlen(cu_seqlens, B, device)
    _check_state("S0", S0, N, H, dk, dv, device)
    _check_state("dS_T", dS_T, N, H, dk, dv, device)
    f32 = dict(device=device, dtype=torch.float32)
    if out is None:
        out = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
               "dv": torch.empty((B, T, H, dv), **f32), "dgate": torch.empty(tuple(gate.shape), **f32),
               "dbeta": torch.empty((B, T, H), **f32),
               "dS0": torch.empty((N, H, dk, dv), **f32) if want_dS0 else None}
    need = (bwd_cw_workspace_bytes if chunked else bwd_workspace_bytes)(B, H, T, dk, dv, N, varlen)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    st = _stream_handle(stream, device)
    fn = _lib().kda_chunk_bwd_cw if chunked else _lib().kda_chunk_bwd
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_T),
                              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dgate"]),
                              _ptr(out["dbeta"]), _ptr(out.get("dS0")), B, H, T, dk, dv, _ptr(cu_seqlens),
                              N if varlen else 0, dt, int(gate_kind), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_bwd_cw" if chunked else "kda_chunk_bwd")
    return out


def bwd_ew_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, N: int = 0, varlen: bool = False) -> int:
    return int(_lib().kda_chunk_bwd_ew_workspace_bytes(B, H, T, dk, dv, N, int(varlen)))


def chunk_bwd_ew(q, k, v, gate, erase, write, dO, S0=None, dS_T=None, cu_seqlens=None,
                 gate_kind: Optional[int] = None, want_dS0: bool = True, out: Optional[dict] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradient of chunk_fwd_ew (kda_chunk_bwd_ew) for L = sum(o * dO) +
    sum(S_T * dS_T). Inputs as for chunk_fwd_ew, dO and dS_T as for chunk_bwd.
    Returns a dict of fp32 tensors dq, dk, dv, dgate, derase, dwrite (input
    layouts) and dS0 ([N,H,dk,dv], or None when not wanted)."""
    B, T, H, dk, dv, gate_kind = _check_seq_inputs(q, k, v, gate, erase[..., 0], gate_kind)
    _check_shape("erase", erase, (B, T, H, dk))
    _check_shape("write", write, (B, T, H, dv))
    for name, t in (("erase", erase), ("write", write)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    if dO.dtype != torch.float32 or tuple(dO.shape) != (B, T, H, dv):
        raise ValueError("dO must be fp32 [%d,%d,%d,%d]" % (B, T, H, dv))
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences (cu_seqlens) need B = 1, got %d" % B)
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("erase", erase), ("write", write), ("dO", dO)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    varlen, N = _check_varlen(cu_seqlens, B, device)
    _check_state("S0", S0, N, H, dk, dv, device)
    _check_state("dS_T", dS_T, N, H, dk, dv, device)
    f32 = dict(device=device, dtype=torch.float32)
    if out is None:
        out = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
               "dv": torch.empty((B, T, H, dv), **f32), "dgate": torch.empty(tuple(gate.shape), **f32),
               "derase": torch.empty((B, T, H, dk), **f32), "dwrite": torch.empty((B, T, H, dv), **f32),
               "dS0": torch.empty((N, H, dk, dv), **f32) if want_dS0 else None}
    need = bwd_ew_workspace_bytes(B, H, T, dk, dv, N, varlen)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    st = _stream_handle(stream, device)
    rc = _lib().kda_chunk_bwd_ew(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(erase), _ptr(write), _ptr(S0), _ptr(dO),
                                 _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dgate"]),
                                 _ptr(out["derase"]), _ptr(out["dwrite"]), _ptr(out.get("dS0")), B, H, T, dk, dv,
                                 _ptr(cu_seqlens), N if varlen else 0, dt, int(gate_kind), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_bwd_ew")
    return out


def gauge_fold(q, k, gate, cu_seqlens=None, gate_kind: Optional[int] = None, stream=None):
    """Gauge fold: returns (q~, k~, gate~, c_T) with c_T int8 [N,H,dk] or
    [N,H]. Inputs as for chunk_fwd."""
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk], got %s" % (tuple(q.shape),))
    B, T, H, dk = q.shape
    _check_shape("k", k, (B, T, H, dk))
    gate_kind = _gate_kind(gate, 3, gate_kind)
    _check_shape("gate", gate, (B, T, H, dk) if gate_kind == GATE_CHANNEL else (B, T, H))
    for name, t in (("k", k), ("gate", gate)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    device = q.device
    for name, t in (("q", q), ("k", k), ("gate", gate)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    varlen, N = _check_varlen(cu_seqlens, B, device)
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
    B, T, H, dk, dv, gate_kind = _check_seq_inputs(q, k, v, gate, beta, gate_kind)
    N = B if cu_seqlens is None else int(cu_seqlens.numel() - 1)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences (cu_seqlens) need B = 1, got %d" % B)
    if S0 is not None and (S0.dtype != torch.float32 or tuple(S0.shape) != (N, H, dk, dv)):
        raise ValueError("S0 must be fp32 [%d,%d,%d,%d]" % (N, H, dk, dv))
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    varlen, N = _check_varlen(cu_seqlens, B, device)
    _check_state("S0", S0, N, H, dk, dv, device)
    if out is None:
        out = torch.empty((B, T, H, dv), device=device, dtype=torch.float32)
    else:
        _check_dev("out", out, device)
        _check_shape("out", out, (B, T, H, dv))
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), device=device, dtype=torch.float32)
    _check_state("S_T", S_T, N, H, dk, dv, device)
    need = fwd_gauge_workspace_bytes(B, H, T, dk, dv, chunk, N, varlen, q.dtype, gate_kind)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
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
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [N,H,dk] and v [N,H,dv]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check_shape("k", k, (N, H, dk))
    _check_shape("v", v, (N, H, dv))
    gate_kind = _gate_kind(gate, 2, gate_kind)
    _check_shape("gate", gate, (N, H, dk) if gate_kind == GATE_CHANNEL else (N, H))
    _check_shape("beta", beta, (N, H))
    for name, t in (("k", k), ("v", v), ("gate", gate), ("beta", beta)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    if S.dtype != torch.float32 or tuple(S.shape) != (N, H, dk, dv):
        raise ValueError("S must be fp32 [%d,%d,%d,%d]" % (N, H, dk, dv))
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("beta", beta), ("S", S)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((N, H, dv), device=device, dtype=torch.float32)
    else:
        _check_dev("out", out, device)
        _check_shape("out", out, (N, H, dv))
    st = _stream_handle(stream, device)
    rc = _lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S), _ptr(out),
                                N, H, dk, dv, dt, int(gate_kind), ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_decode_step")
    return out


def chunk_fwd_ew(q, k, v, gate, erase, write, S0=None, cu_seqlens=None, chunk: int = 64,
                 gate_kind: Optional[int] = None, out: Optional[torch.Tensor] = None, state_out: bool = True,
                 S_T: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise forward with decoupled erase and write gates
    (kda_chunk_fwd_ew): S_t = (I - k (e o k)^T) Diag(alpha) S + k (w o v)^T.
    erase [B,T,H,dk], write [B,T,H,dv] in the inputs' dtype; everything else as
    for chunk_fwd (the erase gate takes beta's place in the shape checks)."""
    B, T, H, dk, dv, gate_kind = _check_seq_inputs(q, k, v, gate, erase[..., 0], gate_kind)
    _check_shape("erase", erase, (B, T, H, dk))
    _check_shape("write", write, (B, T, H, dv))
    for name, t in (("erase", erase), ("write", write)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    N = B if cu_seqlens is None else int(cu_seqlens.numel() - 1)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences (cu_seqlens) need B = 1, got %d" % B)
    if S0 is not None and (S0.dtype != torch.float32 or tuple(S0.shape) != (N, H, dk, dv)):
        raise ValueError("S0 must be fp32 [%d,%d,%d,%d]" % (N, H, dk, dv))
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("erase", erase), ("write", write)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    varlen, N = _check_varlen(cu_seqlens, B, device)
    _check_state("S0", S0, N, H, dk, dv, device)
    if out is None:
        out = torch.empty((B, T, H, dv), device=device, dtype=torch.float32)
    else:
        _check_dev("out", out, device)
        _check_shape("out", out, (B, T, H, dv))
    if S_T is None and state_out:
        S_T = torch.empty((N, H, dk, dv), device=device, dtype=torch.float32)
    _check_state("S_T", S_T, N, H, dk, dv, device)
    need = workspace_bytes(B, H, T, dk, dv, chunk, N, varlen, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=device, dtype=torch.uint8)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    st = _stream_handle(stream, device)
    rc = _lib().kda_chunk_fwd_ew(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(erase), _ptr(write), _ptr(S0), _ptr(out),
                                 _ptr(S_T), B, H, T, dk, dv, chunk, _ptr(cu_seqlens), N if varlen else 0, dt,
                                 int(gate_kind), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_ew")
    return out, S_T


def decode_step_ew(q, k, v, gate, erase, write, S, out: Optional[torch.Tensor] = None,
                   gate_kind: Optional[int] = None, stream=None) -> torch.Tensor:
    """One decode step with erase [N,H,dk] and write [N,H,dv] gates
    (kda_decode_step_ew); S [N,H,dk,dv] fp32 updated in place."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [N,H,dk] and v [N,H,dv]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check_shape("k", k, (N, H, dk))
    _check_shape("v", v, (N, H, dv))
    _check_shape("erase", erase, (N, H, dk))
    _check_shape("write", write, (N, H, dv))
    gate_kind = _gate_kind(gate, 2, gate_kind)
    _check_shape("gate", gate, (N, H, dk) if gate_kind == GATE_CHANNEL else (N, H))
    for name, t in (("k", k), ("v", v), ("gate", gate), ("erase", erase), ("write", write)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    if S.dtype != torch.float32 or tuple(S.shape) != (N, H, dk, dv):
        raise ValueError("S must be fp32 [%d,%d,%d,%d]" % (N, H, dk, dv))
    device = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("erase", erase), ("write", write), ("S", S)):
        _check_dev(name, t, device)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((N, H, dv), device=device, dtype=torch.float32)
    else:
        _check_dev("out", out, device)
        _check_shape("out", out, (N, H, dv))
    st = _stream_handle(stream, device)
    rc = _lib().kda_decode_step_ew(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(erase), _ptr(write), _ptr(S),
                                   _ptr(out), N, H, dk, dv, dt, int(gate_kind), ctypes.c_void_p(st) if st else None)
    if rc != KDA_OK:
        raise KDAError(rc, "kda_decode_step_ew")
    return out
