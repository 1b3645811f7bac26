"""ctypes wrapper over the plain-C fp64 recurrence in ``kda_oracle.c``.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Inputs are the exact values handed to the GPU: bf16 or fp32 tensors are
up-converted to fp64 here, so input quantisation is not charged to the kernel.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
# KDA_ORACLE_LIB names a prebuilt copy (the sanitizer build); build() then
# leaves it alone unless forced.
_LIB = os.environ.get("KDA_ORACLE_LIB") or os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP); returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [_dp] * 7 + [_dp] + [ctypes.c_int] * 5 + [_ip] + [ctypes.c_int] * 2
        lib.kda_oracle_decode.restype = ctypes.c_int
        lib.kda_oracle_decode.argtypes = [_dp] * 7 + [ctypes.c_int] * 5
        lib.kda_oracle_fwd_ew.restype = ctypes.c_int
        lib.kda_oracle_fwd_ew.argtypes = [_dp] * 9 + [ctypes.c_int] * 5 + [_ip] + [ctypes.c_int] * 2
        lib.kda_oracle_decode_ew.restype = ctypes.c_int
        lib.kda_oracle_decode_ew.argtypes = [_dp] * 8 + [ctypes.c_int] * 5
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [_dp] * 14 + [ctypes.c_int] * 5 + [_ip] + [ctypes.c_int] * 2
        lib.kda_oracle_bwd_ew.restype = ctypes.c_int
        lib.kda_oracle_bwd_ew.argtypes = [_dp] * 16 + [ctypes.c_int] * 5 + [_ip] + [ctypes.c_int] * 2
        _lib = lib
    return _lib


def threads() -> int:
    """Threads OpenMP will use (OMP_NUM_THREADS, else the process's CPU set)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env:
        try:
            return int(env)
        except ValueError:
            pass
    return len(os.sched_getaffinity(0))


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().to(torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def fwd(q, k, v, gate, beta, S0=None, cu_seqlens=None, gate_kind: int = 0):
    """Run the recurrence over whole sequences. Returns (o, S_T) as fp64 numpy.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; gate: [B,T,H,dk] or [B,T,H]; beta [B,T,H];
    S0: [nseq,H,dk,dv] or None; cu_seqlens: [nseq+1] int offsets (B must be 1).
    """
    lib = _load()
    q, k, v, gate, beta = (_f64(t) for t in (q, k, v, gate, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor)
                                             else cu_seqlens), dtype=np.int32)
        nseq = cu.size - 1
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((nseq, H, dk, dv))
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                            None if s0 is None else _ptr(s0), _ptr(o), _ptr(ST),
                            B, H, T, dk, dv, None if cu is None else cu.ctypes.data_as(_ip), nseq,
                            int(gate_kind))
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments")
    return o, ST


def bwd(q, k, v, gate, beta, dO, S0=None, dS_T=None, cu_seqlens=None, gate_kind: int = 0):
    """Gradient of L = sum(o * dO) + sum(S_T * dS_T) with respect to every
    input of ``fwd`` (reverse-mode adjoint of the token recurrence, fp64).
    Returns a dict of fp64 numpy arrays dq, dk, dv, dgate, dbeta (input
    layouts) and dS0 [nseq,H,dk,dv]."""
    lib = _load()
    q, k, v, gate, beta, dO = (_f64(t) for t in (q, k, v, gate, beta, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor)
                                             else cu_seqlens), dtype=np.int32)
        nseq = cu.size - 1
    s0 = None if S0 is None else _f64(S0)
    dst = None if dS_T is None else _f64(dS_T)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "dgate": np.zeros_like(gate),
           "dbeta": np.zeros_like(beta), "dS0": np.zeros((nseq, H, dk, dv))}
    rc = lib.kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                            None if s0 is None else _ptr(s0), _ptr(dO), None if dst is None else _ptr(dst),
                            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dgate"]),
                            _ptr(out["dbeta"]), _ptr(out["dS0"]), B, H, T, dk, dv,
                            None if cu is None else cu.ctypes.data_as(_ip), nseq, int(gate_kind))
    if rc != 0:
        raise ValueError("kda_oracle_bwd rejected its arguments")
    return out


def fwd_heads(q, k, v, gate, beta, heads, S0=None, cu_seqlens=None, gate_kind: int = 0):
    """The recurrence restricted to a subset of heads (every head is
    independent). Returns (o[..., heads, :], S_T[:, heads]) as fp64 numpy."""
    idx = torch.as_tensor(list(heads), dtype=torch.long)
    sel = lambda t: None if t is None else t.index_select(2, idx)  # noqa: E731
    s0 = None if S0 is None else S0.index_select(1, idx)
    return fwd(sel(q), sel(k), sel(v), sel(gate), beta.index_select(2, idx), s0, cu_seqlens, gate_kind)


def decode_step(q, k, v, gate, beta, S: np.ndarray, gate_kind: int = 0) -> np.ndarray:
    """One decode step; ``S`` (fp64 numpy [N,H,dk,dv]) is updated in place.
    Returns o [N,H,dv] fp64."""
    lib = _load()
    q, k, v, gate, beta = (_f64(t) for t in (q, k, v, gate, beta))
    assert S.dtype == np.float64 and S.flags.c_contiguous
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv))
    rc = lib.kda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S), _ptr(o),
                               N, H, dk, dv, int(gate_kind))
    if rc != 0:
        raise ValueError("kda_oracle_decode rejected its arguments")
    return o


def fwd_ew(q, k, v, gate, erase, write, S0=None, cu_seqlens=None, gate_kind: int = 0):
    """The recurrence with decoupled erase and write gates (Gated DeltaNet-2
    blurb; reading in kda_oracle.c):
        S_t = (I - k_t (e_t o k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t o v_t)^T.
    erase [B,T,H,dk], write [B,T,H,dv]; everything else as for ``fwd``.
    Returns (o, S_T) as fp64 numpy."""
    lib = _load()
    q, k, v, gate, erase, write = (_f64(t) for t in (q, k, v, gate, erase, write))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor)
                                             else cu_seqlens), dtype=np.int32)
        nseq = cu.size - 1
    if erase.shape != k.shape or write.shape != v.shape:
        raise ValueError("erase must be shaped like k and write like v")
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((nseq, H, dk, dv))
    rc = lib.kda_oracle_fwd_ew(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(erase), _ptr(write),
                               None if s0 is None else _ptr(s0), _ptr(o), _ptr(ST), B, H, T, dk, dv,
                               None if cu is None else cu.ctypes.data_as(_ip), nseq, int(gate_kind))
    if rc != 0:
        raise ValueError("kda_oracle_fwd_ew rejected its arguments")
    return o, ST


def decode_step_ew(q, k, v, gate, erase, write, S: np.ndarray, gate_kind: int = 0) -> np.ndarray:
    """One decode step with erase [N,H,dk] and write [N,H,dv] gates; ``S``
    (fp64 numpy [N,H,dk,dv]) is updated in place. Returns o [N,H,dv]."""
    lib = _load()
    q, k, v, gate, erase, write = (_f64(t) for t in (q, k, v, gate, erase, write))
    assert S.dtype == np.float64 and S.flags.c_contiguous
    N, H, dk = q.shape
    dv = v.shape[-1]
    if erase.shape != k.shape or write.shape != v.shape:
        raise ValueError("erase must be shaped like k and write like v")
    o = np.zeros((N, H, dv))
    rc = lib.kda_oracle_decode_ew(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(erase), _ptr(write), _ptr(S),
                                  _ptr(o), N, H, dk, dv, int(gate_kind))
    if rc != 0:
        raise ValueError("kda_oracle_decode_ew rejected its arguments")
    return o


def bwd_ew(q, k, v, gate, erase, write, dO, S0=None, dS_T=None, cu_seqlens=None, gate_kind: int = 0):
    """Gradient of L = sum(o * dO) + sum(S_T * dS_T) for ``fwd_ew`` (reverse-mode
    adjoint of the erase/write token recurrence, fp64). Returns a dict of fp64
    numpy arrays dq, dk, dv, dgate, derase, dwrite (input layouts) and dS0
    [nseq,H,dk,dv]."""
    lib = _load()
    q, k, v, gate, erase, write, dO = (_f64(t) for t in (q, k, v, gate, erase, write, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if erase.shape != k.shape or write.shape != v.shape:
        raise ValueError("erase must be shaped like k and write like v")
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor)
                                             else cu_seqlens), dtype=np.int32)
        nseq = cu.size - 1
    s0 = None if S0 is None else _f64(S0)
    dst = None if dS_T is None else _f64(dS_T)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "dgate": np.zeros_like(gate),
           "derase": np.zeros_like(erase), "dwrite": np.zeros_like(write), "dS0": np.zeros((nseq, H, dk, dv))}
    rc = lib.kda_oracle_bwd_ew(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(erase), _ptr(write),
                               None if s0 is None else _ptr(s0), _ptr(dO), None if dst is None else _ptr(dst),
                               _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dgate"]),
                               _ptr(out["derase"]), _ptr(out["dwrite"]), _ptr(out["dS0"]), B, H, T, dk, dv,
                               None if cu is None else cu.ctypes.data_as(_ip), nseq, int(gate_kind))
    if rc != 0:
        raise ValueError("kda_oracle_bwd_ew rejected its arguments")
    return out
