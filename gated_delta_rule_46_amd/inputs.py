"""Seeded synthetic inputs for the gated delta-rule forward and decode workloads.

This module is shared by the HIP path's tests/bench and by the fp64 oracle's
tests. It draws random numbers and shapes them into the value ranges of the
workloads; it holds none of the recurrence's arithmetic.

Recipe (all draws in fp64 from ``numpy.random.default_rng(seed)``, PCG64, then
rounded once to the storage dtype with torch's round-to-nearest-even):

* q, k ~ N(0, 1), L2-normalised per (token, head) in fp64, then rounded.
* v ~ N(0, 1).
* KDA gate (Complex KDA summary, background "scalar vs channel gate"):
  alpha = exp(-softplus(a)) per channel, a ~ N(mu, 1).
* CKDA gate (Complex KDA summary, method step 1, the "spread" init):
  r = 2*sigmoid(a) - 1 with a ~ N(2*sign_i, 1); sign_i is drawn once per
  (head, channel) and shared over batch and time. beta = 2*sigmoid(b) with b
  a 50/50 mixture of N(+2, 1) and N(-2, 1). About 1% of gates are set to
  exactly +0.0 or -1.0 (half each) and about 1% of betas to exactly 2.0.
* GDN gate (scalar per (token, head)): alpha = exp(-softplus(a)), a ~ N(4, 1).
* beta = sigmoid(b), b ~ N(0, 1) for KDA and GDN.
* Variable-length lengths: 8 draws from U{4096..32768} with a generator of
  their own seeded like the tensors.

Draw order: q, k, v, gate variates, beta variates, masks, S0.

Backward inputs (``cotangents``): dO ~ N(0, 1) and dS_T ~ N(0, 1), fp32, from a
generator of their own seeded with seed + 7919.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

GATE_CHANNEL = 0
GATE_SCALAR = 1


@dataclasses.dataclass
class Workload:
    """One batch of forward (or one decode step's) inputs, as CPU tensors."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    gate: torch.Tensor
    beta: torch.Tensor
    S0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    gate_kind: int

    @property
    def n_seqs(self) -> int:
        return self.B if self.cu_seqlens is None else int(self.cu_seqlens.numel() - 1)

    @property
    def dtype(self) -> torch.dtype:
        return self.q.dtype

    def tokens(self) -> int:
        return self.B * self.T


# ---------------------------------------------------------------- primitives

def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def kda_gate(rng, shape, mu: float) -> np.ndarray:
    """Positive channel gate exp(-softplus(a)), a ~ N(mu, 1)."""
    return np.exp(-_softplus(rng.normal(mu, 1.0, size=shape)))


def ckda_gate_beta(rng, gshape, bshape, signs: np.ndarray):
    """Signed gate in [-1, 1] and beta in [0, 2] with the stress masks.

    ``signs`` broadcasts against ``gshape`` (one sign per head and channel).
    """
    a = rng.normal(0.0, 1.0, size=gshape) + 2.0 * signs
    gate = 2.0 * _sigmoid(a) - 1.0
    comp = rng.random(size=bshape) < 0.5
    b = rng.normal(0.0, 1.0, size=bshape) + np.where(comp, 2.0, -2.0)
    beta = 2.0 * _sigmoid(b)
    gmask = rng.random(size=gshape)
    gate = np.where(gmask < 0.005, 0.0, np.where(gmask < 0.01, -1.0, gate))
    bmask = rng.random(size=bshape)
    beta = np.where(bmask < 0.01, 2.0, beta)
    return gate, beta


def signed_zero_gates(gate: torch.Tensor, seed: int, frac: float = 0.03) -> torch.Tensor:
    """A copy of ``gate`` with about ``frac`` of its elements replaced, in
    equal parts, by -0.0, +0.0 and -1.0 (a stress mix of both zero signs and
    exact sign flips; any dtype with signed zeros)."""
    u = torch.from_numpy(np.random.default_rng(seed + 104729).random(size=tuple(gate.shape)))
    out = gate.clone()
    out[u < frac] = -1.0
    out[u < 2.0 * frac / 3.0] = 0.0
    out[u < frac / 3.0] = -0.0
    return out


def spread_signs(rng, H: int, dk: int) -> np.ndarray:
    return np.where(rng.random(size=(H, dk)) < 0.5, -1.0, 1.0)


# ---------------------------------------------------------------- generic

def make_forward(name: str, *, B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                 dtype: torch.dtype = torch.bfloat16, gate: str = "kda", gate_mu: float = 3.0,
                 seed: int = 0, lengths=None, s0_std: float = 0.0) -> Workload:
    """Forward inputs. ``gate`` is one of "kda", "ckda", "gdn"; ``lengths``
    packs variable-length sequences into one B=1 stream."""
    rng = np.random.default_rng(seed)
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    q = _l2n(rng.standard_normal((B, T, H, dk)))
    k = _l2n(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    gate_kind = GATE_CHANNEL
    if gate == "kda":
        g = kda_gate(rng, (B, T, H, dk), gate_mu)
        beta = _sigmoid(rng.standard_normal((B, T, H)))
    elif gate == "gdn":
        gate_kind = GATE_SCALAR
        g = kda_gate(rng, (B, T, H), gate_mu)
        beta = _sigmoid(rng.standard_normal((B, T, H)))
    elif gate == "ckda":
        signs = spread_signs(rng, H, dk)
        g, beta = ckda_gate_beta(rng, (B, T, H, dk), (B, T, H), signs)
    else:
        raise ValueError(gate)
    n_seq = B if lengths is None else len(lengths)
    S0 = None
    if s0_std > 0.0:
        S0 = torch.from_numpy(rng.normal(0.0, s0_std, size=(n_seq, H, dk, dv))).float()
    cu = None
    if lengths is not None:
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return Workload(name, _round(q, dtype), _round(k, dtype), _round(v, dtype), _round(g, dtype),
                    _round(beta, dtype), S0, cu, B, H, T, dk, dv, chunk, gate_kind)


@dataclasses.dataclass
class EraseWriteWorkload:
    """Forward inputs with decoupled erase [B,T,H,dk] and write [B,T,H,dv]
    gates in place of beta."""
    w: Workload
    erase: torch.Tensor
    write: torch.Tensor


def erase_write_gates(w: Workload, seed: int, erase: str = "bimodal"):
    """Erase and write gates for workload ``w`` (a generator of their own,
    seeded with seed + 15485863): erase e = 2 sigmoid(b) per (token, head,
    key channel) with b a 50/50 mixture of N(+2, 1) and N(-2, 1) ("bimodal",
    the Complex KDA beta recipe applied per channel, with about 1% of the
    values exactly 2.0 and 1% exactly 0.0), or e = sigmoid(N(0, 1))
    ("sigmoid"); write w = sigmoid(N(0, 1)) per (token, head, value channel)."""
    rng = np.random.default_rng(seed + 15485863)
    es = (w.B, w.T, w.H, w.dk)
    if erase == "bimodal":
        comp = rng.random(size=es) < 0.5
        e = 2.0 * _sigmoid(rng.normal(0.0, 1.0, size=es) + np.where(comp, 2.0, -2.0))
        m = rng.random(size=es)
        e = np.where(m < 0.01, 2.0, np.where(m < 0.02, 0.0, e))
    elif erase == "sigmoid":
        e = _sigmoid(rng.standard_normal(es))
    else:
        raise ValueError(erase)
    wr = _sigmoid(rng.standard_normal((w.B, w.T, w.H, w.dv)))
    return EraseWriteWorkload(w, _round(e, w.dtype), _round(wr, w.dtype))


def gdn2_ckda_fwd(seed: int = 0, B: int = 2, H: int = 16, T: int = 8192) -> EraseWriteWorkload:
    """Erase/write gates combined with Complex KDA's signed gates (the pages'
    future-work combination) at the Complex KDA workload's shape: B=2, H=16,
    T=8192, d=128, bf16, chunk 64; alpha by the Complex KDA recipe, erase
    bimodal in [0, 2], write sigmoid."""
    w = make_forward("gdn2_ckda_b2_h16_t8192", B=B, H=H, T=T, dk=128, dv=128, chunk=64, gate="ckda", seed=seed)
    return erase_write_gates(w, seed)


def cotangents(w: Workload, seed: int = 0, with_dS_T: bool = True):
    """Output gradients for a backward call on ``w``: dO [B,T,H,dv] and dS_T
    [N,H,dk,dv] (or None), fp32 CPU tensors."""
    rng = np.random.default_rng(seed + 7919)
    dO = torch.from_numpy(rng.standard_normal((w.B, w.T, w.H, w.dv))).float()
    dST = None
    if with_dS_T:
        dST = torch.from_numpy(rng.standard_normal((w.n_seqs, w.H, w.dk, w.dv))).float()
    return dO, dST


def varlen_lengths(seed: int = 0, n: int = 8, lo: int = 4096, hi: int = 32768):
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi, size=n, endpoint=True)]


# ---------------------------------------------------------------- the five workloads

def tiny_kda(seed: int = 0) -> Workload:
    """B=1, H=1, T=64, dk=dv=16, fp32, chunk 16, a ~ N(2, 1), S0 = 0."""
    return make_forward("tiny_kda_fp32", B=1, H=1, T=64, dk=16, dv=16, chunk=16,
                        dtype=torch.float32, gate="kda", gate_mu=2.0, seed=seed)


def kda_fwd(seed: int = 0, B: int = 4, H: int = 16, T: int = 4096) -> Workload:
    """KDA forward: B=4, H=16, T=4096, d=128, bf16, a ~ N(3, 1), chunk 64."""
    return make_forward("kda_b4_h16_t4096", B=B, H=H, T=T, dk=128, dv=128, chunk=64,
                        gate="kda", gate_mu=3.0, seed=seed)


def ckda_fwd(seed: int = 0, B: int = 2, H: int = 16, T: int = 8192) -> Workload:
    """Complex KDA forward: B=2, H=16, T=8192, d=128, bf16, spread init, stress masks."""
    return make_forward("ckda_b2_h16_t8192", B=B, H=H, T=T, dk=128, dv=128, chunk=64,
                        gate="ckda", seed=seed)


def gdn_varlen(seed: int = 0, H: int = 32, lengths=None) -> Workload:
    """GDN scalar gate, 8 packed sequences (lengths U{4096..32768}), H=32, d=128."""
    if lengths is None:
        lengths = varlen_lengths(seed)
    return make_forward("gdn_varlen_h32", B=1, H=H, T=0, dk=128, dv=128, chunk=64,
                        gate="gdn", gate_mu=4.0, seed=seed, lengths=lengths)


@dataclasses.dataclass
class DecodeWorkload:
    """Decode inputs: an fp32 state and a list of per-step token inputs."""
    name: str
    S: torch.Tensor
    steps: list  # of dicts q, k, v, gate, beta (CPU tensors)
    N: int
    H: int
    dk: int
    dv: int
    gate_kind: int


def ckda_decode(seed: int = 0, N: int = 256, H: int = 32, d: int = 128, n_steps: int = 128,
                s_std: float = 0.01, dtype: torch.dtype = torch.bfloat16) -> DecodeWorkload:
    """Decode: N sequences, H heads, fp32 state ~ N(0, 0.01^2); per step bf16
    q, k (L2-normalised), v ~ N(0, 1), CKDA-range gate and beta (the Complex KDA
    spread recipe, fresh variates each step; one sign per head and channel)."""
    rng = np.random.default_rng(seed)
    signs = spread_signs(rng, H, d)
    steps = []
    for _ in range(n_steps):
        q = _l2n(rng.standard_normal((N, H, d)))
        k = _l2n(rng.standard_normal((N, H, d)))
        v = rng.standard_normal((N, H, d))
        g, beta = ckda_gate_beta(rng, (N, H, d), (N, H), signs)
        steps.append(dict(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype),
                          gate=_round(g, dtype), beta=_round(beta, dtype)))
    S = torch.from_numpy(rng.normal(0.0, s_std, size=(N, H, d, d))).float()
    return DecodeWorkload("ckda_decode_n%d_h%d" % (N, H), S, steps, N, H, d, d, GATE_CHANNEL)


CONFIGS = {
    1: tiny_kda,
    2: kda_fwd,
    3: ckda_fwd,
    4: gdn_varlen,
    5: ckda_decode,
}
