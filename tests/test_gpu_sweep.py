"""Seeded randomized parity sweep: forward, backward and gauge route over
random shapes (every supported dk, dv and chunk), both input dtypes, all gate
kinds, fixed-length and packed sequences with ragged lengths, against the
fp64 oracle with the same metrics and bars as the dedicated tests.

A second generator draws longer sequences (up to 2,000 tokens), more heads
(up to 8) and packed batches of up to 8 sequences; KDA_SWEEP_LARGE sets how
many of those cases run (default 40). The decode step is swept on random
shapes too, several steps in place."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_46_amd import inputs

pytestmark = pytest.mark.gpu

FWD_TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
NAMES = ("dq", "dk", "dv", "dgate", "dbeta", "dS0")


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_46_amd import kda as m
    m.library()
    return m


def err(x, ref):
    x = x.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(ref * ref)))
    d = float(np.max(np.abs(x - ref)))
    return d / rms if rms > 0 else d


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    dv = int(rng.choice([16, 32, 64, 128]))
    chunk = int(rng.choice([16, 32, 64]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    gate = str(rng.choice(["kda", "ckda", "gdn"]))
    H = int(rng.integers(1, 4))
    if rng.random() < 0.4:
        lengths = [int(x) for x in rng.integers(0, 160, size=int(rng.integers(1, 5)))]
        if sum(lengths) == 0:
            lengths[0] = 7
        w = inputs.make_forward("sweep%d" % seed, B=1, H=H, T=0, dk=dk, dv=dv, chunk=chunk, dtype=dtype, gate=gate,
                                gate_mu=float(rng.uniform(1, 4)), seed=seed, lengths=lengths,
                                s0_std=float(rng.choice([0.0, 0.3])))
    else:
        w = inputs.make_forward("sweep%d" % seed, B=int(rng.integers(1, 3)), H=H, T=int(rng.integers(1, 200)), dk=dk,
                                dv=dv, chunk=chunk, dtype=dtype, gate=gate, gate_mu=float(rng.uniform(1, 4)), seed=seed,
                                s0_std=float(rng.choice([0.0, 0.3])))
    return w


def random_large_case(seed):
    rng = np.random.default_rng(50000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    dv = int(rng.choice([16, 32, 64, 128]))
    chunk = int(rng.choice([16, 32, 64]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    gate = str(rng.choice(["kda", "ckda", "gdn"]))
    H = int(rng.integers(1, 9))
    if rng.random() < 0.4:
        lengths = [int(x) for x in rng.integers(0, 700, size=int(rng.integers(1, 9)))]
        if sum(lengths) == 0:
            lengths[0] = 7
        return inputs.make_forward("large%d" % seed, B=1, H=H, T=0, dk=dk, dv=dv, chunk=chunk, dtype=dtype,
                                   gate=gate, gate_mu=float(rng.uniform(1, 4)), seed=seed, lengths=lengths,
                                   s0_std=float(rng.choice([0.0, 0.3])))
    return inputs.make_forward("large%d" % seed, B=int(rng.integers(1, 4)), H=H, T=int(rng.integers(1, 2000)),
                               dk=dk, dv=dv, chunk=chunk, dtype=dtype, gate=gate, gate_mu=float(rng.uniform(1, 4)),
                               seed=seed, s0_std=float(rng.choice([0.0, 0.3])))


def dev(t):
    return None if t is None else t.cuda()


@pytest.mark.parametrize("seed", range(24))
def test_forward_sweep(kda, seed):
    w = random_case(seed)
    print("case", w.name, "B", w.B, "H", w.H, "T", w.T, "dk", w.dk, "dv", w.dv, "chunk", w.chunk, w.q.dtype,
          "gate kind", w.gate_kind, "varlen", w.cu_seqlens is not None, flush=True)
    o, ST = kda.chunk_fwd(dev(w.q), dev(w.k), dev(w.v), dev(w.gate), dev(w.beta), S0=dev(w.S0),
                          cu_seqlens=dev(w.cu_seqlens), chunk=w.chunk, gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0, w.cu_seqlens, w.gate_kind)
    tol = FWD_TOL[w.q.dtype]
    assert err(o, ro) <= tol and err(ST, rS) <= tol, (err(o, ro), err(ST, rS))


@pytest.mark.parametrize("seed", range(12))
def test_backward_sweep(kda, seed):
    w = random_case(100 + seed)
    print("case", w.name, "B", w.B, "H", w.H, "T", w.T, "dk", w.dk, "dv", w.dv, w.q.dtype, "gate kind", w.gate_kind,
          "varlen", w.cu_seqlens is not None, flush=True)
    dO, dST = inputs.cotangents(w, seed=seed, with_dS_T=seed % 3 != 0)
    r = oracle.bwd(w.q, w.k, w.v, w.gate, w.beta, dO, w.S0, dST, w.cu_seqlens, w.gate_kind)
    # the token form everywhere, the chunkwise form where it applies (dk 64, 128)
    for chunked in (False, True) if w.dk in (64, 128) else (False,):
        g = kda.chunk_bwd(dev(w.q), dev(w.k), dev(w.v), dev(w.gate), dev(w.beta), dev(dO), S0=dev(w.S0),
                          dS_T=dev(dST), cu_seqlens=dev(w.cu_seqlens), gate_kind=w.gate_kind, chunked=chunked)
        torch.cuda.synchronize()
        errs = {n: err(g[n], r[n]) for n in NAMES}
        assert max(errs.values()) <= 1e-4, (chunked, errs)


@pytest.mark.parametrize("seed", range(8))
def test_gauge_route_sweep(kda, seed):
    w = random_case(200 + seed)
    print("case", w.name, "B", w.B, "H", w.H, "T", w.T, "dk", w.dk, "dv", w.dv, w.q.dtype, "gate kind", w.gate_kind,
          flush=True)
    o, ST = kda.chunk_fwd_gauge(dev(w.q), dev(w.k), dev(w.v), dev(w.gate), dev(w.beta), S0=dev(w.S0),
                                cu_seqlens=dev(w.cu_seqlens), chunk=w.chunk, gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0, w.cu_seqlens, w.gate_kind)
    tol = FWD_TOL[w.q.dtype]
    assert err(o, ro) <= tol and err(ST, rS) <= tol, (err(o, ro), err(ST, rS))


@pytest.mark.parametrize("seed", range(int(os.environ.get("KDA_SWEEP_LARGE", "40"))))
def test_large_sweep(kda, seed):
    """Forward (three cases in five), backward and gauge route on the larger shapes."""
    w = random_large_case(seed)
    kind = ("fwd", "fwd", "fwd", "bwd", "gauge")[seed % 5]
    print("case", kind, w.name, "B", w.B, "H", w.H, "T", w.T, "dk", w.dk, "dv", w.dv, "chunk", w.chunk, w.q.dtype,
          "gate kind", w.gate_kind, "varlen", w.cu_seqlens is not None, flush=True)
    if kind == "bwd":
        dO, dST = inputs.cotangents(w, seed=seed, with_dS_T=seed % 2 == 0)
        r = oracle.bwd(w.q, w.k, w.v, w.gate, w.beta, dO, w.S0, dST, w.cu_seqlens, w.gate_kind)
        for chunked in (False, True) if w.dk in (64, 128) else (False,):
            g = kda.chunk_bwd(dev(w.q), dev(w.k), dev(w.v), dev(w.gate), dev(w.beta), dev(dO), S0=dev(w.S0),
                              dS_T=dev(dST), cu_seqlens=dev(w.cu_seqlens), gate_kind=w.gate_kind, chunked=chunked)
            torch.cuda.synchronize()
            errs = {n: err(g[n], r[n]) for n in NAMES}
            assert max(errs.values()) <= 1e-4, (chunked, errs)
        return
    fn = kda.chunk_fwd if kind == "fwd" else kda.chunk_fwd_gauge
    o, ST = fn(dev(w.q), dev(w.k), dev(w.v), dev(w.gate), dev(w.beta), S0=dev(w.S0), cu_seqlens=dev(w.cu_seqlens),
               chunk=w.chunk, gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0, w.cu_seqlens, w.gate_kind)
    tol = FWD_TOL[w.q.dtype]
    assert err(o, ro) <= tol and err(ST, rS) <= tol, (err(o, ro), err(ST, rS))


@pytest.mark.parametrize("seed", range(16))
def test_decode_sweep(kda, seed):
    """Decode steps in place on random N, H, dk, dv, dtype and gate kind, against
    the oracle's step applied to the same fp64 state."""
    rng = np.random.default_rng(7000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    dv = int(rng.choice([16, 32, 64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    gate = str(rng.choice(["kda", "ckda", "gdn"]))
    gk = 1 if gate == "gdn" else 0
    N, H, steps = int(rng.integers(1, 41)), int(rng.integers(1, 9)), int(rng.integers(3, 9))
    print("case decode", seed, "N", N, "H", H, "dk", dk, "dv", dv, dtype, gate, "steps", steps, flush=True)
    S = torch.from_numpy(rng.normal(0, 0.3, (N, H, dk, dv))).float()
    Sd = S.cuda()
    Sr = S.double().numpy().copy()
    for st in range(steps):
        w = inputs.make_forward("dec", B=N, H=H, T=1, dk=dk, dv=dv, dtype=dtype, gate=gate, seed=100 * seed + st)
        q, k, v, g, b = (t[:, 0].contiguous() for t in (w.q, w.k, w.v, w.gate, w.beta))
        o = kda.decode_step(q.cuda(), k.cuda(), v.cuda(), g.cuda(), b.cuda(), Sd, gate_kind=gk)
        ro = oracle.decode_step(q, k, v, g, b, Sr, gate_kind=gk)
        torch.cuda.synchronize()
        assert err(o, ro) < (1e-5 if dtype == torch.float32 else 1e-3)
    assert err(Sd, Sr) < 1e-5
