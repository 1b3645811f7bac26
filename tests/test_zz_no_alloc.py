"""kda_chunk_fwd_noalloc (the forward without a caller workspace, for callers
that cannot allocate) through the C ABI against kda_chunk_fwd on the same
inputs: the two share every kernel, so o and S_T must agree bit for bit.
Two calls in a row, the second smaller than the first (the fixed scratch
keeps the first call's contents, stale status word included), plus packed
sequences, and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_46_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_46_amd import kda as m
    m.library()
    return m


def _P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run_both(kda, w):
    lib = kda.library()
    d = lambda t: None if t is None else t.cuda()  # noqa: E731
    q, k, v, g, b, s0, cu = (d(x) for x in (w.q, w.k, w.v, w.gate, w.beta, w.S0, w.cu_seqlens))
    N = w.n_seqs
    dt = kda.KDA_BF16 if w.dtype == torch.bfloat16 else kda.KDA_F32
    nan = dict(device="cuda", dtype=torch.float32)
    o1 = torch.full((w.B, w.T, w.H, w.dv), float("nan"), **nan)
    S1 = torch.full((N, w.H, w.dk, w.dv), float("nan"), **nan)
    o2, S2 = o1.clone(), S1.clone()
    need = lib.kda_chunk_fwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, N, int(cu is not None), dt)
    assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    Nn = N if cu is not None else 0
    print("case", w.name, "B", w.B, "H", w.H, "T", w.T, "dk", w.dk, "dv", w.dv, "chunk", w.chunk, "need", need,
          flush=True)
    rc = lib.kda_chunk_fwd(_P(q), _P(k), _P(v), _P(g), _P(b), _P(s0), _P(o1), _P(S1), w.B, w.H, w.T, w.dk, w.dv,
                           w.chunk, _P(cu), Nn, dt, w.gate_kind, _P(ws), need, None)
    assert rc == kda.KDA_OK
    rc = lib.kda_chunk_fwd_noalloc(_P(q), _P(k), _P(v), _P(g), _P(b), _P(s0), _P(o2), _P(S2), w.B, w.H, w.T, w.dk,
                                   w.dv, w.chunk, _P(cu), Nn, dt, w.gate_kind, None)
    assert rc == kda.KDA_OK
    torch.cuda.synchronize()
    assert torch.isfinite(o2).all() and torch.isfinite(S2).all()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_noalloc_matches_workspace_call_twice(kda):
    big = inputs.make_forward("noalloc_big", B=2, H=8, T=1000, dk=128, dv=128, chunk=64, gate="ckda", seed=91,
                              s0_std=0.2)
    small = inputs.make_forward("noalloc_small", B=1, H=3, T=77, dk=128, dv=64, chunk=64, gate="kda", seed=92)
    _run_both(kda, big)
    _run_both(kda, small)


def test_noalloc_varlen_and_fp32(kda):
    _run_both(kda, inputs.make_forward("noalloc_vl", B=1, H=4, T=0, dk=128, dv=128, chunk=64, gate="gdn", seed=93,
                                       lengths=[300, 0, 1, 129, 64]))
    _run_both(kda, inputs.make_forward("noalloc_f32", B=3, H=2, T=50, dk=32, dv=16, chunk=16,
                                       dtype=torch.float32, gate="ckda", seed=94, s0_std=0.1))


def test_noalloc_rejects_oversized(kda):
    lib = kda.library()
    F = ctypes.c_void_p(0x10000)
    # Complex KDA workload: 4,096 blocks of 74 KiB, well past the fixed scratch
    rc = lib.kda_chunk_fwd_noalloc(F, F, F, F, F, None, F, None, 2, 16, 8192, 128, 128, 64, None, 0, kda.KDA_BF16, 0,
                                   None)
    assert rc == kda.KDA_ESCRATCH
    assert "scratch" in kda.strerror(rc)
