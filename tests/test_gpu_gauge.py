"""GPU checks of the gauge route (kda_gauge_fold, kda_chunk_fwd_gauge)
through the C ABI: the fold bit-exact against the oracle's fold (sign and
magnitude work on exact values), and the route's o and S_T against the
oracle's direct Complex KDA run with the forward's error metric and bars
(1e-4 fp32 inputs, 2e-2 bf16 inputs)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import gauge
from gated_delta_rule_46_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


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
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(x - ref))) / rms if rms > 0 else float(np.max(np.abs(x - ref)))


def bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


FOLD_CASES = [
    ("ckda", torch.bfloat16, 128, 700, None, False),
    ("ckda", torch.float32, 64, 300, None, False),
    ("gdn", torch.bfloat16, 32, 513, None, False),
    ("ckda", torch.bfloat16, 16, 0, [260, 0, 1, 255, 40], False),
    # -0.0, +0.0 and -1.0 gates mixed in: -0.0 counts as positive (no sign
    # flip), its folded gate is +0.0, and c_T matches bit for bit
    ("ckda", torch.bfloat16, 128, 400, None, True),
    ("ckda", torch.float32, 32, 0, [100, 1, 0, 77], True),
    ("gdn", torch.bfloat16, 64, 333, None, True),
    ("gdn", torch.float32, 16, 129, None, True),
]


@pytest.mark.parametrize("gate,dtype,dk,T,lengths,szero", FOLD_CASES)
def test_fold_bit_exact(kda, gate, dtype, dk, T, lengths, szero):
    w = inputs.make_forward("fold", B=1 if lengths else 2, H=3, T=T, dk=dk, dv=16, dtype=dtype, gate=gate,
                            lengths=lengths, seed=T + dk)
    if gate == "gdn":   # make the scalar gates signed: flip every third token's sign
        g = w.gate.clone()
        g[:, ::3] = -g[:, ::3]
        w.gate = g
    if szero:
        w.gate = inputs.signed_zero_gates(w.gate, seed=T, frac=0.06 if gate == "ckda" else 0.3)
        negz = (w.gate.view(torch.int16 if dtype == torch.bfloat16 else torch.int32) ==
                (-32768 if dtype == torch.bfloat16 else -2 ** 31))
        assert int(negz.sum()) > 0
    print("case", gate, dtype, "dk", dk, "T", w.T, "lengths", lengths, "signed zeros", szero, flush=True)
    d = lambda t: None if t is None else t.cuda()  # noqa: E731
    qo, ko, go, sign = kda.gauge_fold(d(w.q), d(w.k), d(w.gate), cu_seqlens=d(w.cu_seqlens), gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    rq, rk, rg, rc = gauge.fold(w.q, w.k, w.gate, w.cu_seqlens, w.gate_kind)
    np.testing.assert_array_equal(bits(qo), bits(rq))
    np.testing.assert_array_equal(bits(ko), bits(rk))
    np.testing.assert_array_equal(bits(go), bits(rg))
    np.testing.assert_array_equal(sign.cpu().numpy().reshape(rc.shape), rc)
    if szero:   # every folded gate is non-negative, -0.0 included (it becomes +0.0)
        assert not bool(torch.signbit(go.cpu()).any())


ROUTE_CASES = [
    ("ckda", torch.bfloat16, 128, 128, 64, 300),
    ("ckda", torch.float32, 64, 32, 32, 100),
    ("kda", torch.bfloat16, 128, 64, 64, 129),
]


@pytest.mark.parametrize("gate,dtype,dk,dv,chunk,T", ROUTE_CASES)
def test_gauge_route_parity(kda, gate, dtype, dk, dv, chunk, T):
    w = inputs.make_forward("route", B=2, H=2, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype, gate=gate, seed=T,
                            s0_std=0.3)
    print("case route", gate, dtype, dk, dv, chunk, T, flush=True)
    d = lambda t: None if t is None else t.cuda()  # noqa: E731
    o, ST = kda.chunk_fwd_gauge(d(w.q), d(w.k), d(w.v), d(w.gate), d(w.beta), S0=d(w.S0), chunk=chunk,
                                gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0, None, w.gate_kind)
    eo, eS = err(o, ro), err(ST, rS)
    print("  err o %.2e S %.2e" % (eo, eS), flush=True)
    assert eo <= TOL[dtype] and eS <= TOL[dtype]


def test_gauge_route_varlen_scalar(kda):
    w = inputs.make_forward("route_vl", B=1, H=2, T=0, dk=64, dv=64, chunk=32, dtype=torch.float32, gate="gdn",
                            lengths=[70, 0, 33, 300], s0_std=0.2, seed=4)
    g = w.gate.clone()
    g[:, 1::4] = -g[:, 1::4]
    w.gate = g
    d = lambda t: None if t is None else t.cuda()  # noqa: E731
    o, ST = kda.chunk_fwd_gauge(d(w.q), d(w.k), d(w.v), d(w.gate), d(w.beta), S0=d(w.S0), cu_seqlens=d(w.cu_seqlens),
                                chunk=32, gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0, w.cu_seqlens, w.gate_kind)
    assert err(o, ro) <= 1e-4 and err(ST, rS) <= 1e-4


def test_gauge_route_full_size_every_head(kda):
    """The Complex KDA workload (with -0.0 gates mixed in) through the gauge
    route; the oracle runs every (sequence, head) pair directly over all 8192
    tokens, and each head is checked on its own."""
    w = inputs.ckda_fwd(seed=0)
    w.gate = inputs.signed_zero_gates(w.gate, seed=5, frac=0.015)
    d = lambda t: t.cuda()  # noqa: E731
    o, ST = kda.chunk_fwd_gauge(d(w.q), d(w.k), d(w.v), d(w.gate), d(w.beta), chunk=64)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta)
    eo, eS = err(o, ro), err(ST, rS)
    worst = max(max(err(o[:, :, h], ro[:, :, h]), err(ST[:, h], rS[:, h])) for h in range(w.H))
    print("  full size err o %.2e S %.2e worst head %.2e" % (eo, eS, worst), flush=True)
    assert eo <= 2e-2 and eS <= 2e-2 and worst <= 2e-2
