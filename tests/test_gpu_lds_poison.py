"""The LDS-poisoning debug build (libkda_lds_poison.so: the same sources built
with KDA_LDS_POISON, so that every kernel fills its workgroup's LDS with
0xFFFFFFFF -- NaN as fp32, fp16 and bf16 -- before its own code) against the
fp64 oracle: one case per kernel and launch shape. A kernel that read LDS it
had not written first would carry NaN into its results here. Same bars as
the normal build's parity tests; the calls go through the same binding, with
its library switched to the debug build for this module."""
import os

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_46_amd import inputs

import test_gpu_bwd as tok_bwd
import test_gpu_cbwd as cw_bwd
import test_gpu_ew as ew
import test_gpu_parity as par

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_46_amd import build
    from gated_delta_rule_46_amd import kda as m
    assert os.path.exists(build.POISON_LIB), "the LDS-poisoning build is missing (__graft_entry__.build() makes it)"
    with m.using_library(build.POISON_LIB) as lib:
        assert lib._name == build.POISON_LIB
        yield m


FWD = [
    # gate, dtype, dk, dv, chunk, B, H, T -- the state walker each shape takes
    ("ckda", BF16, 128, 128, 64, 1, 2, 300),   # one slice per workgroup, operands in registers
    ("kda", BF16, 128, 128, 64, 4, 16, 130),   # two slices per workgroup, staged in LDS (512 slices)
    ("gdn", BF16, 128, 16, 64, 2, 160, 70),    # one slice per workgroup, staged in LDS (320 slices)
    ("ckda", BF16, 64, 64, 64, 2, 3, 150),     # two waves per slice (dk = 64)
    ("kda", F32, 128, 64, 64, 2, 2, 100),      # one wave per slice, fp32 inputs
    ("ckda", BF16, 32, 16, 16, 2, 3, 45),      # one wave per slice, chunk 16
]


@pytest.mark.parametrize("gate,dtype,dk,dv,chunk,B,H,T", FWD)
def test_poisoned_forward(kda, gate, dtype, dk, dv, chunk, B, H, T):
    w = inputs.make_forward("poison_%s" % gate, B=B, H=H, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype, gate=gate,
                            seed=T + dv, s0_std=0.2)
    par.check(kda, w)


def test_poisoned_forward_varlen(kda):
    w = inputs.make_forward("poison_varlen", B=1, H=2, T=0, dk=128, dv=128, chunk=64, gate="gdn",
                            lengths=[130, 0, 1, 64, 77], s0_std=0.1, seed=9)
    par.check(kda, w)


def test_poisoned_erase_write_forward(kda):
    w = inputs.make_forward("poison_ew", B=2, H=3, T=200, dk=128, dv=128, chunk=64, gate="ckda", seed=4,
                            s0_std=0.3)
    ew.check(kda, inputs.erase_write_gates(w, seed=4))


@pytest.mark.parametrize("gate_kind", [0, 1])
def test_poisoned_decode(kda, gate_kind):
    dw = inputs.ckda_decode(N=4, H=2, d=128, n_steps=3)
    S = dw.S.cuda()
    Sr = dw.S.double().numpy().copy()
    for st in dw.steps:
        g = st["gate"] if gate_kind == 0 else st["gate"][..., 0].contiguous()
        o = kda.decode_step(*(x.cuda() for x in (st["q"], st["k"], st["v"], g, st["beta"])), S,
                            gate_kind=gate_kind)
        ro = oracle.decode_step(st["q"], st["k"], st["v"], g, st["beta"], Sr, gate_kind=gate_kind)
        torch.cuda.synchronize()
        assert np.isfinite(o.cpu().numpy()).all()
        assert par.err(o.cpu(), ro) <= 2e-2
    assert par.err(S.cpu(), Sr) <= 2e-2


@pytest.mark.parametrize("gate,dtype,dk,dv,T", [("ckda", BF16, 128, 128, 77), ("gdn", F32, 64, 32, 130)])
def test_poisoned_chunkwise_backward(kda, gate, dtype, dk, dv, T):
    w = inputs.make_forward("poison_cbwd", B=2, H=3, T=T, dk=dk, dv=dv, dtype=dtype, gate=gate, gate_mu=2.0,
                            seed=T, s0_std=0.3)
    cw_bwd.check(kda, w)


def test_poisoned_token_backward(kda):
    w = inputs.make_forward("poison_bwd", B=2, H=3, T=70, dk=32, dv=16, dtype=BF16, gate="ckda", seed=7,
                            s0_std=0.3)
    tok_bwd.check(kda, w)


def test_poisoned_erase_write_backward(kda):
    w = inputs.make_forward("poison_bwd_ew", B=2, H=3, T=70, dk=128, dv=32, dtype=BF16, gate="ckda", seed=8,
                            s0_std=0.3)
    ew.check_bwd(kda, inputs.erase_write_gates(w, seed=8))


def test_poisoned_gauge_route(kda):
    w = inputs.make_forward("poison_route", B=2, H=2, T=129, dk=128, dv=64, chunk=64, gate="ckda", seed=5,
                            s0_std=0.3)
    o, ST = kda.chunk_fwd_gauge(w.q.cuda(), w.k.cuda(), w.v.cuda(), w.gate.cuda(), w.beta.cuda(), S0=w.S0.cuda(),
                                chunk=64, gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0, None, w.gate_kind)
    assert np.isfinite(o.cpu().numpy()).all()
    assert par.err(o.cpu(), ro) <= 2e-2 and par.err(ST.cpu(), rS) <= 2e-2
