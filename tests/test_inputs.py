"""The seeded generators produce the documented shapes, ranges and stress
patterns (no GPU)."""
import numpy as np
import torch

from gated_delta_rule_46_amd import inputs


def test_varlen_lengths_seed0():
    assert inputs.varlen_lengths(0) == [28485, 22359, 18751, 11831, 12922, 5270, 6253, 4569]


def test_tiny_shapes_and_dtype():
    w = inputs.tiny_kda()
    assert w.q.shape == (1, 64, 1, 16) and w.q.dtype == torch.float32
    assert w.gate.shape == (1, 64, 1, 16) and w.beta.shape == (1, 64, 1)
    assert w.S0 is None and w.chunk == 16
    n = w.k.double().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-6)
    assert (w.gate > 0).all() and (w.gate < 1).all()


def test_ckda_ranges_and_masks():
    w = inputs.make_forward("c", B=2, H=4, T=2048, dk=128, dv=128, gate="ckda")
    g = w.gate.float()
    assert w.gate.dtype == torch.bfloat16
    assert g.min() >= -1 and g.max() <= 1
    zf = (g == 0).float().mean().item()
    mf = (g == -1).float().mean().item()
    assert 0.003 < zf < 0.008 and 0.003 < mf < 0.008
    b = w.beta.float()
    assert b.min() >= 0 and b.max() <= 2
    assert 0.005 < (b == 2).float().mean().item() < 0.02
    # spread init: about half of the (head, channel) signs are negative,
    # shared over batch and time
    neg = (g < 0).float().mean(dim=(0, 1))
    assert 0.3 < (neg > 0.5).float().mean().item() < 0.7


def test_gdn_varlen_shape():
    w = inputs.gdn_varlen(lengths=[100, 37, 250])
    assert w.B == 1 and w.T == 387 and w.gate.shape == (1, 387, 32)
    assert w.cu_seqlens.tolist() == [0, 100, 137, 387]
    assert w.gate_kind == inputs.GATE_SCALAR


def test_decode_shapes():
    d = inputs.ckda_decode(N=4, H=2, d=16, n_steps=3)
    assert d.S.shape == (4, 2, 16, 16) and d.S.dtype == torch.float32
    assert len(d.steps) == 3 and d.steps[0]["q"].shape == (4, 2, 16)
    assert abs(d.S.std().item() - 0.01) < 0.002


def test_seeded_determinism():
    a = inputs.kda_fwd(B=1, H=2, T=64)
    b = inputs.kda_fwd(B=1, H=2, T=64)
    assert torch.equal(a.q, b.q) and torch.equal(a.gate, b.gate)
    c = inputs.kda_fwd(seed=1, B=1, H=2, T=64)
    assert not torch.equal(a.q, c.q)
    assert np.isfinite(a.v.float().numpy()).all()
