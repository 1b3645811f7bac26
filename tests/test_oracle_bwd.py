"""Pins for the fp64 oracle's gradient (``oracle.bwd``).

The gradient is fixed by the forward recurrence alone: it is the derivative of
L = sum_t <o_t, dO_t> + <S_T, dS_T>. Central finite differences of the
(separately pinned) forward oracle check every component on tiny inputs,
including negative and exactly zero gates, beta up to 2, non-zero initial
states, the scalar gate and packed variable-length input with an empty
sequence. L is linear in each single gate, beta, v, q and S0 entry and
quadratic in each k entry, so central differences are exact up to rounding
for every component. A closed form for the frozen state (alpha = 1, beta = 0)
checks the assembled gradients directly.
"""
import numpy as np
import pytest
import torch

import oracle


def _inputs(rng, B, T, H, dk, dv, gate_kind, lengths=None):
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    gshape = (B, T, H, dk) if gate_kind == 0 else (B, T, H)
    g = rng.uniform(-1, 1, gshape)
    flat = g.reshape(-1)
    flat[rng.choice(flat.size, max(1, flat.size // 10), replace=False)] = 0.0
    flat[rng.choice(flat.size, max(1, flat.size // 10), replace=False)] = -1.0
    b = rng.uniform(0, 2, (B, T, H))
    b.reshape(-1)[rng.integers(0, b.size)] = 2.0
    nseq = B if lengths is None else len(lengths)
    S0 = rng.standard_normal((nseq, H, dk, dv))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((nseq, H, dk, dv))
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return dict(q=q, k=k, v=v, gate=g, beta=b, S0=S0), dO, dST, cu


def _loss(x, dO, dST, cu, gate_kind):
    o, ST = oracle.fwd(*(torch.from_numpy(x[n]) for n in ("q", "k", "v", "gate", "beta")),
                       torch.from_numpy(x["S0"]), cu, gate_kind)
    return float((o * dO).sum() + (ST * dST).sum())


CASES = [
    dict(B=2, T=6, H=2, dk=3, dv=2, gate_kind=0),
    dict(B=1, T=7, H=1, dk=4, dv=3, gate_kind=1),
    dict(B=1, T=0, H=2, dk=3, dv=2, gate_kind=0, lengths=[4, 0, 3]),
]


@pytest.mark.parametrize("case", CASES, ids=["channel", "scalar", "varlen"])
def test_gradient_equals_finite_differences(case):
    case = dict(case)
    gk = case["gate_kind"]
    rng = np.random.default_rng(11 + gk)
    x, dO, dST, cu = _inputs(rng, case["B"], case["T"], case["H"], case["dk"], case["dv"], gk,
                             case.get("lengths"))
    g = oracle.bwd(*(torch.from_numpy(x[n]) for n in ("q", "k", "v", "gate", "beta")), torch.from_numpy(dO),
                   torch.from_numpy(x["S0"]), torch.from_numpy(dST), cu, gk)
    h = 1e-5
    names = {"q": "dq", "k": "dk", "v": "dv", "gate": "dgate", "beta": "dbeta", "S0": "dS0"}
    for name, gname in names.items():
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            keep = x[name][idx]
            x[name][idx] = keep + h
            lp = _loss(x, dO, dST, cu, gk)
            x[name][idx] = keep - h
            lm = _loss(x, dO, dST, cu, gk)
            x[name][idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(g[gname], num, rtol=0, atol=1e-8 * scale, err_msg=name)


def test_frozen_state_closed_form():
    """alpha = 1, beta = 0: S_t = S0 for every t, so o_t = S0^T q_t and
    S_T = S0. Then dq_t = S0 dO_t, dS0 = dS_T + sum_t q_t dO_t^T, dv = 0,
    dk_t = 0 (u = 0 and dpred = 0), dbeta_t = (v_t - S0^T k_t) . (D_t^T k_t)
    with D_t = dS_T + sum_{s >= t} q_s dO_s^T, and dalpha_t[i] =
    sum_j D_t[i, j] S0[i, j]."""
    rng = np.random.default_rng(5)
    T, dk, dv = 9, 5, 4
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    dO = rng.standard_normal((1, T, 1, dv))
    dST = rng.standard_normal((1, 1, dk, dv))
    g = oracle.bwd(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), torch.ones(1, T, 1, dk,
                   dtype=torch.float64), torch.zeros(1, T, 1, dtype=torch.float64), torch.from_numpy(dO),
                   torch.from_numpy(S0), torch.from_numpy(dST))
    s0 = S0[0, 0]
    D = dST[0, 0].copy()
    for t in range(T - 1, -1, -1):
        D = D + np.outer(q[0, t, 0], dO[0, t, 0])
        np.testing.assert_allclose(g["dq"][0, t, 0], s0 @ dO[0, t, 0], atol=1e-12)
        np.testing.assert_allclose(g["dbeta"][0, t, 0], (v[0, t, 0] - s0.T @ k[0, t, 0]) @ (D.T @ k[0, t, 0]),
                                   atol=1e-11)
        np.testing.assert_allclose(g["dgate"][0, t, 0], (D * s0).sum(axis=1), atol=1e-11)
    np.testing.assert_allclose(g["dS0"][0, 0], D, atol=1e-12)
    assert np.all(g["dv"] == 0) and np.all(g["dk"] == 0)


def test_scalar_gate_is_sum_of_channel_gradients():
    """A scalar gate equals the same value broadcast over the channels, so its
    gradient is the sum over channels of the channel-gate gradient."""
    rng = np.random.default_rng(8)
    x, dO, dST, _ = _inputs(rng, 2, 10, 2, 6, 5, 1)
    t = {n: torch.from_numpy(x[n]) for n in x}
    g1 = oracle.bwd(t["q"], t["k"], t["v"], t["gate"], t["beta"], torch.from_numpy(dO), t["S0"],
                    torch.from_numpy(dST), None, 1)
    gb = t["gate"][..., None].expand(2, 10, 2, 6).contiguous()
    g0 = oracle.bwd(t["q"], t["k"], t["v"], gb, t["beta"], torch.from_numpy(dO), t["S0"], torch.from_numpy(dST),
                    None, 0)
    np.testing.assert_allclose(g1["dgate"], g0["dgate"].sum(-1), atol=1e-12)
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        np.testing.assert_allclose(g1[n], g0[n], atol=1e-12)


def test_one_token_state_gradient_closed_form():
    """One token: S_1 = Diag(alpha)S0 + beta k (v - S0^T Diag(alpha) k)^T and
    o = S_1^T q, so dS0 = Diag(alpha)(D - beta k (D^T k)^T) with
    D = dS_T + q dO^T. Dropping the delta-term correction (a plausible slip in
    an adjoint) changes dS0 by far more than rounding."""
    rng = np.random.default_rng(3)
    x, dO, dST, _ = _inputs(rng, 1, 1, 1, 4, 3, 0)
    g = oracle.bwd(*(torch.from_numpy(x[n]) for n in ("q", "k", "v", "gate", "beta")), torch.from_numpy(dO),
                   torch.from_numpy(x["S0"]), torch.from_numpy(dST), None, 0)
    k0, a0, b0 = x["k"][0, 0, 0], x["gate"][0, 0, 0], x["beta"][0, 0, 0]
    D = dST[0, 0] + np.outer(x["q"][0, 0, 0], dO[0, 0, 0])
    right = a0[:, None] * (D - b0 * np.outer(k0, D.T @ k0))
    np.testing.assert_allclose(g["dS0"][0, 0], right, atol=1e-12)
    planted = a0[:, None] * D
    assert np.abs(planted - right).max() > 1e-3


# ------------------------------------------------------------------ erase/write gates (oracle.bwd_ew)

def _ew_inputs(rng, B, T, H, dk, dv, gate_kind, lengths=None):
    x, dO, dST, cu = _inputs(rng, B, T, H, dk, dv, gate_kind, lengths)
    B, T = x["q"].shape[:2]
    x = {n: x[n] for n in ("q", "k", "v", "gate", "S0")}
    x["erase"] = rng.uniform(-0.5, 2.0, (B, T, H, dk))    # negative, zero-crossing and above-one erase entries
    x["write"] = rng.uniform(-0.5, 2.0, (B, T, H, dv))
    x["erase"].reshape(-1)[rng.integers(0, x["erase"].size)] = 0.0
    return x, dO, dST, cu


def _ew_loss(x, dO, dST, cu, gate_kind):
    o, ST = oracle.fwd_ew(*(torch.from_numpy(x[n]) for n in ("q", "k", "v", "gate", "erase", "write")),
                          torch.from_numpy(x["S0"]), cu, gate_kind)
    return float((o * dO).sum() + (ST * dST).sum())


@pytest.mark.parametrize("case", CASES, ids=["channel", "scalar", "varlen"])
def test_erase_write_gradient_equals_finite_differences(case):
    """Every component of oracle.bwd_ew against central differences of the
    (separately pinned) oracle.fwd_ew. L is affine in each single q, v, gate,
    erase, write and S0 entry and quadratic in each k entry (k reads through
    e o k and writes along k), so central differences are exact up to
    rounding."""
    case = dict(case)
    gk = case["gate_kind"]
    rng = np.random.default_rng(21 + gk)
    x, dO, dST, cu = _ew_inputs(rng, case["B"], case["T"], case["H"], case["dk"], case["dv"], gk,
                                case.get("lengths"))
    g = oracle.bwd_ew(*(torch.from_numpy(x[n]) for n in ("q", "k", "v", "gate", "erase", "write")),
                      torch.from_numpy(dO), torch.from_numpy(x["S0"]), torch.from_numpy(dST), cu, gk)
    h = 1e-5
    names = {"q": "dq", "k": "dk", "v": "dv", "gate": "dgate", "erase": "derase", "write": "dwrite", "S0": "dS0"}
    for name, gname in names.items():
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            keep = x[name][idx]
            x[name][idx] = keep + h
            lp = _ew_loss(x, dO, dST, cu, gk)
            x[name][idx] = keep - h
            lm = _ew_loss(x, dO, dST, cu, gk)
            x[name][idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(g[gname], num, rtol=0, atol=1e-8 * scale, err_msg=name)


def test_erase_write_gradient_reduces_to_beta_form():
    """With e = beta 1 (every key channel) and w = beta 1 (every value channel)
    the erase/write recurrence is the beta recurrence, so dq, dk, dv, dgate
    and dS0 equal oracle.bwd's, and by the chain rule dbeta = sum over
    channels of derase plus sum over channels of dwrite."""
    rng = np.random.default_rng(13)
    x, dO, dST, _ = _inputs(rng, 2, 9, 2, 5, 4, 0)
    t = {n: torch.from_numpy(x[n]) for n in x}
    b = t["beta"]
    e = b[..., None].expand(*b.shape, 5).contiguous()
    w = b[..., None].expand(*b.shape, 4).contiguous()
    gb = oracle.bwd(t["q"], t["k"], t["v"], t["gate"], b, torch.from_numpy(dO), t["S0"], torch.from_numpy(dST))
    ge = oracle.bwd_ew(t["q"], t["k"], t["v"], t["gate"], e, w, torch.from_numpy(dO), t["S0"],
                       torch.from_numpy(dST))
    for n in ("dq", "dk", "dv", "dgate", "dS0"):
        np.testing.assert_allclose(ge[n], gb[n], atol=1e-11, err_msg=n)
    np.testing.assert_allclose(ge["derase"].sum(-1) + ge["dwrite"].sum(-1), gb["dbeta"], atol=1e-11)
