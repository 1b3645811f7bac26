"""Pins for the fp64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: closed forms
from the Complex KDA summary, textbook special cases (linear attention and the
ungated delta rule from the CyFA blog post, section 2), invariants (norm bound,
eigenvalue count, gauge identity, sequence splitting) and a second dense
formulation on tiny inputs. A plausible slip in the oracle -- a dropped term,
the gate applied after the delta term, a transposed state, a wrong sign --
fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t(x):
    return torch.from_numpy(np.array(x, dtype=np.float64, copy=True))


def run1(q, k, v, a, b, S0=None, gate_kind=0):
    """Oracle on one sequence, one head. Shapes [T,dk] etc."""
    T, dk = k.shape
    dv = v.shape[1]
    g = a[None, :, None] if a.ndim == 2 else a[None, :, None]
    o, S = oracle.fwd(_t(q[None, :, None]), _t(k[None, :, None]), _t(v[None, :, None]), _t(g),
                      _t(b[None, :, None]), None if S0 is None else _t(S0[None, None]),
                      gate_kind=gate_kind)
    return o[0, :, 0], S[0, 0]


def oracle_transition(k, alpha, beta):
    """The oracle's one-token transition read off as a matrix: start from
    S0 = I (dv = dk), v = 0, one token; then S_1 = A S0 = A."""
    dk = k.size
    a = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (dk,))
    _, S = run1(np.zeros((1, dk)), k[None], np.zeros((1, dk)), a[None], np.array([beta]),
                S0=np.eye(dk))
    return S


def unit(rng, d):
    x = rng.standard_normal(d)
    return x / np.linalg.norm(x)


# ------------------------------------------------------------------ second formulation

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("gate_kind", [0, 1])
def test_dense_products_agree(seed, gate_kind):
    """Token recurrence == explicit products of dense transitions (tiny)."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 9, 5, 4
    q = rng.standard_normal((T, dk))
    k = np.stack([unit(rng, dk) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, dk) if gate_kind == 0 else (T,))
    a.flat[rng.integers(0, a.size, 3)] = 0.0   # exact zero gates
    a.flat[rng.integers(0, a.size, 2)] = -1.0
    b = rng.uniform(0, 2, T)
    b[rng.integers(0, T)] = 2.0
    S0 = rng.standard_normal((dk, dv))
    o1, S1 = run1(q, k, v, a, b, S0, gate_kind=gate_kind)
    o2, S2 = dense.run(q, k, v, a, b, S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ Householder special cases

def test_householder_beta_cases():
    """Unit k: beta=0 identity, beta=1 projection, beta=2 exact reflection
    (Complex KDA summary, background: delta rule and Householder reflection)."""
    rng = np.random.default_rng(3)
    d = 6
    k = unit(rng, d)
    one = np.ones(d)
    A0 = oracle_transition(k, one, 0.0)
    np.testing.assert_allclose(A0, np.eye(d), atol=1e-14)
    A1 = oracle_transition(k, one, 1.0)
    np.testing.assert_allclose(A1 @ A1, A1, atol=1e-14)          # idempotent
    np.testing.assert_allclose(A1 @ k, np.zeros(d), atol=1e-14)  # removes the k component
    A2 = oracle_transition(k, one, 2.0)
    np.testing.assert_allclose(A2 @ A2, np.eye(d), atol=1e-14)   # involution
    np.testing.assert_allclose(A2 @ k, -k, atol=1e-14)           # flips k
    w = unit(rng, d)
    w -= (w @ k) * k
    np.testing.assert_allclose(A2 @ w, w, atol=1e-14)            # fixes k-perp


def test_gate_then_delta_order_commutator():
    """The transition is (I - beta k k^T) Diag(alpha): gate first. The two
    orders differ by the commutator beta k_i k_j (alpha_i - alpha_j)
    (Complex KDA summary, motivation), which is non-zero for a channel gate."""
    rng = np.random.default_rng(4)
    d = 5
    k = unit(rng, d)
    alpha = rng.uniform(-1, 1, d)
    beta = 1.3
    A = oracle_transition(k, alpha, beta)
    H = np.eye(d) - beta * np.outer(k, k)
    D = np.diag(alpha)
    np.testing.assert_allclose(A, H @ D, atol=1e-14)
    comm = beta * np.outer(k, k) * (alpha[:, None] - alpha[None, :])
    np.testing.assert_allclose(A - D @ H, comm, atol=1e-14)
    assert np.abs(comm).max() > 1e-2
    # scalar gate: the two orders agree
    As = oracle_transition(k, np.full(d, 0.7), beta)
    np.testing.assert_allclose(As, np.diag(np.full(d, 0.7)) @ H, atol=1e-14)


# ------------------------------------------------------------------ 2-D rotation construction

def _golden_rotation():
    rows = []
    with open(os.path.join(GOLDEN, "rotation_2d.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return rows


@pytest.mark.parametrize("row", _golden_rotation())
def test_rotation_2d_golden(row):
    """2-D construction of the Complex KDA summary (core method): entries,
    discriminant and eigenvalue modulus of A = (I - 2 k k^T) Diag(alpha, 1)."""
    t_over_pi, alpha, beta, a11, a12, a21, a22, disc, modulus = row
    t = t_over_pi * math.pi
    k = np.array([math.cos(t), math.sin(t)])
    A = oracle_transition(k, np.array([alpha, 1.0]), beta)
    np.testing.assert_allclose(A, [[a11, a12], [a21, a22]], atol=1e-13)
    assert math.isclose((1 - alpha) ** 2 * math.cos(2 * t) ** 2 + 4 * alpha, disc, abs_tol=1e-13)
    ev = np.linalg.eigvals(A)
    if modulus < 0:
        assert np.all(np.abs(ev.imag) < 1e-12)
    else:
        assert np.all(np.abs(ev.imag) > 1e-6)
        np.testing.assert_allclose(np.abs(ev), [modulus, modulus], atol=1e-12)


@pytest.mark.parametrize("d", [2, 4, 16])
def test_rotation_sequence_returns(d):
    """alpha = (-1, 1, ...), beta = 2, k = (cos t, sin t, 0...), v = 0: each
    token rotates the top two state rows by 2t; with t = pi/8 eight tokens
    return the state exactly (Complex KDA summary, core method)."""
    t = math.pi / 8
    T, dv = 8, 3
    k = np.zeros((T, d))
    k[:, 0], k[:, 1] = math.cos(t), math.sin(t)
    a = np.ones((T, d))
    a[:, 0] = -1.0
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((d, dv))
    q = rng.standard_normal((T, d))
    o, S = run1(q, k, np.zeros((T, dv)), a, np.full(T, 2.0), S0)
    np.testing.assert_allclose(S, S0, atol=1e-13)
    R = np.array([[math.cos(2 * t), -math.sin(2 * t)], [math.sin(2 * t), math.cos(2 * t)]])
    # after the first token: o_0 = S_1^T q_0 with S_1 = R S0 on rows 0, 1
    S1 = S0.copy()
    S1[:2] = R @ S0[:2]
    np.testing.assert_allclose(o[0], S1.T @ q[0], atol=1e-13)


@pytest.mark.parametrize("seed", range(20))
def test_complex_pair_modulus_general_beta(seed):
    """2-D, alpha < 0: det A = alpha (1 - beta), so a complex pair has modulus
    sqrt(-alpha (beta - 1)); it is complex exactly when the discriminant is
    negative (at beta = 2 this is the summary's sqrt(-alpha))."""
    rng = np.random.default_rng(seed)
    alpha = -rng.uniform(0.05, 1.0)
    beta = rng.uniform(1.0, 2.0)
    t = rng.uniform(0, math.pi)
    k = np.array([math.cos(t), math.sin(t)])
    A = oracle_transition(k, np.array([alpha, 1.0]), beta)
    tr, det = np.trace(A), np.linalg.det(A)
    assert math.isclose(det, alpha * (1 - beta), abs_tol=1e-13)
    ev = np.linalg.eigvals(A)
    if tr * tr - 4 * det < -1e-9:
        np.testing.assert_allclose(np.abs(ev), math.sqrt(-alpha * (beta - 1)), atol=1e-12)
    if beta == 2.0:
        assert math.isclose(tr * tr - 4 * det, (1 - alpha) ** 2 * math.cos(2 * t) ** 2 + 4 * alpha,
                            abs_tol=1e-12)


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("seed", range(30))
def test_nonexpansive_and_one_complex_pair(seed):
    """For unit k, alpha in [-1, 1], beta in [0, 2]: ||A||_2 <= 1 and at most
    one conjugate pair of non-real eigenvalues (Complex KDA summary, core
    method and method step 3)."""
    rng = np.random.default_rng(100 + seed)
    d = int(rng.integers(2, 9))
    k = unit(rng, d)
    alpha = rng.uniform(-1, 1, d)
    beta = rng.uniform(0, 2) if seed % 3 else 2.0
    A = oracle_transition(k, alpha, beta)
    assert np.linalg.norm(A, 2) <= 1 + 1e-12
    ev = np.linalg.eigvals(A)
    assert np.sum(np.abs(ev.imag) > 1e-9) <= 2


def test_state_norm_nonincreasing_without_writes():
    """With v = 0 the state only passes through non-expansive transitions, so
    its Frobenius norm never grows."""
    rng = np.random.default_rng(6)
    T, d = 64, 8
    k = np.stack([unit(rng, d) for _ in range(T)])
    a = rng.uniform(-1, 1, (T, d))
    b = rng.uniform(0, 2, T)
    S = rng.standard_normal((d, 3))
    prev = np.linalg.norm(S)
    for t in range(T):
        _, S = run1(np.zeros((1, d)), k[t:t + 1], np.zeros((1, 3)), a[t:t + 1], b[t:t + 1], S)
        n = np.linalg.norm(S)
        assert n <= prev * (1 + 1e-13)
        prev = n


# ------------------------------------------------------------------ textbook special cases

def test_frozen_state_beta0_alpha1():
    """beta = 0, alpha = 1: the transition is the identity and nothing is
    written, so S_t = S0 and o_t = S0^T q_t."""
    rng = np.random.default_rng(7)
    T, dk, dv = 20, 6, 5
    q = rng.standard_normal((T, dk))
    k = np.stack([unit(rng, dk) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((dk, dv))
    o, S = run1(q, k, v, np.ones((T, dk)), np.zeros(T), S0)
    np.testing.assert_allclose(S, S0, atol=0)
    np.testing.assert_allclose(o, q @ S0, atol=1e-13)


def test_linear_attention_orthogonal_keys():
    """alpha = 1, mutually orthogonal keys, S0 = 0: the delta term never sees a
    previous write, so S_T = sum_t beta_t k_t v_t^T; with beta = 1 this is
    linear attention's S_t = S_{t-1} + k_t v_t^T (CyFA blog post, 2.1)."""
    rng = np.random.default_rng(8)
    dk, dv = 8, 5
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q.T                                   # T = dk orthonormal keys
    T = dk
    v = rng.standard_normal((T, dv))
    q = rng.standard_normal((T, dk))
    b = rng.uniform(0.1, 2.0, T)
    _, S = run1(q, k, v, np.ones((T, dk)), b)
    np.testing.assert_allclose(S, np.einsum("t,ti,tj->ij", b, k, v), atol=1e-13)
    o, S = run1(q, k, v, np.ones((T, dk)), np.ones(T))
    lin = np.cumsum(np.einsum("ti,tj->tij", k, v), axis=0)
    np.testing.assert_allclose(S, lin[-1], atol=1e-13)
    np.testing.assert_allclose(o, np.einsum("tij,ti->tj", lin, q), atol=1e-13)


def test_ungated_delta_rule_step():
    """alpha = 1, beta = 1 is the plain delta rule
    S_t = S_{t-1} + k_t (v_t - S_{t-1}^T k_t)^T (CyFA blog post, 2.2); a unit
    key then retrieves exactly: S_t^T k_t = v_t."""
    rng = np.random.default_rng(9)
    dk, dv, T = 7, 4, 12
    S = rng.standard_normal((dk, dv))
    for t in range(T):
        k = unit(rng, dk)
        v = rng.standard_normal(dv)
        o, S_new = run1(k[None], k[None], v[None], np.ones((1, dk)), np.ones(1), S)
        np.testing.assert_allclose(S_new, S + np.outer(k, v - S.T @ k), atol=1e-13)
        np.testing.assert_allclose(o[0], v, atol=1e-13)      # q = k reads v back
        S = S_new


def test_zero_gate_cuts_history():
    """A token whose gate is 0 in every channel erases the state, so later
    outputs do not depend on anything before it."""
    rng = np.random.default_rng(10)
    T, dk, dv, cut = 24, 6, 4, 11
    q = rng.standard_normal((T, dk))
    k = np.stack([unit(rng, dk) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, dk))
    a[cut] = 0.0
    a[cut, ::2] = -0.0
    b = rng.uniform(0, 2, T)
    o1, S1 = run1(q, k, v, a, b, rng.standard_normal((dk, dv)))
    k2, v2, a2, b2 = k.copy(), v.copy(), a.copy(), b.copy()
    k2[:cut] = np.stack([unit(rng, dk) for _ in range(cut)])
    v2[:cut] = rng.standard_normal((cut, dv))
    a2[:cut] = rng.uniform(-1, 1, (cut, dk))
    b2[:cut] = rng.uniform(0, 2, cut)
    o2, S2 = run1(q, k2, v2, a2, b2, None)
    np.testing.assert_array_equal(o1[cut:], o2[cut:])
    np.testing.assert_array_equal(S1, S2)


# ------------------------------------------------------------------ structural identities

def test_gauge_identity():
    """Cumulative gate signs absorbed into q and k give a positive-gate run
    with the same outputs and a sign-flipped state (Complex KDA summary,
    method step 5): with c_t = prod_{s<=t} sign(alpha_s) (sign(0) = +1),
    CKDA(q, k, alpha) = KDA(c*q, c*k, |alpha|) and S_T = Diag(c_T) S~_T."""
    rng = np.random.default_rng(11)
    T, dk, dv = 40, 6, 5
    q = rng.standard_normal((T, dk))
    k = np.stack([unit(rng, dk) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, dk))
    a[5, 2] = 0.0
    a[9, 1] = -1.0
    b = rng.uniform(0, 2, T)
    o1, S1 = run1(q, k, v, a, b)
    c = np.cumprod(np.where(a < 0, -1.0, 1.0), axis=0)
    o2, S2 = run1(c * q, c * k, v, np.abs(a), b)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(S1, c[-1][:, None] * S2, atol=1e-13)


def test_split_resume_equals_one_pass():
    """Running T1 tokens, handing S_T on as S0, then the rest equals one pass."""
    rng = np.random.default_rng(12)
    T, dk, dv = 50, 6, 4
    q = rng.standard_normal((T, dk))
    k = np.stack([unit(rng, dk) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, dk))
    b = rng.uniform(0, 2, T)
    S0 = rng.standard_normal((dk, dv))
    o, S = run1(q, k, v, a, b, S0)
    for cut in (1, 17, 33, 49):
        oa, Sa = run1(q[:cut], k[:cut], v[:cut], a[:cut], b[:cut], S0)
        ob, Sb = run1(q[cut:], k[cut:], v[cut:], a[cut:], b[cut:], Sa)
        np.testing.assert_allclose(np.concatenate([oa, ob]), o, atol=1e-13)
        np.testing.assert_allclose(Sb, S, atol=1e-13)


def test_varlen_equals_separate_and_scalar_equals_broadcast():
    """Packed sequences with offsets equal separate runs; a scalar gate equals
    the channel gate with all channels equal."""
    from gated_delta_rule_46_amd import inputs
    w = inputs.make_forward("t", B=1, H=3, T=0, dk=8, dv=4, gate="gdn", lengths=[5, 1, 9, 3],
                            dtype=torch.float32, s0_std=0.5)
    o, S = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0, w.cu_seqlens, gate_kind=1)
    cu = w.cu_seqlens.tolist()
    for s in range(4):
        sl = slice(cu[s], cu[s + 1])
        os_, Ss = oracle.fwd(w.q[:, sl], w.k[:, sl], w.v[:, sl], w.gate[:, sl], w.beta[:, sl],
                             w.S0[s:s + 1], gate_kind=1)
        np.testing.assert_array_equal(o[:, sl], os_)
        np.testing.assert_array_equal(S[s], Ss[0])
    gch = w.gate[..., None].expand(*w.gate.shape, 8).contiguous()
    oc, Sc = oracle.fwd(w.q, w.k, w.v, gch, w.beta, w.S0, w.cu_seqlens, gate_kind=0)
    np.testing.assert_array_equal(o, oc)
    np.testing.assert_array_equal(S, Sc)


def test_decode_equals_forward():
    """A decode step is the forward's loop body: prefill(T) followed by decode
    steps equals one forward over T + steps tokens."""
    from gated_delta_rule_46_amd import inputs
    w = inputs.make_forward("t", B=3, H=2, T=12, dk=8, dv=6, gate="ckda", dtype=torch.float32,
                            s0_std=0.3)
    o, S = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0)
    pre = 9
    o1, S1 = oracle.fwd(w.q[:, :pre], w.k[:, :pre], w.v[:, :pre], w.gate[:, :pre],
                        w.beta[:, :pre], w.S0)
    St = S1.copy()
    for t in range(pre, 12):
        od = oracle.decode_step(w.q[:, t], w.k[:, t], w.v[:, t], w.gate[:, t], w.beta[:, t], St)
        np.testing.assert_allclose(od, o[:, t], atol=1e-13)
    np.testing.assert_allclose(St, S, atol=1e-13)
    np.testing.assert_allclose(o1, o[:, :pre], atol=1e-13)


def test_heads_subset_matches_full():
    from gated_delta_rule_46_amd import inputs
    w = inputs.make_forward("t", B=2, H=5, T=10, dk=8, dv=4, gate="kda", dtype=torch.float32)
    o, S = oracle.fwd(w.q, w.k, w.v, w.gate, w.beta)
    oh, Sh = oracle.fwd_heads(w.q, w.k, w.v, w.gate, w.beta, [1, 4])
    np.testing.assert_array_equal(oh, o[:, :, [1, 4]])
    np.testing.assert_array_equal(Sh, S[:, [1, 4]])


# ------------------------------------------------------------------ planted mistakes

def test_pins_catch_planted_mistakes():
    """Each plausible slip, planted in a throwaway copy of the recurrence,
    fails one of the closed forms above."""
    def variant(mistake):
        def step(S, k, v, a, b):
            if mistake == "delta_then_gate":
                S = S + b * np.outer(k, v - S.T @ k)
                return a[:, None] * S
            Sg = a[:, None] * S
            if mistake == "read_before_gate":
                pred = S.T @ k
            else:
                pred = Sg.T @ k
            if mistake == "sign":
                return Sg - b * np.outer(k, v - pred)
            if mistake == "no_beta":
                return Sg + np.outer(k, v - pred)
            return Sg + b * np.outer(k, v - pred)
        return step

    rng = np.random.default_rng(13)
    d = 4
    k = unit(rng, d)
    alpha = rng.uniform(-1, 1, d)
    S0 = np.eye(d)
    good = variant(None)(S0, k, np.zeros(d), alpha, 1.3)
    np.testing.assert_allclose(good, oracle_transition(k, alpha, 1.3), atol=1e-14)
    for m in ("delta_then_gate", "read_before_gate", "sign", "no_beta"):
        bad = variant(m)(S0, k, np.zeros(d), alpha, 1.3)
        assert np.abs(bad - good).max() > 1e-3, m


@pytest.mark.parametrize("gate_kind", [0, 1])
def test_gauge_fold_reproduces_direct_run(gate_kind):
    """oracle.gauge.fold, fed to the forward oracle with the final state's rows
    flipped by c_T, reproduces the direct Complex KDA run (the gauge identity
    of the Complex KDA summary, method step 5), also per packed sequence, with
    exact zero and -1 gates and an empty sequence."""
    from oracle import gauge
    rng = np.random.default_rng(21 + gate_kind)
    lengths = [9, 0, 14, 5]
    T, H, dk, dv = sum(lengths), 2, 5, 3
    q = rng.standard_normal((1, T, H, dk))
    k = rng.standard_normal((1, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, dv))
    a = rng.uniform(-1, 1, (1, T, H, dk) if gate_kind == 0 else (1, T, H))
    a.reshape(-1)[[3, 17]] = 0.0
    a.reshape(-1)[[5, 11]] = -1.0
    b = rng.uniform(0, 2, (1, T, H))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S0 = rng.standard_normal((len(lengths), H, dk, dv))
    o1, S1 = oracle.fwd(_t(q), _t(k), _t(v), _t(a), _t(b), _t(S0), cu, gate_kind)
    qf, kf, af, cT = gauge.fold(_t(q), _t(k), _t(a), cu, gate_kind)
    assert (af.numpy() >= 0).all()
    o2, S2 = oracle.fwd(qf, kf, _t(v), af, _t(b), _t(S0), cu, gate_kind)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    flip = cT.astype(np.float64)[..., None]           # [nseq, H, gdim, 1]
    np.testing.assert_allclose(S1, flip * S2, atol=1e-12)
    # an exclusive product (c_{t-1}) in place of the inclusive one breaks it
    c_excl = np.ones_like(a)
    for s_ in range(len(lengths)):
        t0, t1 = cu[s_], cu[s_ + 1]
        if t1 > t0:
            sg = np.where(a[0, t0:t1] < 0, -1.0, 1.0)
            c_excl[0, t0:t1] = np.concatenate([np.ones_like(sg[:1]), np.cumprod(sg, axis=0)[:-1]])
    ce = c_excl if gate_kind == 0 else c_excl[..., None]
    o3, _ = oracle.fwd(_t(q * ce), _t(k * ce), _t(v), _t(np.abs(a)), _t(b), _t(S0), cu, gate_kind)
    assert np.abs(o3 - o1).max() > 1e-3
