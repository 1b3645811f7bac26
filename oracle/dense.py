"""Dense-matrix formulation of the gated delta rule, for tiny inputs.

TEST INFRASTRUCTURE ONLY. Independent of ``kda_oracle.c``: instead of the
delta form it builds each transition matrix explicitly and forms the state as
a sum of products of transitions,

    A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
          (Complex KDA summary, background "diagonal-plus-rank-one transitions")
    Phi_{t,s} = A_t A_{t-1} ... A_{s+1}          (Phi_{t,t} = I)
    S_t = Phi_{t,0} S_0 + sum_{s<=t} Phi_{t,s} beta_s k_s v_s^T
    o_t = S_t^T q_t.
"""
from __future__ import annotations

import numpy as np


def transition(k: np.ndarray, alpha: np.ndarray, beta: float) -> np.ndarray:
    """A = (I - beta k k^T) Diag(alpha); ``alpha`` is a vector or a scalar."""
    k = np.asarray(k, dtype=np.float64)
    d = k.size
    alpha = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (d,))
    return (np.eye(d) - beta * np.outer(k, k)) @ np.diag(alpha)


def run(q, k, v, alpha, beta, S0=None):
    """One sequence, one head. q, k [T,dk]; v [T,dv]; alpha [T,dk] or [T];
    beta [T]; S0 [dk,dv]. Returns (o [T,dv], S_T [dk,dv]) in fp64."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    A = [transition(k[t], alpha[t], beta[t]) for t in range(T)]
    o = np.zeros((T, dv))
    S = S0
    for t in range(T):
        # Phi_{t,s} for s = t, t-1, ..., -1 built right to left.
        phi = np.eye(dk)
        St = beta[t] * np.outer(k[t], v[t])
        for s in range(t - 1, -1, -1):
            phi = phi @ A[s + 1]
            St = St + phi @ (beta[s] * np.outer(k[s], v[s]))
        phi = phi @ A[0]
        S = St + phi @ S0
        o[t] = S.T @ q[t]
    return o, S


def transition_ew(k: np.ndarray, alpha: np.ndarray, erase: np.ndarray) -> np.ndarray:
    """Erase/write-gate transition A = (I - k (e o k)^T) Diag(alpha) (Gated
    DeltaNet-2 blurb, channel-wise erase gate; reading as in kda_oracle.c)."""
    k = np.asarray(k, dtype=np.float64)
    d = k.size
    alpha = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (d,))
    return (np.eye(d) - np.outer(k, np.asarray(erase, dtype=np.float64) * k)) @ np.diag(alpha)


def run_ew(q, k, v, alpha, erase, write, S0=None):
    """Dense products for the erase/write-gate recurrence: transitions
    A_t = (I - k_t (e_t o k_t)^T) Diag(alpha_t) and writes k_t (w_t o v_t)^T.
    q, k, erase [T,dk]; v, write [T,dv]; alpha [T,dk] or [T]. Returns
    (o [T,dv], S_T [dk,dv])."""
    q, k, v, erase, write = (np.asarray(x, dtype=np.float64) for x in (q, k, v, erase, write))
    alpha = np.asarray(alpha, dtype=np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    A = [transition_ew(k[t], alpha[t], erase[t]) for t in range(T)]
    X = [np.outer(k[t], write[t] * v[t]) for t in range(T)]
    o = np.zeros((T, dv))
    S = S0
    for t in range(T):
        phi = np.eye(dk)
        St = X[t].copy()
        for s in range(t - 1, -1, -1):
            phi = phi @ A[s + 1]
            St = St + phi @ X[s]
        phi = phi @ A[0]
        S = St + phi @ S0
        o[t] = S.T @ q[t]
    return o, S
