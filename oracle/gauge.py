"""Gauge transform of Complex KDA onto positive gates, plain numpy.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Complex KDA summary, method step 5: the cumulative signs of the gates can be
absorbed into the keys and queries so that a positive-gate run reproduces the
outputs. With s_t = -1 where alpha_t < 0 and +1 elsewhere (zero and -0.0
included: a zero gate cuts the history, so its sign is immaterial), per
sequence and key channel

    c_t = s_1 s_2 ... s_t               (inclusive of token t)
    q~_t = c_t q_t,  k~_t = c_t k_t,  alpha~_t = |alpha_t|

and the positive-gate run's final state S~_T relates to the original one by
S_T = Diag(c_T) S~_T (the identity the oracle pins check). For a scalar gate
the sign is one per (token, head) and c_t multiplies every channel.
"""
from __future__ import annotations

import numpy as np
import torch


def fold(q, k, gate, cu_seqlens=None, gate_kind: int = 0):
    """Returns (q~, k~, alpha~, c_T): the first three as tensors of the input
    dtype (every value is an input value with its sign changed or cleared, so
    the conversion back is exact); c_T as an int8 numpy array [nseq, H, gdim]
    of +1 / -1."""
    dtype = q.dtype
    qd, kd, ad = (x.detach().cpu().double().numpy() for x in (q, k, gate))
    B, T, H, dk = qd.shape
    if cu_seqlens is None:
        bounds = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens)
        bounds = [(0, int(cu[s]), int(cu[s + 1])) for s in range(cu.size - 1)]
    gdim = dk if gate_kind == 0 else 1
    qo, ko = qd.copy(), kd.copy()
    ao = np.abs(ad)
    cT = np.ones((len(bounds), H, gdim), dtype=np.int8)
    for si, (b, t0, t1) in enumerate(bounds):
        if t1 <= t0:
            continue
        a = ad[b, t0:t1].reshape(t1 - t0, H, gdim)
        c = np.cumprod(np.where(a < 0, -1.0, 1.0), axis=0)          # [len, H, gdim]
        qo[b, t0:t1] = qd[b, t0:t1] * c
        ko[b, t0:t1] = kd[b, t0:t1] * c
        cT[si] = c[-1].astype(np.int8)
    conv = lambda x: torch.from_numpy(x).to(dtype)  # noqa: E731
    return conv(qo), conv(ko), conv(ao), cT
