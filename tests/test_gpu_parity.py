"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Metric: err = max|x_gpu - x_ref| / rms(x_ref), separately for o and the final
state. Bar: 1e-4 with fp32 inputs, 2e-2 with bf16 inputs (fp32 state).
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_46_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_46_amd import kda as m
    m.library()   # loud failure if the library is missing
    return m


def err(x, ref):
    x = x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(x - ref))) / rms if rms > 0 else float(np.max(np.abs(x - ref)))


def to_dev(w):
    d = lambda t: None if t is None else t.cuda()  # noqa: E731
    return d(w.q), d(w.k), d(w.v), d(w.gate), d(w.beta), d(w.S0), d(w.cu_seqlens)


def gpu_fwd(kda, w, chunk=None, S0=None):
    q, k, v, g, b, s0, cu = to_dev(w)
    if S0 is not None:
        s0 = S0.cuda()
    o, ST = kda.chunk_fwd(q, k, v, g, b, S0=s0, cu_seqlens=cu, chunk=chunk or w.chunk, gate_kind=w.gate_kind)
    torch.cuda.synchronize()
    return o.cpu(), ST.cpu()


def ref_fwd(w, S0=None):
    return oracle.fwd(w.q, w.k, w.v, w.gate, w.beta, w.S0 if S0 is None else S0, w.cu_seqlens, w.gate_kind)


def check(kda, w, chunk=None, tol=None):
    print("case", w.name, "B", w.B, "H", w.H, "T", w.T, "dk", w.dk, "dv", w.dv, "chunk", chunk or w.chunk,
          flush=True)
    o, ST = gpu_fwd(kda, w, chunk)
    ro, rS = ref_fwd(w)
    tol = tol or TOL[w.dtype]
    eo, eS = err(o, ro), err(ST, rS)
    assert np.isfinite(o.numpy()).all() and np.isfinite(ST.numpy()).all()
    assert eo <= tol and eS <= tol, (eo, eS)
    return eo, eS


# ------------------------------------------------------------------ tiny fp32 workload

def test_tiny_fp32(kda):
    w = inputs.tiny_kda()
    eo, eS = check(kda, w)
    print("tiny fp32 err o %.2e S %.2e" % (eo, eS))


# ------------------------------------------------------------------ small, several chunks and a ragged tail

SMALL = [
    # gate, dtype, dk, dv, chunk, T
    ("kda", torch.bfloat16, 128, 128, 64, 200),
    ("ckda", torch.bfloat16, 128, 128, 64, 200),
    ("gdn", torch.bfloat16, 128, 128, 64, 200),
    ("kda", torch.bfloat16, 128, 128, 32, 77),
    ("ckda", torch.bfloat16, 128, 128, 16, 70),
    ("kda", torch.bfloat16, 64, 32, 64, 130),
    ("ckda", torch.bfloat16, 32, 64, 32, 97),
    ("gdn", torch.bfloat16, 16, 128, 16, 45),
    ("kda", torch.bfloat16, 128, 16, 64, 1),
    ("ckda", torch.bfloat16, 16, 16, 64, 64),
    ("kda", torch.float32, 128, 128, 64, 150),
    ("ckda", torch.float32, 64, 64, 32, 100),
    ("gdn", torch.float32, 32, 16, 16, 50),
    ("ckda", torch.float32, 16, 32, 64, 65),
]


@pytest.mark.parametrize("gate,dtype,dk,dv,chunk,T", SMALL)
def test_small_parity(kda, gate, dtype, dk, dv, chunk, T):
    w = inputs.make_forward("small_%s" % gate, B=2, H=3, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype,
                            gate=gate, gate_mu=3.0, seed=T + dk)
    check(kda, w)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nonzero_initial_state(kda, dtype):
    w = inputs.make_forward("s0", B=2, H=2, T=96, dk=128, dv=64, chunk=32, dtype=dtype, gate="ckda",
                            s0_std=0.3, seed=5)
    check(kda, w)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_varlen_small(kda, dtype):
    w = inputs.make_forward("varlen", B=1, H=2, T=0, dk=64, dv=64, chunk=32, dtype=dtype, gate="gdn",
                            lengths=[37, 1, 130, 64, 5], s0_std=0.1, seed=9)
    check(kda, w)


def test_varlen_empty_sequence_keeps_state(kda):
    w = inputs.make_forward("varlen0", B=1, H=2, T=0, dk=32, dv=32, chunk=16, dtype=torch.float32,
                            gate="kda", lengths=[20, 0, 11], s0_std=0.5, seed=3)
    o, ST = gpu_fwd(kda, w)
    np.testing.assert_array_equal(ST[1].numpy(), w.S0[1].numpy())
    check(kda, w)


# ------------------------------------------------------------------ special cases (fp32 inputs)

def _run(kda, q, k, v, g, b, S0=None, chunk=16, gate_kind=0):
    t = lambda x: torch.as_tensor(x, dtype=torch.float32).contiguous().cuda()  # noqa: E731
    o, ST = kda.chunk_fwd(t(q), t(k), t(v), t(g), t(b), S0=None if S0 is None else t(S0), chunk=chunk,
                          gate_kind=gate_kind)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), ST.cpu().double().numpy()


def test_frozen_state_beta0(kda):
    """beta = 0, alpha = 1: S_T = S0 and o_t = S0^T q_t."""
    rng = np.random.default_rng(1)
    B, T, H, d = 1, 50, 2, 32
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d))
    S0 = rng.standard_normal((B, H, d, d))
    o, ST = _run(kda, q, k, v, np.ones((B, T, H, d)), np.zeros((B, T, H)), S0, chunk=32)
    np.testing.assert_allclose(ST, S0, atol=1e-6)
    np.testing.assert_allclose(o, np.einsum("bthi,bhij->bthj", q, S0), atol=1e-4)


def test_exact_retrieval(kda):
    """Unit k, beta = 1, alpha = 1 and q = k: o_t = v_t (projection)."""
    rng = np.random.default_rng(2)
    B, T, H, d = 2, 40, 1, 64
    k = rng.standard_normal((B, T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d))
    o, _ = _run(kda, k, k, v, np.ones((B, T, H, d)), np.ones((B, T, H)), chunk=16)
    np.testing.assert_allclose(o, v, atol=2e-4)


def test_rotation_returns(kda):
    """alpha = (-1, 1, ...), beta = 2, k = (cos t, sin t, 0, ...), v = 0: each
    token rotates the top two state rows by 2t; 8 tokens at t = pi/8 return."""
    d, T = 16, 64
    t = math.pi / 8
    k = np.zeros((1, T, 1, d))
    k[..., 0], k[..., 1] = math.cos(t), math.sin(t)
    a = np.ones((1, T, 1, d))
    a[..., 0] = -1.0
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((1, 1, d, d))
    q = rng.standard_normal((1, T, 1, d))
    for chunk in (16, 32, 64):
        o, ST = _run(kda, q, k, np.zeros((1, T, 1, d)), a, np.full((1, T, 1), 2.0), S0, chunk=chunk)
        np.testing.assert_allclose(ST, S0, atol=1e-4)
        ro, _ = oracle.fwd(torch.tensor(q), torch.tensor(k), torch.zeros(1, T, 1, d), torch.tensor(a),
                           torch.full((1, T, 1), 2.0, dtype=torch.float64), torch.tensor(S0))
        assert err(o, ro) < 1e-4


def test_zero_gate_cuts_history(kda):
    """A token whose gate is 0 in every channel erases the state: outputs after
    it do not depend on anything before it."""
    w = inputs.make_forward("cut", B=1, H=2, T=150, dk=64, dv=32, chunk=64, dtype=torch.float32,
                            gate="ckda", seed=4)
    cut = 70
    w.gate[:, cut] = 0.0
    o1, S1 = gpu_fwd(kda, w)
    w2 = inputs.make_forward("cut2", B=1, H=2, T=150, dk=64, dv=32, chunk=64, dtype=torch.float32,
                             gate="ckda", seed=40)
    for name in ("q", "k", "v", "gate", "beta"):
        getattr(w2, name)[:, cut:] = getattr(w, name)[:, cut:]
    o2, S2 = gpu_fwd(kda, w2)
    assert err(o2[:, cut:], o1[:, cut:].double().numpy()) < 1e-5
    assert err(S2, S1.double().numpy()) < 1e-5


def test_gauge_identity_gpu(kda):
    """CKDA(q, k, alpha) = KDA(c q, c k, |alpha|) with S_T = Diag(c_T) S~_T,
    c_t the cumulative gate sign (sign(0) = +1)."""
    w = inputs.make_forward("gauge", B=1, H=2, T=130, dk=32, dv=32, chunk=32, dtype=torch.float32,
                            gate="ckda", seed=6)
    o1, S1 = gpu_fwd(kda, w)
    c = torch.cumprod(torch.where(w.gate < 0, -1.0, 1.0), dim=1)
    w.q, w.k, w.gate = (c * w.q).contiguous(), (c * w.k).contiguous(), w.gate.abs().contiguous()
    o2, S2 = gpu_fwd(kda, w)
    assert err(o2, o1.double().numpy()) < 1e-4
    cT = c[0, -1]                      # [H, dk]
    assert err(cT[:, :, None] * S2, S1.double().numpy()) < 1e-4


# ------------------------------------------------------------------ invariants

def test_chunk_size_invariance(kda):
    """chunk 16, 32, 64 and the token-by-token oracle (chunk 1) agree."""
    w = inputs.make_forward("inv", B=2, H=2, T=333, dk=128, dv=64, dtype=torch.bfloat16, gate="ckda", seed=8)
    ro, rS = ref_fwd(w)
    outs = {}
    for c in (16, 32, 64):
        o, ST = gpu_fwd(kda, w, chunk=c)
        assert err(o, ro) < 2e-2 and err(ST, rS) < 2e-2
        outs[c] = (o, ST)
    assert err(outs[16][0], outs[64][0].double().numpy()) < 2e-2


def test_split_resume(kda):
    """S_T handed on as S0 at arbitrary cut points equals one pass."""
    w = inputs.make_forward("split", B=1, H=2, T=300, dk=64, dv=64, chunk=32, dtype=torch.float32,
                            gate="kda", seed=11)
    o, S = gpu_fwd(kda, w)
    S0 = None
    parts = []
    for a_, b_ in ((0, 45), (45, 46), (46, 190), (190, 300)):
        wp = inputs.Workload("p", *(t[:, a_:b_].contiguous() for t in (w.q, w.k, w.v, w.gate, w.beta)),
                             None, None, 1, 2, b_ - a_, 64, 64, 32, 0)
        op, S0 = gpu_fwd(kda, wp, S0=S0)
        parts.append(op)
    assert err(torch.cat(parts, 1), o.double().numpy()) < 1e-4
    assert err(S0, S.double().numpy()) < 1e-4


def test_varlen_equals_separate(kda):
    w = inputs.make_forward("vs", B=1, H=2, T=0, dk=32, dv=32, chunk=16, dtype=torch.float32, gate="ckda",
                            lengths=[19, 50, 3], s0_std=0.2, seed=12)
    o, S = gpu_fwd(kda, w)
    cu = w.cu_seqlens.tolist()
    for s in range(3):
        sl = slice(cu[s], cu[s + 1])
        ws = inputs.Workload("s", *(t[:, sl].contiguous() for t in (w.q, w.k, w.v, w.gate, w.beta)),
                             w.S0[s:s + 1].contiguous(), None, 1, 2, cu[s + 1] - cu[s], 32, 32, 16, 0)
        os_, Ss = gpu_fwd(kda, ws)
        assert err(os_, o[:, sl].double().numpy()) < 1e-5
        assert err(Ss, S[s:s + 1].double().numpy()) < 1e-5


def test_scalar_gate_equals_broadcast_channel_gate(kda):
    w = inputs.make_forward("sc", B=1, H=2, T=90, dk=64, dv=32, chunk=32, dtype=torch.float32, gate="gdn",
                            seed=13)
    o1, S1 = gpu_fwd(kda, w)
    w.gate = w.gate[..., None].expand(*w.gate.shape, 64).contiguous()
    w.gate_kind = 0
    o2, S2 = gpu_fwd(kda, w)
    assert err(o2, o1.double().numpy()) < 1e-5 and err(S2, S1.double().numpy()) < 1e-5


@pytest.mark.parametrize("dk,dv,T", [(128, 64, 300), (64, 128, 129), (128, 32, 65)])
def test_walker_paths_small(kda, dk, dv, T):
    """64-token chunks with bf16 inputs: dk = 128 takes the one-slice walker
    (operands loaded into registers), dk = 64 the two-waves-per-slice walker;
    nonzero initial state, ragged tail, each value width."""
    w = inputs.make_forward("walk", B=2, H=3, T=T, dk=dk, dv=dv, chunk=64, dtype=torch.bfloat16, gate="ckda",
                            s0_std=0.2, seed=dk + dv + T)
    check(kda, w)


def test_walkers_agree(kda):
    """With more 16-column value slices than CUs the state walk runs two
    slices per workgroup staged through LDS, with fewer it runs one slice per
    workgroup fed straight from memory; both do the same arithmetic. A batch
    of four sequences (B4 H16 dv128: 512 slices) and its first sequence alone
    (128 slices) give that sequence bit-identical outputs, and the batch
    matches the oracle."""
    w = inputs.make_forward("walk4", B=4, H=16, T=200, dk=128, dv=128, chunk=64, dtype=torch.bfloat16, gate="ckda",
                            s0_std=0.2, seed=5)
    o4, S4 = gpu_fwd(kda, w)
    w1 = dataclasses.replace(w, B=1, **{x: getattr(w, x)[:1].contiguous() for x in ("q", "k", "v", "gate", "beta", "S0")})
    o1, S1 = gpu_fwd(kda, w1)
    assert torch.equal(o4[:1], o1) and torch.equal(S4[:1], S1)
    ro, rS = ref_fwd(w)
    assert err(o4, ro) <= 2e-2 and err(S4, rS) <= 2e-2


@pytest.mark.parametrize("gate,B,H,T,s0", [("ckda", 1, 2, 1611, 0.3), ("kda", 2, 3, 3000, 0.0),
                                           ("gdn", 1, 4, 1536, 0.2), ("ckda", 3, 1, 4097, 0.1)])
def test_long_sequences_few_heads(kda, gate, B, H, T, s0):
    """Long sequences at few heads (bf16, dk = dv = 128, chunk 64: the
    one-slice walker with far fewer slices than CUs): 24 to 65 chunks, ragged
    last chunks and exactly 24 chunks, with and without an initial state; o
    and S_T against the oracle."""
    w = inputs.make_forward("long", B=B, H=H, T=T, dk=128, dv=128, chunk=64, dtype=torch.bfloat16, gate=gate,
                            s0_std=s0, seed=T + H)
    check(kda, w)


def test_stage_split_equals_single_call(kda):
    """The forward as one call equals its two stages called one after the
    other (prep into a caller-provided workspace, then the state walk) bit
    for bit, and the oracle within the bf16 bar."""
    w = inputs.make_forward("split", B=2, H=2, T=2100, dk=128, dv=128, chunk=64, dtype=torch.bfloat16, gate="ckda",
                            s0_std=0.2, seed=21)
    q, k, v, g, b, s0, _ = to_dev(w)
    o1, S1 = kda.chunk_fwd(q, k, v, g, b, S0=s0, chunk=64)
    wsb = kda.workspace_bytes(w.B, w.H, w.T, 128, 128, 64)
    ws = torch.empty(wsb, device="cuda", dtype=torch.uint8)
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    kda.chunk_fwd(q, k, v, g, b, S0=s0, chunk=64, out=o2, S_T=S2, workspace=ws, stage=kda.STAGE_PREP)
    kda.chunk_fwd(q, k, v, g, b, S0=s0, chunk=64, out=o2, S_T=S2, workspace=ws, stage=kda.STAGE_STATE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    ro, rS = ref_fwd(w)
    assert err(o1, ro) <= 2e-2 and err(S1, rS) <= 2e-2


def test_deterministic(kda):
    w = inputs.make_forward("det", B=1, H=4, T=257, dk=128, dv=128, dtype=torch.bfloat16, gate="ckda", seed=14)
    o1, S1 = gpu_fwd(kda, w)
    o2, S2 = gpu_fwd(kda, w)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ------------------------------------------------------------------ decode

def _norm_keeping_gates(rng, gshape, bshape):
    """|alpha| = 1 with random signs, and beta = 2 (a reflection) for half the
    tokens, U(0, 2) otherwise: the state norm stays near its start instead of
    decaying, so growth from a wrong sign or term would show."""
    g = np.where(rng.random(gshape) < 0.5, -1.0, 1.0)
    b = np.where(rng.random(bshape) < 0.5, 2.0, 2.0 * rng.random(bshape))
    return torch.tensor(g, dtype=torch.float32), torch.tensor(b, dtype=torch.float32)


def test_side_stream_bit_identical(kda):
    """Every call enqueues on the stream it is given: forward, backward and
    decode launched on a second stream (default priority, workspace taken
    from the device pool on that stream) give the default stream's results
    bit for bit."""
    w = inputs.make_forward("stream", B=2, H=3, T=150, dk=128, dv=64, chunk=64, dtype=torch.bfloat16, gate="ckda",
                            s0_std=0.3, seed=21)
    q, k, v, g, b, s0, _ = to_dev(w)
    dO, dST = (t.cuda() for t in inputs.cotangents(w, seed=21))
    o1, S1 = kda.chunk_fwd(q, k, v, g, b, S0=s0, chunk=64)
    g1 = kda.chunk_bwd(q, k, v, g, b, dO, S0=s0, dS_T=dST)
    Sd1 = s0.clone()
    od1 = kda.decode_step(q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(), g[:, 0].contiguous(),
                          b[:, 0].contiguous(), Sd1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        o2, S2 = kda.chunk_fwd(q, k, v, g, b, S0=s0, chunk=64, stream=side)
        g2 = kda.chunk_bwd(q, k, v, g, b, dO, S0=s0, dS_T=dST, stream=side)
        Sd2 = s0.clone()
        od2 = kda.decode_step(q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(),
                              g[:, 0].contiguous(), b[:, 0].contiguous(), Sd2, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n
    assert torch.equal(od1, od2) and torch.equal(Sd1, Sd2)


def test_graph_replay_matches_eager(kda):
    """The forward (caller-supplied workspace) and a decode step enqueue kernels
    only, so a caller can capture them in a graph: three replays, each on new
    inputs copied into the captured buffers and with eager calls in between,
    each equal bit for bit to an eager call on the same inputs."""
    B, H, T, dk, dv = 2, 2, 200, 128, 64

    def make(seed):
        w = inputs.make_forward("graph", B=B, H=H, T=T, dk=dk, dv=dv, chunk=64, dtype=torch.bfloat16, gate="ckda",
                                s0_std=0.3, seed=seed)
        return [t.cuda() for t in (w.q, w.k, w.v, w.gate, w.beta, w.S0)]

    static = make(30)
    ws = torch.empty(kda.workspace_bytes(B, H, T, dk, dv, 64), device="cuda", dtype=torch.uint8)
    o = torch.empty((B, T, H, dv), device="cuda")
    ST = torch.empty((B, H, dk, dv), device="cuda")
    Sd = torch.empty((B, H, dk, dv), device="cuda")
    od = torch.empty((B, H, dv), device="cuda")

    def step():
        q, k, v, g, b, s0 = static
        kda.chunk_fwd(q, k, v, g, b, S0=s0, chunk=64, out=o, S_T=ST, workspace=ws)
        Sd.copy_(ST)
        kda.decode_step(q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(), g[:, 0].contiguous(),
                        b[:, 0].contiguous(), Sd, out=od)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        new = make(31 + rep)
        for dst, src in zip(static, new):
            dst.copy_(src)
        q, k, v, g, b, s0 = new
        o_e, ST_e = kda.chunk_fwd(q, k, v, g, b, S0=s0, chunk=64)   # eager, own workspace
        Sd_e = ST_e.clone()
        od_e = kda.decode_step(q[:, 0].contiguous(), k[:, 0].contiguous(), v[:, 0].contiguous(),
                               g[:, 0].contiguous(), b[:, 0].contiguous(), Sd_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(ST, ST_e), rep
        assert torch.equal(od, od_e) and torch.equal(Sd, Sd_e), rep


def test_no_write_state_norm_nonincreasing(kda):
    """With v = 0 every token maps S to A_t S, A_t = (I - beta k k^T) Diag(alpha);
    with unit k, beta in [0, 2] and |alpha| <= 1 the spectral norm of A_t is at
    most 1 (Complex KDA summary, stability of the transition), so the
    Frobenius norm of the state never grows: checked after every decode step
    and, through the chunked forward, at prefix lengths that cross chunk
    boundaries. fp32 inputs (k unit to fp32 rounding); the slack covers fp32
    rounding only."""
    rng = np.random.default_rng(61)
    # decode: 48 steps in place from a random state
    dw = inputs.ckda_decode(seed=6, N=4, H=2, d=64, n_steps=48, s_std=1.0, dtype=torch.float32)
    S = dw.S.cuda()
    n0 = torch.linalg.matrix_norm(dw.S.double())
    prev = n0
    for st in dw.steps:
        g, b = _norm_keeping_gates(rng, tuple(st["gate"].shape), tuple(st["beta"].shape))
        v0 = torch.zeros_like(st["v"])
        kda.decode_step(st["q"].cuda(), st["k"].cuda(), v0.cuda(), g.cuda(), b.cuda(), S)
        torch.cuda.synchronize()
        n = torch.linalg.matrix_norm(S.cpu().double())
        assert bool((n <= prev * (1 + 1e-5)).all()), float((n / prev).max())
        prev = n
    print("decode: norm ratio after 48 steps %.3f..%.3f" % (float((prev / n0).min()), float((prev / n0).max())))
    # chunked forward: S_T of growing prefixes
    w = inputs.make_forward("nowrite", B=2, H=2, T=200, dk=64, dv=32, chunk=64, dtype=torch.float32,
                            gate="ckda", s0_std=1.0, seed=16)
    g, b = _norm_keeping_gates(rng, tuple(w.gate.shape), tuple(w.beta.shape))
    w = dataclasses.replace(w, v=torch.zeros_like(w.v), gate=g, beta=b)
    n0 = prev = torch.linalg.matrix_norm(w.S0.double())
    for T in (30, 64, 100, 128, 170, 200):
        wp = dataclasses.replace(w, q=w.q[:, :T].contiguous(), k=w.k[:, :T].contiguous(), v=w.v[:, :T].contiguous(),
                                 gate=w.gate[:, :T].contiguous(), beta=w.beta[:, :T].contiguous(), T=T)
        _, ST = gpu_fwd(kda, wp)
        n = torch.linalg.matrix_norm(ST.double())
        assert bool((n <= prev * (1 + 1e-4)).all()), (T, float((n / prev).max()))
        prev = n
    print("forward: norm ratio after 200 tokens %.3f..%.3f" % (float((prev / n0).min()), float((prev / n0).max())))


@pytest.mark.parametrize("dtype,dk,dv,gk", [(torch.bfloat16, 128, 128, 0), (torch.float32, 64, 32, 0),
                                            (torch.bfloat16, 16, 64, 1), (torch.float32, 32, 128, 1)])
def test_decode_parity(kda, dtype, dk, dv, gk):
    N, H, steps = 6, 3, 5
    rng = np.random.default_rng(dk + dv)
    S = torch.from_numpy(rng.normal(0, 0.3, (N, H, dk, dv))).float()
    Sd = S.cuda()
    Sr = S.double().numpy().copy()
    for st in range(steps):
        w = inputs.make_forward("d", B=N, H=H, T=1, dk=dk, dv=dv, dtype=dtype, gate="gdn" if gk else "ckda",
                                seed=st)
        q, k, v, g, b = (t[:, 0].contiguous() for t in (w.q, w.k, w.v, w.gate, w.beta))
        o = kda.decode_step(q.cuda(), k.cuda(), v.cuda(), g.cuda(), b.cuda(), Sd, gate_kind=gk)
        ro = oracle.decode_step(q, k, v, g, b, Sr, gate_kind=gk)
        torch.cuda.synchronize()
        tol = 1e-5 if dtype == torch.float32 else 1e-3
        assert err(o.cpu(), ro) < tol
    assert err(Sd.cpu(), Sr) < 1e-5


def test_decode_equals_forward_step(kda):
    """prefill(T) on the GPU then decode steps equals one forward of T + steps."""
    w = inputs.make_forward("pf", B=3, H=2, T=70, dk=64, dv=64, chunk=32, dtype=torch.float32, gate="ckda",
                            s0_std=0.2, seed=15)
    o_full, S_full = gpu_fwd(kda, w)
    pre = 66
    wp = inputs.Workload("pre", *(t[:, :pre].contiguous() for t in (w.q, w.k, w.v, w.gate, w.beta)),
                         w.S0, None, 3, 2, pre, 64, 64, 32, 0)
    _, S = gpu_fwd(kda, wp)
    S = S.cuda()
    for t in range(pre, 70):
        o = kda.decode_step(*(x[:, t].contiguous().cuda() for x in (w.q, w.k, w.v, w.gate, w.beta)), S)
        torch.cuda.synchronize()
        assert err(o.cpu(), o_full[:, t].double().numpy()) < 1e-4
    assert err(S.cpu(), S_full.double().numpy()) < 1e-4


# ------------------------------------------------------------------ signed zero gates

@pytest.mark.parametrize("gate,dtype,dk,dv,chunk,T", [("ckda", torch.bfloat16, 128, 128, 64, 300),
                                                      ("ckda", torch.float32, 64, 32, 32, 150),
                                                      ("gdn", torch.bfloat16, 128, 64, 64, 200),
                                                      ("gdn", torch.float32, 32, 16, 16, 97)])
def test_signed_zero_gates_forward(kda, gate, dtype, dk, dv, chunk, T):
    """About 3% of the gates set, in equal parts, to -0.0, +0.0 and -1.0: a
    zero of either sign zeroes its state row exactly and adds no sign, -1.0
    flips it (Complex KDA summary, method steps 3 and 5)."""
    w = inputs.make_forward("szero_%s" % gate, B=2, H=3, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype, gate=gate,
                            seed=T + dk, s0_std=0.3)
    w = dataclasses.replace(w, gate=inputs.signed_zero_gates(w.gate, seed=T))
    nz = int((w.gate.view(torch.int16 if dtype == torch.bfloat16 else torch.int32) ==
              (-32768 if dtype == torch.bfloat16 else -2 ** 31)).sum())
    assert nz > 0   # the case really holds -0.0 gates
    check(kda, w)


def test_signed_zero_gates_decode(kda):
    """Decode steps with -0.0, +0.0 and -1.0 gates (channel and scalar kinds)."""
    for gk, dtype in ((0, torch.bfloat16), (1, torch.bfloat16), (0, torch.float32)):
        N, H, dk, dv = 8, 3, 128, 64
        rng = np.random.default_rng(5 + gk)
        S = torch.from_numpy(rng.normal(0, 0.3, (N, H, dk, dv))).float()
        Sd, Sr = S.cuda(), S.double().numpy().copy()
        for st in range(6):
            w = inputs.make_forward("dz", B=N, H=H, T=1, dk=dk, dv=dv, dtype=dtype, gate="gdn" if gk else "ckda",
                                    seed=40 + st)
            q, k, v, g, b = (t[:, 0].contiguous() for t in (w.q, w.k, w.v, w.gate, w.beta))
            g = inputs.signed_zero_gates(g, seed=st, frac=0.3 if gk else 0.06)
            o = kda.decode_step(q.cuda(), k.cuda(), v.cuda(), g.cuda(), b.cuda(), Sd, gate_kind=gk)
            ro = oracle.decode_step(q, k, v, g, b, Sr, gate_kind=gk)
            torch.cuda.synchronize()
            assert err(o.cpu(), ro) < TOL[dtype] / 20
        assert err(Sd.cpu(), Sr) < TOL[dtype] / 20


def test_c_abi_direct_call(kda):
    """kda_chunk_fwd called straight through ctypes with raw device pointers
    (no binding code in between), on real data, against the oracle; the
    status word left in the workspace reads KDA_OK."""
    import ctypes
    w = inputs.make_forward("abi", B=2, H=3, T=130, dk=128, dv=128, chunk=64, gate="ckda", seed=77, s0_std=0.2)
    q, k, v, g, b, s0, _ = to_dev(w)
    o = torch.full((2, 130, 3, 128), float("nan"), device="cuda")
    ST = torch.full((2, 3, 128, 128), float("nan"), device="cuda")
    lib = kda.library()
    need = lib.kda_chunk_fwd_workspace_bytes(2, 3, 130, 128, 128, 64, 2, 0, kda.KDA_BF16)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")   # stale contents, status word included
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = lib.kda_chunk_fwd(P(q), P(k), P(v), P(g), P(b), P(s0), P(o), P(ST), 2, 3, 130, 128, 128, 64, None, 2,
                           kda.KDA_BF16, 0, P(ws), need, None)
    assert rc == kda.KDA_OK
    torch.cuda.synchronize()
    ro, rS = ref_fwd(w)
    assert err(o.cpu(), ro) <= 2e-2 and err(ST.cpu(), rS) <= 2e-2
    assert kda.fwd_status(ws) == kda.KDA_OK
    assert int(ws[:4].cpu().view(torch.int32).item()) == 0


# ------------------------------------------------------------------ full-size workloads, every head

def _full(kda, w):
    """The whole workload in the launch configuration the benchmark times;
    the oracle recomputes every (sequence, head) pair."""
    print("case", w.name, "full size, every head", flush=True)
    q, k, v, g, b, s0, cu = to_dev(w)
    N = w.n_seqs
    need = kda.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, N, cu is not None, w.dtype)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    o, ST = kda.chunk_fwd(q, k, v, g, b, S0=s0, cu_seqlens=cu, chunk=w.chunk, gate_kind=w.gate_kind, workspace=ws)
    assert kda.fwd_status(ws) == kda.KDA_OK
    o, ST = o.cpu(), ST.cpu()
    del q, k, v, g, b
    ro, rS = ref_fwd(w)
    eo, eS = err(o, ro), err(ST, rS)
    # per-head errors too, so that one bad head cannot hide behind the global rms
    per_head = [max(err(o[:, :, h], ro[:, :, h]), err(ST[:, h], rS[:, h])) for h in range(w.H)]
    per_seq = []
    if w.cu_seqlens is not None:
        cu_h = w.cu_seqlens.tolist()
        for s_ in range(N):
            a, z = cu_h[s_], cu_h[s_ + 1]
            per_seq.append(max(err(o[:, a:z], ro[:, a:z]) if z > a else 0.0, err(ST[s_], rS[s_])))
    else:
        per_seq = [max(err(o[s_], ro[s_]), err(ST[s_], rS[s_])) for s_ in range(w.B)]
    print("%s err o %.3e S %.3e; worst head %.3e, worst sequence %.3e" % (w.name, eo, eS, max(per_head),
                                                                          max(per_seq)), flush=True)
    assert eo <= 2e-2 and eS <= 2e-2
    assert max(per_head) <= 2e-2 and max(per_seq) <= 2e-2


def test_full_kda_b4_h16_t4096(kda):
    _full(kda, inputs.kda_fwd())


def test_full_ckda_b2_h16_t8192(kda):
    _full(kda, inputs.ckda_fwd())


def test_full_ckda_signed_zero_gates(kda):
    """The Complex KDA workload with 3% of its gates replaced by -0.0, +0.0
    and -1.0 in equal parts."""
    w = inputs.ckda_fwd()
    _full(kda, dataclasses.replace(w, name="ckda_szero", gate=inputs.signed_zero_gates(w.gate, seed=3)))


def test_full_gdn_varlen_h32(kda):
    _full(kda, inputs.gdn_varlen())


def test_full_decode_n256_h32(kda):
    """128 in-place steps at N=256, H=32; the oracle follows every (sequence,
    head) state and every step's output."""
    dw = inputs.ckda_decode(n_steps=128)
    Sd = dw.S.cuda()
    Sr = dw.S.double().numpy().copy()
    worst = 0.0
    for i, st in enumerate(dw.steps):
        o = kda.decode_step(*(st[x].cuda() for x in ("q", "k", "v", "gate", "beta")), Sd)
        ro = oracle.decode_step(st["q"], st["k"], st["v"], st["gate"], st["beta"], Sr)
        worst = max(worst, err(o.cpu(), ro))
        if i % 32 == 31:
            print("decode step %d worst err o %.3e" % (i + 1, worst), flush=True)
    torch.cuda.synchronize()
    Sg = Sd.cpu().double().numpy()
    eS = err(Sg, Sr)
    per_pair = float(np.max(np.abs(Sg - Sr).max(axis=(2, 3)) / np.sqrt(np.mean(Sr * Sr))))
    print("decode max err o %.3e S %.3e (worst pair %.3e)" % (worst, eS, per_pair), flush=True)
    assert worst <= 2e-2 and eS <= 2e-2 and per_pair <= 2e-2
