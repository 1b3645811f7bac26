"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_46_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_46_amd import build
        build.build()
    return kda.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    assert lib.kda_version() == 100
    for code in (0, -1, -2, -3, -4, -5):
        assert kda.strerror(code)
    assert kda.strerror(-99) == "unknown status"
    assert lib.kda_last_hip_error() == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def chunk(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, S0=None, o=FAKE, S_T=None, B=1, H=2, T=8,
             dk=16, dv=16, chunk=16, cu=None, N=0, dtype=kda.KDA_BF16, gate_kind=0, ws=FAKE, wsb=0,
             stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd(*[a[x] for x in ("q", "k", "v", "gate", "beta", "S0", "o", "S_T", "B", "H",
                                                 "T", "dk", "dv", "chunk", "cu", "N", "dtype",
                                                 "gate_kind", "ws", "wsb", "stream")])


def test_chunk_validation(lib):
    assert chunk(lib, B=0) == kda.KDA_EINVAL
    assert chunk(lib, H=-1) == kda.KDA_EINVAL
    assert chunk(lib, dk=24) == kda.KDA_ENOTSUP
    assert chunk(lib, dv=256) == kda.KDA_ENOTSUP
    assert chunk(lib, chunk=128) == kda.KDA_ENOTSUP
    assert chunk(lib, dtype=7) == kda.KDA_ENOTSUP
    assert chunk(lib, gate_kind=2) == kda.KDA_ENOTSUP
    assert chunk(lib, q=None) == kda.KDA_EINVAL
    assert chunk(lib, o=None) == kda.KDA_EINVAL
    assert chunk(lib, q=FAKE + 1) == kda.KDA_EALIGN                   # bf16 needs 2-byte alignment
    assert chunk(lib, dtype=kda.KDA_F32, k=FAKE + 2) == kda.KDA_EALIGN
    assert chunk(lib, ws=FAKE + 8) == kda.KDA_EALIGN
    assert chunk(lib, wsb=1) == kda.KDA_EINVAL                        # workspace too small
    assert chunk(lib, cu=FAKE, B=2, N=2) == kda.KDA_EINVAL            # varlen needs B == 1
    assert chunk(lib, cu=FAKE, N=0) == kda.KDA_EINVAL
    assert chunk(lib, N=3) == kda.KDA_EINVAL                          # N != B without offsets


def test_decode_validation(lib):
    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, S=FAKE, o=FAKE, N=2, H=2, dk=16, dv=16,
                 dtype=kda.KDA_BF16, gate_kind=0, stream=None)
        a.update(kw)
        return lib.kda_decode_step(*a.values())
    assert dec(N=0) == kda.KDA_EINVAL
    assert dec(dk=48) == kda.KDA_ENOTSUP
    assert dec(dtype=3) == kda.KDA_ENOTSUP
    assert dec(gate_kind=-1) == kda.KDA_ENOTSUP
    assert dec(S=None) == kda.KDA_EINVAL
    assert dec(S=FAKE + 4) == kda.KDA_EALIGN                           # state needs 16 bytes
    assert dec(o=FAKE + 8) == kda.KDA_EALIGN


def test_workspace_bytes(lib):
    f = kda.workspace_bytes
    assert f(1, 2, 64, 24, 16, 16) == 0
    a = f(1, 2, 64, 16, 16, 16)
    assert a > 0 and a % 256 == 0
    hdr = f(1, 2, 0, 16, 16, 16)                                     # status header only
    assert hdr == 256
    assert f(2, 2, 64, 16, 16, 16) - hdr == 2 * (a - hdr)
    assert f(1, 2, 65, 16, 16, 16) > a                                # ragged tail adds a chunk
    assert f(1, 16, 8192, 128, 128, 64) > f(1, 16, 8192, 128, 128, 64, dtype=None) * 0  # defined
    v = f(1, 2, 100, 16, 16, 16, N=5, varlen=True)
    assert v >= f(1, 2, 100, 16, 16, 16)
    assert f(2, 2, 100, 16, 16, 16, N=5, varlen=True) == 0           # varlen needs B == 1


def test_bwd_validation(lib):
    def bwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, S0=None, dO=FAKE, dST=None, gq=FAKE, gk=FAKE,
                 gv=FAKE, gg=FAKE, gb=FAKE, gS0=None, B=1, H=2, T=8, dk=16, dv=16, cu=None, N=0,
                 dtype=kda.KDA_BF16, gate_kind=0, ws=FAKE, wsb=0, stream=None)
        a.update(kw)
        return lib.kda_chunk_bwd(*a.values())
    assert bwd(B=0) == kda.KDA_EINVAL
    assert bwd(dk=24) == kda.KDA_ENOTSUP
    assert bwd(dv=8) == kda.KDA_ENOTSUP
    assert bwd(dtype=5) == kda.KDA_ENOTSUP
    assert bwd(gate_kind=3) == kda.KDA_ENOTSUP
    assert bwd(dO=None) == kda.KDA_EINVAL
    assert bwd(gq=None) == kda.KDA_EINVAL
    assert bwd(dO=FAKE + 4) == kda.KDA_EALIGN                         # dO is read 16 bytes at a time
    assert bwd(gv=FAKE + 8) == kda.KDA_EALIGN
    assert bwd(gS0=FAKE + 4) == kda.KDA_EALIGN
    assert bwd(q=FAKE + 1) == kda.KDA_EALIGN
    assert bwd(wsb=1) == kda.KDA_EINVAL                               # workspace too small
    assert bwd(cu=FAKE, B=2, N=2) == kda.KDA_EINVAL
    assert bwd(N=4) == kda.KDA_EINVAL
    assert kda.bwd_workspace_bytes(1, 2, 64, 24, 16) == 0
    w = kda.bwd_workspace_bytes(1, 2, 64, 16, 16)
    assert w > 0 and w % 256 == 0
    assert kda.bwd_workspace_bytes(1, 2, 65, 16, 16) > w              # one more checkpoint and token
    assert kda.bwd_workspace_bytes(2, 2, 64, 16, 16, N=2, varlen=True) == 0


def test_bwd_cw_validation(lib):
    def bwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, S0=None, dO=FAKE, dST=None, gq=FAKE, gk=FAKE,
                 gv=FAKE, gg=FAKE, gb=FAKE, gS0=None, B=1, H=2, T=8, dk=64, dv=16, cu=None, N=0,
                 dtype=kda.KDA_BF16, gate_kind=0, ws=FAKE, wsb=0, stream=None)
        a.update(kw)
        return lib.kda_chunk_bwd_cw(*a.values())
    assert bwd(B=0) == kda.KDA_EINVAL
    assert bwd(dk=32) == kda.KDA_ENOTSUP                              # dk 64 or 128 only
    assert bwd(dv=8) == kda.KDA_ENOTSUP
    assert bwd(dtype=5) == kda.KDA_ENOTSUP
    assert bwd(gate_kind=3) == kda.KDA_ENOTSUP
    assert bwd(dO=None) == kda.KDA_EINVAL
    assert bwd(gq=None) == kda.KDA_EINVAL
    assert bwd(dO=FAKE + 4) == kda.KDA_EALIGN                         # dO rows are read 16 bytes at a time
    assert bwd(gv=FAKE + 2) == kda.KDA_EALIGN
    assert bwd(q=FAKE + 1) == kda.KDA_EALIGN
    assert bwd(ws=FAKE + 8) == kda.KDA_EALIGN
    assert bwd(wsb=1) == kda.KDA_EINVAL                               # workspace too small
    assert bwd(ws=None) == kda.KDA_EINVAL                             # the library never allocates
    assert bwd(cu=FAKE, B=2, N=2) == kda.KDA_EINVAL
    assert bwd(N=4) == kda.KDA_EINVAL
    w = kda.bwd_cw_workspace_bytes(1, 2, 64, 64, 16)
    assert w > 0 and kda.bwd_cw_workspace_bytes(1, 2, 65, 64, 16) > w  # one more chunk
    assert kda.bwd_cw_workspace_bytes(1, 2, 64, 32, 16) == 0


def test_gauge_validation(lib):
    def fold(**kw):
        a = dict(q=FAKE, k=FAKE, gate=FAKE, qo=FAKE, ko=FAKE, go=FAKE, sign=None, B=1, H=2, T=8, dk=16, cu=None,
                 N=0, dtype=kda.KDA_BF16, gate_kind=0, ws=FAKE, wsb=0, stream=None)
        a.update(kw)
        return lib.kda_gauge_fold(*a.values())
    assert fold(B=0) == kda.KDA_EINVAL
    assert fold(dk=12) == kda.KDA_ENOTSUP
    assert fold(gate_kind=2) == kda.KDA_ENOTSUP
    assert fold(qo=None) == kda.KDA_EINVAL
    assert fold(q=FAKE + 2) == kda.KDA_EALIGN                         # read 8 channels (16 bytes) at a time
    assert fold(go=FAKE + 2) == kda.KDA_EALIGN                        # channel gate likewise
    assert fold(wsb=1) == kda.KDA_EINVAL
    args = ("q", "k", "v", "gate", "beta", "S0", "o", "S_T", "B", "H", "T", "dk", "dv", "chunk", "cu", "N", "dtype",
            "gate_kind", "ws", "wsb", "stream")

    def route(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, S0=None, o=FAKE, S_T=None, B=1, H=2, T=8,
                 dk=16, dv=16, chunk=16, cu=None, N=0, dtype=kda.KDA_BF16, gate_kind=0, ws=FAKE, wsb=0,
                 stream=None)
        a.update(kw)
        return lib.kda_chunk_fwd_gauge(*[a[x] for x in args])
    assert route(B=0) == kda.KDA_EINVAL
    assert route(chunk=8) == kda.KDA_ENOTSUP
    assert route(o=None) == kda.KDA_EINVAL
    assert route(q=FAKE + 2) == kda.KDA_EALIGN
    assert route(wsb=1) == kda.KDA_EINVAL
    assert kda.fwd_gauge_workspace_bytes(1, 2, 64, 16, 16, 16) > kda.workspace_bytes(1, 2, 64, 16, 16, 16)


def test_null_workspace_rejected(lib):
    """The library never allocates: a NULL workspace is an argument error for
    every call that needs scratch space, caught before any HIP call."""
    assert chunk(lib, ws=None, wsb=0) == kda.KDA_EINVAL
    assert chunk(lib, ws=None, wsb=1 << 30) == kda.KDA_EINVAL
    assert chunk(lib, ws=None, T=0, S_T=FAKE) == kda.KDA_EINVAL
    assert lib.kda_chunk_bwd(*([FAKE] * 5 + [None, FAKE, None] + [FAKE] * 5 + [None, 1, 2, 8, 16, 16, None, 0,
                                                                                  kda.KDA_BF16, 0, None, 0, None])) \
        == kda.KDA_EINVAL
    assert lib.kda_gauge_fold(*([FAKE] * 6 + [None, 1, 2, 8, 16, None, 0, kda.KDA_BF16, 0, None, 0, None])) \
        == kda.KDA_EINVAL
    assert lib.kda_chunk_fwd_gauge(*([FAKE] * 5 + [None, FAKE, None, 1, 2, 8, 16, 16, 16, None, 0, kda.KDA_BF16, 0,
                                                   None, 0, None])) == kda.KDA_EINVAL


def test_status_word_mapping(lib):
    """The forward's status word (first 4 bytes of its workspace) maps to
    KDA_OK when zero and to KDA_EWAIT when a state-pass wait expired."""
    assert lib.kda_chunk_fwd_status(0) == kda.KDA_OK
    assert kda.status_from_word(0) == kda.KDA_OK
    for word in (1, 3, 0x80000001, 0xFFFFFFFF):
        assert kda.status_from_word(word) == kda.KDA_EWAIT
    assert "wait" in kda.strerror(kda.KDA_EWAIT)


def _cpu_inputs(B=1, T=8, H=2, dk=16, dv=16, scalar=False):
    import torch
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)  # noqa: E731
    return dict(q=z(B, T, H, dk), k=z(B, T, H, dk), v=z(B, T, H, dv),
                gate=z(B, T, H) if scalar else z(B, T, H, dk), beta=z(B, T, H))


def test_binding_rejects_mismatched_shapes(lib):
    """The Python binding checks every tensor's full shape (and the gate's
    rank against gate_kind) before it touches a device: a short v, a wrong
    gate rank or a mismatched S0 would otherwise let a kernel read past an
    allocation."""
    import torch
    base = _cpu_inputs()
    bad = [
        dict(k=torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16)),
        dict(v=torch.zeros(1, 7, 2, 16, dtype=torch.bfloat16)),
        dict(gate=torch.zeros(1, 8, 2, 8, dtype=torch.bfloat16)),
        dict(gate=torch.zeros(1, 8, 2, 16, 1, dtype=torch.bfloat16)),
        dict(beta=torch.zeros(1, 8, 3, dtype=torch.bfloat16)),
        dict(beta=torch.zeros(1, 8, 2, 1, dtype=torch.bfloat16)),
    ]
    for change in bad:
        a = dict(base, **change)
        with pytest.raises(ValueError):
            kda.chunk_fwd(**a)
        with pytest.raises(ValueError):
            kda.chunk_fwd_gauge(**a)
        with pytest.raises(ValueError):
            kda.chunk_bwd(**a, dO=torch.zeros(1, 8, 2, 16))
    # scalar gate passed with the channel kind, channel gate with the scalar kind
    with pytest.raises(ValueError):
        kda.chunk_fwd(**_cpu_inputs(scalar=True), gate_kind=kda.GATE_CHANNEL)
    with pytest.raises(ValueError):
        kda.chunk_fwd(**base, gate_kind=kda.GATE_SCALAR)
    with pytest.raises(ValueError):
        kda.gauge_fold(base["q"], base["k"], base["gate"], gate_kind=kda.GATE_SCALAR)
    with pytest.raises(ValueError):
        kda.gauge_fold(base["q"], base["k"][:, :4].contiguous(), base["gate"])
    # states
    with pytest.raises(ValueError):
        kda.chunk_fwd(**base, S0=torch.zeros(1, 2, 16, 8))
    with pytest.raises(ValueError):
        kda.chunk_fwd_gauge(**base, S0=torch.zeros(2, 2, 16, 16))
    with pytest.raises(ValueError):
        kda.chunk_fwd(**base, S0=torch.zeros(1, 2, 16, 16, dtype=torch.float64))
    with pytest.raises(ValueError):
        kda.chunk_bwd(**base, dO=torch.zeros(1, 8, 2, 8))
    with pytest.raises(ValueError):
        kda.chunk_bwd(**base, dO=torch.zeros(1, 8, 2, 16), dS_T=torch.zeros(1, 2, 8, 16))
    # varlen needs B = 1
    b2 = _cpu_inputs(B=2)
    with pytest.raises(ValueError):
        kda.chunk_fwd(**b2, cu_seqlens=torch.tensor([0, 4, 8], dtype=torch.int32))
    # decode
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)  # noqa: E731
    S = torch.zeros(3, 2, 16, 16)
    dec = dict(q=z(3, 2, 16), k=z(3, 2, 16), v=z(3, 2, 16), gate=z(3, 2, 16), beta=z(3, 2), S=S)
    for change in (dict(k=z(3, 2, 32)), dict(v=z(2, 2, 16)), dict(gate=z(3, 2, 8)), dict(beta=z(3, 1)),
                   dict(S=torch.zeros(3, 2, 16, 32)), dict(gate=z(3, 2, 16, 1))):
        with pytest.raises(ValueError):
            kda.decode_step(**dict(dec, **change))
    with pytest.raises(ValueError):
        kda.decode_step(**dict(dec, gate=z(3, 2)), gate_kind=kda.GATE_CHANNEL)


def test_erase_write_validation(lib):
    args = ("q", "k", "v", "gate", "erase", "write", "S0", "o", "S_T", "B", "H", "T", "dk", "dv", "chunk", "cu", "N",
            "dtype", "gate_kind", "ws", "wsb", "stream")

    def fwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, erase=FAKE, write=FAKE, S0=None, o=FAKE, S_T=None, B=1, H=2, T=8,
                 dk=16, dv=16, chunk=16, cu=None, N=0, dtype=kda.KDA_BF16, gate_kind=0, ws=FAKE, wsb=1 << 30,
                 stream=None)
        a.update(kw)
        return lib.kda_chunk_fwd_ew(*[a[x] for x in args])
    assert fwd(B=0) == kda.KDA_EINVAL
    assert fwd(dk=48) == kda.KDA_ENOTSUP
    assert fwd(erase=None) == kda.KDA_EINVAL
    assert fwd(write=None) == kda.KDA_EINVAL
    assert fwd(erase=FAKE + 4) == kda.KDA_EALIGN
    assert fwd(write=FAKE + 2) == kda.KDA_EALIGN
    assert fwd(ws=None) == kda.KDA_EINVAL
    assert fwd(wsb=1) == kda.KDA_EINVAL

    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, erase=FAKE, write=FAKE, S=FAKE, o=FAKE, N=2, H=2, dk=16, dv=16,
                 dtype=kda.KDA_BF16, gate_kind=0, stream=None)
        a.update(kw)
        return lib.kda_decode_step_ew(*a.values())
    assert dec(N=0) == kda.KDA_EINVAL
    assert dec(erase=None) == kda.KDA_EINVAL
    assert dec(write=None) == kda.KDA_EINVAL
    assert dec(erase=FAKE + 1) == kda.KDA_EALIGN
    assert dec(S=FAKE + 4) == kda.KDA_EALIGN
    assert dec(gate_kind=5) == kda.KDA_ENOTSUP


def test_erase_write_bwd_validation(lib):
    def bwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, erase=FAKE, write=FAKE, S0=None, dO=FAKE, dST=None, gq=FAKE,
                 gk=FAKE, gv=FAKE, gg=FAKE, ge=FAKE, gw=FAKE, gS0=None, B=1, H=2, T=8, dk=16, dv=16, cu=None, N=0,
                 dtype=kda.KDA_BF16, gate_kind=0, ws=FAKE, wsb=1 << 30, stream=None)
        a.update(kw)
        return lib.kda_chunk_bwd_ew(*a.values())
    assert bwd(B=0) == kda.KDA_EINVAL
    assert bwd(dk=24) == kda.KDA_ENOTSUP
    assert bwd(dtype=5) == kda.KDA_ENOTSUP
    assert bwd(gate_kind=3) == kda.KDA_ENOTSUP
    assert bwd(erase=None) == kda.KDA_EINVAL
    assert bwd(write=None) == kda.KDA_EINVAL
    assert bwd(ge=None) == kda.KDA_EINVAL
    assert bwd(gw=None) == kda.KDA_EINVAL
    assert bwd(erase=FAKE + 1) == kda.KDA_EALIGN
    assert bwd(gw=FAKE + 4) == kda.KDA_EALIGN                         # grad_write is written 16 bytes at a time
    assert bwd(dO=FAKE + 4) == kda.KDA_EALIGN
    assert bwd(ws=None) == kda.KDA_EINVAL                             # the library never allocates
    assert bwd(wsb=1) == kda.KDA_EINVAL
    assert bwd(cu=FAKE, B=2, N=2) == kda.KDA_EINVAL
    # one more per-row partial sum (de) in place of dbeta's: more workspace than the beta form
    w = kda.bwd_ew_workspace_bytes(1, 2, 64, 16, 16)
    assert w > kda.bwd_workspace_bytes(1, 2, 64, 16, 16) and w % 256 == 0
    assert kda.bwd_ew_workspace_bytes(1, 2, 64, 24, 16) == 0
    assert kda.bwd_ew_workspace_bytes(2, 2, 64, 16, 16, N=2, varlen=True) == 0


def test_lds_poison_build_exports_every_declared_symbol():
    """The LDS-poisoning debug build is the same library: it loads and exports
    every declared symbol (its GPU test runs the kernels through it)."""
    from gated_delta_rule_46_amd import build
    if not os.path.exists(build.POISON_LIB):
        build.build(poison=True)
    plib = kda.load(build.POISON_LIB)
    for n in declared_functions():
        assert hasattr(plib, n), n
    assert plib.kda_version() == 100
