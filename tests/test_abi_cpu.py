"""C ABI checks that need no GPU: the library loads, exports every declared symbol, and
rejects bad requests on the host before any device work (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

torch = pytest.importorskip("torch")
import chunkwise_causal_linear_amd as fla  # noqa: E402

BOGUS = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced on error paths
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)


def declared_functions():
    """Every function declared by the public headers (include/*.h)."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            names |= set(re.findall(r"^\s*(?:int|double|const char \*)\s*(fla_\w+)\s*\(",
                                    text, re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fla.LIB_PATH):
        pytest.skip("HIP library not built")
    return fla.load_library()


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(fla.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (fla_\w+)$", out, re.M))
    assert set(declared_functions()) <= exported


def test_library_is_built_for_gfx950():
    if not os.path.exists(fla.LIB_PATH):
        pytest.skip("HIP library not built")
    blob = open(fla.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_status_strings(lib):
    assert fla.status_string(0) == "ok"
    for s in (-1, -2, -3, 42):
        assert isinstance(fla.status_string(s), str) and fla.status_string(s)


def fwd_raw(lib, *, q=BOGUS, k=BOGUS, v=BOGUS, gate=None, init=None, out=BOGUS, fin=None,
            B=1, H=1, T=64, dk=64, dv=64, chunk=64, flags=0):
    return lib.fla_linattn_fwd(q, k, v, gate, init, out, fin, B, H, T, dk, dv, chunk, flags, None)


@pytest.mark.parametrize("kw,expected", [
    (dict(flags=1 << 7), fla.FLA_ERR_INVALID_ARG),                       # unknown flag bit
    (dict(flags=fla.FLA_DECAY_GAMMA | fla.FLA_DECAY_GATE, gate=BOGUS), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=fla.FLA_DECAY_TOKEN | fla.FLA_DECAY_GATE, gate=BOGUS), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=fla.FLA_DECAY_TOKEN | fla.FLA_DECAY_GAMMA, gate=BOGUS), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=fla.FLA_DECAY_TOKEN), fla.FLA_ERR_INVALID_ARG),          # token bit, no values
    (dict(flags=fla.FLA_DECAY_GAMMA), fla.FLA_ERR_INVALID_ARG),          # decay bit, no values
    (dict(gate=BOGUS), fla.FLA_ERR_INVALID_ARG),                          # values, no decay bit
    (dict(q=None), fla.FLA_ERR_INVALID_ARG),
    (dict(out=None), fla.FLA_ERR_INVALID_ARG),
    (dict(B=0), fla.FLA_ERR_INVALID_ARG),
    (dict(H=0), fla.FLA_ERR_INVALID_ARG),
    (dict(T=-1), fla.FLA_ERR_INVALID_ARG),
    (dict(q=MISALIGNED), fla.FLA_ERR_INVALID_ARG),
    (dict(fin=MISALIGNED), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=fla.FLA_DECAY_GATE, gate=MISALIGNED), fla.FLA_ERR_INVALID_ARG),
    (dict(dk=48), fla.FLA_ERR_UNSUPPORTED),
    (dict(dv=512), fla.FLA_ERR_UNSUPPORTED),
    (dict(chunk=2048), fla.FLA_ERR_UNSUPPORTED),
    (dict(chunk=96), fla.FLA_ERR_UNSUPPORTED),
    (dict(chunk=8), fla.FLA_ERR_UNSUPPORTED),
])
def test_fwd_rejects_on_host(lib, kw, expected):
    assert fwd_raw(lib, **kw) == expected


def test_segments_override_rejects_negative(lib):
    rc = lib.fla_linattn_fwd_segments(BOGUS, BOGUS, BOGUS, None, None, BOGUS, None, 1, 1, 64, 64,
                                      64, 64, 0, -1, None)
    assert rc == fla.FLA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,expected", [
    (dict(state=None), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=1 << 9), fla.FLA_ERR_INVALID_ARG),
    (dict(dk=24), fla.FLA_ERR_UNSUPPORTED),
    (dict(q=MISALIGNED), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=fla.FLA_DECAY_GATE), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=fla.FLA_DECAY_TOKEN), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=fla.FLA_DECAY_TOKEN | fla.FLA_DECAY_GATE, gate=BOGUS), fla.FLA_ERR_INVALID_ARG),
])
def test_step_rejects_on_host(lib, kw, expected):
    a = dict(q=BOGUS, k=BOGUS, v=BOGUS, gate=None, state=BOGUS, out=BOGUS, B=1, H=1, dk=64,
             dv=64, flags=0)
    a.update(kw)
    rc = lib.fla_linattn_step(a["q"], a["k"], a["v"], a["gate"], a["state"], a["out"], a["B"],
                              a["H"], a["dk"], a["dv"], a["flags"], None)
    assert rc == expected


def bwd_raw(lib, *, q=BOGUS, k=BOGUS, v=BOGUS, gate=None, init=None, do=BOGUS, dfin=None,
            dq=BOGUS, dk=BOGUS, dv=BOGUS, dg=None, dinit=None, B=1, H=1, T=64, dkd=64, dvd=64,
            chunk=64, flags=0):
    return lib.fla_linattn_bwd(q, k, v, gate, init, do, dfin, dq, dk, dv, dg, dinit, B, H, T,
                               dkd, dvd, chunk, flags, None)


@pytest.mark.parametrize("kw,expected", [
    (dict(flags=fla.FLA_NORMALIZE), fla.FLA_ERR_UNSUPPORTED),
    (dict(chunk=48), fla.FLA_ERR_UNSUPPORTED),
    (dict(chunk=2048), fla.FLA_ERR_UNSUPPORTED),
    (dict(dkd=32), fla.FLA_ERR_UNSUPPORTED),
    (dict(dvd=16), fla.FLA_ERR_UNSUPPORTED),
    (dict(dkd=256), fla.FLA_ERR_UNSUPPORTED),                      # fp32 tiles > LDS
    (dict(flags=fla.FLA_DECAY_GAMMA, gate=BOGUS, dg=BOGUS), fla.FLA_ERR_INVALID_ARG),
    (dict(dg=BOGUS), fla.FLA_ERR_INVALID_ARG),                     # no decay, no gradient
    (dict(flags=fla.FLA_DECAY_GATE), fla.FLA_ERR_INVALID_ARG),     # gate bit, no values
    (dict(dq=None), fla.FLA_ERR_INVALID_ARG),
    (dict(do=None), fla.FLA_ERR_INVALID_ARG),
    (dict(do=MISALIGNED), fla.FLA_ERR_INVALID_ARG),
    (dict(dinit=MISALIGNED), fla.FLA_ERR_INVALID_ARG),
    (dict(T=-1), fla.FLA_ERR_INVALID_ARG),
    (dict(flags=1 << 8), fla.FLA_ERR_INVALID_ARG),
])
def test_bwd_rejects_on_host(lib, kw, expected):
    assert bwd_raw(lib, **kw) == expected


def test_layout_and_varlen_rejects_on_host(lib):
    # token-major rows wider than 2^20 elements
    assert fwd_raw(lib, flags=fla.FLA_LAYOUT_BTHD, H=1 << 14, dk=128, dv=128) == fla.FLA_ERR_UNSUPPORTED
    assert bwd_raw(lib, flags=fla.FLA_LAYOUT_BTHD, H=1 << 14, dkd=128, dvd=128) == fla.FLA_ERR_UNSUPPORTED
    # backward over packed sequences: offsets required and 8-byte aligned, at least one
    # sequence, no normaliser
    bvl = lambda cu, **kw: lib.fla_linattn_bwd_varlen(
        BOGUS, BOGUS, BOGUS, None, None, BOGUS, None, BOGUS, BOGUS, BOGUS, None, None, cu,
        kw.get("n", 1), kw.get("T", 64), 1, 64, 64, 64, kw.get("flags", 0), None)
    assert bvl(None) == fla.FLA_ERR_INVALID_ARG
    assert bvl(ctypes.c_void_p((1 << 20) + 4)) == fla.FLA_ERR_INVALID_ARG
    assert bvl(BOGUS, n=0) == fla.FLA_ERR_INVALID_ARG
    assert bvl(BOGUS, flags=fla.FLA_NORMALIZE) == fla.FLA_ERR_UNSUPPORTED
    assert bvl(BOGUS, flags=fla.FLA_DECAY_GATE) == fla.FLA_ERR_INVALID_ARG   # gate missing
    # packed sequences: offsets required and 8-byte aligned
    vl = lambda cu, **kw: lib.fla_linattn_fwd_varlen(BOGUS, BOGUS, BOGUS, None, None, BOGUS, None,
                                                     cu, kw.get("n", 1), kw.get("T", 64), 1, 64,
                                                     64, 64, kw.get("flags", 0), None)
    assert vl(None) == fla.FLA_ERR_INVALID_ARG
    assert vl(ctypes.c_void_p((1 << 20) + 4)) == fla.FLA_ERR_INVALID_ARG
    assert vl(BOGUS, n=0) == fla.FLA_ERR_INVALID_ARG
    assert vl(BOGUS, flags=fla.FLA_DECAY_GATE) == fla.FLA_ERR_INVALID_ARG   # gate missing


def test_schedule_choice(lib):
    # enough (b, h, 64-wide value slice) units: one streaming launch
    assert fla.segments_for(8, 16, 16384, 128, 128, 64, fla.FLA_BF16 | fla.FLA_DECAY_GATE) == 1
    assert fla.segments_for(32, 4, 2048, 256, 256, 64, fla.FLA_BF16 | fla.FLA_DECAY_GAMMA) == 1
    # 8 heads over a million tokens: the sequence is cut into segments
    assert fla.segments_for(1, 8, 1 << 20, 128, 128, 128, fla.FLA_BF16 | fla.FLA_DECAY_GAMMA) == 64
    # too short to cut
    assert fla.segments_for(1, 1, 256, 64, 64, 64, fla.FLA_PHI_ELU1 | fla.FLA_NORMALIZE) == 1
    # chunk sizes above 128 run as 64-token sub-chunks: the same schedule as chunk 64
    f = fla.FLA_BF16 | fla.FLA_DECAY_GAMMA
    for c in (256, 512, 1024):
        assert fla.segments_for(1, 8, 1 << 20, 128, 128, c, f) == \
            fla.segments_for(1, 8, 1 << 20, 128, 128, 64, f)


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(fla, "_lib", None)
    monkeypatch.setattr(fla, "LIB_PATH", "/nonexistent/libfla_linattn.so")
    with pytest.raises(ImportError):
        fla.load_library()


def test_gdn_rejects_on_host(lib):
    def gdn(**kw):
        a = dict(q=BOGUS, k=BOGUS, v=BOGUS, al=BOGUS, be=BOGUS, init=None, out=BOGUS, fin=None,
                 B=1, H=1, T=64, dk=64, dv=64, chunk=64, flags=0)
        a.update(kw)
        return lib.fla_gdn_fwd(a["q"], a["k"], a["v"], a["al"], a["be"], a["init"], a["out"],
                               a["fin"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["chunk"],
                               a["flags"], None)
    assert gdn(flags=fla.FLA_DECAY_GATE) == fla.FLA_ERR_INVALID_ARG
    assert gdn(flags=fla.FLA_NORMALIZE) == fla.FLA_ERR_INVALID_ARG
    assert gdn(al=None) == fla.FLA_ERR_INVALID_ARG
    assert gdn(be=ctypes.c_void_p((1 << 20) + 2)) == fla.FLA_ERR_INVALID_ARG
    assert gdn(q=MISALIGNED) == fla.FLA_ERR_INVALID_ARG
    assert gdn(T=-1) == fla.FLA_ERR_INVALID_ARG
    assert gdn(chunk=48) == fla.FLA_ERR_UNSUPPORTED
    assert gdn(chunk=2048) == fla.FLA_ERR_UNSUPPORTED
    assert gdn(dk=32) == fla.FLA_ERR_UNSUPPORTED
    assert gdn(dv=96) == fla.FLA_ERR_UNSUPPORTED
    assert gdn(dk=256) == fla.FLA_ERR_UNSUPPORTED
    assert gdn(dk=128) == fla.FLA_ERR_UNSUPPORTED                     # fp32 dk = 128


def test_binding_rejects_strided_and_mistyped_tensors():
    # checked in Python before the library is called, so CPU tensors suffice
    q = torch.zeros(2, 3, 5, 64, dtype=torch.bfloat16)
    state = torch.zeros(2, 3, 64, 64, dtype=torch.float32)
    step_q = q[:, :, 1]                      # the usual decode slice: strided, 16-byte aligned
    assert not step_q.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        fla.step(step_q, step_q.contiguous(), step_q.contiguous(), state)
    with pytest.raises(ValueError, match="contiguous"):
        fla.fwd(q, q, q.transpose(2, 3)[..., :5, :].transpose(2, 3), None)
    qc = step_q.contiguous()
    with pytest.raises(ValueError, match="dtype"):
        fla.step(qc, qc.float(), qc, state)
    with pytest.raises(ValueError, match="float32"):
        fla.step(qc, qc, qc, state.double())
    with pytest.raises(ValueError, match="float32"):
        fla.fwd(q, q, q, torch.ones(2, 3, 5, 64, dtype=torch.bfloat16), decay_kind="gate")
    with pytest.raises(ValueError, match="GPU"):
        fla.step(qc, qc, qc, state)


def test_chunk_pattern_probe_rejects_on_host(lib):
    def pat(**kw):
        a = dict(q=BOGUS, k=BOGUS, g=BOGUS, v=BOGUS, out=BOGUS, B=1, H=1, T=64, dk=128, dv=128)
        a.update(kw)
        return lib.fla_probe_chunk_pattern(a["q"], a["k"], a["g"], a["v"], a["out"], a["B"],
                                           a["H"], a["T"], a["dk"], a["dv"], None)
    assert pat(q=None) == -1
    assert pat(out=MISALIGNED) == -1
    assert pat(dk=64) == -1
    assert pat(dv=96) == -1
    assert pat(dv=512) == -1
    assert pat(T=0) == -1
    assert pat(B=0) == -1
    assert pat(T=(1 << 36) + 1) == -1
