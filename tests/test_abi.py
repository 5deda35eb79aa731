"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/had.h, and rejects bad arguments with the documented
status before any HIP call."""

import ctypes
import os
import re

import pytest

import sparse_attention_had_amd as had
from sparse_attention_had_amd import Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    return had.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "had.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(had_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for fn in ["had_pack", "had_attention", "had_logits", "had_select", "had_words_per_row",
               "had_pack_workspace_bytes", "had_forward", "had_forward_workspace_bytes",
               "had_status_string", "had_last_error"]:
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    for fn in declared_functions():
        assert hasattr(lib, fn), fn


@pytest.mark.parametrize("name", ["libhad_popcount.so", "libhad_fusedq.so"])
def test_measurement_builds_export_every_declared_symbol(name):
    """The measurement builds (vector-ALU logit stage; Q's pack inside the
    attention launch) are the same C ABI."""
    path = os.path.join(ROOT, "sparse_attention_had_amd", name)
    assert os.path.exists(path), f"{name} not built"
    alt = ctypes.CDLL(path)
    for fn in declared_functions():
        assert hasattr(alt, fn), fn


def test_words_per_row_and_status_strings(lib):
    assert [lib.had_words_per_row(d) for d in (1, 31, 32, 33, 64, 128, 256)] == [1, 1, 1, 2, 2, 4, 8]
    assert lib.had_status_string(0) == b"HAD_OK"
    assert lib.had_status_string(1) == b"HAD_ERR_INVALID_ARG"
    assert lib.had_status_string(2) == b"HAD_ERR_UNSUPPORTED"
    assert lib.had_status_string(4) == b"HAD_ERR_HIP"


def test_pack_workspace_bytes(lib):
    assert lib.had_pack_workspace_bytes(Shape(1, 1, 128, 64)) >= 16
    assert lib.had_pack_workspace_bytes(Shape(0, 1, 128, 64)) == 0
    big = Shape(8, 12, 1024, 64)
    assert lib.had_forward_workspace_bytes(big) == 2 * lib.had_pack_workspace_bytes(big)
    assert lib.had_forward_workspace_bytes(Shape(1, 0, 1, 1)) == 0


# Fake, never-dereferenced device addresses: every call below must fail its
# host-side checks before anything is enqueued.
A16 = 0x10000
A16B = 0x20000
A16C = 0x30000


def _attn(lib, q=A16, k=A16B, v=A16C, dt=1, shape=(1, 1, 128, 64), topn=32, scale=0.125,
          causal=0, out=0x40000):
    return lib.had_attention(q, k, v, dt, Shape(*shape), topn, scale, causal, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID),
    (dict(k=None), INVALID),
    (dict(v=None), INVALID),
    (dict(out=None), INVALID),
    (dict(q=A16 + 2), INVALID),          # qbits not 4-byte aligned
    (dict(v=A16C + 4), INVALID),         # v not 16-byte aligned
    (dict(out=0x40000 + 8), INVALID),    # out not 16-byte aligned
    (dict(dt=7), INVALID),
    (dict(topn=0), INVALID),
    (dict(topn=-3), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(causal=2), INVALID),
    (dict(shape=(0, 1, 128, 64)), INVALID),
    (dict(shape=(1, 1, 128, 0)), INVALID),
    (dict(shape=(1, -1, 128, 64)), INVALID),
    (dict(shape=(1, 1, 128, 257)), UNSUPPORTED),
    (dict(shape=(1, 1, 65537, 64)), UNSUPPORTED),
])
def test_attention_rejects_bad_arguments(lib, kw, status):
    assert _attn(lib, **kw) == status
    assert lib.had_last_error() != b""


def test_pack_rejects_bad_arguments(lib):
    s = Shape(1, 1, 128, 64)
    assert lib.had_pack(None, s, A16, None, None, 0, None, None) == INVALID
    assert lib.had_pack(A16, s, None, None, None, 0, None, None) == INVALID
    assert lib.had_pack(A16 + 1, s, A16B, None, None, 0, None, None) == INVALID
    # sigma requested without (or with a too small) workspace
    assert lib.had_pack(A16, s, A16B, A16C, None, 0, None, None) == INVALID
    assert lib.had_pack(A16, s, A16B, A16C, 0x50000, 8, None, None) == INVALID
    assert lib.had_pack(A16, Shape(1, 1, 0, 64), A16B, None, None, 0, None, None) == INVALID
    assert lib.had_pack(A16, Shape(1, 1, 8, 300), A16B, None, None, 0, None, None) == UNSUPPORTED
    # key caches longer than the attention limit can be packed, up to the cache limit
    assert lib.had_pack_workspace_bytes(Shape(1, 1, 70000, 64)) > 0
    assert lib.had_pack(A16, Shape(1, 1, (1 << 22) + 1, 64), A16B, None, None, 0, None, None) == UNSUPPORTED


def _fwd(lib, q=A16, k=0x40000, v=0x60000, vdt=1, shape=None, topn=8, scale=0.125, causal=0,
         qb=0x70000, kb=0x80000, out=0x90000, sq=None, sk=None, ws=None, wsb=0, st=None):
    shape = shape or Shape(1, 2, 100, 64)
    return lib.had_forward(q, k, v, vdt, shape, topn, scale, causal, qb, kb, out, sq, sk, ws, wsb,
                           st, None)


def test_forward_rejects_bad_arguments(lib):
    assert _fwd(lib, q=None) == INVALID
    assert _fwd(lib, k=A16 + 2) == INVALID
    assert _fwd(lib, qb=None) == INVALID
    assert _fwd(lib, v=A16 + 4) == INVALID
    assert _fwd(lib, out=None) == INVALID
    assert _fwd(lib, topn=0) == INVALID
    assert _fwd(lib, scale=-1.0) == INVALID
    assert _fwd(lib, causal=2) == INVALID
    assert _fwd(lib, vdt=7) == INVALID
    assert _fwd(lib, st=A16 + 2) == INVALID
    # a sigma without (or with a too small / unaligned) workspace
    assert _fwd(lib, sq=0xA0000) == INVALID
    assert _fwd(lib, sk=0xA0000, ws=0xB0000, wsb=16) == INVALID
    assert _fwd(lib, sq=0xA0000, ws=0xB0008, wsb=1 << 20) == INVALID
    assert _fwd(lib, shape=Shape(1, 1, 8, 257)) == UNSUPPORTED
    assert _fwd(lib, shape=Shape(1, 1, 65537, 8)) == UNSUPPORTED
    assert lib.had_last_error() != b""


def test_decode_rejects_bad_arguments(lib):
    D = had.DecodeShape
    ok = D(1, 2, 4, 1000, 1024, 64)
    ws_bytes = lib.had_decode_workspace_bytes(ok)
    assert ws_bytes > 0
    assert lib.had_decode_workspace_bytes(D(1, 2, 4, 1000, 999, 64)) == 0   # k_stride < n_k

    def dec(q=A16, k=A16B, v=A16C, vdt=1, s=ok, p0=996, topn=8, scale=0.125, causal=1,
            out=0x40000, ws=0x100000, wsb=ws_bytes):
        return lib.had_decode(q, k, v, vdt, s, p0, topn, scale, causal, out, ws, wsb, None)

    assert dec(q=None) == INVALID
    assert dec(v=A16C + 2) == INVALID
    assert dec(vdt=5) == INVALID
    assert dec(p0=-1) == INVALID
    assert dec(topn=0) == INVALID
    assert dec(scale=float("nan")) == INVALID
    assert dec(causal=3) == INVALID
    assert dec(ws=None) == INVALID
    assert dec(ws=0x100010) == INVALID
    assert dec(wsb=ws_bytes - 1) == INVALID
    assert dec(s=D(1, 2, 0, 1000, 1024, 64)) == INVALID
    assert dec(s=D(1, 2, 65537, 1000, 1024, 64)) == UNSUPPORTED
    assert dec(s=D(1, 2, 4, 1000, 1024, 300)) == UNSUPPORTED
    assert dec(s=D(1, 2, 4, 1000, (1 << 22) + 1, 64)) == UNSUPPORTED
    assert lib.had_last_error() != b""

    def fwd(q=A16, k=A16B, wsb=ws_bytes, s=ok):
        return lib.had_decode_forward(q, k, A16C, 1, s, 996, 8, 0.125, 1, 0x40000, 0x100000, wsb, None)

    assert fwd(q=None) == INVALID
    assert fwd(q=A16 + 2) == INVALID
    assert fwd(k=None) == INVALID
    assert fwd(wsb=ws_bytes - 1) == INVALID
    assert fwd(s=D(1, 2, 65537, 1000, 1024, 64)) == UNSUPPORTED
    assert lib.had_last_error() != b""


def test_topn_mass_rejects_bad_arguments(lib):
    s = Shape(2, 3, 100, 64)
    f = lib.had_topn_mass
    assert f(A16, A16B, s, 0.125, 0, 0.9, 0, 6, None, None) == INVALID
    assert f(A16, A16B, s, 0.0, 0, 0.9, 0, 6, A16C, None) == INVALID
    assert f(A16, A16B, s, 0.125, 0, 0.0, 0, 6, A16C, None) == INVALID
    assert f(A16, A16B, s, 0.125, 0, float("inf"), 0, 6, A16C, None) == INVALID
    assert f(A16, A16B, s, 0.125, 2, 0.9, 0, 6, A16C, None) == INVALID
    assert f(A16, A16B, s, 0.125, 0, 0.9, 4, 3, A16C, None) == INVALID
    assert f(None, A16B, s, 0.125, 0, 0.9, 0, 6, A16C, None) == INVALID
    assert f(A16, A16B, Shape(2, 3, 100, 300), 0.125, 0, 0.9, 0, 6, A16C, None) == UNSUPPORTED


def test_calibration_rejects_bad_arguments(lib):
    s = Shape(1, 2, 100, 64)
    wsb = lib.had_pack_workspace_bytes(s)
    c = lib.had_pack_calibrate
    assert c(A16, s, A16B, None, 0x50000, wsb, None, None) == INVALID
    assert c(A16, s, A16B, A16C + 4, 0x50000, wsb, None, None) == INVALID
    assert c(A16, s, A16B, A16C, None, wsb, None, None) == INVALID
    assert c(A16, s, A16B, A16C, 0x50000, wsb - 1, None, None) == INVALID
    assert c(None, s, A16B, A16C, 0x50000, wsb, None, None) == INVALID
    assert c(A16, Shape(1, 2, 100, 257), A16B, A16C, 0x50000, wsb, None, None) == UNSUPPORTED
    assert lib.had_sigma_from_state(None, A16, None) == INVALID
    assert lib.had_sigma_from_state(A16, None, None) == INVALID


def test_select_and_logits_reject_bad_ranges(lib):
    s = Shape(2, 3, 100, 64)
    assert lib.had_select(A16, A16B, s, 0, 0, 0, 6, A16C, None) == INVALID
    assert lib.had_select(A16, A16B, s, 8, 0, 0, 7, A16C, None) == INVALID
    assert lib.had_select(A16, A16B, s, 8, 0, -1, 2, A16C, None) == INVALID
    assert lib.had_select(A16, A16B, s, 8, 3, 0, 6, A16C, None) == INVALID
    assert lib.had_select(None, A16B, s, 8, 0, 0, 6, A16C, None) == INVALID
    assert lib.had_logits(A16, A16B, s, 0, 6, 0, 101, A16C, None) == INVALID
    assert lib.had_logits(A16, A16B, s, 5, 2, 0, 10, A16C, None) == INVALID
    assert lib.had_logits(A16, A16B, s, 0, 6, 99, 2, A16C, None) == INVALID
    assert lib.had_logits(A16, A16B, s, 0, 6, 0, 10, None, None) == INVALID


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("HAD_LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(had, "_lib", None)
    with pytest.raises(RuntimeError, match="libhad.so not found"):
        had.load_library()


def test_forward_noalloc_rejects_bad_arguments_before_any_hip_call(lib):
    s = Shape(1, 2, 128, 64)

    def f(q=A16, k=A16B, v=A16C, vdt=1, shape=s, topn=8, scale=0.125, causal=0, qb=0x50000,
          kb=0x60000, out=0x40000, sq=0x70000, sk=0x70010, st=None):
        return lib.had_forward_noalloc(q, k, v, vdt, shape, topn, scale, causal, qb, kb, out, sq, sk,
                                       st, None)

    assert f(q=None) == INVALID
    assert f(k=A16B + 2) == INVALID
    assert f(qb=None) == INVALID
    assert f(out=0x40004) == INVALID
    assert f(vdt=9) == INVALID
    assert f(topn=0) == INVALID
    assert f(scale=-1.0) == INVALID
    assert f(causal=2) == INVALID
    assert f(sq=0x70002) == INVALID
    assert f(st=0x80002) == INVALID
    assert f(shape=Shape(1, 2, 128, 0)) == INVALID
    assert f(shape=Shape(1, 2, 70000, 64)) == UNSUPPORTED
    assert lib.had_last_error() != b""


def test_backward_rejects_bad_arguments(lib):
    s = Shape(2, 3, 100, 64)
    wsb = lib.had_backward_workspace_bytes(s)
    assert wsb >= 2 * 3 * 100 * 20
    assert lib.had_backward_workspace_bytes(Shape(2, 3, 100, 129)) == 0
    assert lib.had_backward_workspace_bytes(Shape(0, 3, 100, 64)) == 0

    def f(qb=A16, kb=A16B, v=A16C, vdt=1, shape=s, topn=8, scale=0.125, causal=0, out=0x40000,
          dout=0x50000, sq=None, sk=None, dq=0x60000, dk=0x70000, dv=0x80000, ws=0x100000, n=wsb):
        return lib.had_backward(qb, kb, v, vdt, shape, topn, scale, causal, out, dout, sq, sk, dq, dk,
                                dv, ws, n, None)

    assert f(qb=None) == INVALID
    assert f(dout=None) == INVALID
    assert f(dv=0x80002) == INVALID
    assert f(sq=0x90002) == INVALID
    assert f(vdt=3) == INVALID
    assert f(topn=0) == INVALID
    assert f(scale=float("inf")) == INVALID
    assert f(causal=2) == INVALID
    assert f(ws=None) == INVALID
    assert f(ws=0x100010) == INVALID
    assert f(n=wsb - 1) == INVALID
    assert f(shape=Shape(2, 3, 100, 129)) == UNSUPPORTED
    assert f(shape=Shape(2, 3, 70000, 64)) == UNSUPPORTED
    assert lib.had_last_error() != b""


def test_soft_forward_and_select_reject_bad_arguments(lib):
    s = Shape(2, 3, 100, 64)
    wsb = lib.had_soft_workspace_bytes(s)
    assert wsb >= 2 * 3 * 100 * 64 * 4  # the soft key rows
    assert lib.had_soft_workspace_bytes(Shape(2, 3, 100, 129)) == 0
    assert lib.had_soft_workspace_bytes(Shape(2, 3, 1025, 64)) == 0
    assert lib.had_soft_workspace_bytes(Shape(0, 3, 100, 64)) == 0

    def f(q=A16, k=A16B, v=A16C, vdt=1, shape=s, topn=8, scale=0.125, c=0.5, causal=0, sq=None, sk=None,
          out=0x40000, ws=0x100000, n=wsb):
        return lib.had_soft_forward(q, k, v, vdt, shape, topn, scale, c, causal, sq, sk, out, ws, n, None)

    assert f(q=None) == INVALID
    assert f(out=None) == INVALID
    assert f(k=0x20002) == INVALID
    assert f(sq=0x90002) == INVALID
    assert f(vdt=3) == INVALID
    assert f(topn=0) == INVALID
    assert f(scale=0.0) == INVALID
    assert f(c=0.0) == INVALID
    assert f(c=float("nan")) == INVALID
    assert f(c=float("inf")) == INVALID
    assert f(causal=2) == INVALID
    assert f(ws=None) == INVALID
    assert f(ws=0x100010) == INVALID
    assert f(n=wsb - 1) == INVALID
    assert f(shape=Shape(2, 3, 100, 129)) == UNSUPPORTED
    assert f(shape=Shape(2, 3, 1025, 64)) == UNSUPPORTED
    assert f(shape=Shape(2, 0, 100, 64)) == INVALID
    assert lib.had_last_error() != b""

    def g(q=A16, k=A16B, shape=s, topn=8, c=0.5, causal=0, b0=0, bc=6, keep=0x40000, ws=0x100000, n=wsb):
        return lib.had_soft_select(q, k, shape, topn, c, causal, None, None, b0, bc, keep, ws, n, None)

    assert g(keep=None) == INVALID
    assert g(b0=-1) == INVALID
    assert g(bc=0) == INVALID
    assert g(b0=3, bc=4) == INVALID
    assert g(c=-1.0) == INVALID
    assert g(n=0) == INVALID
    assert g(shape=Shape(2, 3, 2000, 64)) == UNSUPPORTED
