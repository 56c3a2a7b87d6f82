"""The C-ABI library on the CPU: it loads, exports every symbol include/attn.h
declares, and rejects bad arguments before touching the GPU.

Every call here fails argument checking, which runs before any HIP call, so
no kernel is launched (the device pointers below are fake).
"""
from __future__ import annotations

import ctypes
import re
import subprocess
from pathlib import Path

import pytest

from scaled_dot_product_10_amd import _lib

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "attn.h"

OK, NULL, SHAPE, UNSUP, SCALE, ALIGN, ALIAS = 0, 1, 2, 3, 4, 5, 6

A = 0x7f0000000000  # fake, 16-byte aligned "device" addresses, far apart
Bp = A + (1 << 36)
C = A + (2 << 36)
Dp = A + (3 << 36)
E = A + (4 << 36)


def header_symbols():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_header_symbols_are_exported(L):
    syms = header_symbols()
    assert len(syms) == 24, syms
    nm = subprocess.run(["nm", "-D", "--defined-only", str(_lib.LIB_PATH)], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", nm, flags=re.M))
    missing = [s for s in syms if s not in exported]
    assert not missing, missing
    for s in syms:
        assert hasattr(L, s)


def test_binding_covers_header():
    assert sorted(_lib.SIGNATURES) == header_symbols()


def test_library_links_no_oracle():
    deps = subprocess.run(["ldd", str(_lib.LIB_PATH)], capture_output=True, text=True).stdout
    assert "oracle" not in deps
    nm = subprocess.run(["nm", "-D", str(_lib.LIB_PATH)], capture_output=True, text=True).stdout
    assert "oracle_" not in nm


def test_status_strings(L):
    for code, name in _lib.STATUS.items():
        assert _lib.attn_status_str(code).startswith(name)
    assert "unknown" in _lib.attn_status_str(99)


def test_byte_helpers(L):
    assert _lib.attn_scores_bytes(4, 16, 4096) == 4 * 16 * 4096 * 4096 * 4
    assert _lib.attn_probs_bytes(4, 16, 4096, 2) == 4 * 16 * 4096 * 4096 * 2
    assert _lib.attn_probs_bytes(1, 1, 8, 3) == 0
    assert _lib.attn_scores_bytes(0, 1, 8) == 0
    assert _lib.attn_scores_bytes(1 << 30, 1 << 30, 1 << 30) == 0
    assert _lib.attn_bwd_workspace_bytes(4, 16, 4096) == 4 * 16 * 4096 * 4
    assert _lib.attn_bwd_workspace_bytes(1, 0, 8) == 0


FWD = [_lib.attn_fwd_bf16, _lib.attn_fwd_f32]


def fwd_args(**kw):
    a = dict(q=A, k=Bp, v=C, out=Dp, lse=E, B=1, Hq=2, Hkv=1, S=16, D=64, scale=0.125, causal=1, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "out", "lse", "B", "Hq", "Hkv", "S", "D", "scale", "causal", "stream")]


@pytest.mark.parametrize("fn", FWD, ids=lambda f: f.__name__)
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(out=None), NULL),
    (dict(B=0), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=0), SHAPE), (dict(S=0), SHAPE), (dict(S=-5), SHAPE),
    (dict(Hq=3, Hkv=2), SHAPE), (dict(B=1 << 30, Hq=1 << 30, Hkv=1 << 30), SHAPE),
    (dict(D=32), UNSUP), (dict(D=96), UNSUP), (dict(D=256), UNSUP), (dict(causal=2), UNSUP),
    (dict(causal=-1), UNSUP),
    (dict(scale=float("nan")), SCALE), (dict(scale=float("inf")), SCALE), (dict(scale=0.0), SCALE),
    (dict(scale=-0.1), SCALE),
    (dict(q=A + 8), ALIGN), (dict(k=Bp + 4), ALIGN), (dict(v=C + 2), ALIGN), (dict(out=Dp + 1), ALIGN),
    (dict(lse=E + 2), ALIGN),
    (dict(out=A), ALIAS), (dict(out=Bp + 64), ALIAS), (dict(lse=C + 16), ALIAS), (dict(lse=Dp), ALIAS),
])
def test_fwd_rejects(fn, kw, code):
    assert fn(*fwd_args(**kw)) == code


def test_stamped_rejects():
    f = _lib.attn_fwd_bf16_stamped
    ST = A + (10 << 36)
    # the forward's own checks come first
    assert f(*fwd_args(q=None)[:-1], ST, None) == NULL
    assert f(*fwd_args(D=96)[:-1], ST, None) == UNSUP
    assert f(*fwd_args(out=A)[:-1], ST, None) == ALIAS
    assert f(*fwd_args()[:-1], None, None) == NULL
    assert f(*fwd_args()[:-1], ST + 4, None) == ALIGN
    assert f(*fwd_args()[:-1], A + 64, None) == ALIAS   # stamps over q
    assert f(*fwd_args()[:-1], Dp, None) == ALIAS       # stamps over out
    assert f(*fwd_args()[:-1], E - 8, None) == ALIAS    # stamps running into lse
    # B * Hq * ceil(S / 128) records of 8 words
    assert _lib.attn_fwd_bf16_stamp_bytes(4, 16, 4096) == 4 * 16 * 32 * 8 * 8
    assert _lib.attn_fwd_bf16_stamp_bytes(1, 1, 1) == 64
    assert _lib.attn_fwd_bf16_stamp_bytes(0, 1, 8) == 0


def test_fp8_rejects():
    f = _lib.attn_fwd_fp8
    base = dict(q=A, k=Bp, v=C, out=Dp, lse=E, B=1, Hq=2, Hkv=1, S=16, D=128, scale=0.1, qs=0.01, ks=0.01, vs=0.01,
                causal=1, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return f(*[a[n] for n in ("q", "k", "v", "out", "lse", "B", "Hq", "Hkv", "S", "D", "scale", "qs", "ks", "vs",
                                  "causal", "stream")])

    assert call(q=None) == NULL
    assert call(Hq=3, Hkv=2) == SHAPE
    assert call(D=96) == UNSUP
    assert call(qs=0.0) == SCALE
    assert call(vs=float("inf")) == SCALE
    assert call(scale=1e30, qs=1e30) == SCALE
    assert call(k=Bp + 8) == ALIGN
    assert call(out=Bp) == ALIAS
    assert call(lse=Dp + 64) == ALIAS


def test_local_rejects():
    f = _lib.attn_fwd_local_bf16
    args = [A, Bp, C, Dp, E, 1, 2, 1, 16, 64, 0.125]
    assert f(*args, 0, None) == UNSUP
    assert f(*args, -3, None) == UNSUP
    assert f(None, *args[1:], 4, None) == NULL
    assert f(A, Bp, C, A, E, 1, 2, 1, 16, 64, 0.125, 4, None) == ALIAS
    assert f(A, Bp, C, Dp, E, 1, 2, 1, 16, 64, float("nan"), 4, None) == SCALE


def test_blockmask_rejects():
    f = _lib.attn_fwd_blockmask_bf16
    M = E + (1 << 24)  # a mask range apart from every tensor

    def call(**kw):
        a = dict(q=A, k=Bp, v=C, out=Dp, lse=E, mask=M, sb=0, sh=0, B=2, Hq=4, Hkv=2, S=300, D=64, scale=0.125,
                 causal=1, stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(mask=None) == NULL
    assert call(q=None) == NULL
    assert call(S=131073) == UNSUP
    assert call(D=96) == UNSUP
    assert call(causal=2) == UNSUP
    assert call(sb=-1) == SHAPE
    assert call(sh=-5) == SHAPE
    assert call(sb=1 << 62) == SHAPE
    assert call(scale=float("inf")) == SCALE
    assert call(mask=Dp + 100) == ALIAS  # inside out
    assert call(mask=E + 8) == ALIAS     # inside lse
    assert call(mask=Dp - 10, sb=0, sh=0) == ALIAS  # 25 flags (5 x 5 blocks) reach into out
    assert call(out=Bp) == ALIAS


def test_splitkv_noalloc_rejects():
    """The allocation-free split-KV takes the same checks (no workspace
    argument) and refuses, before any HIP call, a call whose partial results
    would not fit the library's fixed scratch."""
    f = _lib.attn_fwd_splitkv_bf16_noalloc
    TOO_LARGE = 8

    def call(**kw):
        a = dict(q=A, k=Bp, v=C, out=Dp, lse=E, B=1, Hq=4, Hkv=2, Sq=1, Skv=100, D=128, scale=0.1, causal=1,
                 nsplit=4, stream=None)
        a.update(kw)
        return f(*[a[n] for n in ("q", "k", "v", "out", "lse", "B", "Hq", "Hkv", "Sq", "Skv", "D", "scale",
                                  "causal", "nsplit", "stream")])

    cap = _lib.attn_splitkv_noalloc_max_bytes()
    assert cap == 16 << 20
    assert call(q=None) == NULL
    assert call(out=None) == NULL
    assert call(Sq=101) == SHAPE
    assert call(Hq=3) == SHAPE
    assert call(D=80) == UNSUP
    assert call(nsplit=0) == UNSUP
    assert call(scale=0.0) == SCALE
    assert call(lse=E + 2) == ALIGN
    assert call(out=A) == ALIAS
    # 64 x 64 rows x 129 floats x 16 splits = 33.8 MB > 16 MiB
    assert _lib.attn_splitkv_workspace_bytes(1, 64, 64, 128, 16) > cap
    assert call(Hq=64, Hkv=8, Sq=64, Skv=4096, nsplit=16) == TOO_LARGE
    assert _lib.STATUS[TOO_LARGE] == "ATTN_ERR_TOO_LARGE"
    assert _lib.attn_status_str(TOO_LARGE).startswith("ATTN_ERR_TOO_LARGE")


def test_splitkv_rejects_and_sizes():
    f = _lib.attn_fwd_splitkv_bf16
    ws = E + (1 << 30)

    def call(**kw):
        a = dict(q=A, k=Bp, v=C, out=Dp, lse=E, ws=ws, B=1, Hq=4, Hkv=2, Sq=1, Skv=100, D=128, scale=0.1, causal=1,
                 nsplit=4, stream=None)
        a.update(kw)
        return f(*[a[n] for n in ("q", "k", "v", "out", "lse", "ws", "B", "Hq", "Hkv", "Sq", "Skv", "D", "scale",
                                  "causal", "nsplit", "stream")])

    assert call(ws=None) == NULL
    assert call(q=None) == NULL
    assert call(Sq=101) == SHAPE
    assert call(Sq=0) == SHAPE
    assert call(Hq=3) == SHAPE
    assert call(D=80) == UNSUP
    assert call(nsplit=0) == UNSUP
    assert call(nsplit=5000) == UNSUP
    assert call(causal=2) == UNSUP
    assert call(scale=-1.0) == SCALE
    assert call(ws=ws + 4) == ALIGN
    assert call(ws=A) == ALIAS
    assert call(out=Bp) == ALIAS
    assert _lib.attn_splitkv_workspace_bytes(2, 8, 3, 128, 5) == 5 * 2 * 8 * 3 * 129 * 4
    assert _lib.attn_splitkv_workspace_bytes(2, 8, 3, 100, 5) == 0
    assert _lib.attn_splitkv_workspace_bytes(2, 8, 3, 128, 0) == 0
    assert _lib.attn_splitkv_default_splits(8, 32, 8, 1, 4096) == 8     # 64 units -> 8 splits
    assert _lib.attn_splitkv_default_splits(1, 1, 1, 1, 100) == 1       # one 128-key chunk
    assert _lib.attn_splitkv_default_splits(1, 4, 3, 1, 100) == 0


def test_qk_rejects():
    f = _lib.attn_qk_gemm_bf16
    assert f(None, Bp, C, 1, 1, 1, 8, 64, None) == NULL
    assert f(A, Bp, None, 1, 1, 1, 8, 64, None) == NULL
    assert f(A, Bp, C, 1, 2, 3, 8, 64, None) == SHAPE
    assert f(A, Bp, C, 1, 1, 1, 8, 80, None) == UNSUP
    assert f(A, Bp, C + 4, 1, 1, 1, 8, 64, None) == ALIGN
    assert f(A, Bp, A, 1, 1, 1, 8, 64, None) == ALIAS
    assert _lib.attn_qk_gemm_f32(A, Bp, C, 1, 1, 1, 0, 64, None) == SHAPE


def test_softmax_rejects():
    f = _lib.attn_masked_softmax_bf16
    assert f(None, Bp, C, 1, 1, 8, 0.1, 1, None) == NULL
    assert f(A, None, C, 1, 1, 8, 0.1, 1, None) == NULL
    assert f(A, Bp, C, 1, 0, 8, 0.1, 1, None) == SHAPE
    assert f(A, Bp, C, 1, 1, 8, 0.1, 3, None) == UNSUP
    assert f(A, Bp, C, 1, 1, 8, float("nan"), 1, None) == SCALE
    assert f(A, Bp + 8, C, 1, 1, 8, 0.1, 1, None) == ALIGN
    assert f(A, A + 16, C, 1, 1, 8, 0.1, 1, None) == ALIAS
    assert _lib.attn_masked_softmax_f32(A, Bp, A + 4, 1, 1, 8, 0.1, 1, None) == ALIAS


def test_pv_rejects():
    f = _lib.attn_pv_gemm_bf16
    assert f(A, None, C, 1, 1, 1, 8, 64, None) == NULL
    assert f(A, Bp, C, 1, 4, 3, 8, 64, None) == SHAPE
    assert f(A, Bp, C, 1, 1, 1, 8, 100, None) == UNSUP
    assert f(A + 2, Bp, C, 1, 1, 1, 8, 64, None) == ALIGN
    assert f(A, Bp, Bp, 1, 1, 1, 8, 64, None) == ALIAS
    assert _lib.attn_pv_gemm_f32(A, Bp, C, 0, 1, 1, 8, 64, None) == SHAPE


F = A + (5 << 36)
G_ = A + (6 << 36)
H_ = A + (7 << 36)
I_ = A + (8 << 36)
J_ = A + (9 << 36)


def bwd_args(**kw):
    a = dict(q=A, k=Bp, v=C, out=Dp, dout=E, lse=F, dq=G_, dk=H_, dv=I_, delta=J_, B=1, Hq=2, Hkv=1, S=16, D=64,
             scale=0.125, causal=1, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "delta", "B", "Hq", "Hkv", "S",
                           "D", "scale", "causal", "stream")]


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(out=None), NULL), (dict(dout=None), NULL), (dict(lse=None), NULL),
    (dict(dq=None), NULL), (dict(dk=None), NULL), (dict(dv=None), NULL), (dict(delta=None), NULL),
    (dict(B=0), SHAPE), (dict(Hq=3, Hkv=2), SHAPE), (dict(S=0), SHAPE),
    (dict(D=96), UNSUP), (dict(causal=2), UNSUP), (dict(scale=float("nan")), SCALE), (dict(scale=0.0), SCALE),
    (dict(dout=E + 8), ALIGN), (dict(dq=G_ + 2), ALIGN), (dict(delta=J_ + 2), ALIGN), (dict(lse=F + 1), ALIGN),
    (dict(dq=A), ALIAS), (dict(dk=Bp + 32), ALIAS), (dict(dv=E), ALIAS), (dict(delta=F), ALIAS),
    (dict(dk=G_ + 16), ALIAS), (dict(delta=I_), ALIAS),
])
def test_bwd_rejects(kw, code):
    assert _lib.attn_bwd_bf16(*bwd_args(**kw)) == code


def test_missing_library_is_loud(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", tmp_path / "libattn.so")
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.lib()


# ---------------------------------------------------------------------------
# The torch front end checks every tensor's dtype and exact shape before the
# device (the C ABI cannot see buffer sizes, so an undersized out, lse or
# score buffer would otherwise be written out of bounds).  CPU tensors reach
# every shape check here; with correct shapes they stop at the GPU check.
# ---------------------------------------------------------------------------
torch = pytest.importorskip("torch")
from scaled_dot_product_10_amd import api  # noqa: E402


def _t(*shape, dtype=None):
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _raises(match, fn, *a, exc=ValueError, **kw):
    with pytest.raises(exc, match=match):
        fn(*a, **kw)


def test_api_fwd_checks_shapes():
    q, k, v = _t(1, 4, 8, 64), _t(1, 2, 8, 64), _t(1, 2, 8, 64)
    _raises("k must have shape", api.fwd, q, _t(1, 2, 9, 64), v)
    _raises("v must have shape", api.fwd, q, k, _t(1, 2, 8, 32))
    _raises("out must have shape", api.fwd, q, k, v, out=_t(1, 4, 7, 64))
    _raises("lse must have shape", api.fwd, q, k, v, lse=_t(1, 4, 7, dtype=torch.float32))
    _raises("lse must be", api.fwd, q, k, v, lse=_t(1, 4, 8), exc=TypeError)
    _raises("out must be", api.fwd, q, k, v, out=_t(1, 4, 8, 64, dtype=torch.float32), exc=TypeError)
    _raises("must be a GPU tensor", api.fwd, q, k, v)


def test_api_unfused_checks_shapes():
    q, k = _t(1, 2, 8, 64), _t(1, 1, 8, 64)
    _raises("k must have shape", api.qk_gemm, q, _t(1, 1, 8, 128))
    _raises("scores must have shape", api.qk_gemm, q, k, scores=_t(1, 2, 8, 7, dtype=torch.float32))
    _raises("must be a GPU tensor", api.qk_gemm, q, k)
    sc = _t(1, 2, 8, 8, dtype=torch.float32)
    _raises("p must have shape", api.masked_softmax, sc, scale=0.1, p=_t(1, 2, 8, 4))
    _raises("lse must have shape", api.masked_softmax, sc, scale=0.1, lse=_t(1, 2, 9, dtype=torch.float32))
    _raises("must be a GPU tensor", api.masked_softmax, sc, scale=0.1)
    p, v = _t(1, 2, 8, 8), _t(1, 1, 8, 64)
    _raises("p must be", api.pv_gemm, _t(1, 2, 8, 9), v)
    _raises("v must have shape", api.pv_gemm, p, _t(1, 1, 9, 64))
    _raises("v must have shape", api.pv_gemm, p, _t(2, 1, 8, 64))
    _raises("out must have shape", api.pv_gemm, p, v, out=_t(1, 2, 8, 32))
    _raises("must be a GPU tensor", api.pv_gemm, p, v)


def test_api_bwd_splitkv_fp8_check_shapes():
    q, k, v = _t(1, 2, 8, 64), _t(1, 1, 8, 64), _t(1, 1, 8, 64)
    lse = _t(1, 2, 8, dtype=torch.float32)
    _raises("out must have shape", api.bwd, q, k, v, _t(1, 2, 8, 32), lse, q)
    _raises("dout must have shape", api.bwd, q, k, v, q, lse, _t(1, 2, 4, 64))
    _raises("lse must have shape", api.bwd, q, k, v, q, _t(1, 2, 9, dtype=torch.float32), q)
    _raises("delta must have shape", api.bwd, q, k, v, q, lse, q, delta=_t(1, 1, 8, dtype=torch.float32))
    _raises("must be a GPU tensor", api.bwd, q, k, v, q, lse, q)
    qd, kd = _t(1, 2, 1, 64), _t(1, 1, 40, 64)
    _raises("v must have shape", api.fwd_splitkv, qd, kd, _t(1, 1, 39, 64), nsplit=2)
    _raises("out must have shape", api.fwd_splitkv, qd, kd, kd, nsplit=2, out=_t(1, 2, 2, 64))
    _raises("lse must have shape", api.fwd_splitkv, qd, kd, kd, nsplit=2, lse=_t(1, 2, 2, dtype=torch.float32))
    _raises("workspace must be", api.fwd_splitkv, qd, kd, kd, nsplit=2, workspace=_t(1, dtype=torch.float32))
    _raises("must be a GPU tensor", api.fwd_splitkv, qd, kd, kd, nsplit=2)
    u8 = torch.uint8
    q8, k8 = _t(1, 2, 8, 64, dtype=u8), _t(1, 1, 8, 64, dtype=u8)
    _raises("v must have shape", api.fwd_fp8, q8, k8, _t(1, 1, 8, 128, dtype=u8), 1.0, 1.0, 1.0)
    _raises("out must have shape", api.fwd_fp8, q8, k8, k8, 1.0, 1.0, 1.0, out=_t(1, 2, 8, 32))
    _raises("lse must have shape", api.fwd_fp8, q8, k8, k8, 1.0, 1.0, 1.0, lse=_t(2, 2, 8, dtype=torch.float32))
    _raises("must be a GPU tensor", api.fwd_fp8, q8, k8, k8, 1.0, 1.0, 1.0)
