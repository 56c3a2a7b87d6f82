"""CPU fp64 oracle for causal scaled dot-product attention (test infrastructure).

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package.  The HIP library never loads it, and it never loads the
HIP library: the two share no code.  The arithmetic lives in
``attn_oracle.c`` (plain C, double precision, POSIX threads); this module only
compiles it with gcc and marshals numpy arrays.

Functions and the passages they follow (four web pages on attention
profiling; each function's C counterpart states the definition it writes out):

* ``attn_fwd``   -- softmax(scale * q k^T + causal mask) v and the per-row
  log-sum-exp: the formula in the ainews.cool "technical deep-dive", with the
  five-step causal pipeline of the Hugging Face article's "Naive Attention"
  section (insight.aitobox.com rendering).
* ``attn_fwd_local`` -- the same with a causal sliding window (query i sees
  its own key and the window - 1 before it): one of the special masks that
  the ai-manual.ru tutorial names as the reason for custom kernels.
* ``attn_fwd_blockmask`` -- the same with a block mask (one flag per block
  of 64 queries x 64 keys, combined with the causal mask): the block-sparse
  masks of the same passages.  Rows with no visible key: out 0, lse -inf.
* ``attn_fwd_kv`` -- Sq queries against Skv >= Sq keys and values, the
  queries being the last Sq positions (a decode step; the split-KV path).
* ``attn_spread`` -- the spread of v around out under the attention weights
  (no output of the method: the ingredient of the fp8 path's error bound).
* ``qk_scores``  -- step 1 of that pipeline (q k^T, unscaled).
* ``masked_softmax`` -- steps 2-4 (scale, mask with -inf, softmax).
* ``pv``         -- step 5 (attn v).
* ``attn_bwd`` (with ``attn_bwd_rows`` / ``attn_bwd_keys`` for sampled rows)
  -- dq, dk, dv: the chain-rule derivative of ``attn_fwd`` for a given
  gradient of its output (no gradient reaches lse).  The pages only warn
  that the flash backward is easy to get wrong (ai-manual.ru tutorial,
  section 6).

Every function is pinned by tests in ``tests/test_oracle_pins.py`` against
closed forms, invariants, hand-derived fixtures and independent library
routines; see that file for which pin covers which part.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "attn_oracle.c"
LIB = HERE / "liboracle.so"

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def compile_oracle(out: Path = LIB, plant: int = 0) -> Path:
    """Compile the oracle with gcc.  ``plant`` selects a deliberate-mistake
    variant (tests only); 0 is the real oracle."""
    out = Path(out)
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           f"-DORACLE_PLANT={int(plant)}", str(SRC), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path = LIB):
        path = Path(path)
        if not path.exists() or (path == LIB and path.stat().st_mtime < SRC.stat().st_mtime):
            compile_oracle(path)  # missing, or older than its source
        self.path = path
        self.lib = ctypes.CDLL(str(path))
        L = self.lib
        L.oracle_attn_fwd_rows.restype = ctypes.c_int
        L.oracle_attn_fwd_rows.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64,
                                           ctypes.c_double, ctypes.c_int, _ptr, _i64, _ptr, _ptr,
                                           ctypes.c_int]
        L.oracle_attn_fwd_local_rows.restype = ctypes.c_int
        L.oracle_attn_fwd_local_rows.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64,
                                                 ctypes.c_double, ctypes.c_int, _i64, _ptr, _i64, _ptr,
                                                 _ptr, ctypes.c_int]
        L.oracle_attn_fwd_blockmask_rows.restype = ctypes.c_int
        L.oracle_attn_fwd_blockmask_rows.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64,
                                                     ctypes.c_double, ctypes.c_int, _ptr, _i64, _i64, _ptr,
                                                     _i64, _ptr, _ptr, ctypes.c_int]
        L.oracle_attn_fwd_kv_rows.restype = ctypes.c_int
        L.oracle_attn_fwd_kv_rows.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _i64,
                                              ctypes.c_double, ctypes.c_int, _ptr, _i64, _ptr, _ptr,
                                              ctypes.c_int]
        L.oracle_attn_fwd_spread_rows.restype = ctypes.c_int
        L.oracle_attn_fwd_spread_rows.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64,
                                                  ctypes.c_double, ctypes.c_int, _ptr, _i64, _ptr, _ptr,
                                                  ctypes.c_int]
        L.oracle_qk_scores_rows.restype = ctypes.c_int
        L.oracle_qk_scores_rows.argtypes = [_ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _ptr, _i64,
                                            _ptr, ctypes.c_int]
        L.oracle_masked_softmax_rows.restype = ctypes.c_int
        L.oracle_masked_softmax_rows.argtypes = [_ptr, _i64, _i64, _i64, ctypes.c_double,
                                                 ctypes.c_int, _ptr, _i64, _ptr, _ptr, ctypes.c_int]
        L.oracle_pv_rows.restype = ctypes.c_int
        L.oracle_pv_rows.argtypes = [_ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _ptr, _i64, _ptr,
                                     ctypes.c_int]
        L.oracle_attn_bwd_rows.restype = ctypes.c_int
        L.oracle_attn_bwd_rows.argtypes = [_ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64,
                                           ctypes.c_double, ctypes.c_int, _ptr, _i64, _ptr, _ptr,
                                           _ptr, ctypes.c_int]
        L.oracle_attn_bwd_keys.restype = ctypes.c_int
        L.oracle_attn_bwd_keys.argtypes = [_ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64,
                                           ctypes.c_double, ctypes.c_int, _ptr, _ptr, _ptr, _i64,
                                           _ptr, _ptr, ctypes.c_int]
        L.oracle_plant_id.restype = ctypes.c_int
        L.oracle_plant_id.argtypes = []

    @property
    def plant(self) -> int:
        return int(self.lib.oracle_plant_id())

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _f32(x) -> np.ndarray:
        a = np.ascontiguousarray(x, dtype=np.float32)
        return a

    @staticmethod
    def _rows(rows, total: int) -> np.ndarray:
        if rows is None:
            return np.arange(total, dtype=np.int64)
        return np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)

    @staticmethod
    def _threads(nthreads):
        if nthreads:
            return int(nthreads)
        try:
            return len(os.sched_getaffinity(0))  # the CPUs this process may run on
        except AttributeError:
            return os.cpu_count() or 1

    @staticmethod
    def _check(rc: int, name: str):
        if rc != 0:
            raise RuntimeError(f"{name} failed with code {rc}")

    # -- attention forward --------------------------------------------------
    def attn_fwd(self, q, k, v, scale: float, causal: bool, rows=None, nthreads=None):
        """out, lse for q ``[B,Hq,S,D]``, k/v ``[B,Hkv,S,D]``.

        With ``rows=None`` returns out ``[B,Hq,S,D]`` and lse ``[B,Hq,S]``;
        otherwise ``rows`` indexes the flattened ``[B,Hq,S]`` row space and
        out is ``[len(rows), D]``, lse ``[len(rows)]``.
        """
        q, k, v = self._f32(q), self._f32(k), self._f32(v)
        B, Hq, S, D = q.shape
        Hkv = k.shape[1]
        assert k.shape == (B, Hkv, S, D) and v.shape == k.shape
        r = self._rows(rows, B * Hq * S)
        out = np.empty((r.size, D), dtype=np.float64)
        lse = np.empty((r.size,), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                           B, Hq, Hkv, S, D, float(scale), int(bool(causal)),
                                           r.ctypes.data, r.size, out.ctypes.data,
                                           lse.ctypes.data, self._threads(nthreads))
        self._check(rc, "oracle_attn_fwd_rows")
        if rows is None:
            return out.reshape(B, Hq, S, D), lse.reshape(B, Hq, S)
        return out, lse

    def attn_fwd_blockmask(self, q, k, v, scale: float, causal: bool, mask, rows=None, nthreads=None):
        """Attention with a block mask: ``mask`` is ``[Bm, Hm, nqb, nkb]``
        (any dtype; nonzero = visible) with Bm in (1, B), Hm in (1, Hq) and
        nqb = nkb = ceil(S / 64); a size-1 batch or head axis broadcasts.
        Same shapes and ``rows`` as ``attn_fwd``."""
        q, k, v = self._f32(q), self._f32(k), self._f32(v)
        B, Hq, S, D = q.shape
        Hkv = k.shape[1]
        assert k.shape == (B, Hkv, S, D) and v.shape == k.shape
        nb = (S + 63) // 64
        m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        assert m.ndim == 4 and m.shape[2:] == (nb, nb) and m.shape[0] in (1, B) and m.shape[1] in (1, Hq)
        msh = nb * nb if m.shape[1] > 1 else 0
        msb = m.shape[1] * nb * nb if m.shape[0] > 1 else 0
        r = self._rows(rows, B * Hq * S)
        out = np.empty((r.size, D), dtype=np.float64)
        lse = np.empty((r.size,), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_blockmask_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                                     B, Hq, Hkv, S, D, float(scale), int(bool(causal)),
                                                     m.ctypes.data, msb, msh, r.ctypes.data, r.size,
                                                     out.ctypes.data, lse.ctypes.data, self._threads(nthreads))
        self._check(rc, "oracle_attn_fwd_blockmask_rows")
        if rows is None:
            return out.reshape(B, Hq, S, D), lse.reshape(B, Hq, S)
        return out, lse

    def attn_fwd_local(self, q, k, v, scale: float, window: int, rows=None, nthreads=None):
        """Causal sliding-window attention: query i sees keys
        max(0, i-window+1)..i.  Same shapes and ``rows`` as ``attn_fwd``."""
        q, k, v = self._f32(q), self._f32(k), self._f32(v)
        B, Hq, S, D = q.shape
        Hkv = k.shape[1]
        assert k.shape == (B, Hkv, S, D) and v.shape == k.shape and int(window) >= 1
        r = self._rows(rows, B * Hq * S)
        out = np.empty((r.size, D), dtype=np.float64)
        lse = np.empty((r.size,), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_local_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                                 B, Hq, Hkv, S, D, float(scale), 1, int(window),
                                                 r.ctypes.data, r.size, out.ctypes.data,
                                                 lse.ctypes.data, self._threads(nthreads))
        self._check(rc, "oracle_attn_fwd_local_rows")
        if rows is None:
            return out.reshape(B, Hq, S, D), lse.reshape(B, Hq, S)
        return out, lse

    def attn_fwd_kv(self, q, k, v, scale: float, causal: bool, rows=None, nthreads=None):
        """q ``[B,Hq,Sq,D]`` against k, v ``[B,Hkv,Skv,D]`` (Sq <= Skv): the queries
        are the last Sq positions, so causal query i sees keys 0..Skv-Sq+i.
        Returns out ``[B,Hq,Sq,D]``, lse ``[B,Hq,Sq]`` (or per listed row)."""
        q, k, v = self._f32(q), self._f32(k), self._f32(v)
        B, Hq, Sq, D = q.shape
        Hkv, Skv = k.shape[1], k.shape[2]
        assert k.shape == (B, Hkv, Skv, D) and v.shape == k.shape
        r = self._rows(rows, B * Hq * Sq)
        out = np.empty((r.size, D), dtype=np.float64)
        lse = np.empty((r.size,), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_kv_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                              B, Hq, Hkv, Sq, Skv, D, float(scale), int(bool(causal)),
                                              r.ctypes.data, r.size, out.ctypes.data, lse.ctypes.data,
                                              self._threads(nthreads))
        self._check(rc, "oracle_attn_fwd_kv_rows")
        if rows is None:
            return out.reshape(B, Hq, Sq, D), lse.reshape(B, Hq, Sq)
        return out, lse

    def attn_spread(self, q, k, v, scale: float, causal: bool, rows=None, nthreads=None):
        """Spread of v around out, per (row, d): sw = sum_j p_j |v_j - out| / l
        and su = sum_j |v_j - out| / l with p_j = exp(s_j - max s), l = sum p_j.
        Bounds how far out moves when the weights are rounded (fp8 path)."""
        q, k, v = self._f32(q), self._f32(k), self._f32(v)
        B, Hq, S, D = q.shape
        Hkv = k.shape[1]
        r = self._rows(rows, B * Hq * S)
        sw = np.empty((r.size, D), dtype=np.float64)
        su = np.empty((r.size, D), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_spread_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                                  B, Hq, Hkv, S, D, float(scale), int(bool(causal)),
                                                  r.ctypes.data, r.size, sw.ctypes.data, su.ctypes.data,
                                                  self._threads(nthreads))
        self._check(rc, "oracle_attn_fwd_spread_rows")
        if rows is None:
            return sw.reshape(B, Hq, S, D), su.reshape(B, Hq, S, D)
        return sw, su

    # -- unfused steps ------------------------------------------------------
    def qk_scores(self, q, k, rows=None, nthreads=None):
        """Unscaled scores q k^T: ``[B,Hq,S,S]`` (or ``[len(rows), S]``)."""
        q, k = self._f32(q), self._f32(k)
        B, Hq, S, D = q.shape
        Hkv = k.shape[1]
        assert k.shape == (B, Hkv, S, D)
        r = self._rows(rows, B * Hq * S)
        out = np.empty((r.size, S), dtype=np.float64)
        rc = self.lib.oracle_qk_scores_rows(q.ctypes.data, k.ctypes.data, B, Hq, Hkv, S, D,
                                            r.ctypes.data, r.size, out.ctypes.data,
                                            self._threads(nthreads))
        self._check(rc, "oracle_qk_scores_rows")
        return out.reshape(B, Hq, S, S) if rows is None else out

    def masked_softmax(self, scores, scale: float, causal: bool, rows=None, nthreads=None):
        """p, lse from fp32 scores ``[B,H,S,S]`` (or per listed row)."""
        x = self._f32(scores)
        B, H, S, S2 = x.shape
        assert S == S2
        r = self._rows(rows, B * H * S)
        p = np.empty((r.size, S), dtype=np.float64)
        lse = np.empty((r.size,), dtype=np.float64)
        rc = self.lib.oracle_masked_softmax_rows(x.ctypes.data, B, H, S, float(scale),
                                                 int(bool(causal)), r.ctypes.data, r.size,
                                                 p.ctypes.data, lse.ctypes.data,
                                                 self._threads(nthreads))
        self._check(rc, "oracle_masked_softmax_rows")
        if rows is None:
            return p.reshape(B, H, S, S), lse.reshape(B, H, S)
        return p, lse

    def pv(self, p, v, rows=None, nthreads=None):
        """out = p v for p ``[B,Hq,S,S]``, v ``[B,Hkv,S,D]``."""
        p, v = self._f32(p), self._f32(v)
        B, Hq, S, S2 = p.shape
        Hkv, D = v.shape[1], v.shape[3]
        assert S == S2 and v.shape == (B, Hkv, S, D)
        r = self._rows(rows, B * Hq * S)
        out = np.empty((r.size, D), dtype=np.float64)
        rc = self.lib.oracle_pv_rows(p.ctypes.data, v.ctypes.data, B, Hq, Hkv, S, D,
                                     r.ctypes.data, r.size, out.ctypes.data,
                                     self._threads(nthreads))
        self._check(rc, "oracle_pv_rows")
        return out.reshape(B, Hq, S, D) if rows is None else out


    # -- backward -----------------------------------------------------------
    def _bwd_args(self, q, k, v, dout):
        q, k, v, dout = self._f32(q), self._f32(k), self._f32(v), self._f32(dout)
        B, Hq, S, D = q.shape
        Hkv = k.shape[1]
        assert k.shape == (B, Hkv, S, D) and v.shape == k.shape and dout.shape == q.shape
        return q, k, v, dout, (B, Hq, Hkv, S, D)

    def attn_bwd_rows(self, q, k, v, dout, scale: float, causal: bool, rows=None, nthreads=None):
        """Pass 1 for query rows (indices into the flattened ``[B,Hq,S]``):
        lse, delta ``[n]`` and dq ``[n, D]``."""
        q, k, v, dout, (B, Hq, Hkv, S, D) = self._bwd_args(q, k, v, dout)
        r = self._rows(rows, B * Hq * S)
        lse = np.empty((r.size,), np.float64)
        delta = np.empty((r.size,), np.float64)
        dq = np.empty((r.size, D), np.float64)
        rc = self.lib.oracle_attn_bwd_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                           dout.ctypes.data, B, Hq, Hkv, S, D, float(scale),
                                           int(bool(causal)), r.ctypes.data, r.size,
                                           lse.ctypes.data, delta.ctypes.data, dq.ctypes.data,
                                           self._threads(nthreads))
        self._check(rc, "oracle_attn_bwd_rows")
        return lse, delta, dq

    def attn_bwd_keys(self, q, k, v, dout, scale: float, causal: bool, lse_all, delta_all,
                      keys=None, nthreads=None):
        """Pass 2 for key rows (indices into the flattened ``[B,Hkv,S]``):
        dk, dv ``[n, D]``.  lse_all, delta_all: pass 1 over every query row."""
        q, k, v, dout, (B, Hq, Hkv, S, D) = self._bwd_args(q, k, v, dout)
        la = np.ascontiguousarray(lse_all, np.float64).reshape(-1)
        da = np.ascontiguousarray(delta_all, np.float64).reshape(-1)
        assert la.size == B * Hq * S and da.size == la.size
        r = self._rows(keys, B * Hkv * S)
        dk = np.empty((r.size, D), np.float64)
        dv = np.empty((r.size, D), np.float64)
        rc = self.lib.oracle_attn_bwd_keys(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                           dout.ctypes.data, B, Hq, Hkv, S, D, float(scale),
                                           int(bool(causal)), la.ctypes.data, da.ctypes.data,
                                           r.ctypes.data, r.size, dk.ctypes.data, dv.ctypes.data,
                                           self._threads(nthreads))
        self._check(rc, "oracle_attn_bwd_keys")
        return dk, dv

    def attn_bwd(self, q, k, v, dout, scale: float, causal: bool, nthreads=None):
        """dq ``[B,Hq,S,D]``, dk and dv ``[B,Hkv,S,D]`` for output gradient dout."""
        B, Hq, S, D = np.shape(q)
        Hkv = np.shape(k)[1]
        lse, delta, dq = self.attn_bwd_rows(q, k, v, dout, scale, causal, nthreads=nthreads)
        dk, dv = self.attn_bwd_keys(q, k, v, dout, scale, causal, lse, delta, nthreads=nthreads)
        return (dq.reshape(B, Hq, S, D), dk.reshape(B, Hkv, S, D), dv.reshape(B, Hkv, S, D))


_DEFAULT = None


def default() -> Oracle:
    """The real (unplanted) oracle, compiled on first use if needed."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(LIB)
        assert _DEFAULT.plant == 0
    return _DEFAULT
