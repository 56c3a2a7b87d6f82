"""torch-tensor front end of libattn.

PyTorch only provides device memory and the current stream here: every
function checks tensor dtypes/devices/contiguity, allocates the outputs with
torch, and hands raw pointers to the C ABI, which launches libattn's own
kernels.  A non-zero status raises :class:`AttnError`.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import AttnError

_SUFFIX = {torch.bfloat16: "bf16", torch.float32: "f32"}


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(t: torch.Tensor, name: str, dtype=None, ndim=4):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libattn has no CPU path)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise(code: int, name: str):
    if code != _lib.ATTN_OK:
        raise AttnError(code, name)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = True, scale: float | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True, window: int | None = None,
        block_mask: torch.Tensor | None = None):
    """Fused attention forward.  q ``[B,Hq,S,D]``, k/v ``[B,Hkv,S,D]``, bf16 or fp32.

    Returns ``(out, lse)``; ``lse`` is float32 ``[B,Hq,S]`` (None if ``lse=False``).
    ``scale`` defaults to 1/sqrt(D).  ``window`` (bf16, causal only): each query
    sees its own key and the ``window - 1`` before it (``attn_fwd_local_bf16``).
    ``block_mask`` (bf16): bool or uint8 ``[Bm, Hm, nb, nb]`` on the device,
    nb = ceil(S / 64), Bm in (1, B), Hm in (1, Hq) (size-1 or stride-0 axes
    broadcast), last two axes contiguous; nonzero = the 64 x 64 block of
    (query, key) pairs is visible, combined with ``causal``
    (``attn_fwd_blockmask_bf16``).  Queries that see no key: out 0, lse -inf.
    """
    if q.dtype not in _SUFFIX:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(t, n, q.dtype)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D) or tuple(v.shape) != (B, Hkv, S, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q.dtype)
    if lse is True:
        lse = torch.empty((B, Hq, S), device=q.device, dtype=torch.float32)
    elif lse is False:
        lse = None
    elif lse is not None:
        _check(lse, "lse", torch.float32, 3)
    lp = lse.data_ptr() if lse is not None else None
    if block_mask is not None:
        if q.dtype != torch.bfloat16 or window is not None:
            raise ValueError("a block mask needs bf16 tensors and no window")
        nb = (S + 63) // 64
        m = block_mask
        if m.dtype == torch.bool:
            m = m.view(torch.uint8)
        if m.dtype != torch.uint8 or m.device != q.device or m.dim() != 4:
            raise ValueError("block_mask must be a 4-d bool or uint8 tensor on q's device")
        if tuple(m.shape[2:]) != (nb, nb) or m.shape[0] not in (1, B) or m.shape[1] not in (1, Hq):
            raise ValueError(f"block_mask shape {tuple(m.shape)}: expected [1 or {B}, 1 or {Hq}, {nb}, {nb}]")
        if m.stride(3) != 1 or m.stride(2) != nb:
            raise ValueError("block_mask: the last two axes must be contiguous")
        sb = m.stride(0) if m.shape[0] > 1 else 0
        sh = m.stride(1) if m.shape[1] > 1 else 0
        code = _lib.attn_fwd_blockmask_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp,
                                            m.data_ptr(), sb, sh, B, Hq, Hkv, S, D, float(scale),
                                            int(bool(causal)), _stream(q.device))
        _raise(code, "attn_fwd_blockmask_bf16")
        return out, lse
    if window is not None:
        if q.dtype != torch.bfloat16 or not causal:
            raise ValueError("a sliding window needs bf16 tensors and causal=True")
        code = _lib.attn_fwd_local_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp,
                                        B, Hq, Hkv, S, D, float(scale), int(window), _stream(q.device))
        _raise(code, "attn_fwd_local_bf16")
        return out, lse
    fn = getattr(_lib, "attn_fwd_" + _SUFFIX[q.dtype])
    code = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp,
              B, Hq, Hkv, S, D, float(scale), int(bool(causal)), _stream(q.device))
    _raise(code, "attn_fwd_" + _SUFFIX[q.dtype])
    return out, lse


def qk_gemm(q: torch.Tensor, k: torch.Tensor, scores: torch.Tensor | None = None) -> torch.Tensor:
    """Step 1: float32 scores ``[B,Hq,S,S]`` = q k^T (unscaled, unmasked)."""
    if q.dtype not in _SUFFIX:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if scores is None:
        scores = torch.empty((B, Hq, S, S), device=q.device, dtype=torch.float32)
    else:
        _check(scores, "scores", torch.float32)
    fn = getattr(_lib, "attn_qk_gemm_" + _SUFFIX[q.dtype])
    _raise(fn(q.data_ptr(), k.data_ptr(), scores.data_ptr(), B, Hq, Hkv, S, D, _stream(q.device)),
           "attn_qk_gemm_" + _SUFFIX[q.dtype])
    return scores


def masked_softmax(scores: torch.Tensor, *, scale: float, causal: bool = True, dtype=torch.bfloat16,
                   p: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True):
    """Steps 2-4: p = softmax(scale * scores + mask) in ``dtype``; returns ``(p, lse)``."""
    _check(scores, "scores", torch.float32)
    B, H, S, S2 = scores.shape
    if S != S2:
        raise ValueError("scores must be [B,H,S,S]")
    if dtype not in _SUFFIX:
        raise TypeError(f"unsupported dtype {dtype}")
    if p is None:
        p = torch.empty((B, H, S, S), device=scores.device, dtype=dtype)
    else:
        _check(p, "p", dtype)
    if lse is True:
        lse = torch.empty((B, H, S), device=scores.device, dtype=torch.float32)
    elif lse is False:
        lse = None
    fn = getattr(_lib, "attn_masked_softmax_" + _SUFFIX[dtype])
    _raise(fn(scores.data_ptr(), p.data_ptr(), lse.data_ptr() if lse is not None else None, B, H, S, float(scale),
              int(bool(causal)), _stream(scores.device)), "attn_masked_softmax_" + _SUFFIX[dtype])
    return p, lse


def pv_gemm(p: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Step 5: out ``[B,Hq,S,D]`` = p v in p's dtype."""
    if p.dtype not in _SUFFIX:
        raise TypeError(f"unsupported dtype {p.dtype}")
    _check(p, "p", p.dtype)
    _check(v, "v", p.dtype)
    B, Hq, S, _ = p.shape
    Hkv, D = v.shape[1], v.shape[3]
    if out is None:
        out = torch.empty((B, Hq, S, D), device=p.device, dtype=p.dtype)
    else:
        _check(out, "out", p.dtype)
    fn = getattr(_lib, "attn_pv_gemm_" + _SUFFIX[p.dtype])
    _raise(fn(p.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, S, D, _stream(p.device)),
           "attn_pv_gemm_" + _SUFFIX[p.dtype])
    return out


def unfused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = True, scale: float | None = None):
    """The three unfused steps back to back (three launches).  Returns ``(out, lse)``."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    scores = qk_gemm(q, k)
    p, lse = masked_softmax(scores, scale=scale, causal=causal, dtype=q.dtype)
    del scores
    return pv_gemm(p, v), lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, causal: bool = True, scale: float | None = None, delta: torch.Tensor | None = None):
    """Gradients of the fused forward (bf16).  ``out``, ``lse``: the forward's
    results for the same q, k, v, causal and scale; ``dout``: dL/dout.

    Returns ``(dq, dk, dv)``, bf16, shaped like q, k, v.  ``delta`` (float32
    ``[B,Hq,S]``, optional) is the workspace; it is allocated when absent.
    """
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check(t, n, torch.bfloat16)
    _check(lse, "lse", torch.float32, 3)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D) or tuple(v.shape) != (B, Hkv, S, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, S):
        raise ValueError("out/dout must be shaped like q and lse [B,Hq,S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if delta is None:
        delta = torch.empty((B, Hq, S), device=q.device, dtype=torch.float32)
    else:
        _check(delta, "delta", torch.float32, 3)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    code = _lib.attn_bwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                              lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                              B, Hq, Hkv, S, D, float(scale), int(bool(causal)), _stream(q.device))
    _raise(code, "attn_bwd_bf16")
    return dq, dk, dv


def fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = True,
                scale: float | None = None, nsplit: int | None = None, workspace: torch.Tensor | None = None,
                out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True):
    """Split-KV forward (bf16): q ``[B,Hq,Sq,D]`` against k, v ``[B,Hkv,Skv,D]``
    with Sq <= Skv; the queries are the last Sq positions (a decode step).

    Returns ``(out, lse)``.  ``nsplit`` defaults to the library's suggestion;
    ``workspace`` (float32, ``attn_splitkv_workspace_bytes`` bytes) is
    allocated when absent.
    """
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(t, n, torch.bfloat16)
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Skv, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if nsplit is None:
        nsplit = _lib.attn_splitkv_default_splits(B, Hq, Hkv, Sq, Skv)
    nbytes = _lib.attn_splitkv_workspace_bytes(B, Hq, Sq, D, nsplit)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4) // 4,), device=q.device, dtype=torch.float32)
    elif workspace.dtype != torch.float32 or workspace.numel() * 4 < nbytes or not workspace.is_contiguous():
        raise ValueError(f"workspace must be contiguous float32 of at least {nbytes} bytes")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16)
    if lse is True:
        lse = torch.empty((B, Hq, Sq), device=q.device, dtype=torch.float32)
    elif lse is False:
        lse = None
    elif lse is not None:
        _check(lse, "lse", torch.float32, 3)
    code = _lib.attn_fwd_splitkv_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                                      B, Hq, Hkv, Sq, Skv, D, float(scale), int(bool(causal)), int(nsplit),
                                      _stream(q.device))
    _raise(code, "attn_fwd_splitkv_bf16")
    return out, lse


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_scale: float, k_scale: float, v_scale: float, *,
            causal: bool = True, scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | bool | None = True):
    """fp8 forward: q ``[B,Hq,S,D]``, k/v ``[B,Hkv,S,D]`` hold e4m3fn codes
    (``torch.uint8`` or ``torch.float8_e4m3fn``) with per-tensor scales.
    Returns ``(out, lse)``; out is bf16."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must hold e4m3fn codes (uint8 or float8_e4m3fn), got {t.dtype}")
        _check(t, n)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D) or tuple(v.shape) != (B, Hkv, S, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, S, D), device=q.device, dtype=torch.bfloat16)
    else:
        _check(out, "out", torch.bfloat16)
    if lse is True:
        lse = torch.empty((B, Hq, S), device=q.device, dtype=torch.float32)
    elif lse is False:
        lse = None
    elif lse is not None:
        _check(lse, "lse", torch.float32, 3)
    code = _lib.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None, B, Hq, Hkv, S, D, float(scale),
                             float(q_scale), float(k_scale), float(v_scale), int(bool(causal)), _stream(q.device))
    _raise(code, "attn_fwd_fp8")
    return out, lse
