"""torch-tensor front end of libattn.

PyTorch only provides device memory and the current stream here: every
function checks each tensor's dtype, exact shape, contiguity and device (all
on the first input's GPU), allocates the outputs it is not given with torch,
and hands raw pointers to the C ABI, which launches libattn's own kernels.
The C ABI cannot see buffer sizes, so these checks are what keeps an
undersized caller buffer from being written out of bounds.  A non-zero status
raises :class:`AttnError`.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import AttnError

_SUFFIX = {torch.bfloat16: "bf16", torch.float32: "f32"}


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(t: torch.Tensor, name: str, dtype=None, ndim=4, shape=None):
    """Type, dtype, rank, exact shape and contiguity of one tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_gpu(**tensors):
    """Every tensor given (None skipped) on one GPU: the first one's.  Run
    after the shape checks, so those report the same way on any device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (libattn has no CPU path)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


def _lse_arg(lse, shape):
    """``lse=True``: allocate later (returns True); False/None: no lse; a
    tensor: checked."""
    if lse is True:
        return True
    if lse is False or lse is None:
        return None
    _check(lse, "lse", torch.float32, 3, shape)
    return lse


def _alloc_lse(lse, shape, device):
    return torch.empty(shape, device=device, dtype=torch.float32) if lse is True else lse


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
    if not isinstance(q, torch.Tensor) or q.dtype not in _SUFFIX:
        raise TypeError(f"unsupported q: {getattr(q, 'dtype', type(q))}")
    _check(q, "q", q.dtype)
    B, Hq, S, D = q.shape
    _check(k, "k", q.dtype)
    Hkv = k.shape[1]
    _check(k, "k", q.dtype, shape=(B, Hkv, S, D))
    _check(v, "v", q.dtype, shape=(B, Hkv, S, D))
    if out is not None:
        _check(out, "out", q.dtype, shape=q.shape)
    lse = _lse_arg(lse, (B, Hq, S))
    dev = _same_gpu(q=q, k=k, v=v, out=out, lse=lse if lse is not True else None)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    lse = _alloc_lse(lse, (B, Hq, S), dev)
    lp = lse.data_ptr() if lse is not None else None
    if block_mask is not None:
        if q.dtype != torch.bfloat16 or window is not None:
            raise ValueError("a block mask needs bf16 tensors and no window")
        nb = (S + 63) // 64
        m = block_mask
        if m.dtype == torch.bool:
            m = m.view(torch.uint8)
        if m.dtype != torch.uint8 or m.device != dev or m.dim() != 4:
            raise ValueError("block_mask must be a 4-d bool or uint8 tensor on q's device")
        if tuple(m.shape[2:]) != (nb, nb) or m.shape[0] not in (1, B) or m.shape[1] not in (1, Hq):
            raise ValueError(f"block_mask shape {tuple(m.shape)}: expected [1 or {B}, 1 or {Hq}, {nb}, {nb}]")
        if m.stride(3) != 1 or m.stride(2) != nb:
            raise ValueError("block_mask: the last two axes must be contiguous")
        sb = m.stride(0) if m.shape[0] > 1 else 0
        sh = m.stride(1) if m.shape[1] > 1 else 0
        code = _lib.attn_fwd_blockmask_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp,
                                            m.data_ptr(), sb, sh, B, Hq, Hkv, S, D, float(scale),
                                            int(bool(causal)), _stream(dev))
        _raise(code, "attn_fwd_blockmask_bf16")
        return out, lse
    if window is not None:
        if q.dtype != torch.bfloat16 or not causal:
            raise ValueError("a sliding window needs bf16 tensors and causal=True")
        code = _lib.attn_fwd_local_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp,
                                        B, Hq, Hkv, S, D, float(scale), int(window), _stream(dev))
        _raise(code, "attn_fwd_local_bf16")
        return out, lse
    fn = getattr(_lib, "attn_fwd_" + _SUFFIX[q.dtype])
    code = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp,
              B, Hq, Hkv, S, D, float(scale), int(bool(causal)), _stream(dev))
    _raise(code, "attn_fwd_" + _SUFFIX[q.dtype])
    return out, lse


def qk_gemm(q: torch.Tensor, k: torch.Tensor, scores: torch.Tensor | None = None) -> torch.Tensor:
    """Step 1: float32 scores ``[B,Hq,S,S]`` = q k^T (unscaled, unmasked)."""
    if not isinstance(q, torch.Tensor) or q.dtype not in _SUFFIX:
        raise TypeError(f"unsupported q: {getattr(q, 'dtype', type(q))}")
    _check(q, "q", q.dtype)
    B, Hq, S, D = q.shape
    _check(k, "k", q.dtype)
    Hkv = k.shape[1]
    _check(k, "k", q.dtype, shape=(B, Hkv, S, D))
    if scores is not None:
        _check(scores, "scores", torch.float32, shape=(B, Hq, S, S))
    dev = _same_gpu(q=q, k=k, scores=scores)
    if scores is None:
        scores = torch.empty((B, Hq, S, S), device=dev, dtype=torch.float32)
    fn = getattr(_lib, "attn_qk_gemm_" + _SUFFIX[q.dtype])
    _raise(fn(q.data_ptr(), k.data_ptr(), scores.data_ptr(), B, Hq, Hkv, S, D, _stream(dev)),
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
    if p is not None:
        _check(p, "p", dtype, shape=(B, H, S, S))
    lse = _lse_arg(lse, (B, H, S))
    dev = _same_gpu(scores=scores, p=p, lse=lse if lse is not True else None)
    if p is None:
        p = torch.empty((B, H, S, S), device=dev, dtype=dtype)
    lse = _alloc_lse(lse, (B, H, S), dev)
    fn = getattr(_lib, "attn_masked_softmax_" + _SUFFIX[dtype])
    _raise(fn(scores.data_ptr(), p.data_ptr(), lse.data_ptr() if lse is not None else None, B, H, S, float(scale),
              int(bool(causal)), _stream(dev)), "attn_masked_softmax_" + _SUFFIX[dtype])
    return p, lse


def pv_gemm(p: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Step 5: out ``[B,Hq,S,D]`` = p v in p's dtype."""
    if not isinstance(p, torch.Tensor) or p.dtype not in _SUFFIX:
        raise TypeError(f"unsupported p: {getattr(p, 'dtype', type(p))}")
    _check(p, "p", p.dtype)
    B, Hq, S, S2 = p.shape
    if S != S2:
        raise ValueError("p must be [B,Hq,S,S]")
    _check(v, "v", p.dtype)
    Hkv, D = v.shape[1], v.shape[3]
    _check(v, "v", p.dtype, shape=(B, Hkv, S, D))
    if out is not None:
        _check(out, "out", p.dtype, shape=(B, Hq, S, D))
    dev = _same_gpu(p=p, v=v, out=out)
    if out is None:
        out = torch.empty((B, Hq, S, D), device=dev, dtype=p.dtype)
    fn = getattr(_lib, "attn_pv_gemm_" + _SUFFIX[p.dtype])
    _raise(fn(p.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, S, D, _stream(dev)),
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
    _check(q, "q", torch.bfloat16)
    B, Hq, S, D = q.shape
    _check(k, "k", torch.bfloat16)
    Hkv = k.shape[1]
    _check(k, "k", torch.bfloat16, shape=(B, Hkv, S, D))
    _check(v, "v", torch.bfloat16, shape=(B, Hkv, S, D))
    _check(out, "out", torch.bfloat16, shape=q.shape)
    _check(dout, "dout", torch.bfloat16, shape=q.shape)
    _check(lse, "lse", torch.float32, 3, (B, Hq, S))
    if delta is not None:
        _check(delta, "delta", torch.float32, 3, (B, Hq, S))
    dev = _same_gpu(q=q, k=k, v=v, out=out, dout=dout, lse=lse, delta=delta)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if delta is None:
        delta = torch.empty((B, Hq, S), device=dev, dtype=torch.float32)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    code = _lib.attn_bwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                              lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                              B, Hq, Hkv, S, D, float(scale), int(bool(causal)), _stream(dev))
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
    _check(q, "q", torch.bfloat16)
    B, Hq, Sq, D = q.shape
    _check(k, "k", torch.bfloat16)
    Hkv, Skv = k.shape[1], k.shape[2]
    _check(k, "k", torch.bfloat16, shape=(B, Hkv, Skv, D))
    _check(v, "v", torch.bfloat16, shape=(B, Hkv, Skv, D))
    if out is not None:
        _check(out, "out", torch.bfloat16, shape=q.shape)
    lse = _lse_arg(lse, (B, Hq, Sq))
    if nsplit is None:
        nsplit = _lib.attn_splitkv_default_splits(B, Hq, Hkv, Sq, Skv)
    nbytes = _lib.attn_splitkv_workspace_bytes(B, Hq, Sq, D, nsplit)
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.float32
                                  or workspace.numel() * 4 < nbytes or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be contiguous float32 of at least {nbytes} bytes")
    dev = _same_gpu(q=q, k=k, v=v, out=out, lse=lse if lse is not True else None, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4) // 4,), device=dev, dtype=torch.float32)
    if out is None:
        out = torch.empty_like(q)
    lse = _alloc_lse(lse, (B, Hq, Sq), dev)
    code = _lib.attn_fwd_splitkv_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                                      B, Hq, Hkv, Sq, Skv, D, float(scale), int(bool(causal)), int(nsplit),
                                      _stream(dev))
    _raise(code, "attn_fwd_splitkv_bf16")
    return out, lse


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_scale: float, k_scale: float, v_scale: float, *,
            causal: bool = True, scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | bool | None = True):
    """fp8 forward: q ``[B,Hq,S,D]``, k/v ``[B,Hkv,S,D]`` hold e4m3fn codes
    (``torch.uint8`` or ``torch.float8_e4m3fn``) with per-tensor scales.
    Returns ``(out, lse)``; out is bf16."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must hold e4m3fn codes (uint8 or float8_e4m3fn), got {getattr(t, 'dtype', type(t))}")
    _check(q, "q")
    B, Hq, S, D = q.shape
    _check(k, "k")
    Hkv = k.shape[1]
    _check(k, "k", shape=(B, Hkv, S, D))
    _check(v, "v", shape=(B, Hkv, S, D))
    if out is not None:
        _check(out, "out", torch.bfloat16, shape=(B, Hq, S, D))
    lse = _lse_arg(lse, (B, Hq, S))
    dev = _same_gpu(q=q, k=k, v=v, out=out, lse=lse if lse is not True else None)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, S, D), device=dev, dtype=torch.bfloat16)
    lse = _alloc_lse(lse, (B, Hq, S), dev)
    code = _lib.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None, B, Hq, Hkv, S, D, float(scale),
                             float(q_scale), float(k_scale), float(v_scale), int(bool(causal)), _stream(dev))
    _raise(code, "attn_fwd_fp8")
    return out, lse
