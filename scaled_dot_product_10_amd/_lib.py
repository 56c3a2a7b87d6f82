"""ctypes binding of libattn's C ABI (include/attn.h), one Python function per
C symbol with the same name and the same arguments (device pointers as ints,
the stream as an int handle or None).  Argument marshalling only.

The library must be built (``python -m scaled_dot_product_10_amd.build``);
there is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libattn.so"

ATTN_OK = 0
STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL_POINTER",
    2: "ATTN_ERR_BAD_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_BAD_SCALE",
    5: "ATTN_ERR_MISALIGNED",
    6: "ATTN_ERR_ALIAS",
    7: "ATTN_ERR_HIP",
    8: "ATTN_ERR_TOO_LARGE",
}

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_i64 = ctypes.c_int64

# symbol -> (restype, argtypes)
SIGNATURES = {
    "attn_fwd_bf16": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]),
    "attn_fwd_f32": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]),
    "attn_fwd_bf16_stamped": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _p]),
    "attn_fwd_bf16_stamp_bytes": (ctypes.c_size_t, [_i, _i, _i]),
    "attn_fwd_fp8": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _f, _f, _f, _i, _p]),
    "attn_fwd_local_bf16": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]),
    "attn_fwd_blockmask_bf16": (_i, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i, _i, _i, _i, _i, _f, _i, _p]),
    "attn_qk_gemm_bf16": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "attn_qk_gemm_f32": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "attn_masked_softmax_bf16": (_i, [_p, _p, _p, _i, _i, _i, _f, _i, _p]),
    "attn_masked_softmax_f32": (_i, [_p, _p, _p, _i, _i, _i, _f, _i, _p]),
    "attn_pv_gemm_bf16": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "attn_pv_gemm_f32": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "attn_fwd_splitkv_bf16": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _p]),
    "attn_splitkv_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "attn_splitkv_default_splits": (_i, [_i, _i, _i, _i, _i]),
    "attn_fwd_splitkv_bf16_noalloc": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _p]),
    "attn_splitkv_noalloc_max_bytes": (ctypes.c_size_t, []),
    "attn_bwd_bf16": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]),
    "attn_bwd_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i]),
    "attn_scores_bytes": (ctypes.c_size_t, [_i, _i, _i]),
    "attn_probs_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "attn_status_str": (ctypes.c_char_p, [_i]),
    "attn_last_hip_error": (_i, []),
}

_LIB = None


class AttnError(RuntimeError):
    def __init__(self, code: int, name: str):
        msg = lib().attn_status_str(code).decode()
        if code == 7:
            msg += f" (hipError {lib().attn_last_hip_error()})"
        super().__init__(f"{name}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libattn.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m scaled_dot_product_10_amd.build` "
                "(or __graft_entry__.build()); libattn has no fallback path")
        L = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _call(name: str, *args) -> int:
    return int(getattr(lib(), name)(*args))


def attn_fwd_bf16(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, stream) -> int:
    return _call("attn_fwd_bf16", q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, stream)


def attn_fwd_bf16_stamped(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, stamps, stream) -> int:
    return _call("attn_fwd_bf16_stamped", q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, stamps, stream)


def attn_fwd_bf16_stamp_bytes(B, Hq, S) -> int:
    return int(lib().attn_fwd_bf16_stamp_bytes(B, Hq, S))


def attn_fwd_f32(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, stream) -> int:
    return _call("attn_fwd_f32", q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, stream)


def attn_fwd_fp8(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, q_scale, k_scale, v_scale, causal, stream) -> int:
    return _call("attn_fwd_fp8", q, k, v, out, lse, B, Hq, Hkv, S, D, scale, q_scale, k_scale, v_scale, causal,
                 stream)


def attn_fwd_local_bf16(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, window, stream) -> int:
    return _call("attn_fwd_local_bf16", q, k, v, out, lse, B, Hq, Hkv, S, D, scale, window, stream)


def attn_fwd_blockmask_bf16(q, k, v, out, lse, block_mask, mask_stride_b, mask_stride_h, B, Hq, Hkv, S, D, scale,
                            causal, stream) -> int:
    return _call("attn_fwd_blockmask_bf16", q, k, v, out, lse, block_mask, mask_stride_b, mask_stride_h, B, Hq, Hkv,
                 S, D, scale, causal, stream)


def attn_qk_gemm_bf16(q, k, scores, B, Hq, Hkv, S, D, stream) -> int:
    return _call("attn_qk_gemm_bf16", q, k, scores, B, Hq, Hkv, S, D, stream)


def attn_qk_gemm_f32(q, k, scores, B, Hq, Hkv, S, D, stream) -> int:
    return _call("attn_qk_gemm_f32", q, k, scores, B, Hq, Hkv, S, D, stream)


def attn_masked_softmax_bf16(scores, p, lse, B, H, S, scale, causal, stream) -> int:
    return _call("attn_masked_softmax_bf16", scores, p, lse, B, H, S, scale, causal, stream)


def attn_masked_softmax_f32(scores, p, lse, B, H, S, scale, causal, stream) -> int:
    return _call("attn_masked_softmax_f32", scores, p, lse, B, H, S, scale, causal, stream)


def attn_pv_gemm_bf16(p, v, out, B, Hq, Hkv, S, D, stream) -> int:
    return _call("attn_pv_gemm_bf16", p, v, out, B, Hq, Hkv, S, D, stream)


def attn_pv_gemm_f32(p, v, out, B, Hq, Hkv, S, D, stream) -> int:
    return _call("attn_pv_gemm_f32", p, v, out, B, Hq, Hkv, S, D, stream)


def attn_fwd_splitkv_bf16(q, k, v, out, lse, workspace, B, Hq, Hkv, Sq, Skv, D, scale, causal, nsplit,
                          stream) -> int:
    return _call("attn_fwd_splitkv_bf16", q, k, v, out, lse, workspace, B, Hq, Hkv, Sq, Skv, D, scale, causal,
                 nsplit, stream)


def attn_splitkv_workspace_bytes(B, Hq, Sq, D, nsplit) -> int:
    return int(lib().attn_splitkv_workspace_bytes(B, Hq, Sq, D, nsplit))


def attn_splitkv_default_splits(B, Hq, Hkv, Sq, Skv) -> int:
    return int(lib().attn_splitkv_default_splits(B, Hq, Hkv, Sq, Skv))


def attn_fwd_splitkv_bf16_noalloc(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, nsplit, stream) -> int:
    return _call("attn_fwd_splitkv_bf16_noalloc", q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, nsplit,
                 stream)


def attn_splitkv_noalloc_max_bytes() -> int:
    return int(lib().attn_splitkv_noalloc_max_bytes())


def attn_bwd_bf16(q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, S, D, scale, causal, stream) -> int:
    return _call("attn_bwd_bf16", q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, S, D, scale, causal,
                 stream)


def attn_bwd_workspace_bytes(B, Hq, S) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, S))


def attn_scores_bytes(B, Hq, S) -> int:
    return int(lib().attn_scores_bytes(B, Hq, S))


def attn_probs_bytes(B, Hq, S, elem_bytes) -> int:
    return int(lib().attn_probs_bytes(B, Hq, S, elem_bytes))


def attn_status_str(code: int) -> str:
    return lib().attn_status_str(code).decode()


def attn_last_hip_error() -> int:
    return int(lib().attn_last_hip_error())
