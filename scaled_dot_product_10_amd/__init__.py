"""libattn for MI355X: fused causal scaled dot-product attention forward
(hand-written HIP for gfx950) behind a C ABI, with a thin torch front end.

    from scaled_dot_product_10_amd import fwd
    out, lse = fwd(q, k, v, causal=True)          # q,k,v bf16 [B,H,S,D] on the GPU

Submodules: ``api`` (torch front end), ``_lib`` (ctypes binding of the C
ABI), ``inputs`` (seeded synthetic inputs), ``build`` (hipcc build).
The torch front end is imported lazily so that ``inputs`` and ``build`` work
without touching the GPU stack.
"""

__all__ = ["fwd", "qk_gemm", "masked_softmax", "pv_gemm", "unfused", "AttnError"]


def __getattr__(name):
    if name in __all__:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
