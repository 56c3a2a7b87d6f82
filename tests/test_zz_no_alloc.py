"""attn_fwd_splitkv_bf16_noalloc: the split-KV forward with its partial
results in the library's fixed per-GPU scratch instead of a caller workspace.

Called through the C ABI twice in a row on one GPU, the second time with a
smaller input (so stale contents of the larger first call sit in the
scratch), each result compared element by element with attn_fwd_splitkv_bf16
on the same inputs and split count (the same kernels: bit for bit) and with
the fp64 oracle within the forward's tolerances.  Also: no device memory is
allocated by the calls, and a call that needs more than the scratch is
refused before any launch.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import gpu_util as G
from scaled_dot_product_10_amd import _lib, inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _make(B, Hq, Hkv, Sq, Skv, D, seed):
    q, k, v = inputs.make_qkv(B, Hq, Hkv, Skv, D, "bf16", seed)
    qs = inputs.Tensor(bits=np.ascontiguousarray(q.bits[:, :, Skv - Sq:]),
                       f32=np.ascontiguousarray(q.f32[:, :, Skv - Sq:]), dtype="bf16")
    return qs, k, v


def _run(case, seed, orc):
    B, Hq, Hkv, Sq, Skv, D, causal, nsplit = case
    q, k, v = _make(B, Hq, Hkv, Sq, Skv, D, seed)
    Q, K, V = G.dev(q), G.dev(k), G.dev(v)
    sc = 1.0 / math.sqrt(D)
    sp = torch.cuda.current_stream().cuda_stream
    # the existing entry point, with its caller-owned workspace
    ws = torch.empty((_lib.attn_splitkv_workspace_bytes(B, Hq, Sq, D, nsplit) // 4,), device=Q.device,
                     dtype=torch.float32)
    out_ref = torch.empty_like(Q)
    lse_ref = torch.empty((B, Hq, Sq), device=Q.device, dtype=torch.float32)
    assert _lib.attn_fwd_splitkv_bf16(Q.data_ptr(), K.data_ptr(), V.data_ptr(), out_ref.data_ptr(),
                                      lse_ref.data_ptr(), ws.data_ptr(), B, Hq, Hkv, Sq, Skv, D, sc, int(causal),
                                      nsplit, sp) == 0
    out = torch.full_like(Q, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), device=Q.device, dtype=torch.float32)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    rc = _lib.attn_fwd_splitkv_bf16_noalloc(Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(),
                                            lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, sc, int(causal), nsplit, sp)
    assert rc == 0, _lib.attn_status_str(rc)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, "the allocation-free call allocated device memory"
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
    ref_o, ref_l = orc.attn_fwd_kv(q.f32, k.f32, v.f32, sc, causal)
    G.check_close(f"noalloc {case}", G.host(out), ref_o, "bf16", G.host(lse), ref_l, keys=Skv)


def test_two_calls_second_smaller(orc):
    # first: a B2 Hq32 Hkv8 decode step against 8192 keys in 24 splits
    _run((2, 32, 8, 1, 8192, 128, True, 24), 4101, orc)
    # second: fewer rows, fewer splits, D = 64, several queries, not causal
    _run((1, 4, 2, 3, 700, 64, False, 5), 4102, orc)


def test_too_large_is_refused():
    B, Hq, Hkv, Sq, Skv, D = 1, 64, 8, 64, 4096, 128
    cap = _lib.attn_splitkv_noalloc_max_bytes()
    assert cap == 16 << 20
    nsplit = 16
    assert _lib.attn_splitkv_workspace_bytes(B, Hq, Sq, D, nsplit) > cap
    Q = torch.zeros((B, Hq, Sq, D), device="cuda", dtype=torch.bfloat16)
    K = torch.zeros((B, Hkv, Skv, D), device="cuda", dtype=torch.bfloat16)
    out = torch.full_like(Q, 3.0)
    rc = _lib.attn_fwd_splitkv_bf16_noalloc(Q.data_ptr(), K.data_ptr(), K.data_ptr(), out.data_ptr(), None, B, Hq,
                                            Hkv, Sq, Skv, D, 0.1, 1, nsplit, torch.cuda.current_stream().cuda_stream)
    assert rc == 8 and _lib.STATUS[rc] == "ATTN_ERR_TOO_LARGE"
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call must not launch"
