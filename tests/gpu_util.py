"""Helpers for the GPU parity tests: host<->device transfer of generator
tensors, row sampling and error statistics.  No attention arithmetic here."""
from __future__ import annotations

import sys

import numpy as np

# the parity bar: max-abs / mean-abs error of out against the fp64 oracle
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}
# lse is not bounded by the pages.  Every bf16 kernel whose lse is checked
# here (fused forward, window and block masks, split-KV, the unfused softmax)
# normalises by the float32 sum of the *unrounded* weights p = 2^(s c - m c),
# so the bf16 rounding of P does not reach lse.  What does, for a row of n keys:
#   - the float32 score s (exact bf16 products, float32 accumulation of D of
#     them): |ds| <= gamma_D sum_d |q_d k_d|, about 1.3e-7 after the factor
#     c = scale * log2(e) for N(0,1) inputs at D = 128 (gamma_D = D u / (1 - D u),
#     u = 2^-24);
#   - the fma s c - m c and the hardware exp2 / log2 (about one unit in the
#     last place each), and the few rescales of l when the reference moves:
#     a few 2^-23 relative each, under 1e-5 together, plus u |lse| for the
#     final rounding;
#   - the float32 sum of n terms, accumulated as per-tile partial sums (n / 64
#     tiles, a few more levels inside a tile and across lanes): relative
#     gamma_(n/64 + 8) of l, so the same in lse.
# Hence LSE_TOL_CONST + (ceil(n / 64) + 8) * 2^-24 for bf16: 2.4e-5 at
# n = 4096, 1.4e-4 at n = 131072.  A test that knows n passes it as ``keys``;
# otherwise the bound at the largest n tested (131072) applies.  Inputs with
# large logits add the gamma_D term explicitly (see the fused tests).
# The fp8 path (weights rounded to e4m3) derives its own bound in its tests.
LSE_TOL_CONST = 2e-5
LSE_MAX_KEYS = 131072
LSE_TOL = {"f32": 1e-5}


def lse_bound(dtype, keys=None):
    if dtype != "bf16":
        return LSE_TOL[dtype]
    n = LSE_MAX_KEYS if keys is None else int(keys)
    return LSE_TOL_CONST + (-(-n // 64) + 8) * 2.0**-24


# Backward gradients have no bound on the pages; errors are taken relative to
# the size of the exact gradient (max |ref| for the max error, mean |ref| for
# the mean error).  The bf16 kernels round p and ds to bf16 (relative 2^-8 at
# most, bf16's unit roundoff) before the products that consume them and round
# dq, dk, dv to bf16 (the same); float32 accumulates everything else.  The
# rounding errors have both signs and mostly cancel in the sums (measured: at
# most 5.8e-3 and 2.7e-3 of the gradient's size over the test shapes); the
# bounds leave a margin of about two.  A gradient that is
# exactly zero (S = 1, causal query 0) is met only by the float32 rounding of
# dp - delta, about D * 2^-24 * |dout| |v| ~ 1e-5 here, so the sizes are
# floored at GRAD_FLOOR.
GRAD_TOL = (1e-2, 5e-3)
GRAD_FLOOR = 1e-2


def check_grad(name, got, ref, tol=GRAD_TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    scale_max = max(float(np.abs(ref).max()), GRAD_FLOOR) if ref.size else 1.0
    scale_mean = max(float(np.abs(ref).mean()), GRAD_FLOOR) if ref.size else 1.0
    rel_max = float(d.max()) / scale_max if d.size else 0.0
    rel_mean = float(d.mean()) / scale_mean if d.size else 0.0
    report(name, rel_max=rel_max, rel_mean=rel_mean, ref_max=scale_max)
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    assert rel_max <= tol[0], f"{name}: max err {rel_max:.3e} of max|ref| > {tol[0]}"
    assert rel_mean <= tol[1], f"{name}: mean err {rel_mean:.3e} of mean|ref| > {tol[1]}"


def persistent_launch(B, Hq, S, causal) -> bool:
    """Whether attn_fwd_bf16 takes the persistent schedule for this grid: one
    workgroup per compute unit over whole rounds of units (causal: pairs of
    query tiles), mirroring the launch code's choice."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nq = (S + 255) // 256
    split = S > 256 and B * Hq * nq <= (256 if causal else 128)  # the key-split form
    if split or S < 256 or (causal and nq % 2):
        return False
    units = B * Hq * (nq // 2 if causal else nq)
    return units % cus == 0


def dev(t, device="cuda"):
    import torch

    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).to(device)


def host(x) -> np.ndarray:
    """Exact float64 image of a bf16/fp32 device tensor."""
    return x.detach().float().cpu().numpy().astype(np.float64)


def sample_rows(B, H, S, n_random, seed, tile=128):
    """Flattened [B,H,S] row indices: first/last rows, tile edges and random rows."""
    rng = np.random.default_rng(seed)
    edge = sorted({0, 1, 2, 31, 32, 63, 64, tile - 1, tile, tile + 1, S // 2, S - 2, S - 1} & set(range(S)))
    rows = []
    for bh in sorted({0, B * H - 1, int(rng.integers(B * H))}):
        rows += [bh * S + i for i in edge]
    rows += list(rng.integers(0, B * H * S, n_random))
    return np.unique(np.array(rows, dtype=np.int64))


def errs(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def report(name, **vals):
    msg = " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in vals.items())
    print(f"[{name}] {msg}", file=sys.stderr, flush=True)


def check_close(name, got, ref, dtype, lse_got=None, lse_ref=None, lse_tol=None, keys=None):
    mx, mean = errs(got, ref)
    tol_max, tol_mean = TOL[dtype]
    vals = dict(max_abs=mx, mean_abs=mean)
    if lse_got is not None:
        vals["lse_max"] = errs(lse_got, lse_ref)[0]
    report(name, **vals)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert mx <= tol_max, f"{name}: max abs err {mx:.3e} > {tol_max}"
    assert mean <= tol_mean, f"{name}: mean abs err {mean:.3e} > {tol_mean}"
    if lse_got is not None:
        tol = lse_bound(dtype, keys) if lse_tol is None else lse_tol
        assert vals["lse_max"] <= tol, f"{name}: lse err {vals['lse_max']:.3e} > {tol:.3e}"
