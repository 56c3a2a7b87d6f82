"""Seeded synthetic inputs for the attention forward and the unfused trio.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle.  It draws random numbers and rounds them to the storage dtype; it does
none of the attention arithmetic.

Workload shape follows the tutorial pages: q, k, v are ``[B, H, S, D]`` tensors
filled with iid standard normals (``torch.randn`` in the Russian tutorial
"Profiling Attention in PyTorch", section 1).  Here they come from numpy's
PCG64 (``default_rng(seed).standard_normal(dtype=float32)``), drawn in the
order q, k, v, then rounded to bfloat16 with round-to-nearest-even when the
config is bf16.  The oracle and the GPU see bit-identical values: the oracle
gets the float32 image of each bf16 value (exact), the GPU gets the bf16 bits.
For the fp8 path the same draws are quantised to e4m3fn codes with one
power-of-two scale per tensor; the oracle gets code value x scale (exact).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs are finite by construction (standard normals), so NaN handling is
    not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 image of bfloat16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A host tensor in its storage dtype plus its exact float32 image.

    ``bits`` is uint16 (bf16 payload) for bf16, float32 for fp32.
    ``f32`` holds the exact values as float32 (what the oracle consumes).
    """

    bits: np.ndarray
    f32: np.ndarray
    dtype: str  # "bf16" | "f32"


def _finish(x32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Tensor(bits=bits, f32=bf16_bits_to_f32(bits), dtype=dtype)
    if dtype == "f32":
        x32 = np.ascontiguousarray(x32, dtype=np.float32)
        return Tensor(bits=x32, f32=x32, dtype=dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_qkv(B: int, Hq: int, Hkv: int, S: int, D: int, dtype: str, seed: int):
    """Draw q ``[B,Hq,S,D]``, k and v ``[B,Hkv,S,D]`` iid N(0,1) in that order."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    return _finish(q, dtype), _finish(k, dtype), _finish(v, dtype)


def make_dout(B: int, Hq: int, S: int, D: int, dtype: str, seed: int) -> Tensor:
    """Output gradient ``[B,Hq,S,D]`` for the backward, iid N(0,1), drawn from
    a stream of its own (PCG64 seeded with ``[seed, 1]``), so q, k, v of the
    same seed are unchanged."""
    rng = np.random.default_rng([seed, 1])
    return _finish(rng.standard_normal((B, Hq, S, D), dtype=np.float32), dtype)


# ---------------------------------------------------------------------------
# fp8 (OCP E4M3, "e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
# infinities; exponent 15 with mantissa 7 is NaN, so the largest finite value
# is 448; exponent 0 holds subnormals m/8 * 2^-6.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float32 value of e4m3fn codes (uint8); NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return (sign * val).astype(np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest e4m3fn code, ties to even, clamping
    to +-448 first (inputs are finite)."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.abs(x)
    # grid spacing at |x|: 2^(e-3) in the normal range e >= -6, 2^-9 below
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6)
    step = 2.0 ** (e - 3)
    q = a / step
    r = np.floor(q)
    frac = q - r
    r = r + ((frac > 0.5) | ((frac == 0.5) & (r % 2 == 1)))  # nearest, ties to even multiple
    mag = r * step  # exact multiple of the grid (may step up to the next binade)
    # encode the magnitude: subnormal if < 2^-6
    ee = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    sub = mag < 2.0 ** -6
    code_sub = np.round(mag / 2.0 ** -9).astype(np.int64)
    mant = np.round((mag / 2.0 ** ee - 1.0) * 8).astype(np.int64)
    code_norm = ((ee + 7).astype(np.int64) << 3) | mant
    code = np.where(sub, code_sub, code_norm)
    return (sign | code).astype(np.uint8)


@dataclass
class Fp8Tensor:
    """e4m3fn codes with a per-tensor scale: value = decode(code) * scale.
    ``f32`` is that value (exact in float32: the scale is a power of two)."""

    codes: np.ndarray
    scale: float
    f32: np.ndarray


def to_fp8(x32: np.ndarray) -> Fp8Tensor:
    """Per-tensor power-of-two scale that maps max |x| inside +-448, then
    round-to-nearest-even to e4m3fn."""
    amax = float(np.max(np.abs(x32))) if x32.size else 0.0
    scale = 2.0 ** int(np.ceil(np.log2(amax / E4M3_MAX))) if amax > 0 else 1.0
    codes = e4m3_encode(np.asarray(x32, np.float64) / scale)
    return Fp8Tensor(codes=codes, scale=scale, f32=(e4m3_decode(codes).astype(np.float64) * scale).astype(np.float32))


def make_qkv_fp8(B: int, Hq: int, Hkv: int, S: int, D: int, seed: int):
    """The same N(0,1) draws as make_qkv (same seed), quantised to e4m3fn
    with one power-of-two scale per tensor."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    return to_fp8(q), to_fp8(k), to_fp8(v)


def make_qkv_fp8_ramp(B: int, Hq: int, Hkv: int, S: int, D: int, step: float, seed: int):
    """fp8 inputs whose scores move by about ``step`` (log2 units, after the
    1/sqrt(D) scale) from one block of 64 keys to the next: q near the
    all-ones vector, key j near the all-a_j vector with
    a_j = step * (j // 64) / (sqrt(D) log2(e)), both with N(0, 0.3^2) noise,
    v N(0,1); each quantised to e4m3fn with a power-of-two scale."""
    rng = np.random.default_rng(seed)
    a = step * (np.arange(S) // 64) / (np.sqrt(D) * np.log2(np.e))
    q = 1.0 + 0.3 * rng.standard_normal((B, Hq, S, D))
    k = a[None, None, :, None] + 0.3 * rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    return to_fp8(q.astype(np.float32)), to_fp8(k.astype(np.float32)), to_fp8(v.astype(np.float32))


def make_scores(B: int, H: int, S: int, D: int, seed: int) -> np.ndarray:
    """Raw (unscaled) score-like matrix ``[B,H,S,S]`` fp32 for the masked softmax alone.

    A dot product of two D-long N(0,1) vectors has variance D, so the entries
    are N(0, D): after the 1/sqrt(D) scale the logits are N(0,1), as they are
    in the full pipeline.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, S, S), dtype=np.float32)
    x *= np.float32(np.sqrt(D))
    return x


def make_probs(B: int, H: int, S: int, causal: bool, dtype: str, seed: int) -> Tensor:
    """Probability-like matrix ``[B,H,S,S]`` for the PV product alone.

    Row i holds uniform draws in [0, 2/n_i) on its n_i visible keys
    (n_i = i+1 when causal, S otherwise) and zeros elsewhere, so rows sum to
    about one and carry the causal zero pattern, like real softmax output.
    """
    rng = np.random.default_rng(seed)
    x = rng.random((B, H, S, S), dtype=np.float32)
    n = (np.arange(S, dtype=np.float32) + 1.0) if causal else np.full(S, float(S), np.float32)
    x *= (np.float32(2.0) / n)[:, None]
    if causal:
        x *= np.tril(np.ones((S, S), dtype=np.float32))
    return _finish(x, dtype)


# The five workloads of the method's headline measurements.  Seeds are fixed so
# every run (tests, bench, smoke) sees the same values.
CONFIGS = {
    "C1": dict(dtype="f32", B=1, Hq=1, Hkv=1, S=128, D=64, causal=True, seed=1),
    "C2": dict(dtype="bf16", B=1, Hq=32, Hkv=32, S=2048, D=128, causal=True, seed=2),
    "C3": dict(dtype="bf16", B=4, Hq=16, Hkv=16, S=4096, D=128, causal=True, seed=3),
    "C4": dict(dtype="bf16", B=2, Hq=32, Hkv=32, S=8192, D=128, causal=True, seed=4),
    "C5": dict(dtype="bf16", B=8, Hq=32, Hkv=8, S=4096, D=128, causal=True, seed=5),
}

