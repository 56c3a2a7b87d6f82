"""fp8 forward (attn_fwd_fp8) against the fp64 oracle on the dequantised inputs.

The inputs are the generator's N(0,1) draws rounded to e4m3fn with one
power-of-two scale per tensor; the oracle computes exact attention on those
values.  The kernel stores each weight as 2^(s c - mc + 7) rounded to e4m3,
with mc an integer reference at or below the row's running max, multiplies it
back by an exact power of two inside the P.V product, and normalises by the
sum of the rounded values.  So out is the convex combination of v rows under
weights p_j (1 + e_j) + a_j (max p = 1) with |e_j| <= 2^-4 (half a unit in
e4m3's last place) and |a_j| <= 2^-17 (half the smallest subnormal step,
2^-9 / 2, over the stored value 2^7 of a weight equal to the max).  Hence, per
element,
    |out - ref| <= (2^-4 sw + 2^-17 su) / (1 - 2^-4 - S 2^-17) + 2^-8 |ref| + 1e-5
with sw, su the oracle's weighted and unweighted spread of v around out
(l >= 1 is the oracle's sum of p_j), 2^-8 |ref| covering the bf16 store and
1e-5 the float32 sums.  lse moves by at most -ln(1 - 2^-4 - S 2^-17) plus
float32 rounding.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import gpu_util as G
from scaled_dot_product_10_amd import api, inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DELTA = 2.0 ** -4
ABS_P = 2.0 ** -17


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def codes(t):
    return torch.from_numpy(np.ascontiguousarray(t.codes)).to("cuda")


def check_fp8(orc, name, q, k, v, causal, out, lse, rows=None):
    B, Hq, S, D = q.f32.shape
    sc = 1.0 / math.sqrt(D)
    ref_o, ref_l = orc.attn_fwd(q.f32, k.f32, v.f32, sc, causal, rows=rows)
    sw, su = orc.attn_spread(q.f32, k.f32, v.f32, sc, causal, rows=rows)
    got = G.host(out).reshape(ref_o.shape)
    gl = G.host(lse).reshape(ref_l.shape)
    bound = (DELTA * sw + ABS_P * su) / (1 - DELTA - S * ABS_P) + 2.0 ** -8 * np.abs(ref_o) + 1e-5
    err = np.abs(got - ref_o)
    lse_bound = -math.log(1 - DELTA - S * ABS_P) + 1e-5
    lerr = float(np.max(np.abs(gl - ref_l)))
    G.report(name, max_abs=float(err.max()), mean_abs=float(err.mean()), worst_frac_of_bound=float((err / bound).max()),
             lse_max=lerr)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(gl))
    assert np.all(err <= bound), f"{name}: error above the rounding bound at {int(np.sum(err > bound))} elements"
    assert lerr <= lse_bound, f"{name}: lse err {lerr:.3e} > {lse_bound:.3e}"


SMALL = [(1, 1, 1, 1, 128), (1, 2, 1, 17, 64), (1, 2, 2, 200, 128), (2, 4, 2, 130, 64), (1, 3, 1, 333, 128),
         (1, 2, 2, 640, 128), (1, 1, 1, 1000, 64)]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}kv{}S{}D{}".format(*s))
def test_small_full_compare(orc, shape, causal):
    B, Hq, Hkv, S, D = shape
    q, k, v = inputs.make_qkv_fp8(B, Hq, Hkv, S, D, seed=6000 + S + D)
    out, lse = api.fwd_fp8(codes(q), codes(k), codes(v), q.scale, k.scale, v.scale, causal=causal)
    torch.cuda.synchronize()
    check_fp8(orc, f"fp8 {shape} causal={causal}", q, k, v, causal, out, lse)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_c3_sampled(orc, causal):
    c = inputs.CONFIGS["C3"]
    B, Hq, Hkv, S, D = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"]
    q, k, v = inputs.make_qkv_fp8(B, Hq, Hkv, S, D, c["seed"])
    out, lse = api.fwd_fp8(codes(q), codes(k), codes(v), q.scale, k.scale, v.scale, causal=causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())
    rows = G.sample_rows(B, Hq, S, n_random=200, seed=c["seed"])
    idx = torch.from_numpy(rows).to(out.device)
    check_fp8(orc, f"fp8 C3 causal={causal} rows={rows.size}", q, k, v, causal, out.view(-1, D)[idx],
              lse.view(-1)[idx], rows=rows)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("step", [3.0, 20.0, 70.0, -20.0], ids=lambda s: f"step{s:+g}")
@pytest.mark.parametrize("shape", [(1, 2, 1, 520, 64), (1, 2, 2, 300, 128)], ids=lambda s: "H{1}kv{2}S{3}D{4}".format(*s))
def test_moving_reference(orc, shape, step, causal):
    """Scores that rise (or fall) by `step` log2 units per 64 keys: the stored
    weights' reference moves every block (+3), moves past 64 above the
    accumulators' and forces their rescaling (+20 after four blocks, +70 at
    once), or never moves and the early weights dominate (-20)."""
    B, Hq, Hkv, S, D = shape
    q, k, v = inputs.make_qkv_fp8_ramp(B, Hq, Hkv, S, D, step, seed=6200 + S)
    out, lse = api.fwd_fp8(codes(q), codes(k), codes(v), q.scale, k.scale, v.scale, causal=causal)
    torch.cuda.synchronize()
    check_fp8(orc, f"fp8 ramp {step:+g} {shape} causal={causal}", q, k, v, causal, out, lse)


# Causal grids of 256 to 768 workgroups (several per compute unit, the head
# groups of the XCD schedule, ragged S, GQA); every element compared.
GRIDS = [(1, 64, 8, 2000, 64), (2, 64, 16, 1000, 128), (1, 256, 32, 1500, 64)]


@pytest.mark.parametrize("shape", GRIDS, ids=lambda s: "B{}H{}kv{}S{}D{}".format(*s))
def test_grid_full_compare(orc, shape):
    B, Hq, Hkv, S, D = shape
    q, k, v = inputs.make_qkv_fp8(B, Hq, Hkv, S, D, seed=6400 + S + D)
    out, lse = api.fwd_fp8(codes(q), codes(k), codes(v), q.scale, k.scale, v.scale, causal=True)
    torch.cuda.synchronize()
    check_fp8(orc, f"fp8 grid {shape}", q, k, v, True, out, lse)


@pytest.mark.parametrize("step", [20.0, 70.0, -20.0], ids=lambda s: f"step{s:+g}")
def test_grid_moving_reference(orc, step):
    """The ramps of test_moving_reference over 512 workgroups."""
    B, Hq, Hkv, S, D = 1, 128, 16, 1024, 128
    q, k, v = inputs.make_qkv_fp8_ramp(B, Hq, Hkv, S, D, step, seed=6500 + int(step))
    out, lse = api.fwd_fp8(codes(q), codes(k), codes(v), q.scale, k.scale, v.scale, causal=True)
    torch.cuda.synchronize()
    check_fp8(orc, f"fp8 grid ramp {step:+g}", q, k, v, True, out, lse)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_long_sequence_sampled(orc, causal):
    """S = 32768: the weights' reference keeps moving over 512 key tiles."""
    B, Hq, Hkv, S, D = 1, 2, 1, 32768, 128
    q, k, v = inputs.make_qkv_fp8(B, Hq, Hkv, S, D, seed=6300)
    out, lse = api.fwd_fp8(codes(q), codes(k), codes(v), q.scale, k.scale, v.scale, causal=causal)
    torch.cuda.synchronize()
    rows = G.sample_rows(B, Hq, S, n_random=40, seed=6301, tile=256)
    idx = torch.from_numpy(rows).to(out.device)
    check_fp8(orc, f"fp8 S=32768 causal={causal} rows={rows.size}", q, k, v, causal, out.view(-1, D)[idx],
              lse.view(-1)[idx], rows=rows)


def test_gqa_and_row0():
    """Causal row 0 sees key 0 only: its one weight w cancels in w v / w, so
    out = v_0 * v_scale rounded to bf16, for every head of a GQA group."""
    q, k, v = inputs.make_qkv_fp8(2, 4, 2, 300, 128, seed=6100)
    out, _ = api.fwd_fp8(codes(q), codes(k), codes(v), q.scale, k.scale, v.scale, causal=True)
    torch.cuda.synchronize()
    ref = torch.from_numpy(np.repeat(v.f32[:, :, 0, :], 2, axis=1)).to(torch.bfloat16)
    assert torch.equal(out[:, :, 0, :].cpu(), ref)
