"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the fact it checks.  ``tests/test_oracle_pins.py`` runs
them on the real oracle (all must pass) and on builds that carry a planted
mistake (each must be caught by at least one pin).

What pins what:
  attention forward (formula of the ainews.cool deep-dive; five-step causal
  pipeline of the Hugging Face article's "Naive Attention" section):
    hand-derived worked examples (tests/golden/hand_cases.json), the S=2, D=1
    closed form, causal row 0 = v_0, q = 0 -> running prefix mean of v with
    lse = ln(i+1), identical keys -> uniform weights, key shift invariance,
    affinity in v, one-hot v exposing the weights (rows sum to 1, zero above
    the diagonal, log-ratio = scaled key difference), last causal row = last
    non-causal row, S = 1, grouped-query heads = repeated heads, the
    hard-attention limit, and torch's float64 CPU scaled_dot_product_attention
    plus torch.logsumexp as an independent library routine.
  step 1 (q k^T): numpy matmul, exact integer products.
  steps 2-4 (scale, -inf mask, softmax): hand fixtures, scipy.special.softmax
    and logsumexp, rows sum to one, zero above the diagonal.
  step 5 (attn v): numpy matmul, exact integer products.
  composition: steps 1-5 chained equal the fused forward.
  causal sliding window (one of the special masks the ai-manual.ru tutorial
    names as the reason for custom kernels): window >= S equals causal,
    window 1 gives out_i = v_i, each row equals the last row of the causal
    attention over its own window, torch's float64 SDPA with an explicit band
    mask.
  queries against a longer key/value sequence (decode, split-KV): Sq = Skv
    equals the square forward, each query row equals the square causal
    forward's row at its position, and torch's float64 SDPA with an explicit
    bottom-right mask.
  spread of v around out (fp8 error bound ingredient): the S = 2 closed form,
    zero for one key and for constant v.
  backward (chain-rule derivative of the forward; the ai-manual.ru tutorial,
  section 6, only warns that the flash backward is easy to get wrong):
    central finite differences of sum(dout * out) through the pinned forward
    (GQA, causal and not), torch's float64 autograd through its
    scaled_dot_product_attention, the invariants sum_j dk_j = 0 and
    sum_j dv_j = sum_i dout_i, delta_i = dout_i . out_i, S = 1 and causal
    row 0 closed forms, linearity in dout.
"""
from __future__ import annotations

import json
import math
from fractions import Fraction
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden" / "hand_cases.json"

TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _frac(s) -> float:
    return float(Fraction(str(s)))


def _scale(s) -> float:
    return {"ln2": math.log(2.0), "ln3": math.log(3.0)}[s] if isinstance(s, str) else float(s)


def _randn(shape, seed):
    return _rng(seed).standard_normal(shape).astype(np.float32)


# --------------------------------------------------------------------------
# attention forward
# --------------------------------------------------------------------------

def pin_golden_attention(orc):
    cases = json.loads(GOLDEN.read_text())
    tol = cases["tol"]
    for c in cases["attention"]:
        q = np.array(c["q"], np.float32)
        k = np.array(c["k"], np.float32)
        v = np.array(c["v"], np.float32)
        out, lse = orc.attn_fwd(q, k, v, _scale(c["scale"]), c["causal"])
        exp_out = np.vectorize(_frac)(np.array(c["out"], dtype=object)).astype(np.float64)
        exp_lse = np.log(np.vectorize(_frac)(np.array(c["lse_exp"], dtype=object)).astype(np.float64))
        _close(out, exp_out, tol, c["name"] + " out")
        _close(lse, exp_lse, tol, c["name"] + " lse")


def pin_s2_d1_closed_form(orc):
    """S=2, D=1: row 1 = (e^{a} x + e^{b} y) / (e^{a} + e^{b}), a = sc*q1*k0, b = sc*q1*k1."""
    r = _rng(11)
    for trial in range(20):
        qv, kv, vv = (r.standard_normal(2).astype(np.float32) for _ in range(3))
        sc = float(r.uniform(0.2, 2.0))
        q = qv.reshape(1, 1, 2, 1)
        k = kv.reshape(1, 1, 2, 1)
        v = vv.reshape(1, 1, 2, 1)
        q64, k64, v64 = qv.astype(np.float64), kv.astype(np.float64), vv.astype(np.float64)
        for causal in (True, False):
            out, lse = orc.attn_fwd(q, k, v, sc, causal)
            a, b = sc * q64[1] * k64[0], sc * q64[1] * k64[1]
            row1 = (math.exp(a) * v64[0] + math.exp(b) * v64[1]) / (math.exp(a) + math.exp(b))
            _close(out[0, 0, 1, 0], row1, 1e-12, "S2 row1")
            _close(lse[0, 0, 1], math.log(math.exp(a) + math.exp(b)), 1e-12, "S2 lse1")
            if causal:
                _close(out[0, 0, 0, 0], v64[0], 0.0, "S2 causal row0")
                _close(lse[0, 0, 0], sc * q64[0] * k64[0], 1e-12, "S2 causal lse0")
            else:
                c0, c1 = sc * q64[0] * k64[0], sc * q64[0] * k64[1]
                row0 = (math.exp(c0) * v64[0] + math.exp(c1) * v64[1]) / (math.exp(c0) + math.exp(c1))
                _close(out[0, 0, 0, 0], row0, 1e-12, "S2 noncausal row0")


def pin_causal_row0(orc):
    """Causal row 0 sees key 0 only: out = v_0 exactly, lse = scale * q_0 . k_0."""
    for (B, Hq, Hkv, S, D, seed) in [(2, 4, 2, 37, 16, 1), (1, 3, 1, 5, 64, 2)]:
        q = _randn((B, Hq, S, D), seed)
        k = _randn((B, Hkv, S, D), seed + 100)
        v = _randn((B, Hkv, S, D), seed + 200)
        sc = 1.0 / math.sqrt(D)
        out, lse = orc.attn_fwd(q, k, v, sc, True)
        g = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                kvh = h // g
                _close(out[b, h, 0], v[b, kvh, 0].astype(np.float64), 0.0, "row0 out")
                dot = sum(float(q[b, h, 0, d]) * float(k[b, kvh, 0, d]) for d in range(D))
                _close(lse[b, h, 0], sc * dot, 1e-12, "row0 lse")


def pin_zero_queries(orc):
    """q = 0: all logits 0 -> out_i = mean(v_0..v_i), lse_i = ln(i+1) (causal);
    mean of all v and ln S otherwise."""
    B, Hq, Hkv, S, D = 1, 2, 2, 23, 8
    q = np.zeros((B, Hq, S, D), np.float32)
    k = _randn((B, Hkv, S, D), 3)
    v = _randn((B, Hkv, S, D), 4)
    v64 = v.astype(np.float64)
    out, lse = orc.attn_fwd(q, k, v, 0.3, True)
    for i in range(S):
        _close(out[:, :, i], v64[:, :, : i + 1].mean(axis=2), 1e-12, "zero-q prefix mean")
        _close(lse[:, :, i], np.full((B, Hq), math.log(i + 1)), 1e-12, "zero-q lse")
    out, lse = orc.attn_fwd(q, k, v, 0.3, False)
    for i in range(S):
        _close(out[:, :, i], v64.mean(axis=2), 1e-12, "zero-q mean")
        _close(lse[:, :, i], np.full((B, Hq), math.log(S)), 1e-12, "zero-q lse S")


def pin_identical_keys(orc):
    """k_j = kappa for all j: uniform weights; lse_i = scale q_i.kappa + ln(i+1)."""
    B, H, S, D = 1, 1, 17, 8
    q = _randn((B, H, S, D), 5)
    kappa = _randn((D,), 6)
    k = np.broadcast_to(kappa, (B, H, S, D)).copy()
    v = _randn((B, H, S, D), 7)
    sc = 0.7
    out, lse = orc.attn_fwd(q, k, v, sc, True)
    v64 = v.astype(np.float64)
    for i in range(S):
        _close(out[0, 0, i], v64[0, 0, : i + 1].mean(axis=0), 1e-12, "identical keys out")
        qk = sum(float(q[0, 0, i, d]) * float(kappa[d]) for d in range(D))
        _close(lse[0, 0, i], sc * qk + math.log(i + 1), 1e-12, "identical keys lse")


def pin_shift_keys(orc):
    """k_j -> k_j + c: out unchanged, lse_i -> lse_i + scale q_i.c."""
    B, H, S, D = 1, 2, 19, 4
    # small integers and halves keep k + c exact in float32
    r = _rng(8)
    q = r.integers(-3, 4, (B, H, S, D)).astype(np.float32) / 2
    k = r.integers(-3, 4, (B, H, S, D)).astype(np.float32) / 2
    v = _randn((B, H, S, D), 9)
    c = np.array([0.5, -1.0, 1.5, 2.0], np.float32)
    sc = 0.4
    for causal in (True, False):
        o1, l1 = orc.attn_fwd(q, k, v, sc, causal)
        o2, l2 = orc.attn_fwd(q, k + c, v, sc, causal)
        _close(o2, o1, 1e-12, "shift out")
        _close(l2 - l1, sc * (q.astype(np.float64) @ c.astype(np.float64)), 1e-12, "shift lse")


def pin_affine_v(orc):
    """v -> alpha v + beta: out -> alpha out + beta (weights sum to one)."""
    B, Hq, Hkv, S, D = 2, 2, 1, 21, 8
    q = _randn((B, Hq, S, D), 10)
    k = _randn((B, Hkv, S, D), 11)
    v = (_rng(12).integers(-8, 9, (B, Hkv, S, D))).astype(np.float32)
    alpha, beta = 0.5, 3.0
    for causal in (True, False):
        o1, _ = orc.attn_fwd(q, k, v, 0.35, causal)
        o2, _ = orc.attn_fwd(q, k, (alpha * v + beta).astype(np.float32), 0.35, causal)
        _close(o2, alpha * o1 + beta, 1e-11, "affine v")


def pin_onehot_weights(orc):
    """v = identity (D = S) makes out the weight matrix itself."""
    S = 12
    q = _randn((1, 1, S, 6), 13)
    k = _randn((1, 1, S, 6), 14)
    sc = 0.6
    q6 = np.zeros((1, 1, S, S), np.float32)
    k6 = np.zeros((1, 1, S, S), np.float32)
    q6[..., :6] = q
    k6[..., :6] = k
    v = np.eye(S, dtype=np.float32).reshape(1, 1, S, S)
    for causal in (True, False):
        w, _ = orc.attn_fwd(q6, k6, v, sc, causal)
        w = w[0, 0]
        assert np.all(w >= 0), "weights negative"
        _close(w.sum(axis=1), np.ones(S), 1e-12, "weights sum")
        if causal:
            assert np.all(np.triu(w, 1) == 0.0), "weight above the diagonal"
        q64, k64 = q[0, 0].astype(np.float64), k[0, 0].astype(np.float64)
        for i in range(S):
            jmax = i if causal else S - 1
            for j in range(jmax + 1):
                expect = sc * float(q64[i] @ (k64[j] - k64[0]))
                _close(math.log(w[i, j]) - math.log(w[i, 0]), expect, 1e-10, "log-ratio")


def pin_last_row(orc):
    """The last causal row sees every key, as the non-causal row does."""
    q = _randn((2, 2, 33, 16), 15)
    k = _randn((2, 2, 33, 16), 16)
    v = _randn((2, 2, 33, 16), 17)
    oc, lc = orc.attn_fwd(q, k, v, 0.25, True)
    on, ln_ = orc.attn_fwd(q, k, v, 0.25, False)
    _close(oc[:, :, -1], on[:, :, -1], 1e-13, "last row out")
    _close(lc[:, :, -1], ln_[:, :, -1], 1e-13, "last row lse")


def pin_s1(orc):
    """S = 1: out = v, lse = scale q.k (both modes)."""
    q = _randn((3, 4, 1, 64), 18)
    k = _randn((3, 2, 1, 64), 19)
    v = _randn((3, 2, 1, 64), 20)
    for causal in (True, False):
        out, lse = orc.attn_fwd(q, k, v, 0.125, causal)
        kk = np.repeat(k, 2, axis=1).astype(np.float64)
        vv = np.repeat(v, 2, axis=1).astype(np.float64)
        _close(out, vv, 0.0, "S1 out")
        _close(lse, 0.125 * np.sum(q.astype(np.float64) * kk, axis=-1), 1e-12, "S1 lse")


def pin_gqa(orc):
    """Hkv < Hq equals multi-head attention with k, v repeated per group
    (query head h reads key/value head h // (Hq/Hkv))."""
    B, Hq, Hkv, S, D = 2, 6, 2, 14, 8
    q = _randn((B, Hq, S, D), 21)
    k = _randn((B, Hkv, S, D), 22)
    v = _randn((B, Hkv, S, D), 23)
    for causal in (True, False):
        o1, l1 = orc.attn_fwd(q, k, v, 0.3, causal)
        o2, l2 = orc.attn_fwd(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), 0.3, causal)
        _close(o1, o2, 0.0, "gqa out")
        _close(l1, l2, 0.0, "gqa lse")


def pin_hard_limit(orc):
    """Large scale: the weight concentrates on the largest logit, out -> v_argmax."""
    B, H, S, D = 1, 1, 16, 4
    r = _rng(24)
    q = r.integers(-4, 5, (B, H, S, D)).astype(np.float32)
    k = r.integers(-4, 5, (B, H, S, D)).astype(np.float32)
    v = _randn((B, H, S, D), 25)
    sc = 60.0
    for causal in (True, False):
        out, _ = orc.attn_fwd(q, k, v, sc, causal)
        for i in range(S):
            jmax = i if causal else S - 1
            dots = [int(np.dot(q[0, 0, i].astype(np.int64), k[0, 0, j].astype(np.int64))) for j in range(jmax + 1)]
            best = max(dots)
            if dots.count(best) != 1:
                continue  # tie: the limit averages the tied values
            j = dots.index(best)
            _close(out[0, 0, i], v[0, 0, j].astype(np.float64), 1e-6, "hard limit")


def pin_torch_sdpa(orc):
    """torch's float64 CPU scaled_dot_product_attention (an independent library
    implementation) and torch.logsumexp agree with the oracle."""
    import torch

    for (B, Hq, Hkv, S, D, seed) in [(2, 4, 4, 29, 16, 30), (1, 6, 2, 40, 32, 31), (1, 2, 1, 7, 64, 32)]:
        q = _randn((B, Hq, S, D), seed)
        k = _randn((B, Hkv, S, D), seed + 1)
        v = _randn((B, Hkv, S, D), seed + 2)
        sc = 1.0 / math.sqrt(D)
        g = Hq // Hkv
        tq = torch.from_numpy(q.astype(np.float64))
        tk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(g, dim=1)
        tv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(g, dim=1)
        for causal in (True, False):
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=sc)
            logits = torch.matmul(tq, tk.transpose(-2, -1)) * sc
            if causal:
                mask = torch.ones(S, S, dtype=torch.bool).triu(1)
                logits = logits.masked_fill(mask, float("-inf"))
            ref_lse = torch.logsumexp(logits, dim=-1)
            out, lse = orc.attn_fwd(q, k, v, sc, causal)
            _close(out, ref.numpy(), 1e-12, "torch sdpa out")
            _close(lse, ref_lse.numpy(), 1e-12, "torch lse")


ATTN_PINS = [
    pin_golden_attention, pin_s2_d1_closed_form, pin_causal_row0, pin_zero_queries,
    pin_identical_keys, pin_shift_keys, pin_affine_v, pin_onehot_weights, pin_last_row,
    pin_s1, pin_gqa, pin_hard_limit, pin_torch_sdpa,
]


# --------------------------------------------------------------------------
# unfused steps
# --------------------------------------------------------------------------

def pin_qk_numpy(orc):
    """Step 1 equals numpy's matmul (per kv-head group)."""
    B, Hq, Hkv, S, D = 2, 4, 2, 19, 24
    q = _randn((B, Hq, S, D), 40)
    k = _randn((B, Hkv, S, D), 41)
    ref = np.matmul(q.astype(np.float64), np.repeat(k, 2, axis=1).astype(np.float64).transpose(0, 1, 3, 2))
    _close(orc.qk_scores(q, k), ref, 1e-12, "qk numpy")
    rows = np.array([0, 5, B * Hq * S - 1], np.int64)
    _close(orc.qk_scores(q, k, rows=rows), ref.reshape(-1, S)[rows], 1e-12, "qk rows")


def pin_qk_integer(orc):
    """Step 1 on small integers is exact: compare with int64 arithmetic."""
    r = _rng(42)
    q = r.integers(-9, 10, (1, 2, 9, 7))
    k = r.integers(-9, 10, (1, 2, 9, 7))
    ref = np.matmul(q, k.transpose(0, 1, 3, 2)).astype(np.float64)
    _close(orc.qk_scores(q.astype(np.float32), k.astype(np.float32)), ref, 0.0, "qk exact")


def pin_golden_softmax(orc):
    cases = json.loads(GOLDEN.read_text())
    for c in cases["masked_softmax"]:
        x = np.array(c["x"], np.float32)
        p, lse = orc.masked_softmax(x, _scale(c["scale"]), c["causal"])
        exp_p = np.vectorize(_frac)(np.array(c["p"], dtype=object)).astype(np.float64)
        exp_lse = np.log(np.vectorize(_frac)(np.array(c["lse_exp"], dtype=object)).astype(np.float64))
        _close(p, exp_p, cases["tol"], c["name"] + " p")
        _close(lse, exp_lse, cases["tol"], c["name"] + " lse")


def pin_softmax_scipy(orc):
    """Steps 2-4 equal scipy.special.softmax / logsumexp on the masked,
    scaled logits; rows sum to one; entries above the diagonal are zero."""
    from scipy.special import logsumexp, softmax

    B, H, S = 2, 3, 31
    x = _randn((B, H, S, S), 43) * 8
    sc = 0.2
    for causal in (True, False):
        t = sc * x.astype(np.float64)
        if causal:
            t = np.where(np.triu(np.ones((S, S), bool), 1), -np.inf, t)
        p, lse = orc.masked_softmax(x, sc, causal)
        _close(p, softmax(t, axis=-1), 1e-13, "softmax scipy")
        _close(lse, logsumexp(t, axis=-1), 1e-12, "lse scipy")
        _close(p.sum(axis=-1), np.ones((B, H, S)), 1e-12, "rows sum")
        if causal:
            assert np.all(p[..., np.triu(np.ones((S, S), bool), 1)] == 0.0)


def pin_pv_numpy(orc):
    """Step 5 equals numpy's matmul (per kv-head group)."""
    B, Hq, Hkv, S, D = 2, 4, 1, 17, 12
    p = _rng(44).random((B, Hq, S, S)).astype(np.float32)
    v = _randn((B, Hkv, S, D), 45)
    ref = np.matmul(p.astype(np.float64), np.repeat(v, 4, axis=1).astype(np.float64))
    _close(orc.pv(p, v), ref, 1e-12, "pv numpy")


def pin_pv_integer(orc):
    r = _rng(46)
    p = r.integers(-5, 6, (1, 1, 11, 11))
    v = r.integers(-5, 6, (1, 1, 11, 3))
    _close(orc.pv(p.astype(np.float32), v.astype(np.float32)), np.matmul(p, v).astype(np.float64), 0.0, "pv exact")


def pin_chain_equals_fused(orc):
    """Steps 1-5 chained give the fused forward's out and lse."""
    B, Hq, Hkv, S, D = 1, 4, 2, 26, 16
    q = _randn((B, Hq, S, D), 47)
    k = _randn((B, Hkv, S, D), 48)
    v = _randn((B, Hkv, S, D), 49)
    sc = 0.25
    for causal in (True, False):
        scores = orc.qk_scores(q, k)
        # the chain's hand-offs are float32 here only because the oracle's
        # inputs are float32 arrays; compare at float32 resolution
        p, lse = orc.masked_softmax(scores.astype(np.float32), sc, causal)
        out = orc.pv(p.astype(np.float32), v)
        fo, fl = orc.attn_fwd(q, k, v, sc, causal)
        _close(out, fo, 1e-5, "chain out")
        _close(lse, fl, 1e-5, "chain lse")


STEP_PINS = [pin_qk_numpy, pin_qk_integer, pin_golden_softmax, pin_softmax_scipy,
             pin_pv_numpy, pin_pv_integer, pin_chain_equals_fused]

# --------------------------------------------------------------------------
# causal sliding window
# --------------------------------------------------------------------------

def pin_local_wide_is_causal(orc):
    """A window of at least S keys hides nothing the causal mask shows."""
    q = _randn((2, 4, 33, 16), 100)
    k = _randn((2, 2, 33, 16), 101)
    v = _randn((2, 2, 33, 16), 102)
    out, lse = orc.attn_fwd(q, k, v, 0.25, True)
    for w in (33, 34, 1000):
        o2, l2 = orc.attn_fwd_local(q, k, v, 0.25, w)
        _close(o2, out, 0.0, f"window {w} = causal out")
        _close(l2, lse, 0.0, f"window {w} = causal lse")


def pin_local_w1(orc):
    """Window 1: every query sees only its own key, so out_i = v_i exactly and
    lse_i = scale q_i . k_i."""
    q = _randn((1, 2, 20, 8), 103)
    k = _randn((1, 1, 20, 8), 104)
    v = _randn((1, 1, 20, 8), 105)
    out, lse = orc.attn_fwd_local(q, k, v, 0.5, 1)
    _close(out, np.repeat(v, 2, axis=1).astype(np.float64), 0.0, "window 1 out")
    ref = 0.5 * np.einsum("bhsd,bhsd->bhs", q.astype(np.float64), np.repeat(k, 2, axis=1).astype(np.float64))
    _close(lse, ref, 1e-12, "window 1 lse")


def pin_local_subproblem(orc):
    """Row i with window W is the last row of causal attention over keys
    i-W+1..i alone (the pinned causal forward on a shorter sequence)."""
    B, H, S, D, W = 1, 2, 40, 8, 7
    q = _randn((B, H, S, D), 106)
    k = _randn((B, H, S, D), 107)
    v = _randn((B, H, S, D), 108)
    out, lse = orc.attn_fwd_local(q, k, v, 0.3, W)
    for i in (0, 3, 6, 7, 20, S - 1):
        lo = max(0, i - W + 1)
        o2, l2 = orc.attn_fwd(q[:, :, lo:i + 1], k[:, :, lo:i + 1], v[:, :, lo:i + 1], 0.3, True)
        _close(out[:, :, i], o2[:, :, -1], 1e-14, f"subproblem row {i}")
        _close(lse[:, :, i], l2[:, :, -1], 1e-14, f"subproblem lse {i}")


def pin_local_torch(orc):
    """torch's float64 CPU scaled_dot_product_attention with an explicit band
    mask (j <= i and j > i - W) agrees."""
    import torch

    B, Hq, Hkv, S, D = 2, 4, 2, 50, 16
    q = _randn((B, Hq, S, D), 109)
    k = _randn((B, Hkv, S, D), 110)
    v = _randn((B, Hkv, S, D), 111)
    sc = 1 / math.sqrt(D)
    tq = torch.from_numpy(q.astype(np.float64))
    tk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(2, dim=1)
    tv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(2, dim=1)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    for W in (1, 5, 16, 49):
        band = (j <= i) & (j > i - W)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=band, scale=sc)
        out, _ = orc.attn_fwd_local(q, k, v, sc, W)
        _close(out, ref.numpy(), 1e-12, f"torch band W={W}")


LOCAL_PINS = [pin_local_wide_is_causal, pin_local_w1, pin_local_subproblem, pin_local_torch]


# --------------------------------------------------------------------------
# block mask (64 x 64 blocks)
# --------------------------------------------------------------------------

def _expand_mask(mask, S):
    """Element mask [Bm, Hm, S, S] of a block mask (each flag covers 64 x 64)."""
    e = np.repeat(np.repeat(np.asarray(mask) != 0, 64, axis=2), 64, axis=3)
    return e[:, :, :S, :S]


def pin_blockmask_ones(orc):
    """An all-ones block mask hides nothing: plain attention, bit for bit,
    also when the mask is broadcast over batch and heads."""
    q = _randn((2, 4, 150, 8), 130)
    k = _randn((2, 2, 150, 8), 131)
    v = _randn((2, 2, 150, 8), 132)
    for causal in (True, False):
        a, la = orc.attn_fwd(q, k, v, 0.3, causal)
        for shape in ((1, 1, 3, 3), (2, 4, 3, 3)):
            b, lb = orc.attn_fwd_blockmask(q, k, v, 0.3, causal, np.ones(shape, np.uint8))
            _close(b, a, 0.0, f"ones mask {shape} causal={causal}")
            _close(lb, la, 0.0, f"ones mask lse {shape} causal={causal}")


def pin_blockmask_diagonal(orc):
    """A block-diagonal mask splits the sequence into independent 64-key
    segments: rows of segment r equal attention (causal or full) over that
    segment alone (the pinned forward on the sliced tensors)."""
    B, H, S, D = 1, 2, 170, 8
    q = _randn((B, H, S, D), 133)
    k = _randn((B, H, S, D), 134)
    v = _randn((B, H, S, D), 135)
    m = np.eye(3, dtype=np.uint8)[None, None]
    for causal in (True, False):
        out, lse = orc.attn_fwd_blockmask(q, k, v, 0.4, causal, m)
        for r0 in (0, 64, 128):
            r1 = min(r0 + 64, S)
            o2, l2 = orc.attn_fwd(q[:, :, r0:r1], k[:, :, r0:r1], v[:, :, r0:r1], 0.4, causal)
            _close(out[:, :, r0:r1], o2, 1e-14, f"segment {r0} causal={causal}")
            _close(lse[:, :, r0:r1], l2, 1e-14, f"segment lse {r0} causal={causal}")


def pin_blockmask_torch(orc):
    """torch's float64 CPU scaled_dot_product_attention with the element mask
    the block flags expand to (and j <= i when causal), on random per-(b, h)
    masks; rows left with no visible key give out 0 and lse -inf (torch's
    softmax would give NaN there, so those rows are checked on their own)."""
    import torch

    B, Hq, Hkv, S, D = 2, 4, 2, 150, 16
    nb = 3
    q = _randn((B, Hq, S, D), 136)
    k = _randn((B, Hkv, S, D), 137)
    v = _randn((B, Hkv, S, D), 138)
    sc = 1 / math.sqrt(D)
    tq = torch.from_numpy(q.astype(np.float64))
    tk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(2, dim=1)
    tv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(2, dim=1)
    rng = _rng(139)
    for causal in (True, False):
        for dens in (0.3, 0.6):
            m = (rng.random((B, Hq, nb, nb)) < dens).astype(np.uint8)
            m[0, 1, 2, :] = 0  # one query block that sees nothing
            em = _expand_mask(m, S)
            if causal:
                em = em & np.tril(np.ones((S, S), bool))[None, None]
            out, lse = orc.attn_fwd_blockmask(q, k, v, sc, causal, m)
            seen = em.any(axis=3)
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(em),
                                                                   scale=sc).numpy()
            _close(out[seen], ref[seen], 1e-12, f"torch block mask causal={causal} density={dens}")
            s = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), np.repeat(k, 2, axis=1).astype(np.float64)) * sc
            s = np.where(em, s, -np.inf)
            mx = s.max(axis=3, keepdims=True)
            with np.errstate(divide="ignore"):  # log 0 = -inf on the rows that see nothing
                ref_l = (mx[..., 0] + np.log(np.exp(s - np.where(np.isfinite(mx), mx, 0)).sum(axis=3)))
            _close(lse[seen], ref_l[seen], 1e-12, f"block mask lse causal={causal} density={dens}")
            assert (~seen).any(), "the pin needs a row with no visible key"
            assert np.all(out[~seen] == 0.0) and np.all(lse[~seen] == -np.inf), "empty rows: out 0, lse -inf"


def pin_blockmask_broadcast(orc):
    """A mask broadcast over batch (or heads) equals the same flags written
    out for every batch (or head)."""
    q = _randn((2, 3, 130, 8), 140)
    k = _randn((2, 3, 130, 8), 141)
    v = _randn((2, 3, 130, 8), 142)
    rng = _rng(143)
    per_head = (rng.random((1, 3, 3, 3)) < 0.5).astype(np.uint8)
    per_batch = (rng.random((2, 1, 3, 3)) < 0.5).astype(np.uint8)
    for m, full in ((per_head, np.repeat(per_head, 2, axis=0)), (per_batch, np.repeat(per_batch, 3, axis=1))):
        a, la = orc.attn_fwd_blockmask(q, k, v, 0.3, False, m)
        b, lb = orc.attn_fwd_blockmask(q, k, v, 0.3, False, full)
        assert np.array_equal(a, b), f"broadcast {m.shape}"
        assert np.array_equal(la, lb), f"broadcast lse {m.shape}"  # -inf rows included


BLOCK_PINS = [pin_blockmask_ones, pin_blockmask_diagonal, pin_blockmask_torch, pin_blockmask_broadcast]


# --------------------------------------------------------------------------
# queries against a longer key/value sequence
# --------------------------------------------------------------------------

def pin_kv_square(orc):
    """Sq = Skv is the square forward, causal and not, bit for bit."""
    q = _randn((2, 4, 21, 8), 120)
    k = _randn((2, 2, 21, 8), 121)
    v = _randn((2, 2, 21, 8), 122)
    for causal in (True, False):
        a, la = orc.attn_fwd(q, k, v, 0.35, causal)
        b, lb = orc.attn_fwd_kv(q, k, v, 0.35, causal)
        _close(b, a, 0.0, f"kv square out causal={causal}")
        _close(lb, la, 0.0, f"kv square lse causal={causal}")


def pin_kv_suffix_rows(orc):
    """Query i of Sq is position Skv-Sq+i: with the earlier positions filled
    in, the square causal forward's rows Skv-Sq.. equal the decode rows."""
    B, Hq, Hkv, Skv, D = 1, 4, 2, 50, 16
    full_q = _randn((B, Hq, Skv, D), 123)
    k = _randn((B, Hkv, Skv, D), 124)
    v = _randn((B, Hkv, Skv, D), 125)
    sq_out, sq_lse = orc.attn_fwd(full_q, k, v, 0.25, True)
    for Sq in (1, 3, 17):
        out, lse = orc.attn_fwd_kv(full_q[:, :, Skv - Sq:], k, v, 0.25, True)
        _close(out, sq_out[:, :, Skv - Sq:], 1e-15, f"suffix rows Sq={Sq}")
        _close(lse, sq_lse[:, :, Skv - Sq:], 1e-15, f"suffix lse Sq={Sq}")
        nc, _ = orc.attn_fwd_kv(full_q[:, :, Skv - Sq:], k, v, 0.25, False)
        _close(nc[:, :, -1], sq_out[:, :, -1], 1e-15, "last row sees every key")


def pin_kv_torch(orc):
    """torch's float64 CPU SDPA with an explicit bottom-right causal mask."""
    import torch

    B, Hq, Hkv, Sq, Skv, D = 2, 6, 3, 5, 37, 16
    q = _randn((B, Hq, Sq, D), 126)
    k = _randn((B, Hkv, Skv, D), 127)
    v = _randn((B, Hkv, Skv, D), 128)
    sc = 1 / math.sqrt(D)
    tq = torch.from_numpy(q.astype(np.float64))
    tk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(2, dim=1)
    tv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(2, dim=1)
    mask = torch.arange(Skv)[None, :] <= (Skv - Sq + torch.arange(Sq))[:, None]
    for causal in (True, False):
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask if causal else None,
                                                               scale=sc)
        out, _ = orc.attn_fwd_kv(q, k, v, sc, causal)
        _close(out, ref.numpy(), 1e-12, f"torch kv causal={causal}")


KV_PINS = [pin_kv_square, pin_kv_suffix_rows, pin_kv_torch]


# --------------------------------------------------------------------------
# spread of v around out (fp8 error bound)
# --------------------------------------------------------------------------

def pin_spread_closed_forms(orc):
    """S = 2: with weights w0, w1 = 1 - w0, sw = 2 w0 w1 |v0 - v1| and
    su = (|v0 - out| + |v1 - out|) / l, l = 1 + exp(-|s0 - s1|).  S = 1 and a
    constant v give zero spread."""
    q = np.array([[[[1.0, 0.5]]] * 1], np.float32).reshape(1, 1, 1, 2)
    q = np.concatenate([q, q], axis=2)  # two identical queries
    k = np.array([[[[0.5, 1.0], [1.5, -0.5]]]], np.float32)
    v = np.array([[[[2.0, -1.0], [0.5, 3.0]]]], np.float32)
    sc = 0.7
    sw, su = orc.attn_spread(q, k, v, sc, False)
    s0 = sc * (1.0 * 0.5 + 0.5 * 1.0)
    s1 = sc * (1.0 * 1.5 + 0.5 * -0.5)
    w0 = 1 / (1 + math.exp(s1 - s0))
    w1 = 1 - w0
    out = w0 * v[0, 0, 0].astype(np.float64) + w1 * v[0, 0, 1].astype(np.float64)
    l = 1 + math.exp(-abs(s0 - s1))
    exp_sw = 2 * w0 * w1 * np.abs(v[0, 0, 0] - v[0, 0, 1]).astype(np.float64)
    exp_su = (np.abs(v[0, 0, 0] - out) + np.abs(v[0, 0, 1] - out)) / l
    _close(sw[0, 0, 1], exp_sw, 1e-14, "spread S=2 sw")
    _close(su[0, 0, 1], exp_su, 1e-14, "spread S=2 su")
    swc, suc = orc.attn_spread(q, k, v, sc, True)
    _close(swc[0, 0, 0], np.zeros(2), 0.0, "spread causal row 0 (one key) sw")
    _close(suc[0, 0, 0], np.zeros(2), 0.0, "spread causal row 0 (one key) su")
    _close(swc[0, 0, 1], exp_sw, 1e-14, "spread causal row 1 = full row 1")
    qq = _randn((1, 2, 9, 4), 130)
    kk = _randn((1, 2, 9, 4), 131)
    vv = np.ones((1, 2, 9, 4), np.float32) * np.float32(1.5)
    sw, su = orc.attn_spread(qq, kk, vv, 0.5, True)
    _close(sw, np.zeros_like(sw), 1e-15, "constant v sw")
    _close(su, np.zeros_like(su), 1e-15, "constant v su")


SPREAD_PINS = [pin_spread_closed_forms]


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def _dyadic(shape, seed, lo=-2.0, hi=2.0):
    """Values on a 2^-8 grid: x +- 2^-14 stays exact in float32."""
    r = _rng(seed)
    return (np.round(r.uniform(lo, hi, shape) * 256) / 256).astype(np.float32)


def pin_bwd_finite_diff(orc):
    """dq, dk, dv equal central differences of L = sum(dout * out) taken
    through the (separately pinned) forward, with a step of 2^-14."""
    h = 2.0 ** -14
    for (B, Hq, Hkv, S, D, causal, seed) in [(1, 2, 1, 5, 3, True, 60), (1, 2, 1, 5, 3, False, 61),
                                             (2, 2, 2, 4, 2, True, 62)]:
        q = _dyadic((B, Hq, S, D), seed)
        k = _dyadic((B, Hkv, S, D), seed + 10)
        v = _dyadic((B, Hkv, S, D), seed + 20)
        do = _dyadic((B, Hq, S, D), seed + 30)
        sc = 0.75

        def loss(qq, kk, vv):
            out, _ = orc.attn_fwd(qq, kk, vv, sc, causal)
            return float(np.sum(out * do.astype(np.float64)))

        dq, dk, dv = orc.attn_bwd(q, k, v, do, sc, causal)
        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            num = np.zeros(x.shape)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += np.float32(h)
                xm[idx] -= np.float32(h)
                args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
                args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(g, num, 1e-6, f"finite differences {name} causal={causal}")


def pin_bwd_torch(orc):
    """torch's float64 CPU autograd through scaled_dot_product_attention (an
    independent library implementation) gives the same dq, dk, dv."""
    import torch

    for (B, Hq, Hkv, S, D, seed) in [(2, 4, 2, 23, 16, 70), (1, 3, 3, 30, 8, 71), (1, 4, 1, 9, 32, 72)]:
        q = _randn((B, Hq, S, D), seed)
        k = _randn((B, Hkv, S, D), seed + 1)
        v = _randn((B, Hkv, S, D), seed + 2)
        do = _randn((B, Hq, S, D), seed + 3)
        sc = 1.0 / math.sqrt(D)
        g = Hq // Hkv
        for causal in (True, False):
            tq = torch.from_numpy(q.astype(np.float64)).requires_grad_()
            tk = torch.from_numpy(k.astype(np.float64)).requires_grad_()
            tv = torch.from_numpy(v.astype(np.float64)).requires_grad_()
            out = torch.nn.functional.scaled_dot_product_attention(
                tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), is_causal=causal, scale=sc)
            out.backward(torch.from_numpy(do.astype(np.float64)))
            dq, dk, dv = orc.attn_bwd(q, k, v, do, sc, causal)
            _close(dq, tq.grad.numpy(), 1e-11, "torch dq")
            _close(dk, tk.grad.numpy(), 1e-11, "torch dk")
            _close(dv, tv.grad.numpy(), 1e-11, "torch dv")


def pin_bwd_invariants(orc):
    """Rows of ds sum to zero, so sum_j dk_j = 0; rows of p sum to one, so
    sum_j dv_j = sum of dout over the group's queries; delta_i = dout_i . out_i
    and pass 1's lse equals the forward's."""
    B, Hq, Hkv, S, D = 2, 6, 2, 37, 8
    q = _randn((B, Hq, S, D), 80)
    k = _randn((B, Hkv, S, D), 81)
    v = _randn((B, Hkv, S, D), 82)
    do = _randn((B, Hq, S, D), 83)
    sc = 0.4
    g = Hq // Hkv
    for causal in (True, False):
        dq, dk, dv = orc.attn_bwd(q, k, v, do, sc, causal)
        _close(dk.sum(axis=2), np.zeros((B, Hkv, D)), 1e-12, "sum dk")
        ref = do.astype(np.float64).reshape(B, Hkv, g, S, D).sum(axis=(2, 3))
        _close(dv.sum(axis=2), ref, 1e-11, "sum dv")
        lse, delta, _ = orc.attn_bwd_rows(q, k, v, do, sc, causal)
        out, flse = orc.attn_fwd(q, k, v, sc, causal)
        _close(delta, np.sum(out * do.astype(np.float64), axis=-1).reshape(-1), 1e-12, "delta")
        _close(lse, flse.reshape(-1), 1e-12, "pass-1 lse")


def pin_bwd_special(orc):
    """S = 1: out = v_0, so dv_0 = sum of dout over the group and dq = dk = 0.
    Causal query 0 sees one key, so dq_0 = 0; causal key S-1 is seen only by
    query S-1.  Gradients are linear in dout (doubling is exact)."""
    q = _randn((1, 4, 1, 5), 90)
    k = _randn((1, 2, 1, 5), 91)
    v = _randn((1, 2, 1, 5), 92)
    do = _randn((1, 4, 1, 5), 93)
    for causal in (True, False):
        dq, dk, dv = orc.attn_bwd(q, k, v, do, 0.3, causal)
        _close(dq, np.zeros_like(dq), 0.0, "S=1 dq")
        _close(dk, np.zeros_like(dk), 0.0, "S=1 dk")
        _close(dv, do.astype(np.float64).reshape(1, 2, 2, 1, 5).sum(axis=2), 1e-15, "S=1 dv")
    B, Hq, S, D = 1, 1, 12, 6
    q = _randn((B, Hq, S, D), 94)
    k = _randn((B, Hq, S, D), 95)
    v = _randn((B, Hq, S, D), 96)
    do = _randn((B, Hq, S, D), 97)
    dq, dk, dv = orc.attn_bwd(q, k, v, do, 0.5, True)
    _close(dq[0, 0, 0], np.zeros(D), 0.0, "causal dq_0")
    _, lse = orc.attn_fwd(q, k, v, 0.5, True)
    p_last = math.exp(0.5 * float(np.dot(q[0, 0, -1].astype(np.float64), k[0, 0, -1])) - lse[0, 0, -1])
    _close(dv[0, 0, -1], p_last * do[0, 0, -1].astype(np.float64), 1e-14, "causal dv_last")
    dq2, dk2, dv2 = orc.attn_bwd(q, k, v, 2 * do, 0.5, True)
    _close(dq2, 2 * dq, 0.0, "linear dq")
    _close(dk2, 2 * dk, 0.0, "linear dk")
    _close(dv2, 2 * dv, 0.0, "linear dv")


BWD_PINS = [pin_bwd_finite_diff, pin_bwd_torch, pin_bwd_invariants, pin_bwd_special]

ALL_PINS = ATTN_PINS + STEP_PINS + LOCAL_PINS + BLOCK_PINS + KV_PINS + SPREAD_PINS + BWD_PINS
