"""The CPU oracle against its pins, and planted mistakes against the pins."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


# Each planted variant is compiled from attn_oracle.c with -DORACLE_PLANT=n.
PLANTS = {
    1: "scale dropped",
    2: "K operand read transposed",
    3: "causal mask off by one",
    4: "sign of the exponent flipped",
    5: "GQA heads grouped by stride",
    6: "normalisation dropped",
    7: "lse in base 2",
    8: "backward delta left out",
    9: "backward dk scale dropped",
    10: "backward dq uses v for k",
    11: "backward key pass mask flipped",
    12: "backward dk dv from one head of the group",
    13: "sliding window one key too wide",
    14: "decode queries aligned top-left",
    15: "block mask transposed",
    16: "block mask batch and head strides swapped",
}


@pytest.fixture(scope="module")
def planted(tmp_path_factory):
    d = tmp_path_factory.mktemp("planted")
    libs = {}
    for n in PLANTS:
        path = oracle.compile_oracle(d / f"liboracle_plant{n}.so", plant=n)
        libs[n] = oracle.Oracle(path)
        assert libs[n].plant == n
    return libs


@pytest.mark.parametrize("n", sorted(PLANTS), ids=lambda n: PLANTS[n].replace(" ", "_"))
def test_planted_mistake_is_caught(planted, n):
    orc = planted[n]
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake: {PLANTS[n]}"


def test_rows_match_full(orc):
    """Sampled rows return the same values as the full computation."""
    rng = np.random.default_rng(50)
    q = rng.standard_normal((2, 4, 20, 8)).astype(np.float32)
    k = rng.standard_normal((2, 2, 20, 8)).astype(np.float32)
    v = rng.standard_normal((2, 2, 20, 8)).astype(np.float32)
    out, lse = orc.attn_fwd(q, k, v, 0.3, True)
    rows = np.array([0, 1, 19, 20, 77, 159], np.int64)
    o2, l2 = orc.attn_fwd(q, k, v, 0.3, True, rows=rows)
    assert np.array_equal(o2, out.reshape(-1, 8)[rows])
    assert np.array_equal(l2, lse.reshape(-1)[rows])


def test_bad_rows_rejected(orc):
    q = np.zeros((1, 1, 4, 2), np.float32)
    with pytest.raises(RuntimeError):
        orc.attn_fwd(q, q, q, 1.0, True, rows=np.array([4], np.int64))
    with pytest.raises(RuntimeError):
        orc.attn_fwd(q, q, q, 1.0, True, rows=np.array([-1], np.int64))


def test_bwd_rows_keys_match_full(orc):
    """Sampled query rows and key rows of the backward equal the full result."""
    rng = np.random.default_rng(51)
    q = rng.standard_normal((2, 4, 20, 8)).astype(np.float32)
    k = rng.standard_normal((2, 2, 20, 8)).astype(np.float32)
    v = rng.standard_normal((2, 2, 20, 8)).astype(np.float32)
    do = rng.standard_normal((2, 4, 20, 8)).astype(np.float32)
    dq, dk, dv = orc.attn_bwd(q, k, v, do, 0.3, True)
    rows = np.array([0, 19, 20, 77, 159], np.int64)
    lse, delta, dq2 = orc.attn_bwd_rows(q, k, v, do, 0.3, True, rows=rows)
    assert np.array_equal(dq2, dq.reshape(-1, 8)[rows])
    la, da, _ = orc.attn_bwd_rows(q, k, v, do, 0.3, True)
    keys = np.array([0, 7, 39, 79], np.int64)
    dk2, dv2 = orc.attn_bwd_keys(q, k, v, do, 0.3, True, la, da, keys=keys)
    assert np.array_equal(dk2, dk.reshape(-1, 8)[keys])
    assert np.array_equal(dv2, dv.reshape(-1, 8)[keys])
