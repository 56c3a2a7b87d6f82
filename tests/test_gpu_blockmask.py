"""Block-masked forward (attn_fwd_blockmask_bf16) against the fp64 oracle.

One flag per 64 queries x 64 keys; query i sees key j when the flag of
(i / 64, j / 64) is set (and j <= i when causal).  Small shapes are compared
over every element for random masks of several densities, with a query block
that sees nothing and one that sees everything, ragged S, D 64/128 and GQA;
the B4 H16 S4096 D128 workload and a 40000-key sequence (more tiles than one
pass of the workgroup's list building covers) on sampled rows.  Rows that see
no key must give out 0 and lse -inf.  An all-ones mask must reproduce the
unmasked kernel bit for bit; a broadcast mask must equal its written-out copy.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import gpu_util as G
from scaled_dot_product_10_amd import api, inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def nblk(S):
    return (S + 63) // 64


def random_mask(Bm, Hm, S, density, seed):
    """Random flags with, per (b, h), one query block that sees nothing and
    one that sees every key block (when there are at least two)."""
    nb = nblk(S)
    rng = np.random.default_rng(seed)
    m = (rng.random((Bm, Hm, nb, nb)) < density).astype(np.uint8)
    if nb >= 2:
        m[:, :, 1, :] = 0
        m[:, :, 0, :] = 1
    return m


def check_masked(name, out, lse, ref_o, ref_l, D):
    """Rows with a visible key against the oracle; rows without: exactly out 0
    and lse -inf."""
    got_o = G.host(out).reshape(-1, D)
    got_l = G.host(lse).reshape(-1)
    ref_o = np.asarray(ref_o).reshape(-1, D)
    ref_l = np.asarray(ref_l).reshape(-1)
    empty = ~np.isfinite(ref_l)
    assert np.all(got_o[empty] == 0.0), f"{name}: rows that see nothing must be 0"
    assert np.all(got_l[empty] == -np.inf), f"{name}: rows that see nothing must have lse -inf"
    G.check_close(name, got_o[~empty], ref_o[~empty], "bf16", got_l[~empty], ref_l[~empty])
    return int(empty.sum())


SHAPES = [(1, 2, 1, 100, 64), (2, 4, 2, 300, 128), (1, 2, 2, 64, 128), (1, 1, 1, 1, 64), (1, 3, 1, 520, 64),
          (1, 2, 1, 1000, 128), (2, 2, 2, 257, 64)]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("density", [0.25, 0.7])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}kv{}S{}D{}".format(*s))
def test_small_full_compare(orc, shape, density, causal):
    B, Hq, Hkv, S, D = shape
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, D, "bf16", seed=7000 + S + D)
    m = random_mask(B, Hq, S, density, seed=7100 + S)
    sc = 1.0 / math.sqrt(D)
    out, lse = api.fwd(G.dev(q), G.dev(k), G.dev(v), causal=causal, scale=sc,
                       block_mask=torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = orc.attn_fwd_blockmask(q.f32, k.f32, v.f32, sc, causal, m)
    check_masked(f"blockmask {shape} d={density} causal={causal}", out, lse, ref_o, ref_l, D)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_all_ones_is_unmasked(causal):
    # 288 workgroups of 256 queries: the plain kernel runs the same schedule
    # as the block-mask one (smaller grids split each workgroup's key range
    # between its two wave groups, which sums in another order), so the two
    # agree bit for bit
    q, k, v = inputs.make_qkv(2, 48, 2, 700, 128, "bf16", seed=7200)
    Q, K, V = G.dev(q), G.dev(k), G.dev(v)
    o1, l1 = api.fwd(Q, K, V, causal=causal)
    ones = torch.ones((1, 1, nblk(700), nblk(700)), dtype=torch.bool, device="cuda")
    o2, l2 = api.fwd(Q, K, V, causal=causal, block_mask=ones)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_mask():
    q, k, v = inputs.make_qkv(1, 2, 1, 300, 64, "bf16", seed=7201)
    zeros = torch.zeros((1, 2, nblk(300), nblk(300)), dtype=torch.uint8, device="cuda")
    out, lse = api.fwd(G.dev(q), G.dev(k), G.dev(v), causal=False, block_mask=zeros)
    torch.cuda.synchronize()
    assert bool((out == 0).all()) and bool(torch.isneginf(lse).all())


def test_broadcast_and_strided_masks():
    B, Hq, Hkv, S, D = 2, 4, 2, 400, 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, D, "bf16", seed=7202)
    Q, K, V = G.dev(q), G.dev(k), G.dev(v)
    nb = nblk(S)
    per_head = torch.from_numpy(random_mask(1, Hq, S, 0.5, 7203)).cuda()
    full = per_head.expand(B, Hq, nb, nb).contiguous()
    o1, l1 = api.fwd(Q, K, V, causal=True, block_mask=per_head)
    o2, l2 = api.fwd(Q, K, V, causal=True, block_mask=full)
    o3, l3 = api.fwd(Q, K, V, causal=True, block_mask=per_head.expand(B, Hq, nb, nb))  # stride 0 over batch
    big = torch.from_numpy(random_mask(B, 2 * Hq, S, 0.5, 7204)).cuda()
    o4, l4 = api.fwd(Q, K, V, causal=True, block_mask=big[:, ::2])  # head stride 2 nb^2
    o5, l5 = api.fwd(Q, K, V, causal=True, block_mask=big[:, ::2].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert torch.equal(o4, o5) and torch.equal(l4, l5)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_c3_sampled(orc, causal):
    c = inputs.CONFIGS["C3"]
    B, Hq, Hkv, S, D = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"]
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, D, "bf16", c["seed"])
    m = random_mask(B, Hq, S, 0.3, seed=7300)
    sc = 1.0 / math.sqrt(D)
    out, lse = api.fwd(G.dev(q), G.dev(k), G.dev(v), causal=causal, scale=sc, block_mask=torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    rows = G.sample_rows(B, Hq, S, n_random=300, seed=c["seed"], tile=256)
    ref_o, ref_l = orc.attn_fwd_blockmask(q.f32, k.f32, v.f32, sc, causal, m, rows=rows)
    idx = torch.from_numpy(rows).to(out.device)
    n_empty = check_masked(f"C3 blockmask causal={causal} rows={rows.size}", out.view(-1, D)[idx],
                           lse.view(-1)[idx], ref_o, ref_l, D)
    assert n_empty > 0  # query block 1 sees nothing


def test_long_sequence_sampled(orc):
    """40000 keys: 625 key tiles, more than the 512 threads that build the
    list in one pass."""
    B, Hq, Hkv, S, D = 1, 2, 1, 40000, 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, D, "bf16", seed=7400)
    m = random_mask(B, Hq, S, 0.1, seed=7401)
    sc = 1.0 / math.sqrt(D)
    out, lse = api.fwd(G.dev(q), G.dev(k), G.dev(v), causal=False, scale=sc, block_mask=torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    rows = G.sample_rows(B, Hq, S, n_random=60, seed=7402, tile=256)
    ref_o, ref_l = orc.attn_fwd_blockmask(q.f32, k.f32, v.f32, sc, False, m, rows=rows)
    idx = torch.from_numpy(rows).to(out.device)
    check_masked(f"S=40000 blockmask rows={rows.size}", out.view(-1, D)[idx], lse.view(-1)[idx], ref_o, ref_l, D)


def test_max_sequence(orc):
    """S = 131072, the block mask's limit: 2048 key tiles, the longest list a
    workgroup can hold (causal, so late workgroups list up to all of them)."""
    B, Hq, Hkv, S, D = 1, 1, 1, 131072, 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, D, "bf16", seed=7500)
    nb = nblk(S)
    rng = np.random.default_rng(7501)
    m = (rng.random((1, 1, nb, nb)) < 0.05).astype(np.uint8)
    m[0, 0, -1, :] = 1  # the last query block lists every tile
    np.fill_diagonal(m[0, 0], 1)
    sc = 1.0 / math.sqrt(D)
    out, lse = api.fwd(G.dev(q), G.dev(k), G.dev(v), causal=True, scale=sc, block_mask=torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    rows = G.sample_rows(B, Hq, S, n_random=30, seed=7502, tile=256)
    ref_o, ref_l = orc.attn_fwd_blockmask(q.f32, k.f32, v.f32, sc, True, m, rows=rows)
    idx = torch.from_numpy(rows).to(out.device)
    check_masked(f"S=131072 blockmask rows={rows.size}", out.view(-1, D)[idx], lse.view(-1)[idx], ref_o, ref_l, D)
