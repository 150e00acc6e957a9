"""Pins of the oracle against things other than itself (CPU only).

* an independent numpy brute force (tests/bruteforce.py) on tiny inputs;
* the TopK rule against a full sort, and its special cases;
* constructed exact ties (lower block index wins, -0.0 == +0.0);
* dense causal GQA attention (torch's scaled_dot_product_attention in
  float64) when k covers every block;
* the softmax normalisation invariant (constant values);
* the causal limit: later blocks whose index keys would win are never kept;
* decode == prefill with a one-token chunk; page-shuffle and in-group head
  permutation invariance;
* a hand-worked example with the diagram's structure (tests/golden).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from msa_inputs import Shape, make_decode_case, make_prefill_case, PagedCache, DecodeCase
from tests import bruteforce

TINY = Shape(num_q_heads=6, num_kv_heads=2, head_dim=16, num_idx_heads=3, idx_dim=8,
             block_size=4, top_k=3)
TINY1 = Shape(num_q_heads=3, num_kv_heads=1, head_dim=8, num_idx_heads=1, idx_dim=4,
              block_size=16, top_k=2)


def _cmp_decode(case, tol=1e-12):
    o = oracle.decode(case)
    r = bruteforce.decode(case)
    np.testing.assert_array_equal(o["sel"], r["sel"])
    for s, L in enumerate(case.lengths):
        own = (L - 1) // case.shape.block_size
        for g in range(case.shape.num_kv_heads):
            np.testing.assert_array_equal(o["pooled"][s, g, :own], r["pooled"][s][g])
            assert np.all(np.isneginf(o["pooled"][s, g, own:]))
    np.testing.assert_allclose(o["out"], r["out"], rtol=tol, atol=tol)
    return o


@pytest.mark.parametrize("shape,lengths,seed", [
    (TINY, [37, 9, 1, 4, 5, 17], 11),
    (TINY, [64, 63, 65], 12),
    (TINY1, [300, 16, 17], 13),
    (Shape(num_q_heads=4, num_kv_heads=2, head_dim=8, num_idx_heads=2, idx_dim=4,
           block_size=1, top_k=5), [12, 1, 2, 6], 14),
])
def test_decode_matches_bruteforce(shape, lengths, seed):
    _cmp_decode(make_decode_case(shape, lengths, seed))


def test_decode_paged_poisoned_matches_bruteforce():
    case = make_decode_case(TINY, [41, 7, 28, 13], 21, shuffle_pages=True, poison_frac=0.3)
    _cmp_decode(case)


@pytest.mark.parametrize("P,C,seed", [(0, 19, 31), (13, 22, 32), (16, 8, 33), (5, 1, 34),
                                      (37, 40, 35)])
def test_prefill_matches_bruteforce(P, C, seed):
    case = make_prefill_case(TINY, P, C, seed, shuffle_pages=True, poison_frac=0.2)
    o = oracle.prefill(case)
    r = bruteforce.prefill(case)
    np.testing.assert_array_equal(o["sel"], r["sel"])
    B = TINY.block_size
    for tau in range(case.num_tiles):
        own = P // B + tau
        for g in range(TINY.num_kv_heads):
            np.testing.assert_array_equal(o["pooled"][tau, g, :own], r["pooled"][tau][g])
    np.testing.assert_allclose(o["out"], r["out"], rtol=1e-12, atol=1e-12)


def test_selection_never_beyond_the_causal_limit():
    """Index keys of the chunk's later blocks are set to the tile queries'
    direction, so they would outrank every earlier block if a tile could see
    them: each tile still keeps only blocks up to its own diagonal block, and
    its pooled scores past that block stay unscored."""
    P, C = 24, 40
    case = make_prefill_case(TINY, P, C, 44, shuffle_pages=True)
    B = TINY.block_size
    c = case.cache
    direction = case.idx_q.float().sum(dim=(0, 1, 2))  # [d_i]
    direction = (8.0 * direction / direction.norm()).to(torch.bfloat16)
    for b in range(P // B + 1, (P + C - 1) // B + 1):
        page = int(c.block_table[0, b])
        c.idx_k[page] = direction
    o = oracle.prefill(case)
    r = bruteforce.prefill(case)
    np.testing.assert_array_equal(o["sel"], r["sel"])
    for tau in range(case.num_tiles):
        own = P // B + tau
        kept = o["sel"][tau]
        assert kept.max() == own and (kept[kept >= 0] <= own).all()
        assert np.isneginf(o["pooled"][tau, :, own:]).all()


def test_prefill_tile_subset_equals_full():
    case = make_prefill_case(TINY, 21, 30, 41)
    full = oracle.prefill(case)
    part = oracle.prefill(case, tiles=[0, 3, 7])
    for tau in [0, 3, 7]:
        np.testing.assert_array_equal(part["sel"][tau], full["sel"][tau])
        q0, q1 = oracle.tile_rows(case, tau)
        np.testing.assert_array_equal(part["out"][q0:q1], full["out"][q0:q1])
    assert np.all(part["sel"][1] == -2) and np.isnan(part["out"][oracle.tile_rows(case, 1)[0]]).all()


# ---------------------------------------------------------------- TopK rule
def _by_sort(scores, own, k):
    order = sorted(range(own), key=lambda b: (-scores[b], b))
    keep = sorted(order[:min(k - 1, own)] + [own])
    return keep + [-1] * (k - len(keep))


def test_select_matches_full_sort_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(400):
        own = int(rng.integers(0, 40))
        k = int(rng.integers(1, 12))
        scores = rng.integers(-3, 4, size=max(own, 1)).astype(np.float64)  # many ties
        got = oracle.select(scores[:own], own, k).tolist()
        assert got == _by_sort(scores, own, k), (own, k, scores[:own])


def test_select_special_cases():
    s = np.arange(10, dtype=np.float64)[::-1].copy()  # block 0 best
    assert oracle.select(s, 10, 1).tolist() == [10]                 # k=1: own only
    assert oracle.select(s, 10, 11).tolist() == list(range(11))     # k > own: all
    assert oracle.select(s, 10, 13).tolist() == list(range(11)) + [-1, -1]
    assert oracle.select(s, 0, 4).tolist() == [0, -1, -1, -1]       # first block
    assert oracle.select(s, 10, 4).tolist() == [0, 1, 2, 10]
    z = np.array([0.0, -0.0, 0.0, -1.0])                            # -0.0 == +0.0
    assert oracle.select(z, 4, 2).tolist() == [0, 4]
    z = np.array([-1.0, -0.0, 0.0, -1.0])
    assert oracle.select(z, 4, 2).tolist() == [1, 4]


def test_constructed_exact_ties_lower_index_wins():
    shape = Shape(num_q_heads=4, num_kv_heads=2, head_dim=8, num_idx_heads=2, idx_dim=8,
                  block_size=4, top_k=3)
    case = make_decode_case(shape, [40], 51)
    ik = case.cache.idx_k
    # copy block 2 into blocks 5 and 8: pooled scores become bit-equal
    for dst in (5, 8):
        ik[dst] = ik[2]
    # make block 2's content the clear winner for both groups
    ik[2] = (ik[2].float() * 0 + 3.0).to(torch.bfloat16)
    for dst in (5, 8):
        ik[dst] = ik[2]
    case.idx_q[:] = torch.abs(case.idx_q)
    o = oracle.decode(case)
    for g in range(2):
        assert o["pooled"][0, g, 2] == o["pooled"][0, g, 5] == o["pooled"][0, g, 8]
        assert o["sel"][0, g].tolist() == [2, 5, 9]  # two of the three tied blocks: 2 and 5
    _cmp_decode(case)


def test_signed_zero_tie():
    shape = Shape(num_q_heads=2, num_kv_heads=1, head_dim=4, num_idx_heads=1, idx_dim=4,
                  block_size=2, top_k=2)
    case = make_decode_case(shape, [9], 52)
    case.idx_q[:] = 1.0
    ik = case.cache.idx_k
    ik[:] = -torch.abs(ik) - 0.5          # every block scores below zero
    ik[1] = -0.0                           # block 1: products -0.0, score zero
    ik[3] = 0.0                            # block 3: products +0.0, score zero
    o = oracle.decode(case)
    assert o["pooled"][0, 0, 1] == 0.0 and o["pooled"][0, 0, 3] == 0.0
    assert o["sel"][0, 0].tolist() == [1, 4]


# -------------------------------------------------------- dense equivalence
def _dense_causal(q, K, V, scale, G):
    """Textbook causal GQA attention, float64, via torch SDPA.
    q [Hq][Lq][D] at positions P..P+Lq-1, K/V [Hkv][L][D]."""
    Hq, Lq, _ = q.shape
    L = K.shape[1]
    Kx = torch.from_numpy(K).repeat_interleave(G, dim=0)
    Vx = torch.from_numpy(V).repeat_interleave(G, dim=0)
    pos = torch.arange(L - Lq, L)
    mask = torch.arange(L)[None, :] <= pos[:, None]
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), Kx, Vx, attn_mask=mask, scale=scale).numpy()


def test_decode_dense_when_k_covers_all_blocks():
    shape = Shape(num_q_heads=8, num_kv_heads=2, head_dim=16, num_idx_heads=2, idx_dim=8,
                  block_size=8, top_k=64)
    case = make_decode_case(shape, [200, 8, 9, 511], 61, shuffle_pages=True)
    o = oracle.decode(case)
    for s, L in enumerate(case.lengths):
        K, V, _ = bruteforce.logical(case, s, L)
        q = bruteforce.f64(case.q[s])[:, None, :]
        ref = _dense_causal(q, K, V, shape.softmax_scale, shape.group_size)[:, 0]
        np.testing.assert_allclose(o["out"][s], ref, rtol=1e-11, atol=1e-12)
        nb = (L - 1) // 8 + 1
        assert o["sel"][s, 0, :nb].tolist() == list(range(nb))


def test_prefill_dense_when_k_covers_all_blocks():
    shape = Shape(num_q_heads=4, num_kv_heads=2, head_dim=16, num_idx_heads=2, idx_dim=8,
                  block_size=8, top_k=40)
    case = make_prefill_case(shape, 45, 70, 62)
    o = oracle.prefill(case)
    K, V, _ = bruteforce.logical(case, 0, 115)
    q = bruteforce.f64(case.q).transpose(1, 0, 2)
    ref = _dense_causal(q, K, V, shape.softmax_scale, 2).transpose(1, 0, 2)
    np.testing.assert_allclose(o["out"], ref, rtol=1e-11, atol=1e-12)


def test_constant_values_give_that_value():
    case = make_decode_case(TINY, [50, 23], 71, shuffle_pages=True)
    u = torch.randn(TINY.num_kv_heads, TINY.head_dim, dtype=torch.float64)
    u_bf = u.to(torch.bfloat16)
    case.cache.v[:] = u_bf[None, :, None, :]
    o = oracle.decode(case)
    G = TINY.group_size
    for j in range(TINY.num_q_heads):
        np.testing.assert_allclose(o["out"][:, j], u_bf[j // G].double().numpy()[None].repeat(2, 0),
                                   rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------- invariances
def test_decode_equals_prefill_with_one_token_chunk():
    for L, seed in [(33, 81), (1, 82), (4, 83), (5, 84)]:
        d = make_decode_case(TINY, [L], seed)
        p = make_prefill_case(TINY, L - 1, 1, seed)
        # same cache content, and the chunk query equals the decode query
        p.cache = d.cache
        p.q, p.idx_q = d.q.clone(), d.idx_q.clone()
        od, op = oracle.decode(d), oracle.prefill(p)
        np.testing.assert_array_equal(od["sel"][0], op["sel"][0])
        np.testing.assert_array_equal(od["out"][0], op["out"][0])


def test_page_shuffle_invariance():
    a = make_decode_case(TINY, [45, 12, 30], 91)
    b = make_decode_case(TINY, [45, 12, 30], 91)
    n = a.cache.num_pages
    perm = torch.from_numpy(np.random.default_rng(3).permutation(n))
    inv = torch.argsort(perm)
    for name in ("k", "v", "idx_k"):
        setattr(b.cache, name, getattr(a.cache, name)[perm].clone())
    b.cache.block_table = inv[a.cache.block_table.long()].to(torch.int32)
    oa, ob = oracle.decode(a), oracle.decode(b)
    np.testing.assert_array_equal(oa["sel"], ob["sel"])
    np.testing.assert_array_equal(oa["out"], ob["out"])


def test_head_permutation_within_group_permutes_outputs():
    a = make_decode_case(TINY, [47, 20], 92)
    b = make_decode_case(TINY, [47, 20], 92)
    perm = [2, 0, 1, 5, 3, 4]          # permutes heads inside each group of 3
    b.q = a.q[:, perm].clone()
    oa, ob = oracle.decode(a), oracle.decode(b)
    np.testing.assert_array_equal(oa["out"][:, perm], ob["out"])
    np.testing.assert_array_equal(oa["sel"], ob["sel"])


# ----------------------------------------------------------- hand-worked
def test_handworked_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "t0_handworked.json")
    g = json.load(open(path))
    sh = Shape(**g["shape"], scale=g["softmax_scale"])
    L, B = g["seq_len"], sh.block_size
    nb = (L + B - 1) // B
    bf = lambda x: torch.tensor(x, dtype=torch.float64).to(torch.bfloat16)
    k = torch.zeros(nb * B, sh.num_kv_heads, sh.head_dim)
    v = torch.zeros(nb * B, sh.num_kv_heads, sh.head_dim)
    ik = torch.zeros(nb * B, sh.idx_dim)
    k[:L] = torch.tensor(g["k"], dtype=torch.float64).permute(1, 0, 2).float()
    v[:L] = torch.tensor(g["v"], dtype=torch.float64).permute(1, 0, 2).float()
    ik[:L] = torch.tensor(g["idx_k"]).float()
    cache = PagedCache(
        k=k.view(nb, B, sh.num_kv_heads, sh.head_dim).permute(0, 2, 1, 3).contiguous().to(torch.bfloat16),
        v=v.view(nb, B, sh.num_kv_heads, sh.head_dim).permute(0, 2, 1, 3).contiguous().to(torch.bfloat16),
        idx_k=ik.view(nb, B, sh.idx_dim).contiguous().to(torch.bfloat16),
        block_table=torch.arange(nb, dtype=torch.int32)[None], num_pages=nb, max_blocks=nb,
        lengths=[L])
    case = DecodeCase(sh, cache, bf([g["q"]]), bf([g["idx_q"]]),
                      torch.tensor([L], dtype=torch.int32), [L])
    o = oracle.decode(case)
    np.testing.assert_array_equal(o["pooled"][0, :, :3], np.array(g["expected_pooled"], float))
    np.testing.assert_array_equal(o["sel"][0], np.array(g["expected_sel"]))
    np.testing.assert_allclose(o["out"][0], np.array(g["expected_out"]), rtol=1e-14, atol=1e-14)
