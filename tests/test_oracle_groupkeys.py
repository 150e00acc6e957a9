"""Pins of the oracle's per-group index keys (CPU): the ablation of the single
shared index-key head ("MiniMax wird dünn", section 1, Schritt 1: K_idx has
one head shared by every group), where each KV group scores its blocks
against an index-key head of its own.

* decode and prefill against the numpy brute force with per-group keys;
* when every group's key head is a copy of one head, the results equal the
  shared-head method's bit for bit (pooled scores, selections, outputs);
* a group reads only its own key head: redrawing another group's head leaves
  the group's pooled scores, selection and output unchanged, redrawing its own
  head changes its pooled scores;
* appends with per-group index keys restore the generated cache.
"""
import numpy as np
import pytest
import torch

import oracle
from msa_inputs import Shape, build_paged_cache, make_decode_case, make_prefill_case
from tests import bruteforce
from tests.append_util import holed_copy, new_token_batch
from tests.test_oracle_pins import _cmp_decode

GK = Shape(num_q_heads=6, num_kv_heads=3, head_dim=16, num_idx_heads=2, idx_dim=8,
           block_size=4, top_k=3, idx_k_heads=3)


@pytest.mark.parametrize("lengths,seed", [([37, 9, 1, 4, 5, 17, 64], 111), ([100, 33], 112)])
def test_decode_group_keys_matches_bruteforce(lengths, seed):
    _cmp_decode(make_decode_case(GK, lengths, seed, shuffle_pages=True, poison_frac=0.2))


@pytest.mark.parametrize("P,C,seed", [(0, 19, 113), (13, 22, 114), (37, 40, 115)])
def test_prefill_group_keys_matches_bruteforce(P, C, seed):
    case = make_prefill_case(GK, P, C, seed, shuffle_pages=True, poison_frac=0.2)
    o, r = oracle.prefill(case), bruteforce.prefill(case)
    np.testing.assert_array_equal(o["sel"], r["sel"])
    np.testing.assert_allclose(o["out"], r["out"], rtol=1e-12, atol=1e-12)


def test_identical_group_heads_equal_the_shared_head():
    shared = Shape(num_q_heads=6, num_kv_heads=3, head_dim=16, num_idx_heads=2, idx_dim=8,
                   block_size=4, top_k=3)
    a = make_decode_case(shared, [60, 23, 41], 116, shuffle_pages=True)
    b = make_decode_case(GK, [60, 23, 41], 116, shuffle_pages=True)
    b.cache.k, b.cache.v, b.q, b.idx_q = a.cache.k, a.cache.v, a.q, a.idx_q
    b.cache.idx_k = a.cache.idx_k[:, None].expand(-1, 3, -1, -1).contiguous()
    oa, ob = oracle.decode(a), oracle.decode(b)
    np.testing.assert_array_equal(oa["sel"], ob["sel"])
    np.testing.assert_array_equal(oa["pooled"], ob["pooled"])
    np.testing.assert_array_equal(oa["out"], ob["out"])


def test_group_reads_only_its_own_key_head():
    case = make_decode_case(GK, [60, 23, 41], 118, shuffle_pages=True)
    base = oracle.decode(case)
    G = GK.num_q_heads // GK.num_kv_heads
    rng = np.random.default_rng(119)
    for h in range(GK.num_kv_heads):
        alt = make_decode_case(GK, [60, 23, 41], 118, shuffle_pages=True)
        redraw = torch.from_numpy(rng.standard_normal(alt.cache.idx_k[:, h].shape)).to(torch.bfloat16)
        alt.cache.idx_k[:, h] = redraw
        res = oracle.decode(alt)
        for g in range(GK.num_kv_heads):
            heads = slice(g * G, (g + 1) * G)
            if g == h:
                assert not np.array_equal(res["pooled"][:, g], base["pooled"][:, g])
            else:
                np.testing.assert_array_equal(res["pooled"][:, g], base["pooled"][:, g])
                np.testing.assert_array_equal(res["sel"][:, g], base["sel"][:, g])
                np.testing.assert_array_equal(res["out"][:, heads], base["out"][:, heads])


def test_append_group_keys_restores_the_cache():
    shape = Shape(num_q_heads=8, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=4,
                  idx_k_heads=2)
    lengths = [700, 300]
    full = build_paged_cache(shape, lengths, seed=117, shuffle_pages=True, poison_frac=0.05)
    starts = [L - 70 - 9 for L in lengths]
    kn, vn, xn = new_token_batch(full, shape, starts, 70)
    assert xn.shape == (2, 70, 2, 64)
    hole = holed_copy(full, shape, starts, 70)
    arrays = [np.ascontiguousarray(t.view(torch.int16).numpy()) for t in (hole.k, hole.v, hole.idx_k)]
    oracle.cache_append(shape, *arrays, full.block_table, kn, vn, xn, starts)
    for a, t in zip(arrays, (full.k, full.v, full.idx_k)):
        np.testing.assert_array_equal(a, t.view(torch.int16).numpy())
