"""Pins of the oracle's forced blocks (CPU): the first `sink_blocks` blocks and
the `local_blocks` blocks just before the own block are always kept, count
toward k, and are never ranked ("MiniMax wird dünn", section 2: the dropped
sliding-window branch is probably replaced by an attention sink or local
attention; the forced blocks are the plainest form of that).

* the rule against an independent full-sort implementation with many ties;
* special cases: no forced blocks = the plain rule; sink + local = k-1 keeps
  exactly the forced blocks whatever the scores; short sequences keep all;
* decode and prefill against the numpy brute force with forced blocks;
* with sink + local = k-1 the output is textbook attention restricted to the
  sink tokens and the causal local window (torch SDPA with that mask);
* the index keys of forced blocks do not influence the selection.
"""
import numpy as np
import pytest
import torch

import oracle
from msa_inputs import Shape, make_decode_case, make_prefill_case
from tests import bruteforce
from tests.test_oracle_pins import _cmp_decode

FORCED = Shape(num_q_heads=6, num_kv_heads=2, head_dim=16, num_idx_heads=3, idx_dim=8,
               block_size=4, top_k=5, sink_blocks=1, local_blocks=2)


def test_select_forced_matches_full_sort_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(600):
        own = int(rng.integers(0, 40))
        k = int(rng.integers(1, 12))
        sink = int(rng.integers(0, k))
        local = int(rng.integers(0, k - sink))
        scores = rng.integers(-3, 4, size=max(own, 1)).astype(np.float64)
        got = oracle.select(scores[:own], own, k, sink, local).tolist()
        want = bruteforce.topk_sorted(scores, own, k, sink, local).tolist()
        assert got == want, (own, k, sink, local, scores[:own])


def test_select_forced_special_cases():
    s = np.arange(20, dtype=np.float64)              # block 19 best, block 0 worst
    assert oracle.select(s, 20, 6, 0, 0).tolist() == oracle.select(s, 20, 6).tolist()
    # sink + local = k-1: the forced blocks and own only, whatever the scores
    assert oracle.select(s, 20, 6, 2, 3).tolist() == [0, 1, 17, 18, 19, 20]
    assert oracle.select(-s, 20, 6, 2, 3).tolist() == [0, 1, 17, 18, 19, 20]
    # one slot left: the best of blocks 2..17 (block 17)
    assert oracle.select(s, 20, 6, 2, 2).tolist() == [0, 1, 17, 18, 19, 20]
    assert oracle.select(-s, 20, 6, 2, 2).tolist() == [0, 1, 2, 18, 19, 20]
    # forced ranges overlapping on a short sequence
    assert oracle.select(s, 3, 6, 2, 3).tolist() == [0, 1, 2, 3, -1, -1]
    assert oracle.select(s, 0, 3, 1, 1).tolist() == [0, -1, -1]
    with pytest.raises(ValueError):
        oracle.select(s, 20, 4, 2, 2)                 # sink + local > k-1


@pytest.mark.parametrize("lengths,seed", [([37, 9, 1, 4, 5, 17, 64], 81), ([100, 33], 82)])
def test_decode_forced_matches_bruteforce(lengths, seed):
    _cmp_decode(make_decode_case(FORCED, lengths, seed, shuffle_pages=True, poison_frac=0.2))


@pytest.mark.parametrize("P,C,seed", [(0, 19, 83), (13, 22, 84), (37, 40, 85)])
def test_prefill_forced_matches_bruteforce(P, C, seed):
    case = make_prefill_case(FORCED, P, C, seed, shuffle_pages=True, poison_frac=0.2)
    o, r = oracle.prefill(case), bruteforce.prefill(case)
    np.testing.assert_array_equal(o["sel"], r["sel"])
    np.testing.assert_allclose(o["out"], r["out"], rtol=1e-12, atol=1e-12)


def test_sink_plus_local_window_is_masked_dense_attention():
    shape = Shape(num_q_heads=8, num_kv_heads=2, head_dim=16, num_idx_heads=2, idx_dim=8,
                  block_size=8, top_k=6, sink_blocks=2, local_blocks=3)
    case = make_decode_case(shape, [200, 9, 61, 333], 86, shuffle_pages=True)
    o = oracle.decode(case)
    B, G = shape.block_size, shape.group_size
    for s, L in enumerate(case.lengths):
        K, V, _ = bruteforce.logical(case, s, L)
        own = (L - 1) // B
        t = np.arange(L)
        keep = (t < 2 * B) | (t >= max(own - 3, 0) * B)     # sink tokens + window up to now
        q = torch.from_numpy(bruteforce.f64(case.q[s])[:, None, :])
        Kx = torch.from_numpy(K).repeat_interleave(G, dim=0)
        Vx = torch.from_numpy(V).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, Kx, Vx, attn_mask=torch.from_numpy(keep)[None, :], scale=shape.softmax_scale)
        np.testing.assert_allclose(o["out"][s], ref[:, 0].numpy(), rtol=1e-11, atol=1e-12)


def test_forced_blocks_index_keys_do_not_matter():
    case = make_decode_case(FORCED, [120, 77], 87)
    a = oracle.decode(case)["sel"]
    B = FORCED.block_size
    for s, L in enumerate(case.lengths):
        own = (L - 1) // B
        for b in [0, own - 1, own - 2]:
            page = int(case.cache.block_table[s, b])
            case.cache.idx_k[page] = 50.0 if b % 2 else -50.0
    b2 = oracle.decode(case)["sel"]
    np.testing.assert_array_equal(a, b2)
