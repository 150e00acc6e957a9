"""Pins of the oracle's cache append (CPU): appending the rows of some tokens
into a cache whose slots for them were punched out must give back, bit for bit,
the cache the seeded generator built with those tokens in place.  The
generator lays the pages out independently of the oracle, so a wrong page,
slot, head, dimension or an untransposed V page fails the comparison."""
import numpy as np
import pytest
import torch

import oracle
from msa_inputs import Shape, build_paged_cache
from tests.append_util import holed_copy, new_token_batch

SHAPES = [Shape(num_q_heads=8, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=4),
          Shape(num_q_heads=12, num_kv_heads=3, num_idx_heads=2, block_size=128, top_k=4)]


def _host(t):
    return np.ascontiguousarray(t.view(torch.int16).numpy())


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("n_new,tail", [(1, 0), (150, 0), (70, 37), (1, 5)])
def test_append_restores_the_generated_cache(shape, n_new, tail):
    lengths = [700, 300, 1000]
    full = build_paged_cache(shape, lengths, seed=11, shuffle_pages=True, poison_frac=0.05)
    # new tokens end `tail` positions before each sequence's last token
    starts = [L - n_new - tail for L in lengths]
    k_new, v_new, idx_new = new_token_batch(full, shape, starts, n_new)
    hole = holed_copy(full, shape, starts, n_new)
    k, v, ik = _host(hole.k), _host(hole.v), _host(hole.idx_k)
    assert not np.array_equal(k, _host(full.k))  # the punch removed something
    oracle.cache_append(shape, k, v, ik, full.block_table, k_new, v_new, idx_new, starts)
    assert np.array_equal(k, _host(full.k))
    assert np.array_equal(v, _host(full.v))
    assert np.array_equal(ik, _host(full.idx_k))


def test_append_rejects_positions_past_the_table():
    shape = SHAPES[0]
    full = build_paged_cache(shape, [128], seed=3)
    k, v, ik = _host(full.k), _host(full.v), _host(full.idx_k)
    kn = torch.zeros(1, 1, shape.num_kv_heads, shape.head_dim, dtype=torch.bfloat16)
    xn = torch.zeros(1, 1, shape.idx_dim, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        oracle.cache_append(shape, k, v, ik, full.block_table, kn, kn, xn, [full.max_blocks * 64])
