"""Helpers of the cache-append tests: read the rows of given token positions
out of a paged cache (by the page layout alone), and punch those slots out of
a copy of the cache so that an append has to restore them."""
from __future__ import annotations

import copy

import torch

from msa_inputs import POISON


def token_rows(cache, shape, seq: int, positions):
    """k, v [n][Hkv][D] and idx_k [n][d_i] of the listed positions of one sequence."""
    B = shape.block_size
    pos = torch.as_tensor(list(positions), dtype=torch.long, device=cache.k.device)
    pages = cache.block_table[seq].to(pos.device).long()[pos // B]
    slots = pos % B
    k = cache.k[pages, :, slots, :]
    v = cache.v[pages, :, slots, :]
    if cache.idx_k.dim() == 4:  # per-group index keys: [n][Hkv][d_i]
        idx = cache.idx_k[pages, :, slots, :]
    else:
        idx = cache.idx_k[pages, slots, :]
    return k.contiguous(), v.contiguous(), idx.contiguous()


def new_token_batch(cache, shape, starts, n_new):
    """k_new, v_new [batch][n_new][Hkv][D], idx_new [batch][n_new][d_i] (or
    [batch][n_new][Hkv][d_i] with per-group index keys) holding the tokens
    start[s] .. start[s]+n_new-1 of every sequence."""
    rows = [token_rows(cache, shape, s, range(st, st + n_new)) for s, st in enumerate(starts)]
    return (torch.stack([r[0] for r in rows]), torch.stack([r[1] for r in rows]),
            torch.stack([r[2] for r in rows]))


def holed_copy(cache, shape, starts, n_new):
    """A copy of the cache with the slots of the new tokens set to POISON."""
    c = copy.copy(cache)
    c.k, c.v, c.idx_k = cache.k.clone(), cache.v.clone(), cache.idx_k.clone()
    B = shape.block_size
    for s, st in enumerate(starts):
        pos = torch.arange(st, st + n_new, device=cache.k.device)
        pages = cache.block_table[s].to(pos.device).long()[pos // B]
        slots = pos % B
        c.k[pages, :, slots, :] = POISON
        c.v[pages, :, slots, :] = POISON
        if c.idx_k.dim() == 4:
            c.idx_k[pages, :, slots, :] = POISON
        else:
            c.idx_k[pages, slots, :] = POISON
    return c


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))
