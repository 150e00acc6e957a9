"""Pins of the oracle's entry points that take a selection or a query range
from the caller (CPU only): the sparse branch for a given selection
(attend_decode, attend_prefill) and single pooled scores (block_scores).

The GPU parity tests compare the kernels with exactly these functions, so each
is pinned on its own:
* fed the oracle's own selection, attend_decode / attend_prefill reproduce
  decode() / prefill() bit for bit; block_scores over all eligible blocks
  reproduces the pooled rows of decode() / prefill() bit for bit;
* on arbitrary valid selections (fewer blocks than k, -1 padding, a near-tie
  swap, forced blocks, tiles listed out of order) they match the numpy brute
  force, which is written independently (tests/bruteforce.py);
* prefill cases include partial first tiles (prior length not a multiple of
  the block size) and ragged last tiles.
"""
import numpy as np
import pytest

import oracle
from msa_inputs import Shape, make_decode_case, make_prefill_case
from tests import bruteforce
from tests.test_oracle_forced import FORCED
from tests.test_oracle_groupkeys import GK
from tests.test_oracle_pins import TINY, TINY1

DECODE_CASES = [
    (TINY, [37, 9, 1, 4, 5, 17], 301, dict(shuffle_pages=True, poison_frac=0.3)),
    (TINY1, [300, 16, 17], 302, {}),
    (FORCED, [37, 9, 1, 64], 303, dict(shuffle_pages=True, poison_frac=0.2)),
    (GK, [37, 9, 64], 304, dict(shuffle_pages=True, poison_frac=0.2)),
]
PREFILL_CASES = [
    (TINY, 13, 22, 311),   # partial first tile (13 % 4 = 1), ragged last tile
    (TINY, 16, 9, 312),    # aligned start, ragged last tile
    (TINY, 6, 1, 313),     # one query inside one tile
    (TINY1, 21, 40, 314),  # partial first tile, 16-token blocks
    (FORCED, 30, 13, 315),
]


def random_selection(rng, own: int, k: int) -> list:
    """A valid selection row: distinct blocks <= own, ascending, -1 padded,
    at least one block (the own block is included with probability 3/4)."""
    n = int(rng.integers(0, min(k - 1, own) + 1)) if own > 0 else 0
    rest = sorted(rng.choice(own, size=n, replace=False).tolist()) if n else []
    if rng.random() < 0.75 or not rest:
        rest = sorted(rest + [own])
    return rest + [-1] * (k - len(rest))


def near_tie_swap(sel_row: list, scores: np.ndarray, own: int) -> list:
    """The oracle's selection with its weakest chosen block replaced by the best
    unchosen eligible block (what a GPU could return on a near tie)."""
    kept = [b for b in sel_row if b >= 0 and b != own]
    others = [b for b in range(own) if b not in kept]
    if not kept or not others:
        return list(sel_row)
    weakest = min(kept, key=lambda b: (scores[b], -b))
    best = max(others, key=lambda b: (scores[b], -b))
    row = sorted([b for b in kept if b != weakest] + [best, own])
    return row + [-1] * (len(sel_row) - len(row))


def _decode_sel_variants(case, o, rng):
    sh = case.shape
    B, k = sh.block_size, sh.top_k
    rand = np.zeros_like(o["sel"])
    swap = np.zeros_like(o["sel"])
    for s, L in enumerate(case.lengths):
        own = (L - 1) // B
        for g in range(sh.num_kv_heads):
            rand[s, g] = random_selection(rng, own, k)
            swap[s, g] = near_tie_swap(o["sel"][s, g].tolist(), o["pooled"][s, g], own)
    return rand, swap


@pytest.mark.parametrize("shape,lengths,seed,kw", DECODE_CASES)
def test_attend_decode_given_selection(shape, lengths, seed, kw):
    case = make_decode_case(shape, lengths, seed, **kw)
    o = oracle.decode(case)
    np.testing.assert_array_equal(oracle.attend_decode(case, o["sel"]), o["out"])
    rng = np.random.default_rng(seed)
    for sel in _decode_sel_variants(case, o, rng):
        np.testing.assert_allclose(oracle.attend_decode(case, sel),
                                   bruteforce.attend_decode(case, sel), rtol=1e-12, atol=1e-12)


def _prefill_random_sel(case, rng):
    sh = case.shape
    sel = np.zeros((case.num_tiles, sh.num_kv_heads, sh.top_k), dtype=np.int32)
    for t in range(case.num_tiles):
        own = case.prior_len // sh.block_size + t
        for g in range(sh.num_kv_heads):
            sel[t, g] = random_selection(rng, own, sh.top_k)
    return sel


@pytest.mark.parametrize("shape,P,C,seed", PREFILL_CASES)
def test_attend_prefill_given_selection(shape, P, C, seed):
    case = make_prefill_case(shape, P, C, seed, shuffle_pages=True, poison_frac=0.2)
    o = oracle.prefill(case)
    np.testing.assert_array_equal(oracle.attend_prefill(case, o["sel"]), o["out"])
    rng = np.random.default_rng(seed)
    sel = _prefill_random_sel(case, rng)
    np.testing.assert_allclose(oracle.attend_prefill(case, sel),
                               bruteforce.attend_prefill(case, sel), rtol=1e-12, atol=1e-12)
    # listed tiles, out of order: only their rows are written, from their own rows of sel
    nt = case.num_tiles
    tiles = sorted({nt - 1, 0, nt // 2}, reverse=True)
    got = oracle.attend_prefill(case, sel, tiles=tiles)
    ref = bruteforce.attend_prefill(case, sel, tiles=tiles)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(got[ok], ref[ok], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape,lengths,seed,kw", DECODE_CASES)
def test_block_scores_decode(shape, lengths, seed, kw):
    case = make_decode_case(shape, lengths, seed, **kw)
    o = oracle.decode(case)
    for s, L in enumerate(case.lengths):
        own = (L - 1) // shape.block_size
        if own == 0:
            continue
        for g in range(shape.num_kv_heads):
            got = oracle.block_scores(case, g, range(own), seq=s)
            np.testing.assert_array_equal(got, o["pooled"][s, g, :own])
            np.testing.assert_array_equal(got, bruteforce.block_scores(case, g, range(own), seq=s))


@pytest.mark.parametrize("shape,P,C,seed", PREFILL_CASES)
def test_block_scores_prefill(shape, P, C, seed):
    case = make_prefill_case(shape, P, C, seed, shuffle_pages=True, poison_frac=0.2)
    o = oracle.prefill(case)
    for t in range(case.num_tiles):
        own = P // shape.block_size + t
        if own == 0:
            continue
        for g in range(shape.num_kv_heads):
            got = oracle.block_scores(case, g, range(own), tile=t)
            np.testing.assert_array_equal(got, o["pooled"][t, g, :own])
            np.testing.assert_array_equal(got, bruteforce.block_scores(case, g, range(own), tile=t))


def test_tile_rows_partial_tiles():
    """Tile query ranges against a direct count of which chunk positions fall in
    each absolute block."""
    for P, C, B in [(13, 22, 4), (16, 9, 4), (6, 1, 4), (0, 5, 4), (1000, 700, 128)]:
        case = make_prefill_case(Shape(num_q_heads=2, num_kv_heads=1, head_dim=8,
                                       num_idx_heads=1, idx_dim=4, block_size=B, top_k=2),
                                 P, C, 1)
        rows = [oracle.tile_rows(case, t) for t in range(case.num_tiles)]
        for t, (q0, q1) in enumerate(rows):
            want = [i for i in range(C) if (P + i) // B == P // B + t]
            assert list(range(q0, q1)) == want
