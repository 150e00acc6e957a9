"""GPU parity of MSA chunked prefill (index score + pooling per tile, TopK per
tile, sparse attention with the causal diagonal block) against the oracle,
through the C ABI.  Marked gpu."""
import sys

import numpy as np
import pytest
import torch

import oracle
from msa_inputs import Shape, GQA64, make_prefill_case, make_workload
from tests.gpu_util import check_out, check_pooled, check_selection, run_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(what):
    print("\n[gpu prefill] " + what, flush=True)
    sys.stdout.flush()


def _full_check(case):
    g = run_prefill(case)
    np.testing.assert_array_equal(g["sel"], g["sel_steps"])
    P = oracle.prepare(case)
    ref = oracle.prefill(case, prepared=P)
    sh = case.shape
    B = sh.block_size
    kinds = []
    for t in range(case.num_tiles):
        own = case.prior_len // B + t
        for gi in range(sh.num_kv_heads):
            check_pooled(g["pooled"][t, gi, :own], ref["pooled"][t, gi, :own], "t%d g%d" % (t, gi))
            kinds.append(check_selection(g["sel"][t, gi], ref["pooled"][t, gi], own, sh.top_k))
    ref_out = oracle.attend_prefill(case, g["sel"], prepared=P)
    worst = check_out(g["out"], ref_out)
    return worst, kinds


@pytest.mark.parametrize("shape,P,C,seed", [
    (GQA64, 0, 300, 201),                   # first chunk, ragged last tile
    (GQA64, 1000, 700, 202),                # unaligned prior: partial first tile
    (GQA64, 4096, 512, 203),                # aligned
    (Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8),
     3000, 333, 204),
    (Shape(num_q_heads=8, num_kv_heads=4, num_idx_heads=2, block_size=128, top_k=3),
     2500, 1, 205),                         # one-token chunk
    (Shape(num_q_heads=32, num_kv_heads=2, num_idx_heads=8, block_size=64, top_k=12),
     5000, 200, 206),
])
def test_prefill_small(shape, P, C, seed):
    _announce("P=%d C=%d %s" % (P, C, shape))
    case = make_prefill_case(shape, P, C, seed, device=DEV, shuffle_pages=True, poison_frac=0.05)
    worst, kinds = _full_check(case)
    print("worst row err %.3g, selections %s" % (worst, {k: kinds.count(k) for k in set(kinds)}))


def test_prefill_mid_size_several_tiles():
    _announce("P=8000 C=1100")
    case = make_prefill_case(GQA64, 8000, 1100, 207, device=DEV, shuffle_pages=True)
    worst, kinds = _full_check(case)
    print("worst row err %.3g, selections %s" % (worst, {k: kinds.count(k) for k in set(kinds)}))


@pytest.mark.timeout(600)
def test_prefill_workload_full_size_sampled():
    """prefill_P1M_C8k in the benchmark's launch configuration (33 key ranges
    of at most 256 blocks per (tile, group)), checked against the oracle on
    eight whole tiles -- the first two, the last two and four seeded ones --
    in all eight groups: every pooled score of every eligible block, every
    selection (against the oracle's own scores), and the output of every query
    of those tiles over the kept blocks."""
    _announce("prefill_P1M_C8k (8 whole tiles)")
    case = make_workload("prefill_P1M_C8k", DEV)
    g = run_prefill(case)
    np.testing.assert_array_equal(g["sel"], g["sel_steps"])
    sh = case.shape
    B, k = sh.block_size, sh.top_k
    nt = case.num_tiles
    rng = np.random.default_rng(44)
    middle = sorted(rng.choice(np.arange(2, nt - 2), size=4, replace=False).tolist())
    tiles = [0, 1] + middle + [nt - 2, nt - 1]
    P = oracle.prepare(case, kv_pages=[])
    # pooled scores and selections of the listed tiles (its outputs, computed
    # on zeroed K/V pages, are not used)
    ref = oracle.prefill(case, tiles=tiles, prepared=P)
    print("oracle scored tiles %s" % tiles, flush=True)
    bt = case.cache.block_table.cpu().numpy()
    pages = set()
    kinds = []
    for t in tiles:
        own = case.prior_len // B + t
        for gi in range(sh.num_kv_heads):
            check_pooled(g["pooled"][t, gi, :own], ref["pooled"][t, gi, :own],
                         "tile %d group %d" % (t, gi))
            kinds.append(check_selection(g["sel"][t, gi], ref["pooled"][t, gi], own, k))
            pages.update(int(bt[0, b]) for b in g["sel"][t, gi] if b >= 0)
    P.fill_pages(case, pages)
    ref_out = oracle.attend_prefill(case, g["sel"], tiles=tiles, prepared=P)
    rows = np.concatenate([np.arange(*oracle.tile_rows(case, t)) for t in tiles])
    worst = check_out(g["out"][rows], ref_out[rows])
    print("worst row err %.3g over %d queries, selections %s" % (
        worst, len(rows), {kk: kinds.count(kk) for kk in set(kinds)}))
