"""GPU parity of MSA decode (index score + pooling, TopK, sparse attention)
against the oracle, through the C ABI.  Marked gpu."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_long_10_amd as msa
import oracle
from msa_inputs import Shape, GQA64, make_decode_case, make_workload
from tests.gpu_util import (check_out, check_pooled, check_selection, params_of, run_decode)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(what):
    print("\n[gpu decode] " + what, flush=True)
    sys.stdout.flush()


def _full_check(case, exact_sel=False):
    """Oracle on the whole cache (small cases)."""
    g = run_decode(case)
    P = oracle.prepare(case)
    ref = oracle.decode(case, prepared=P)
    sh = case.shape
    kinds = []
    for s, L in enumerate(case.lengths):
        own = (L - 1) // sh.block_size
        for gi in range(sh.num_kv_heads):
            check_pooled(g["pooled"][s, gi, :own], ref["pooled"][s, gi, :own], "s%d g%d" % (s, gi))
            kinds.append(check_selection(g["sel"][s, gi], ref["pooled"][s, gi], own, sh.top_k,
                                         exact_only=exact_sel))
    ref_out = oracle.attend_decode(case, g["sel"], prepared=P)
    worst = check_out(g["out"], ref_out)
    return g, ref, worst, kinds


def _big_check(case):
    """Oracle with only the needed K/V pages on the host (long contexts)."""
    g = run_decode(case)
    P = oracle.prepare(case, kv_pages=[])
    ref = oracle.decode(case, prepared=P)        # scores + selection (K/V unused here)
    sh = case.shape
    bt = case.cache.block_table.cpu().numpy()
    kinds, pages = [], set()
    for s, L in enumerate(case.lengths):
        own = (L - 1) // sh.block_size
        for gi in range(sh.num_kv_heads):
            check_pooled(g["pooled"][s, gi, :own], ref["pooled"][s, gi, :own], "s%d g%d" % (s, gi))
            kinds.append(check_selection(g["sel"][s, gi], ref["pooled"][s, gi], own, sh.top_k))
            pages.update(int(bt[s, b]) for b in g["sel"][s, gi] if b >= 0)
    P.fill_pages(case, pages)
    ref_out = oracle.attend_decode(case, g["sel"], prepared=P)
    worst = check_out(g["out"], ref_out)
    return g, worst, kinds


SMALL = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8)


@pytest.mark.parametrize("lengths,seed", [
    ([1, 63, 64, 65, 1000, 4097, 130, 448, 449], 101),
    ([5000, 12345, 777], 102),
])
def test_decode_small_ragged(lengths, seed):
    _announce("small ragged %s" % lengths)
    case = make_decode_case(SMALL, lengths, seed, device=DEV, shuffle_pages=True, poison_frac=0.05)
    _, _, worst, kinds = _full_check(case)
    print("worst row err %.3g, selections %s" % (worst, {k: kinds.count(k) for k in set(kinds)}))


def _log_uniform_lengths(n, lo, hi, seed, fixed):
    rng = np.random.default_rng(seed)
    drawn = np.exp(rng.uniform(np.log(lo), np.log(hi), n - len(fixed))).astype(int)
    return list(fixed) + [int(x) for x in drawn]


# Batches of 2..64 sequences whose full (block, sequence) grid exceeds 10240
# workgroups take the compact index kernel (a walk over the real blocks found
# from a scan of the lengths): 48 x 255 and 64 x 187 blocks here, with empty
# and one-block sequences among them.
@pytest.mark.parametrize("shape,n,hi,fixed,seed", [
    (SMALL, 48, 16384, [1, 64, 65, 16384, 2], 104),
    (Shape(num_q_heads=32, num_kv_heads=8, num_idx_heads=4, block_size=64, top_k=8), 64, 12000,
     [12000, 1, 128, 129], 105),
])
def test_decode_compact_grid(shape, n, hi, fixed, seed):
    lengths = _log_uniform_lengths(n, 1, hi, seed, fixed)
    _announce("compact grid: %d sequences up to %d tokens" % (n, max(lengths)))
    case = make_decode_case(shape, lengths, seed, device=DEV, shuffle_pages=True, poison_frac=0.05)
    _, _, worst, kinds = _full_check(case)
    print("worst row err %.3g, selections %s" % (worst, {k: kinds.count(k) for k in set(kinds)}))


@pytest.mark.parametrize("shape", [
    Shape(num_q_heads=8, num_kv_heads=8, num_idx_heads=1, block_size=128, top_k=16),
    Shape(num_q_heads=12, num_kv_heads=4, num_idx_heads=2, block_size=128, top_k=5),
    Shape(num_q_heads=64, num_kv_heads=4, num_idx_heads=8, block_size=64, top_k=64),
    Shape(num_q_heads=16, num_kv_heads=4, num_idx_heads=16, block_size=128, top_k=1),
    Shape(num_q_heads=3, num_kv_heads=3, num_idx_heads=4, block_size=64, top_k=2),
    Shape(num_q_heads=48, num_kv_heads=16, num_idx_heads=4, block_size=128, top_k=9),
])
def test_decode_shape_variants(shape):
    _announce("shape %s" % (shape,))
    case = make_decode_case(shape, [9000, 257, 128, 3333], 103, device=DEV, shuffle_pages=True)
    _, _, worst, _ = _full_check(case)
    print("worst row err %.3g" % worst)



# The selection's register tiers switch on the longest row of the batch
# (max_seq_len): the fused TopK keeps 4 scores per thread up to 1024 ranked
# blocks and 32 above; the separate TopK launch (more than 1024 slot
# workgroups) keeps 16 up to 4096 blocks and 32 above; past 8192 blocks
# both re-read the scores from memory (the general path).  Each edge from
# both sides, beside short rows of the same batch.
EDGE_FUSED = Shape(num_q_heads=8, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8)
EDGE_SPLIT = Shape(num_q_heads=8, num_kv_heads=2, num_idx_heads=2, block_size=64, top_k=64)


@pytest.mark.parametrize("shape,own,others,seed", [
    (EDGE_FUSED, 1024, [3000, 1], 111),
    (EDGE_FUSED, 1025, [3000, 65], 112),
    (EDGE_SPLIT, 4096, [1, 64, 65, 5000, 30000, 65600, 9000, 129], 113),
    (EDGE_SPLIT, 4097, [1, 64, 65, 5000, 30000, 65600, 9000, 129], 114),
    (EDGE_FUSED, 8192, [3000, 1], 115),
    (EDGE_FUSED, 8193, [3000, 65], 116),
    (EDGE_SPLIT, 8193, [1, 64, 65, 5000, 30000, 65600, 9000, 129], 117),
])
def test_decode_selection_tier_edges(shape, own, others, seed):
    lengths = [own * shape.block_size + 1] + others
    _announce("selection tier edge: %d ranked blocks, %d slot workgroups"
              % (own, len(lengths) * shape.num_kv_heads * shape.top_k))
    case = make_decode_case(shape, lengths, seed, device=DEV, shuffle_pages=True, poison_frac=0.02)
    g, worst, kinds = _big_check(case)
    print("worst row err %.3g, selections %s" % (worst, {k: kinds.count(k) for k in set(kinds)}))

def test_decode_workload_b1_L4k():
    _announce("decode_b1_L4k")
    case = make_workload("decode_b1_L4k", DEV)
    _, _, worst, kinds = _full_check(case)
    print("worst row err %.3g, selections %s" % (worst, kinds))


@pytest.mark.parametrize("name", ["decode_b8_L128k", "decode_b1_L1M", "decode_paged_b32"])
def test_decode_workload_full_size(name):
    _announce(name)
    case = make_workload(name, DEV)
    g, worst, kinds = _big_check(case)
    print("worst row err %.3g, selections %s" % (worst, {k: kinds.count(k) for k in set(kinds)}))
    if case.shifted:
        # shifted blocks are kept far more often than chance (k-1 of ~own)
        hit = sum(len(set(v) & set(g["sel"][s, gi].tolist()))
                  for (s, gi), v in case.shifted.items())
        tot = sum(len(v) for v in case.shifted.values())
        own = (case.lengths[0] - 1) // case.shape.block_size
        chance = (case.shape.top_k - 1) / own
        print("shifted blocks kept: %d of %d (chance %.3f)" % (hit, tot, chance))
        assert hit >= 10 * chance * tot


def test_decode_constructed_exact_ties():
    _announce("exact ties")
    case = make_decode_case(SMALL, [3000, 2000], 104, device=DEV)
    ik = case.cache.idx_k
    bt = case.cache.block_table
    # make blocks 3, 9, 20, 31 bit-identical and the clear best of sequence 0;
    # blocks 5 and 6 identical in sequence 1
    src = int(bt[0, 3])
    ik[src] = (ik[src].float() * 0.5 + 1.5).to(torch.bfloat16)
    for b in (9, 20, 31):
        ik[int(bt[0, b])] = ik[src]
    ik[int(bt[1, 6])] = ik[int(bt[1, 5])]
    case.idx_q[:] = case.idx_q.abs()
    g, ref, _, _ = _full_check(case, exact_sel=True)
    for gi in range(SMALL.num_kv_heads):
        row = g["sel"][0, gi].tolist()
        assert {3, 9, 20, 31} <= set(row)
    np.testing.assert_array_equal(g["sel"], ref["sel"])


@pytest.mark.parametrize("extra", [1, 2, 4, 6])
def test_decode_ties_across_the_cut(extra):
    """keep + extra blocks with bit-identical index keys are the clear best of
    each sequence: only keep of them fit, so the cut falls inside the tie and
    the lowest block indices must win (reading: score descending, then block
    index ascending).  extra <= 4 is settled by dropping the worst candidates
    one at a time, 6 by sorting them; both against the oracle bit for bit."""
    _announce("ties across the cut, %d extra" % extra)
    keep = SMALL.top_k - 1
    case = make_decode_case(SMALL, [5000, 2300], 110 + extra, device=DEV)
    ik = case.cache.idx_k
    bt = case.cache.block_table
    rng = np.random.default_rng(extra)
    for s, L in enumerate(case.lengths):
        own = (L - 1) // SMALL.block_size
        tied = sorted(rng.choice(own, size=keep + extra, replace=False).tolist())
        src = int(bt[s, tied[0]])
        ik[src] = (ik[src].float() * 0.5 + 1.5).to(torch.bfloat16)
        for b in tied[1:]:
            ik[int(bt[s, b])] = ik[src]
    case.idx_q[:] = case.idx_q.abs()
    g, ref, _, _ = _full_check(case, exact_sel=True)
    for s, L in enumerate(case.lengths):
        own = (L - 1) // SMALL.block_size
        for gi in range(SMALL.num_kv_heads):
            assert g["sel"][s, gi].tolist()[-1] == own
    np.testing.assert_array_equal(g["sel"], ref["sel"])


def test_decode_tie_fallback_paths():
    _announce("all-equal and heavily tied scores")
    # every pooled score equal: the lowest indices win
    case = make_decode_case(SMALL, [6000, 3001], 105, device=DEV)
    case.cache.idx_k.zero_()
    g, ref, _, _ = _full_check(case, exact_sel=True)
    for s, L in enumerate(case.lengths):
        own = (L - 1) // SMALL.block_size
        assert g["sel"][s, 0].tolist() == list(range(SMALL.top_k - 1)) + [own]
    # few distinct values, hundreds of blocks per value: histogram refinement
    case = make_decode_case(SMALL, [40000, 20000], 106, device=DEV)
    q = case.cache.idx_k.float()
    case.cache.idx_k.copy_((torch.round(q * 2) / 2).clamp(-1, 1).to(torch.bfloat16))
    case.idx_q.fill_(0.25)
    _full_check(case, exact_sel=True)


def test_decode_deterministic():
    _announce("determinism")
    case = make_decode_case(GQA64, [70000, 9999, 131072], 107, device=DEV, shuffle_pages=True)
    a = run_decode(case, with_pooled=False)
    b = run_decode(case, with_pooled=False)
    np.testing.assert_array_equal(a["sel"], b["sel"])
    assert np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_decode_workspace_contents_do_not_change_results(fill):
    """The workspace's contents on entry do not matter: zero bytes, 0xFF bytes
    and random bytes give the same selection and bit-identical outputs, on two
    calls in a row.  Covers the fused TopK (batch 2) and the separate TopK
    launch (batch 9: more than 1024 slot workgroups)."""
    _announce("workspace contents: %s" % fill)
    for lengths, seed in [([70000, 131072], 108), ([9000 + 4000 * i for i in range(9)], 109)]:
        case = make_decode_case(GQA64, lengths, seed, device=DEV, shuffle_pages=True)
        ref = run_decode(case, with_pooled=False)
        p = params_of(GQA64)
        ws = torch.empty(msa.msa_decode_workspace_bytes(p, case.batch, case.cache.max_blocks),
                         dtype=torch.uint8, device=DEV)
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(255)
        else:
            ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=DEV))
        for rep in range(2):
            got = run_decode(case, with_pooled=False, ws=ws)
            np.testing.assert_array_equal(got["sel"], ref["sel"])
            assert np.array_equal(got["out"], ref["out"]), (fill, rep)
