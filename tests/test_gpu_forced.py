"""GPU parity of the forced sink and local-window blocks (decode and prefill)
against the oracle, through the C ABI.  Marked gpu."""
import sys

import numpy as np
import pytest

import oracle
from msa_inputs import GQA64, Shape, make_decode_case, make_prefill_case, make_workload
from tests.gpu_util import check_out, check_pooled, check_selection, run_decode, run_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(what):
    print("\n[gpu forced] " + what, flush=True)
    sys.stdout.flush()


def _check_decode(case, full=True):
    g = run_decode(case)
    sh = case.shape
    P = oracle.prepare(case, kv_pages=None if full else [])
    ref = oracle.decode(case, prepared=P)
    bt = case.cache.block_table.cpu().numpy()
    pages = set()
    kinds = []
    for s, L in enumerate(case.lengths):
        own = (L - 1) // sh.block_size
        for gi in range(sh.num_kv_heads):
            check_pooled(g["pooled"][s, gi, :own], ref["pooled"][s, gi, :own])
            kinds.append(check_selection(g["sel"][s, gi], ref["pooled"][s, gi], own, sh.top_k,
                                         sink=sh.sink_blocks, local=sh.local_blocks))
            pages.update(int(bt[s, b]) for b in g["sel"][s, gi] if b >= 0)
    if not full:
        P.fill_pages(case, pages)
    worst = check_out(g["out"], oracle.attend_decode(case, g["sel"], prepared=P))
    return worst, kinds


@pytest.mark.parametrize("sink,local,k", [(1, 0, 4), (0, 2, 4), (1, 2, 5), (2, 1, 4), (1, 3, 5)])
def test_decode_forced_small(sink, local, k):
    shape = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=k,
                  sink_blocks=sink, local_blocks=local)
    _announce("decode sink=%d local=%d k=%d" % (sink, local, k))
    case = make_decode_case(shape, [1, 64, 65, 200, 700, 1000, 129], 91, device=DEV,
                            shuffle_pages=True, poison_frac=0.05)
    worst, kinds = _check_decode(case)
    print("worst row err %.3g, %s" % (worst, {x: kinds.count(x) for x in set(kinds)}))


def test_decode_forced_1M():
    """decode_b1_L1M with one sink block and two local blocks (13 chosen by TopK)."""
    _announce("decode_b1_L1M sink=1 local=2")
    w = make_workload("decode_b1_L1M", device=DEV)
    w.shape = Shape(num_q_heads=64, num_kv_heads=8, sink_blocks=1, local_blocks=2)
    worst, kinds = _check_decode(w, full=False)
    print("worst row err %.3g, %s" % (worst, {x: kinds.count(x) for x in set(kinds)}))


def test_decode_forced_large_batch_separate_topk():
    """Enough (sequence, group, slot) workgroups that TopK runs in its own launch."""
    shape = Shape(num_q_heads=64, num_kv_heads=8, top_k=16, sink_blocks=2, local_blocks=1)
    _announce("decode batch 10 x 8 groups x 16 slots, sink=2 local=1")
    case = make_decode_case(shape, [3000 + 977 * i for i in range(10)], 92, device=DEV,
                            shuffle_pages=True)
    worst, kinds = _check_decode(case, full=False)
    print("worst row err %.3g" % worst)


@pytest.mark.parametrize("sink,local", [(1, 1), (0, 3), (2, 0)])
def test_prefill_forced(sink, local):
    shape = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=6,
                  sink_blocks=sink, local_blocks=local)
    _announce("prefill sink=%d local=%d" % (sink, local))
    case = make_prefill_case(shape, 3000, 333, 93, device=DEV, shuffle_pages=True,
                             poison_frac=0.05)
    g = run_prefill(case)
    np.testing.assert_array_equal(g["sel"], g["sel_steps"])
    P = oracle.prepare(case)
    ref = oracle.prefill(case, prepared=P)
    B = shape.block_size
    for t in range(case.num_tiles):
        own = case.prior_len // B + t
        for gi in range(shape.num_kv_heads):
            check_pooled(g["pooled"][t, gi, :own], ref["pooled"][t, gi, :own])
            check_selection(g["sel"][t, gi], ref["pooled"][t, gi], own, shape.top_k,
                            sink=sink, local=local)
    check_out(g["out"], oracle.attend_prefill(case, g["sel"], prepared=P))
