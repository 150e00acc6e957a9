"""GPU parity of per-group index keys (one index-key head per KV group, the
ablation of the single shared head) against the oracle, through the C ABI:
decode (small and 1M), prefill, batched prefill and the appends.  Marked gpu."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_long_10_amd as msa
import oracle
from msa_inputs import GQA64, Shape, make_prefill_case, make_varlen_prefill_case, make_workload
from tests.append_util import holed_copy, new_token_batch, same_bits
from tests.gpu_util import check_out, check_pooled, check_selection, params_of, run_prefill
from tests.test_gpu_forced import _check_decode
from msa_inputs import make_decode_case

pytestmark = pytest.mark.gpu

DEV = "cuda"
SMALL = [Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=4,
               idx_k_heads=2),
         Shape(num_q_heads=24, num_kv_heads=3, num_idx_heads=2, block_size=128, top_k=5,
               idx_k_heads=3),
         Shape(num_q_heads=64, num_kv_heads=8, num_idx_heads=8, block_size=64, top_k=6,
               idx_k_heads=8, sink_blocks=1, local_blocks=1)]


def _announce(what):
    print("\n[gpu group keys] " + what, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("shape", SMALL)
def test_decode_group_keys_small(shape):
    _announce("decode %s" % (shape,))
    case = make_decode_case(shape, [1, 64, 65, 700, 1000, 129], 121, device=DEV,
                            shuffle_pages=True, poison_frac=0.05)
    worst, kinds = _check_decode(case)
    print("worst row err %.3g, %s" % (worst, {x: kinds.count(x) for x in set(kinds)}))


def test_decode_group_keys_1M():
    _announce("decode_b1_L1M with 8 index-key heads")
    w = make_workload("decode_b1_L1M", device=DEV)
    sh = Shape(num_q_heads=64, num_kv_heads=8, idx_k_heads=8)
    case = make_decode_case(sh, w.lengths, 3, device=DEV)
    worst, kinds = _check_decode(case, full=False)
    print("worst row err %.3g" % worst)


@pytest.mark.parametrize("shape", SMALL[:2])
def test_prefill_group_keys(shape):
    _announce("prefill %s" % (shape,))
    case = make_prefill_case(shape, 3000, 333, 122, device=DEV, shuffle_pages=True,
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
            check_selection(g["sel"][t, gi], ref["pooled"][t, gi], own, shape.top_k)
    check_out(g["out"], oracle.attend_prefill(case, g["sel"], prepared=P))


def test_varlen_group_keys():
    shape = SMALL[0]
    _announce("batched prefill %s" % (shape,))
    from tests.test_gpu_varlen import run_varlen, _tile_offsets
    case = make_varlen_prefill_case(shape, [0, 1000, 130], [300, 700, 1], 123, device=DEV,
                                    shuffle_pages=True)
    out, sel = run_varlen(case)
    out, sel = out.cpu().numpy().astype(np.float64), sel.cpu().numpy()
    toff, qs = _tile_offsets(case), case.q_start
    for s in range(case.batch):
        one = case.sequence(s)
        P = oracle.prepare(one)
        ref = oracle.prefill(one, prepared=P)
        my = sel[toff[s]:toff[s] + one.num_tiles]
        for t in range(one.num_tiles):
            own = one.prior_len // shape.block_size + t
            for g in range(shape.num_kv_heads):
                check_selection(my[t, g], ref["pooled"][t, g], own, shape.top_k)
        check_out(out[qs[s]:qs[s] + one.chunk_len], oracle.attend_prefill(one, my, prepared=P))


def test_appends_group_keys():
    shape = SMALL[1]
    _announce("appends %s" % (shape,))
    lengths = [700, 420, 1000]
    case = make_decode_case(shape, lengths, 124, device=DEV, shuffle_pages=True)
    full = case.cache
    starts = [L - 150 for L in lengths]
    kn, vn, xn = new_token_batch(full, shape, starts, 150)
    hole = holed_copy(full, shape, starts, 150)
    kv = msa.make_kv_mut(hole.k, hole.v, hole.idx_k, full.block_table)
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    msa.msa_cache_append(params_of(shape), kv, kn, vn, xn, st, len(starts), 150)
    torch.cuda.synchronize()
    assert same_bits(hole.k, full.k) and same_bits(hole.v, full.v)
    assert same_bits(hole.idx_k, full.idx_k)
    from tests.test_gpu_append import _decode_append_matches
    _decode_append_matches(case, check_oracle=True)
