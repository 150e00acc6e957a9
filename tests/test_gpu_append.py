"""GPU parity of the cache append and of the decode step with the append fused
in, through the C ABI.  Marked gpu.

* msa_cache_append into a cache whose slots for the new tokens were punched
  out must give back the generated cache bit for bit (and the oracle's append
  of the same rows into the same punched host copy gives the same bits).
* msa_decode_append on a punched cache must write the current tokens and give
  the same outputs and selections, bit for bit, as msa_decode on the cache
  that already holds them; the outputs are also checked against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_long_10_amd as msa
import oracle
from msa_inputs import GQA64, Shape, make_decode_case, make_prefill_case, make_workload
from tests.append_util import holed_copy, new_token_batch, same_bits
from tests.gpu_util import check_out, params_of, run_decode

pytestmark = pytest.mark.gpu

DEV = "cuda"
SMALL = [Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=4),
         Shape(num_q_heads=24, num_kv_heads=3, num_idx_heads=2, block_size=128, top_k=5)]


def _announce(what):
    print("\n[gpu append] " + what, flush=True)
    sys.stdout.flush()


def _append_and_compare(shape, full, starts, n_new):
    kn, vn, xn = new_token_batch(full, shape, starts, n_new)
    hole = holed_copy(full, shape, starts, n_new)
    host = [np.ascontiguousarray(t.cpu().view(torch.int16).numpy())
            for t in (hole.k, hole.v, hole.idx_k)]
    kv = msa.make_kv_mut(hole.k, hole.v, hole.idx_k, full.block_table)
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    msa.msa_cache_append(params_of(shape), kv, kn, vn, xn, st, len(starts), n_new)
    torch.cuda.synchronize()
    assert same_bits(hole.k, full.k) and same_bits(hole.v, full.v)
    assert same_bits(hole.idx_k, full.idx_k)
    oracle.cache_append(shape, *host, full.block_table, kn, vn, xn, starts)
    for a, t in zip(host, (hole.k, hole.v, hole.idx_k)):
        np.testing.assert_array_equal(a, t.cpu().view(torch.int16).numpy())


@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("n_new,tail", [(1, 0), (150, 0), (70, 37), (300, 3)])
def test_cache_append_small(shape, n_new, tail):
    lengths = [700, 420, 1000]
    _announce("cache append %s n_new=%d tail=%d" % (shape, n_new, tail))
    case = make_decode_case(shape, lengths, 31, device=DEV, shuffle_pages=True, poison_frac=0.05)
    starts = [L - n_new - tail for L in lengths]
    _append_and_compare(shape, case.cache, starts, n_new)


def test_cache_append_prefill_chunk_1M():
    """The 8192-token chunk of the 1M prefill workload, appended after 1,048,576 tokens."""
    _announce("cache append of the prefill_P1M_C8k chunk")
    case = make_workload("prefill_P1M_C8k", device=DEV)
    _append_and_compare(case.shape, case.cache, [case.prior_len], case.chunk_len)


def _decode_append_matches(case, check_oracle):
    sh = case.shape
    starts = [L - 1 for L in case.lengths]
    kn, vn, xn = new_token_batch(case.cache, sh, starts, 1)
    kn, vn, xn = kn[:, 0].contiguous(), vn[:, 0].contiguous(), xn[:, 0].contiguous()
    ref = run_decode(case, with_pooled=False)
    hole = holed_copy(case.cache, sh, starts, 1)
    p = params_of(sh)
    kv = msa.make_kv_mut(hole.k, hole.v, hole.idx_k, case.cache.block_table)
    batch, maxL, mb = case.batch, max(case.lengths), case.cache.max_blocks
    out = torch.full((batch, sh.num_q_heads, sh.head_dim), float("nan"), device=DEV)
    sel = torch.full((batch, sh.num_kv_heads, sh.top_k), -7, dtype=torch.int32, device=DEV)
    ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8, device=DEV)
    msa.msa_decode_append(p, kv, kn, vn, xn, case.q, case.idx_q, case.seq_lens, batch, maxL, out,
                          sel, ws)
    torch.cuda.synchronize()
    assert same_bits(hole.k, case.cache.k) and same_bits(hole.v, case.cache.v)
    assert same_bits(hole.idx_k, case.cache.idx_k)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref["sel"])
    np.testing.assert_array_equal(out.cpu().numpy().astype(np.float64), ref["out"])
    if check_oracle:
        check_out(ref["out"], oracle.attend_decode(case, ref["sel"]))


@pytest.mark.parametrize("shape", SMALL)
def test_decode_append_small(shape):
    _announce("decode append %s" % (shape,))
    lengths = [1, 64, 65, 700, 129, 1000, 128]
    case = make_decode_case(shape, lengths, 41, device=DEV, shuffle_pages=True, poison_frac=0.05)
    _decode_append_matches(case, check_oracle=True)


def test_decode_append_1M():
    """The decode_b1_L1M workload in the launch configuration of the benchmark."""
    _announce("decode append decode_b1_L1M")
    case = make_workload("decode_b1_L1M", device=DEV)
    _decode_append_matches(case, check_oracle=False)


def test_decode_append_paged_b32():
    _announce("decode append decode_paged_b32")
    case = make_workload("decode_paged_b32", device=DEV)
    _decode_append_matches(case, check_oracle=False)
