"""GPU parity of the batched variable-length prefill (several sequences'
chunks in one call, paged caches) against the oracle run sequence by
sequence, and bit-for-bit against one msa_prefill_chunk call per sequence.
Marked gpu."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_long_10_amd as msa
import oracle
from msa_inputs import GQA64, Shape, log_uniform_lengths, make_varlen_prefill_case
from tests.gpu_util import check_out, check_selection, kv_of, params_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(what):
    print("\n[gpu varlen] " + what, flush=True)
    sys.stdout.flush()


def run_varlen(case):
    sh = case.shape
    p = params_of(sh)
    kv = kv_of(case)
    mb = case.cache.max_blocks
    rows = sum(case.chunk_lens)
    tiles = sum(case.num_tiles_of(s) for s in range(case.batch))
    out = torch.full((rows, sh.num_q_heads, sh.head_dim), float("nan"), device=DEV)
    sel = torch.full((tiles, sh.num_kv_heads, sh.top_k), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(msa.msa_prefill_varlen_workspace_bytes(p, case.prior_lens, case.chunk_lens, mb),
                     dtype=torch.uint8, device=DEV)
    pd = torch.tensor(case.prior_lens, dtype=torch.int32, device=DEV)
    cd = torch.tensor(case.chunk_lens, dtype=torch.int32, device=DEV)
    msa.msa_prefill_varlen(p, kv, case.q, case.idx_q, pd, cd, case.prior_lens, case.chunk_lens,
                           out, sel, ws)
    torch.cuda.synchronize()
    return out, sel


def _tile_offsets(case):
    offs, acc = [], 0
    for s in range(case.batch):
        offs.append(acc)
        acc += case.num_tiles_of(s)
    return offs


@pytest.mark.parametrize("shape", [
    GQA64,
    Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8),
    Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=6, sink_blocks=1,
          local_blocks=2),
])
def test_varlen_prefill_small(shape):
    priors, chunks = [0, 1000, 4096, 130, 5000, 64], [300, 700, 512, 1, 200, 64]
    _announce("%s priors %s chunks %s" % (shape, priors, chunks))
    case = make_varlen_prefill_case(shape, priors, chunks, 301, device=DEV, shuffle_pages=True,
                                    poison_frac=0.05)
    out, sel = run_varlen(case)
    out, sel = out.cpu().numpy().astype(np.float64), sel.cpu().numpy()
    B = shape.block_size
    toff, qs = _tile_offsets(case), case.q_start
    for s in range(case.batch):
        one = case.sequence(s)
        P = oracle.prepare(one)
        ref = oracle.prefill(one, prepared=P)
        nt = one.num_tiles
        my_sel = sel[toff[s]:toff[s] + nt]
        for t in range(nt):
            own = one.prior_len // B + t
            for g in range(shape.num_kv_heads):
                check_selection(my_sel[t, g], ref["pooled"][t, g], own, shape.top_k,
                                sink=shape.sink_blocks, local=shape.local_blocks)
        check_out(out[qs[s]:qs[s] + one.chunk_len], oracle.attend_prefill(one, my_sel, prepared=P),
                  "sequence %d" % s)


@pytest.mark.timeout(600)
def test_varlen_prefill_paged_b32_equals_single_calls():
    """The 32 sequences of the paged decode workload (log-uniform lengths in
    [4096, 524288], shuffled pages) each prefilling its last 512 tokens: four
    sequences against the oracle, and all 32 bit for bit against one
    msa_prefill_chunk call per sequence."""
    lengths = log_uniform_lengths(32, 4096, 524288, 5)
    chunk = 512
    priors = [L - chunk for L in lengths]
    _announce("paged b32, 512-token chunks")
    case = make_varlen_prefill_case(GQA64, priors, [chunk] * 32, 5, device=DEV,
                                    shuffle_pages=True, poison_frac=0.01)
    out, sel = run_varlen(case)
    p = params_of(GQA64)
    toff, qs = _tile_offsets(case), case.q_start
    # four sequences against the oracle: the shortest, the longest and two
    # seeded others (pooled scores via the selection rule, and every output row)
    order = sorted(range(case.batch), key=lambda s: lengths[s])
    rng = np.random.default_rng(77)
    picked = sorted({order[0], order[-1]} |
                    set(rng.choice(order[1:-1], size=2, replace=False).tolist()))
    sel_h, out_h = sel.cpu().numpy(), out.cpu().numpy().astype(np.float64)
    B = GQA64.block_size
    for s in picked:
        one = case.sequence(s)
        P = oracle.prepare(one, kv_pages=[])
        ref = oracle.prefill(one, prepared=P)
        nt = one.num_tiles
        my_sel = sel_h[toff[s]:toff[s] + nt]
        bt = one.cache.block_table.cpu().numpy()
        for t in range(nt):
            own = one.prior_len // B + t
            for gi in range(GQA64.num_kv_heads):
                check_selection(my_sel[t, gi], ref["pooled"][t, gi], own, GQA64.top_k)
        P.fill_pages(one, {int(bt[0, b]) for b in my_sel.reshape(-1) if b >= 0})
        worst = check_out(out_h[qs[s]:qs[s] + chunk],
                          oracle.attend_prefill(one, my_sel, prepared=P), "sequence %d" % s)
        print("sequence %d (L=%d) against the oracle: worst row err %.3g" % (s, lengths[s], worst),
              flush=True)
    for s in range(case.batch):
        one = case.sequence(s)
        kv = msa.make_kv(one.cache.k, one.cache.v, one.cache.idx_k, one.cache.block_table)
        o1 = torch.full((chunk, GQA64.num_q_heads, GQA64.head_dim), float("nan"), device=DEV)
        s1 = torch.full((one.num_tiles, GQA64.num_kv_heads, GQA64.top_k), -7, dtype=torch.int32,
                        device=DEV)
        ws = torch.empty(msa.msa_prefill_workspace_bytes(p, one.prior_len, chunk,
                                                         one.cache.max_blocks),
                         dtype=torch.uint8, device=DEV)
        msa.msa_prefill_chunk(p, kv, one.q, one.idx_q, one.prior_len, chunk, o1, s1, ws)
        torch.cuda.synchronize()
        assert torch.equal(sel[toff[s]:toff[s] + one.num_tiles], s1), "sequence %d" % s
        assert torch.equal(out[qs[s]:qs[s] + chunk], o1), "sequence %d" % s
