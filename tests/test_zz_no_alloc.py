"""msa_decode_noalloc (the kernels' scratch in the library's static device
array instead of a caller workspace) against msa_decode through the C ABI:
two calls in a row, the second with a smaller input, each identical to
msa_decode on a fresh workspace (same kernels, so bit for bit); outputs also
checked against the oracle.  A call needing more than the static scratch is
rejected with MSA_ERR_WORKSPACE.  Marked gpu."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import block_sparse_long_10_amd as msa
import oracle
from msa_inputs import GQA64, Shape, make_decode_case
from tests.gpu_util import check_out, check_selection, kv_of, params_of, run_decode

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(case):
    sh = case.shape
    out = torch.full((case.batch, sh.num_q_heads, sh.head_dim), float("nan"), device=DEV)
    sel = torch.full((case.batch, sh.num_kv_heads, sh.top_k), -7, dtype=torch.int32, device=DEV)
    msa.msa_decode_noalloc(params_of(sh), kv_of(case), case.q, case.idx_q, case.seq_lens,
                           case.batch, max(case.lengths), out, sel)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), sel.cpu().numpy()


def test_decode_noalloc_matches_decode_twice_shrinking():
    for lengths, seed, shape in [
            ([131072, 70001, 9999, 4097], 151, GQA64),                # larger first
            ([5000], 152, Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4,
                                block_size=64, top_k=8))]:            # then smaller
        print("\n[gpu noalloc] lengths %s" % lengths, flush=True)
        sys.stdout.flush()
        case = make_decode_case(shape, lengths, seed, device=DEV, shuffle_pages=True,
                                poison_frac=0.02)
        out, sel = _noalloc(case)
        ref = run_decode(case, with_pooled=False)
        np.testing.assert_array_equal(sel, ref["sel"])
        assert np.array_equal(out, ref["out"])
        P = oracle.prepare(case, kv_pages=[])
        oref = oracle.decode(case, prepared=P)
        B = shape.block_size
        bt = case.cache.block_table.cpu().numpy()
        pages = set()
        for s, L in enumerate(lengths):
            own = (L - 1) // B
            for g in range(shape.num_kv_heads):
                check_selection(sel[s, g], oref["pooled"][s, g], own, shape.top_k)
                pages.update(int(bt[s, b]) for b in sel[s, g] if b >= 0)
        P.fill_pages(case, pages)
        check_out(out, oracle.attend_decode(case, sel, prepared=P))


def test_decode_noalloc_replays_in_a_graph():
    """Captured in a HIP graph (the callers it is for), then replayed three
    times; between the replays, eager work and an eager msa_decode_noalloc
    on another input, which leaves its own contents in the shared scratch.
    Every replay equals the eager call bit for bit."""
    print("\n[gpu noalloc] graph capture and replays", flush=True)
    sys.stdout.flush()
    shape = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8)
    case = make_decode_case(shape, [9000, 777, 1, 4097], 154, device=DEV, shuffle_pages=True,
                            poison_frac=0.02)
    other = make_decode_case(GQA64, [70001, 3000], 155, device=DEV, shuffle_pages=True)
    ref_out, ref_sel = _noalloc(case)
    sh = case.shape
    out = torch.full((case.batch, sh.num_q_heads, sh.head_dim), float("nan"), device=DEV)
    sel = torch.full((case.batch, sh.num_kv_heads, sh.top_k), -7, dtype=torch.int32, device=DEV)
    p, kv = params_of(sh), kv_of(case)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            msa.msa_decode_noalloc(p, kv, case.q, case.idx_q, case.seq_lens, case.batch,
                                   max(case.lengths), out, sel)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        sel.fill_(-7)
        _noalloc(other)  # the scratch now holds another call's contents
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(sel.cpu().numpy(), ref_sel, err_msg="replay %d" % rep)
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref_out), "replay %d" % rep
        assert torch.isfinite(junk)


def test_decode_noalloc_rejects_beyond_the_static_scratch():
    sh = GQA64
    case = make_decode_case(sh, [300], 153, device=DEV)
    p = params_of(sh)
    c = case.cache
    # a block table that claims 200K blocks per sequence for 16 sequences:
    # pooled scores alone would take 16*8*200000*4 bytes > 32 MiB
    kv = msa.PagedKV(c.k.data_ptr(), c.v.data_ptr(), c.idx_k.data_ptr(),
                     c.block_table.data_ptr(), c.num_pages, 200000)
    st = msa.lib().msa_decode_noalloc(ctypes.byref(p), ctypes.byref(kv), case.q.data_ptr(),
                                      case.idx_q.data_ptr(), case.seq_lens.data_ptr(), 16, 300,
                                      case.q.data_ptr(), None, None)
    assert st == -3
    assert "static scratch" in msa.msa_last_error()
