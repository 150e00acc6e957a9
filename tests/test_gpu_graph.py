"""MSA calls captured in one HIP graph (through torch's graph capture of the
C ABI calls on the capture stream) and replayed: several decode layers, and a
chunked plus a batched prefill.  The eager decode layers are checked against
the oracle layer by layer; every replay, with eager work and synchronisations
between the replays, must give the eager outputs bit for bit.  Marked gpu."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_long_10_amd as msa
import oracle
from msa_inputs import (TENSOR_IDS, DecodeCase, PagedCache, Shape, make_decode_case,
                        make_prefill_case, make_varlen_prefill_case, normal_bf16)
from tests.gpu_util import check_out, check_selection, params_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("append", [False, True])
def test_multi_layer_decode_graph_replays(append):
    print("\n[gpu graph] 4-layer decode graph, append=%s" % append, flush=True)
    sys.stdout.flush()
    shape = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=4)
    lengths = [900, 65, 1500]
    case = make_decode_case(shape, lengths, 51, device="cuda", shuffle_pages=True,
                            poison_frac=0.05)
    c, p = case.cache, params_of(shape)
    n_layers, batch, maxL, mb = 4, case.batch, max(lengths), c.max_blocks
    layers = []
    for l in range(n_layers):
        ik = normal_bf16(tuple(c.idx_k.shape), 600 + l, TENSOR_IDS["idx_k"], "cuda")
        q = normal_bf16(tuple(case.q.shape), 600 + l, TENSOR_IDS["q"], "cuda")
        iq = normal_bf16(tuple(case.idx_q.shape), 600 + l, TENSOR_IDS["idx_q"], "cuda")
        layers.append((ik, q, iq))
    pos = torch.tensor([L - 1 for L in lengths], dtype=torch.long, device="cuda")
    rows = torch.arange(batch, device="cuda")
    pages = c.block_table.long()[rows, pos // 64]
    slots = pos % 64
    kn = c.k[pages, :, slots, :].contiguous()
    vn = c.v[pages, :, slots, :].contiguous()
    outs = torch.empty(n_layers, batch, shape.num_q_heads, shape.head_dim, device="cuda")
    sels = torch.empty(n_layers, batch, shape.num_kv_heads, shape.top_k, dtype=torch.int32,
                       device="cuda")
    ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
                     device="cuda")

    def token():
        for l, (ik, q, iq) in enumerate(layers):
            if append:
                kv = msa.make_kv_mut(c.k, c.v, ik, c.block_table)
                xn = ik[pages, slots, :].contiguous()
                msa.msa_decode_append(p, kv, kn, vn, xn, q, iq, case.seq_lens, batch, maxL,
                                      outs[l], sels[l], ws)
            else:
                kv = msa.make_kv(c.k, c.v, ik, c.block_table)
                msa.msa_decode(p, kv, q, iq, case.seq_lens, batch, maxL, outs[l], sels[l], ws)

    token()
    torch.cuda.synchronize()
    ref_out, ref_sel = outs.clone(), sels.clone()
    assert torch.isfinite(ref_out).all()
    # every layer of the eager run against the oracle on that layer's index
    # keys and queries (the replays below must then equal it bit for bit)
    for l, (ik, q, iq) in enumerate(layers):
        one = DecodeCase(shape, PagedCache(k=c.k, v=c.v, idx_k=ik, block_table=c.block_table,
                                           num_pages=c.num_pages, max_blocks=c.max_blocks,
                                           lengths=list(lengths)),
                         q, iq, case.seq_lens, list(lengths))
        P = oracle.prepare(one)
        ref = oracle.decode(one, prepared=P)
        gsel = ref_sel[l].cpu().numpy()
        for sq, L in enumerate(lengths):
            own = (L - 1) // shape.block_size
            for gi in range(shape.num_kv_heads):
                check_selection(gsel[sq, gi], ref["pooled"][sq, gi], own, shape.top_k)
        check_out(ref_out[l].cpu().numpy().astype(np.float64),
                  oracle.attend_decode(one, gsel, prepared=P), "layer %d" % l)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            token()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        outs.fill_(float("nan"))
        sels.fill_(-9)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref_out), "replay %d" % rep
        assert torch.equal(sels, ref_sel), "replay %d" % rep
        assert torch.isfinite(junk)


def test_prefill_graph_replays():
    """A chunked prefill of one sequence and a batched prefill of four,
    captured in one HIP graph and replayed three times with eager work and
    synchronisations in between: every replay equals the eager run bit for
    bit (the batched call's tile map is rebuilt on the device in each replay)."""
    print("\n[gpu graph] prefill chunk + batched prefill graph", flush=True)
    sys.stdout.flush()
    shape = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=6)
    p = params_of(shape)
    one = make_prefill_case(shape, 3000, 333, 71, device="cuda", shuffle_pages=True,
                            poison_frac=0.05)
    kv1 = msa.make_kv(one.cache.k, one.cache.v, one.cache.idx_k, one.cache.block_table)
    out1 = torch.empty(one.chunk_len, shape.num_q_heads, shape.head_dim, device="cuda")
    sel1 = torch.empty(one.num_tiles, shape.num_kv_heads, shape.top_k, dtype=torch.int32,
                       device="cuda")
    ws1 = torch.empty(msa.msa_prefill_workspace_bytes(p, one.prior_len, one.chunk_len,
                                                      one.cache.max_blocks),
                      dtype=torch.uint8, device="cuda")
    priors, chunks = [0, 1000, 130, 5000], [300, 700, 1, 200]
    var = make_varlen_prefill_case(shape, priors, chunks, 72, device="cuda", shuffle_pages=True)
    kvv = msa.make_kv(var.cache.k, var.cache.v, var.cache.idx_k, var.cache.block_table)
    pl = torch.tensor(priors, dtype=torch.int32, device="cuda")
    cl = torch.tensor(chunks, dtype=torch.int32, device="cuda")
    tiles = sum((pr + c + 63) // 64 - pr // 64 for pr, c in zip(priors, chunks))
    outv = torch.empty(sum(chunks), shape.num_q_heads, shape.head_dim, device="cuda")
    selv = torch.empty(tiles, shape.num_kv_heads, shape.top_k, dtype=torch.int32, device="cuda")
    wsv = torch.empty(msa.msa_prefill_varlen_workspace_bytes(p, priors, chunks,
                                                            var.cache.max_blocks),
                      dtype=torch.uint8, device="cuda")

    def step():
        msa.msa_prefill_chunk(p, kv1, one.q, one.idx_q, one.prior_len, one.chunk_len, out1,
                              sel1, ws1)
        msa.msa_prefill_varlen(p, kvv, var.q, var.idx_q, pl, cl, priors, chunks, outv, selv,
                               wsv)

    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in (out1, sel1, outv, selv)]
    assert torch.isfinite(refs[0]).all() and torch.isfinite(refs[2]).all()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out1, outv):
            t.fill_(float("nan"))
        for t in (sel1, selv):
            t.fill_(-9)
        wsv.fill_(0xFF)  # the device-built tile map must be rebuilt by the replay
        ws1.fill_(0xFF)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out1, sel1, outv, selv), refs):
            assert torch.equal(got, ref), "replay %d" % rep
        assert torch.isfinite(junk)
