"""Several MSA decode layers captured in one HIP graph (through torch's graph
capture of the C ABI calls on the capture stream) and replayed: every replay,
with eager work and synchronisations between the replays, must give the eager
outputs bit for bit.  Marked gpu."""
import sys

import pytest
import torch

import block_sparse_long_10_amd as msa
from msa_inputs import TENSOR_IDS, Shape, make_decode_case, normal_bf16
from tests.gpu_util import params_of

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
    vn = c.v[pages, :, :, slots].contiguous()
    outs = torch.empty(n_layers, batch, shape.num_q_heads, shape.head_dim, device="cuda")
    sels = torch.empty(n_layers, batch, shape.num_kv_heads, shape.top_k, dtype=torch.int32,
                       device="cuda")
    ws = torch.empty(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
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
