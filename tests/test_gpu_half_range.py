"""GPU parity when the staged V leaves the range in which the prefill
kernel's half-precision P.V product is exact: values above 2^15 (the half
form would overflow or lose the bound) and blocks whose values are all below
2^-8.  The workgroups that meet such a block must hand their rows to the bf16
launch, whose results are checked against the oracle like any other.  V is
scaled by powers of two, which bfloat16 represents exactly: by 2^14 (values
past the half range, which would overflow) and by 2^-20 (values deep in the
half subnormals, about 6% relative spacing, which the 2e-3 bound would
reject if they were used).  Marked gpu."""
import sys

import pytest
import torch

import oracle
from msa_inputs import Shape, make_prefill_case
from tests.gpu_util import check_out, check_pooled, check_selection, run_prefill

pytestmark = pytest.mark.gpu

SHAPES = [
    Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=128, top_k=4),
    Shape(num_q_heads=24, num_kv_heads=3, num_idx_heads=2, block_size=64, top_k=6),
]


def _check(case, shape, prior):
    g = run_prefill(case)
    P = oracle.prepare(case)
    ref = oracle.prefill(case, prepared=P)
    for t in range(case.num_tiles):
        own = prior // shape.block_size + t
        for gi in range(shape.num_kv_heads):
            check_pooled(g["pooled"][t, gi, :own], ref["pooled"][t, gi, :own])
            check_selection(g["sel"][t, gi], ref["pooled"][t, gi], own, shape.top_k)
    check_out(g["out"], oracle.attend_prefill(case, g["sel"], prepared=P))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scale,every", [(2.0 ** 14, 3), (2.0 ** -20, 1), (2.0 ** -20, 4)])
def test_prefill_v_outside_half_range(shape, scale, every):
    prior, chunk = 1000, 300
    print("\n[gpu half range] %s scale=2^%d every %d pages" % (shape, round(torch.log2(
        torch.tensor(scale)).item()), every), flush=True)
    sys.stdout.flush()
    case = make_prefill_case(shape, prior, chunk, 94, device="cuda", shuffle_pages=True)
    v = case.cache.v
    pages = torch.arange(0, v.shape[0], every, device=v.device)
    v[pages] = v[pages] * scale
    _check(case, shape, prior)


def test_varlen_prefill_v_outside_half_range():
    """The batched call: sequences whose kept V includes scaled pages hand
    their workgroups to the bf16 launch, the others stay in half; every
    sequence is checked against the oracle."""
    import numpy as np
    from msa_inputs import make_varlen_prefill_case
    from tests.test_gpu_varlen import _tile_offsets, run_varlen

    shape = SHAPES[0]
    priors, chunks = [0, 1000, 4096, 130, 5000], [300, 700, 512, 1, 200]
    print("\n[gpu half range] varlen %s" % (shape,), flush=True)
    sys.stdout.flush()
    case = make_varlen_prefill_case(shape, priors, chunks, 95, device="cuda",
                                    shuffle_pages=True)
    v = case.cache.v
    pages = torch.arange(0, v.shape[0], 5, device=v.device)
    v[pages] = v[pages] * 2.0 ** 14
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
                check_selection(my_sel[t, g], ref["pooled"][t, g], own, shape.top_k)
        check_out(out[qs[s]:qs[s] + one.chunk_len], oracle.attend_prefill(one, my_sel, prepared=P),
                  "sequence %d" % s)
