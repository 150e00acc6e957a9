"""Seeded random configurations of the whole path on the GPU, each against the
oracle through the C ABI: group sizes, index heads, block size, k, forced sink
and local blocks, shared or per-group index keys, ragged lengths (decode),
prior / chunk positions (prefill) and batches of them (batched prefill), paged
and poisoned caches.  The draws are
fixed by the seeds, so every run checks the same configurations.  Marked gpu."""
import random
import sys

import pytest

import oracle
from msa_inputs import Shape, make_decode_case, make_prefill_case, make_varlen_prefill_case
from tests.gpu_util import check_out, check_pooled, check_selection, run_decode, run_prefill
from tests.test_gpu_varlen import run_varlen

pytestmark = pytest.mark.gpu

DEV = "cuda"


def random_shape(rng, prefill=False):
    """A configuration inside the documented support set (include/msa.h); for
    prefill also block_size * num_idx_heads <= 512."""
    hkv = rng.choice([1, 2, 3, 4, 8])
    group = rng.choice([g for g in (1, 2, 3, 4, 8, 16) if g * hkv <= 64])
    B = rng.choice([64, 128])
    ni = rng.choice([n for n in (1, 2, 4, 8, 16) if n * hkv <= 64 and (not prefill or n * B <= 512)])
    k = rng.choice([1, 2, 3, 5, 8, 13, 16, 31, 64])
    forced = rng.random() < 0.4 and k >= 2
    sink = rng.randint(0, k - 1) if forced else 0
    local = rng.randint(0, k - 1 - sink) if forced else 0
    ik = hkv if (hkv > 1 and rng.random() < 0.3) else 1
    return Shape(num_q_heads=hkv * group, num_kv_heads=hkv, num_idx_heads=ni, block_size=B,
                 top_k=k, sink_blocks=sink, local_blocks=local, idx_k_heads=ik)


def _announce(what):
    print("\n[gpu random] " + what, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    rng = random.Random(1000 + seed)
    shape = random_shape(rng)
    lengths = [rng.choice([1, rng.randint(2, 300), rng.randint(300, 6000), rng.randint(6000, 30000)])
               for _ in range(rng.randint(1, 5))]
    _announce("decode seed %d %s lengths %s" % (seed, shape, lengths))
    case = make_decode_case(shape, lengths, 5000 + seed, device=DEV, shuffle_pages=True,
                            poison_frac=0.05)
    g = run_decode(case)
    P = oracle.prepare(case)
    ref = oracle.decode(case, prepared=P)
    for s, L in enumerate(lengths):
        own = (L - 1) // shape.block_size
        for gi in range(shape.num_kv_heads):
            check_pooled(g["pooled"][s, gi, :own], ref["pooled"][s, gi, :own])
            check_selection(g["sel"][s, gi], ref["pooled"][s, gi], own, shape.top_k,
                            sink=shape.sink_blocks, local=shape.local_blocks)
    worst = check_out(g["out"], oracle.attend_decode(case, g["sel"], prepared=P))
    print("worst row err %.3g" % worst)


@pytest.mark.parametrize("seed", range(8))
def test_random_prefill(seed):
    rng = random.Random(2000 + seed)
    shape = random_shape(rng, prefill=True)
    prior = rng.choice([0, rng.randint(1, 500), rng.randint(500, 9000)])
    chunk = rng.choice([1, rng.randint(2, 200), rng.randint(200, 700)])
    _announce("prefill seed %d %s P=%d C=%d" % (seed, shape, prior, chunk))
    case = make_prefill_case(shape, prior, chunk, 6000 + seed, device=DEV, shuffle_pages=True,
                             poison_frac=0.05)
    g = run_prefill(case)
    P = oracle.prepare(case)
    ref = oracle.prefill(case, prepared=P)
    B = shape.block_size
    for t in range(case.num_tiles):
        own = prior // B + t
        for gi in range(shape.num_kv_heads):
            check_pooled(g["pooled"][t, gi, :own], ref["pooled"][t, gi, :own])
            check_selection(g["sel"][t, gi], ref["pooled"][t, gi], own, shape.top_k,
                            sink=shape.sink_blocks, local=shape.local_blocks)
    worst = check_out(g["out"], oracle.attend_prefill(case, g["sel"], prepared=P))
    print("worst row err %.3g" % worst)


@pytest.mark.parametrize("seed", range(6))
def test_random_varlen(seed):
    """msa_prefill_varlen over 1-6 sequences of random prior and chunk
    lengths (empty priors and one-token chunks among them), each sequence's
    selections and outputs against the oracle run on that sequence alone."""
    rng = random.Random(3000 + seed)
    shape = random_shape(rng, prefill=True)
    n = rng.randint(1, 6)
    priors = [rng.choice([0, rng.randint(1, 600), rng.randint(600, 7000)]) for _ in range(n)]
    chunks = [rng.choice([1, rng.randint(2, 150), rng.randint(150, 500)]) for _ in range(n)]
    _announce("varlen seed %d %s priors %s chunks %s" % (seed, shape, priors, chunks))
    case = make_varlen_prefill_case(shape, priors, chunks, 7000 + seed, device=DEV,
                                    shuffle_pages=True, poison_frac=0.05)
    out, sel = run_varlen(case)
    out, sel = out.cpu().numpy().astype("float64"), sel.cpu().numpy()
    B = shape.block_size
    worst, t0 = 0.0, 0
    for s in range(n):
        one = case.sequence(s)
        P = oracle.prepare(one)
        ref = oracle.prefill(one, prepared=P)
        nt = one.num_tiles
        my_sel = sel[t0:t0 + nt]
        t0 += nt
        for t in range(nt):
            own = one.prior_len // B + t
            for gi in range(shape.num_kv_heads):
                check_selection(my_sel[t, gi], ref["pooled"][t, gi], own, shape.top_k,
                                sink=shape.sink_blocks, local=shape.local_blocks)
        q0 = case.q_start[s]
        worst = max(worst, check_out(out[q0:q0 + one.chunk_len],
                                     oracle.attend_prefill(one, my_sel, prepared=P),
                                     "sequence %d" % s))
    print("worst row err %.3g" % worst)
