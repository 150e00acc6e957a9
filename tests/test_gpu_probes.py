"""The measurement kernels of include/msa_probes.h on the GPU: the read
stream visits every 16-byte word of its buffer (a single word whose fold
equals the probe's constant, placed at chosen positions, must reach the
sink), the MFMA loop runs to completion, and the latency chain ends where
the same chain followed on the host ends.  Marked gpu."""
import sys

import pytest
import torch

import block_sparse_long_10_amd as msa

pytestmark = pytest.mark.gpu

PROBE_MAGIC = 0x9E3779B9


@pytest.mark.parametrize("words,workgroups,pos", [
    (1, 1, 0),                       # a single word
    (4096, 3, 4095),                 # tail of the grid-stride loop
    (1 << 20, 512, 0),
    (1 << 20, 512, (1 << 20) - 1),
    (1 << 20, 512, 777_777),         # inside the 8-deep unrolled body
    ((1 << 20) + 13, 4096, (1 << 20) + 12),
])
def test_read_stream_visits_every_word(words, workgroups, pos):
    print("\n[gpu probes] read stream words=%d wg=%d pos=%d" % (words, workgroups, pos), flush=True)
    sys.stdout.flush()
    buf = torch.zeros(words, 4, dtype=torch.int32, device="cuda")
    buf[pos, 0] = torch.tensor(PROBE_MAGIC, dtype=torch.int64).to(torch.int32)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    msa.msa_probe_read_stream(buf, workgroups, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) & 0xFFFFFFFF == PROBE_MAGIC


def test_read_stream_without_the_constant_writes_nothing():
    buf = torch.ones(1 << 16, 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    msa.msa_probe_read_stream(buf, 64, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == 0


def test_mfma_loop_runs():
    print("\n[gpu probes] mfma loop", flush=True)
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    msa.msa_probe_mfma_bf16(64, 256, sink)
    torch.cuda.synchronize()
    assert float(sink[0].item()) == 0.0


@pytest.mark.parametrize("n,steps,start", [(1, 5, 0), (1000, 0, 7), (1000, 137, 3), (4096, 5000, 0)])
def test_latency_chain_follows_the_table(n, steps, start):
    print("\n[gpu probes] latency chain n=%d steps=%d" % (n, steps), flush=True)
    sys.stdout.flush()
    g = torch.Generator().manual_seed(n + steps)
    table = torch.randperm(n, generator=g).to(torch.int32)
    table[n // 2] = n + 5  # outside the table: the chain restarts at 0
    p = start
    for _ in range(steps):
        p = int(table[p])
        if not 0 <= p < n:
            p = 0
    sink = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    msa.msa_probe_latency_chain(table.cuda(), steps, start, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == p

