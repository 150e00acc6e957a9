"""The timeline build (libmsa_timeline.so, include/msa_timeline.h) on the GPU.
It runs in a child process, since a process loads one of the two libraries.
The child checks that the marks of the watched decode attention workgroup
are reached and come in the order of its chain, on the fused selection with 4
and with 32 scores per thread.  Its outputs and selections must equal those
of libmsa.so, computed here in the parent, bit for bit: the marks only add
stores.  Marked gpu."""
import os
import subprocess
import sys

import numpy as np
import pytest

import block_sparse_long_10_amd as msa
from msa_inputs import Shape, make_decode_case
from tests.gpu_util import run_decode

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPE = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8)
CASES = [([3000, 777], 121),           # rows of at most 1024 blocks: 4 scores per thread
         ([1100 * 64 + 5, 4000], 122)]  # a row of 1100 blocks: 32 scores per thread

CHILD = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import block_sparse_long_10_amd as msa
msa.use_timeline_library()
from msa_inputs import Shape, make_decode_case
from tests.gpu_util import run_decode
shape = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8)
lengths = [int(x) for x in sys.argv[3].split(",")]
case = make_decode_case(shape, lengths, int(sys.argv[4]), device="cuda", shuffle_pages=True)
chain = ["start", "scores_in", "range", "bin", "counted", "gathered", "selected", "block_known",
         "kv_in", "scores", "softmax", "pv", "waves_done", "combined", "stored", "counted_in"]
for rep in range(3):
    msa.msa_timeline_clear()
    g = run_decode(case, with_pooled=False)
    m = msa.msa_timeline_read()
    t = [m[k] for k in chain]
    assert all(v > 0 for v in t), m
    assert t == sorted(t), m
    assert 0 < m["index_end"] <= m["start"] + 100, m   # (10 ns ticks)
    assert m["merged"] >= m["start"], m
print("marks ok", flush=True)
np.savez(sys.argv[2], out=g["out"], sel=g["sel"])
"""


@pytest.mark.parametrize("lengths,seed", CASES)
def test_timeline_build_marks_and_results(lengths, seed, tmp_path):
    lib = os.path.join(os.path.dirname(msa.library_path()), "libmsa_timeline.so")
    if not os.path.exists(lib):
        pytest.skip("libmsa_timeline.so is not built")
    print("\n[gpu timeline] lengths %s" % lengths, flush=True)
    sys.stdout.flush()
    ref = run_decode(make_decode_case(SHAPE, lengths, seed, device="cuda", shuffle_pages=True),
                     with_pooled=False)
    npz = str(tmp_path / "timeline_out.npz")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, npz, ",".join(map(str, lengths)),
                        str(seed)], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    got = np.load(npz)
    np.testing.assert_array_equal(got["sel"], ref["sel"])
    assert np.array_equal(got["out"], ref["out"])
