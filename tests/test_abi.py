"""The C ABI library on the CPU: it loads, exports every entry point that
include/msa.h declares, and rejects bad arguments on the host before anything
is launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_long_10_amd as msa
from block_sparse_long_10_amd import Params, PagedKV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "msa_probes.h")]
TIMELINE_HEADER = os.path.join(ROOT, "include", "msa_timeline.h")
TIMELINE_LIB = os.path.join(os.path.dirname(msa.library_path()), "libmsa_timeline.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000  # a non-null address; never dereferenced by a rejected call


def declared_functions(headers=HEADERS):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["msa_decode", "msa_prefill_chunk", "msa_decode_workspace_bytes",
              "msa_prefill_workspace_bytes", "msa_last_error", "msa_index_score_decode",
              "msa_index_score_prefill", "msa_block_topk_prefill", "msa_sparse_attn_prefill",
              "msa_cache_append", "msa_decode_append", "msa_prefill_varlen",
              "msa_prefill_varlen_workspace_bytes", "msa_probe_read_stream",
              "msa_probe_mfma_bf16", "msa_probe_latency_chain"]:
        assert n in names


def test_library_loads_and_exports_every_declared_symbol():
    L = ctypes.CDLL(msa.library_path())
    for n in declared_functions():
        assert hasattr(L, n), n
    assert msa.msa_version().startswith("msa-mi355x")


def _timeline_lib():
    if not os.path.exists(TIMELINE_LIB):
        pytest.skip("libmsa_timeline.so is not built (block_sparse_long_10_amd/build.py builds it)")
    return ctypes.CDLL(TIMELINE_LIB)


def test_timeline_library_exports_the_same_entry_points_and_the_marks():
    """libmsa_timeline.so (the -DMSA_TIMELINE build) exports every entry point
    of msa.h and msa_probes.h plus those of msa_timeline.h; libmsa.so exports
    none of the latter."""
    T = _timeline_lib()
    extra = declared_functions([TIMELINE_HEADER])
    assert extra == ["msa_timeline_clear", "msa_timeline_read"]
    for n in declared_functions() + extra:
        assert hasattr(T, n), n
    L = ctypes.CDLL(msa.library_path())
    for n in extra:
        assert not hasattr(L, n), n


def test_timeline_mark_numbers_match_the_binding():
    """The MSA_MARK_* numbers of msa_timeline.h are 0 .. MSA_NUM_MARKS-1 in
    the order of the binding's TIMELINE_MARKS names."""
    text = open(TIMELINE_HEADER).read()
    marks = {m.group(1).lower(): int(m.group(2))
             for m in re.finditer(r"#define MSA_MARK_([A-Z_]+) (\d+)", text)}
    num = int(re.search(r"#define MSA_NUM_MARKS (\d+)", text).group(1))
    assert sorted(marks.values()) == list(range(num))
    assert [k for k, _ in sorted(marks.items(), key=lambda kv: kv[1])] == msa.TIMELINE_MARKS


def test_timeline_read_rejects_bad_arguments():
    T = _timeline_lib()
    T.msa_timeline_read.restype = ctypes.c_int
    T.msa_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    T.msa_last_error.restype = ctypes.c_char_p
    assert T.msa_timeline_read(None, 64) == INVALID
    assert b"NULL" in T.msa_last_error()
    buf = (ctypes.c_uint64 * 4)()
    assert T.msa_timeline_read(ctypes.cast(buf, ctypes.c_void_p), 4) == INVALID
    assert b"MSA_NUM_MARKS" in T.msa_last_error()


def good_params(**kw):
    p = dict(num_q_heads=64, num_kv_heads=8, head_dim=128, num_idx_heads=4, idx_dim=64,
             block_size=128, top_k=16, softmax_scale=128 ** -0.5)
    p.update(kw)
    return Params(**p)


def fake_kv(num_pages=100, max_blocks=50):
    return PagedKV(FAKE, FAKE, FAKE, FAKE, num_pages, max_blocks)


def decode_status(p, kv, batch=2, max_seq_len=1000, ws_bytes=None, **null):
    L = msa.lib()
    if ws_bytes is None:
        ws_bytes = L.msa_decode_workspace_bytes(ctypes.byref(p), batch, kv.max_blocks_per_seq) \
            if p is not None and kv is not None else 0
    args = dict(q=FAKE, idx_q=FAKE, seq_lens=FAKE, out=FAKE, ws=FAKE)
    args.update(null)
    return L.msa_decode(ctypes.byref(p) if p is not None else None,
                        ctypes.byref(kv) if kv is not None else None, args["q"], args["idx_q"],
                        args["seq_lens"], batch, max_seq_len, args["out"], None, args["ws"],
                        ws_bytes, None)


@pytest.mark.parametrize("change,status,msg", [
    (dict(num_q_heads=60), INVALID, "multiple"),
    (dict(top_k=0), INVALID, ">= 1"),
    (dict(head_dim=64), UNSUPPORTED, "head_dim"),
    (dict(idx_dim=128), UNSUPPORTED, "idx_dim"),
    (dict(block_size=32), UNSUPPORTED, "block_size"),
    (dict(top_k=65), UNSUPPORTED, "top_k"),
    (dict(num_idx_heads=3), UNSUPPORTED, "num_idx_heads"),
    (dict(num_idx_heads=16), UNSUPPORTED, "num_kv_heads * num_idx_heads"),
    (dict(num_q_heads=256), UNSUPPORTED, "group size"),
    (dict(softmax_scale=float("inf")), INVALID, "finite"),
    (dict(sink_blocks=-1), INVALID, "sink"),
    (dict(sink_blocks=8, local_blocks=8), INVALID, "top_k - 1"),
    (dict(num_idx_k_heads=3), UNSUPPORTED, "num_idx_k_heads"),
])
def test_decode_rejects_bad_params(change, status, msg):
    assert decode_status(good_params(**change), fake_kv()) == status
    assert msg in msa.msa_last_error()


def test_decode_rejects_bad_arguments():
    p = good_params()
    assert decode_status(None, fake_kv()) == INVALID
    assert decode_status(p, None) == INVALID
    assert decode_status(p, PagedKV(FAKE, None, FAKE, FAKE, 10, 10)) == INVALID
    assert decode_status(p, fake_kv(num_pages=0)) == INVALID
    assert decode_status(p, fake_kv(), q=None) == INVALID
    assert decode_status(p, fake_kv(), out=None) == INVALID
    assert decode_status(p, fake_kv(), batch=0) == INVALID
    assert decode_status(p, fake_kv(), max_seq_len=0) == INVALID
    assert decode_status(p, fake_kv(max_blocks=4), max_seq_len=513) == INVALID
    assert "max_seq_len" in msa.msa_last_error()
    need = msa.lib().msa_decode_workspace_bytes(ctypes.byref(p), 2, 50)
    assert decode_status(p, fake_kv(), ws_bytes=need - 1) == WORKSPACE
    assert decode_status(p, fake_kv(), ws=None) == WORKSPACE


def test_workspace_sizes():
    L = msa.lib()
    p = good_params()
    a = L.msa_decode_workspace_bytes(ctypes.byref(p), 1, 8192)
    b = L.msa_decode_workspace_bytes(ctypes.byref(p), 8, 8192)
    assert 0 < a < b
    assert a >= 8 * 8192 * 4  # pooled scores alone
    assert L.msa_decode_workspace_bytes(ctypes.byref(good_params(head_dim=64)), 1, 10) == 0
    pf = L.msa_prefill_workspace_bytes(ctypes.byref(p), 1048576, 8192, 8256)
    assert pf >= 64 * 8 * 8256 * 4
    assert L.msa_prefill_workspace_bytes(ctypes.byref(p), 0, 0, 10) == 0


def test_prefill_rejects_bad_arguments():
    L = msa.lib()
    p = good_params()
    kv = fake_kv(num_pages=100, max_blocks=40)
    ws = L.msa_prefill_workspace_bytes(ctypes.byref(p), 1000, 100, 40)

    def st(prior, chunk, params=p, kvv=kv, wsb=ws, q=FAKE):
        return L.msa_prefill_chunk(ctypes.byref(params), ctypes.byref(kvv), q, FAKE, prior, chunk,
                                   FAKE, None, FAKE, wsb, None)

    assert st(1000, 0) == INVALID
    assert st(-1, 10) == INVALID
    assert st(5000, 200) == INVALID       # beyond max_blocks * block_size
    assert st(1000, 100, q=None) == INVALID
    assert st(1000, 100, wsb=ws - 1) == WORKSPACE
    big = good_params(num_kv_heads=4, num_q_heads=32, num_idx_heads=8)
    assert st(1000, 100, params=big) == UNSUPPORTED   # block_size * num_idx_heads > 512
    assert L.msa_index_score_prefill(ctypes.byref(p), ctypes.byref(kv), None, 10, 10, FAKE,
                                     None) == INVALID
    assert L.msa_block_topk_prefill(ctypes.byref(p), 10, 10, 40, FAKE, None, None) == INVALID
    assert L.msa_sparse_attn_prefill(ctypes.byref(p), ctypes.byref(kv), FAKE, 10, 10, None, FAKE,
                                     None) == INVALID


def test_binding_has_no_cpu_path():
    p = msa.make_params(8, 1, block_size=64, top_k=8)
    k = torch.zeros(4, 1, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="GPU tensor"):
        msa.make_kv(k, k, torch.zeros(4, 64, 64, dtype=torch.bfloat16),
                    torch.zeros(1, 4, dtype=torch.int32))


def test_append_entry_points_reject_bad_arguments():
    from block_sparse_long_10_amd import PagedKVMut
    L = msa.lib()
    p = good_params()
    kv = PagedKVMut(FAKE, FAKE, FAKE, FAKE, 100, 40)

    def app(params=p, kvv=kv, k=FAKE, v=FAKE, x=FAKE, start=FAKE, batch=2, n_new=5):
        return L.msa_cache_append(ctypes.byref(params) if params is not None else None,
                                  ctypes.byref(kvv) if kvv is not None else None,
                                  k, v, x, start, batch, n_new, None)

    assert app(params=None) == INVALID
    assert app(kvv=None) == INVALID
    assert app(kvv=PagedKVMut(FAKE, None, FAKE, FAKE, 100, 40)) == INVALID
    assert app(v=None) == INVALID
    assert app(start=None) == INVALID
    assert app(n_new=0) == INVALID
    assert app(batch=0) == INVALID
    assert app(n_new=40 * 128 + 1) == INVALID
    assert "n_new" in msa.msa_last_error()
    assert app(params=good_params(head_dim=64)) == UNSUPPORTED
    ws = L.msa_decode_workspace_bytes(ctypes.byref(p), 2, 40)

    def dec(kvv=kv, k=FAKE, q=FAKE, wsb=ws):
        return L.msa_decode_append(ctypes.byref(p), ctypes.byref(kvv), k, FAKE, FAKE, q, FAKE, FAKE,
                                   2, 1000, FAKE, None, FAKE, wsb, None)

    assert dec(k=None) == INVALID
    assert dec(q=None) == INVALID
    assert dec(kvv=PagedKVMut(FAKE, FAKE, None, FAKE, 100, 40)) == INVALID
    assert dec(wsb=ws - 1) == WORKSPACE


def test_varlen_prefill_rejects_bad_arguments():
    L = msa.lib()
    p = good_params()
    kv = fake_kv(num_pages=100, max_blocks=40)

    def arr(v):
        return ctypes.cast((ctypes.c_int32 * len(v))(*v), ctypes.c_void_p)

    def st(prior, chunk, batch=None, wsb=None, host=True, q=FAKE):
        batch = len(prior) if batch is None else batch
        ph, ch = (arr(prior), arr(chunk)) if host else (None, None)
        if wsb is None:
            wsb = L.msa_prefill_varlen_workspace_bytes(ctypes.byref(p), ph, ch, batch, 40)
        return L.msa_prefill_varlen(ctypes.byref(p), ctypes.byref(kv), q, FAKE, FAKE, FAKE, ph, ch,
                                    batch, FAKE, None, FAKE, wsb, None)

    assert st([0, 100], [10, 0]) == INVALID            # empty chunk
    assert st([-1], [10]) == INVALID
    assert st([5000], [200]) == INVALID               # beyond max_blocks * block_size
    assert st([10], [10], batch=0) == INVALID
    assert st([10], [10], host=False, wsb=1 << 20) == INVALID
    assert st([10], [10], q=None) == INVALID
    need = L.msa_prefill_varlen_workspace_bytes(ctypes.byref(p), arr([10, 300]), arr([5, 40]), 2, 40)
    assert need > 0
    assert st([10, 300], [5, 40], wsb=need - 1) == WORKSPACE
    assert L.msa_prefill_varlen_workspace_bytes(ctypes.byref(p), arr([10]), arr([0]), 1, 40) == 0


@pytest.mark.parametrize("args,msg", [
    ((None, 1024, 8, FAKE), "NULL"),
    ((FAKE, 1024, 8, None), "NULL"),
    ((FAKE, 0, 8, FAKE), "multiple of 16"),
    ((FAKE, 1000, 8, FAKE), "multiple of 16"),
    ((FAKE, 1024, 0, FAKE), "workgroups"),
    ((FAKE, 1024, (1 << 20) + 1, FAKE), "workgroups"),
])
def test_read_stream_probe_rejects_bad_arguments(args, msg):
    assert msa.lib().msa_probe_read_stream(*args, None) == INVALID
    assert msg in msa.msa_last_error()


@pytest.mark.parametrize("args,msg", [
    ((0, 8, FAKE), "iters"),
    ((1 << 25, 8, FAKE), "iters"),
    ((16, 0, FAKE), "workgroups"),
    ((16, 8, None), "NULL"),
])
def test_mfma_probe_rejects_bad_arguments(args, msg):
    assert msa.lib().msa_probe_mfma_bf16(*args, None) == INVALID
    assert msg in msa.msa_last_error()


@pytest.mark.parametrize("args,msg", [
    ((None, 16, 4, 0, FAKE), "NULL"),
    ((FAKE, 16, 4, 0, None), "NULL"),
    ((FAKE, 0, 4, 0, FAKE), "n must be"),
    ((FAKE, 16, 4, 16, FAKE), "start"),
    ((FAKE, 16, 4, -1, FAKE), "start"),
    ((FAKE, 16, -1, 0, FAKE), "steps"),
    ((FAKE, 16, (1 << 24) + 1, 0, FAKE), "steps"),
])
def test_latency_probe_rejects_bad_arguments(args, msg):
    assert msa.lib().msa_probe_latency_chain(*args, None) == INVALID
    assert msg in msa.msa_last_error()


_NO_DEVICE_SCRIPT = r"""
import ctypes, sys
import block_sparse_long_10_amd as msa
from block_sparse_long_10_amd import Params, PagedKV
L = msa.lib()
F = 0x10000
p = Params(num_q_heads=64, num_kv_heads=8, head_dim=128, num_idx_heads=4, idx_dim=64,
           block_size=128, top_k=16, softmax_scale=128 ** -0.5)
kv = PagedKV(F, F, F, F, 100, 50)
calls = {
    "decode": lambda: L.msa_decode(ctypes.byref(p), ctypes.byref(kv), F, F, F, 2, 1000, F, None, F,
                                   L.msa_decode_workspace_bytes(ctypes.byref(p), 2, 50), None),
    "prefill": lambda: L.msa_prefill_chunk(ctypes.byref(p), ctypes.byref(kv), F, F, 1000, 100, F,
                                           None, F,
                                           L.msa_prefill_workspace_bytes(ctypes.byref(p), 1000,
                                                                         100, 50), None),
    "index": lambda: L.msa_index_score_decode(ctypes.byref(p), ctypes.byref(kv), F, F, 2, 1000,
                                              F, None),
}
for name, call in calls.items():
    st = call()
    err = msa.msa_last_error()
    print(name, st, err)
    if st != -4 or not err:
        sys.exit(1)
"""


def test_launching_call_without_a_device_returns_hip_error():
    """With no GPU visible, a call that passes host validation reaches its
    first launch, which fails: the call returns MSA_ERR_HIP with a message and
    nothing crashes.  Run in a child process with every device hidden; skipped
    where a GPU is visible to this process (then the fake pointers could
    reach a real launch)."""
    import subprocess
    import sys
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; the no-device path is checked on hosts without one")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", _NO_DEVICE_SCRIPT], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(" -4 ") == 3, r.stdout
