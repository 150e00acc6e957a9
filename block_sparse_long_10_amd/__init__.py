"""MiniMax Sparse Attention (MSA) decode and chunked prefill on MI355X (gfx950).

A thin ctypes binding of ``libmsa.so`` (include/msa.h).  The functions carry
the C names and only marshal arguments: every step of the computation runs in
the library's HIP kernels.  Tensors must be CUDA (HIP) tensors of the dtype
and layout the header states; work is enqueued on torch's current stream.
There is no CPU fallback: without the built library, or with host tensors,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MSAError", "Params", "PagedKV", "make_params", "make_kv", "library_path",
    "msa_decode_workspace_bytes", "msa_decode", "msa_decode_noalloc", "msa_index_score_decode",
    "msa_prefill_workspace_bytes", "msa_prefill_chunk", "msa_index_score_prefill",
    "msa_block_topk_prefill", "msa_sparse_attn_prefill", "msa_last_error", "msa_version",
    "PagedKVMut", "make_kv_mut", "msa_cache_append", "msa_decode_append",
    "msa_prefill_varlen_workspace_bytes", "msa_prefill_varlen", "msa_probe_read_stream",
    "msa_probe_mfma_bf16", "msa_probe_latency_chain", "use_timeline_library", "msa_timeline_clear",
    "msa_timeline_read", "TIMELINE_MARKS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmsa.so")
_TIMELINE_LIB_PATH = os.path.join(_HERE, "libmsa_timeline.so")

MSA_OK = 0
STATUS_NAMES = {0: "MSA_OK", -1: "MSA_ERR_INVALID_ARGUMENT", -2: "MSA_ERR_UNSUPPORTED",
                -3: "MSA_ERR_WORKSPACE", -4: "MSA_ERR_HIP"}


class MSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("sink_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
                ("num_idx_k_heads", ctypes.c_int32)]


class PagedKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("idx_k", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32)]


class PagedKVMut(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("idx_k", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def use_timeline_library() -> None:
    """Load libmsa_timeline.so (include/msa_timeline.h: the same entry points
    plus the wall-clock marks) instead of libmsa.so.  Must come before the
    first call into the library."""
    global _LIB_PATH
    if _lib is not None:
        raise RuntimeError("the library is already loaded from %s" % _LIB_PATH)
    _LIB_PATH = _TIMELINE_LIB_PATH


def lib():
    """The loaded libmsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libmsa.so is not built; run __graft_entry__.build() or "
                              "python block_sparse_long_10_amd/build.py")
        L = ctypes.CDLL(_LIB_PATH)
        P, K = ctypes.POINTER(Params), ctypes.POINTER(PagedKV)
        KM = ctypes.POINTER(PagedKVMut)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sigs = {
            "msa_decode_workspace_bytes": (sz, [P, i32, i32]),
            "msa_decode": (ctypes.c_int, [P, K, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]),
            "msa_decode_noalloc": (ctypes.c_int, [P, K, vp, vp, vp, i32, i32, vp, vp, vp]),
            "msa_index_score_decode": (ctypes.c_int, [P, K, vp, vp, i32, i32, vp, vp]),
            "msa_prefill_workspace_bytes": (sz, [P, i32, i32, i32]),
            "msa_prefill_chunk": (ctypes.c_int, [P, K, vp, vp, i32, i32, vp, vp, vp, sz, vp]),
            "msa_index_score_prefill": (ctypes.c_int, [P, K, vp, i32, i32, vp, vp]),
            "msa_block_topk_prefill": (ctypes.c_int, [P, i32, i32, i32, vp, vp, vp]),
            "msa_sparse_attn_prefill": (ctypes.c_int, [P, K, vp, i32, i32, vp, vp, vp]),
            "msa_cache_append": (ctypes.c_int, [P, KM, vp, vp, vp, vp, i32, i32, vp]),
            "msa_decode_append": (ctypes.c_int, [P, KM, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp,
                                                 vp, sz, vp]),
            "msa_prefill_varlen_workspace_bytes": (sz, [P, vp, vp, i32, i32]),
            "msa_prefill_varlen": (ctypes.c_int, [P, K, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                                  sz, vp]),
            "msa_last_error": (ctypes.c_char_p, []),
            "msa_version": (ctypes.c_char_p, []),
            "msa_probe_read_stream": (ctypes.c_int, [vp, sz, i32, vp, vp]),
            "msa_probe_mfma_bf16": (ctypes.c_int, [i32, i32, vp, vp]),
            "msa_probe_latency_chain": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
        }
        if hasattr(L, "msa_timeline_read"):  # the timeline build only
            sigs["msa_timeline_clear"] = (ctypes.c_int, [])
            sigs["msa_timeline_read"] = (ctypes.c_int, [vp, i32])
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def msa_last_error() -> str:
    return lib().msa_last_error().decode()


def msa_version() -> str:
    return lib().msa_version().decode()


def _check(status: int) -> None:
    if status != MSA_OK:
        raise MSAError(status, msa_last_error())


def _dev(t: Optional[torch.Tensor], dtype, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor (no CPU path exists)" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_params(num_q_heads: int, num_kv_heads: int, head_dim: int = 128, num_idx_heads: int = 4,
                idx_dim: int = 64, block_size: int = 128, top_k: int = 16,
                softmax_scale: Optional[float] = None, sink_blocks: int = 0,
                local_blocks: int = 0, num_idx_k_heads: int = 1) -> Params:
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    return Params(num_q_heads, num_kv_heads, head_dim, num_idx_heads, idx_dim, block_size, top_k,
                  float(softmax_scale), sink_blocks, local_blocks, num_idx_k_heads)


def make_kv(k: torch.Tensor, v: torch.Tensor, idx_k: torch.Tensor,
            block_table: torch.Tensor) -> PagedKV:
    """Paged cache descriptor: k [P][Hkv][B][D], v [P][Hkv][B][D], idx_k [P][B][d_i] or
    [P][Hkv][B][d_i] (bf16), block_table int32 [batch][max_blocks]."""
    kv = PagedKV(_dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
                 _dev(idx_k, torch.bfloat16, "idx_k"), _dev(block_table, torch.int32, "block_table"),
                 int(k.shape[0]), int(block_table.shape[-1]))
    kv._keep = (k, v, idx_k, block_table)
    return kv


def make_kv_mut(k: torch.Tensor, v: torch.Tensor, idx_k: torch.Tensor,
                block_table: torch.Tensor) -> PagedKVMut:
    """Writable paged cache descriptor (same layouts as make_kv), for the calls that append."""
    kv = PagedKVMut(_dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
                    _dev(idx_k, torch.bfloat16, "idx_k"),
                    _dev(block_table, torch.int32, "block_table"),
                    int(k.shape[0]), int(block_table.shape[-1]))
    kv._keep = (k, v, idx_k, block_table)
    return kv


def msa_cache_append(params: Params, kv: PagedKVMut, k_new, v_new, idx_k_new, start_pos,
                     batch: int, n_new: int, stream=None) -> None:
    _check(lib().msa_cache_append(ctypes.byref(params), ctypes.byref(kv),
                                  _dev(k_new, torch.bfloat16, "k_new"),
                                  _dev(v_new, torch.bfloat16, "v_new"),
                                  _dev(idx_k_new, torch.bfloat16, "idx_k_new"),
                                  _dev(start_pos, torch.int32, "start_pos"), batch, n_new,
                                  _stream(stream)))


def msa_decode_append(params: Params, kv: PagedKVMut, k_new, v_new, idx_k_new, q, idx_q,
                      seq_lens, batch: int, max_seq_len: int, out, sel=None, workspace=None,
                      stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msa_decode_append(ctypes.byref(params), ctypes.byref(kv),
                                   _dev(k_new, torch.bfloat16, "k_new"),
                                   _dev(v_new, torch.bfloat16, "v_new"),
                                   _dev(idx_k_new, torch.bfloat16, "idx_k_new"),
                                   _dev(q, torch.bfloat16, "q"), _dev(idx_q, torch.bfloat16, "idx_q"),
                                   _dev(seq_lens, torch.int32, "seq_lens"), batch, max_seq_len,
                                   _dev(out, torch.float32, "out"), _dev(sel, torch.int32, "sel"),
                                   _dev(workspace, None, "workspace"), ws_bytes, _stream(stream)))


def msa_decode_workspace_bytes(params: Params, batch: int, max_blocks_per_seq: int) -> int:
    return int(lib().msa_decode_workspace_bytes(ctypes.byref(params), batch, max_blocks_per_seq))


def msa_decode(params: Params, kv: PagedKV, q, idx_q, seq_lens, batch: int, max_seq_len: int,
               out, sel=None, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msa_decode(ctypes.byref(params), ctypes.byref(kv),
                            _dev(q, torch.bfloat16, "q"), _dev(idx_q, torch.bfloat16, "idx_q"),
                            _dev(seq_lens, torch.int32, "seq_lens"), batch, max_seq_len,
                            _dev(out, torch.float32, "out"), _dev(sel, torch.int32, "sel"),
                            _dev(workspace, None, "workspace"), ws_bytes, _stream(stream)))


def msa_decode_noalloc(params: Params, kv: PagedKV, q, idx_q, seq_lens, batch: int,
                       max_seq_len: int, out, sel=None, stream=None) -> None:
    _check(lib().msa_decode_noalloc(ctypes.byref(params), ctypes.byref(kv),
                                    _dev(q, torch.bfloat16, "q"),
                                    _dev(idx_q, torch.bfloat16, "idx_q"),
                                    _dev(seq_lens, torch.int32, "seq_lens"), batch, max_seq_len,
                                    _dev(out, torch.float32, "out"),
                                    _dev(sel, torch.int32, "sel"), _stream(stream)))


def msa_index_score_decode(params: Params, kv: PagedKV, idx_q, seq_lens, batch: int,
                           max_seq_len: int, pooled, stream=None) -> None:
    _check(lib().msa_index_score_decode(ctypes.byref(params), ctypes.byref(kv),
                                        _dev(idx_q, torch.bfloat16, "idx_q"),
                                        _dev(seq_lens, torch.int32, "seq_lens"), batch,
                                        max_seq_len, _dev(pooled, torch.float32, "pooled"),
                                        _stream(stream)))


def msa_prefill_workspace_bytes(params: Params, prior_len: int, chunk_len: int,
                                max_blocks_per_seq: int) -> int:
    return int(lib().msa_prefill_workspace_bytes(ctypes.byref(params), prior_len, chunk_len,
                                                 max_blocks_per_seq))


def msa_prefill_chunk(params: Params, kv: PagedKV, q, idx_q, prior_len: int, chunk_len: int,
                      out, sel=None, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msa_prefill_chunk(ctypes.byref(params), ctypes.byref(kv),
                                   _dev(q, torch.bfloat16, "q"), _dev(idx_q, torch.bfloat16, "idx_q"),
                                   prior_len, chunk_len, _dev(out, torch.float32, "out"),
                                   _dev(sel, torch.int32, "sel"), _dev(workspace, None, "workspace"),
                                   ws_bytes, _stream(stream)))


def msa_index_score_prefill(params: Params, kv: PagedKV, idx_q, prior_len: int, chunk_len: int,
                            pooled, stream=None) -> None:
    _check(lib().msa_index_score_prefill(ctypes.byref(params), ctypes.byref(kv),
                                         _dev(idx_q, torch.bfloat16, "idx_q"), prior_len, chunk_len,
                                         _dev(pooled, torch.float32, "pooled"), _stream(stream)))


def msa_block_topk_prefill(params: Params, prior_len: int, chunk_len: int, max_blocks_per_seq: int,
                           pooled, sel, stream=None) -> None:
    _check(lib().msa_block_topk_prefill(ctypes.byref(params), prior_len, chunk_len,
                                        max_blocks_per_seq, _dev(pooled, torch.float32, "pooled"),
                                        _dev(sel, torch.int32, "sel"), _stream(stream)))


def msa_sparse_attn_prefill(params: Params, kv: PagedKV, q, prior_len: int, chunk_len: int, sel,
                            out, stream=None) -> None:
    _check(lib().msa_sparse_attn_prefill(ctypes.byref(params), ctypes.byref(kv),
                                         _dev(q, torch.bfloat16, "q"), prior_len, chunk_len,
                                         _dev(sel, torch.int32, "sel"),
                                         _dev(out, torch.float32, "out"), _stream(stream)))


def _host_i32(values):
    arr = (ctypes.c_int32 * len(values))(*[int(x) for x in values])
    return arr


def msa_prefill_varlen_workspace_bytes(params: Params, prior_lens, chunk_lens,
                                       max_blocks_per_seq: int) -> int:
    """prior_lens, chunk_lens: host sequences of ints."""
    n = len(prior_lens)
    return int(lib().msa_prefill_varlen_workspace_bytes(
        ctypes.byref(params), ctypes.cast(_host_i32(prior_lens), ctypes.c_void_p),
        ctypes.cast(_host_i32(chunk_lens), ctypes.c_void_p), n, max_blocks_per_seq))


def msa_prefill_varlen(params: Params, kv: PagedKV, q, idx_q, prior_lens, chunk_lens,
                       prior_lens_host, chunk_lens_host, out, sel=None, workspace=None,
                       stream=None) -> None:
    """prior_lens, chunk_lens: int32 GPU tensors [batch]; the *_host arguments
    are host sequences of the same values."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ph, ch = _host_i32(prior_lens_host), _host_i32(chunk_lens_host)
    _check(lib().msa_prefill_varlen(ctypes.byref(params), ctypes.byref(kv),
                                    _dev(q, torch.bfloat16, "q"),
                                    _dev(idx_q, torch.bfloat16, "idx_q"),
                                    _dev(prior_lens, torch.int32, "prior_lens"),
                                    _dev(chunk_lens, torch.int32, "chunk_lens"),
                                    ctypes.cast(ph, ctypes.c_void_p),
                                    ctypes.cast(ch, ctypes.c_void_p), len(prior_lens_host),
                                    _dev(out, torch.float32, "out"), _dev(sel, torch.int32, "sel"),
                                    _dev(workspace, None, "workspace"), ws_bytes,
                                    _stream(stream)))


# ------------------------------------------------------------ measurement
def msa_probe_read_stream(src: torch.Tensor, workgroups: int, sink: torch.Tensor,
                          stream=None) -> None:
    """One non-temporal read pass over src (any dtype, contiguous GPU tensor)."""
    _check(lib().msa_probe_read_stream(_dev(src, None, "src"), src.numel() * src.element_size(),
                                       workgroups, _dev(sink, None, "sink"), _stream(stream)))


def msa_probe_mfma_bf16(iters: int, workgroups: int, sink: torch.Tensor, stream=None) -> None:
    """32768 * 16 * iters * workgroups flops of v_mfma_f32_32x32x16_bf16."""
    _check(lib().msa_probe_mfma_bf16(iters, workgroups, _dev(sink, None, "sink"), _stream(stream)))


def msa_probe_latency_chain(next_: torch.Tensor, steps: int, start: int, sink: torch.Tensor,
                            stream=None) -> None:
    """steps dependent loads p = next_[p] from p = start (next_: int32 GPU table)."""
    _check(lib().msa_probe_latency_chain(_dev(next_, torch.int32, "next"), next_.numel(), steps,
                                         start, _dev(sink, torch.int32, "sink"), _stream(stream)))


# Mark numbers of include/msa_timeline.h, in order.
TIMELINE_MARKS = ["start", "scores_in", "range", "bin", "counted", "gathered", "selected",
                  "block_known", "kv_in", "scores", "softmax", "pv", "waves_done", "combined",
                  "stored", "counted_in", "merged", "index_end"]


def _timeline_lib():
    L = lib()
    if not hasattr(L, "msa_timeline_read"):
        raise RuntimeError("%s has no timeline marks; call use_timeline_library() first" % _LIB_PATH)
    return L


def msa_timeline_clear() -> None:
    """Sets every mark to 0 (synchronises the device)."""
    _check(_timeline_lib().msa_timeline_clear())


def msa_timeline_read() -> dict:
    """The marks, {name: 10 ns clock ticks, 0 if not reached} (synchronises
    the device)."""
    buf = (ctypes.c_uint64 * len(TIMELINE_MARKS))()
    _check(_timeline_lib().msa_timeline_read(ctypes.cast(buf, ctypes.c_void_p), len(buf)))
    return dict(zip(TIMELINE_MARKS, list(buf)))
