"""MSA reference oracle (plain C, fp64) -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It loads ``libmsa_oracle.so`` (built
from ``msa_oracle.c`` with gcc) through ctypes and takes its inputs from the
seeded cases of ``msa_inputs``; tensors on a GPU are copied to the host.

The definition it implements, and the readings taken where the source page
is silent, are stated in the header of ``msa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, IEEE arithmetic, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                               _SRC, "-o", _LIB + ".tmp", "-lm"])
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("softmax_scale", ctypes.c_double),
                ("sink_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
                ("num_idx_k_heads", ctypes.c_int32)]


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("idx_k", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32)]


_lib = None
_lib_path = None  # set by use_library(); None = the built oracle


def use_library(path: Optional[str]) -> None:
    """Point the wrappers at another build of msa_oracle.c (None = default).

    Used by the tests that compile deliberately broken copies of the oracle to
    show that the pins catch them."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


def lib():
    global _lib
    if _lib is None:
        path = _lib_path or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        P, C = ctypes.POINTER(_Params), ctypes.POINTER(_Cache)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.msa_oracle_decode.argtypes = [P, C, vp, vp, vp, i32, vp, vp, vp]
        L.msa_oracle_attend_decode.argtypes = [P, C, vp, vp, i32, vp, vp]
        L.msa_oracle_prefill.argtypes = [P, C, vp, vp, i32, i32, vp, i32, vp, vp, vp]
        L.msa_oracle_attend_prefill.argtypes = [P, C, vp, i32, i32, vp, i32, vp, vp]
        L.msa_oracle_select.argtypes = [vp, i32, i32, vp]
        L.msa_oracle_select_forced.argtypes = [vp, i32, i32, i32, i32, vp]
        L.msa_oracle_block_scores.argtypes = [P, C, i32, vp, i32, i32, i32, vp, i32, vp]
        L.msa_oracle_append.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32]
        for f in ("msa_oracle_decode", "msa_oracle_attend_decode", "msa_oracle_prefill",
                  "msa_oracle_attend_prefill", "msa_oracle_select", "msa_oracle_max_threads",
                  "msa_oracle_block_scores", "msa_oracle_append", "msa_oracle_select_forced"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def max_threads() -> int:
    return int(lib().msa_oracle_max_threads())


def _host_u16(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return np.ascontiguousarray(t.detach().cpu().view(torch.int16).numpy())


def _host_i32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.int32))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class _Prepared:
    """Host copies of a case's cache, kept alive for the C calls.

    With ``kv_pages`` given, only those pages of K and V are copied; the other
    pages of the host arrays stay zero (and, being calloc'ed, take no memory),
    which lets very long contexts be checked for the blocks actually used."""

    def __init__(self, case, kv_pages=None):
        sh, cache = case.shape, case.cache
        self.params = _Params(sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.num_idx_heads,
                              sh.idx_dim, sh.block_size, sh.top_k, sh.softmax_scale,
                              sh.sink_blocks, sh.local_blocks, sh.idx_k_heads)
        if kv_pages is None:
            self.k = _host_u16(cache.k)
            self.v = _host_u16(cache.v)
        else:
            self.k = np.zeros(tuple(cache.k.shape), dtype=np.int16)
            self.v = np.zeros(tuple(cache.v.shape), dtype=np.int16)
            self.fill_pages(case, kv_pages)
        self.idx_k = _host_u16(cache.idx_k)
        self.bt = _host_i32(cache.block_table)
        self.cache = _Cache(_ptr(self.k), _ptr(self.v), _ptr(self.idx_k), _ptr(self.bt),
                            cache.num_pages, cache.max_blocks)
        self.q = _host_u16(case.q)
        self.idx_q = _host_u16(case.idx_q)


    def fill_pages(self, case, pages):
        """Copy the listed pages of K and V into the host arrays."""
        idx = torch.as_tensor(sorted(set(int(p) for p in pages)), dtype=torch.long)
        if idx.numel() == 0:
            return
        dev = case.cache.k.device
        self.k[idx.numpy()] = case.cache.k[idx.to(dev)].cpu().view(torch.int16).numpy()
        self.v[idx.numpy()] = case.cache.v[idx.to(dev)].cpu().view(torch.int16).numpy()


def prepare(case, kv_pages=None) -> _Prepared:
    return _Prepared(case, kv_pages)


def decode(case, prepared: Optional[_Prepared] = None, want_pooled: bool = True) -> dict:
    """Oracle decode: out [batch][Hq][D] f64, sel [batch][Hkv][k], pooled."""
    P = prepared or _Prepared(case)
    sh = case.shape
    batch = case.batch
    lens = _host_i32(case.lengths)
    out = np.zeros((batch, sh.num_q_heads, sh.head_dim), dtype=np.float64)
    sel = np.zeros((batch, sh.num_kv_heads, sh.top_k), dtype=np.int32)
    pooled = (np.zeros((batch, sh.num_kv_heads, case.cache.max_blocks), dtype=np.float64)
              if want_pooled else None)
    rc = lib().msa_oracle_decode(ctypes.byref(P.params), ctypes.byref(P.cache), _ptr(P.q),
                                 _ptr(P.idx_q), _ptr(lens), batch, _ptr(out), _ptr(sel),
                                 _ptr(pooled))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return {"out": out, "sel": sel, "pooled": pooled}


def attend_decode(case, sel, prepared: Optional[_Prepared] = None) -> np.ndarray:
    """Oracle sparse branch for a given selection sel [batch][Hkv][k]."""
    P = prepared or _Prepared(case)
    sh = case.shape
    lens = _host_i32(case.lengths)
    s = _host_i32(sel)
    out = np.zeros((case.batch, sh.num_q_heads, sh.head_dim), dtype=np.float64)
    rc = lib().msa_oracle_attend_decode(ctypes.byref(P.params), ctypes.byref(P.cache),
                                        _ptr(P.q), _ptr(lens), case.batch, _ptr(s), _ptr(out))
    if rc != 0:
        raise ValueError("oracle attend rejected its arguments")
    return out


def tile_rows(case, tile: int):
    """Chunk-query index range [q0, q1) of prefill tile ``tile``."""
    B = case.shape.block_size
    own = case.prior_len // B + tile
    q0 = max(0, own * B - case.prior_len)
    q1 = min(case.chunk_len, (own + 1) * B - case.prior_len)
    return q0, q1


def prefill(case, tiles: Optional[Sequence[int]] = None, prepared: Optional[_Prepared] = None,
            want_pooled: bool = True) -> dict:
    """Oracle prefill for the listed tiles (all if None).

    Returns out [C][Hq][D] (NaN for rows of tiles not computed),
    sel [num_tiles][Hkv][k] (-2 where not computed), pooled
    [num_tiles][Hkv][max_blocks] (NaN where not computed, -inf where not scored).
    """
    P = prepared or _Prepared(case)
    sh = case.shape
    nt = case.num_tiles
    tl = None if tiles is None else _host_i32(list(tiles))
    out = np.full((case.chunk_len, sh.num_q_heads, sh.head_dim), np.nan, dtype=np.float64)
    sel = np.full((nt, sh.num_kv_heads, sh.top_k), -2, dtype=np.int32)
    pooled = (np.full((nt, sh.num_kv_heads, case.cache.max_blocks), np.nan, dtype=np.float64)
              if want_pooled else None)
    rc = lib().msa_oracle_prefill(ctypes.byref(P.params), ctypes.byref(P.cache), _ptr(P.q),
                                  _ptr(P.idx_q), case.prior_len, case.chunk_len, _ptr(tl),
                                  0 if tl is None else len(tl), _ptr(out), _ptr(sel),
                                  _ptr(pooled))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    return {"out": out, "sel": sel, "pooled": pooled}


def attend_prefill(case, sel, tiles: Optional[Sequence[int]] = None,
                   prepared: Optional[_Prepared] = None) -> np.ndarray:
    """Oracle sparse branch of prefill for a given selection [num_tiles][Hkv][k]."""
    P = prepared or _Prepared(case)
    sh = case.shape
    tl = None if tiles is None else _host_i32(list(tiles))
    s = _host_i32(sel)
    out = np.full((case.chunk_len, sh.num_q_heads, sh.head_dim), np.nan, dtype=np.float64)
    rc = lib().msa_oracle_attend_prefill(ctypes.byref(P.params), ctypes.byref(P.cache),
                                         _ptr(P.q), case.prior_len, case.chunk_len, _ptr(tl),
                                         0 if tl is None else len(tl), _ptr(s), _ptr(out))
    if rc != 0:
        raise ValueError("oracle attend rejected its arguments")
    return out


def select(scores: np.ndarray, own: int, k: int, sink_blocks: int = 0,
           local_blocks: int = 0) -> np.ndarray:
    """The TopK rule alone: scores of blocks 0..own-1 -> sorted selection
    (with forced sink / local blocks when given)."""
    sc = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    sel = np.zeros(k, dtype=np.int32)
    if sink_blocks == 0 and local_blocks == 0:
        rc = lib().msa_oracle_select(_ptr(sc) if own > 0 else None, own, k, _ptr(sel))
    else:
        rc = lib().msa_oracle_select_forced(_ptr(sc) if own > 0 else None, own, k, sink_blocks,
                                            local_blocks, _ptr(sel))
    if rc != 0:
        raise ValueError("oracle select rejected its arguments")
    return sel


def block_scores(case, group: int, blocks: Sequence[int], seq: int = 0, tile: Optional[int] = None,
                 prepared: Optional[_Prepared] = None) -> np.ndarray:
    """Pooled index scores of the listed blocks, for decode sequence ``seq`` or,
    when ``tile`` is given, for that prefill tile."""
    P = prepared or _Prepared(case, kv_pages=[])
    bl = _host_i32(list(blocks))
    out = np.zeros(len(bl), dtype=np.float64)
    if tile is None:
        sh = case.shape
        row = sh.num_kv_heads * sh.num_idx_heads * sh.idx_dim
        iq = P.idx_q.reshape(case.batch, -1)[seq]
        iq = np.ascontiguousarray(iq[:row])
        q0, q1, s = 0, 1, seq
    else:
        iq = P.idx_q
        q0, q1 = tile_rows(case, tile)
        s = 0
    rc = lib().msa_oracle_block_scores(ctypes.byref(P.params), ctypes.byref(P.cache), s, _ptr(iq),
                                       q0, q1, group, _ptr(bl), len(bl), _ptr(out))
    if rc != 0:
        raise ValueError("oracle block_scores rejected its arguments")
    return out


def cache_append(shape, k: np.ndarray, v: np.ndarray, idx_k: np.ndarray, block_table,
                 k_new, v_new, idx_new, start_pos) -> None:
    """Oracle cache append, in place on host arrays of bfloat16 bits (int16).

    k [P][Hkv][B][D], v [P][Hkv][B][D], idx_k [P][B][d_i] (or [P][Hkv][B][d_i]
    with per-group index keys); k_new, v_new [batch][n_new][Hkv][D] and
    idx_new [batch][n_new][d_i] (or [batch][n_new][Hkv][d_i]) (tensors or
    arrays); start_pos [batch]: position of each sequence's first new token.
    """
    params = _Params(shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.num_idx_heads,
                     shape.idx_dim, shape.block_size, shape.top_k, shape.softmax_scale,
                     shape.sink_blocks, shape.local_blocks, shape.idx_k_heads)
    for a in (k, v, idx_k):
        assert a.dtype == np.int16 and a.flags["C_CONTIGUOUS"]
    bt = _host_i32(block_table)
    kn = k_new if isinstance(k_new, np.ndarray) else _host_u16(k_new)
    vn = v_new if isinstance(v_new, np.ndarray) else _host_u16(v_new)
    xn = idx_new if isinstance(idx_new, np.ndarray) else _host_u16(idx_new)
    kn, vn, xn = (np.ascontiguousarray(a) for a in (kn, vn, xn))
    st = _host_i32(start_pos)
    batch, n_new = int(kn.shape[0]), int(kn.shape[1])
    rc = lib().msa_oracle_append(ctypes.byref(params), _ptr(k), _ptr(v), _ptr(idx_k), _ptr(bt),
                                 int(bt.shape[-1]), _ptr(kn), _ptr(vn), _ptr(xn), _ptr(st),
                                 batch, n_new)
    if rc != 0:
        raise ValueError("oracle append rejected its arguments")
