"""Seeded synthetic inputs for MiniMax Sparse Attention (MSA) decode and prefill.

This module is shared by the test oracle and the HIP path, so it holds none of
the method's arithmetic: it only draws random tensors, builds page tables and
sequence lengths, and applies the structured key shift of the decode-batch
workload.  Every tensor is produced once and then handed to both sides, so the
oracle and the kernels always read identical bits.

Random streams
--------------
Each tensor is drawn from its own stream, keyed by ``(seed, tensor_id)``:
q 0, k 1, v 2, idx_q 3, idx_k 4, lengths 5, page permutation 6, shifted-block
choice 7.
* On the CPU the stream is numpy's counter-based Philox bit generator (4x64,
  10 rounds) with key ``[seed, tensor_id]``; normals come from numpy's
  ``standard_normal`` and are rounded float64 -> float32 -> bfloat16 (round to
  nearest even at each step).  These values are platform independent.
* On a GPU the stream is torch's CUDA generator seeded with
  ``seed * 1_000_003 + tensor_id``; ``torch.randn`` in float32, then rounded
  to bfloat16.  Values differ from the CPU stream; tests copy the GPU tensors
  back to the host for the oracle.
Integer draws (lengths, permutations, shifted blocks) always use the CPU
stream, so page tables and lengths are identical on every device.

Paged layout (one page = one KV block of ``block_size`` tokens)
---------------------------------------------------------------
* ``k``     bf16 ``[num_pages][Hkv][B][D]``   (token-major keys)
* ``v``     bf16 ``[num_pages][Hkv][B][D]``   (token-major values)
* ``idx_k`` bf16 ``[num_pages][B][d_i]``      (one index-key head shared by all groups;
  ``[num_pages][Hkv][B][d_i]`` when the shape asks for one head per group)
* ``block_table`` int32 ``[batch][max_blocks]``: logical block -> physical page
Pages never referenced by a block table ("poison pages") and the slots past a
sequence's last token are filled with ``POISON`` so that any read outside the
valid tokens changes the result.  Unused block-table entries point at a poison
page (never at an invalid id), so a stray read is wrong but never faults.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "idx_q": 3, "idx_k": 4,
              "lengths": 5, "perm": 6, "shift": 7}

POISON = 30000.0  # exactly representable in bfloat16


@dataclasses.dataclass(frozen=True)
class Shape:
    """Head counts and block parameters of one MSA attention layer."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int = 128
    num_idx_heads: int = 4
    idx_dim: int = 64
    block_size: int = 128
    top_k: int = 16
    scale: Optional[float] = None  # softmax scale; None means 1/sqrt(head_dim)
    sink_blocks: int = 0           # blocks always kept from the start of the sequence
    local_blocks: int = 0          # blocks always kept just before the own block
    idx_k_heads: int = 1           # index-key heads: 1 (shared) or num_kv_heads (per group)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return float(self.scale) if self.scale is not None else 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass
class Workload:
    """One named workload: shapes, sizes and the recipe of its inputs."""
    name: str
    kind: str                      # "decode" or "prefill"
    shape: Shape
    seed: int
    batch: int = 1
    seq_len: int = 0               # decode, fixed length
    log_uniform: Optional[tuple] = None  # decode, (lo, hi) lengths
    prior_len: int = 0             # prefill
    chunk_len: int = 0             # prefill
    shuffle_pages: bool = False
    poison_frac: float = 0.0
    shift_frac: float = 0.0
    description: str = ""


GQA64 = Shape(num_q_heads=64, num_kv_heads=8)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("decode_b1_L4k", "decode",
             Shape(num_q_heads=8, num_kv_heads=1, block_size=64, top_k=8),
             seed=1, batch=1, seq_len=4096,
             description="decode, batch 1, L=4096, 8 q heads / 1 KV head, "
                         "B=64, top-k 8"),
    Workload("decode_b8_L128k", "decode", GQA64, seed=2, batch=8,
             seq_len=131072, shift_frac=0.01,
             description="decode, batch 8 x L=131072, 64/8 heads, B=128, "
                         "top-k 16, 1% of blocks shifted +2 sigma"),
    Workload("decode_b1_L1M", "decode", GQA64, seed=3, batch=1,
             seq_len=1048576,
             description="decode, batch 1, L=1,048,576, 64/8 heads, B=128, "
                         "top-k 16"),
    Workload("prefill_P1M_C8k", "prefill", GQA64, seed=4,
             prior_len=1048576, chunk_len=8192,
             description="prefill chunk of 8192 queries after 1,048,576 "
                         "tokens, 64/8 heads, B=128, top-k 16 per tile"),
    Workload("decode_paged_b32", "decode", GQA64, seed=5, batch=32,
             log_uniform=(4096, 524288), shuffle_pages=True,
             poison_frac=0.01,
             description="paged decode, 32 sequences, L log-uniform in "
                         "[4096, 524288], shuffled pages, 1% poison pages"),
]}


def _philox(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(
        key=np.array([seed, tensor_id], dtype=np.uint64)))


def normal_bf16(shape: Sequence[int], seed: int, tensor_id: int,
                device="cpu") -> torch.Tensor:
    """iid N(0,1) values rounded to bfloat16, from stream (seed, tensor_id)."""
    shape = tuple(int(s) for s in shape)
    device = torch.device(device)
    if device.type == "cpu":
        x = _philox(seed, tensor_id).standard_normal(shape, dtype=np.float64)
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + tensor_id)
    n = math.prod(shape)
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    step = 1 << 28
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        out[lo:hi] = torch.randn(hi - lo, generator=gen, device=device,
                                 dtype=torch.float32).to(torch.bfloat16)
    return out.view(shape)


def log_uniform_lengths(batch: int, lo: int, hi: int, seed: int) -> List[int]:
    """L_s = round(lo * (hi/lo)**u_s), u_s ~ U[0,1) from stream (seed, 5)."""
    u = _philox(seed, TENSOR_IDS["lengths"]).random(batch)
    return [int(round(lo * (hi / lo) ** float(x))) for x in u]


@dataclasses.dataclass
class PagedCache:
    k: torch.Tensor
    v: torch.Tensor
    idx_k: torch.Tensor
    block_table: torch.Tensor      # int32 [batch][max_blocks]
    num_pages: int
    max_blocks: int
    lengths: List[int]             # tokens present in the cache per sequence


def build_paged_cache(shape: Shape, lengths: Sequence[int], seed: int,
                      device="cpu", shuffle_pages: bool = False,
                      poison_frac: float = 0.0,
                      max_blocks: Optional[int] = None) -> PagedCache:
    """Random paged K/V/index-key cache holding ``lengths[s]`` tokens each."""
    B = shape.block_size
    nblocks = [(L + B - 1) // B for L in lengths]
    used = sum(nblocks)
    if max_blocks is None:
        max_blocks = max(nblocks)
    assert max_blocks >= max(nblocks)
    n_poison = int(round(poison_frac * used))
    if any(nb < max_blocks for nb in nblocks) and n_poison == 0:
        n_poison = 1  # unused table entries need a harmless target
    num_pages = used + n_poison
    if shuffle_pages:
        perm = _philox(seed, TENSOR_IDS["perm"]).permutation(num_pages)
    else:
        perm = np.arange(num_pages)
    table = np.empty((len(lengths), max_blocks), dtype=np.int32)
    pos = 0
    poison_pages = perm[used:]
    for s, nb in enumerate(nblocks):
        table[s, :nb] = perm[pos:pos + nb]
        table[s, nb:] = poison_pages[0] if n_poison else 0
        pos += nb
    Hkv, D, di = shape.num_kv_heads, shape.head_dim, shape.idx_dim
    k = normal_bf16((num_pages, Hkv, B, D), seed, TENSOR_IDS["k"], device)
    v = normal_bf16((num_pages, Hkv, B, D), seed, TENSOR_IDS["v"], device)
    if shape.idx_k_heads > 1:
        idx_k = normal_bf16((num_pages, shape.idx_k_heads, B, di), seed, TENSOR_IDS["idx_k"],
                            device)
    else:
        idx_k = normal_bf16((num_pages, B, di), seed, TENSOR_IDS["idx_k"], device)
    if n_poison:
        pp = torch.as_tensor(poison_pages, dtype=torch.long, device=k.device)
        k[pp] = POISON
        v[pp] = POISON
        idx_k[pp] = POISON
    for s, L in enumerate(lengths):
        tail = L % B
        if tail:
            page = int(table[s, nblocks[s] - 1])
            k[page, :, tail:, :] = POISON
            v[page, :, tail:, :] = POISON
            idx_k[page, ..., tail:, :] = POISON
    return PagedCache(k=k, v=v, idx_k=idx_k,
                      block_table=torch.from_numpy(table).to(k.device),
                      num_pages=num_pages, max_blocks=max_blocks,
                      lengths=list(lengths))


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm()


def shift_blocks(shape: Shape, cache: PagedCache, idx_q: torch.Tensor,
                 q: torch.Tensor, frac: float, seed: int) -> Dict:
    """Shift the keys of a few blocks toward their group's query direction.

    For each (sequence, group) pick round(frac * c) distinct blocks among the
    blocks before the current one (c = (L-1)//B), and add 2 * (unit vector of
    the group's summed index queries) to every index key in them, and
    2 * (unit vector of the group's summed attention queries) to the group's
    attention keys.  Values are rounded back to bfloat16.  Returns the chosen
    blocks per (sequence, group).
    """
    B, G = shape.block_size, shape.group_size
    rng = _philox(seed, TENSOR_IDS["shift"])
    chosen = {}
    for s, L in enumerate(cache.lengths):
        c = (L - 1) // B
        n = int(round(frac * c))
        for g in range(shape.num_kv_heads):
            if n == 0:
                chosen[(s, g)] = []
                continue
            blocks = sorted(int(b) for b in rng.choice(c, size=n, replace=False))
            chosen[(s, g)] = blocks
            u = _unit(idx_q[s, g].float().sum(0))
            w = _unit(q[s, g * G:(g + 1) * G].float().sum(0))
            pages = cache.block_table[s, blocks].long()
            if cache.idx_k.dim() == 4:  # per-group index keys: this group's head only
                cache.idx_k[pages, g] = (cache.idx_k[pages, g].float() + 2.0 * u).to(torch.bfloat16)
            else:
                cache.idx_k[pages] = (cache.idx_k[pages].float() + 2.0 * u).to(torch.bfloat16)
            cache.k[pages, g] = (cache.k[pages, g].float() + 2.0 * w).to(torch.bfloat16)
    return chosen


@dataclasses.dataclass
class DecodeCase:
    shape: Shape
    cache: PagedCache
    q: torch.Tensor          # bf16 [batch][Hq][D]
    idx_q: torch.Tensor      # bf16 [batch][Hkv][n_i][d_i]
    seq_lens: torch.Tensor   # int32 [batch] (same device as q)
    lengths: List[int]
    shifted: Optional[Dict] = None

    @property
    def batch(self) -> int:
        return len(self.lengths)


@dataclasses.dataclass
class PrefillCase:
    shape: Shape
    cache: PagedCache
    q: torch.Tensor          # bf16 [C][Hq][D]
    idx_q: torch.Tensor      # bf16 [C][Hkv][n_i][d_i]
    prior_len: int
    chunk_len: int

    @property
    def num_tiles(self) -> int:
        B = self.shape.block_size
        return (self.prior_len + self.chunk_len + B - 1) // B - self.prior_len // B


def make_decode_case(shape: Shape, lengths: Sequence[int], seed: int,
                     device="cpu", shuffle_pages=False, poison_frac=0.0,
                     shift_frac=0.0, max_blocks=None) -> DecodeCase:
    lengths = [int(L) for L in lengths]
    assert all(L >= 1 for L in lengths)
    cache = build_paged_cache(shape, lengths, seed, device, shuffle_pages,
                              poison_frac, max_blocks)
    batch = len(lengths)
    q = normal_bf16((batch, shape.num_q_heads, shape.head_dim), seed,
                    TENSOR_IDS["q"], device)
    idx_q = normal_bf16((batch, shape.num_kv_heads, shape.num_idx_heads,
                         shape.idx_dim), seed, TENSOR_IDS["idx_q"], device)
    shifted = None
    if shift_frac > 0:
        shifted = shift_blocks(shape, cache, idx_q, q, shift_frac, seed)
    seq_lens = torch.tensor(lengths, dtype=torch.int32, device=q.device)
    return DecodeCase(shape, cache, q, idx_q, seq_lens, lengths, shifted)


def make_prefill_case(shape: Shape, prior_len: int, chunk_len: int, seed: int,
                      device="cpu", shuffle_pages=False,
                      poison_frac=0.0) -> PrefillCase:
    assert prior_len >= 0 and chunk_len >= 1
    cache = build_paged_cache(shape, [prior_len + chunk_len], seed, device,
                              shuffle_pages, poison_frac)
    q = normal_bf16((chunk_len, shape.num_q_heads, shape.head_dim), seed,
                    TENSOR_IDS["q"], device)
    idx_q = normal_bf16((chunk_len, shape.num_kv_heads, shape.num_idx_heads,
                         shape.idx_dim), seed, TENSOR_IDS["idx_q"], device)
    return PrefillCase(shape, cache, q, idx_q, prior_len, chunk_len)


@dataclasses.dataclass
class VarlenPrefillCase:
    """Chunks of several sequences for one batched prefill call: sequence s has
    prior_lens[s] cached tokens before its chunk of chunk_lens[s] queries; the
    chunks' rows of q / idx_q are packed sequence after sequence."""
    shape: Shape
    cache: PagedCache            # lengths[s] = prior_lens[s] + chunk_lens[s]
    q: torch.Tensor              # bf16 [total_rows][Hq][D]
    idx_q: torch.Tensor          # bf16 [total_rows][Hkv][n_i][d_i]
    prior_lens: List[int]
    chunk_lens: List[int]

    @property
    def batch(self) -> int:
        return len(self.prior_lens)

    @property
    def q_start(self) -> List[int]:
        out, acc = [], 0
        for c in self.chunk_lens:
            out.append(acc)
            acc += c
        return out

    def num_tiles_of(self, s: int) -> int:
        B = self.shape.block_size
        P, C = self.prior_lens[s], self.chunk_lens[s]
        return (P + C + B - 1) // B - P // B

    def sequence(self, s: int) -> PrefillCase:
        """Sequence s alone, as a one-sequence prefill case sharing the tensors."""
        c = self.cache
        one = PagedCache(k=c.k, v=c.v, idx_k=c.idx_k, block_table=c.block_table[s:s + 1],
                         num_pages=c.num_pages, max_blocks=c.max_blocks,
                         lengths=[c.lengths[s]])
        r0, n = self.q_start[s], self.chunk_lens[s]
        return PrefillCase(self.shape, one, self.q[r0:r0 + n], self.idx_q[r0:r0 + n],
                           self.prior_lens[s], n)


def make_varlen_prefill_case(shape: Shape, prior_lens: Sequence[int], chunk_lens: Sequence[int],
                             seed: int, device="cpu", shuffle_pages=False,
                             poison_frac=0.0) -> VarlenPrefillCase:
    priors, chunks = [int(p) for p in prior_lens], [int(c) for c in chunk_lens]
    assert len(priors) == len(chunks) and all(p >= 0 for p in priors) and all(c >= 1 for c in chunks)
    cache = build_paged_cache(shape, [p + c for p, c in zip(priors, chunks)], seed, device,
                              shuffle_pages, poison_frac)
    rows = sum(chunks)
    q = normal_bf16((rows, shape.num_q_heads, shape.head_dim), seed, TENSOR_IDS["q"], device)
    idx_q = normal_bf16((rows, shape.num_kv_heads, shape.num_idx_heads, shape.idx_dim), seed,
                        TENSOR_IDS["idx_q"], device)
    return VarlenPrefillCase(shape, cache, q, idx_q, priors, chunks)


def make_workload(name: str, device="cpu"):
    """Inputs of a named workload of ``WORKLOADS``."""
    w = WORKLOADS[name]
    if w.kind == "prefill":
        return make_prefill_case(w.shape, w.prior_len, w.chunk_len, w.seed,
                                 device, w.shuffle_pages, w.poison_frac)
    if w.log_uniform is not None:
        lengths = log_uniform_lengths(w.batch, *w.log_uniform, w.seed)
    else:
        lengths = [w.seq_len] * w.batch
    return make_decode_case(w.shape, lengths, w.seed, device, w.shuffle_pages,
                            w.poison_frac, w.shift_frac)
