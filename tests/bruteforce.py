"""Independent numpy brute force of MSA, for pinning the oracle on tiny inputs.

Written from the definition in a different form than the oracle: the paged
cache is first gathered into logical per-sequence arrays, token scores are one
matrix product, block pooling is a reshape + max, TopK is a full sort by
(score descending, block ascending), and attention is a vectorised softmax.
It shares no code with ``oracle/`` and must not import it.
"""
from __future__ import annotations

import numpy as np
import torch


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def logical(case, s: int, length: int):
    """Gather sequence s's first ``length`` tokens: K,V [Hkv][L][D], IK [L][d_i]
    (IK [Hkv][L][d_i] with per-group index keys)."""
    sh, cache = case.shape, case.cache
    B = sh.block_size
    nb = (length + B - 1) // B
    pages = cache.block_table[s, :nb].cpu().numpy().astype(np.int64)
    k = f64(cache.k)[pages]                      # [nb][Hkv][B][D]
    v = f64(cache.v)[pages]                      # [nb][Hkv][B][D]
    ik = f64(cache.idx_k)[pages]                 # [nb][B][d_i] or [nb][Hkv][B][d_i]
    K = k.transpose(1, 0, 2, 3).reshape(sh.num_kv_heads, nb * B, sh.head_dim)[:, :length]
    V = v.transpose(1, 0, 2, 3).reshape(sh.num_kv_heads, nb * B, sh.head_dim)[:, :length]
    if ik.ndim == 4:
        IK = ik.transpose(1, 0, 2, 3).reshape(ik.shape[1], nb * B, sh.idx_dim)[:, :length]
    else:
        IK = ik.reshape(nb * B, sh.idx_dim)[:length]
    return K, V, IK


def topk_sorted(scores: np.ndarray, own: int, k: int, sink: int = 0, local: int = 0) -> np.ndarray:
    """Forced blocks (the first `sink`, the last `local` before own) plus the best
    of the rest by a full sort, plus own; the forced ones count toward k."""
    forced = [b for b in range(own) if b < sink or b >= own - local]
    rest = [b for b in range(own) if b not in forced]
    order = sorted(rest, key=lambda b: (-scores[b], b))
    n = max(0, min(k - 1 - len(forced), len(rest)))
    keep = sorted(forced + order[:n] + [own])
    return np.array(keep + [-1] * (k - len(keep)), dtype=np.int32)


def pool_blocks(tok_scores: np.ndarray, own: int, B: int) -> np.ndarray:
    """tok_scores [rows][L] -> per-block max over rows and tokens, blocks < own."""
    if own == 0:
        return np.zeros(0)
    return tok_scores[:, :own * B].reshape(tok_scores.shape[0], own, B).max(axis=(0, 2))


def softmax_attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    z = scale * (K @ qv)
    w = np.exp(z - z.max())
    return (w / w.sum()) @ V


def tokens_of(sel: np.ndarray, B: int, last_pos: int) -> np.ndarray:
    toks = [np.arange(b * B, (b + 1) * B) for b in sel if b >= 0]
    t = np.concatenate(toks)
    return t[t <= last_pos]


def decode(case):
    sh = case.shape
    B, H, G, k = sh.block_size, sh.num_kv_heads, sh.group_size, sh.top_k
    outs, sels, pools = [], [], []
    for s, L in enumerate(case.lengths):
        K, V, IK = logical(case, s, L)
        own = (L - 1) // B
        qi = f64(case.idx_q[s])                          # [Hkv][n_i][d_i]
        sc = qi @ IK.T if IK.ndim == 2 else qi @ IK.transpose(0, 2, 1)  # [Hkv][n_i][L]
        pooled = [pool_blocks(sc[g], own, B) for g in range(H)]
        sel = np.stack([topk_sorted(pooled[g], own, k, sh.sink_blocks, sh.local_blocks)
                        for g in range(H)])
        q = f64(case.q[s])
        out = np.stack([softmax_attend(q[j], K[j // G][tokens_of(sel[j // G], B, L - 1)],
                                       V[j // G][tokens_of(sel[j // G], B, L - 1)],
                                       sh.softmax_scale)
                        for j in range(sh.num_q_heads)])
        outs.append(out)
        sels.append(sel)
        pools.append(pooled)
    return {"out": np.stack(outs), "sel": np.stack(sels), "pooled": pools}


def prefill(case):
    sh = case.shape
    B, H, G, k = sh.block_size, sh.num_kv_heads, sh.group_size, sh.top_k
    P, C = case.prior_len, case.chunk_len
    K, V, IK = logical(case, 0, P + C)
    qi = f64(case.idx_q)                                 # [C][Hkv][n_i][d_i]
    q = f64(case.q)
    first = P // B
    out = np.zeros((C, sh.num_q_heads, sh.head_dim))
    sels, pools = [], []
    for tau in range(case.num_tiles):
        own = first + tau
        q0, q1 = max(0, own * B - P), min(C, (own + 1) * B - P)
        sel_t, pool_t = [], []
        for g in range(H):
            rows = qi[q0:q1, g].reshape(-1, sh.idx_dim)  # tile queries x heads
            ikg = IK if IK.ndim == 2 else IK[g]
            pooled = pool_blocks(rows @ ikg.T, own, B)
            sel_t.append(topk_sorted(pooled, own, k, sh.sink_blocks, sh.local_blocks))
            pool_t.append(pooled)
        sel_t = np.stack(sel_t)
        for i in range(q0, q1):
            for j in range(sh.num_q_heads):
                t = tokens_of(sel_t[j // G], B, P + i)
                out[i, j] = softmax_attend(q[i, j], K[j // G][t], V[j // G][t], sh.softmax_scale)
        sels.append(sel_t)
        pools.append(pool_t)
    return {"out": out, "sel": np.stack(sels), "pooled": pools}


def attend_decode(case, sel):
    """Sparse branch alone for a given selection sel [batch][Hkv][k] (any valid
    blocks, -1 padded): head j of sequence s over the tokens <= L_s - 1 of
    sel[s][j // G]."""
    sh = case.shape
    B, G = sh.block_size, sh.group_size
    sel = np.asarray(sel)
    outs = []
    for s, L in enumerate(case.lengths):
        K, V, _ = logical(case, s, L)
        q = f64(case.q[s])
        outs.append(np.stack([
            softmax_attend(q[j], K[j // G][tokens_of(sel[s, j // G], B, L - 1)],
                           V[j // G][tokens_of(sel[s, j // G], B, L - 1)], sh.softmax_scale)
            for j in range(sh.num_q_heads)]))
    return np.stack(outs)


def attend_prefill(case, sel, tiles=None):
    """Prefill sparse branch alone for a given selection sel [num_tiles][Hkv][k]:
    every query of the listed tiles (all if None) over the tokens of its
    tile's kept blocks up to its own position.  Rows of other tiles are NaN."""
    sh = case.shape
    B, G = sh.block_size, sh.group_size
    P, C = case.prior_len, case.chunk_len
    K, V, _ = logical(case, 0, P + C)
    q = f64(case.q)
    sel = np.asarray(sel)
    out = np.full((C, sh.num_q_heads, sh.head_dim), np.nan)
    for tau in (range(case.num_tiles) if tiles is None else tiles):
        own = P // B + tau
        for i in range(max(0, own * B - P), min(C, (own + 1) * B - P)):
            for j in range(sh.num_q_heads):
                t = tokens_of(sel[tau, j // G], B, P + i)
                out[i, j] = softmax_attend(q[i, j], K[j // G][t], V[j // G][t], sh.softmax_scale)
    return out


def block_scores(case, group, blocks, seq=0, tile=None):
    """Pooled index scores of the listed blocks: decode sequence ``seq``
    (its index queries), or prefill tile ``tile`` (the queries inside the
    tile's own block)."""
    sh = case.shape
    B = sh.block_size
    blocks = [int(b) for b in blocks]
    nb = max(blocks) + 1 if blocks else 0
    if tile is None:
        _, _, IK = logical(case, seq, nb * B)
        rows = f64(case.idx_q[seq])[group]                   # [n_i][d_i]
    else:
        P, C = case.prior_len, case.chunk_len
        _, _, IK = logical(case, 0, nb * B)
        own = P // B + tile
        q0, q1 = max(0, own * B - P), min(C, (own + 1) * B - P)
        rows = f64(case.idx_q)[q0:q1, group].reshape(-1, sh.idx_dim)
    ikg = IK if IK.ndim == 2 else IK[group]
    tok = rows @ ikg.T                                      # [rows][nb*B]
    return np.array([tok[:, b * B:(b + 1) * B].max() for b in blocks])
