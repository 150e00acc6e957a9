"""Helpers of the GPU parity tests: run the HIP path through the C ABI binding
and compare it with the oracle under the stated tolerances.

Tolerances
----------
* pooled index scores (fp32 MFMA sums of 64 exact bf16 products vs fp64):
  |gpu - ref| <= 1e-5 * (|ref| + 8)
* selection: identical to the oracle, except where the oracle's scores at the
  k-th boundary are within 1e-5 relative of each other (near tie); then the
  GPU set must contain every block above the tie band and take the rest from
  the band, and the output is compared with the oracle's attention over the
  GPU's own selection.  Constructed exact ties are checked bit-exactly.
* attention output: per (query, head) row, max|gpu - ref| / max|ref| <= 2e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_long_10_amd as msa

POOLED_RTOL = 1e-5
POOLED_ATOL_SCALE = 8.0
GAP_REL = 1e-5
OUT_ROW_TOL = 2e-3


def params_of(shape):
    return msa.make_params(shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                           shape.num_idx_heads, shape.idx_dim, shape.block_size, shape.top_k,
                           shape.softmax_scale, shape.sink_blocks, shape.local_blocks,
                           shape.idx_k_heads)


def kv_of(case):
    c = case.cache
    return msa.make_kv(c.k, c.v, c.idx_k, c.block_table)


def run_decode(case, with_pooled=True, ws=None):
    sh = case.shape
    p, kv = params_of(sh), kv_of(case)
    dev = case.q.device
    batch, maxL, mb = case.batch, max(case.lengths), case.cache.max_blocks
    out = torch.full((batch, sh.num_q_heads, sh.head_dim), float("nan"), device=dev)
    sel = torch.full((batch, sh.num_kv_heads, sh.top_k), -7, dtype=torch.int32, device=dev)
    if ws is None:  # (contents on entry do not matter; test_gpu_decode checks that)
        ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
                         device=dev)
    msa.msa_decode(p, kv, case.q, case.idx_q, case.seq_lens, batch, maxL, out, sel, ws)
    res = {}
    if with_pooled:
        pooled = torch.full((batch, sh.num_kv_heads, mb), float("nan"), device=dev)
        msa.msa_index_score_decode(p, kv, case.idx_q, case.seq_lens, batch, maxL, pooled)
        res["pooled"] = pooled
    torch.cuda.synchronize()
    res["out"] = out.cpu().numpy().astype(np.float64)
    res["sel"] = sel.cpu().numpy()
    if with_pooled:
        res["pooled"] = res["pooled"].cpu().numpy().astype(np.float64)
    return res


def run_prefill(case):
    sh = case.shape
    p, kv = params_of(sh), kv_of(case)
    dev = case.q.device
    P, C, mb, nt = case.prior_len, case.chunk_len, case.cache.max_blocks, case.num_tiles
    out = torch.full((C, sh.num_q_heads, sh.head_dim), float("nan"), device=dev)
    sel = torch.full((nt, sh.num_kv_heads, sh.top_k), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(msa.msa_prefill_workspace_bytes(p, P, C, mb), dtype=torch.uint8, device=dev)
    msa.msa_prefill_chunk(p, kv, case.q, case.idx_q, P, C, out, sel, ws)
    # the steps one by one, on their own buffers
    pooled = torch.full((nt, sh.num_kv_heads, mb), float("nan"), device=dev)
    msa.msa_index_score_prefill(p, kv, case.idx_q, P, C, pooled)
    sel2 = torch.full_like(sel, -7)
    msa.msa_block_topk_prefill(p, P, C, mb, pooled, sel2)
    torch.cuda.synchronize()
    return {"out": out.cpu().numpy().astype(np.float64), "sel": sel.cpu().numpy(),
            "pooled": pooled.cpu().numpy().astype(np.float64), "sel_steps": sel2.cpu().numpy()}


def check_pooled(gpu, ref, what=""):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    bound = POOLED_RTOL * (np.abs(ref) + POOLED_ATOL_SCALE)
    bad = ~(err <= bound)
    assert not bad.any(), "%s pooled mismatch at %s: gpu %s ref %s" % (
        what, np.argwhere(bad)[:5].tolist(), gpu[bad][:5], ref[bad][:5])
    return float(err.max()) if err.size else 0.0


def check_selection(gpu_row, scores, own, k, exact_only=False, sink=0, local=0):
    """Validate one GPU selection row against the oracle scores of blocks
    0..own-1 (with `sink` leading and `local` trailing blocks forced).
    Returns "exact" or "near-tie"; raises on a wrong selection."""
    g = [int(b) for b in gpu_row]
    forced = [b for b in range(own) if b < sink or b >= own - local]
    elig = [b for b in range(own) if not (b < sink or b >= own - local)]
    keep = min(k - 1 - len(forced), len(elig))
    kept = [b for b in g if b >= 0]
    assert g[len(kept):] == [-1] * (k - len(kept)), "padding is not -1: %s" % g
    assert kept == sorted(kept) and len(set(kept)) == len(kept), "not ascending: %s" % g
    assert len(kept) == len(forced) + keep + 1 and kept[-1] == own, \
        "own block / count wrong: %s (own %d)" % (g, own)
    assert set(forced) <= set(kept), "forced blocks missing: %s" % g
    chosen = sorted(set(kept[:-1]) - set(forced))
    if keep >= len(elig):
        assert chosen == elig, g
        return "exact"
    s = np.asarray(scores[:own], np.float64)
    order = sorted(elig, key=lambda b: (-s[b], b))
    ref = sorted(order[:keep])
    if chosen == ref:
        return "exact"
    assert not exact_only, "selection %s != oracle %s" % (chosen, ref)
    assert keep >= 1
    s_star, s_next = s[order[keep - 1]], s[order[keep]]

    def in_band(x):
        return abs(x - s_star) <= GAP_REL * max(abs(x), abs(s_star))

    assert in_band(s_next), "selection %s != oracle %s and no near tie" % (chosen, ref)
    above = {b for b in elig if s[b] > s_star and not in_band(s[b])}
    band = {b for b in elig if in_band(s[b])}
    assert above <= set(chosen) <= above | band, "near-tie selection invalid: %s" % chosen
    return "near-tie"


def row_errors(gpu_out, ref_out):
    """max|gpu-ref| / max|ref| per (query, head) row over the head dim."""
    gpu_out, ref_out = np.asarray(gpu_out, np.float64), np.asarray(ref_out, np.float64)
    num = np.abs(gpu_out - ref_out).max(axis=-1)
    den = np.abs(ref_out).max(axis=-1)
    return num / den


def check_out(gpu_out, ref_out, what=""):
    e = row_errors(gpu_out, ref_out)
    assert np.isfinite(gpu_out).all(), what + " output has non-finite values"
    worst = float(e.max())
    assert worst <= OUT_ROW_TOL, "%s worst row error %.3g > %.1g" % (what, worst, OUT_ROW_TOL)
    return worst
