#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

Headline: MSA decode latency per step at a 1,048,576-token context
(decode_b1_L1M: batch 1, 64 query / 8 KV heads, head dim 128, 4 index heads x
64 per group, block 128, top-k 16), one attention layer.  One step is one
msa_decode call: index scores + block max pool, TopK, sparse attention and
the partial merge.  The line also carries the chunked-prefill throughput
(prefill_P1M_C8k: 8192 queries after 1,048,576 tokens) with the MFMA use of
its kernels, the roofline of the dominant decode kernel, and the oracle timed
on the host cores.

Inputs are synthetic and seeded (msa_inputs), generated on the GPU and
resident in HBM before timing.  Decode rotates over several independent
buffer sets (as consecutive layers of a model would) so the 128 MiB of index
keys are never served from the 256 MB Infinity Cache.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, datasheet
DECODE_WORKLOAD = "decode_b1_L1M"
PREFILL_WORKLOAD = "prefill_P1M_C8k"
# the sources the decode index kernel is compiled from (its counters are
# reported only while these are unchanged)
KERNEL_SOURCES = ["block_sparse_long_10_amd/csrc/index_decode.hip",
                  "block_sparse_long_10_amd/csrc/index_block.h",
                  "block_sparse_long_10_amd/csrc/msa_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_index_score_decode_L1M.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the decode index kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def clone_decode_case(case):
    import copy
    c = copy.copy(case)
    c.cache = copy.copy(case.cache)
    c.cache.k = case.cache.k.clone()
    c.cache.v = case.cache.v.clone()
    c.cache.idx_k = case.cache.idx_k.clone()
    c.cache.block_table = case.cache.block_table.clone()
    c.q = case.q.clone()
    c.idx_q = case.idx_q.clone()
    c.seq_lens = case.seq_lens.clone()
    return c


def decode_algorithmic_bytes(case):
    """Bytes a decode step must move at least (per the definition): every
    index key of every eligible block, the K/V of the kept blocks, the
    queries, index queries, block table and the output."""
    sh = case.shape
    B, D, di = sh.block_size, sh.head_dim, sh.idx_dim
    idx_keys = kept_kv = 0
    for L in case.lengths:
        own = (L - 1) // B
        idx_keys += own * B * di * 2
        kept_tokens = min(sh.top_k - 1, own) * B + (L - own * B)
        kept_kv += kept_tokens * D * 2 * 2 * sh.num_kv_heads
    small = (case.q.numel() * 2 + case.idx_q.numel() * 2 + case.cache.block_table.numel() * 4
             + case.batch * sh.num_q_heads * D * 4)
    return idx_keys, kept_kv, small


class _Binding:
    """Parameter and cache descriptors of a seeded case for the C ABI."""

    def __init__(self, msa):
        self.msa = msa

    def params_of(self, sh):
        return self.msa.make_params(sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                                    sh.num_idx_heads, sh.idx_dim, sh.block_size, sh.top_k,
                                    sh.softmax_scale, sh.sink_blocks, sh.local_blocks,
                                    sh.idx_k_heads)

    def kv_of(self, case):
        c = case.cache
        return self.msa.make_kv(c.k, c.v, c.idx_k, c.block_table)


def run_decode_bench(args, torch, msa, mi, gu):
    log("[bench] generating %s x%d buffer sets" % (DECODE_WORKLOAD, args.rotate))
    base = mi.make_workload(DECODE_WORKLOAD, "cuda")
    sets = [base] + [clone_decode_case(base) for _ in range(args.rotate - 1)]
    sh = base.shape
    p = gu.params_of(sh)
    kvs = [gu.kv_of(c) for c in sets]
    batch, maxL, mb = base.batch, max(base.lengths), base.cache.max_blocks
    out = torch.empty(batch, sh.num_q_heads, sh.head_dim, device="cuda")
    sel = torch.empty(batch, sh.num_kv_heads, sh.top_k, dtype=torch.int32, device="cuda")
    ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
                     device="cuda")
    pooled = torch.empty(batch, sh.num_kv_heads, mb, device="cuda")

    def step(i):
        c = sets[i % len(sets)]
        msa.msa_decode(p, kvs[i % len(sets)], c.q, c.idx_q, c.seq_lens, batch, maxL, out, sel, ws)

    def index_only(i):
        c = sets[i % len(sets)]
        msa.msa_index_score_decode(p, kvs[i % len(sets)], c.idx_q, c.seq_lens, batch, maxL,
                                   pooled)

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms

    # decode with the current token's append fused in: each set's own current
    # token is written into its slot again at every step
    kvm = [msa.make_kv_mut(c.cache.k, c.cache.v, c.cache.idx_k, c.cache.block_table) for c in sets]
    cur = [current_token_rows(torch, c) for c in sets]

    def append_step(i):
        c, (kn, vn, xn) = sets[i % len(sets)], cur[i % len(sets)]
        msa.msa_decode_append(p, kvm[i % len(sets)], kn, vn, xn, c.q, c.idx_q, c.seq_lens, batch,
                              maxL, out, sel, ws)

    def per_step(fn, n):
        # events between consecutive steps on the launch stream: one interval per step
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        evs[0].record()
        for i in range(n):
            fn(i)
            evs[i + 1].record()
        torch.cuda.synchronize()
        return sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))

    log("[bench] decode: %d warmup + %d timed steps" % (args.warmup, args.steps))
    ms_step = timed(step, args.steps, args.warmup)
    log("[bench] decode: per-step intervals (one event marker each)")
    ms_each = per_step(step, args.steps)
    log("[bench] decode index kernel alone")
    ms_index = timed(index_only, args.steps, args.warmup)
    log("[bench] decode with the fused append")
    ms_append_step = timed(append_step, args.steps, args.warmup)
    idx_bytes, kv_bytes, small = decode_algorithmic_bytes(base)
    own = (maxL - 1) // sh.block_size
    index_bytes = idx_bytes + base.idx_q.numel() * 2 + base.cache.block_table.numel() * 4 \
        + batch * sh.num_kv_heads * own * 4
    step_bytes = idx_bytes + kv_bytes + small
    return {
        "ms_step": ms_step, "ms_index": ms_index, "index_bytes": index_bytes,
        "step_bytes": step_bytes, "case": base, "sets": sets, "p": p, "kvs": kvs,
        "ms_append_step": ms_append_step, "ms_each": ms_each,
    }


OTHER_DECODE_WORKLOADS = (("decode_b1_L4k", 4), ("decode_b8_L128k", 4), ("decode_paged_b32", 2))


def run_other_decode_bench(args, torch, msa, mi, gu):
    """Step time of the other decode workloads (parity cases; reported for
    context): rotated buffer sets as for the headline, so that the index keys
    are not served from the Infinity Cache where they exceed it."""
    res = {}
    for name, rot in OTHER_DECODE_WORKLOADS:
        log("[bench] decode %s x%d buffer sets" % (name, rot))
        base = mi.make_workload(name, "cuda")
        sets = [base] + [clone_decode_case(base) for _ in range(rot - 1)]
        sh = base.shape
        p = gu.params_of(sh)
        kvs = [gu.kv_of(c) for c in sets]
        batch, maxL, mb = base.batch, max(base.lengths), base.cache.max_blocks
        out = torch.empty(batch, sh.num_q_heads, sh.head_dim, device="cuda")
        sel = torch.empty(batch, sh.num_kv_heads, sh.top_k, dtype=torch.int32, device="cuda")
        ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
                         device="cuda")

        calls = [0]

        def step():
            i = calls[0] % len(sets)
            calls[0] += 1
            c = sets[i]
            msa.msa_decode(p, kvs[i], c.q, c.idx_q, c.seq_lens, batch, maxL, out, sel, ws)

        ms = _timed_ms(torch, step, 50, 5)
        idx_b, kv_b, small = decode_algorithmic_bytes(base)
        total = idx_b + kv_b + small
        res[name] = {"batch": batch, "context_tokens": int(sum(base.lengths)),
                     "us_per_step": round(ms * 1e3, 3), "algorithmic_bytes": total,
                     "gbps": round(total / (ms * 1e-3) / 1e9, 1), "rotated_buffer_sets": rot}
        if args.cpu_budget > 0:
            res[name]["cpu_baseline"] = cpu_baseline(base, max(2.0, args.cpu_budget / 4), name)
        del sets, kvs, base, out, sel, ws
        torch.cuda.empty_cache()
    return res


def current_token_rows(torch, case):
    """k, v [batch][Hkv][D] and idx_k [batch][d_i] of each sequence's current
    token, read out of its page (the rows a decode-with-append call writes)."""
    sh, c = case.shape, case.cache
    B = sh.block_size
    pos = torch.tensor([L - 1 for L in case.lengths], dtype=torch.long, device=c.k.device)
    rows = torch.arange(case.batch, device=c.k.device)
    pages = c.block_table.long()[rows, pos // B]
    slots = pos % B
    return (c.k[pages, :, slots, :].contiguous(), c.v[pages, :, slots, :].contiguous(),
            c.idx_k[pages, slots, :].contiguous())


def run_layers_bench(args, torch, msa, mi, dec):
    """Decode of one token through args.layers MSA layers at the 1M context:
    every layer has its own index keys (so no layer's 128 MiB of index keys is
    served from the Infinity Cache), queries and index queries; the K/V pages
    are shared (each layer reads only its kept blocks, 8 MiB).  The layers run
    eagerly (one msa_decode per layer, back to back) and as one captured HIP
    graph replayed per token; both are reported per layer and per token."""
    base = dec["case"]
    sh = base.shape
    p = dec["p"]
    n = args.layers
    log("[bench] %d-layer decode: generating per-layer index keys" % n)
    c = base.cache
    layers = []
    for l in range(n):
        seed = 1000 + l
        ik = mi.normal_bf16(tuple(c.idx_k.shape), seed, mi.TENSOR_IDS["idx_k"], "cuda")
        q = mi.normal_bf16(tuple(base.q.shape), seed, mi.TENSOR_IDS["q"], "cuda")
        iq = mi.normal_bf16(tuple(base.idx_q.shape), seed, mi.TENSOR_IDS["idx_q"], "cuda")
        layers.append((msa.make_kv(c.k, c.v, ik, c.block_table), q, iq))
    batch, maxL, mb = base.batch, max(base.lengths), c.max_blocks
    outs = torch.empty(n, batch, sh.num_q_heads, sh.head_dim, device="cuda")
    ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
                     device="cuda")

    def token():
        for l, (kv, q, iq) in enumerate(layers):
            msa.msa_decode(p, kv, q, iq, base.seq_lens, batch, maxL, outs[l], None, ws)

    def timed(fn, reps, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = max(1, args.layer_tokens)
    ms_eager = timed(token, reps, 2)
    eager_out = outs.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        token()  # warm the stream before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            token()
    torch.cuda.current_stream().wait_stream(s)
    outs.zero_()
    ms_graph = timed(g.replay, reps, 2)
    same = bool(torch.equal(outs, eager_out))
    log("[bench] %d layers: eager %.1f us/layer, graph %.1f us/layer, replay == eager: %s"
        % (n, ms_eager * 1e3 / n, ms_graph * 1e3 / n, same))
    return {"layers": n, "tokens_timed": reps, "eager_us_per_token": round(ms_eager * 1e3, 2),
            "graph_us_per_token": round(ms_graph * 1e3, 2),
            "eager_us_per_layer": round(ms_eager * 1e3 / n, 3),
            "graph_us_per_layer": round(ms_graph * 1e3 / n, 3),
            "graph_replay_equals_eager": same,
            "note": "per-layer index keys, queries and index queries; K/V pages shared"}


def prefill_algorithmic_flops(sh, P, C):
    """Index flops: every (query, eligible key) pair x all index rows x d_i
    multiply-adds; attention flops: QK and PV over the kept tokens visible to
    each query (exact causal)."""
    B, rows = sh.block_size, sh.num_kv_heads * sh.num_idx_heads
    nt = (P + C + B - 1) // B - P // B
    pairs = 0
    attn_pairs = 0
    for t in range(nt):
        own = P // B + t
        q0, q1 = max(0, own * B - P), min(C, (own + 1) * B - P)
        pairs += (q1 - q0) * own * B
        kept = min(sh.top_k - 1, own) * B
        for i in range(q0, q1):
            attn_pairs += kept + (P + i - own * B + 1)
    return pairs * rows * sh.idx_dim * 2, attn_pairs * sh.num_q_heads * sh.head_dim * 4


def prefill_padded_attn_flops(sh, P, C):
    """Attention flops counted per whole block: every query over its kept
    blocks and its whole diagonal block (the block-granular work, against the
    exact-causal count above)."""
    B = sh.block_size
    nt = (P + C + B - 1) // B - P // B
    pairs = 0
    for t in range(nt):
        own = P // B + t
        q0, q1 = max(0, own * B - P), min(C, (own + 1) * B - P)
        pairs += (q1 - q0) * (min(sh.top_k - 1, own) + 1) * B
    return pairs * sh.num_q_heads * sh.head_dim * 4


def run_prefill_bench(args, torch, msa, mi, gu):
    log("[bench] generating %s" % PREFILL_WORKLOAD)
    case = mi.make_workload(PREFILL_WORKLOAD, "cuda")
    sh = case.shape
    p, kv = gu.params_of(sh), gu.kv_of(case)
    P, C, mb, nt = case.prior_len, case.chunk_len, case.cache.max_blocks, case.num_tiles
    out = torch.empty(C, sh.num_q_heads, sh.head_dim, device="cuda")
    sel = torch.empty(nt, sh.num_kv_heads, sh.top_k, dtype=torch.int32, device="cuda")
    ws = torch.empty(msa.msa_prefill_workspace_bytes(p, P, C, mb), dtype=torch.uint8,
                     device="cuda")
    pooled = torch.empty(nt, sh.num_kv_heads, mb, device="cuda")

    def timed(fn, n, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n, w = args.prefill_steps, args.prefill_warmup
    log("[bench] prefill: %d warmup + %d timed chunks" % (w, n))
    ms_chunk = timed(lambda: msa.msa_prefill_chunk(p, kv, case.q, case.idx_q, P, C, out, sel, ws),
                     n, w)
    ms_index = timed(lambda: msa.msa_index_score_prefill(p, kv, case.idx_q, P, C, pooled), n, w)
    ms_topk = timed(lambda: msa.msa_block_topk_prefill(p, P, C, mb, pooled, sel), n, w)
    ms_attn = timed(lambda: msa.msa_sparse_attn_prefill(p, kv, case.q, P, C, sel, out), n, w)
    # cache append of the chunk (its tokens are rewritten into their own slots)
    B = sh.block_size
    pos = torch.arange(P, P + C, device="cuda")
    pages = case.cache.block_table[0].long()[pos // B]
    slots = pos % B
    k_new = case.cache.k[pages, :, slots, :].contiguous().unsqueeze(0)
    v_new = case.cache.v[pages, :, slots, :].contiguous().unsqueeze(0)
    x_new = case.cache.idx_k[pages, slots, :].contiguous().unsqueeze(0)
    start = torch.tensor([P], dtype=torch.int32, device="cuda")
    kvm = msa.make_kv_mut(case.cache.k, case.cache.v, case.cache.idx_k, case.cache.block_table)
    ms_append = timed(lambda: msa.msa_cache_append(p, kvm, k_new, v_new, x_new, start, 1, C), n, w)
    append_bytes = 2 * C * (2 * sh.num_kv_heads * sh.head_dim * 2 + sh.idx_dim * 2)
    index_flops, attn_flops = prefill_algorithmic_flops(sh, P, C)
    attn_flops_padded = prefill_padded_attn_flops(sh, P, C)
    return {"case": case, "ms_chunk": ms_chunk, "ms_index": ms_index, "ms_topk": ms_topk,
            "ms_attn": ms_attn, "index_flops": index_flops, "attn_flops": attn_flops,
            "attn_flops_padded": attn_flops_padded,
            "ms_append": ms_append, "append_bytes": append_bytes}


def run_varlen_bench(args, torch, msa, mi, gu):
    """Batched prefill over the 32-sequence paged workload: every sequence
    (log-uniform length in [4096, 524288], shuffled pages) prefills its last
    args.varlen_chunk tokens in one msa_prefill_varlen call."""
    w = mi.WORKLOADS["decode_paged_b32"]
    lengths = mi.log_uniform_lengths(w.batch, *w.log_uniform, w.seed)
    C = args.varlen_chunk
    priors = [L - C for L in lengths]
    log("[bench] generating batched prefill over decode_paged_b32 (chunk %d)" % C)
    case = mi.make_varlen_prefill_case(w.shape, priors, [C] * w.batch, w.seed, "cuda",
                                       shuffle_pages=True, poison_frac=w.poison_frac)
    sh = case.shape
    p = gu.params_of(sh)
    c = case.cache
    kv = msa.make_kv(c.k, c.v, c.idx_k, c.block_table)
    rows = C * w.batch
    out = torch.empty(rows, sh.num_q_heads, sh.head_dim, device="cuda")
    ws = torch.empty(msa.msa_prefill_varlen_workspace_bytes(p, priors, [C] * w.batch,
                                                            c.max_blocks),
                     dtype=torch.uint8, device="cuda")
    pd = torch.tensor(priors, dtype=torch.int32, device="cuda")
    cd = torch.tensor([C] * w.batch, dtype=torch.int32, device="cuda")

    def call():
        msa.msa_prefill_varlen(p, kv, case.q, case.idx_q, pd, cd, priors, [C] * w.batch, out,
                               None, ws)

    for _ in range(args.prefill_warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.prefill_steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.prefill_steps
    B = sh.block_size
    pairs = 0
    for P in priors:
        for t in range((P + C + B - 1) // B - P // B):
            own = P // B + t
            q0, q1 = max(0, own * B - P), min(C, (own + 1) * B - P)
            pairs += (q1 - q0) * own * B
    index_flops = pairs * sh.num_kv_heads * sh.num_idx_heads * sh.idx_dim * 2
    return {"workload": "prefill_paged_b32_c%d" % C, "sequences": w.batch, "chunk_len": C,
            "context_tokens": sum(lengths), "ms_per_call": round(ms, 4),
            "tokens_per_s": round(rows / (ms * 1e-3), 1),
            "index_tflops_effective": round(index_flops / (ms * 1e-3) / 1e12, 1)}


def run_group_keys_bench(args, torch, msa, mi, gu):
    """Ablation of the shared index-key head: decode_b1_L1M with one index-key
    head per KV group (8 x 128 MiB of index keys per layer), two buffer sets
    of index keys rotated (the K/V pages are shared)."""
    base = mi.make_workload(DECODE_WORKLOAD, "cuda")
    sh = mi.Shape(num_q_heads=64, num_kv_heads=8, idx_k_heads=8)
    log("[bench] ablation: per-group index keys at 1M")
    c = base.cache
    sets = []
    for r in range(2):
        ik = mi.normal_bf16((c.num_pages, 8, sh.block_size, sh.idx_dim), 300 + r,
                            mi.TENSOR_IDS["idx_k"], "cuda")
        sets.append(msa.make_kv(c.k, c.v, ik, c.block_table))
    p = gu.params_of(sh)
    batch, maxL, mb = base.batch, max(base.lengths), c.max_blocks
    out = torch.empty(batch, sh.num_q_heads, sh.head_dim, device="cuda")
    ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
                     device="cuda")
    pooled = torch.empty(batch, sh.num_kv_heads, mb, device="cuda")

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(20, args.steps // 4)
    ms_step = timed(lambda i: msa.msa_decode(p, sets[i % 2], base.q, base.idx_q, base.seq_lens,
                                             batch, maxL, out, None, ws), n, 5)
    ms_index = timed(lambda i: msa.msa_index_score_decode(p, sets[i % 2], base.idx_q,
                                                          base.seq_lens, batch, maxL, pooled),
                     n, 5)
    own = (maxL - 1) // sh.block_size
    idx_bytes = own * sh.block_size * sh.idx_dim * 2 * 8
    return {"workload": DECODE_WORKLOAD + " with 8 index-key heads",
            "us_per_step": round(ms_step * 1e3, 2),
            "index_kernel_us": round(ms_index * 1e3, 2),
            "index_key_bytes": idx_bytes,
            "index_gbps": round(idx_bytes / (ms_index * 1e-3) / 1e9, 1)}


def _timed_ms(torch, fn, reps, warm):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measured_peaks(torch, msa):
    """The practical roofs, from the library's measurement kernels: a plain
    non-temporal read stream (one wave per 16 KiB chunk, as the decode index
    kernel streams its pages) over 2 GiB, far beyond the 256 MB Infinity
    Cache, and over 128 MiB rotated across four buffers (the size of the
    1M-token index-key stream, launch ramp and tail included); and a loop of
    independent bf16 MFMA chains.  The best launch shape of a small sweep."""
    log("[bench] practical peaks: read stream and bf16 MFMA loop")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nbytes = 1 << 31
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    read = []
    for wg in (8192, 32768, 131072):
        ms = _timed_ms(torch, lambda: msa.msa_probe_read_stream(src, wg, sink), 10, 2)
        read.append((nbytes / (ms * 1e-3) / 1e9, wg))
    del src
    small = 128 << 20
    bufs = [torch.empty(small, dtype=torch.uint8, device="cuda") for _ in range(4)]
    for b in bufs:
        b.fill_(1)
    calls = [0]

    def rotated():
        msa.msa_probe_read_stream(bufs[calls[0] % 4], small // 16384, sink)
        calls[0] += 1

    ms_small = _timed_ms(torch, rotated, 40, 8)
    del bufs
    iters = 4096
    mfma = []
    for wg in (1024, 2048, 4096):
        ms = _timed_ms(torch, lambda: msa.msa_probe_mfma_bf16(iters, wg, sink), 5, 1)
        mfma.append((32768.0 * 16 * iters * wg / (ms * 1e-3) / 1e12, wg))
    (gbps, rwg), (tflops, mwg) = max(read), max(mfma)
    return {"hbm_read_stream_gbps": round(gbps, 1), "read_stream_workgroups": rwg,
            "hbm_read_stream_128mib_gbps": round(small / (ms_small * 1e-3) / 1e9, 1),
            "mfma_bf16_tflops": round(tflops, 1), "mfma_workgroups": mwg,
            "note": "msa_probe_read_stream over 2 GiB, and over 128 MiB rotated over 4 "
                    "buffers (one 16 KiB chunk per workgroup); msa_probe_mfma_bf16 (4 chains "
                    "of v_mfma_f32_32x32x16_bf16 per wave); best of a launch-shape sweep"}


def measured_latency(torch, msa):
    """What one dependent memory round trip and one kernel boundary cost, the
    bound of the decode attention launch (a chain of short dependent steps).
    One lane follows a random single-cycle table (msa_probe_latency_chain,
    vector-memory loads), each call from a fresh random entry, so that no call
    finds the lines of an earlier one in a cache:
      - l2: a 256 KiB table whose whole cycle is walked first in the same
        call (every line then sits in the L2 of the XCD the call runs on);
      - infinity_cache: a 64 MiB table read once by the device beforehand
        (it fits the 256 MB Infinity Cache, not the 4 MB L2 of an XCD);
      - hbm: a 2 GiB table (an eighth of it fits the Infinity Cache).
    The time per load is the difference between calls of 10000 and 2000
    loads (100000 and 20000 for l2), the launch and the warm walk cancelling.  launch_us: the time per launch of
    200 back-to-back one-load launches replayed as a captured HIP graph (no
    host work between them)."""
    import numpy as np
    log("[bench] latency: dependent-load chains and launch cost")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    rng = np.random.default_rng(7)
    res = {}
    for name, nbytes in (("l2", 256 << 10), ("infinity_cache", 64 << 20), ("hbm", 2 << 30)):
        n = nbytes // 4
        perm = torch.randperm(n, device="cuda", generator=gen)
        table = torch.empty(n, dtype=torch.int32, device="cuda")
        table[perm] = torch.roll(perm, -1).to(torch.int32)  # one cycle through all n entries
        del perm
        if name == "infinity_cache":
            torch.sum(table, dtype=torch.int64).item()
        warm = n if name == "l2" else 0

        def chase(k):
            msa.msa_probe_latency_chain(table, warm + k, int(rng.integers(n)), sink)

        ks = (20000, 100000) if name == "l2" else (2000, 10000)
        ms = [_timed_ms(torch, lambda: chase(k), 3, 1) for k in ks]
        res[name + "_ns_per_load"] = round((ms[1] - ms[0]) * 1e6 / (ks[1] - ks[0]), 1)
        del table
    tiny = torch.zeros(1, dtype=torch.int32, device="cuda")
    launches = 200
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        msa.msa_probe_latency_chain(tiny, 1, 0, sink)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for _ in range(launches):
                msa.msa_probe_latency_chain(tiny, 1, 0, sink)
    torch.cuda.current_stream().wait_stream(st)
    res["launch_us"] = round(_timed_ms(torch, g.replay, 5, 2) * 1e3 / launches, 2)
    res["note"] = ("msa_probe_latency_chain: one lane, dependent vector loads through a random "
                   "single-cycle table, a fresh start per call (256 KiB walked whole first in "
                   "the call: L2; 64 MiB read beforehand: Infinity Cache; 2 GiB: mostly HBM); "
                   "ns per load from the difference of two chain lengths; launch_us = time "
                   "per launch of 200 one-load launches in a replayed HIP graph")
    return res


def practical_peaks(torch):
    """What library kernels reach on this machine, for context beside the
    datasheet peaks: a 2 GiB device-to-device copy (bytes read + written per
    second) and an 8192^3 bf16 matrix product (through torch)."""
    log("[bench] library reference: device copy and bf16 GEMM")
    n = 1 << 30  # bf16 elements: 2 GiB
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)

    def timed(fn, reps, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_copy = timed(lambda: b.copy_(a), 10, 2)
    del a, b
    m = 8192
    x = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    ms_mm = timed(lambda: torch.matmul(x, y), 10, 3)
    del x, y
    return {"hbm_copy_gbps": round(2 * 2 * n / (ms_copy * 1e-3) / 1e9, 1),
            "bf16_gemm_tflops": round(2 * m ** 3 / (ms_mm * 1e-3) / 1e12, 1),
            "note": "torch device copy (read + write bytes) and torch.matmul 8192^3 bf16"}


def cpu_model():
    """The host CPU's model name, family/model numbers (which identify the
    generation where the name is generic) and logical core count."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's entry is enough
                key, _, val = line.partition(":")
                info.setdefault(key.strip(), val.strip())
    except OSError:
        pass
    name = info.get("model name", "unknown")
    fam = ("family %s model %s" % (info["cpu family"], info["model"])
           if "cpu family" in info and "model" in info else None)
    return "%s (%s%d logical cores on the host)" % (name, fam + ", " if fam else "",
                                                    os.cpu_count() or 0)


def cpu_baseline(case, budget_s, workload=None):
    """The oracle on the host cores: whole decode steps of the same workload
    (index scores of every block, TopK, attention), repeated for about
    budget_s seconds; K/V pages are copied to the host for the kept blocks."""
    import oracle
    oracle.build()
    workload = workload or DECODE_WORKLOAD
    log("[bench] cpu baseline: oracle decode of %s on the host" % workload)
    P = oracle.prepare(case, kv_pages=[])
    first = oracle.decode(case, prepared=P)
    bt = case.cache.block_table.cpu().numpy()
    pages = {int(bt[s, b]) for s in range(case.batch) for g in range(case.shape.num_kv_heads)
             for b in first["sel"][s, g] if b >= 0}
    P.fill_pages(case, pages)
    times = []
    t_end = time.time() + budget_s
    while time.time() < t_end or not times:
        t0 = time.time()
        oracle.decode(case, prepared=P, want_pooled=False)
        times.append(time.time() - t0)
        if len(times) >= 50:
            break
    times.sort()
    med = times[len(times) // 2]
    return {"value": med * 1e6, "unit": "us/step", "cores": oracle.max_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d full decode steps of %s (median), fp64 C oracle with OpenMP"
                      % (len(times), workload)}


def cpu_prefill_baseline(case, budget_s):
    """The oracle's prefill on the host cores, on a bounded sample of the same
    chunk: whole tiles (index scores of every eligible block, TopK, attention
    of the tile's queries), the first and the last tile, then more tiles while
    the budget lasts, each computed once; the whole K/V cache is copied to the
    host first.  Reported as chunk tokens per second extrapolated from the
    sampled tiles to all of them (an extrapolation)."""
    import oracle
    oracle.build()
    log("[bench] cpu baseline: oracle prefill tiles on the host")
    nt = case.num_tiles
    order = [0, nt - 1] + list(range(1, nt - 1))
    P = oracle.prepare(case)
    done, spent = [], 0.0
    for t in order:
        t0 = time.time()
        oracle.prefill(case, tiles=[t], prepared=P, want_pooled=False)
        spent += time.time() - t0
        done.append(t)
        if len(done) >= 2 and spent >= budget_s:
            break
    per_tile = spent / len(done)
    del P
    return {"value": case.chunk_len / (per_tile * nt), "unit": "tokens/s",
            "cores": oracle.max_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d of %d tiles of %s (%.1f s per tile, each computed once), "
                      "extrapolated to the whole chunk: an extrapolation"
                      % (len(done), nt, PREFILL_WORKLOAD, per_tile)}


COPY_PROBE_BYTES = 128 << 20


def traffic_probe(args, torch, msa, mi, gu):
    """Launches for the FETCH_SIZE / WRITE_SIZE counter runs: a plain device
    copy of COPY_PROBE_BYTES (reads and writes that many bytes), then the
    decode index kernel on rotated buffer sets of decode_b1_L1M."""
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    base = mi.make_workload(DECODE_WORKLOAD, "cuda")
    sets = [base] + [clone_decode_case(base) for _ in range(args.rotate - 1)]
    sh = base.shape
    p = gu.params_of(sh)
    kvs = [gu.kv_of(c) for c in sets]
    pooled = torch.empty(base.batch, sh.num_kv_heads, base.cache.max_blocks, device="cuda")
    for i in range(8):
        c = sets[i % len(sets)]
        msa.msa_index_score_decode(p, kvs[i % len(sets)], c.idx_q, c.seq_lens, base.batch,
                                   max(base.lengths), pooled)
    torch.cuda.synchronize()
    log("[bench] traffic probe done; kernel source hash %s" % kernel_source_hash())


TIMELINE_WORKLOADS = ["decode_b1_L1M", "decode_b8_L128k", "decode_b1_L4k", "decode_paged_b32"]
TIMELINE_LABELS = {
    "index_end": "last decode index workgroup ends",
    "start": "watched attention workgroup starts",
    "scores_in": "selection: length, pooled scores in, thread maxima",
    "range": "selection: range of the maxima (barrier)",
    "bin": "selection: bin of the bound (2 barriers)",
    "counted": "selection: candidates counted (barrier)",
    "gathered": "selection: candidates gathered (barrier)",
    "selected": "selection: worst dropped / sorted, written",
    "block_known": "kept block of the slot known (barrier)",
    "kv_in": "block: page id, K, Q, staged V in",
    "scores": "block: scores and row maxima",
    "softmax": "block: exponentials and row sums",
    "pv": "block: P.V products issued",
    "waves_done": "block: all waves done with V (barrier)",
    "combined": "block: wave outputs in LDS (barrier)",
    "stored": "partial stored (before the store wait)",
    "counted_in": "store wait, hand-off counter back (barrier)",
    "merged": "group 0 merged (its last slot workgroup)",
}


def timeline(args, torch, msa, mi, gu, out_txt, command):
    """Wall-clock marks of one decode attention workgroup (libmsa_timeline.so,
    include/msa_timeline.h): for each workload, warmup + steps msa_decode
    calls on rotated buffer sets, each between a clear and a read of the
    marks (so every call starts on an idle GPU); the table gives the median of
    each mark relative to the watched workgroup's start."""
    import statistics
    lines = ["Decode attention launch: per-workgroup timeline (wall-clock marks)", "",
             "command:", "  " + command, "",
             "Timeline build of the library (libmsa_timeline.so, -DMSA_TIMELINE): thread 0",
             "of the slot-1 workgroup of group 0 of sequence 0 stores the 100 MHz",
             "constant clock (s_memrealtime, 10 ns ticks) at each mark; 'merged' comes",
             "from the workgroup that merges group 0, 'last decode index workgroup ends'",
             "is the latest end over the index launch.  Each call runs on an idle GPU",
             "(the marks are cleared and read around it).  Medians over the timed calls,",
             "in microseconds from the watched workgroup's start; 'step' is the time",
             "since the mark above it.", ""]
    for name in TIMELINE_WORKLOADS:
        base = mi.make_workload(name, "cuda")
        sets = [base] + [clone_decode_case(base) for _ in range(max(0, args.rotate - 1))]
        sh = base.shape
        p = gu.params_of(sh)
        kvs = [gu.kv_of(c) for c in sets]
        batch, maxL, mb = base.batch, max(base.lengths), base.cache.max_blocks
        out = torch.empty(batch, sh.num_q_heads, sh.head_dim, device="cuda")
        sel = torch.empty(batch, sh.num_kv_heads, sh.top_k, dtype=torch.int32, device="cuda")
        ws = torch.zeros(msa.msa_decode_workspace_bytes(p, batch, mb), dtype=torch.uint8,
                         device="cuda")
        rows = []
        for i in range(args.warmup + args.steps):
            c = sets[i % len(sets)]
            msa.msa_timeline_clear()
            msa.msa_decode(p, kvs[i % len(sets)], c.q, c.idx_q, c.seq_lens, batch, maxL, out,
                           sel, ws)
            m = msa.msa_timeline_read()
            if i >= args.warmup:
                rows.append(m)
        del sets, kvs
        torch.cuda.empty_cache()
        log("[bench] timeline %s: %d calls" % (name, len(rows)))
        slots = batch * sh.num_kv_heads * sh.top_k
        lines.append("%s: batch %d, longest row %d blocks, %d slot workgroups, %d timed calls"
                     % (name, batch, (maxL - 1) // sh.block_size, slots, len(rows)))
        lines.append("  %-52s %10s %8s %7s" % ("mark", "since start", "step", "reached"))
        med = {}
        for k in TIMELINE_LABELS:
            d = [(r[k] - r["start"]) / 100.0 for r in rows if r[k] and r["start"]]
            if d:
                med[k] = (statistics.median(d), len(d))
        prev = None
        for k in sorted(med, key=lambda k: med[k][0]):
            t, n = med[k]
            step = "" if prev is None else "%8.2f" % (t - prev)
            lines.append("  %-52s %10.2f %8s %4d/%d" % (TIMELINE_LABELS[k], t, step, n, len(rows)))
            prev = t
        lines.append("")
    if out_txt:
        with open(out_txt, "w") as f:
            f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_PROBE_ITERS, MFMA_PROBE_WORKGROUPS = 1024, 1024


def mfma_probe(args, torch, msa, mi, gu):
    """Launches for the MFMA counter run: the MFMA issue loop (known flops,
    the calibration of SQ_INSTS_VALU_MFMA_MOPS_BF16), then one index, TopK and
    attention launch of prefill_P1M_C8k."""
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    msa.msa_probe_mfma_bf16(MFMA_PROBE_ITERS, MFMA_PROBE_WORKGROUPS, sink)
    torch.cuda.synchronize()
    case = mi.make_workload(PREFILL_WORKLOAD, "cuda")
    sh = case.shape
    p, kv = gu.params_of(sh), gu.kv_of(case)
    P, C, mb, nt = case.prior_len, case.chunk_len, case.cache.max_blocks, case.num_tiles
    out = torch.empty(C, sh.num_q_heads, sh.head_dim, device="cuda")
    sel = torch.empty(nt, sh.num_kv_heads, sh.top_k, dtype=torch.int32, device="cuda")
    pooled = torch.empty(nt, sh.num_kv_heads, mb, device="cuda")
    msa.msa_index_score_prefill(p, kv, case.idx_q, P, C, pooled)
    msa.msa_block_topk_prefill(p, P, C, mb, pooled, sel)
    msa.msa_sparse_attn_prefill(p, kv, case.q, P, C, sel, out)
    torch.cuda.synchronize()
    log("[bench] mfma probe done")


def summarize_mfma(counter_csv, out_txt, command):
    """MFMA work, busy fraction and shader clock per kernel from a counter run
    of --mfma-probe (SQ_INSTS_VALU_MFMA_MOPS_BF16 and _F16,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_CYCLES, GRBM_GUI_ACTIVE, GRBM_COUNT): counted
    flops = MOPS x 512, checked on the issue loop whose flops are known;
    busy = busy cycles / (active cycles x SIMDs); core clock = GRBM_COUNT
    per XCD / dispatch duration (the counter window is a little longer than
    the kernel, so the clock of a short dispatch reads high; it is used, with
    the peak scaled to it, only for dispatches of 5 ms and more).  The
    per-dispatch GRBM counters are sums over the XCDs' GRBM instances, so they
    are divided by the XCD count (Num_Xcc of the run's agent info)."""
    import csv
    import msa_inputs as mi
    n_xcc, n_simd = 8, 1024
    agent_csv = os.path.join(os.path.dirname(counter_csv), "run_agent_info.csv")
    if os.path.exists(agent_csv):
        for r in csv.DictReader(open(agent_csv)):
            if r.get("Name", "").startswith("gfx"):
                n_xcc, n_simd = int(r["Num_Xcc"]), int(r["Simd_Count"])
    w = mi.WORKLOADS[PREFILL_WORKLOAD]
    index_flops, attn_flops = prefill_algorithmic_flops(w.shape, w.prior_len, w.chunk_len)
    B = w.shape.block_size
    known = {"mfma_loop_kernel": 32768.0 * 16 * MFMA_PROBE_ITERS * MFMA_PROBE_WORKGROUPS,
             "index_score_prefill_kernel": float(index_flops),
             "prefill_attn_kernel<%d, true>" % B: float(attn_flops),
             "prefill_attn_kernel<%d, false>" % B: float(attn_flops)}
    rows = {}
    for r in csv.DictReader(open(counter_csv)):
        name = next((k for k in known if k in r["Kernel_Name"]), None)
        if name is None:
            continue
        d = rows.setdefault((name, r["Dispatch_Id"]), {
            "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    lines = ["rocprofv3 MFMA counters (one dispatch each)", "", "command:", "  " + command, "",
             "counted TFLOP = (SQ_INSTS_VALU_MFMA_MOPS_BF16 + _F16) x 512; algorithmic TFLOP "
             "as the bench counts them (exact causal);",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d XCDs x %d SIMDs);"
             % (n_xcc, n_simd),
             "clock = GRBM_COUNT / %d XCDs / duration (GHz; the counter window exceeds the "
             "kernel, so short dispatches read high);" % n_xcc,
             "frac = algorithmic TFLOP/s / 2.5 PFLOP/s dense bf16/fp16 peak (at 2.4 GHz); "
             "frac@clk = the same against that peak scaled to the clock (dispatches >= 5 ms).",
             "",
             "%-32s %10s %9s %7s %7s %9s %7s %7s %8s" % (
                 "kernel", "counted TF", "algo TF", "ratio", "busy %", "us", "clock", "frac",
                 "frac@clk")]
    for (name, _), d in sorted(rows.items()):
        counted = (d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
                   + d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)) * 512
        active = d.get("GRBM_GUI_ACTIVE", 0.0) / n_xcc
        busy = 100.0 * d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(1.0, active * n_simd)
        us = max(d["us"], 1e-3)
        clk = d.get("GRBM_COUNT", 0.0) / n_xcc / us / 1e3       # GHz
        tfs = known[name] / (us * 1e-6) / 1e12
        frac = tfs / BF16_PEAK_TFLOPS
        frac_clk = ("%8.3f" % (tfs / (BF16_PEAK_TFLOPS * clk / 2.4))
                    if clk > 0 and us >= 5000 and counted > 0 else "%8s" % "-")
        lines.append("%-32s %10.4f %9.4f %7.3f %7.1f %9.1f %7.3f %8.3f %s" % (
            name, counted / 1e12, known[name] / 1e12, counted / known[name], busy, us, clk,
            frac if counted > 0 else 0.0, frac_clk))
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_instruction_mix(csv_a, csv_b, out_txt, command):
    """Per-wave instruction mix of the MSA kernels of --mfma-probe from two
    rocprofv3 counter passes (SQ counters; one dispatch each): waves, vector
    instructions other than MFMA, MFMA, transcendental (fp32) and LDS
    instructions per wave and per MFMA, LDS bank-conflict cycles per LDS
    active cycle, and the MFMA busy fraction.  SQ_INSTS_VALU counts the MFMA
    instructions too (the issue loop reads them one for one), so they are
    subtracted."""
    import csv
    n_xcc, n_simd = 8, 1024
    agent_csv = os.path.join(os.path.dirname(csv_a), "run_agent_info.csv")
    if os.path.exists(agent_csv):
        for r in csv.DictReader(open(agent_csv)):
            if r.get("Name", "").startswith("gfx"):
                n_xcc, n_simd = int(r["Num_Xcc"]), int(r["Simd_Count"])
    rows = {}
    for path in (csv_a, csv_b):
        for r in csv.DictReader(open(path)):
            if "msa::" not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("msa::", "")
            d = rows.setdefault(name, {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["rocprofv3 SQ counters: instruction mix per wave (one dispatch of each kernel)", "",
             "commands (two counter passes of the same program):", "  " + command, "",
             "valu = SQ_INSTS_VALU - SQ_INSTS_MFMA (vector instructions other than MFMA); "
             "trans = SQ_INSTS_VALU_TRANS_F32; lds = SQ_INSTS_LDS;",
             "conflict = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS; MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d XCDs x %d SIMDs)" % (n_xcc, n_simd),
             "",
             "%-36s %8s %9s %8s %8s %8s %8s %9s %9s %7s" % (
                 "kernel", "waves", "valu/wv", "mfma/wv", "valu/mf", "trans/mf", "lds/mf",
                 "salu/wv", "conflict", "busy %")]
    for name, d in sorted(rows.items()):
        waves = max(1.0, d.get("SQ_WAVES", 0.0))
        mfma = d.get("SQ_INSTS_MFMA", 0.0)
        valu = d.get("SQ_INSTS_VALU", 0.0) - mfma
        per_mf = (lambda x: "%8.2f" % (x / mfma)) if mfma > 0 else (lambda x: "%8s" % "-")
        lds_act = d.get("SQ_ACTIVE_INST_LDS", 0.0)
        conflict = d.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds_act if lds_act > 0 else 0.0
        active = d.get("GRBM_GUI_ACTIVE", 0.0) / n_xcc
        busy = 100.0 * d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(1.0, active * n_simd)
        lines.append("%-36s %8d %9.0f %8.0f %s %s %s %9.0f %9.3f %7.1f" % (
            name[:36], waves, valu / waves, mfma / waves, per_mf(valu),
            per_mf(d.get("SQ_INSTS_VALU_TRANS_F32", 0.0)), per_mf(d.get("SQ_INSTS_LDS", 0.0)),
            d.get("SQ_INSTS_SALU", 0.0) / waves, conflict, busy))
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_kernel_trace(trace_csv, out_txt, command):
    """Write a short text summary of a rocprofv3 --kernel-trace run: per MSA
    kernel and launch grid (workgroups x, y, z), the dispatch count and the
    average / min / max duration."""
    import csv
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        if "msa::" not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        wg = tuple(int(r["Grid_Size_" + a]) // max(1, int(r["Workgroup_Size_" + a]))
                   for a in "XYZ")
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((name, wg), []).append(us)
    lines = ["rocprofv3 kernel trace (MSA kernels), per kernel and launch grid", "",
             "command:", "  " + command, "",
             "%-60s %-18s %6s %12s %12s %12s" % ("kernel", "workgroups", "calls", "avg us",
                                                  "min us", "max us")]
    for (name, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%-60s %-18s %6d %12.3f %12.3f %12.3f" % (
            name, "%dx%dx%d" % wg, len(v), sum(v) / len(v), min(v), max(v)))
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_kernel_stats(stats_csv, out_txt, command):
    """Write the MSA kernels' rows of a rocprofv3 --stats run (its own
    per-kernel call counts and durations, over every launch grid)."""
    import csv
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        if "msa::" not in r["Name"]:
            continue
        name = r["Name"].split("(")[0].replace("void ", "")
        rows.append((float(r["TotalDurationNs"]), name, int(r["Calls"]),
                     float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                     float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines = ["rocprofv3 --stats (MSA kernels; all launch grids of a kernel together)", "",
             "command:", "  " + command, "",
             "%-60s %6s %12s %12s %12s %8s" % ("kernel", "calls", "avg us", "min us", "max us",
                                              "% time")]
    for _, name, calls, avg, mn, mx, pct in sorted(rows, reverse=True):
        lines.append("%-60s %6d %12.3f %12.3f %12.3f %8.2f" % (name, calls, avg, mn, mx, pct))
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_traffic(fetch_csv, write_csv, out_json, command):
    """HBM bytes per launch of the decode index kernel from FETCH_SIZE and
    WRITE_SIZE runs of --traffic-probe, each scaled by what the counter reads
    for the probe's plain copy of COPY_PROBE_BYTES."""
    import csv
    kib = COPY_PROBE_BYTES / 1024.0

    def load(path, counter):
        copy_vals, kern_vals = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copy_vals.append(v)
            elif "index_score_decode_kernel" in r["Kernel_Name"]:
                kern_vals.append(v)
        return copy_vals[0], sum(kern_vals) / len(kern_vals), len(kern_vals)

    f_copy, f_kern, n = load(fetch_csv, "FETCH_SIZE")
    w_copy, w_kern, _ = load(write_csv, "WRITE_SIZE")
    f_scale, w_scale = kib / f_copy, kib / w_copy
    fetch_b = f_kern * f_scale * 1024.0
    write_b = w_kern * w_scale * 1024.0
    out = {"kernel": "index_score_decode", "workload": DECODE_WORKLOAD,
           "kernel_source_hash": kernel_source_hash(), "command": command,
           "copy_probe_bytes": COPY_PROBE_BYTES,
           "fetch_size_kib_copy": f_copy, "write_size_kib_copy": w_copy,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_size_kib_per_launch": f_kern, "write_size_kib_per_launch": w_kern,
           "launches": n, "hbm_read_bytes_per_launch": round(fetch_b),
           "hbm_write_bytes_per_launch": round(write_b),
           "hbm_bytes_per_launch": round(fetch_b + write_b)}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=4, help="decode buffer sets")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--layers", type=int, default=60,
                    help="layers of the multi-layer decode leg (0 = skip)")
    ap.add_argument("--layer-tokens", type=int, default=20,
                    help="tokens timed in the multi-layer decode leg")
    ap.add_argument("--no-other-decode", action="store_true",
                    help="skip the step times of the other decode workloads")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the per-group index-key ablation leg")
    ap.add_argument("--varlen-chunk", type=int, default=512,
                    help="tokens per sequence of the batched prefill leg (0 = skip)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    ap.add_argument("--summarize-kernel-trace", nargs=3, metavar=("TRACE_CSV", "OUT_TXT", "CMD"),
                    help="write the profiles/ summary of a rocprofv3 kernel-trace run")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON", "CMD"),
                    help="write the profiles/ traffic summary of two counter runs")
    ap.add_argument("--summarize-kernel-stats", nargs=3, metavar=("STATS_CSV", "OUT_TXT", "CMD"),
                    help="write the profiles/ summary of a rocprofv3 --stats run")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("COUNTER_CSV", "OUT_TXT", "CMD"),
                    help="write the profiles/ summary of an MFMA counter run")
    ap.add_argument("--summarize-instruction-mix", nargs=4,
                    metavar=("COUNTER_CSV_A", "COUNTER_CSV_B", "OUT_TXT", "CMD"),
                    help="write the profiles/ instruction-mix summary of two SQ counter runs")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="for rocprofv3 counter runs: the MFMA issue loop (calibration), then "
                         "one index, TopK and attention launch of the 1M prefill; no timing")
    ap.add_argument("--timeline", metavar="OUT_TXT", nargs="?", const="",
                    help="with libmsa_timeline.so: per-workgroup wall-clock marks of the decode "
                         "attention launch (medians over --steps calls after --warmup), "
                         "printed and, given a path, written there; no JSON line")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for rocprofv3 counter runs: one 128 MiB device copy (the "
                         "calibration), then 8 decode index-kernel launches; no timing")
    args = ap.parse_args()
    if args.summarize_kernel_trace:
        summarize_kernel_trace(*args.summarize_kernel_trace)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_instruction_mix:
        summarize_instruction_mix(*args.summarize_instruction_mix)
        return
    if args.summarize_kernel_stats:
        summarize_kernel_stats(*args.summarize_kernel_stats)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_long_10_amd as msa
    import msa_inputs as mi
    gu = _Binding(msa)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.timeline is not None:
        msa.use_timeline_library()
    msa.lib()
    if args.timeline is not None:
        timeline(args, torch, msa, mi, gu, args.timeline,
                 "python bench.py " + " ".join(sys.argv[1:]))
        return
    if args.traffic_probe:
        traffic_probe(args, torch, msa, mi, gu)
        return
    if args.mfma_probe:
        mfma_probe(args, torch, msa, mi, gu)
        return

    dec = run_decode_bench(args, torch, msa, mi, gu)
    lay = run_layers_bench(args, torch, msa, mi, dec) if args.layers > 0 else None
    gk = run_group_keys_bench(args, torch, msa, mi, gu) if not args.no_ablation else None
    other = run_other_decode_bench(args, torch, msa, mi, gu) if not args.no_other_decode else None
    pre = None if args.no_prefill else run_prefill_bench(args, torch, msa, mi, gu)
    var = (run_varlen_bench(args, torch, msa, mi, gu)
           if not args.no_prefill and args.varlen_chunk > 0 else None)
    # after the prefill legs: the MFMA loop and the library GEMM heat the chip,
    # and the prefill index kernel is power-limited
    peaks = practical_peaks(torch)
    roofs = measured_peaks(torch, msa)
    lat = measured_latency(torch, msa)

    case = dec["case"]
    sh = case.shape
    us_step = dec["ms_step"] * 1e3
    index_gbps = dec["index_bytes"] / (dec["ms_index"] * 1e-3) / 1e9
    step_gbps = dec["step_bytes"] / (dec["ms_step"] * 1e-3) / 1e9
    traffic = measured_traffic()
    result = {
        "metric": "MSA decode latency per step at 1M-token context (one attention layer)",
        "value": round(us_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_step"], 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, generated on the GPU)",
        "config": {"workload": DECODE_WORKLOAD, "batch": case.batch, "seq_len": case.lengths[0],
                   "num_q_heads": sh.num_q_heads, "num_kv_heads": sh.num_kv_heads,
                   "head_dim": sh.head_dim, "num_idx_heads": sh.num_idx_heads,
                   "idx_dim": sh.idx_dim, "block_size": sh.block_size, "top_k": sh.top_k,
                   "rotated_buffer_sets": args.rotate},
        "decode_step_gbps": round(step_gbps, 1),
        "decode_step_bytes": dec["step_bytes"],
        "decode_append_us_per_step": round(dec["ms_append_step"] * 1e3, 3),
        "decode_us_per_step_percentiles": dict(
            {q: round(dec["ms_each"][min(len(dec["ms_each"]) - 1, int(f * len(dec["ms_each"])))]
                      * 1e3, 3) for q, f in (("p10", 0.1), ("p50", 0.5), ("p90", 0.9))},
            note="per-call intervals between event markers on the launch stream; each "
                 "includes one marker, which back-to-back steps (value) do not"),
        "roofline": {
            "kernel": "index_score_decode",
            "bound": "hbm",
            "achieved": round(index_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(index_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dec["index_bytes"],
            "avg_launch_us": round(dec["ms_index"] * 1e3, 3),
            "practical_peak": roofs["hbm_read_stream_128mib_gbps"],
            "frac_of_practical": round(index_gbps / roofs["hbm_read_stream_128mib_gbps"], 4),
            "practical_peak_note": "read stream of the same size (128 MiB)",
        },
        "practical_peaks": roofs,
        "latency_probe": lat,
    }
    if pre is not None:
        pc = pre["case"]
        result["prefill"] = {
            "workload": PREFILL_WORKLOAD,
            "prior_len": pc.prior_len, "chunk_len": pc.chunk_len,
            "tokens_per_s": round(pc.chunk_len / (pre["ms_chunk"] * 1e-3), 1),
            "ms_per_chunk": round(pre["ms_chunk"], 4),
            "index_kernel_ms": round(pre["ms_index"], 4),
            "index_tflops": round(pre["index_flops"] / (pre["ms_index"] * 1e-3) / 1e12, 1),
            "index_mfma_frac": round(pre["index_flops"] / (pre["ms_index"] * 1e-3) / 1e12
                                     / BF16_PEAK_TFLOPS, 4),
            "topk_kernel_ms": round(pre["ms_topk"], 4),
            "attn_kernel_ms": round(pre["ms_attn"], 4),
            "attn_tflops": round(pre["attn_flops"] / (pre["ms_attn"] * 1e-3) / 1e12, 1),
            "attn_mfma_frac": round(pre["attn_flops"] / (pre["ms_attn"] * 1e-3) / 1e12
                                    / BF16_PEAK_TFLOPS, 4),
            "index_flops": pre["index_flops"], "attn_flops": pre["attn_flops"],
            "attn_flops_padded": pre["attn_flops_padded"],
            "attn_mfma_frac_padded": round(pre["attn_flops_padded"] / (pre["ms_attn"] * 1e-3)
                                           / 1e12 / BF16_PEAK_TFLOPS, 4),
            "peak_tflops": BF16_PEAK_TFLOPS,
            "practical_peak_tflops": roofs["mfma_bf16_tflops"],
            "index_frac_of_practical": round(pre["index_flops"] / (pre["ms_index"] * 1e-3) / 1e12
                                             / roofs["mfma_bf16_tflops"], 4),
            "attn_frac_of_practical": round(pre["attn_flops"] / (pre["ms_attn"] * 1e-3) / 1e12
                                            / roofs["mfma_bf16_tflops"], 4),
            "chunk_append_us": round(pre["ms_append"] * 1e3, 2),
            "chunk_append_gbps": round(pre["append_bytes"] / (pre["ms_append"] * 1e-3) / 1e9, 1),
        }
    if lay is not None:
        result["multi_layer_decode"] = lay
    if var is not None:
        result["batched_prefill"] = var
    if gk is not None:
        result["ablation_group_index_keys"] = gk
    if other is not None:
        result["other_decode_workloads"] = other
    result["library_reference"] = peaks
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
        if pre is not None:
            result["cpu_baseline_prefill"] = cpu_prefill_baseline(pre["case"], args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
