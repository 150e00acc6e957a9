"""The benchmark's measurement arithmetic on the CPU: algorithmic bytes and
flops against independent counts and the figures of the 1M workloads, the
counter-scaling of the traffic summary, the source-hash gate of the traffic
figure, and the refusal of a multi-GPU run."""
import json
import os
import subprocess
import sys
import types

import pytest
import torch

import bench
from msa_inputs import GQA64, WORKLOADS, Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _prefill_counts_by_query(sh, P, C):
    """(index pairs, attention pairs) counted query by query: query i sits at
    position P + i in absolute block c = (P + i) // B; it scores every key of
    blocks 0 .. c-1 and attends to the kept blocks' keys up to its position."""
    B, idx_pairs, att_pairs = sh.block_size, 0, 0
    for i in range(C):
        pos = P + i
        c = pos // B
        idx_pairs += c * B
        att_pairs += min(sh.top_k - 1, c) * B + (pos - c * B + 1)
    return idx_pairs, att_pairs


@pytest.mark.parametrize("P,C,B,k", [(0, 1, 64, 4), (0, 300, 64, 8), (1000, 700, 128, 16),
                                     (4096, 512, 128, 3), (77, 1, 128, 16)])
def test_prefill_flops_match_a_count_by_query(P, C, B, k):
    sh = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=B, top_k=k)
    idx, att = bench.prefill_algorithmic_flops(sh, P, C)
    ip, ap = _prefill_counts_by_query(sh, P, C)
    rows = sh.num_kv_heads * sh.num_idx_heads
    assert idx == ip * rows * sh.idx_dim * 2
    assert att == ap * sh.num_q_heads * sh.head_dim * 4


@pytest.mark.parametrize("P,C,B,k", [(0, 1, 64, 4), (0, 300, 64, 8), (1000, 700, 128, 16),
                                     (77, 1, 128, 16)])
def test_padded_attention_flops_count_whole_blocks(P, C, B, k):
    # query i in absolute block c: its kept blocks and its whole diagonal block
    sh = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=B, top_k=k)
    pairs = sum((min(k - 1, (P + i) // B) + 1) * B for i in range(C))
    padded = bench.prefill_padded_attn_flops(sh, P, C)
    assert padded == pairs * sh.num_q_heads * sh.head_dim * 4
    assert padded >= bench.prefill_algorithmic_flops(sh, P, C)[1]


def test_prefill_flops_of_the_1m_chunk():
    # 8,622,964,736 query-key pairs x 32 index rows x 128 flop = 35.32 TFLOP;
    # sparse attention 0.5327 TFLOP exact-causal
    w = WORKLOADS["prefill_P1M_C8k"]
    idx, att = bench.prefill_algorithmic_flops(w.shape, w.prior_len, w.chunk_len)
    assert idx == 8_622_964_736 * 32 * 128 == 35_319_663_558_656
    assert att == 532_710_162_432


def _meta_case(shape, lengths, max_blocks):
    batch = len(lengths)
    m = torch.device("meta")
    return types.SimpleNamespace(
        shape=shape, lengths=lengths, batch=batch,
        q=torch.empty(batch, shape.num_q_heads, shape.head_dim, device=m),
        idx_q=torch.empty(batch, shape.num_kv_heads, shape.num_idx_heads, shape.idx_dim, device=m),
        cache=types.SimpleNamespace(block_table=torch.empty(batch, max_blocks, device=m)))


def test_decode_bytes_of_the_1m_step():
    # index keys of the 8191 scored blocks, K/V of 15 kept blocks plus the own
    # block (2048 tokens), q, idx_q, block table and the fp32 output
    case = _meta_case(GQA64, [1 << 20], 8192)
    idx, kv, small = bench.decode_algorithmic_bytes(case)
    assert idx == 8191 * 128 * 64 * 2 == 134_201_344
    assert kv == 2048 * 128 * 2 * 2 * 8 == 8_388_608
    assert small == 64 * 128 * 2 + 8 * 4 * 64 * 2 + 8192 * 4 + 64 * 128 * 4
    assert idx + kv + small == 142_675_968


def test_decode_bytes_of_short_and_partial_sequences():
    sh = Shape(num_q_heads=16, num_kv_heads=2, num_idx_heads=4, block_size=64, top_k=8)
    case = _meta_case(sh, [1, 64, 65, 1000], 20)
    idx, kv, _ = bench.decode_algorithmic_bytes(case)
    owns = [0, 0, 1, 15]
    assert idx == sum(o * 64 * 64 * 2 for o in owns)
    kept = [1, 64, 64 + 1, 7 * 64 + (1000 - 15 * 64)]
    assert kv == sum(t * 128 * 2 * 2 * 2 for t in kept)


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for name, v in rows:
            f.write('"%s","%s",%r\n' % (name, counter, v))


def test_traffic_summary_scales_by_the_copy(tmp_path):
    fetch, write, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    kib = bench.COPY_PROBE_BYTES / 1024
    # FETCH_SIZE reads half of the copy's bytes, WRITE_SIZE all of them
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", kib / 2)] +
                 [("void msa::index_score_decode_kernel<128, 4, 2, false>(...)", 1000.0)] * 4)
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", kib)] +
                 [("void msa::index_score_decode_kernel<128, 4, 2, false>(...)", 10.0)] * 4)
    bench.summarize_traffic(str(fetch), str(write), str(out), "cmd")
    t = json.load(open(out))
    assert t["launches"] == 4
    assert t["hbm_read_bytes_per_launch"] == 2 * 1000 * 1024
    assert t["hbm_write_bytes_per_launch"] == 10 * 1024
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


def test_instruction_mix_summary_subtracts_mfma_from_valu(tmp_path):
    a, b, out = tmp_path / "a.csv", tmp_path / "b.csv", tmp_path / "mix.txt"
    k = "void msa::prefill_attn_kernel<128, true>(...)"
    # two waves: 100 vector instructions of which 20 MFMA; 10 transcendental,
    # 30 LDS; 5 conflict cycles over 50 LDS active cycles
    with open(a, "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for c, v in [("SQ_INSTS_VALU", 100.0), ("SQ_INSTS_LDS", 30.0),
                     ("SQ_LDS_BANK_CONFLICT", 5.0), ("SQ_ACTIVE_INST_LDS", 50.0)]:
            f.write('"%s","%s",%r\n' % (k, c, v))
    with open(b, "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for c, v in [("SQ_INSTS_MFMA", 20.0), ("SQ_INSTS_VALU_TRANS_F32", 10.0),
                     ("SQ_WAVES", 2.0), ("SQ_INSTS_SALU", 8.0)]:
            f.write('"%s","%s",%r\n' % (k, c, v))
    bench.summarize_instruction_mix(str(a), str(b), str(out), "cmd")
    row = [l for l in open(out) if l.startswith("prefill_attn_kernel<128, true>")][0].split()
    # waves, valu/wave, mfma/wave, valu/mfma, trans/mfma, lds/mfma, salu/wave, conflict, busy
    assert row[-9:] == ["2", "40", "10", "4.00", "0.50", "1.50", "4", "0.100", "0.0"]


def test_traffic_figure_is_dropped_when_the_kernel_source_changed(tmp_path, monkeypatch):
    f = tmp_path / "t.json"
    json.dump({"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 5}, open(f, "w"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() == 5
    json.dump({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 5}, open(f, "w"))
    assert bench.measured_traffic() is None


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
