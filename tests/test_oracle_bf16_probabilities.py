"""The bf16-probability diagnostic (oracle/diag_bf16_probabilities.py) on one
tile of the 1M prefill workload's attention shape (CPU only): rounding the
softmax probabilities to bfloat16 alone, by nearest-even or by truncation,
breaks the 2e-3 per-row bound, while the two-term hi + lo form (the decode
kernels') stays far inside it, and so does a single IEEE half (11
significant bits; the prefill kernel's form, with the rounded values also in
the denominator).  The full run (8 tiles, 65,536 rows) is the figure quoted
with the kernels."""
from oracle import diag_bf16_probabilities as diag


def test_bf16_probabilities_need_two_terms():
    r = diag.run(prior_len=8192, chunk_len=128, seed=4)
    assert r["rne"]["worst_row_error"] > 2e-3
    assert r["trunc"]["worst_row_error"] > 2e-3
    assert r["rne_den"]["worst_row_error"] > 2e-3
    assert r["hi_lo"]["worst_row_error"] < 2e-5
    assert r["fp16"]["worst_row_error"] < 1e-3
    assert r["fp16_den"]["worst_row_error"] < 1e-3
