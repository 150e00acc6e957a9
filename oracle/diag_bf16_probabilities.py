"""Diagnostic (test infrastructure, CPU only): how much output error does
rounding the softmax probabilities P to bfloat16 cost, on the 1M-context
prefill workload's attention shape?

The sparse branch ("MiniMax wird dünn", section 1, Schritt 2) is exact softmax
attention over the kept blocks.  The GPU kernels feed P to a 16-bit matrix
product (bf16 or IEEE half); this script measures, with copies of the oracle
whose only change is a rounding of P inside the P.V sum, the worst per-row error
max|o - o_exact| / max|o_exact| (the parity metric) for:
  rne        P rounded to nearest-even bf16, denominator exact
  trunc      P truncated to bf16, denominator exact
  rne_den    P rounded to bf16 in both the P.V sum and the denominator
  hi_lo      P as hi + lo, two bf16 terms (hi = rne(P), lo = rne(P - hi))
  fp16       P rounded to nearest-even IEEE half (11 significant bits,
             subnormal below 2^-14), denominator exact
  fp16_den   P rounded to half in both the P.V sum and the denominator
against the unmodified oracle (fp64 throughout).

Inputs: the 1M prefill workload's per-tile attention shape, at a size the
oracle finishes in seconds: 64 query / 8 KV heads, head dim 128, block 128,
top-k 16 (so every query attends to 15 selected blocks plus its causal
diagonal block, 2048 keys at most, as in the 1M chunk), prior length 8192 and
a chunk of 1024 queries (8 tiles), bf16 N(0,1) from seed 4.  The attention
statistics depend only on the per-query key count and the value distribution,
which are the 1M chunk's.

Run:  python -m oracle.diag_bf16_probabilities   (prints one JSON line)
"""
from __future__ import annotations

import json
import os
import subprocess
import sys
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SRC = os.path.join(HERE, "msa_oracle.c")

# the accumulation of the oracle's attend(): every variant rewrites only this
_ANCHOR = ("  double den = 0.0;\n"
           "  for (int64_t i = 0; i < n; i++) { z[i] = exp(z[i] - zmax); den += z[i]; }\n")

_ROUND_HELPERS = r"""
/* bfloat16 rounding of a positive double (8 significant bits) */
static double diag_bf16(double x, int truncate) {
  if (!(x > 0.0)) return x;
  int e;
  frexp(x, &e);                    /* x = m * 2^e, m in [0.5, 1) */
  double ulp = ldexp(1.0, e - 8);  /* spacing of 8-bit significands */
  double q = x / ulp;
  return (truncate ? floor(q) : nearbyint(q)) * ulp;
}
/* IEEE half rounding of a positive double in [0, 1] (11 significant bits;
   below 2^-14 the spacing stays 2^-24) */
static double diag_fp16(double x) {
  if (!(x > 0.0)) return x;
  int e;
  frexp(x, &e);
  if (e < -13) e = -13;            /* subnormal range: fixed spacing 2^-24 */
  double ulp = ldexp(1.0, e - 11);
  return nearbyint(x / ulp) * ulp;
}
"""

VARIANTS = {
    "rne": "  for (int64_t i = 0; i < n; i++) z[i] = diag_bf16(z[i], 0);\n",
    "trunc": "  for (int64_t i = 0; i < n; i++) z[i] = diag_bf16(z[i], 1);\n",
    "rne_den": None,  # rounded before the denominator is summed
    "hi_lo": ("  for (int64_t i = 0; i < n; i++) {\n"
              "    double hi = diag_bf16(z[i], 0);\n"
              "    z[i] = hi + diag_bf16(z[i] - hi, 0);\n"
              "  }\n"),
    "fp16": "  for (int64_t i = 0; i < n; i++) z[i] = diag_fp16(z[i]);\n",
    "fp16_den": None,
}

# variants that round P before the denominator is summed
_ROUND_IN_DEN = {"rne_den": "diag_bf16(exp(z[i] - zmax), 0)",
                 "fp16_den": "diag_fp16(exp(z[i] - zmax))"}


def variant_source(name: str) -> str:
    text = open(SRC).read()
    assert text.count(_ANCHOR) == 1
    if name in _ROUND_IN_DEN:
        new = ("  double den = 0.0;\n"
               "  for (int64_t i = 0; i < n; i++) {\n"
               "    z[i] = %s;\n"
               "    den += z[i];\n"
               "  }\n" % _ROUND_IN_DEN[name])
    else:
        new = _ANCHOR + VARIANTS[name]
    text = text.replace(_ANCHOR, new)
    anchor = "static int64_t page_of("
    return text.replace(anchor, _ROUND_HELPERS + "\n" + anchor, 1)


def build_variant(name: str, outdir: str) -> str:
    src = os.path.join(outdir, "diag_%s.c" % name)
    lib = os.path.join(outdir, "libdiag_%s.so" % name)
    with open(src, "w") as f:
        f.write(variant_source(name))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", src,
                           "-o", lib, "-lm"])
    return lib


def row_errors(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)


def run(prior_len: int = 8192, chunk_len: int = 1024, seed: int = 4) -> dict:
    import oracle
    from msa_inputs import GQA64, make_prefill_case

    case = make_prefill_case(GQA64, prior_len, chunk_len, seed)
    P = oracle.prepare(case)
    exact = oracle.prefill(case, prepared=P)
    sel = exact["sel"]
    res = {"shape": "64/8 heads, D 128, B 128, k 16", "prior_len": prior_len,
           "chunk_len": chunk_len, "rows": int(chunk_len * GQA64.num_q_heads), "bound": 2e-3}
    with tempfile.TemporaryDirectory() as tmp:
        for name in VARIANTS:
            oracle.use_library(build_variant(name, tmp))
            try:
                got = oracle.attend_prefill(case, sel, prepared=P)
            finally:
                oracle.use_library(None)
            e = row_errors(got, exact["out"])
            res[name] = {"worst_row_error": float(e.max()),
                         "rows_over_bound": int((e > 2e-3).sum()),
                         "p99_row_error": float(np.quantile(e, 0.99))}
    return res


if __name__ == "__main__":
    print(json.dumps(run()))
