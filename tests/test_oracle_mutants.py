"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one of them (CPU only; the copies are compiled into a temporary
directory and never replace the real oracle)."""
import os
import subprocess

import numpy as np
import pytest

import torch

import oracle
from msa_inputs import Shape, build_paged_cache, make_decode_case, make_prefill_case
from tests.append_util import holed_copy, new_token_batch
from tests.test_oracle_forced import FORCED
from tests.test_oracle_groupkeys import GK
from tests import bruteforce
from tests import test_oracle_given_sel as given_sel
from tests.test_oracle_pins import TINY, TINY1, _by_sort
from tests.test_oracle_pins import test_handworked_golden as _golden

SRC = os.path.join(os.path.dirname(oracle.__file__), "msa_oracle.c")
APPEND_SHAPE = Shape(num_q_heads=4, num_kv_heads=2, num_idx_heads=2, block_size=64, top_k=4)

# (name, text in msa_oracle.c, replacement, replace every occurrence)
MUTANTS = [
    ("index heads not pooled", "for (int64_t row = 0; row < nrows; row++)",
     "for (int64_t row = 0; row < nrows; row += ni)", False),
    ("own block scored", "if (b < own)\n", "if (b <= own)\n", False),
    ("ties keep the higher index", "score[b] > score[best]", "score[b] >= score[best]", False),
    ("values read dimension-major", "return bf(c->v[((pg * H + g) * B + t % B) * D + d]);",
     "return bf(c->v[((pg * H + g) * D + d) * B + t % B]);", False),
    ("softmax scale dropped", "z[i] = p->softmax_scale * dot;", "z[i] = dot;", False),
    ("heads mapped to groups round-robin", "int32_t g = j / G;", "int32_t g = j % H;", True),
    ("one block too few", "int32_t kk = k - 1 - n;", "int32_t kk = k - 2 - n;", False),
    ("current token excluded", "if (hi > last_pos + 1) hi = last_pos + 1;",
     "if (hi > last_pos) hi = last_pos;", True),
    ("block table ignored for index keys",
     "  int64_t pg = page_of(c, seq, t, B);\n  return bf(c->idx_k",
     "  int64_t pg = t / B;\n  return bf(c->idx_k", False),
    ("tile queries not pooled", "block_score(p, c, 0, idx_q, q0, q1, g, b)",
     "block_score(p, c, 0, idx_q, q0, q0 + 1, g, b)", False),
    ("softmax not normalised", "out[d] = acc / den;", "out[d] = acc;", False),
    ("index key dims swapped with query", "dot += qry[row * di + d] * key[r * di + d];",
     "dot += qry[row * di + d] * key[d * B + r];", False),
    ("append writes V dimension-major", "v[((pg * H + g) * B + slot) * D + d] = v_new",
     "v[((pg * H + g) * D + d) * B + slot] = v_new", False),
    ("append slot off by one", "const int64_t slot = t % B;", "const int64_t slot = (t + 1) % B;",
     False),
    ("local window one block short", "if (b < n_sink || b >= own - n_local) {",
     "if (b < n_sink || b > own - n_local) {", False),
    ("sink blocks ignored", "if (b < n_sink || b >= own - n_local) {",
     "if (b < 0 || b >= own - n_local) {", False),
    ("per-group index keys read the shared head", "const int32_t head = Hk > 1 ? g : 0;",
     "const int32_t head = 0;", False),
    ("append ignores the block table",
     "const int64_t pg = block_table[(int64_t)s * max_blocks + t / B];",
     "const int64_t pg = t / B;", False),
    # the entry points that take the caller's selection or query range
    ("given selection read from sequence 0's row",
     "sel + ((int64_t)s * H + g) * k,\n             (int64_t)seq_lens[s] - 1",
     "sel + (int64_t)g * k,\n             (int64_t)seq_lens[s] - 1", False),
    ("prefill query sees one token fewer", "(int64_t)prior_len + qi[r], out",
     "(int64_t)prior_len + qi[r] - 1, out", False),
    ("listed tiles take the selection of their list position", "qi[n] = i; qt[n] = list[u];",
     "qi[n] = i; qt[n] = u;", False),
    ("block scores of sequence 0's pages",
     "out[i] = block_score(p, c, seq, idx_q, q0, q1, g, blocks[i]);",
     "out[i] = block_score(p, c, 0, idx_q, q0, q1, g, blocks[i]);", False),
]

# Mistakes planted in the Python wrapper's slicing (oracle/__init__.py):
# (name, text, replacement)
PY_MUTANTS = [
    ("tile rows start one query late", "    q0 = max(0, own * B - case.prior_len)\n",
     "    q0 = max(0, own * B - case.prior_len) + 1\n"),
    ("decode block scores take sequence 0's index queries",
     "        iq = P.idx_q.reshape(case.batch, -1)[seq]\n",
     "        iq = P.idx_q.reshape(case.batch, -1)[0]\n"),
]


def _pins_pass() -> bool:
    """A compact run of the brute-force, TopK and golden pins."""
    try:
        for shape, lengths, seed, kw in [
                (TINY, [37, 9, 1, 4, 5, 17], 11, {}),
                (TINY, [41, 7, 28, 13], 21, dict(shuffle_pages=True, poison_frac=0.3)),
                (TINY1, [300, 16, 17], 13, {})]:
            case = make_decode_case(shape, lengths, seed, **kw)
            o, r = oracle.decode(case), bruteforce.decode(case)
            np.testing.assert_array_equal(o["sel"], r["sel"])
            for s, L in enumerate(case.lengths):
                own = (L - 1) // shape.block_size
                for g in range(shape.num_kv_heads):
                    np.testing.assert_array_equal(o["pooled"][s, g, :own], r["pooled"][s][g])
                    assert np.all(np.isneginf(o["pooled"][s, g, own:]))
            np.testing.assert_allclose(o["out"], r["out"], rtol=1e-12, atol=1e-12)
        for P, C, seed in [(13, 22, 32), (37, 40, 35)]:
            case = make_prefill_case(TINY, P, C, seed, shuffle_pages=True, poison_frac=0.2)
            o, r = oracle.prefill(case), bruteforce.prefill(case)
            np.testing.assert_array_equal(o["sel"], r["sel"])
            np.testing.assert_allclose(o["out"], r["out"], rtol=1e-12, atol=1e-12)
        rng = np.random.default_rng(5)
        for _ in range(100):
            own, k = int(rng.integers(0, 30)), int(rng.integers(1, 10))
            sc = rng.integers(-3, 4, size=max(own, 1)).astype(np.float64)
            assert oracle.select(sc[:own], own, k).tolist() == _by_sort(sc, own, k)
        _golden()
        _append_pin()
        case = make_decode_case(FORCED, [37, 9, 1, 64], 81, shuffle_pages=True, poison_frac=0.2)
        np.testing.assert_array_equal(oracle.decode(case)["sel"], bruteforce.decode(case)["sel"])
        case = make_decode_case(GK, [37, 9, 64], 111, shuffle_pages=True, poison_frac=0.2)
        o, r = oracle.decode(case), bruteforce.decode(case)
        for s, L in enumerate(case.lengths):
            own = (L - 1) // GK.block_size
            for g in range(GK.num_kv_heads):
                np.testing.assert_array_equal(o["pooled"][s, g, :own], r["pooled"][s][g])
        for shape, lengths, seed, kw in given_sel.DECODE_CASES[:2]:
            given_sel.test_attend_decode_given_selection(shape, lengths, seed, kw)
            given_sel.test_block_scores_decode(shape, lengths, seed, kw)
        for shape, P, C, seed in given_sel.PREFILL_CASES[:2]:
            given_sel.test_attend_prefill_given_selection(shape, P, C, seed)
            given_sel.test_block_scores_prefill(shape, P, C, seed)
        given_sel.test_tile_rows_partial_tiles()
    except AssertionError:
        return False
    return True


def _append_pin():
    """Append into punched-out slots must restore the generated cache."""
    shape = APPEND_SHAPE
    lengths = [300, 200]
    full = build_paged_cache(shape, lengths, seed=17, shuffle_pages=True, poison_frac=0.1)
    starts = [L - 70 - 9 for L in lengths]
    kn, vn, xn = new_token_batch(full, shape, starts, 70)
    hole = holed_copy(full, shape, starts, 70)
    arrays = [np.ascontiguousarray(t.view(torch.int16).numpy()) for t in (hole.k, hole.v, hole.idx_k)]
    oracle.cache_append(shape, *arrays, full.block_table, kn, vn, xn, starts)
    for a, t in zip(arrays, (full.k, full.v, full.idx_k)):
        np.testing.assert_array_equal(a, t.view(torch.int16).numpy())


def test_unmutated_copy_passes(tmp_path):
    lib = tmp_path / "liboracle_copy.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", SRC,
                           "-o", str(lib), "-lm"])
    oracle.use_library(str(lib))
    try:
        assert _pins_pass()
    finally:
        oracle.use_library(None)


@pytest.mark.parametrize("name,old,new,every", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, every):
    text = open(SRC).read()
    assert text.count(old) >= 1, name
    if not every:
        assert text.count(old) == 1, name
    mutated = text.replace(old, new) if every else text.replace(old, new, 1)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = tmp_path / ("libmutant_%d.so" % abs(hash(name)))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(src),
                           "-o", str(lib), "-lm"])
    oracle.use_library(str(lib))
    try:
        assert not _pins_pass(), "pins did not catch: " + name
    finally:
        oracle.use_library(None)


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_pins_catch_planted_wrapper_mistake(monkeypatch, name, old, new):
    """The same for the wrapper's own slicing: a mutated copy of
    oracle/__init__.py is loaded as a separate module and its functions are
    swapped into the oracle module for the duration of the test."""
    import types
    path = oracle.__file__
    text = open(path).read()
    assert text.count(old) == 1, name
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = path
    exec(compile(text.replace(old, new), path, "exec"), mod.__dict__)
    for fn in ("tile_rows", "block_scores", "prefill", "attend_prefill", "attend_decode", "decode"):
        monkeypatch.setattr(oracle, fn, getattr(mod, fn))
    assert not _pins_pass(), "pins did not catch: " + name
