"""The oracle pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, index or comparison, a transposed operand), builds it
with the same flags into a temporary library, and runs the whole pin suite
(tests/test_oracle_pins.py) against that library in a child process.  The
suite must fail for every mutant.  The mistakes are planted in the oracle
only, on the CPU; nothing here touches the GPU library.
"""
import os
import subprocess
import sys

import pytest

from oracle.build import SRC, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, original text, planted text): the original must occur exactly once.
MUTANTS = [
    # slot mapping: the new token written at position n instead of n - 1
    ("slot_at_n", "table_stride, n - 1, block_size);", "table_stride, n, block_size);"),
    # store: V rows taken from k_new
    ("store_v_from_k", "memcpy(v_cache + slot * row, v_new + t * row",
     "memcpy(v_cache + slot * row, k_new + t * row"),
    # attention: position's offset inside its block taken as the block index
    ("offset_in_block", "int64_t slot = phys * block_size + j % block_size;",
     "int64_t slot = phys * block_size + j / block_size;"),
    # attention: softmax without subtracting the max
    ("no_max_subtraction", "double w = exp(s[j] - m);", "double w = exp(s[j]);"),
    # attention: interleaved instead of contiguous GQA groups
    ("gqa_interleaved", "                num_kv_heads, h / group, head_dim, block_size, num_blocks,",
     "                num_kv_heads, h % num_kv_heads, head_dim, block_size, num_blocks,"),
    # varlen: new token j misses its own position
    ("varlen_not_inclusive", "cached + j + 1, num_kv_heads,", "cached + j, num_kv_heads,"),
    # sampler: temperature multiplied instead of divided
    ("temperature_times", "s[i] = logits[i] / temperature;", "s[i] = logits[i] * temperature;"),
    # sampler: mask applied to the raw logits before the division by T
    ("mask_before_temperature",
     "        s[i] = logits[i] / temperature;\n        if (mask && !mask[i])\n            s[i] = masked;",
     "        s[i] = ((mask && !mask[i]) ? masked : logits[i]) / temperature;"),
    # sampler: greedy ties to the higher index
    ("greedy_ties_high", "if (v[i] > v[best])", "if (v[i] >= v[best])"),
    # sampler: Gumbel-max ties to the higher index
    ("gumbel_ties_high", "if (best < 0 || key > best_key)", "if (best < 0 || key >= best_key)"),
    # top-k: one token too many
    ("top_k_plus_one", "for (int64_t r = 0; r < top_k; ++r)", "for (int64_t r = 0; r <= top_k && r < vocab; ++r)"),
    # top-k: equal values ordered by the higher index first
    ("top_k_ties_high", "return (a->i > b->i) - (a->i < b->i);", "return (a->i < b->i) - (a->i > b->i);"),
    # nucleus over the whole vocabulary instead of the top-k set
    ("nucleus_over_all_v", "            if (keep[i])\n                asc[n++] = s[i];",
     "            asc[n++] = s[i];"),
    # nucleus: the cumsum compared with p instead of 1 - p
    ("nucleus_target_p", "double target = 1.0 - (double)top_p;", "double target = (double)top_p;"),
    # nucleus: values equal to the threshold dropped
    ("nucleus_strict_tau", "if (keep[i] && !(s[i] >= tau))", "if (keep[i] && !(s[i] > tau))"),
    # margin: only the distance to the upper edge of the threshold group
    ("margin_one_sided", "margin = m1 < m2 ? m1 : m2;", "margin = m2 + 0.0 * m1;"),
    # margin: lower edge taken at the first index reaching 1 - p, not at the
    # start of its tie group
    ("margin_at_for_lo", "double below = lo > 0 ? cum[lo - 1] : 0.0;",
     "double below = at > 0 ? cum[at - 1] : 0.0;"),
]


def _mutate(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: the planted site must occur exactly once"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    # the header sits next to the original source
    (tmp_path / "pkv_oracle.h").write_text(open(os.path.join(os.path.dirname(SRC),
                                                             "pkv_oracle.h")).read())
    return build(src=str(path), out=str(tmp_path / f"liboracle_{name}.so"))


def _run_pins(lib_path):
    env = dict(os.environ, PKV_ORACLE_LIB=lib_path)
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p",
                           "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=300)


def test_pins_pass_on_the_unmodified_source(tmp_path):
    src = open(SRC).read()
    path = tmp_path / "oracle_same.c"
    path.write_text(src)
    (tmp_path / "pkv_oracle.h").write_text(open(os.path.join(os.path.dirname(SRC),
                                                             "pkv_oracle.h")).read())
    lib = build(src=str(path), out=str(tmp_path / "liboracle_same.so"))
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    lib = _mutate(tmp_path, name, old, new)
    r = _run_pins(lib)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-1500:]}"
