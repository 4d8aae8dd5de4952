"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (on the CPU only),
builds it, and runs the pin tests against it in a subprocess; at least one pin
must fail.  This checks the pins, not the GPU path.

Dropping the exclusion of slots used in the current step from the victim scan
is not a mistake the pins can see: with C >= K, when the i-th of m misses is
served at least m - i slots still have a last-use step below t, so the
oldest slot is never one used in this step.  The exclusion is implied by the
LRU order itself, and that mutant is equivalent.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    # LRU: ties go to the highest slot instead of the lowest
    "lru_tie_to_highest_slot": ("if (best < 0 || c->last[v] < c->last[best]) best = v;",
                                "if (best < 0 || c->last[v] <= c->last[best]) best = v;",
                                "test_oracle_lru.py"),
    # LRU: the evicted position stays in the map
    "lru_keeps_evicted_mapping": ("      c->slot_of[old] = -1;\n", "", "test_oracle_lru.py"),
    # LRU: hits do not refresh their last-use step
    "lru_hits_not_refreshed": ("      c->last[s] = t;\n      ++n_hit;", "      ++n_hit;",
                               "test_oracle_lru.py"),
    # top-K: equal scores go to the higher position
    "topk_ties_to_higher_position": ("return (x->pos > y->pos) - (x->pos < y->pos);",
                                     "return (x->pos < y->pos) - (x->pos > y->pos);",
                                     "test_oracle_topk.py"),
    # top-K: negative scores keep their bit order (wrong totalOrder)
    "topk_wrong_negative_order": ("return (b & 0x80000000u) ? ~b : (b | 0x80000000u);",
                                  "return b ^ 0x80000000u;", "test_oracle_topk.py"),
    # dequant: rounding ties away from zero instead of to even
    "bf16_ties_away": ("if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;",
                       "if (frac >= 0.5) fl += 1.0;", "test_oracle_dequant.py"),
    # dequant: subnormal fp16 scales off by one binade
    "fp16_subnormal_exponent": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);",
                                "test_oracle_dequant.py"),
    # dequant: scale group of 32 instead of 64 values
    "scale_group_of_32": ("    int g = j / 64;", "    int g = (j / 32) & 7;",
                          "test_oracle_format.py"),
    # ring: the copyback moves no bytes
    "ring_copyback_skips_rows": ("    memcpy(host_rows + (size_t)p * ORC_ROW_BYTES, r->data + (size_t)e * ORC_ROW_BYTES,\n           ORC_ROW_BYTES);\n",
                                 "", "test_oracle_ring.py"),
    # ring: rows the ring holds go through the LRU cache anyway
    "ring_rows_through_cache": ("    if (orc_ring_row(ring, p) || c->slot_of[p] >= 0) continue;",
                                "    if (c->slot_of[p] >= 0) continue;", "test_oracle_ring.py"),
    # ring: a batch is copied one append late
    "ring_batch_off_by_one": ("if (r->end - r->copied >= r->batch)",
                              "if (r->end - r->copied > r->batch)", "test_oracle_ring.py"),
    # multi-query round: the union keeps duplicate positions
    "union_keeps_duplicates": ("    if (n == 0 || uni[i] != uni[n - 1]) uni[n++] = uni[i];",
                               "    uni[n++] = uni[i];", "test_oracle_mtp.py"),
    # circular replacement: the hand takes pinned slots too
    "circular_ignores_pins": ("    if (c->last[v] != t) return v;", "    return v;",
                              "test_oracle_replacement.py"),
    # clock replacement: hits do not set the reference bit
    "clock_hits_keep_bit": ("      ++n_hit;\n      c->ref[s] = 1;", "      ++n_hit;",
                            "test_oracle_replacement.py"),
    # clock replacement: a set bit is skipped without being cleared
    "clock_bits_not_cleared": ("    if (c->ref[v]) {\n      c->ref[v] = 0;\n      continue;",
                               "    if (c->ref[v]) {\n      continue;",
                               "test_oracle_replacement.py"),
    # attention: the RoPE values left out of the scores
    "attend_scores_without_rope": ("      for (int d = 0; d < ORC_OUT_ELEMS; ++d) acc += bf16_value(qh[d]) * bf16_value(x[d]);",
                                   "      for (int d = 0; d < 512; ++d) acc += bf16_value(qh[d]) * bf16_value(x[d]);",
                                   "test_oracle_attend.py"),
    # attention: exponentials taken without subtracting the largest score
    "attend_no_max_shift": ("      z[i] = exp(z[i] - zmax);", "      z[i] = exp(z[i]);",
                            "test_oracle_attend.py"),
    # attention: the softmax scale not applied
    "attend_scale_ignored": ("      z[i] = scale * acc;", "      z[i] = acc;", "test_oracle_attend.py"),
    # gather: RoPE read two bytes early
    "rope_offset": ("out[512 + k] = (uint16_t)(row[528 + 2 * k] | (row[528 + 2 * k + 1] << 8));",
                    "out[512 + k] = (uint16_t)(row[526 + 2 * k] | (row[526 + 2 * k + 1] << 8));",
                    "test_oracle_format.py"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new, pin_file = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once"
    mutated = tmp_path / "oracle.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liborc_mutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-D_GNU_SOURCE",
                    "-I", os.path.join(ROOT, "oracle"), "-o", str(lib), str(mutated),
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, pin_file)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "the pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
