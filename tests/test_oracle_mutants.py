"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle.c with one plausible error (a dropped term, a
wrong sign or index, an off-by-one in a mask, a transposed byte order ...),
compiled on the CPU into a temporary library; the pin suite then runs in a
subprocess against it and has to fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "causal_excludes_query_key": ("if (causal && t > q) return 0;", "if (causal && t >= q) return 0;"),
    "window_one_key_wider": ("t < q - window + 1) return 0;", "t < q - window) return 0;"),
    "int8_msb_first": ("(word >> (8u * (uint32_t)lane))", "(word >> (8u * (3u - (uint32_t)lane)))"),
    "int8_wrong_sign_offset": ("(int32_t)byte - 256", "(int32_t)byte - 255"),
    "softcap_drops_cap_factor": ("x = cap * tanh(x / cap);", "x = tanh(x / cap);"),
    "gqa_modulo_map": ("int32_t g = h / (p->num_heads / p->num_kv_heads);", "int32_t g = h % p->num_kv_heads;"),
    "paged_offset_shifted": ("return blk * p->block_size + t % p->block_size;",
                             "return blk * p->block_size + (t + 1) % p->block_size;"),
    "scale_dropped": ("double x = scale * dot;", "double x = dot;"),
    "lse_drops_max": ("*lse = M + log(ell);", "*lse = log(ell);"),
    "f16_subnormal_exponent": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "ring_slot_shifted": ("return t % hot_window;", "return (t + 1) % hot_window;"),
    "sparse_clip_one_block_late": ("if (j >= 0 && j <= r && j < nsel)", "if (j >= 0 && j <= r + 1 && j < nsel)"),
    "sparse_layout_shifted": ("int32_t layout = h % c->num_layouts;", "int32_t layout = (h + 1) % c->num_layouts;"),
    "hot_cold_boundary": ("if (t < s->cold_lens[b]) {", "if (t < s->cold_lens[b] - 1) {"),
    "dot_drops_last_dim": ("for (int32_t d = 0; d < D; ++d) dot += qv[d] * row[d];",
                           "for (int32_t d = 0; d < D - 1; ++d) dot += qv[d] * row[d];"),
    "value_scale_uses_key_scale": ("(is_v ? s->v_scale : s->k_scale)[row]", "s->k_scale[row]"),
    "empty_set_lse_zero": ("*lse = -INFINITY;", "*lse = 0.0;"),
    # the write path
    "evict_next_slot": ("const int64_t slot = orc_ring_slot(C, hot_window);",
                        "const int64_t slot = orc_ring_slot(C + 1, hot_window);"),
    "new_token_next_slot": ("const int64_t slot = orc_ring_slot(L, hot_window);",
                            "const int64_t slot = orc_ring_slot(L + 1, hot_window);"),
    "scale_not_rounded_to_f16": ("const float s = (float)orc_f16_to_f64(s16);", "const float s = s32;"),
    "codes_round_half_away": ("const float r = rintf(", "const float r = roundf("),
    "f16_ties_round_up": ("double r = rint(ldexp(v, 10 - e));", "double r = floor(ldexp(v, 10 - e) + 0.5);"),
    "cold_len_not_advanced": ("      C += 1;\n", "      C += 0;\n"),
    "f16_cold_boundary": ("const int32_t in_cold = t < s->cold_lens[b];", "const int32_t in_cold = t <= s->cold_lens[b];"),
    "f16_cold_drops_kv_head": ("base = (paged_row(p, s->cold_block_table, b, t) * p->num_kv_heads + g) * D;",
                               "base = (paged_row(p, s->cold_block_table, b, t) * p->num_kv_heads) * D;"),
    "f16_hot_slot_from_hot_start": (
        "base = (((int64_t)b * s->hot_window + orc_ring_slot(t, s->hot_window)) * p->num_kv_heads + g) * D;",
        "base = (((int64_t)b * s->hot_window + (t - s->cold_lens[b])) * p->num_kv_heads + g) * D;"),
    "window_ring_slot_shifted": ("const int64_t base = (((int64_t)b * s->ring + t % s->ring)",
                          "const int64_t base = (((int64_t)b * s->ring + (t + 1) % s->ring)"),
    "ring_keeps_one_more": ("if (resident > 0 && t < L - resident) continue;",
                            "if (resident > 0 && t < L - resident - 1) continue;"),
    "ring_residency_ignored": ("if (resident > 0 && t < L - resident) continue;", "(void)resident;"),
    "ring_append_next_slot": ("const int64_t slot = L % W;", "const int64_t slot = (L + 1) % W;"),
    "ring_append_length_kept": ("    seq_lens[b] = (int32_t)(L + 1);\n  }\n  return ORC_OK;\n}\n",
                                "    seq_lens[b] = (int32_t)(L + 0);\n  }\n  return ORC_OK;\n}\n"),
    "mq_all_queries_at_first_position": (
        "return (q_pos ? (int64_t)q_pos[b] : (int64_t)seq_lens[b] - queries(p)) + i;",
        "return (q_pos ? (int64_t)q_pos[b] : (int64_t)seq_lens[b] - queries(p)) + 0 * i;"),
    "mq_default_start_at_last_token": ("(int64_t)seq_lens[b] - queries(p)) + i;", "(int64_t)seq_lens[b] - 1) + i;"),
    "mq_query_rows_transposed": ("int32_t b = bq / Qn, qi = bq % Qn;",
                                 "int32_t b = bq % p->num_seqs, qi = bq / p->num_seqs;"),
    "sparse_negative_query_takes_row_zero": ("if (q < 0) return ORC_OK;", "if (q < 0) q = 0;"),
    "sparse_mq_rows_of_first_query": ("local = sel ? sparse_select(csr, h, qp, sel, nblk) : ORC_ENOMEM;",
                                      "local = sel ? sparse_select(csr, h, query_pos(p, q_pos, seq_lens, b, 0), sel, "
                                      "nblk) : ORC_ENOMEM;"),
}
PIN_FILES = ["test_oracle_pins.py", "test_oracle_append_pins.py", "test_oracle_tiered_f16_pins.py",
             "test_oracle_ring_pins.py", "test_oracle_multi_query_pins.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old}"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-std=c11", "-shared", "-fPIC", str(mut), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in PIN_FILES]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
