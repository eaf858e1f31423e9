"""Plant plausible mistakes in a copy of the C oracle and check the pins catch each.

Every mutant is a one-line textual edit of oracle/gqa_oracle.c, compiled with
gcc into a temporary directory and run through ``tests/oracle_pins.py`` in a
child process (a mutant may crash; that counts as caught).  The unmodified
source is run the same way as a control and must pass.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "gqa_oracle.c")

MUTANTS = {
    "modulo_head_map": ("return h / group_size;", "return h % h_kv;"),
    "scale_dropped": ("scores[j] = scale * dot;", "scores[j] = dot;"),
    "causal_off_by_one": ("int n_vis = causal ? first + i + 1 : Lk;",
                          "int n_vis = causal ? first + i : Lk;"),
    "top_left_alignment": ("int n_vis = causal ? first + i + 1 : Lk;",
                           "int n_vis = causal ? i + 1 : Lk;"),
    "softmax_sign": ("scores[j] = exp(scores[j] - m);", "scores[j] = exp(m - scores[j]);"),
    "no_normalisation": ("double p = scores[j] / z;", "double p = scores[j];"),
    "k_v_swapped": ("repeat_kv_slab(k, sb, sj, sh, b, kvh, Lk, d, krep);",
                    "repeat_kv_slab(v, sb, sj, sh, b, kvh, Lk, d, krep);"),
    "transposed_key_index": ("dot += q[c] * krep[(long)j * d + c];",
                             "dot += q[c] * krep[(long)c * n_vis + j];"),
    "decode_reads_whole_cache": ("int n = seqlens[b];", "int n = S;"),
    "append_not_attended": ("grown[b] = seqlens[b] + 1;", "grown[b] = seqlens[b];"),
    "decode_scale_wrong": ("const double scale = 1.0 / sqrt((double)d);",
                           "const double scale = 1.0 / (double)d;"),
    "paged_ignores_table": ("long page = block_table[(long)b * max_blocks + j / page_size];",
                            "long page = (long)b * max_blocks + j / page_size;"),
    "token_major_read_head_major": ("const long sh = d, sj = (long)h_kv * d, sb = (long)S * sj;",
                                    "const long sj = d, sh = (long)S * d, sb = (long)h_kv * sh;"),
    "rope_sin_sign": ("ov[i] = x0 * c - x1 * sn;", "ov[i] = x0 * c + x1 * sn;"),
    "rope_rotate_half_pairs": ("double x0 = xv[2 * i], x1 = xv[2 * i + 1];",
                               "double x0 = xv[i], x1 = xv[half + i];"),
    "rope_keys_not_rotated": ("if (rc == 0) rc = gqa_oracle_rope(k, cos_t, sin_t, k_rot, B, L, h_kv, d);",
                              "if (rc == 0) memcpy(k_rot, k, sizeof(double) * (size_t)B * L * h_kv * d);"),
    "varlen_lengths_ignored": ("if (kv_lens && kv_lens[b] < n_vis) n_vis = kv_lens[b]; /* key padding */",
                               "/* key padding dropped */"),
    "rope_decode_position_off_by_one": ("const long p = seqlens[b];",
                                        "const long p = seqlens[b] > 0 ? seqlens[b] - 1 : 0;"),
    "mask_ignored": ("if (mrow[j] == 0) continue;", "/* keep-mask dropped */"),
    "mask_transposed": ("if (mrow[j] == 0) continue;",
                        "if (j < Lq && mask[((int64_t)b * Lq + j) * (int64_t)Lk + i] == 0) continue;"),
    "mask_causal_dropped": ("if (causal && j > first + i) continue;", "/* causal dropped */"),
    "first_head_of_group_only": ("int kvh = kv_head_of(h, h_q, h_kv);\n                int n = seqlens[b];",
                                 "int kvh = 0;\n                int n = seqlens[b];"),
}


def _build_and_run(tmp_path, source, name):
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"lib{name}.so"
    src.write_text(source)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-ffp-contract=off", str(src), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), str(lib)],
                          capture_output=True, text=True, env=env, timeout=300)


def test_unmutated_oracle_passes_all_pins(tmp_path):
    r = _build_and_run(tmp_path, open(SRC).read(), "control")
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    text = open(SRC).read()
    old, new = MUTANTS[name]
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    r = _build_and_run(tmp_path, text.replace(old, new), name)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout}"
