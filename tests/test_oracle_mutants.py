"""The oracle pins must catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a dropped term, a wrong sign
or index, a swapped operand), builds the copy in a temporary directory and runs the pin
suite against it in a subprocess. Every mutant must make the pins fail. CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "paged_attn_oracle.c")

MUTANTS = {
    "head_map_interleaved": ("const int h = g * G + hh;", "const int h = hh * Hkv + g;"),
    "slot_off_by_one": ("size_t src = (((size_t)page * P + (size_t)(t % P)) * Hkv + g) * D;",
                        "size_t src = (((size_t)page * P + (size_t)((t + 1) % P)) * Hkv + g) * D;"),
    "page_table_ignores_request": ("int64_t page = kv_indices[kv_indptr[r] + t / P];",
                                   "int64_t page = kv_indices[t / P];"),
    "causal_top_left": ("const int n = causal ? kv_len - qlen + i + 1 : kv_len;",
                        "const int n = causal ? i + 1 : kv_len;"),
    "no_max_subtraction": ("double p = exp(s[t] - m);", "double p = exp(s[t]);"),
    "no_normaliser": ("        o[d] /= l;\n", "        o[d] /= 1.0;\n"),
    "lse_without_log": ("return m + log(l);", "return m + l;"),
    "merge_weight_sign": ("double w = exp(lj - M);", "double w = exp(M - lj);"),
    "k_v_swapped": ("V[(size_t)t * D + d] = load_elem(v_pool, dtype, src + d);",
                    "V[(size_t)t * D + d] = load_elem(k_pool, dtype, src + d);"),
    "scale_dropped": ("s[t] = scale * acc;", "s[t] = acc;"),
    "last_key_dropped": ("for (int t = t0; t < t1; ++t) {\n        double p",
                         "for (int t = t0; t < t1 - 1; ++t) {\n        double p"),
    "f16_exponent_bias": ("v = ldexp((double)(f | 0x400), e - 25);", "v = ldexp((double)(f | 0x400), e - 24);"),
    # appending new K/V rows
    "append_top_left_positions": ("const int pos = kv_len - qlen + i;", "const int pos = i;"),
    "append_slot_off_by_one": ("((size_t)page * P + (size_t)(pos % P)) * token_bytes",
                               "((size_t)page * P + (size_t)((pos + 1) % P)) * token_bytes"),
    "append_page_ignores_request": ("const int64_t page = kv_indices[kv_indptr[r] + pos / P];",
                                    "const int64_t page = kv_indices[pos / P];"),
    "append_rows_ignore_request": ("const size_t src = (size_t)(row0 + i) * token_bytes;",
                                   "const size_t src = (size_t)i * token_bytes;"),
    # poisoning freed pages
    "poison_k_pool_only": ("            if (!base)\n                continue;\n            const size_t first",
                           "            if (!base || pool)\n                continue;\n            const size_t first"),
    "poison_half_page": ("for (int64_t e = 0; e < page_elems; ++e) {", "for (int64_t e = 0; e < page_elems / 2; ++e) {"),
    "poison_negative_bf16_nan": ("dtype == 1 ? 0x7E00u : 0x7FC0u", "dtype == 1 ? 0x7E00u : 0xFFC0u"),
    # rotary embedding
    "rope_sin_sign": ("y[i1] = x1 * c - x2 * s;", "y[i1] = x1 * c + x2 * s;"),
    "rope_interleaved_pairs": ("const size_t i1 = base + (size_t)i, i2 = base + (size_t)i + (size_t)half;",
                               "const size_t i1 = base + 2 * (size_t)i, i2 = base + 2 * (size_t)i + 1;"),
    "rope_frequency_exponent": ("pow(theta, -2.0 * i / head_dim)", "pow(theta, -1.0 * i / head_dim)"),
    "rope_angle_in_double": ("const float a = (float)positions[r] * f;",
                             "const double a = (double)positions[r] * (double)f;"),
    "rope_position_off_by_one": ("const float a = (float)positions[r] * f;",
                                 "const float a = (float)(positions[r] + 1) * f;"),
    "append_k_v_swapped": ("memcpy((char *)v_pool + dst, (const char *)v_new + src, token_bytes);",
                           "memcpy((char *)v_pool + dst, (const char *)k_new + src, token_bytes);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                           str(lib), str(mpath), "-lm"])
    env = dict(os.environ, FL_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout


def test_unmutated_copy_passes(tmp_path):
    """Control: the same build-and-run route with no planted mistake passes the pins."""
    mpath = tmp_path / "copy.c"
    shutil.copy(SRC, mpath)
    lib = tmp_path / "libcopy.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                           str(lib), str(mpath), "-lm"])
    env = dict(os.environ, FL_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
