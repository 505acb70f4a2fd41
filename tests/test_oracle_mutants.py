"""Planted mistakes in the oracle must fail its pins.

Each mutant is a one-line edit of a copy of ``oracle/lora_oracle.c`` (a
dropped term, a wrong index or sign, a transposed operand, a lost flag, ...),
compiled with gcc into a temporary library and run against
``tests/test_oracle.py`` in a subprocess.  A mutant that every pin accepts
would mean the pins do not pin that part of the oracle.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lora_oracle.c")

MUTANTS = {
    "shrink_drops_first_term": ("for (int32_t h = 0; h < H; ++h) acc +=",
                                "for (int32_t h = 1; h < H; ++h) acc +="),
    "shrink_reversed_index": ("dec[xt[h]] * dec[aj[h]]", "dec[xt[h]] * dec[aj[H - 1 - h]]"),
    "shrink_wrong_adapter": ("A + ((int64_t)id * r + j) * H", "A + ((int64_t)((id + 1) % L) * r + j) * H"),
    "expand_transposed_B": ("acc += vt[j] * dec[bc[j]]",
                            "acc += vt[j] * dec[B[((int64_t)id * r + j) * n + c]]"),
    "expand_wrong_sign": ("acc += vt[j] * dec[bc[j]]", "acc -= vt[j] * dec[bc[j]]"),
    "expand_ignores_add_flag": ("(add ? dec[yt[c]] : 0.0)", "dec[yt[c]]"),
    "expand_drops_last_rank": ("for (int32_t j = 0; j < r; ++j) acc += vt[j]",
                               "for (int32_t j = 0; j < r - 1; ++j) acc += vt[j]"),
    "expand_ignores_col_off": ("y0 + (int64_t)t * ldy + col_off;", "y0 + (int64_t)t * ldy;"),
    "expand_zeroes_inactive_rows": ("for (int32_t c = 0; c < n; ++c) o[c] = dec[yt[c]];",
                                    "for (int32_t c = 0; c < n; ++c) o[c] = 0.0;"),
    "f16_exponent_bias": ("expo - 25);", "expo - 24);"),
    "f16_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "bf16_wrong_half": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "segments_unstable": ("for (int32_t t = 0; t < T; ++t)\n      if (ids[t] == a)",
                          "for (int32_t t = T - 1; t >= 0; --t)\n      if (ids[t] == a)"),
    "segments_bad_not_counted": ("if (ids[t] != -1) ++bad;", ";"),
    "segments_tail_start": ("seg_start[s] = t_active;", "seg_start[s] = 0;"),
    "segments_longest": ("if (len > longest) longest = len;", ";"),
    "rank_bin_16": ("if (r <= 16) return 16;", "if (r <= 8) return 16;"),
    "slice_stride_ignored": ("oracle_expand(dtype, v + s * v_slice_stride,",
                             "oracle_expand(dtype, v,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", str(lib), str(path), "-lm"])
    env = dict(os.environ, LORA_ORACLE_MUTANT_LIB=str(lib), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle.py")],
                         env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} passed every pin:\n{res.stdout[-2000:]}"
