"""The oracle's pins catch plausible mistakes.

Each case copies oracle/pa_oracle.c, plants one mistake (a wrong head
mapping, a dropped scale, an untruncated tail, a transposed index, ...),
builds the copy and runs the oracle pin tests against it in a child process
(PA_ORACLE_LIB points the oracle at the copy).  Every planted mistake must
make at least one pin fail.  Nothing here touches the GPU library.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")

MUTANTS = {
    "gqa_head_mapping": ("kv = h / G;", "kv = h % Hkv;"),
    "dropped_scale": ("z[t] = scale * acc;", "z[t] = acc;"),
    "untruncated_tail": ("for (int64_t t = 0; t < L; ++t) {\n            double acc",
                         "for (int64_t t = 0; t < L + (L % bs ? 1 : 0); ++t) {\n            double acc"),
    "block_offset_transposed": ("((phys * bs + t) * Hkv + kv) * D + d",
                                "((t * NB + phys) * Hkv + kv) * D + d"),
    "table_transposed": ("block_tables[s * max_nb + j]", "block_tables[j * S + s]"),
    "k_used_as_v": ("o[d] += z[t] * V[t * D + d];", "o[d] += z[t] * K[t * D + d];"),
    "unnormalised": ("z[t] /= denom;", "z[t] /= 1.0;"),
    "v_takes_k_scale": ("? v_scale : 1.0", "? k_scale : 1.0"),
    "query_index": ("qbase = (s * H + h) * D", "qbase = (h * S + s) * D"),
    "e4m3_subnormal_bias": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "e4m3_ties_away": ("pick = (c & 1) ? c + 1 : c;", "pick = c + 1;"),
    "e4m3_nan_saturates": ("return sign | 0x7F;\n    double a", "return sign | 0x7E;\n    double a"),
    "bf16_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "append_slot_split": ("blk = slot / bs, off = slot % bs", "blk = slot % NB, off = slot / NB"),
    "append_skips_scale": ("float yk = xk * k_inv;", "float yk = xk;"),
    "multi_excludes_self": ("(int32_t)(L - q_len + i + 1)", "(int32_t)(L - q_len + i)"),
    "multi_not_causal": ("(int32_t)(L - q_len + i + 1)", "(int32_t)(L)"),
    "multi_token_not_relative": ("const int64_t i = tok - query_start_loc[s];",
                                 "const int64_t i = tok - query_start_loc[0];"),
    "multi_wrong_sequence": ("while (query_start_loc[s + 1] <= tok)",
                             "while (query_start_loc[s + 1] < tok)"),
}

PIN_FILES = ["tests/test_oracle_decode.py", "tests/test_oracle_append.py",
             "tests/test_oracle_codecs.py", "tests/test_oracle_decode_multi.py"]


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(tmp, "libmutant.so")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-ffp-contract=off", "-o", lib, path, "-lm"], check=True)
        env = dict(os.environ, PA_ORACLE_LIB=lib)
        res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not slow",
                              *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                             timeout=600)
    assert res.returncode != 0, f"mutant {name} passed every pin:\n{res.stdout[-2000:]}"
