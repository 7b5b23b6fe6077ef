"""Each plausible mistake planted in a copy of the oracle (on the CPU) must
make at least one pin fail; this is what shows the pins are not vacuous."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from oracle_pins import PINS

# (id, text in kvc_oracle.c, replacement); every occurrence is replaced
MUTANTS = [
    ("top_left_alignment", "int64_t last = old_len + t;", "int64_t last = t;"),
    ("head_map_modulo", "const int64_t h = hq / group;", "const int64_t h = hq % Hk;"),
    ("default_scale_uses_Dv", "resolve_scale(has_scale, scale, D, &sc)",
     "resolve_scale(has_scale, scale, Dv, &sc)"),
    ("no_max_subtraction", "attention_row[j] = exp(attention_row[j] - mx);",
     "attention_row[j] = exp(attention_row[j]);"),
    ("min_instead_of_max", "if (attention_row[j] > mx) mx = attention_row[j];",
     "if (attention_row[j] < mx) mx = attention_row[j];"),
    ("append_off_by_one", "int64_t slot = lengths[b] + t;", "int64_t slot = lengths[b] + t + 1;"),
    ("lengths_not_advanced", "lengths_out[b] = lengths[b] + n;", "lengths_out[b] = lengths[b];"),
    ("no_normalisation", "attention_row[j] = attention_row[j] / z;",
     "attention_row[j] = attention_row[j];"),
    ("context_from_keys", "load_elem(value_updated, voff + d, dtype)",
     "load_elem(key_updated, voff + d, dtype)"),
    ("invalid_row_kept", "if (t >= n) return KVC_ORACLE_OK;", "if (t > n) return KVC_ORACLE_OK;"),
    ("scale_dropped", "attention_row[j] = sc * dot;", "attention_row[j] = dot;"),
    ("bf16_shift", "(uint32_t)((const uint16_t *)base)[idx] << 16;",
     "(uint32_t)((const uint16_t *)base)[idx] << 15;"),
    ("mask_ignored", "while (n < Q && mask_row[n] != 0) n++;", "while (n < Q) n++;"),
    ("non_prefix_accepted", "if (mask_row[t] != 0) return KVC_ORACLE_ROW_NOT_PREFIX;",
     "if (mask_row[t] == 2) return KVC_ORACLE_ROW_NOT_PREFIX;"),
    ("overflow_accepted", "if (len + n > M) return KVC_ORACLE_ROW_OVERFLOW;",
     "if (len + n > M + 1) return KVC_ORACLE_ROW_OVERFLOW;"),
    ("tail_not_copied", "memcpy(key_cache_out, key_cache, (size_t)(B * Hk * M * D * e));",
     "memset(key_cache_out, 0, (size_t)(B * Hk * M * D * e));"),
    ("key_stride_Dv", "const int64_t koff = ((b * Hk + h) * M + j) * D;",
     "const int64_t koff = ((b * Hk + h) * M + j) * Dv;"),
    ("query_row_fixed", "const int64_t qoff = ((b * Hq + hq) * Q + t) * D;",
     "const int64_t qoff = ((b * Hq + hq) * Q) * D;"),
    ("last_slot_dropped", "for (int64_t j = 0; j <= last; j++) {\n    const int64_t koff",
     "for (int64_t j = 0; j < last; j++) {\n    const int64_t koff"),
    ("value_head_zero", "const int64_t voff = ((b * Hk + h) * M + j) * Dv;",
     "const int64_t voff = ((b * Hk + 0) * M + j) * Dv;"),
]


# Runs the pins against one oracle build in a child process and prints the
# name of the first pin that fails.  A child process keeps a mutant that
# writes out of bounds (the overflow one does) away from the test runner.
RUNNER = r"""
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle
from oracle_pins import PINS
orc = oracle.Oracle(sys.argv[1])
for pin in PINS:
    try:
        pin(orc)
    except (AssertionError, ValueError, FloatingPointError):
        print(pin.__name__, flush=True)
        sys.exit(0)
sys.exit(3)
"""


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("mid,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, mid, find, repl):
    assert source.count(find) >= 1, f"mutation site for {mid} missing from kvc_oracle.c"
    src = tmp_path / "kvc_oracle.c"
    src.write_text(source.replace(find, repl))
    shutil.copy(os.path.join(os.path.dirname(oracle.SOURCE), "kvc_oracle.h"), tmp_path)
    lib = str(tmp_path / f"libmut_{mid}.so")
    oracle.build(str(src), lib)
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests_dir)
    r = subprocess.run([sys.executable, "-c", RUNNER, lib, root, tests_dir],
                       capture_output=True, text=True, timeout=600)
    caught_by = r.stdout.strip()
    assert caught_by.startswith("pin_"), f"mutant {mid} passed every pin (rc {r.returncode})"
