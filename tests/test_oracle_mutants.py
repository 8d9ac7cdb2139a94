"""Plausible mistakes planted in copies of the oracle (on the CPU only) must each trip at
least one pin: evidence that the pins constrain every step of the oracle."""
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "paged_oracle.c")

# (name, text in the oracle, planted replacement)
MUTANTS = [
    ("diagonal_key_dropped", "j <= q_pos; ++j) {\n                    const double* kj", "j < q_pos; ++j) {\n                    const double* kj"),
    ("query_position_shifted", "q_pos = length - t + i;", "q_pos = length - t + i - (i > 0);"),
    ("gqa_interleaved", "kvh = h / group;", "kvh = h % num_kv_heads;"),
    ("softmax_sign", "exp(s[j] - m)", "exp(m - s[j])"),
    ("no_max_subtraction", "exp(s[j] - m)", "exp(s[j])"),
    ("normalisation_dropped", "acc[d] / l;", "acc[d];"),
    ("scale_dropped", "s[j] = scale * dot;", "s[j] = dot;"),
    ("slot_offset_transposed", "* block_size + p % block_size;", "* block_size + p / block_size;"),
    ("block_index_off_by_one", "table_row[p / block_size]", "table_row[(p + 1) / block_size]"),
    ("kv_operand_swapped", "const double* vj = ctx_v", "const double* vj = ctx_k"),
    ("scratch_slot_wrong", "const int64_t scratch = num_slots - 1;", "const int64_t scratch = 0;"),
    ("bf16_truncates", "ldexp(rint(ldexp(x, -q)), q)", "ldexp(trunc(ldexp(x, -q)), q)"),
    ("bf16_via_float", "double r = ldexp(rint(ldexp(x, -q)), q);", "double r = ldexp(rint(ldexp((double)(float)x, -q)), q);"),
    ("padding_rows_not_cleared", "store_elem(out, i * qrow + e, dtype, 0.0);", "store_elem(out, i * qrow + e, dtype, 1.0);"),
    ("head_offset_in_q", "row * qrow + (int64_t)h * head_dim + d, dtype);", "row * qrow + (int64_t)(h / 2) * head_dim + d, dtype);"),
    ("window_one_key_too_many", "? q_pos - window + 1 : 0;", "? q_pos - window : 0;"),
    ("window_ignored", "? q_pos - window + 1 : 0;", "? 0 : 0;"),
    ("window_one_key_too_few", "? q_pos - window + 1 : 0;", "? q_pos - window + 2 : 0;"),
    ("copy_half_block", "for (int64_t b = 0; b < block_bytes; ++b) to[b] = from[b];",
     "for (int64_t b = 0; b < block_bytes / 2; ++b) to[b] = from[b];"),
    ("copy_wrong_destination", "unsigned char* to = (unsigned char*)dst + dst_block[i] * block_bytes;",
     "unsigned char* to = (unsigned char*)dst + src_block[i] * block_bytes;"),
    ("copy_pairs_misaligned", "const unsigned char* from = (const unsigned char*)src + src_block[i] * block_bytes;",
     "const unsigned char* from = (const unsigned char*)src + src_block[i ? i - 1 : 0] * block_bytes;"),
    ("fp8_exponent_bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 6)"),
    ("fp8_round_half_up", "const double r = ldexp(rint(ldexp(a, -q)), q);", "const double r = ldexp(floor(ldexp(a, -q) + 0.5), q);"),
    ("fp8_scale_constant", "amax / 448.0f", "amax / 240.0f"),
    ("fp8_scale_of_wrong_head", "(double)scale[slot * num_kv_heads + e / head_dim]", "(double)scale[slot * num_kv_heads]"),
    ("fp8_subnormals_flushed", "if (Er < -6) return sign | (uint8_t)ldexp(r, 9);", "if (Er < -6) return sign;"),
]


RUNNER = r"""
import sys
import oracle
from tests import oracle_pins as P
oracle._LIB = oracle.load_library(sys.argv[1])
caught = []
for check in P.ALL_CHECKS + [lambda o: P.check_chunking_invariance(o, long_prompt=False)]:
    try:
        check(oracle)
    except Exception:
        caught.append(getattr(check, "__name__", "chunking"))
print("CAUGHT", " ".join(caught))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutant {name}: pattern not found in the oracle"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(src), "-o",
                           lib_path, "-lm"])
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    # a mutant may also crash (e.g. read past a table row): that counts as caught too
    proc = subprocess.run([sys.executable, "-c", RUNNER, lib_path], cwd=root, capture_output=True,
                          text=True, timeout=600, env=dict(os.environ, OMP_NUM_THREADS="2"))
    if proc.returncode != 0:
        return
    line = [l for l in proc.stdout.splitlines() if l.startswith("CAUGHT")][-1]
    assert line.split()[1:], f"planted mistake {name} passed every pin"
