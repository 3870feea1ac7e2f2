"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of ``oracle/kev_oracle.c`` with one plausible mistake
(a dropped term, a wrong index or sign, a swapped operand), compiled with gcc
into a temporary directory.  The pins of ``oracle_pins`` run against it in a
child process; at least one pin must fail.  The product code is not involved.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    "dropped_scale": ("w[j] = s * scale;", "w[j] = s;"),
    "diagonal_not_visible": ("attend(qv, kbuf, vbuf, i - a + 1, d, w,", "attend(qv, kbuf, vbuf, i - a, d, w,"),
    "gqa_modulo_map": ("int32_t g = h / (heads / kv_heads);", "int32_t g = h % kv_heads;"),
    "missing_normalisation": ("out[c] = acc / z;", "out[c] = acc;"),
    "scores_against_v": ("s += qv[c] * kv[(size_t)j * d + c];", "s += qv[c] * vv[(size_t)j * d + c];"),
    "bf16_widen_shift": ("uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;",
                         "uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 15;"),
    "decode_stale_row_instead_of_new_k": (
        "kbuf[(size_t)(L - 1) * d + c] = widen(k_new, dtype, src);",
        "kbuf[(size_t)(L - 1) * d + c] = widen(pool, dtype, kbase + (size_t)(L - 1) * d + c);"),
    "decode_v_from_k_plane": ("size_t vbase = kbase + (size_t)kv_heads * plane;", "size_t vbase = kbase;"),
    "max_not_subtracted": ("w[j] = exp(w[j] - m);", "w[j] = exp(w[j]);"),
    "q_head_from_kv_head": ("qv[c] = widen(q, dtype, ((size_t)i * heads + h) * d + c);",
                            "qv[c] = widen(q, dtype, ((size_t)i * heads + h / (heads / kv_heads)) * d + c);"),
    "decode_slot_by_request_index": ("size_t kbase = (size_t)slot_ids[r] * slot_elems",
                                     "size_t kbase = (size_t)(r % n_slots) * slot_elems"),
    "decode_group_modulo": ("int32_t r = (int32_t)(u / heads), h = (int32_t)(u % heads), g = h / G;",
                            "int32_t r = (int32_t)(u / heads), h = (int32_t)(u % heads), g = h % kv_heads;"),
    "exp_sign_flipped": ("w[j] = exp(w[j] - m);", "w[j] = exp(m - w[j]);"),
    "store_slot_by_question_index": ("size_t kdst = (size_t)slot_ids[s] * slot_elems + (size_t)g * plane +",
                                     "size_t kdst = (size_t)(s % n_slots) * slot_elems + (size_t)g * plane +"),
    "store_row_off_by_one": ("(size_t)(i - cu[s]) * d;", "(size_t)(i - cu[s] + 1) * d;"),
    "store_k_from_v": ("memcpy((char *)pool_after + kdst * esz, (const char *)k + src * esz, esz * d);",
                       "memcpy((char *)pool_after + kdst * esz, (const char *)v + src * esz, esz * d);"),
    "chunk_causal_limit_off_by_one": ("attend(qv, kbuf, vbuf, P + i + 1,", "attend(qv, kbuf, vbuf, P + i,"),
    "chunk_prefix_keys_from_v_plane": (
        "kbuf[e] = widen(pool, dtype, kbase + e);", "kbuf[e] = widen(pool, dtype, vbase + e);"),
    "chunk_rows_overwrite_prefix": ("kbuf[(size_t)(P + j) * d + c] = widen(k, dtype, src);",
                                    "kbuf[(size_t)j * d + c] = widen(k, dtype, src);"),
    "chunk_stored_at_row_zero": ("size_t row = (size_t)(prefix_lens[s] + i - cu[s]);", "size_t row = (size_t)(i - cu[s]);"),
    "paged_block_of_next_position": ("size_t at = (size_t)table[p / block_size] * block_elems",
                                     "size_t at = (size_t)table[(p + 1) / block_size] * block_elems"),
    "paged_row_ignores_block_offset": ("(size_t)(p % block_size) * d;\n                    for",
                                       "(size_t)(p / block_size) * d;\n                    for"),
    "paged_v_from_k_plane": ("vbuf[(size_t)p * d + c] = widen(pool, dtype, at + (size_t)kv_heads * head_rows + c);",
                             "vbuf[(size_t)p * d + c] = widen(pool, dtype, at + c);"),
    "paged_append_into_first_block": ("int32_t blk = block_tables[(size_t)r * max_blocks + p / block_size];",
                                      "int32_t blk = block_tables[(size_t)r * max_blocks];"),
    "append_k_into_v_plane": (
        "memcpy((char *)pool_after + kdst * esz, (const char *)k_new + src * esz, esz * d);",
        "memcpy((char *)pool_after + vdst * esz, (const char *)k_new + src * esz, esz * d);"),
}

RUNNER = r"""
import json, sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle
from oracle_pins import ALL_PINS
orc = oracle.Oracle(sys.argv[1])
failed = []
for pin in ALL_PINS:
    try:
        pin(orc)
    except Exception as e:
        failed.append([pin.__name__, type(e).__name__])
print(json.dumps(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / f"{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_oracle(str(mutated), str(tmp_path / f"lib{name}.so"))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-c", RUNNER, lib, ROOT, HERE], capture_output=True,
                       text=True, env=env, timeout=300)
    if p.returncode != 0:
        # a crash of the mutant also counts as caught, but say why
        assert p.returncode < 0 or "Error" in p.stderr, p.stderr[-2000:]
        return
    failed = json.loads(p.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"
