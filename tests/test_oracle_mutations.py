"""Planted mistakes in a copy of the oracle must fail the pins.

Each case rewrites one expression of oracle/pkv_oracle.c into a plausible bug (a
swapped index, a dropped term, a wrong sign, an off-by-one), builds that copy
into a temporary library, and runs the pin tests against it in a subprocess.
The pins must reject every mutant; the unmodified oracle must pass them.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")

MUTANTS = {
    "offset_uses_division": ("int64_t o = t % block_size;", "int64_t o = t / block_size;"),
    "block_uses_modulo": ("int64_t blk = t / block_size;", "int64_t blk = t % block_size;"),
    "head_and_offset_swapped": ("((phys * num_kv_heads + h) * block_size + off) * head_dim + d",
                                "((phys * num_kv_heads + off) * block_size + h) * head_dim + d"),
    "scale_dropped": ("z[t - t0] = scale * acc;", "z[t - t0] = acc;"),
    "gqa_modulo_mapping": ("h / group, 0, n,", "h % num_kv_heads, 0, n,"),
    "append_at_n": ("max_blocks_per_seq,\n                           block_size, num_blocks, n - 1,",
                    "max_blocks_per_seq,\n                           block_size, num_blocks, n,"),
    "merge_weight_sign": ("double w = exp(lse[p] - M);", "double w = exp(M - lse[p]);"),
    "lse_missing_log_sum": ("*lse = m + log(l);", "*lse = m;"),
    "fp16_exponent_bias": ("e - 25);", "e - 24);"),
    "value_head_zero": ("const uint16_t *v = v_pool + oracle_elem_offset(phys, g, off, 0, "
                        "num_kv_heads,\n                                                        "
                        "block_size, head_dim);\n        double w = exp(z[t - t0] - m);",
                        "const uint16_t *v = v_pool + oracle_elem_offset(phys, 0, off, 0, "
                        "num_kv_heads,\n                                                        "
                        "block_size, head_dim);\n        double w = exp(z[t - t0] - m);"),
    "missing_normalisation": ("        o[d] /= l;\n    *lse = m + log(l);",
                              "        o[d] /= 1.0;\n    *lse = m + log(l);"),
    "slotted_value_head_zero": ("block_size, head_dim);\n            const double w = exp(z[t] - m);",
                                "block_size, head_dim) - g * block_size * head_dim;\n"
                                "            const double w = exp(z[t] - m);"),
    "slotted_missing_normalisation": ("            for (int64_t d = 0; d < head_dim; ++d)\n"
                                      "                o[d] /= l;",
                                      "            for (int64_t d = 0; d < head_dim; ++d)\n"
                                      "                o[d] /= 1.0;"),
    "last_token_skipped": ("for (int64_t t = t0; t < t1; ++t) {\n        int64_t phys, off;\n        int rc",
                           "for (int64_t t = t0; t < t1 - 1; ++t) {\n        int64_t phys, off;\n        int rc"),
    # block copy: the anchors end at the slot copy's header, which follows it
    "copy_direction_swapped": ("head_dim);\n                    k_pool[to] = k_pool[from];\n"
                               "                    v_pool[to] = v_pool[from];\n                }\n"
                               "    return OR_OK;\n}\n\n/* ---- slot copy",
                               "head_dim);\n                    k_pool[from] = k_pool[to];\n"
                               "                    v_pool[to] = v_pool[from];\n                }\n"
                               "    return OR_OK;\n}\n\n/* ---- slot copy"),
    "copy_skips_values": ("head_dim);\n                    k_pool[to] = k_pool[from];\n"
                          "                    v_pool[to] = v_pool[from];\n                }\n"
                          "    return OR_OK;\n}\n\n/* ---- slot copy",
                          "head_dim);\n                    k_pool[to] = k_pool[from];\n"
                          "                }\n    return OR_OK;\n}\n\n/* ---- slot copy"),
    "copy_last_row_dropped": ("for (int64_t off = 0; off < block_size; ++off)",
                              "for (int64_t off = 0; off < block_size - 1; ++off)"),
    "slot_copy_ignores_destination_offset": ("int64_t to = oracle_elem_offset(c[2], h, c[3] + r, d,",
                                             "int64_t to = oracle_elem_offset(c[2], h, r, d,"),
    "slot_copy_ignores_source_offset": ("int64_t from = oracle_elem_offset(c[0], h, c[1] + r, d,",
                                        "int64_t from = oracle_elem_offset(c[0], h, r, d,"),
    "slot_copy_drops_last_row": ("for (int64_t r = 0; r < c[4]; ++r)",
                                 "for (int64_t r = 0; r < c[4] - 1; ++r)"),
    "slot_copy_skips_values": ("block_size, head_dim);\n                    k_pool[to] = k_pool[from];\n"
                               "                    v_pool[to] = v_pool[from];",
                               "block_size, head_dim);\n                    k_pool[to] = k_pool[from];"),
    "slot_offset_dropped": ("*off = so + (t - start);", "*off = (t - start);"),
    "segment_end_inclusive": ("if (t < start + len) {", "if (t <= start + len) {"),
    "slotted_append_at_n": ("rc = oracle_locate_slotted(row, ns, block_size, num_blocks, n - 1, &phys, &off);",
                            "rc = oracle_locate_slotted(row, ns, block_size, num_blocks, n, &phys, &off);"),
    "slotted_append_skips_values": ("                k_pool[at] = kn[d];\n                v_pool[at] = vn[d];",
                                    "                k_pool[at] = kn[d];"),
    "slotted_append_value_head_zero": ("const uint16_t *vn = v_new + (s * num_kv_heads + h) * head_dim;",
                                       "const uint16_t *vn = v_new + (s * num_kv_heads) * head_dim;"),
    "segment_start_not_advanced": ("        start += len;\n    }\n    return OR_ETABLE;",
                                   "    }\n    return OR_ETABLE;"),
}


def _build(tmp_path, text, name):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    str(src), "-lm"], check=True)
    return str(so)


def _run_pins(lib_path):
    env = dict(os.environ, PKV_ORACLE_LIB=lib_path, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_oracle_cow.py"),
           os.path.join(ROOT, "tests", "test_oracle_slotted.py"),
           os.path.join(ROOT, "tests", "test_oracle_slot_cow.py")]
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes(tmp_path):
    with open(SRC) as f:
        text = f.read()
    r = _run_pins(_build(tmp_path, text, "orig"))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    r = _run_pins(_build(tmp_path, text.replace(old, new), name))
    assert r.returncode != 0, f"mutant {name} passed every pin"
