"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one. Each mutant is a one-token change (a shift, a sign, an index,
a comparison, a dropped rounding term); it is compiled on the CPU into a
temporary library and the oracle pin tests run against it in a subprocess.
A mutant that passes every pin would mean the pins cannot tell that mistake
from the correct oracle.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "uzip_oracle.c")

MUTANTS = {
    "exponent_shift": ("return (uint8_t)((x >> 7) & 0xffu);", "return (uint8_t)((x >> 8) & 0xffu);"),
    "signmant_sign_bit": ("(((x >> 8) & 0x80u) | (x & 0x7fu))", "(((x >> 9) & 0x80u) | (x & 0x7fu))"),
    "merge_sign_shift": ("(((unsigned)a & 0x80u) << 8)", "(((unsigned)a & 0x80u) << 7)"),
    "tie_to_larger_exponent": ("hist[e] > hist[best]", "hist[e] >= hist[best]"),
    "nibble_order": ("if (i % 2 == 0) out[L.codes + i / 2] |= (uint8_t)code;",
                     "if (i % 2 == 1) out[L.codes + i / 2] |= (uint8_t)code;"),
    "dummy_code_15": ("unsigned code = (k < 0) ? 0u : (unsigned)k;",
                      "unsigned code = (k < 0) ? 15u : (unsigned)k;"),
    "global_positions": ("put_u16(out + L.pos + 2 * j, (uint16_t)(i - lo));",
                         "put_u16(out + L.pos + 2 * j, (uint16_t)(i));"),
    "inclusive_offsets": ("put_u32(out + L.offs + 4 * c, (uint32_t)j);",
                          "put_u32(out + L.offs + 4 * c, (uint32_t)(j + 1));"),
    "rne_ties_away": ("if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;",
                      "if (lo >= 0x8000u) hi += 1;"),
    "rne_truncate": ("if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;", ";"),
    "add_becomes_sub": ("orc_bf16_to_f32(a) + orc_bf16_to_f32(b)", "orc_bf16_to_f32(a) - orc_bf16_to_f32(b)"),
    "nan_payload_kept": ("return 0x7FC0;", "return (uint16_t)(u >> 16);"),
    "section_alignment": ("return (v + 255u) & ~(uint64_t)255u;", "return (v + 127u) & ~(uint64_t)127u;"),
    "patch_drops_signmant": ("y[i] = orc_merge(in[L.sm + i], in[L.val + j]);",
                             "y[i] = orc_merge(0, in[L.val + j]);"),
    "validate_equal_positions": ("if (j > j0 && p <= get_u16", "if (j > j0 && p < get_u16"),
    "validate_skips_nibble": ("if (code != 0) return -3;", "if (code > 15) return -3;"),
    "sum_order_reversed": ("volatile float s = orc_bf16_to_f32(v[0]);\n"
                           "    for (uint32_t i = 1; i < k; i++) s = s + orc_bf16_to_f32(v[(uint64_t)i * stride]);",
                           "volatile float s = orc_bf16_to_f32(v[(uint64_t)(k - 1) * stride]);\n"
                           "    for (uint32_t i = k - 1; i-- > 0;) s = s + orc_bf16_to_f32(v[(uint64_t)i * stride]);"),
    "sum_in_binary64": ("volatile float s = orc_bf16_to_f32(v[0]);", "volatile double s = orc_bf16_to_f32(v[0]);"),
    "sum_skips_first_input": ("for (uint32_t i = 1; i < k; i++) s = s +", "for (uint32_t i = 2; i < k; i++) s = s +"),
    "s15_sentinel_14": ("unsigned code = (k < 0) ? 15u : (unsigned)k;          /* the sentinel */",
                        "unsigned code = (k < 0) ? 14u : (unsigned)k;          /* the sentinel */"),
    "s15_uses_16_codes": ("    for (int k = 0; k < 15; k++)\n        if (dec[k] == e) return k;\n    return -1;\n}\n\nstatic orc_layout orcs_layout_of",
                          "    for (int k = 0; k < 16; k++)\n        if (dec[k] == e) return k;\n    return -1;\n}\n\nstatic orc_layout orcs_layout_of"),
    "s15_keeps_position_section": ("    L.val = L.pos;\n    L.total = L.val + m;",
                                   "    L.val = L.pos + orc_align(2 * m);\n    L.total = L.val + m;"),
    "fp8_sign_shift": ("(uint8_t)(((x >> 5) & 0x4u) | (x & 0x3u))", "(uint8_t)(((x >> 4) & 0x4u) | (x & 0x3u))"),
    "fp8_exponent_width": ("(uint8_t)((x >> 2) & 0x1fu)", "(uint8_t)((x >> 2) & 0x0fu)"),
    "fp8_msb_first_bits": ("sec[b / 8] |= (uint8_t)(1u << (b % 8));", "sec[b / 8] |= (uint8_t)(0x80u >> (b % 8));"),
    "fp8_sm_section_length": ("static uint64_t orc8_sm_bytes(uint64_t n) { return (3 * n + 7) / 8; }",
                              "static uint64_t orc8_sm_bytes(uint64_t n) { return (3 * n) / 8 + 1; }"),
    "z7_codes_from_zero": ("        if (dec[k] == e) return k + 1;", "        if (dec[k] == e) return k;"),
    "z7_top8_codes": ("    for (int k = 0; k < 7; k++)\n        if (dec[k] == e) return k + 1;",
                      "    for (int k = 0; k < 8; k++)\n        if (dec[k] == e) return k + 1;"),
    "z7_msb_first_planes": ("return (unsigned)(i % 8); }", "return 7u - (unsigned)(i % 8); }"),
    "z7_keeps_position_section": ("/* no position section */\n    L.val = L.pos;\n    L.total = L.val + m;\n    return L;\n}\n\nstatic unsigned orcz_get_code",
                                  "/* no position section */\n    L.val = L.pos + orc_align(2 * m);\n    L.total = L.val + m;\n    return L;\n}\n\nstatic unsigned orcz_get_code"),
    "t8_seven_codes": ("    for (int k = 0; k < 8; k++)\n        if (dec[k] == e) return k;\n    return -1;\n}\n\nstatic orc_layout orct8_layout_of",
                       "    for (int k = 0; k < 7; k++)\n        if (dec[k] == e) return k;\n    return -1;\n}\n\nstatic orc_layout orct8_layout_of"),
    "t8_nibble_sized_codes": ("    L.offs = L.codes + orc_align((3 * n + 7) / 8);\n    L.pos = L.offs + orc_align(4 * (nch + 1));\n    L.val = L.pos + orc_align(2 * m);",
                              "    L.offs = L.codes + orc_align((n + 1) / 2);\n    L.pos = L.offs + orc_align(4 * (nch + 1));\n    L.val = L.pos + orc_align(2 * m);"),
}

PIN_TESTS = ["tests/test_oracle_split.py", "tests/test_oracle_codec.py", "tests/test_oracle_reduce.py",
             "tests/test_oracle_reduce_k.py", "tests/test_oracle_fp8.py", "tests/test_oracle_s15.py",
             "tests/test_oracle_z7.py", "tests/test_oracle_t8.py"]


def _run(name, a, b, tmp):
    src = open(SRC).read()
    assert src.count(a) >= 1, name
    path = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"lib{name}.so")
    open(path, "w").write(src.replace(a, b, 1))
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-o", lib, path],
                   check=True)
    env = dict(os.environ, UZIP_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu and not slow", *PIN_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            futs = [ex.submit(_run, n, a, b, tmp) for n, (a, b) in MUTANTS.items()]
            results = dict(f.result() for f in futs)
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    # rc 1 = tests failed; anything else (2 = collection error) is not a catch
    assert all(rc == 1 for rc in results.values()), results
