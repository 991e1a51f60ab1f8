"""The oracle's pins catch plausible mistakes: each case plants one mistake in a
copy of oracle/mtp_oracle.c (on the CPU), builds it, and runs the oracle's pin
tests against that build (MTP_ORACLE_LIB); at least one pin must fail.

The mistakes are readings a careful implementer could get wrong: the order of
the NVFP4 scale arithmetic at a global scale that is not a power of two
(a / 6 / s_g for a / f32(6 s_g), S or d kept in double, d from the unrounded
G / 2688), tie rounding, nibble order, constants, the concat order, the gamma
offset, eps, truncation, the argmax tie rule and the next rows' formulas.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mtp_oracle.c")
PIN_FILES = ["tests/test_oracle_codecs.py", "tests/test_oracle_quant.py", "tests/test_oracle_math.py",
             "tests/test_oracle_next.py"]

# name -> list of (text in mtp_oracle.c, replacement); each text occurs exactly once
MUTATIONS = {
    "nvfp4_a_over_6_over_sg": [("float ad = a / d; /* f32 division */", "float ad = a / 6.0f / c->sg;")],
    "nvfp4_S_in_double": [("float S = (float)oracle_e4m3_decode(sb) * c->sg; /* f32 multiply */",
                           "double S = oracle_e4m3_decode(sb) * (double)c->sg;")],
    "nvfp4_d_from_unrounded_G": [("float d = 6.0f * s;     /* f32 multiply of the rounded global scale */",
                                  "float d = (G == 0.0f) ? 6.0f : (float)(6.0 * (double)G / 2688.0);")],
    "nvfp4_6sg_unrounded": [("float ad = a / d; /* f32 division */",
                             "float ad = (float)((double)a / (6.0 * (double)c->sg));")],
    "nvfp4_global_constant": [("float sg = G / 2688.0f; /* f32 division */", "float sg = G / 2687.0f;")],
    "nvfp4_swapped_nibbles": [("c->codes[byte] = (uint8_t)((c->codes[byte] & 0xF0u) | q);",
                               "c->codes[byte] = (uint8_t)((c->codes[byte] & 0x0Fu) | (uint8_t)(q << 4));"),
                              ("c->codes[byte] = (uint8_t)((c->codes[byte] & 0x0Fu) | (uint8_t)(q << 4));\n      }",
                               "c->codes[byte] = (uint8_t)((c->codes[byte] & 0xF0u) | q);\n      }")],
    "ties_round_up": [("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;")],
    "e4m3_subnormal_quantum": [("if (e < -6) e = -6; /* subnormals share the quantum 2^-9 */", "if (e < -7) e = -7;")],
    "fp8_constant": [("float s = a / 448.0f; /* f32 division */", "float s = a / 447.0f;")],
    "rms_no_eps": [("double r = 1.0 / sqrt(ms + (double)eps);", "double r = 1.0 / sqrt(ms);")],
    "rms_no_gamma_offset": [("double g = oracle_bf16_decode(gamma[i]) + (double)gamma_offset;",
                             "double g = oracle_bf16_decode(gamma[i]);")],
    "concat_swapped": [("oracle_rms_norm(e, gamma_embed, h, eps, gamma_offset, c);\n"
                        "    oracle_rms_norm(target_hidden + bi * h, gamma_hidden, h, eps, gamma_offset, c + h);",
                        "oracle_rms_norm(e, gamma_embed, h, eps, gamma_offset, c + h);\n"
                        "    oracle_rms_norm(target_hidden + bi * h, gamma_hidden, h, eps, gamma_offset, c);")],
    "fc_row_stride": [("const uint16_t *wr = fc_w + j * 2 * h;", "const uint16_t *wr = fc_w + j * h;")],
    "truncation_off_by_one": [("? mtp_vocab_size : vocab;", "? mtp_vocab_size - 1 : vocab;")],
    "argmax_ge": [("for (int64_t i = 0; i < n; ++i)\n    if (v[i] > bv) {",
                   "for (int64_t i = 0; i < n; ++i)\n    if (v[i] >= bv) {")],
    "logprob_no_max_shift": [("for (int64_t i = 0; i < n; ++i) sum += exp(v[i] - m);",
                              "for (int64_t i = 0; i < n; ++i) sum += exp(v[i]);")],
    "logprob_sign": [("return -log(sum);", "return log(sum);")],
    "mask_short_by_one_word": [("if (wi >= mask_words) break;", "if (wi + 1 >= mask_words) break;")],
    "mask_bit_order": [("if ((((uint32_t)mask[wi]) >> (i % 32) & 1u) == 0u) continue;",
                        "if ((((uint32_t)mask[wi]) >> (31 - i % 32) & 1u) == 0u) continue;")],
    "split_no_branch_rounding": [("double be = oracle_bf16_decode(oracle_bf16_encode(se));", "double be = se;")],
    "split_subtract": [("u[j] = oracle_bf16_encode(be + bh);", "u[j] = oracle_bf16_encode(be - bh);")],
    "bf16_overflow_at_max": [("if (rv > ldexp(255.0, 120)) return sign | 0x7F80u;",
                              "if (rv >= ldexp(255.0, 120)) return sign | 0x7F80u;")],
    "bf16_subnormal_quantum": [("if (e < -126) e = -126; /* subnormal range shares the smallest quantum */",
                                "if (e < -125) e = -125; /* subnormal range shares the smallest quantum */")],
    "bf16_range_truncates": [("((uint16_t *)c->out)[i] = oracle_bf16_encode((double)f);",
                              "((uint16_t *)c->out)[i] = (uint16_t)(u >> 16);")],
}


def _mutant_source(src: str, subs) -> str:
    for old, new in subs:
        assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
        src = src.replace(old, new)
    return src


def _run_mutant(name: str, tmpdir: str) -> tuple[int, str]:
    with open(SRC) as f:
        src = _mutant_source(f.read(), MUTATIONS[name])
    c_path = os.path.join(tmpdir, f"{name}.c")
    so_path = os.path.join(tmpdir, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-w", "-o", so_path,
                    c_path, "-lm", "-lpthread"], check=True)
    env = dict(os.environ, MTP_ORACLE_LIB=so_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results():
    with tempfile.TemporaryDirectory(prefix="oracle_mutants_") as d:
        with concurrent.futures.ThreadPoolExecutor(4) as ex:
            futs = {n: ex.submit(_run_mutant, n, d) for n in MUTATIONS}
            yield {n: f.result() for n, f in futs.items()}


def test_mutation_sites_exist():
    with open(SRC) as f:
        src = f.read()
    for name, subs in MUTATIONS.items():
        _mutant_source(src, subs)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(mutant_results, name):
    rc, out = mutant_results[name]
    # pytest exit code 1: tests ran and at least one failed (not a crash or a collection error)
    assert rc == 1, f"mutation {name} not caught (exit {rc}):\n{out}"
