"""Plant plausible mistakes in a copy of the oracle (on the CPU) and show that the
pins catch each one. The copy is built in a temporary directory; the real oracle is
untouched."""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.c")

# (name, text in mla_oracle.c, replacement)
MUTANTS = [
    ("causal_off_by_one", "int64_t n = L - J->q_len + j + 1;", "int64_t n = L - J->q_len + j;"),
    ("drop_rope", "for (int d = 0; d < ORACLE_D_QK; ++d) dot +=",
     "for (int d = 0; d < ORACLE_D_V; ++d) dot +="),
    ("wrong_slot", "(page * ORACLE_PAGE + i % ORACLE_PAGE) * row_bytes, kd);\n    double dot",
     "(page * ORACLE_PAGE + (i + 1) % ORACLE_PAGE) * row_bytes, kd);\n    double dot"),
    ("log2_lse", "J->out_lse[idx] = m + log(l);", "J->out_lse[idx] = m + log2(l);"),
    ("scale_on_lse", "J->out_lse[idx] = m + log(l);",
     "J->out_lse[idx] = m + log(l) + log(J->output_scale);"),
    ("subnormal_exponent", "v = ldexp((double)mant, -9);", "v = ldexp((double)mant, -10);"),
    ("v_from_rope", "acc[d] += w * kd[d];", "acc[d] += w * kd[d + 64];"),
    ("no_max_shift_sign", "double w = exp(s[i] - m);", "double w = exp(m - s[i]);"),
    ("sink_sign", "double l = J->sinks ? exp(sigma - m) : 0.0;",
     "double l = J->sinks ? exp(m - sigma) : 0.0;"),
    ("sink_head_index", "J->sinks[r % J->heads]", "J->sinks[0]"),
    ("sink_outside_max", "if (sigma > m) m = sigma;", ""),
    ("bf16_ties_away", "double r = nearbyint(v / quantum) * quantum;",
     "double r = round(v / quantum) * quantum;"),
    ("bf16_short_significand", "double quantum = ldexp(1.0, e - 7);",
     "double quantum = ldexp(1.0, e - 6);"),
    ("bounds_start_off_by_one", "if (start > k0) k0 = start;",
     "if (start + 1 > k0) k0 = start + 1;"),
    ("bounds_end_inclusive", "if (end < k1) k1 = end;", "if (end + 1 < k1) k1 = end + 1;"),
    ("bounds_end_past_causal", "if (end < k1) k1 = end;", "if (end < L) k1 = end;"),
    ("bounds_of_request_0", "start = J->bounds[2 * (int64_t)b],", "start = J->bounds[0],"),
    ("empty_row_divides", "if (l == 0.0) { /* no visible key and no sink */",
     "if (l == -1.0) {"),
    ("mx_scale_not_strict", "while (e < 127 && amax >= ldexp(448.0, e)) ++e;",
     "while (e < 127 && amax > ldexp(448.0, e)) ++e;"),
    ("mx_no_saturation", "if (e == -127) {", "if (0) {"),
    ("mx_saturate_zeros", "(xb[i] != 0.0 ? 0x7E : 0x00)", "0x7E"),
    ("mx_saturate_to_nan", "(xb[i] != 0.0 ? 0x7E : 0x00)", "(xb[i] != 0.0 ? 0x7F : 0x00)"),
    ("mx_ties_odd", "(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    ("mx_sign_of_zero", "(signbit(y) ? 0x80 : 0)", "(y < 0 ? 0x80 : 0)"),
    ("bf16_bias", "v = ldexp(128.0 + mant, expo - 127 - 7);",
     "v = ldexp(128.0 + mant, expo - 126 - 7);"),
    ("bf16_row_stride", "(J->bf16 ? 2 : 1)", "(J->bf16 ? 1 : 1)"),
    ("bf16_byte_order", "(uint16_t)(src[2 * d] | (src[2 * d + 1] << 8))",
     "(uint16_t)(src[2 * d + 1] | (src[2 * d] << 8))"),
    ("bf16_subnormal", "v = ldexp((double)mant, -126 - 7);", "v = ldexp((double)mant, -126 - 8);"),
    ("mx_amax_skips_first", "for (int i = 0; i < block; ++i) {\n        if (!isfinite",
     "for (int i = 1; i < block; ++i) {\n        if (!isfinite"),
]


def _build_mutant(tmpdir, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    path_c = os.path.join(tmpdir, "mutant.c")
    path_so = os.path.join(tmpdir, "libmutant.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
                    "-o", path_so, path_c, "-lm"], check=True)
    return path_so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    with tempfile.TemporaryDirectory() as d:
        lib = _build_mutant(d, old, new)
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib_path=lib)
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
        assert caught, f"no pin caught mutant {name}"
