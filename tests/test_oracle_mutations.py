"""The oracle's pins must fail on plausible mistakes (CPU only).

Each case compiles a copy of the oracle with one planted mistake and runs the pin
suite against it in a subprocess; the suite must fail. This shows the pins are
sensitive to: the tie-break, the visibility rule, the raw tail, the relu, the
weight index, the head grouping, the softmax scale, the bf16 rounding, the
compression range, the FP8 cache's rounding, scale and dequantization, and the
attention backward's softmax Jacobian and scale.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qsa_ref.c")

MUTATIONS = {
    "tie_to_higher_index": ("return (x->blk > y->blk) - (x->blk < y->blk);",
                            "return (x->blk < y->blk) - (x->blk > y->blk);"),
    "visibility_floor_t_over_bs": ("return (t + 1) / d->block_size;",
                                   "return t / d->block_size;"),
    "raw_tail_dropped": ("for (int64_t j = nv * bs; j <= p.t; ++j)",
                         "for (int64_t j = nv * bs; j < p.t; ++j)", 2),
    "no_relu": ("static double relu(double x) { return x > 0.0 ? x : 0.0; }",
                "static double relu(double x) { return x; }"),
    "weight_of_head0": ("s += (double)w_row[h] * relu(dot);",
                        "s += (double)w_row[0] * relu(dot);"),
    "interleaved_head_groups": ("int64_t g = h / (Hq / Hkv);", "int64_t g = h % Hkv;", 2),
    "no_softmax_scale": ("z[i] = dot * scale;", "z[i] = dot;", 2),
    "bf16_truncation": ("double r = ldexp(nearbyint(ldexp(x, -qe)), qe);",
                        "double r = ldexp(trunc(ldexp(x, -qe)), qe);"),
    "compress_three_tokens": ("for (int64_t i = 0; i < bs; ++i)\n                    s +=",
                              "for (int64_t i = 0; i < bs - 1; ++i)\n                    s +="),
    "e4m3_quantum_halved": ("int qe = (e < -5 ? -5 : e) - 4;", "int qe = (e < -5 ? -5 : e) - 5;"),
    "e4m3_truncation": ("double r = ldexp(nearbyint(ldexp(a, -qe)), qe);",
                        "double r = ldexp(trunc(ldexp(a, -qe)), qe);"),
    "fp8_scale_ignored": ("return e4m3_value(s->f8[r * D + c]) * (double)s->scale[r];",
                          "return e4m3_value(s->f8[r * D + c]);"),
    "fp8_amax_over_256": ("float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;",
                          "float s = amax > 0.0 ? (float)(amax / 256.0) : 1.0f;"),
    "backward_no_softmax_jacobian": ("const double ds = z[i] * (dp[i] - pdp);",
                                     "const double ds = z[i] * dp[i];"),
    "backward_dk_unscaled": ("dk[r * D + c] += scale * ds * bf16_value(qh[c]);",
                             "dk[r * D + c] += ds * bf16_value(qh[c]);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    old, new, *count = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == (count[0] if count else 1), f"mutation anchor for {name} not found"
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "qsa_ref.c")
        open(c, "w").write(src.replace(old, new))
        subprocess.run(["cp", os.path.join(ROOT, "oracle", "qsa_ref.h"), tmp], check=True)
        lib = os.path.join(tmp, "libmut.so")
        subprocess.run(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", c, "-o", lib,
                        "-lm", "-lpthread"], check=True)
        env = dict(os.environ, QSA_ORACLE_LIB=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                            "-k", "not prefill_1x1024 and not needles"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
