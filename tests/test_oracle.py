"""The oracle against its pins, and the pins against broken copies of the oracle.

CPU only. A pin is a fact the oracle must reproduce that does not come from
the oracle itself (closed forms, library routines, the pages' figures); see
``oracle_pins``. The mutation half plants plausible mistakes in a copy of the
oracle's C source (a transposed operand, a dropped term, a wrong sign, a
wrong rounding) and checks that at least one pin catches each.
"""
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


# (name, text in gemm_oracle.c, replacement)
MUTANTS = [
    ("transposed_B_at", "dec_one(dtype, B, k * N + j)", "dec_one(dtype, B, j * K + k)"),
    ("minus_sign", "acc[j] += p;", "acc[j] -= p;"),
    ("dropped_first_term", "for (int64_t k = 0; k < K; ++k) {\n          const double a",
     "for (int64_t k = 1; k < K; ++k) {\n          const double a"),
    ("dropped_last_term_at", "for (int64_t k = 0; k < K; ++k) {\n      const double p",
     "for (int64_t k = 0; k + 1 < K; ++k) {\n      const double p"),
    ("signed_abs_sum", "s[j] += fabs(p);", "s[j] += p;"),
    ("bias_wrong_index", "v += (double)bias[j];", "v += (double)bias[0];"),
    ("gelu_no_sqrt2", "erfc(-v / sqrt(2.0))", "erfc(-v)"),
    ("gelu_one_plus_erf", "0.5 * v * erfc(-v / sqrt(2.0))", "0.5 * v * (1.0 + erf(v / sqrt(2.0)))"),
    ("gelu_tanh_form", "0.5 * v * erfc(-v / sqrt(2.0))",
     "0.5 * v * (1.0 + tanh(0.7978845608 * (v + 0.044715 * v * v * v)))"),
    ("scale_after_bias", "if (flags & OR_SCALE) v = scale * v;\n  if (flags & OR_BIAS) v += (double)bias[j];",
     "if (flags & OR_BIAS) v += (double)bias[j];\n  if (flags & OR_SCALE) v = scale * v;"),
    ("resid_before_gelu", "if (flags & OR_GELU) v = oracle_gelu(v);\n  if (flags & OR_RESID) v += dec_one(resid_dtype, resid, ij);",
     "if (flags & OR_RESID) v += dec_one(resid_dtype, resid, ij);\n  if (flags & OR_GELU) v = oracle_gelu(v);"),
    ("resid_transposed", "dec_one(resid_dtype, resid, ij)", "dec_one(resid_dtype, resid, (ij % 4) * 3 + ij / 4)"),
    ("f16_exponent_bias", "e - 25", "e - 24"),
    ("f16_subnormal_scale", "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    ("bf16_shift", "(uint32_t)h << 16", "(uint32_t)h << 15"),
    ("round_truncates", "nearbyint(ldexp(a, -q))", "floor(ldexp(a, -q))"),
    ("round_ties_away", "nearbyint(ldexp(a, -q))", "round(ldexp(a, -q))"),
    ("no_overflow_to_inf", "if (r >= ldexp(1.0, emax + 1)) r = INFINITY;", ""),
    ("ulp_off_by_one", "return ldexp(1.0, lead - (p - 1));", "return ldexp(1.0, lead - p);"),
    ("a_row_stride_N", "arow[k] = dec_one(dtype, A, i * K + k)", "arow[k] = dec_one(dtype, A, i * N + k)"),
    ("f16acc_not_rounded", "acc = round_fmt(acc + dec_one(OR_F16, A, i * K + k) * dec_one(OR_F16, B, k * N + j), 11,\n                        -14, 15);",
     "acc = acc + dec_one(OR_F16, A, i * K + k) * dec_one(OR_F16, B, k * N + j);"),
    ("f16acc_bf16_rounding", "11,\n                        -14, 15);", "8,\n                        -126, 127);"),
    ("f16acc_transposed_B", "dec_one(OR_F16, B, k * N + j)", "dec_one(OR_F16, B, j * K + k)"),
    ("softmax_no_max", "sum += exp(scale * (double)x[c] - m);", "sum += exp(scale * (double)x[c]);"),
    ("softmax_scale_dropped", "ref[r * cols + c] = exp(scale * (double)x[c] - m) / sum;",
     "ref[r * cols + c] = exp((double)x[c] - m) / sum;"),
    ("softmax_last_column_dropped", "for (int64_t c = 0; c < cols; ++c) sum += exp",
     "for (int64_t c = 0; c + 1 < cols; ++c) sum += exp"),
]

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
for name, path in {paths!r}:
    lib = oracle.load(path)
    verdict = "MISSED"
    for pin in oracle_pins.PINS:
        try:
            pin(lib)
        except Exception as e:
            verdict = "CAUGHT " + pin.__name__ + " " + type(e).__name__
            break
    print("VERDICT", name, verdict, flush=True)
"""


def _run_pins(paths):
    """Every mutant library in `paths` ([(name, path)]) through the pins in one
    process (the pins import torch and scipy, which take seconds to load)."""
    return subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, paths=paths)],
                          capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module")
def mutant_runs(tmp_path_factory):
    """Build every mutant (in parallel), run them all through the pins at once; the
    verdict lines by mutant name, with the libraries for a rerun."""
    from concurrent.futures import ThreadPoolExecutor
    d = tmp_path_factory.mktemp("mutants")
    src = open(oracle.SRC).read()
    paths = []
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"mutation site for {name} not unique/present"
        (d / f"{name}.c").write_text(src.replace(old, new))
        paths.append((name, str(d / f"lib_{name}.so")))
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(lambda np_: oracle.build(str(d / f"{np_[0]}.c"), np_[1]), paths))
    out = _run_pins(paths)
    verdicts = {}
    for line in out.stdout.splitlines():
        if line.startswith("VERDICT "):
            _, name, v = line.split(" ", 2)
            verdicts[name] = v
    return verdicts, dict(paths)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(mutant_runs, name, old, new):
    """Each planted mistake in the oracle fails at least one pin."""
    verdicts, paths = mutant_runs
    v = verdicts.get(name)
    if v is None:
        # the shared run ended before this mutant (one crashed): run it alone, where
        # a crash of the mutant counts as caught as well
        out = _run_pins([(name, paths[name])])
        assert out.returncode != 0 or "CAUGHT" in out.stdout, (name, out.stdout,
                                                                out.stderr[-500:])
        return
    assert v.startswith("CAUGHT"), (name, v)
