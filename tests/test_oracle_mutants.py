"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below is a copy of ``oracle/moe_oracle.c`` with one deliberate
slip of the kind a hand-written oracle could contain: a dropped term, a wrong
sign, index or operand, a max for a sum, a tie broken the wrong way.  Every
mutant is compiled on its own and the pin suites (``test_oracle_pins.py``,
``test_oracle_mlp_pins.py``) are run against it in a subprocess; the test
passes only if each mutant makes at least one pin fail.  A mutant whose
search text no longer occurs in the source fails the test too, so the list
follows the oracle as it changes.

The two slowest pins (the exhaustive E4M3 neighbour sweep and the torch cast
cross-check) are left out of the mutant runs to keep this test short; the
rounding mutant is caught by the hand-derived rounding fixture instead.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

# name -> (text in moe_oracle.c, replacement)
MUTANTS = {
    "exp: degree-7 term dropped": (
        "float p = c7;\n    p = fmaf(p, r, c6);", "float p = c6;"),
    "exp: low part of ln2 dropped": (
        "r = fmaf(-n, 1.4286068e-6f, r);", "r = r;"),
    "group score: max instead of sum": (
        "sum = (i == 0) ? s[best] : sum + s[best];",
        "sum = (i == 0) ? s[best] : (s[best] > sum ? s[best] : sum);"),
    "ties: higher index wins": ("return ia < ib;", "return ia > ib;"),
    "expert select: worst first": (
        "if (taken[e] || !gkept[e / Eg]) continue;\n                if (best < 0 || ahead(s[e], e, s[best], best))",
        "if (taken[e] || !gkept[e / Eg]) continue;\n                if (best < 0 || ahead(s[best], best, s[e], e))"),
    "softmax weights: sign flipped": (
        "uu[j] = orc_exp_r(l[sel[j]] - l0);", "uu[j] = orc_exp_r(l0 - l[sel[j]]);"),
    "layout: rank offsets per expert index": (
        "off_r[r] = off_e[r * Er];", "off_r[r] = off_e[r];"),
    "layout: rank counts pairs, not tokens": ("hit[e / Er] = 1;", "hit[e / Er] += 1;"),
    "layout: descending token order inside an expert": (
        "for (int t = 0; t < T; ++t)\n        for (int j = 0; j < k; ++j) {\n            const int e = idx[(size_t)t * k + j];\n            const int rank",
        "for (int t = T - 1; t >= 0; --t)\n        for (int j = 0; j < k; ++j) {\n            const int e = idx[(size_t)t * k + j];\n            const int rank"),
    "layout: aligned regions over-rounded": (
        "span = (span + A - 1) / A * A;", "span = (span + A) / A * A;"),
    "dispatch: wrong scale divisor": ("scale = a / 448.0f;", "scale = a / 447.0f;"),
    "e4m3: ties away from even": ("else c = (lo % 2 == 0) ? lo : hi;", "else c = hi;"),
    "bf16: truncation instead of nearest": (
        "const double r = nearbyint(a / q) * q;", "const double r = floor(a / q) * q;"),
    "pow2 scale: chosen against 256 instead of 448": (
        "while (ldexp(448.0, e) < (double)a) ++e;", "while (ldexp(256.0, e) < (double)a) ++e;"),
    "ue8m0: exponent bias 126": (
        "(uint8_t)(ilogbf(scale) + 127);", "(uint8_t)(ilogbf(scale) + 126);"),
    "combine: weights of reversed slots": (
        "acc += (double)w[(size_t)t * k + j] *", "acc += (double)w[(size_t)t * k + (k - 1 - j)] *"),
    "dispatch backward: last slot overwrites": (
        "acc += (double)bf16_to_f32(grad_recv[(size_t)p * H + c]);",
        "acc = (double)bf16_to_f32(grad_recv[(size_t)p * H + c]);"),
    "combine backward: router gradient ignores y": (
        "dot += g * (double)bf16_to_f32(y[(size_t)p * H + c]);", "dot += g;"),
    "mlp: gate and up swapped": (
        "const double g = h[j], u = h[I + j];", "const double g = h[I + j], u = h[j];"),
    "mlp: silu sign flipped": (
        "const double a = g / (1.0 + exp(-g)) * u;", "const double a = g / (1.0 + exp(g)) * u;"),
    "mlp: W1 scale row block always 0": (
        "c->w1s + ((size_t)e * S2I + n / 128) * SH;", "c->w1s + ((size_t)e * S2I) * SH;"),
    "mlp: x scale block always 0": (
        "(double)c->xs[(size_t)p * SH + k / 128];", "(double)c->xs[(size_t)p * SH];"),
    "mlp: W2 scales of expert 0": (
        "c->w2s + ((size_t)e * (H / 128) + n / 128) * SI;", "c->w2s + ((size_t)0 * (H / 128) + n / 128) * SI;"),
    "mlp: W2 of the previous expert": (
        "c->w2 + ((size_t)e * H + n) * I;", "c->w2 + ((size_t)(e > 0 ? e - 1 : 0) * H + n) * I;"),
    "mlp: act scale block always 0": (
        "(double)c->as[(size_t)p * SI + k / 128];", "(double)c->as[(size_t)p * SI];"),
}

SLOW = ["tests/test_oracle_pins.py::test_e4m3_exhaustive_neighbour_check",
        "tests/test_oracle_pins.py::test_e4m3_matches_torch_cast"]


def _run_mutant(name, text, repl, workdir):
    src = open(SRC).read()
    if src.count(text) != 1:
        return name, "search text occurs %d times" % src.count(text)
    tag = "".join(c if c.isalnum() else "_" for c in name)
    csrc = os.path.join(workdir, tag + ".c")
    so = os.path.join(workdir, tag + ".so")
    with open(csrc, "w") as f:
        f.write(src.replace(text, repl))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           "-I", os.path.dirname(SRC), "-o", so, csrc, "-lm"])
    env = dict(os.environ, CGL_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "tests/test_oracle_pins.py", "tests/test_oracle_mlp_pins.py"] + [a for s in SLOW for a in ("--deselect", s)]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    if r.returncode == 0:
        return name, "survived: every pin passed"
    if r.returncode not in (1,):
        return name, "pin run ended with status %d:\n%s" % (r.returncode, r.stdout[-2000:] + r.stderr[-2000:])
    return name, None


@pytest.mark.slow
def test_every_mutant_fails_a_pin(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda kv: _run_mutant(kv[0], kv[1][0], kv[1][1], str(tmp_path)), MUTANTS.items()))
    problems = {n: msg for n, msg in results if msg}
    assert not problems, problems


def test_unmutated_oracle_passes_the_fast_pins(tmp_path):
    """The harness itself: the real oracle, built the same way, passes."""
    name, msg = _run_mutant("identity", "int orc_route(", "int orc_route(", str(tmp_path))
    assert msg == "survived: every pin passed"
