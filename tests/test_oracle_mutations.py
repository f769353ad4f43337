"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a scratch copy of the oracle's C
sources (a textual substitution that must match exactly once), builds that
copy with the oracle's own flags, and runs the pin suites against it in a
child process.  The case passes only when at least one pin fails: a mistake
the pins cannot see would leave that part of the oracle unpinned.

Nothing here touches the real oracle library or the GPU path.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
SOURCES = ["svdq_oracle.c", "awq_oracle.c", "qkv_oracle.c", "mxfp4_oracle.c"]
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_awq_pins.py",
             "tests/test_oracle_mx_pins.py", "tests/test_oracle_qkv_pins.py"]

# (id, file, text in the oracle, planted replacement)
MUTATIONS = [
    # smoothing as a division instead of a product with the fp32 reciprocal
    ("smooth_division", "svdq_oracle.c",
     "bf16_to_float(X[m * K + k]) * inv[k]", "bf16_to_float(X[m * K + k]) / lam[k]"),
    # code from a division by the scale instead of a product with fl32(1/s)
    ("code_division", "svdq_oracle.c", "float y = p[j] * inv;", "float y = p[j] / s;"),
    # W4A16 code and zero point from divisions
    ("awq_code_division", "awq_oracle.c", "const float y = w[j] * inv;",
     "const float y = w[j] / s;"),
    ("awq_zero_division", "awq_oracle.c", "const float zl = -lo * inv;",
     "const float zl = -lo / s;"),
    # ties away from zero instead of to even
    ("code_roundf", "svdq_oracle.c", "float c = rintf(y);", "float c = roundf(y);"),
    # scale as amax times a rounded 1/7
    ("scale_recip7", "svdq_oracle.c", "float s = amax / 7.0f;", "float s = amax * (1.0f / 7.0f);"),
    # codes in natural field order instead of the halves interleaved
    ("field_order", "svdq_oracle.c", "return 2 * (e % 8) + e / 8;", "return e;"),
    # the sign in the field's bit 3 instead of bit 5
    ("sign_bit", "svdq_oracle.c", "(blk[e] < 0 ? 32u : 0u)", "(blk[e] < 0 ? 8u : 0u)"),
    # the third image word folded into the wrong word (free bits of the other word)
    ("fold_word", "svdq_oracle.c", "return is_free_bit(o) ? o : 32 + o;",
     "return is_free_bit(o) ? 32 + o : o;"),
    # L2 read transposed
    ("l2_transposed", "svdq_oracle.c", "L2[(int64_t)i * N + n]", "L2[n * r + i]"),
    # bias dropped
    ("bias_dropped", "svdq_oracle.c", "acc += (double)bf16_to_float(bias[n]);", "(void)0;"),
    # GELU in its tanh form
    ("gelu_tanh", "svdq_oracle.c", "return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
     "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    # bf16 output rounded twice (fp64 -> fp32 -> bf16)
    ("bf16_double_round", "svdq_oracle.c", "double a = fabs(v);", "double a = fabs((double)(float)v);"),
    # one scale of the pair dropped from the rescale
    ("rescale_drops_sw", "svdq_oracle.c",
     "acc += (double)sa[m * G + g] * (double)sw[n * G + g] * (double)s;",
     "acc += (double)sa[m * G + g] * (double)s;"),
    # down-projection with L1 transposed
    ("l1_transposed", "svdq_oracle.c", "bf16_to_float(L1[k * r + i])", "bf16_to_float(L1[i * K + k])"),
    # W4A16 range that does not always contain zero
    ("awq_range_no_zero", "awq_oracle.c", "float lo = 0.0f, hi = 0.0f;",
     "float lo = w[0], hi = w[0];"),
    # MXFP4 ties away from the even code
    ("mx_ties_odd", "mxfp4_oracle.c", "(d == db && (c & 1) == 0)", "(d == db && (c & 1) == 1)"),
    # MXFP4 scale exponent off by one
    ("mx_scale_off_by_one", "mxfp4_oracle.c", "int e = (e2 - 1) - 2;", "int e = (e2 - 1) - 1;"),
    # rotary turn with the sine's sign flipped
    ("rotary_sign", "qkv_oracle.c", "const double o0 = va * c - vbv * sn;",
     "const double o0 = va * c + vbv * sn;"),
    # RMS norm without its epsilon
    ("rms_no_eps", "qkv_oracle.c", "sqrt(ss / (double)D + eps)", "sqrt(ss / (double)D)"),
]


def _build(srcdir, lib):
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-shared", "-fPIC"] + [os.path.join(srcdir, s) for s in SOURCES] + ["-o", lib, "-lm"]
    subprocess.check_call(cmd)


@pytest.mark.parametrize("mid,fname,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, mid, fname, old, new):
    srcdir = tmp_path / "src"
    srcdir.mkdir()
    for s in SOURCES:
        shutil.copy(os.path.join(ORACLE, s), srcdir / s)
    text = (srcdir / fname).read_text()
    assert text.count(old) == 1, "mutation %s: its target text must occur exactly once" % mid
    (srcdir / fname).write_text(text.replace(old, new))
    lib = str(tmp_path / "liboracle_mut.so")
    _build(str(srcdir), lib)
    env = dict(os.environ, SVDQ_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + PIN_FILES,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, ("mutation %s: the pins did not fail (rc %d)\n%s"
                               % (mid, r.returncode, r.stdout[-2000:]))
