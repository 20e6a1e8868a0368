"""The oracle's pins catch plausible mistakes.

Each mutant below plants one mistake in a copy of oracle/vc_oracle.c (a wrong
rounding, a dropped term, a flipped sign, a wrong index or bound), builds it
with the oracle's own compiler flags and runs the oracle pin suites against it
(through the VC_ORACLE_LIB hook of oracle/oracle.py) in a subprocess.  Every
mutant must make at least one pin fail.  CPU only."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "vc_oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_scores.py", "tests/test_oracle_v4.py",
        "tests/test_oracle_smoothq.py"]

# (name, exact text in vc_oracle.c, replacement)
MUTANTS = [
    ("expcast_floor", "float y = rintf(fmaf(s_raw, alpha, beta));", "float y = floorf(fmaf(s_raw, alpha, beta));"),
    ("expcast_bias_64", "const float bias = (float)(56 + 8 * P->expcast_k);",
     "const float bias = (float)(64 + 8 * P->expcast_k);"),
    ("rescale_sign", "r = isinf(M) ? 0.0 : exp2(((double)M - (double)Mn) / 8.0);",
     "r = isinf(M) ? 0.0 : exp2(((double)Mn - (double)M) / 8.0);"),
    ("rowsum_not_rescaled", "ell = ell * r + lb;", "ell = ell + lb;"),
    ("restore_dropped", "acc[c] = acc[c] * r + lb * (double)mup[(size_t)b * d + c] + pv;",
     "acc[c] = acc[c] * r + pv;"),
    ("tail_keys_included", "int j0 = b * 128, j1 = j0 + 128 < N ? j0 + 128 : N;",
     "int j0 = b * 128, j1 = j0 + 128;"),
    ("kmeans_norm_dropped", "D = cc[k] - 2 * dot;", "D = -2 * dot;"),
    ("kmeans_mean_truncated", "c[(size_t)k * d + ch] = llrint((double)sum[(size_t)k * d + ch] / (double)cnt[k]);",
     "c[(size_t)k * d + ch] = (int64_t)((double)sum[(size_t)k * d + ch] / (double)cnt[k]);"),
    ("kmeans_shift_14", "return 13 - e;", "return 14 - e;"),
    ("sort_unstable", "for (int j = 0; j < N; ++j) perm[start[labels[j]]++] = j;",
     "for (int j = N - 1; j >= 0; --j) perm[start[labels[j]]++] = j;"),
    ("ksmooth_missing", "kbar[c] = fixed_mean(s, N);", "kbar[c] = 0.0f;"),
    ("e4m3_ties_up", "int m = (int)rint((2.0 * fr - 1.0) * 8.0);", "int m = (int)floor((2.0 * fr - 1.0) * 8.0 + 0.5);"),
    ("scale_inverse_off", "*inv = 448.0f / amax;", "*inv = 440.0f / amax;"),
    ("demean_next_block", "        float xx = r * inv[c];",
     "        float xx = (v[(size_t)perm[p] * d + c] - mu[(size_t)(((p / 128) + 1) % nblk) * d + c]) * inv[c];"),
    ("repair_smallest", "if (best < 0 || err[p] > err[best]) best = p;", "if (best < 0 || err[p] < err[best]) best = p;"),
    ("repair_error_unweighted", "float t = sv[c] * dl;", "float t = dl;"),
    ("v4_groups_strided", "int oc_v4_group(int k) { return k >> 5; }", "int oc_v4_group(int k) { return (k >> 4) & 3; }"),
    ("e2m1_ties_odd", "if (dc < db || (dc == db && (c & 1) == 0)) best = c;",
     "if (dc < db || (dc == db && (c & 1) == 1)) best = c;"),
    ("mx_exponent_off", "int x = e - 3;", "int x = e - 2;"),
    ("smoothq_kbar_dropped", "delta = fmaf(qm[c], k[(size_t)perm[p] * d + c] - kbar[c], delta);",
     "delta = fmaf(qm[c], k[(size_t)perm[p] * d + c], delta);"),
]


def _run_mutant(m, tmp):
    name, old, new = m
    src = open(SRC).read()
    if src.count(old) != 1:
        return name, "site", f"text found {src.count(old)} times"
    msrc = os.path.join(tmp, f"{name}.c")
    mlib = os.path.join(tmp, f"lib{name}.so")
    open(msrc, "w").write(src.replace(old, new))
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-mfma", "-fPIC", "-shared", msrc, "-o", mlib, "-lm"]
    cp = subprocess.run(cmd, capture_output=True, text=True)
    if cp.returncode != 0:
        return name, "build", cp.stderr[-400:]
    env = dict(os.environ, VC_ORACLE_LIB=mlib, OMP_NUM_THREADS="2")
    cp = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, ("killed" if cp.returncode != 0 else "survived"), cp.stdout[-600:]


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(4) as ex:
            res = list(ex.map(lambda m: _run_mutant(m, tmp), MUTANTS))
    bad = [(n, s, out) for n, s, out in res if s != "killed"]
    assert not bad, "\n".join(f"{n}: {s}\n{out}" for n, s, out in bad)
