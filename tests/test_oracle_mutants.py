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
    ("score_fp32_sum", "  double s = 0.0;\n  for (int c = 0; c < d; ++c) s += DEC[a[c]] * DEC[b[c]];",
     "  float s = 0.0f;\n  for (int c = 0; c < d; ++c) s += (float)(DEC[a[c]] * DEC[b[c]]);"),
    ("mean_denominator", "return (float)(((double)sum * 0x1p-24) / (double)n);",
     "return (float)(((double)sum * 0x1p-24) / (double)(n + 1));"),
    ("fx24_truncated", "static int64_t fx24(float x) { return llrintf(x * 16777216.0f); }",
     "static int64_t fx24(float x) { return (int64_t)(x * 16777216.0f); }"),
    ("repair_count_floor", "m = ceil((double)P->rho * (double)P->N);", "m = floor((double)P->rho * (double)P->N);"),
    ("lazy_max_ignored", "Mn = (isinf(M) || (tmax - M) > P->tau) ? tmax : M;", "Mn = (isinf(M) || tmax > M) ? tmax : M;"),
    ("warm_start_truncated", "int64_t x = llrintf(ldexpf(cent[i], sh));", "int64_t x = (int64_t)(ldexpf(cent[i], sh));"),
    ("repair_without_max", "DEC[oc_expcast(s, alpha, bias - M)];", "DEC[oc_expcast(s, alpha, bias)];"),
    ("repair_first_block_scale", "    float alpha = (sq[a] * sk[b]) * c0;\n    float s = raw_score",
     "    float alpha = (sq[a] * sk[0]) * c0;\n    float s = raw_score"),
    ("output_row_perm", "const int p = (P->flags & OC_PERMUTE_Q) ? o->iperm[(size_t)slot * N + row] : row;",
     "const int p = (P->flags & OC_PERMUTE_Q) ? o->perm[(size_t)slot * N + row] : row;"),
    ("forgy_duplicates", "int32_t j = i + (int32_t)(r % (uint64_t)(N - i));", "int32_t j = (int32_t)(r % (uint64_t)N);"),
    ("code_clamp_127", "if (y > 126.0f) return 126;", "if (y > 127.0f) return 127;"),
    ("e4m3_saturate_nan", "    code = 0x7e;\n  } else if (a < ldexp(1.0, -6)) {", "    code = 0x7f;\n  } else if (a < ldexp(1.0, -6)) {"),
    ("mx_exponent_floor", "return x < -126 ? -126 : (x > 127 ? 127 : x);", "return x < -127 ? -127 : (x > 127 ? 127 : x);"),
    ("kmeans_ties_high", "if (k == 0 || D < bestD) {", "if (k == 0 || D <= bestD) {"),
    ("e4m3_subnormal_scale", "    v = ldexp((double)m, -9);", "    v = ldexp((double)m, -10);"),
    ("exact_scale_dropped", "      s[j] = t * scale;", "      s[j] = t;"),
    ("exact_weight_squared", "      double w = exp(s[j] - mx);", "      double w = exp(2.0 * (s[j] - mx));"),
    ("empty_cluster_zeroed", "    for (int k = 0; k < C; ++k)\n      if (cnt[k] > 0)",
     "    for (int k = 0; k < C; ++k)\n      if (cnt[k] == 0) for (int ch = 0; ch < d; ++ch) c[(size_t)k * d + ch] = 0; else if (cnt[k] > 0)"),
    ("forgy_head_index", "uint64_t st = seed ^ (0x9E3779B97F4A7C15ull * (uint64_t)(head + 1));",
     "uint64_t st = seed ^ (0x9E3779B97F4A7C15ull * (uint64_t)(head + 2));"),
    ("tail_mean_full_block", "        mu[(size_t)b * d + c] = fixed_mean(s, p1 - p0);", "        mu[(size_t)b * d + c] = fixed_mean(s, 128);"),
    ("zero_amax_scale", "    *s = 1.0f;\n    *inv = 1.0f;", "    *s = 0.0f;\n    *inv = 1.0f;"),
    ("expcast_floor_code_1", "  if (!(y > 0.0f)) return 0; /* also maps -inf (masked keys) to 0 */",
     "  if (!(y > 0.0f)) return 1;"),
    ("e4m3_sign_dropped", "  uint8_t sign = signbit(xf) ? 0x80 : 0x00;", "  uint8_t sign = (xf < 0.0f) ? 0x80 : 0x00;"),
    ("repair_ties_later", "if (best < 0 || err[p] > err[best]) best = p;", "if (best < 0 || err[p] >= err[best]) best = p;"),
    ("smoothq_mean_unpermuted", "for (int p = p0; p < p1; ++p) sum += fx24(q[(size_t)((P->flags & OC_PERMUTE_Q) ? perm[p] : p) * d + c]);",
     "for (int p = p0; p < p1; ++p) sum += fx24(q[(size_t)p * d + c]);"),
    ("smoothq_code_alpha", "code[j - j0] = dq ? oc_expcast(S[j - j0], 1.0f, beta) : oc_expcast(S[j - j0], alpha, beta);",
     "code[j - j0] = dq ? oc_expcast(S[j - j0], alpha, beta) : oc_expcast(S[j - j0], alpha, beta);"),
    ("q_unpermuted_codes", "      int jq = (P->flags & OC_PERMUTE_Q) ? perm[p] : p, jk = perm[p];",
     "      int jq = p, jk = perm[p];"),
    ("v4_repair_delta_unscaled", "  if (!v4) return (float)oc_e4m3_decode(code);", "  if (!v4 || p >= 0) return (float)oc_e4m3_decode(code);"),
    ("bf16_round_truncated", "  u += 0x7fffu + ((u >> 16) & 1u);\n  return (uint16_t)(u >> 16);\n}",
     "  return (uint16_t)(u >> 16);\n}"),
    ("code_gain_ln", "return (float)(8.0 * 1.4426950408889634074 * (double)sm_scale_of(P));",
     "return (float)(8.0 * (double)sm_scale_of(P));"),
    ("default_scale_inverse_d", "return P->sm_scale > 0.0f ? P->sm_scale : (float)(1.0 / sqrt((double)P->d));",
     "return P->sm_scale > 0.0f ? P->sm_scale : (float)(1.0 / (double)P->d);"),
    ("warm_clamp_narrow", "c[i] = x < -8192 ? -8192 : (x > 8191 ? 8191 : x);", "c[i] = x < -4096 ? -4096 : (x > 4095 ? 4095 : x);"),
    ("v4_value_exponent_off", "  return ldexpf((float)oc_e2m1_decode(code), X);", "  return ldexpf((float)oc_e2m1_decode(code), X + 1);"),
    ("smoothq_repair_term_dropped",
     "double pw = dq ? DEC[oc_expcast(fmaf(s, alpha, dq[j]), 1.0f, bias - M)] : DEC[oc_expcast(s, alpha, bias - M)];",
     "double pw = dq ? DEC[oc_expcast(s, alpha, bias - M)] : DEC[oc_expcast(s, alpha, bias - M)];"),
    ("mup_unscaled", "    for (int c = 0; c < d; ++c) mup[(size_t)b * d + c] = mu[(size_t)b * d + c] * inv[c];",
     "    for (int c = 0; c < d; ++c) mup[(size_t)b * d + c] = mu[(size_t)b * d + c];"),
    ("output_scale_dropped", "  for (int c = 0; c < d; ++c) out[c] = (double)sv[c] * acc[c] / ell;",
     "  for (int c = 0; c < d; ++c) out[c] = acc[c] / ell;"),
    ("qblock_scale_of_key", "    float alpha = (sq[a] * sk[b]) * c0;\n    float smax",
     "    float alpha = (sk[a] * sk[b]) * c0;\n    float smax"),
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
