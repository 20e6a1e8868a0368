/*
 * vc_oracle.c -- plain CPU oracle for VC-Attention FP8 (V-Smooth + ExpCast-FP8).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant generator with the HIP
 * library: every step below is written from the source pages and from the OCP
 * 8-bit floating point definition, in the order those describe it, with no
 * blocking or fusion beyond what the method states.
 *
 * Sources (the pages are web articles about VC-Attention):
 *   [P1] "VC-Attention et FLUX 3 accelerent la generation d'images sur Blackwell"
 *        (ip73.fr), introduction (block scales fixed by the block maximum; V-Smooth
 *        reorders value tokens by a light online clustering; ExpCast-FP8 maps
 *        log-domain scores straight to E4M3 probability codes) and section
 *        "Le compromis entre vitesse et fidelite" (repair budget rho = 0.005 picks
 *        the tokens with the largest quantisation error and corrects their residual).
 *   [P5] "VC-Attention acelera atencao em modelos de video de IA em ate 3,58x sem
 *        retreinamento" (noticiai.com.br): section "Por que a atencao e o gargalo"
 *        (Q/K smoothing of earlier methods; FP32 softmax is the slowest stage),
 *        section "V-Smooth: corrigindo outliers de valor" (Group / Demean / Restore),
 *        section "ExpCast-FP8: eliminando o gargalo do softmax" (an E4M3 byte read
 *        as an integer is about 8*log2(v)+56; one fused multiply-add writes it).
 *   OCP "8-bit Floating Point Specification (OFP8)", E4M3 format.
 *
 * Readings taken where the pages are silent (each is also listed in the design
 * notes of the repository):
 *   - k-means is Lloyd's algorithm with a fixed iteration count on fixed-point
 *     values: per (batch, head) every value is scaled by 2^sh, the largest power
 *     of two that keeps max|v| * 2^sh below 2^13, and rounded to an integer u
 *     (the "lightweight" clustering: 14-bit values, exact integer distances).
 *     Forgy initial centroids are drawn by a seeded splitmix64 partial
 *     Fisher-Yates shuffle; the distance is ||c||^2 - 2 u.c computed exactly in
 *     integers; ties go to the lowest cluster id; a non-empty cluster moves to
 *     the mean of its members rounded to the nearest integer (ties to even), an
 *     empty one keeps its centroid; labels are those of the last assignment.
 *     With OC_WARM_START the Lloyd rounds start instead from the centroids
 *     passed in the output array (those of a previous denoising step): each is
 *     scaled by 2^sh of the current values, rounded to the nearest integer (ties
 *     to even) and clamped to [-2^13, 2^13 - 1].
 *   - means (K channel mean, V block means, centroids) are exact sums of values
 *     rounded to 2^-24 fixed point, divided once in fp64, rounded to fp32.
 *   - the permutation is a stable sort of positions by cluster id; Q follows it
 *     when VC_PERMUTE_Q is set and the output is written back in original order.
 *   - ExpCast code = clamp(rne(fma_f32(S_raw, alpha, bias - M)), 0, 126) with
 *     bias = 56 + 8k (k = 8 by default): the shift 8k cancels between P.V and the
 *     row sum; the row maximum M moves once per 128-key block, before that block's
 *     codes, and only when the block maximum exceeds it by more than tau code
 *     units (tau = 0 is the textbook online softmax).
 *   - the row sum adds the decoded codes that P.V uses; Restore adds
 *     (row sum of the block) * (block mean) to the accumulator.
 *   - raw scores S_raw = q.k of the E4M3 codes: the exact dot product of the
 *     decoded codes, rounded once to fp32.  The pages run this product on FP8
 *     tensor cores and fix no accumulation precision; the exact sum is the plain
 *     reading.  OC_MFMA_RULE (a diagnostic, never the reference) replaces it by
 *     a model of one FP8 matrix instruction measured on gfx950 (16x16x128
 *     E4M3): the 128 channels form 16 groups of 8 consecutive channels; inside a
 *     group every product is cut toward zero to a multiple of 2^(E-13), E being
 *     the largest exponent sum e(q)+e(k) over the group's nonzero products
 *     (e = exponent field - 7, or -6 for subnormals); the group sums are added
 *     and rounded once to fp32.  It is fitted to probe measurements, so it only
 *     serves to explain code differences, not to decide parity.
 *   - repair: m = ceil(rho*N) tokens per (batch, head) with the largest
 *     sum_c (sV_c * delta_c)^2, ties to the lower position; their residual error
 *     delta (in V code units, stored as bf16) is added with codes formed from the
 *     final row maximum; the row sum is left unchanged. *
 *   - 4-bit residual (OC_V4): the pages also run V-Smooth with the residual in
 *     NVFP4 [P5 "V-Smooth", Demean]; here in the gfx950-native MX form.  Per
 *     128-position block, channel and group of 32 consecutive positions (key
 *     k of the block is in group k/32: the MX block of the OCP Microscaling
 *     format is 32 consecutive elements), X = floor(log2 max|r|) - 2 kept in
 *     [-126, 127] (2^X a normal fp32 scale; -126 for an all-zero group), and the
 *     code is E2M1(r * 2^-X), nearest with ties to the even code, saturating at
 *     6, no negative zero.  There
 *     is no per-channel scale (sV = 1, mu' = mu), the repair error and the
 *     stored repair residuals are in real units, and P stays the ExpCast FP8
 *     code (the pages apply ExpCast only at 8 bits, so P's format is ours).
 *   - Q smoothing (OC_SMOOTH_Q): the pages name the query and key smoothing of
 *     earlier methods (SageAttention2) [P5 "Por que a atencao e o gargalo"];
 *     here each 128-position query block b subtracts its channel mean qbar_b
 *     (an exact fixed-point mean, like the V means) before its codes and scale
 *     are formed, and the dropped part returns as a per-key term of the score:
 *     delta_bj = qbar_b . k~_j, an fp32 fma chain over channels 0..127 with the
 *     same fp32 k~ = k - kbar the K codes come from, and d_bj = fp32(c0 *
 *     delta_bj) in code units.  A score becomes t = fma(S_raw, alpha, d_bj); the
 *     block maximum is taken over t, and code = clamp(rne(t + (56 + 8k - M)),
 *     0, 126), the sum an fp32 add.  Repaired keys use the same d.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -mfma -shared -fPIC (fp32 operations
 * must not be contracted; fmaf is always an explicit single-rounding fma).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OC_VSMOOTH 1u
#define OC_REPAIR 2u
#define OC_PERMUTE_Q 4u
#define OC_WARM_START 32u
#define OC_V4 64u
#define OC_SMOOTH_Q 128u
#define OC_MFMA_RULE 256u /* diagnostic score model, see the header */

typedef struct {
  int32_t B, H, N, d;     /* d must be 128 */
  int32_t C, T;           /* clusters, Lloyd iterations */
  uint64_t seed;
  float rho;              /* repair budget */
  float sm_scale;         /* softmax scale (1/sqrt(d) when <= 0) */
  int32_t expcast_k;      /* additive shift k of the ExpCast bias 56 + 8k */
  float tau;              /* lazy-max slack, code units */
  uint32_t flags;
} oc_params;

/* Per-head outputs of the prepare stage; every array holds nheads slots. */
typedef struct {
  int32_t *labels;   /* [nh][N]   cluster id of each original token            */
  int32_t *perm;     /* [nh][N]   position -> original token index              */
  int32_t *iperm;    /* [nh][N]   original token index -> position              */
  float *centroids;  /* [nh][C][d] centroids after the last update               */
  float *kbar;       /* [nh][d]   channel mean of K                             */
  uint8_t *q8;       /* [nh][Npad][d] Q codes, position order                    */
  uint8_t *k8;       /* [nh][Npad][d] K codes (smoothed K), position order       */
  float *sq, *sk;    /* [nh][nblk] block scales                                  */
  float *mu;         /* [nh][nblk][d] block means of V (real units)              */
  float *mup;        /* [nh][nblk][d] block means in V code units (mu * inv)     */
  uint8_t *v8;       /* [nh][Npad][d] residual codes, position order             */
  float *sv, *inv;   /* [nh][d] per-channel residual scale and its inverse       */
  float *err;        /* [nh][N]  repair criterion per position                   */
  int32_t *rep_pos;  /* [nh][mcap] repaired positions, ascending                 */
  uint16_t *rep_delta; /* [nh][mcap][d] bf16 residual error, V code units        */
  int8_t *vexp;      /* [nh][nblk][4][d] MX exponents of the 4-bit residual (OC_V4) */
  float *qbar;       /* [nh][nblk][d] query block means (OC_SMOOTH_Q)            */
  float *qbias;      /* [nh][nblk][Npad] score correction c0 * qbar_b . k~_j in
                        code units, query block b, key position j (OC_SMOOTH_Q) */
  int32_t mcap;      /* capacity of the repair arrays (>= m)                     */
} oc_prep;

/* ------------------------------------------------------------------------- */
/* Scalar formats                                                            */
/* ------------------------------------------------------------------------- */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* bf16 round-to-nearest-even from fp32 (finite inputs). */
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP E4M3 (E4M3FN): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent
 * field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; no infinities. */
double oc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest E4M3 value with ties to even mantissa, magnitudes at or above 448
 * saturate to 448, the sign is kept (so -0 and tiny negatives give 0x80). */
uint8_t oc_e4m3_encode(float xf) {
  double x = (double)xf, a = fabs(x);
  uint8_t sign = signbit(xf) ? 0x80 : 0x00;
  int code;
  if (isnan(xf)) return 0x7f;
  if (a >= 448.0) {
    code = 0x7e;
  } else if (a < ldexp(1.0, -6)) {
    /* subnormal band: multiples of 2^-9; m == 8 is the smallest normal (code 8) */
    code = (int)rint(a * 512.0);
  } else {
    int e;
    double fr = frexp(a, &e); /* a = fr * 2^e, fr in [0.5, 1) */
    int ue = e - 1;           /* a = (2 fr) * 2^ue, 2 fr in [1, 2) */
    int m = (int)rint((2.0 * fr - 1.0) * 8.0);
    if (m == 8) {
      m = 0;
      ue += 1;
    }
    code = ((ue + 7) << 3) | m;
    if (code > 0x7e) code = 0x7e;
  }
  return (uint8_t)(sign | code);
}

/* ExpCast-FP8 [P5 "ExpCast-FP8"]: one fp32 fma from the raw score to the byte. */
/* OCP FP4 E2M1 (OCP Microscaling Formats v1.0): magnitude codes 0..7 are 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.  Used by the 4-bit V residual (OC_V4),
 * the NVFP4 variant of V-Smooth [P5 "V-Smooth", Demean] in the gfx950-native MX
 * form. */
double oc_e2m1_decode(uint8_t c) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[c & 7];
  return (c & 8) ? -v : v;
}

/* Nearest E2M1 value, ties to the even code, saturating at 6; a result of
 * magnitude 0 is the code 0 (no negative zero). */
uint8_t oc_e2m1_encode(float y) {
  float a = fabsf(y);
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double dc = fabs((double)a - oc_e2m1_decode((uint8_t)c));
    double db = fabs((double)a - oc_e2m1_decode((uint8_t)best));
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  if (best == 0) return 0;
  return (uint8_t)(best | (y < 0.0f ? 8 : 0));
}

/* MX shared exponent of a 32-value group whose largest magnitude is a: the X
 * with a * 2^-X in [4, 8), i.e. floor(log2 a) - 2 (E2M1's largest binade starts
 * at 4), kept in [-126, 127] so that the group scale 2^X is a normal fp32 power
 * of two (E8M0's 2^-127 has no normal fp32 form); -126 when the group is all
 * zero. */
int oc_mx_exponent(float a) {
  if (!(a > 0.0f)) return -126;
  int e;
  frexpf(a, &e); /* a = m 2^e with m in [0.5, 1): floor(log2 a) = e - 1 */
  int x = e - 3;
  return x < -126 ? -126 : (x > 127 ? 127 : x);
}

/* 32-key groups of a 128-key block for the 4-bit residual: consecutive
 * positions, key k (0..127) in group k / 32. */
int oc_v4_group(int k) { return k >> 5; }

uint8_t oc_expcast(float s_raw, float alpha, float beta) {
  float y = rintf(fmaf(s_raw, alpha, beta));
  if (!(y > 0.0f)) return 0; /* also maps -inf (masked keys) to 0 */
  if (y > 126.0f) return 126;
  return (uint8_t)y;
}

/* splitmix64 (Steele, Lea, Flood 2014; Vigna's public-domain reference). */
static uint64_t sm64_next(uint64_t *s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Value rounded to the 2^-24 fixed-point grid, as an exact integer. */
static int64_t fx24(float x) { return llrintf(x * 16777216.0f); }

static float fixed_mean(int64_t sum, int64_t n) {
  return (float)(((double)sum * 0x1p-24) / (double)n);
}

/* Block scale and inverse from the block maximum [P1 introduction]. */
static void scale_from_amax(float amax, float *s, float *inv) {
  if (amax < 0x1p-100f) {
    *s = 1.0f;
    *inv = 1.0f;
  } else {
    *s = amax / 448.0f;
    *inv = 448.0f / amax;
  }
}

static int32_t repair_count(const oc_params *P) {
  double m;
  if (!(P->flags & OC_REPAIR) || !(P->rho > 0.0f)) return 0;
  m = ceil((double)P->rho * (double)P->N);
  if (m > P->N) m = P->N;
  return (int32_t)m;
}

int32_t oc_repair_count(const oc_params *P) { return repair_count(P); }

/* ------------------------------------------------------------------------- */
/* Prepare: V-Smooth Group [P5 "V-Smooth", Group]                             */
/* ------------------------------------------------------------------------- */

/* Forgy initial centroid indices: partial Fisher-Yates over [0, N). */
void oc_kmeans_init_indices(uint64_t seed, int64_t head, int32_t N, int32_t C, int32_t *out) {
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
  uint64_t st = seed ^ (0x9E3779B97F4A7C15ull * (uint64_t)(head + 1));
  for (int32_t i = 0; i < N; ++i) idx[i] = i;
  for (int32_t i = 0; i < C; ++i) {
    uint64_t r = sm64_next(&st);
    int32_t j = i + (int32_t)(r % (uint64_t)(N - i));
    int32_t t = idx[i];
    idx[i] = idx[j];
    idx[j] = t;
    out[i] = idx[i];
  }
  free(idx);
}

/* Fixed-point exponent of one head: max|v| * 2^sh < 2^13 <= 2 * max|v| * 2^sh. */
int oc_kmeans_shift(const float *v, int64_t n) {
  float a = 0.0f;
  int e;
  for (int64_t i = 0; i < n; ++i)
    if (fabsf(v[i]) > a) a = fabsf(v[i]);
  if (a == 0.0f) return 0;
  frexpf(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  return 13 - e;
}

static void kmeans_head(const oc_params *P, int64_t head, const float *v /*[N][d]*/,
                        int32_t *labels, float *cent /*[C][d]*/) {
  const int N = P->N, d = P->d, C = P->C;
  const int sh = oc_kmeans_shift(v, (int64_t)N * d);
  int32_t *init = (int32_t *)malloc(sizeof(int32_t) * (size_t)C);
  int32_t *u = (int32_t *)malloc(sizeof(int32_t) * (size_t)N * d);
  int64_t *c = (int64_t *)malloc(sizeof(int64_t) * (size_t)C * d);
  int64_t *cc = (int64_t *)malloc(sizeof(int64_t) * (size_t)C);
  int64_t *sum = (int64_t *)malloc(sizeof(int64_t) * (size_t)C * d);
  int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * (size_t)C);

  for (size_t i = 0; i < (size_t)N * d; ++i) u[i] = (int32_t)llrintf(ldexpf(v[i], sh));
  if (P->flags & OC_WARM_START) {
    /* previous step's centroids, in the current fixed-point scale */
    for (size_t i = 0; i < (size_t)C * d; ++i) {
      int64_t x = llrintf(ldexpf(cent[i], sh));
      c[i] = x < -8192 ? -8192 : (x > 8191 ? 8191 : x);
    }
  } else {
    oc_kmeans_init_indices(P->seed, head, N, C, init);
    for (int k = 0; k < C; ++k)
      for (int ch = 0; ch < d; ++ch) c[(size_t)k * d + ch] = u[(size_t)init[k] * d + ch];
  }

  for (int it = 0; it < P->T; ++it) {
    /* assignment step: argmin_k ||c_k||^2 - 2 u.c_k, exact integers */
    for (int k = 0; k < C; ++k) {
      int64_t s = 0;
      for (int ch = 0; ch < d; ++ch) s += c[(size_t)k * d + ch] * c[(size_t)k * d + ch];
      cc[k] = s;
    }
    for (int j = 0; j < N; ++j) {
      const int32_t *uj = u + (size_t)j * d;
      int best = 0;
      int64_t bestD = 0;
      for (int k = 0; k < C; ++k) {
        int64_t dot = 0, D;
        for (int ch = 0; ch < d; ++ch) dot += (int64_t)uj[ch] * c[(size_t)k * d + ch];
        D = cc[k] - 2 * dot;
        if (k == 0 || D < bestD) {
          best = k;
          bestD = D;
        }
      }
      labels[j] = best;
    }
    /* update step: each non-empty cluster moves to the rounded mean of its members */
    memset(sum, 0, sizeof(int64_t) * (size_t)C * d);
    memset(cnt, 0, sizeof(int64_t) * (size_t)C);
    for (int j = 0; j < N; ++j) {
      int k = labels[j];
      cnt[k] += 1;
      for (int ch = 0; ch < d; ++ch) sum[(size_t)k * d + ch] += u[(size_t)j * d + ch];
    }
    for (int k = 0; k < C; ++k)
      if (cnt[k] > 0)
        for (int ch = 0; ch < d; ++ch) /* |sum| < 2^34: the quotient rounds once, exactly */
          c[(size_t)k * d + ch] = llrint((double)sum[(size_t)k * d + ch] / (double)cnt[k]);
  }
  for (int k = 0; k < C; ++k)
    for (int ch = 0; ch < d; ++ch) cent[(size_t)k * d + ch] = ldexpf((float)c[(size_t)k * d + ch], -sh);
  free(init);
  free(u);
  free(c);
  free(cc);
  free(sum);
  free(cnt);
}

/* ------------------------------------------------------------------------- */
/* Prepare: one (batch, head)                                                 */
/* ------------------------------------------------------------------------- */

static float sm_scale_of(const oc_params *P) {
  return P->sm_scale > 0.0f ? P->sm_scale : (float)(1.0 / sqrt((double)P->d));
}

/* c0 converts a raw score (code units of Q times code units of K, times the two
 * block scales) to ExpCast code units: 8 * log2(e) * softmax scale. */
static float code_gain(const oc_params *P) {
  return (float)(8.0 * 1.4426950408889634074 * (double)sm_scale_of(P));
}

/* Value of residual code `code` of position p, channel c, in the units of the
 * residual x: the E4M3 value (V code units), or with the 4-bit residual the E2M1
 * value times its group's power of two (real units; exact in fp32). */
static float vq_value(const oc_prep *o, int slot, int nblk, int d, int v4, int p, int c, uint8_t code) {
  if (!v4) return (float)oc_e4m3_decode(code);
  int b = p / 128;
  int X = o->vexp[(((size_t)slot * nblk + b) * 4 + oc_v4_group(p - b * 128)) * d + c];
  return ldexpf((float)oc_e2m1_decode(code), X);
}

static void prepare_head(const oc_params *P, int64_t head, const uint16_t *qh, const uint16_t *kh,
                         const uint16_t *vh, oc_prep *o, int slot) {
  const int N = P->N, d = P->d, C = P->C;
  const int nblk = (N + 127) / 128, Npad = nblk * 128;
  const int vs = (P->flags & OC_VSMOOTH) != 0;
  const int v4 = (P->flags & OC_V4) != 0;
  const int sq_on = (P->flags & OC_SMOOTH_Q) != 0;
  const int m = repair_count(P);
  float *q = (float *)malloc(sizeof(float) * (size_t)N * d);
  float *k = (float *)malloc(sizeof(float) * (size_t)N * d);
  float *v = (float *)malloc(sizeof(float) * (size_t)N * d);
  float *x = (float *)malloc(sizeof(float) * (size_t)N * d); /* scaled residual, position order */
  int32_t *labels = o->labels + (size_t)slot * N;
  int32_t *perm = o->perm + (size_t)slot * N;
  int32_t *iperm = o->iperm + (size_t)slot * N;
  float *kbar = o->kbar + (size_t)slot * d;
  uint8_t *q8 = o->q8 + (size_t)slot * Npad * d;
  uint8_t *k8 = o->k8 + (size_t)slot * Npad * d;
  uint8_t *v8 = o->v8 + (size_t)slot * Npad * d;
  float *sq = o->sq + (size_t)slot * nblk, *sk = o->sk + (size_t)slot * nblk;
  float *mu = o->mu + (size_t)slot * nblk * d, *mup = o->mup + (size_t)slot * nblk * d;
  float *sv = o->sv + (size_t)slot * d, *inv = o->inv + (size_t)slot * d;
  float *err = o->err + (size_t)slot * N;

  for (size_t i = 0; i < (size_t)N * d; ++i) {
    q[i] = bf16_to_f32(qh[i]);
    k[i] = bf16_to_f32(kh[i]);
    v[i] = bf16_to_f32(vh[i]);
  }

  /* Group: k-means labels, then a stable sort of positions by label. */
  if (vs) {
    int64_t *start = (int64_t *)calloc((size_t)C + 1, sizeof(int64_t));
    kmeans_head(P, head, v, labels, o->centroids + (size_t)slot * C * d);
    for (int j = 0; j < N; ++j) start[labels[j] + 1] += 1;
    for (int kk = 0; kk < C; ++kk) start[kk + 1] += start[kk];
    for (int j = 0; j < N; ++j) perm[start[labels[j]]++] = j;
    free(start);
  } else {
    for (int j = 0; j < N; ++j) {
      labels[j] = 0;
      perm[j] = j;
    }
    memset(o->centroids + (size_t)slot * C * d, 0, sizeof(float) * (size_t)C * d);
  }
  for (int p = 0; p < N; ++p) iperm[perm[p]] = p;

  /* K smoothing: subtract the channel mean of K over all N tokens [P5 "Por que..."]. */
  for (int c = 0; c < d; ++c) {
    int64_t s = 0;
    for (int j = 0; j < N; ++j) s += fx24(k[(size_t)j * d + c]);
    kbar[c] = fixed_mean(s, N);
  }

  /* Per-128-position-block E4M3 quantisation of Q and smoothed K [P1 intro].
   * With OC_SMOOTH_Q the Q block first subtracts its channel mean. */
  memset(q8, 0, (size_t)Npad * d);
  memset(k8, 0, (size_t)Npad * d);
  for (int b = 0; b < nblk; ++b) {
    int p0 = b * 128, p1 = p0 + 128 < N ? p0 + 128 : N;
    float aq = 0.0f, ak = 0.0f, s, iv;
    float qm[128];
    for (int c = 0; c < d; ++c) {
      int64_t sum = 0;
      if (sq_on)
        for (int p = p0; p < p1; ++p) sum += fx24(q[(size_t)((P->flags & OC_PERMUTE_Q) ? perm[p] : p) * d + c]);
      qm[c] = sq_on ? fixed_mean(sum, p1 - p0) : 0.0f;
      if (sq_on) o->qbar[((size_t)slot * nblk + b) * d + c] = qm[c];
    }
    for (int p = p0; p < p1; ++p) {
      int jq = (P->flags & OC_PERMUTE_Q) ? perm[p] : p, jk = perm[p];
      for (int c = 0; c < d; ++c) {
        float xq = q[(size_t)jq * d + c] - qm[c];
        float xk = k[(size_t)jk * d + c] - kbar[c];
        if (fabsf(xq) > aq) aq = fabsf(xq);
        if (fabsf(xk) > ak) ak = fabsf(xk);
      }
    }
    scale_from_amax(aq, &s, &iv);
    sq[b] = s;
    for (int p = p0; p < p1; ++p) {
      int jq = (P->flags & OC_PERMUTE_Q) ? perm[p] : p;
      for (int c = 0; c < d; ++c) q8[(size_t)p * d + c] = oc_e4m3_encode((q[(size_t)jq * d + c] - qm[c]) * iv);
    }
    scale_from_amax(ak, &s, &iv);
    sk[b] = s;
    for (int p = p0; p < p1; ++p) {
      int jk = perm[p];
      for (int c = 0; c < d; ++c) {
        float xk = k[(size_t)jk * d + c] - kbar[c];
        k8[(size_t)p * d + c] = oc_e4m3_encode(xk * iv);
      }
    }
  }

  /* Score correction of the smoothed queries: d_bj = fp32(c0 * qbar_b . k~_j),
   * the dot product an fp32 fma chain in channel order (padding keys: 0). */
  if (sq_on) {
    const float c0 = code_gain(P);
    for (int b = 0; b < nblk; ++b) {
      const float *qm = o->qbar + ((size_t)slot * nblk + b) * d;
      float *db = o->qbias + ((size_t)slot * nblk + b) * Npad;
      for (int p = 0; p < Npad; ++p) {
        float delta = 0.0f;
        if (p < N)
          for (int c = 0; c < d; ++c) delta = fmaf(qm[c], k[(size_t)perm[p] * d + c] - kbar[c], delta);
        db[p] = p < N ? c0 * delta : 0.0f;
      }
    }
  }

  /* Demean: each 128-position block of permuted V subtracts its own mean
   * [P5 "V-Smooth", Demean]; residuals get one E4M3 scale per channel. */
  for (int b = 0; b < nblk; ++b) {
    int p0 = b * 128, p1 = p0 + 128 < N ? p0 + 128 : N;
    for (int c = 0; c < d; ++c) {
      int64_t s = 0;
      if (vs) {
        for (int p = p0; p < p1; ++p) s += fx24(v[(size_t)perm[p] * d + c]);
        mu[(size_t)b * d + c] = fixed_mean(s, p1 - p0);
      } else {
        mu[(size_t)b * d + c] = 0.0f;
      }
    }
  }
  memset(v8, 0, (size_t)Npad * d);
  if (v4) {
    /* 4-bit residual [P5 "V-Smooth", Demean: NVFP4 at 4 bits], as MXFP4: one
     * power-of-two scale per 32-key group of a block and channel, E2M1 codes of
     * the residual in real units; no per-channel scale (sV = 1). */
    int8_t *vexp = o->vexp + (size_t)slot * nblk * 4 * d;
    for (int c = 0; c < d; ++c) {
      sv[c] = 1.0f;
      inv[c] = 1.0f;
    }
    for (int b = 0; b < nblk; ++b)
      for (int c = 0; c < d; ++c) {
        float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int p = b * 128; p < b * 128 + 128 && p < N; ++p) {
          float r = v[(size_t)perm[p] * d + c] - mu[(size_t)b * d + c];
          int g = oc_v4_group(p - b * 128);
          if (fabsf(r) > a[g]) a[g] = fabsf(r);
        }
        for (int g = 0; g < 4; ++g) vexp[((size_t)b * 4 + g) * d + c] = (int8_t)oc_mx_exponent(a[g]);
      }
    for (int p = 0; p < N; ++p)
      for (int c = 0; c < d; ++c) {
        int b = p / 128, X = vexp[((size_t)b * 4 + oc_v4_group(p - b * 128)) * d + c];
        float r = v[(size_t)perm[p] * d + c] - mu[(size_t)b * d + c];
        x[(size_t)p * d + c] = r;
        v8[(size_t)p * d + c] = oc_e2m1_encode(ldexpf(r, -X));
      }
  } else {
    for (int c = 0; c < d; ++c) {
      float a = 0.0f;
      for (int p = 0; p < N; ++p) {
        float r = v[(size_t)perm[p] * d + c] - mu[(size_t)(p / 128) * d + c];
        if (fabsf(r) > a) a = fabsf(r);
      }
      scale_from_amax(a, &sv[c], &inv[c]);
    }
    for (int p = 0; p < N; ++p)
      for (int c = 0; c < d; ++c) {
        float r = v[(size_t)perm[p] * d + c] - mu[(size_t)(p / 128) * d + c];
        float xx = r * inv[c];
        x[(size_t)p * d + c] = xx;
        v8[(size_t)p * d + c] = oc_e4m3_encode(xx);
      }
  }
  for (int b = 0; b < nblk; ++b)
    for (int c = 0; c < d; ++c) mup[(size_t)b * d + c] = mu[(size_t)b * d + c] * inv[c];

  /* Repair set [P1 "Le compromis..."]: per-position squared quantisation error of
   * the value residual in real units, fp32 fma chain over channels. */
  for (int p = 0; p < N; ++p) {
    float e = 0.0f;
    for (int c = 0; c < d; ++c) {
      float dl = x[(size_t)p * d + c] - vq_value(o, slot, nblk, d, v4, p, c, v8[(size_t)p * d + c]);
      float t = sv[c] * dl;
      e = fmaf(t, t, e);
    }
    err[p] = e;
  }
  if (m > 0) {
    /* top m by (err descending, position ascending): repeated selection of the
     * best remaining position is slow but plainly correct. */
    uint8_t *taken = (uint8_t *)calloc((size_t)N, 1);
    int32_t *sel = o->rep_pos + (size_t)slot * o->mcap;
    uint16_t *dl = o->rep_delta + (size_t)slot * o->mcap * d;
    int32_t n = 0;
    for (int i = 0; i < m; ++i) {
      int best = -1;
      for (int p = 0; p < N; ++p) {
        if (taken[p]) continue;
        if (best < 0 || err[p] > err[best]) best = p;
      }
      taken[best] = 1;
    }
    for (int p = 0; p < N; ++p)
      if (taken[p]) {
        sel[n] = p;
        for (int c = 0; c < d; ++c) {
          float de = x[(size_t)p * d + c] - vq_value(o, slot, nblk, d, v4, p, c, v8[(size_t)p * d + c]);
          dl[(size_t)n * d + c] = f32_to_bf16(de);
        }
        ++n;
      }
    free(taken);
  }
  free(q);
  free(k);
  free(v);
  free(x);
}

/* Prepare the heads listed in heads[0..nheads) (global index b*H + h); slot i of
 * every output array receives heads[i].  Inputs are bf16 [B][H][N][d]. */
int oc_prepare(const oc_params *P, const uint16_t *q, const uint16_t *k, const uint16_t *v,
               const int32_t *heads, int32_t nheads, oc_prep *o) {
  if (P->d != 128 || P->N < 1 || P->C < 1 || P->C > P->N || P->T < 1) return 1;
  if (o->mcap < repair_count(P)) return 2;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < nheads; ++i) {
    size_t off = (size_t)heads[i] * P->N * P->d;
    prepare_head(P, heads[i], q + off, k + off, v + off, o, i);
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Forward: online ExpCast softmax with Restore and repair                    */
/* ------------------------------------------------------------------------- */

/* Decoded value of every code, filled from oc_e4m3_decode before any
 * parallel region (a cache of the decoder, nothing more). */
static double DEC[256];
static int dec_ready = 0;
static void init_dec(void) {
  if (dec_ready) return;
  for (int c = 0; c < 256; ++c) DEC[c] = oc_e4m3_decode((uint8_t)c);
  dec_ready = 1;
}

/* Exact dot product of two E4M3 code rows (every product is a multiple of
 * 2^-18 below 2^18, so the fp64 sum is exact), rounded once to fp32. */
static float exact_score(const uint8_t *a, const uint8_t *b, int d) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) s += DEC[a[c]] * DEC[b[c]];
  return (float)s;
}

/* Exponent of an E4M3 code as the matrix unit aligns it: field - 7 for normal
 * codes, -6 for subnormal ones (their value is m/8 * 2^-6). */
static int code_exp(uint8_t c) {
  int e = (c >> 3) & 15;
  return e ? e - 7 : -6;
}

/* Dot product as the FP8 matrix instruction accumulates it: groups of 8
 * consecutive channels, each product cut toward zero to 13 bits below the
 * group's largest exponent sum, group sums added exactly (all terms are
 * multiples of 2^-31 below 2^24, so the fp64 sum is exact) and rounded once to
 * fp32. */
static float mfma_score(const uint8_t *a, const uint8_t *b, int d) {
  double s = 0.0;
  for (int g = 0; g < d; g += 8) {
    int emax = -1000;
    for (int c = g; c < g + 8; ++c)
      if (DEC[a[c]] != 0.0 && DEC[b[c]] != 0.0) {
        int e = code_exp(a[c]) + code_exp(b[c]);
        if (e > emax) emax = e;
      }
    if (emax == -1000) continue;
    for (int c = g; c < g + 8; ++c) {
      double p = DEC[a[c]] * DEC[b[c]];
      s += ldexp(trunc(ldexp(p, 13 - emax)), emax - 13);
    }
  }
  return (float)s;
}

static float raw_score(const oc_params *P, const uint8_t *a, const uint8_t *b, int d) {
  return (P->flags & OC_MFMA_RULE) ? mfma_score(a, b, d) : exact_score(a, b, d);
}

/* One query row.  pcodes (optional) receives the row's ExpCast codes and pvals
 * (optional) the fp32 value each code rounds, fma(S_raw, alpha, 56 + 8k - M)
 * (t + 56 + 8k - M with smoothed queries), both in key position order; keys past
 * N get code 0 and value -inf. */
static void forward_row(const oc_params *P, const oc_prep *o, int slot, int32_t row, double *out,
                        uint8_t *pcodes, float *pvals) {
  const int N = P->N, d = P->d;
  const int nblk = (N + 127) / 128, Npad = nblk * 128;
  const int m = repair_count(P);
  const uint8_t *q8 = o->q8 + (size_t)slot * Npad * d;
  const uint8_t *k8 = o->k8 + (size_t)slot * Npad * d;
  const uint8_t *v8 = o->v8 + (size_t)slot * Npad * d;
  const float *sq = o->sq + (size_t)slot * nblk, *sk = o->sk + (size_t)slot * nblk;
  const float *mup = o->mup + (size_t)slot * nblk * d;
  const float *sv = o->sv + (size_t)slot * d;
  const int p = (P->flags & OC_PERMUTE_Q) ? o->iperm[(size_t)slot * N + row] : row;
  const int a = p / 128;
  const int v4 = (P->flags & OC_V4) != 0;
  /* smoothed queries: per-key score term of this row's query block, code units */
  const float *dq = (P->flags & OC_SMOOTH_Q) ? o->qbias + ((size_t)slot * nblk + a) * Npad : NULL;
  const float c0 = code_gain(P);
  const float bias = (float)(56 + 8 * P->expcast_k);
  float M = -INFINITY;
  double ell = 0.0, acc[128];
  float S[128];
  uint8_t code[128];

  for (int c = 0; c < d; ++c) acc[c] = 0.0;
  for (int b = 0; b < nblk; ++b) {
    int j0 = b * 128, j1 = j0 + 128 < N ? j0 + 128 : N;
    float alpha = (sq[a] * sk[b]) * c0;
    float smax = -INFINITY, tmax, Mn, beta;
    double r, lb = 0.0;
    for (int j = j0; j < j1; ++j) {
      S[j - j0] = raw_score(P, q8 + (size_t)p * d, k8 + (size_t)j * d, d);
      if (dq) S[j - j0] = fmaf(S[j - j0], alpha, dq[j]); /* t, code units */
      if (S[j - j0] > smax) smax = S[j - j0];
    }
    tmax = dq ? smax : smax * alpha;
    Mn = (isinf(M) || (tmax - M) > P->tau) ? tmax : M;
    beta = bias - Mn;
    r = isinf(M) ? 0.0 : exp2(((double)M - (double)Mn) / 8.0);
    for (int j = j0; j < j1; ++j) {
      /* with smoothed queries fma(t, 1, beta) is the fp32 sum t + beta */
      code[j - j0] = dq ? oc_expcast(S[j - j0], 1.0f, beta) : oc_expcast(S[j - j0], alpha, beta);
      lb += DEC[code[j - j0]];
      if (pcodes) pcodes[j] = code[j - j0];
      if (pvals) pvals[j] = dq ? S[j - j0] + beta : fmaf(S[j - j0], alpha, beta);
    }
    ell = ell * r + lb;
    for (int c = 0; c < d; ++c) {
      double pv = 0.0;
      for (int j = j0; j < j1; ++j) {
        double vv = v4 ? (double)vq_value(o, slot, nblk, d, 1, j, c, v8[(size_t)j * d + c])
                       : DEC[v8[(size_t)j * d + c]];
        pv += DEC[code[j - j0]] * vv;
      }
      acc[c] = acc[c] * r + lb * (double)mup[(size_t)b * d + c] + pv;
    }
    M = Mn;
  }
  for (int j = N; j < Npad; ++j) {
    if (pcodes) pcodes[j] = 0;
    if (pvals) pvals[j] = -INFINITY;
  }

  /* repair: residual error of the selected tokens, weighted by final-M codes */
  for (int i = 0; i < m; ++i) {
    int j = o->rep_pos[(size_t)slot * o->mcap + i];
    int b = j / 128;
    float alpha = (sq[a] * sk[b]) * c0;
    float s = raw_score(P, q8 + (size_t)p * d, k8 + (size_t)j * d, d);
    double pw = dq ? DEC[oc_expcast(fmaf(s, alpha, dq[j]), 1.0f, bias - M)] : DEC[oc_expcast(s, alpha, bias - M)];
    const uint16_t *dl = o->rep_delta + ((size_t)slot * o->mcap + i) * d;
    for (int c = 0; c < d; ++c) acc[c] += pw * (double)bf16_to_f32(dl[c]);
  }
  for (int c = 0; c < d; ++c) out[c] = (double)sv[c] * acc[c] / ell;
}

/* Simulated output rows.  row_slot[i] selects the prepared head, row_index[i] is
 * the query row in ORIGINAL token order; out is [nrows][d] fp64.  pcodes and
 * pvals, when not NULL, receive [nrows][Npad] P codes and the fp32 values they
 * round, in key position order. */
int oc_forward_rows(const oc_params *P, const oc_prep *o, const int32_t *row_slot,
                    const int32_t *row_index, int32_t nrows, double *out, uint8_t *pcodes,
                    float *pvals) {
  const int Npad = ((P->N + 127) / 128) * 128;
  if (P->d != 128) return 1;
  init_dec();
#pragma omp parallel for schedule(dynamic, 4)
  for (int i = 0; i < nrows; ++i)
    forward_row(P, o, row_slot[i], row_index[i], out + (size_t)i * P->d,
                pcodes ? pcodes + (size_t)i * Npad : NULL, pvals ? pvals + (size_t)i * Npad : NULL);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Exact FP64 attention: softmax(q K^T * scale) V from the bf16 inputs.        */
/* ------------------------------------------------------------------------- */

int oc_exact_rows(const oc_params *P, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const int32_t *row_head, const int32_t *row_index, int32_t nrows, double *out) {
  const int N = P->N, d = P->d;
  const double scale = (double)sm_scale_of(P);
  if (d != 128) return 1;
#pragma omp parallel for schedule(dynamic, 4)
  for (int i = 0; i < nrows; ++i) {
    size_t off = (size_t)row_head[i] * N * d;
    const uint16_t *qi = q + off + (size_t)row_index[i] * d;
    double *s = (double *)malloc(sizeof(double) * (size_t)N);
    double mx = -INFINITY, den = 0.0;
    double *o = out + (size_t)i * d;
    for (int j = 0; j < N; ++j) {
      double t = 0.0;
      for (int c = 0; c < d; ++c)
        t += (double)bf16_to_f32(qi[c]) * (double)bf16_to_f32(k[off + (size_t)j * d + c]);
      s[j] = t * scale;
      if (s[j] > mx) mx = s[j];
    }
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j < N; ++j) {
      double w = exp(s[j] - mx);
      den += w;
      for (int c = 0; c < d; ++c) o[c] += w * (double)bf16_to_f32(v[off + (size_t)j * d + c]);
    }
    for (int c = 0; c < d; ++c) o[c] /= den;
    free(s);
  }
  return 0;
}

/* Array helpers used by the pins. */
void oc_e4m3_decode_array(const uint8_t *c, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oc_e4m3_decode(c[i]);
}
void oc_e4m3_encode_array(const float *x, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oc_e4m3_encode(x[i]);
}
void oc_expcast_array(const float *s, float alpha, float beta, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oc_expcast(s[i], alpha, beta);
}
/* Scores of n code-row pairs (rows of d bytes); exact != 0 selects the exact
 * dot product, else the diagnostic FP8 matrix-instruction model. */
void oc_score_array(const uint8_t *a, const uint8_t *b, int64_t n, int32_t d, int32_t exact,
                    float *out) {
  init_dec();
  for (int64_t i = 0; i < n; ++i)
    out[i] = exact ? exact_score(a + i * d, b + i * d, d) : mfma_score(a + i * d, b + i * d, d);
}
void oc_splitmix64_array(uint64_t state, uint64_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = sm64_next(&state);
}

void oc_e2m1_decode_array(const uint8_t *c, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oc_e2m1_decode(c[i]);
}
void oc_e2m1_encode_array(const float *x, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oc_e2m1_encode(x[i]);
}
void oc_mx_exponent_array(const float *a, int32_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oc_mx_exponent(a[i]);
}
