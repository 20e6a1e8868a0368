// Prepare-stage kernels of VC-Attention FP8 for gfx950.
//
// Method (articles on VC-Attention: noticiai.com.br, sections "Por que a atencao
// e o gargalo" and "V-Smooth: corrigindo outliers de valor"; ip73.fr,
// introduction and section "Le compromis entre vitesse et fidelite"):
//   K smoothing     subtract the channel mean of K (softmax ignores it);
//   Q/K codes       one E4M3 scale per 128-token block, set by the block maximum;
//   Group           k-means over value tokens per (batch, head), then K and V (and
//                   Q) are permuted jointly so that clusters are contiguous;
//   Demean          each 128-position block subtracts its own mean, and only the
//                   residual is quantised, E4M3 with one scale per channel;
//   repair set      the ceil(rho*N) positions whose value codes lose the most.
//
// Every decision that yields an integer (cluster id, E4M3 code, selected token)
// is taken in exact integer arithmetic or in a fixed sequence of fp32 operations
// (explicit fma), so that the result does not depend on the order in which
// threads run: means are exact int64 sums of values rounded to a 2^-24 grid,
// divided once in fp64; k-means distances are exact integers on fixed-point
// values.  The library is built with -ffp-contract=off.
#include "vc_internal.h"

namespace vc {
namespace {

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float((h & 0xffffu) << 16); }

// x rounded to the 2^-24 grid, in units of 2^-24, as a double (exact: an
// integer-valued float).  Sums of up to 2^7 such values stay below 2^53 for
// inputs |x| < 2^22, so fp64 adds of them are exact and equal integer sums;
// gfx950 has no float -> int64 convert, so this costs 4 instructions per value
// instead of about 15.
__device__ __forceinline__ double fx24d(float x) {
  return (double)__builtin_rintf(x * 16777216.0f);
}

__device__ __forceinline__ float fixed_mean(long long s, long long n) {
  return (float)(((double)s * 0x1p-24) / (double)n);
}

// Two fp32 -> two OCP E4M3 bytes (round to nearest even) in bits 0..15.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

__device__ __forceinline__ float e4m3_val(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

__device__ __forceinline__ void scale_from_amax(float amax, float* s, float* inv) {
  if (amax < 0x1p-100f) {
    *s = 1.0f;
    *inv = 1.0f;
  } else {
    *s = amax / 448.0f;
    *inv = 448.0f / amax;
  }
}

__device__ __forceinline__ uint16_t f2bf_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint64_t splitmix(uint64_t& st) {
  uint64_t z = (st += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Column of key r inside a 128-key block of the channel-major V codes: the fused
// kernel's accumulator layout gives lane group g the keys 16t+4g+v (t = 0..7,
// v = 0..3) and the PV operand wants them as 32 consecutive bytes.
__device__ __forceinline__ int v_col(int r) { return 32 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3); }

// Column of repair slot s inside a 128-slot group of the repair residuals (bf16
// MFMA operand with 32-wide K chunks): slot 32u+16t'+4g+v -> column 32u+8g+4t'+v.
__device__ __forceinline__ int rep_col(int s) {
  const int u = s >> 5, tp = (s >> 4) & 1, g = (s >> 2) & 3, v = s & 3;
  return 32 * u + 8 * g + 4 * tp + v;
}

// E2M1 (OCP FP4) rounding of y, |y| < 8: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4,
// 6, ties to the even code, saturating at 6; a zero magnitude is code 0 (no
// negative zero).  Returns the code and the value it decodes to (code 0 is
// +0, whatever the sign of y).  Inside the binade
// [2^e, 2^(e+1)) the E2M1 values are the multiples of 2^(e-1) (0.5 below 2),
// and adding M = 2^(max(e,0)+22) leaves exactly that step as the sum's last bit:
// fp32 round-to-nearest-even of a + M, minus M, is the E2M1 rounding, and an
// even last bit is an even code.  The code is read off the rounded value's
// exponent and mantissa bits.  Plain VALU arithmetic, no compares.
__device__ __forceinline__ float e2m1_round(float y, uint32_t* code) {
  const float a = fabsf(y);
  const float M = __uint_as_float(max(__float_as_uint(a) & 0x7f800000u, 127u << 23) + (22u << 23));
  const float r = fminf((a + M) - M, 6.0f);
  // r in {0, 0.5, 1, 1.5, 2, 3, 4, 6}: b = bits >> 22 is 0, 252, 254, 255, ..., 259
  const uint32_t b = __float_as_uint(r) >> 22;
  const uint32_t m = max(b, 251u) - 251u - ((b + 2u) >> 8);
  const uint32_t sgn = (__float_as_uint(y) >> 28) & 8u;
  *code = m | (m != 0u ? sgn : 0u);
  return __uint_as_float(__float_as_uint(r) | ((*code & 8u) << 28));
}

// MX exponent of a group whose largest magnitude is amax: X with amax * 2^-X in
// [4, 8) (E2M1's top binade), kept in [-126, 127] so that 2^X is a normal fp32
// power of two; -126 for an all-zero group.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -126;
  const int x = __builtin_amdgcn_frexp_expf(amax) - 3;  // amax = f 2^e, f in [0.5, 1)
  return x < -126 ? -126 : (x > 127 ? 127 : x);
}

// 32-key group of key r of a block (4-bit residual).
__device__ __forceinline__ int v4_group(int r) { return 2 * (r >> 6) + ((r >> 3) & 1); }

// ---------------------------------------------------------------------------
// K channel sums: fixed-point partial sums over KSUM_CHUNK tokens; with WITH_V
// the same workgroup records max|V| of the chunk (the k-means fixed-point scale,
// needed only when k-means runs).
// grid (nkc, BH), 256 threads: thread = (row r = t/16, 8-channel group t%16).
template <bool WITH_V>
__global__ __launch_bounds__(256) void k_ksum(Args a) {
  __shared__ long long red[16][D];
  __shared__ float wm[4];
  const int bh = blockIdx.y, ch = blockIdx.x, t = threadIdx.x;
  const int cg = t & 15, r = t >> 4;
  const int j0 = ch * KSUM_CHUNK, j1 = min(j0 + KSUM_CHUNK, a.N);
  const uint16_t* kh = a.k + (size_t)bh * a.N * D;
  const uint16_t* vh = a.v + (size_t)bh * a.N * D;
  // a thread sums at most KSUM_CHUNK/16 = 32 rows: exact in fp64 (see fx24d)
  double s[8];
  float vm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0;
  for (int j = j0 + r; j < j1; j += 16) {
    const uint4 u = *reinterpret_cast<const uint4*>(kh + (size_t)j * D + cg * 8);
    s[0] += fx24d(bf2f(u.x));
    s[1] += fx24d(bf2f(u.x >> 16));
    s[2] += fx24d(bf2f(u.y));
    s[3] += fx24d(bf2f(u.y >> 16));
    s[4] += fx24d(bf2f(u.z));
    s[5] += fx24d(bf2f(u.z >> 16));
    s[6] += fx24d(bf2f(u.w));
    s[7] += fx24d(bf2f(u.w >> 16));
    if constexpr (WITH_V) {
      const uint4 w = *reinterpret_cast<const uint4*>(vh + (size_t)j * D + cg * 8);
      vm = fmaxf(vm, fmaxf(fmaxf(fabsf(bf2f(w.x)), fabsf(bf2f(w.x >> 16))),
                           fmaxf(fabsf(bf2f(w.y)), fabsf(bf2f(w.y >> 16)))));
      vm = fmaxf(vm, fmaxf(fmaxf(fabsf(bf2f(w.z)), fabsf(bf2f(w.z >> 16))),
                           fmaxf(fabsf(bf2f(w.w)), fabsf(bf2f(w.w >> 16)))));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[r][cg * 8 + i] = (long long)s[i];
  if constexpr (WITH_V) {
    vm = wave_max(vm);
    if ((t & 63) == 0) wm[t >> 6] = vm;
  }
  __syncthreads();
  if (t < D) {
    long long tot = 0;
    for (int rr = 0; rr < 16; ++rr) tot += red[rr][t];
    a.ksum[((size_t)bh * a.nkc + ch) * D + t] = tot;
  }
  if (WITH_V && t == 0) a.vmaxp[(size_t)bh * a.nkc + ch] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

// K channel mean.  grid BH, 128 threads.
__global__ __launch_bounds__(128) void k_kbar(Args a) {
  const int bh = blockIdx.x, c = threadIdx.x;
  long long tot = 0;
  for (int ch = 0; ch < a.nkc; ++ch) tot += a.ksum[((size_t)bh * a.nkc + ch) * D + c];
  a.kbar[(size_t)bh * D + c] = fixed_mean(tot, a.N);
}

// ---------------------------------------------------------------------------
// k-means on fixed-point values ("lightweight" clustering): per head every V
// value is scaled by 2^sh, the largest power of two keeping max|V| * 2^sh below
// 2^13, and rounded to an integer u; u = 128 * (u >> 7) + (u & 127) with both
// parts in int8, so u.c is exact on int8 MFMA (four products, int32 partial
// sums, combined in int64).  Distances ||c||^2 - 2 u.c are exact integers, so
// the cluster ids do not depend on the order of any accumulation.

typedef int v4i __attribute__((ext_vector_type(4)));

// Fixed-point exponent of the head and the int8 planes of u (token order).
// grid (ceil(N/256), BH), 256 threads: 16 threads per token row (8 channels
// each, 16-byte loads), 16 rows per step.
__global__ __launch_bounds__(256) void k_vfix(Args a) {
  __shared__ float wm[4];
  const int bh = blockIdx.y, t = threadIdx.x;
  float am = 0.0f;
  for (int i = t; i < a.nkc; i += 256) am = fmaxf(am, a.vmaxp[(size_t)bh * a.nkc + i]);
  am = wave_max(am);
  if ((t & 63) == 0) wm[t >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  int e = 0;
  if (am > 0.0f) frexpf(am, &e);
  const int sh = am > 0.0f ? 13 - e : 0;
  if (blockIdx.x == 0 && t == 0) a.kmsh[bh] = sh;
  const int cg = t & 15;
  for (int r = t >> 4; r < 256; r += 16) {
    const int j = blockIdx.x * 256 + r;
    if (j >= a.N) break;
    const size_t o = ((size_t)bh * a.N + j) * D + cg * 8;
    const uint4 u = *reinterpret_cast<const uint4*>(a.v + o);
    const uint32_t h[4] = {u.x, u.y, u.z, u.w};
    uint32_t ph[2] = {0u, 0u}, pl[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (i & 1) ? (h[i >> 1] >> 16) : h[i >> 1];
      const int q = (int)__builtin_rintf(ldexpf(bf2f(bits), sh));
      ph[i >> 2] |= (uint32_t)((q >> 7) & 0xff) << (8 * (i & 3));
      pl[i >> 2] |= (uint32_t)(q & 127) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(a.uhi + o) = make_uint2(ph[0], ph[1]);
    *reinterpret_cast<uint2*>(a.ulo + o) = make_uint2(pl[0], pl[1]);
  }
}

// Forgy initialisation: seeded partial Fisher-Yates over [0, N), centroid k =
// fixed-point value of token idx[k].  The draws do not depend on the swaps, so
// lane i computes draw i and then resolves, on its own, which value the swaps
// leave at position i.  grid BH, 128 threads.
// Sum of one int64 per lane over a wave (exact).
__device__ __forceinline__ long long wave_sum_i64(long long x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum of one int64 per thread over a 128-thread block (exact).  red: 2 slots of
// shared memory.  Every thread gets the total.
__device__ __forceinline__ long long sum128_i64(long long x, long long* red) {
  x = wave_sum_i64(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return red[0] + red[1];
}

__global__ __launch_bounds__(128) void k_km_init(Args a) {
  __shared__ int jdraw[MAX_CLUSTERS];
  __shared__ int idx[MAX_CLUSTERS];
  const int bh = blockIdx.x, C = a.C, t = threadIdx.x;
  if (t < C) {
    // state after t+1 steps of splitmix64 from the head's seed
    uint64_t st = (a.seed ^ (0x9E3779B97F4A7C15ull * (uint64_t)(bh + 1))) +
                  0x9E3779B97F4A7C15ull * (uint64_t)t;
    const uint64_t r = splitmix(st);
    jdraw[t] = t + (int)(r % (uint64_t)(a.N - t));
  }
  __syncthreads();
  if (t < C) {
    // Position t is final after step t (later steps only touch positions >= their
    // own index), so idx[t] is the value at position jdraw[t] just before step t.
    // A position q holds q until the last earlier step k with jdraw[k] == q,
    // after which it holds what position k held just before step k; follow that
    // chain (each link lowers the step index) to an untouched position.
    int pos = jdraw[t], step = t;
    for (;;) {
      int last = -1;
      for (int k = 0; k < step; ++k)
        if (jdraw[k] == pos) last = k;
      if (last < 0) break;
      pos = last;
      step = last;
    }
    idx[t] = pos;
  }
  __syncthreads();
  const int sh = a.kmsh[bh];
  __shared__ long long part[2][MAX_CLUSTERS];
  for (int kk = 0; kk < C; ++kk) {
    const size_t src = ((size_t)bh * a.N + idx[kk]) * D + t;
    const int u = 128 * (int)a.uhi[src] + (int)a.ulo[src];
    a.centfix[((size_t)bh * C + kk) * D + t] = u;
    a.cent[((size_t)bh * C + kk) * D + t] = ldexpf((float)u, -sh);
    const long long s2 = wave_sum_i64((long long)u * u);
    if ((t & 63) == 0) part[t >> 6][kk] = s2;
  }
  __syncthreads();
  if (t < C) a.kmcc[(size_t)bh * C + t] = part[0][t] + part[1][t];
  if (t < C) a.init_idx[(size_t)bh * C + t] = idx[t];
}

// Warm start: the previous step's centroids (fp32, in the workspace) in the
// current fixed-point scale, rounded to the nearest integer (ties to even) and
// clamped to 14 bits.  grid BH, 128 threads (one per channel).
__global__ __launch_bounds__(128) void k_km_warm(Args a) {
  __shared__ long long part[2][MAX_CLUSTERS];
  const int bh = blockIdx.x, C = a.C, t = threadIdx.x;
  const int sh = a.kmsh[bh];
  for (int kk = 0; kk < C; ++kk) {
    const size_t o = ((size_t)bh * C + kk) * D + t;
    const float x = fminf(fmaxf(__builtin_rintf(ldexpf(a.cent[o], sh)), -8192.0f), 8191.0f);
    const int u = (int)x;
    a.centfix[o] = u;
    a.cent[o] = ldexpf((float)u, -sh);
    const long long s2 = wave_sum_i64((long long)u * u);
    if ((t & 63) == 0) part[t >> 6][kk] = s2;
  }
  __syncthreads();
  if (t < C) a.kmcc[(size_t)bh * C + t] = part[0][t] + part[1][t];
}

// Assignment step on int8 MFMA plus per-workgroup member sums.
// grid (nkm, BH), KM_WAVES waves (each takes every KM_WAVES-th 16-token subtile),
// KM_CHUNK tokens per workgroup.  Lane (g, j) of a 16-token subtile loads the
// hi/lo bytes of channels 16g..16g+15 and 64+16g..64+16g+15 of token j as its
// MFMA B operand; after the argmin the same registers are added to the LDS bins
// of the token's cluster, so the planes are read once per iteration.
constexpr int CROW = D + 16;  // padded LDS row (bytes): spreads rows over banks

constexpr int KM_WAVES = 8;  // 8 waves: twice the loads in flight of 4 (measured 13 us
                             // less per Lloyd iteration at N=16544, 48 heads)
// Member sums: two channels per 64-bit LDS add.  Each half holds u + 16384 (in
// [8192, 24575]) summed over at most KM_CHUNK = 2048 tokens (< 2^26), so the low
// half never carries into the high one; the bias is removed with the count.
constexpr int BROW2 = D / 2 + 1;  // LDS row of the packed bins (8-byte words)
static_assert(KM_CHUNK * 24575ll < (1ll << 32), "packed member sums would carry");
constexpr size_t km_smem_bytes(int C) { return (size_t)C * (2 * CROW + 8 * BROW2 + 4); }

__device__ __forceinline__ void add_bins2(unsigned long long* bins, int base, const v4i& h, const v4i& l) {
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    const uint32_t hb = (uint32_t)h[wd] ^ 0x80808080u;  // signed hi byte + 128, as unsigned
    const uint32_t lb = (uint32_t)l[wd];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const uint32_t ua = (((hb >> (16 * pr)) & 0xffu) << 7) + ((lb >> (16 * pr)) & 0xffu);
      const uint32_t ub = (((hb >> (16 * pr + 8)) & 0xffu) << 7) + ((lb >> (16 * pr + 8)) & 0xffu);
      atomicAdd(&bins[base + 2 * wd + pr], (unsigned long long)ua | ((unsigned long long)ub << 32));
    }
  }
}

// NT = number of 16-centroid tiles (C <= 16 NT).  Centroids beyond C get a norm
// of 2^62, so their distance never wins and no lane needs a predicate.
template <int NT>
__global__ __launch_bounds__(64 * KM_WAVES) void k_km_assign(Args a) {
  extern __shared__ __align__(16) unsigned char km_smem[];
  const int C = a.C;
  int8_t* chi = reinterpret_cast<int8_t*>(km_smem);                       // [C][CROW]
  int8_t* clo = chi + C * CROW;                                           // [C][CROW]
  unsigned long long* bins = reinterpret_cast<unsigned long long*>(clo + C * CROW);  // [C][BROW2]
  int* cnt = reinterpret_cast<int*>(bins + C * BROW2);                    // [C]
  const int bh = blockIdx.y, chunk = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, g = lane >> 4, l16 = lane & 15;
  const int* cf = a.centfix + (size_t)bh * C * D;
  for (int e = t; e < C * D; e += 64 * KM_WAVES) {
    const int u = cf[e];
    chi[(e / D) * CROW + (e % D)] = (int8_t)(u >> 7);
    clo[(e / D) * CROW + (e % D)] = (int8_t)(u & 127);
  }
  for (int e = t; e < C * BROW2; e += 64 * KM_WAVES) bins[e] = 0ull;
  if (t < C) cnt[t] = 0;
  // this lane's centroid norms: centroid 16kt + 4g + v
  long long ccr[NT][4];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int k = 16 * kt + 4 * g + v;
      ccr[kt][v] = k < C ? a.kmcc[(size_t)bh * C + k] : (1ll << 62);
    }
  __syncthreads();
  const int8_t* uhi = a.uhi + (size_t)bh * a.N * D;
  const int8_t* ulo = a.ulo + (size_t)bh * a.N * D;
  // wave w takes 16-token subtiles w, w+KM_WAVES, ... of the chunk; the operands
  // of the next subtile are loaded while the current one is processed
  const int first = chunk * KM_CHUNK;
  auto load_sub = [&](int s, v4i& h0, v4i& h1, v4i& l0, v4i& l1) {
    int jj = first + s * 16 + l16;
    jj = jj < a.N ? jj : a.N - 1;  // tail lanes read a valid row, add nothing
    h0 = *reinterpret_cast<const v4i*>(uhi + (size_t)jj * D + 16 * g);
    h1 = *reinterpret_cast<const v4i*>(uhi + (size_t)jj * D + 64 + 16 * g);
    l0 = *reinterpret_cast<const v4i*>(ulo + (size_t)jj * D + 16 * g);
    l1 = *reinterpret_cast<const v4i*>(ulo + (size_t)jj * D + 64 + 16 * g);
  };
  v4i nh0, nh1, nl0, nl1;
  if (first + w * 16 < a.N) load_sub(w, nh0, nh1, nl0, nl1);
#pragma unroll 1
  for (int sub = w; sub < KM_CHUNK / 16; sub += KM_WAVES) {
    if (first + sub * 16 >= a.N) break;  // uniform per wave
    const v4i bh0 = nh0, bh1 = nh1, bl0 = nl0, bl1 = nl1;
    if (sub + KM_WAVES < KM_CHUNK / 16 && first + (sub + KM_WAVES) * 16 < a.N)
      load_sub(sub + KM_WAVES, nh0, nh1, nl0, nl1);
    const int j = first + sub * 16 + l16;
    long long bestD = 0x7fffffffffffffffll;
    int best = 0;
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
      const int kr = 16 * kt + l16;
      const int krow = kr < C ? kr : 0;
      const v4i ah0 = *reinterpret_cast<const v4i*>(chi + krow * CROW + 16 * g);
      const v4i ah1 = *reinterpret_cast<const v4i*>(chi + krow * CROW + 64 + 16 * g);
      const v4i al0 = *reinterpret_cast<const v4i*>(clo + krow * CROW + 16 * g);
      const v4i al1 = *reinterpret_cast<const v4i*>(clo + krow * CROW + 64 + 16 * g);
      const v4i z = {0, 0, 0, 0};
      v4i HH = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah0, bh0, z, 0, 0, 0);
      HH = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah1, bh1, HH, 0, 0, 0);
      v4i HL = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah0, bl0, z, 0, 0, 0);
      HL = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah1, bl1, HL, 0, 0, 0);
      v4i LH = __builtin_amdgcn_mfma_i32_16x16x64_i8(al0, bh0, z, 0, 0, 0);
      LH = __builtin_amdgcn_mfma_i32_16x16x64_i8(al1, bh1, LH, 0, 0, 0);
      v4i LL = __builtin_amdgcn_mfma_i32_16x16x64_i8(al0, bl0, z, 0, 0, 0);
      LL = __builtin_amdgcn_mfma_i32_16x16x64_i8(al1, bl1, LL, 0, 0, 0);
      // lane (g, token l16) holds centroids 16kt + 4g + v; ||c||^2 - 2 u.c with
      // u.c = 2^14 HH + 2^7 (HL + LH) + LL, exact in int64
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const long long Dk = ccr[kt][v] - (long long)HH[v] * 32768 - (long long)(HL[v] + LH[v]) * 256 -
                             (long long)LL[v] * 2;
        const int k = 16 * kt + 4 * g + v;
        best = Dk < bestD ? k : best;
        bestD = Dk < bestD ? Dk : bestD;
      }
    }
    // argmin across the four lane groups; ties go to the lower id
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const long long oD = __shfl_xor(bestD, off, 64);
      const int ob = __shfl_xor(best, off, 64);
      if (oD < bestD || (oD == bestD && ob < best)) { bestD = oD; best = ob; }
    }
    if (j < a.N) {
      if (g == 0) {
        a.labels[(size_t)bh * a.N + j] = best;
        atomicAdd(&cnt[best], 1);
      }
      add_bins2(bins, best * BROW2 + 8 * g, bh0, bl0);
      add_bins2(bins, best * BROW2 + 32 + 8 * g, bh1, bl1);
    }
  }
  __syncthreads();
  int* part = a.kmpart + ((size_t)bh * a.nkm + chunk) * C * D;
  for (int e = t; e < C * D; e += 64 * KM_WAVES) {
    const int c = e / D, ch = e % D;
    const unsigned long long wv = bins[c * BROW2 + (ch >> 1)];
    const uint32_t half = (ch & 1) ? (uint32_t)(wv >> 32) : (uint32_t)wv;
    part[e] = (int)half - 16384 * cnt[c];
  }
  if (t < C) a.kmcnt[((size_t)bh * a.nkm + chunk) * C + t] = cnt[t];
}

// Update step: centroid = member mean rounded to the nearest integer (ties to
// even; |sum| < 2^34 so the fp64 quotient rounds once), empty clusters stay.
// grid (C, BH), 128 threads.
__global__ __launch_bounds__(128) void k_km_update(Args a) {
  const int kk = blockIdx.x, bh = blockIdx.y, c = threadIdx.x, C = a.C;
  long long s = 0, n = 0;
  for (int ch = 0; ch < a.nkm; ++ch) {
    s += a.kmpart[(((size_t)bh * a.nkm + ch) * C + kk) * D + c];
    n += a.kmcnt[((size_t)bh * a.nkm + ch) * C + kk];
  }
  int u;
  if (n > 0) {
    u = (int)__builtin_rint((double)s / (double)n);
    a.centfix[((size_t)bh * C + kk) * D + c] = u;
    a.cent[((size_t)bh * C + kk) * D + c] = ldexpf((float)u, -a.kmsh[bh]);
  } else {
    u = a.centfix[((size_t)bh * C + kk) * D + c];
  }
  __shared__ long long red[2];
  const long long cc = sum128_i64((long long)u * u, red);
  if (c == 0) a.kmcc[(size_t)bh * C + kk] = cc;
}

// ---------------------------------------------------------------------------
// Stable counting sort of positions by cluster id.  grid BH, 1024 threads.
__global__ __launch_bounds__(1024) void k_perm(Args a) {
  __shared__ int base[MAX_CLUSTERS + 1];
  __shared__ int wcnt[16][MAX_CLUSTERS + 1];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6, C = a.C;
  const int* lab = a.labels + (size_t)bh * a.N;
  int* perm = a.perm + (size_t)bh * a.N;
  int* iperm = a.iperm + (size_t)bh * a.N;
  if (t <= MAX_CLUSTERS) base[t] = 0;
  __syncthreads();
  for (int j = t; j < a.N; j += 1024) atomicAdd(&base[lab[j] + 1], 1);
  __syncthreads();
  if (t == 0)
    for (int kk = 0; kk < C; ++kk) base[kk + 1] += base[kk];
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < a.N; j0 += 1024) {
    const int j = j0 + t;
    const int l = j < a.N ? lab[j] : MAX_CLUSTERS;  // sentinel bucket for the tail
    unsigned long long peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 7; ++b) {
      const unsigned long long m = __ballot((l >> b) & 1);
      peers &= ((l >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    for (int e = t; e < 16 * (MAX_CLUSTERS + 1); e += 1024) (&wcnt[0][0])[e] = 0;
    __syncthreads();
    if (rank == 0) wcnt[w][l] = __popcll(peers);
    __syncthreads();
    if (j < a.N) {
      int pre = 0;
      for (int ww = 0; ww < w; ++ww) pre += wcnt[ww][l];
      const int pos = base[l] + pre + rank;
      perm[pos] = j;
      iperm[j] = pos;
    }
    __syncthreads();
    if (t < C) {
      int tot = 0;
      for (int ww = 0; ww < 16; ++ww) tot += wcnt[ww][t];
      base[t] += tot;
    }
    __syncthreads();
  }
}

// Identity permutation (V-Smooth off).  grid (ceil(N/256), BH), 256 threads.
__global__ __launch_bounds__(256) void k_perm_identity(Args a) {
  const int j = blockIdx.x * 256 + threadIdx.x, bh = blockIdx.y;
  if (j < a.N) {
    a.perm[(size_t)bh * a.N + j] = j;
    a.iperm[(size_t)bh * a.N + j] = j;
    a.labels[(size_t)bh * a.N + j] = 0;
  }
}

// ---------------------------------------------------------------------------
// Per-block E4M3 codes of Q (z = 0) and smoothed K (z = 1), and for K the bf16
// copy of the codes.  With VC_SMOOTH_Q a Q block first subtracts its channel
// mean (exact fixed-point sum, as for the V block means), which is kept.
// grid (nblk, BH, 2), 256 threads: thread = (8-channel chunk t%16, rows
// t/16 + 16i), so 16 threads cover one 256-byte row.
__global__ __launch_bounds__(256) void k_qk_quant(Args a) {
  __shared__ float wmax[4];
  __shared__ long long qsum[16][D];
  __shared__ float qmean[D];
  const int blk = blockIdx.x, bh = blockIdx.y, isk = blockIdx.z, t = threadIdx.x;
  const int cg = t & 15, r0 = t >> 4;
  const bool follow = isk || (a.flags & VC_PERMUTE_Q);
  const bool smooth = !isk && (a.flags & VC_SMOOTH_Q);  // uniform over the workgroup
  const uint16_t* src = (isk ? a.k : a.q) + (size_t)bh * a.N * D;
  float kb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) kb[i] = isk ? a.kbar[(size_t)bh * D + cg * 8 + i] : 0.0f;
  float x[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = blk * BLK + r0 + 16 * i;
    if (p < a.N) {
      const int j = follow ? a.perm[(size_t)bh * a.N + p] : p;
      const uint4 u = *reinterpret_cast<const uint4*>(src + (size_t)j * D + cg * 8);
      const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float val = bf2f((e & 1) ? (h[e >> 1] >> 16) : h[e >> 1]);
        if (isk) val = val - kb[e];
        x[i][e] = val;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = 0.0f;
    }
  }
  if (smooth) {
    const int n = min(BLK, a.N - blk * BLK);
    double sm[8];  // 8 rows per thread: exact in fp64 (see fx24d)
#pragma unroll
    for (int e = 0; e < 8; ++e) sm[e] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm[e] += fx24d(x[i][e]);  // rows past N hold 0
#pragma unroll
    for (int e = 0; e < 8; ++e) qsum[r0][cg * 8 + e] = (long long)sm[e];
    __syncthreads();
    if (t < D) {
      long long tot = 0;
      for (int rr = 0; rr < 16; ++rr) tot += qsum[rr][t];
      qmean[t] = fixed_mean(tot, n);
      a.qbar[((size_t)bh * a.nblk + blk) * D + t] = qmean[t];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (blk * BLK + r0 + 16 * i < a.N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = x[i][e] - qmean[cg * 8 + e];
      }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
  amax = wave_max(amax);
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float s, inv;
  scale_from_amax(amax, &s, &inv);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = blk * BLK + r0 + 16 * i;
    uint32_t w0 = 0u, w1 = 0u;
    if (p < a.N) {
      w0 = e4m3x2(x[i][0] * inv, x[i][1] * inv) | (e4m3x2(x[i][2] * inv, x[i][3] * inv) << 16);
      w1 = e4m3x2(x[i][4] * inv, x[i][5] * inv) | (e4m3x2(x[i][6] * inv, x[i][7] * inv) << 16);
    }
    uint8_t* dst = (isk ? a.k8 : a.q8) + ((size_t)bh * a.Npad + p) * D + cg * 8;
    *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
    if (isk && (a.flags & VC_EXACT_SCORES)) {
      // the K codes decoded to bf16 (E4M3 values are exact in bf16)
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wd = e < 2 ? w0 : w1;
        const uint32_t b0 = (wd >> (16 * (e & 1))) & 0xff, b1 = (wd >> (16 * (e & 1) + 8)) & 0xff;
        h[e] = (__float_as_uint(e4m3_val(b0)) >> 16) | (__float_as_uint(e4m3_val(b1)) & 0xffff0000u);
      }
      *reinterpret_cast<uint4*>(a.k16 + ((size_t)bh * a.Npad + p) * D + cg * 8) =
          make_uint4(h[0], h[1], h[2], h[3]);
    }
  }
  if (t == 0) (isk ? a.sk : a.sq)[(size_t)bh * a.nblk + blk] = s;
}

// ---------------------------------------------------------------------------
// Score term of the smoothed queries (VC_SMOOTH_Q): for every query block b and
// key position p, d = fp32(c0 * delta) with delta the fp32 fma chain over
// channels 0..127 of qbar_b[c] * (k[c] - kbar[c]), the same fp32 values the K
// codes are made from; 0 for positions past N.  A product of a (nblk x 128) and
// a (128 x Npad) matrix whose every output accumulates in channel order, so it
// runs on VALU fma, register-tiled: a workgroup computes 16 query blocks x 256
// keys, each thread 4 x 4 outputs; 32 channels at a time pass through LDS
// (k - kbar channel-major, the means channel-major), and per channel a thread
// reads two float4 and issues 16 fma.  grid (ceil(nblk/16), ceil(Npad/256), BH),
// 256 threads; the block groups of one key tile are neighbours, so the key rows
// are fetched from HBM about once.
__global__ __launch_bounds__(256) void k_qbias(Args a) {
  constexpr int QB = 16, KT = 256, CC = 32;
  __shared__ __align__(16) float skt[CC][KT];  // k - kbar, [channel][key]
  __shared__ __align__(16) float sqm[CC][QB];  // qbar, [channel][block]
  const int bh = blockIdx.z, t = threadIdx.x;
  const int b0 = blockIdx.x * QB, nb = min(QB, a.nblk - b0);
  const int p0 = blockIdx.y * KT;
  const int bq = t >> 6, kq = t & 63;  // outputs: blocks 4bq..4bq+3, keys 4kq..4kq+3
  // loader role: key p0 + t of the tile
  const int pl = p0 + t;
  const bool vl = pl < a.N;
  const uint4* row = reinterpret_cast<const uint4*>(a.k + ((size_t)bh * a.N + (vl ? a.perm[(size_t)bh * a.N + pl] : 0)) * D);
  const float* kbar = a.kbar + (size_t)bh * D;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
#pragma unroll 1
  for (int c0 = 0; c0 < D; c0 += CC) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CC / 8; ++i) {
      const uint4 u = row[c0 / 8 + i];
      const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * i + e;
        skt[c][t] = vl ? bf2f((e & 1) ? (h[e >> 1] >> 16) : h[e >> 1]) - kbar[c0 + c] : 0.0f;
      }
    }
    for (int j = t; j < CC * QB; j += 256) {
      const int c = j / QB, bb = j % QB;
      sqm[c][bb] = bb < nb ? a.qbar[((size_t)bh * a.nblk + b0 + bb) * D + c0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < CC; ++c) {
      const float4 qv = *reinterpret_cast<const float4*>(&sqm[c][4 * bq]);
      const float4 kv = *reinterpret_cast<const float4*>(&skt[c][4 * kq]);
      const float qa[4] = {qv.x, qv.y, qv.z, qv.w}, ka[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(qa[i], ka[j], acc[i][j]);
    }
  }
  const int pk = p0 + 4 * kq;
  if (pk < a.Npad) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * bq + i;
      if (b < nb) {
        float4 o;
        o.x = pk + 0 < a.N ? a.c0 * acc[i][0] : 0.0f;
        o.y = pk + 1 < a.N ? a.c0 * acc[i][1] : 0.0f;
        o.z = pk + 2 < a.N ? a.c0 * acc[i][2] : 0.0f;
        o.w = pk + 3 < a.N ? a.c0 * acc[i][3] : 0.0f;
        *reinterpret_cast<float4*>(a.qbias + ((size_t)bh * a.nblk + b0 + b) * a.Npad + pk) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// V block means and block maxima of |V - mu|; with VC_V4 also the maximum of each
// 32-key group (rows r with 2(r/64) + (r/8)%2 = G) and its E8M0 exponent.
// grid (nblk, BH), 256 threads: thread = (8-channel chunk t%16, rows t/16 + 16i),
// so rows i < 4 and i >= 4 of a thread lie in groups (t/128)%2 and 2 + (t/128)%2.
__global__ __launch_bounds__(256) void k_v_stats(Args a) {
  __shared__ long long ssum[16][D];
  __shared__ float smax[2][16][D];
  __shared__ float smu[D];
  const int blk = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int cg = t & 15, r0 = t >> 4;
  const int p0 = blk * BLK, n = min(BLK, a.N - p0);
  const bool vs = (a.flags & VC_VSMOOTH) != 0;
  const uint16_t* vh = a.v + (size_t)bh * a.N * D;
  const int* perm = a.perm + (size_t)bh * a.N;
  float x[8][8];
  double s[8];  // 8 rows per thread: exact in fp64 (see fx24d)
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + 16 * i;
    if (r < n) {
      const uint4 u = *reinterpret_cast<const uint4*>(vh + (size_t)perm[p0 + r] * D + cg * 8);
      const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[i][e] = bf2f((e & 1) ? (h[e >> 1] >> 16) : h[e >> 1]);
        s[e] += fx24d(x[i][e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = 0.0f;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ssum[r0][cg * 8 + e] = (long long)s[e];
  __syncthreads();
  if (t < D) {
    long long tot = 0;
    for (int rr = 0; rr < 16; ++rr) tot += ssum[rr][t];
    smu[t] = vs ? fixed_mean(tot, n) : 0.0f;
  }
  __syncthreads();
  float m[2][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[0][e] = m[1][e] = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (r0 + 16 * i < n) {
#pragma unroll
      for (int e = 0; e < 8; ++e) m[i >> 2][e] = fmaxf(m[i >> 2][e], fabsf(x[i][e] - smu[cg * 8 + e]));
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    smax[0][r0][cg * 8 + e] = m[0][e];
    smax[1][r0][cg * 8 + e] = m[1][e];
  }
  __syncthreads();
  if (t < D) {
    float gm[4];  // group G = 2h + b: rows of half h, threads with (r0/8)%2 = b
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      float mm = 0.0f;
      for (int rr = 0; rr < 8; ++rr) mm = fmaxf(mm, smax[G >> 1][8 * (G & 1) + rr][t]);
      gm[G] = mm;
    }
    const size_t o = ((size_t)bh * a.nblk + blk) * D + t;
    a.mu[o] = smu[t];
    a.bamax[o] = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
    if (a.flags & VC_V4) {
      uint8_t* rec = a.v4s + ((size_t)bh * a.nblk + blk) * V4_SREC;
#pragma unroll
      for (int G = 0; G < 4; ++G) rec[(16 * G + (t & 15)) * 8 + (t >> 4)] = (uint8_t)(mx_exponent(gm[G]) + 127);
    }
  }
}

// Per-channel residual scales.  grid BH, 128 threads (one per channel).
__global__ __launch_bounds__(128) void k_v_scale(Args a) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const float* bm = a.bamax + (size_t)bh * a.nblk * D + c;
  float A[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  int b = 0;
  for (; b + 8 <= a.nblk; b += 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = fmaxf(A[i], bm[(size_t)(b + i) * D]);
  }
  for (; b < a.nblk; ++b) A[0] = fmaxf(A[0], bm[(size_t)b * D]);
  const float amax = fmaxf(fmaxf(fmaxf(A[0], A[1]), fmaxf(A[2], A[3])),
                           fmaxf(fmaxf(A[4], A[5]), fmaxf(A[6], A[7])));
  float s, inv;
  scale_from_amax(amax, &s, &inv);
  if (a.flags & VC_V4) s = inv = 1.0f;  // the 4-bit residual carries its own powers of two
  a.sv[(size_t)bh * D + c] = s;
  a.inv[(size_t)bh * D + c] = inv;
}

// Block means in V code units (mu * inv), fp32 and as a bf16 high/low pair in
// groups of 16 blocks, channel-major (the restore MFMA reads 4 blocks of one
// channel per lane).  grid (nch16, BH), 128 threads (one per channel).
__global__ __launch_bounds__(128) void k_v_mup(Args a) {
  const int grp = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const float inv = a.inv[(size_t)bh * D + c];
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    float x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int b = grp * 16 + j + e;
      x[e] = 0.0f;
      if (b < a.nblk) {
        const size_t o = ((size_t)bh * a.nblk + b) * D + c;
        x[e] = a.mu[o] * inv;
        a.mup[o] = x[e];
      }
    }
    const uint16_t h0 = f2bf_rne(x[0]), h1 = f2bf_rne(x[1]);
    const uint16_t l0 = f2bf_rne(x[0] - __uint_as_float((uint32_t)h0 << 16));
    const uint16_t l1 = f2bf_rne(x[1] - __uint_as_float((uint32_t)h1 << 16));
    hi[j / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[j / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  uint16_t* base = a.mupt + (((size_t)bh * a.nch16 + grp) * 2) * D * 16;
  uint4* dh = reinterpret_cast<uint4*>(base + (size_t)c * 16);
  uint4* dl = reinterpret_cast<uint4*>(base + (size_t)D * 16 + (size_t)c * 16);
  dh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  dh[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
  dl[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  dl[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
}

// Residual codes (channel-major, interleaved) and the repair criterion.
// One thread per row: the thread loads its own row (256 bytes) into registers
// and walks its channels in order (the criterion is an fp32 fma chain over
// channels 0..127).  LDS holds only the transposed code tile, so many
// workgroups share a CU.  grid (nblk, BH), 128 threads.
__global__ __launch_bounds__(128) void k_v_quant(Args a) {
  __shared__ float smu[D], sinv[D], ssv[D];
  __shared__ __align__(16) uint8_t tile[D * BLK];
  const int blk = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int p0 = blk * BLK, n = min(BLK, a.N - p0);
  smu[t] = a.mu[((size_t)bh * a.nblk + blk) * D + t];
  sinv[t] = a.inv[(size_t)bh * D + t];
  ssv[t] = a.sv[(size_t)bh * D + t];
  const int r = t, col = v_col(r), p = p0 + r;
  uint4 row[16];
  if (r < n) {
    const uint4* src = reinterpret_cast<const uint4*>(a.v + ((size_t)bh * a.N + a.perm[(size_t)bh * a.N + p]) * D);
#pragma unroll
    for (int i = 0; i < 16; ++i) row[i] = src[i];
  }
  __syncthreads();
  if (r < n) {
    float e = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t hw[4] = {row[i].x, row[i].y, row[i].z, row[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t h = hw[q];
        const int c = 8 * i + 2 * q;
        const float x0 = (bf2f(h) - smu[c]) * sinv[c];
        const float x1 = (bf2f(h >> 16) - smu[c + 1]) * sinv[c + 1];
        const uint32_t cc = e4m3x2(x0, x1);
        tile[c * BLK + col] = (uint8_t)(cc & 0xff);
        tile[(c + 1) * BLK + col] = (uint8_t)(cc >> 8);
        const float t0 = ssv[c] * (x0 - e4m3_val(cc & 0xff));
        e = __builtin_fmaf(t0, t0, e);
        const float t1 = ssv[c + 1] * (x1 - e4m3_val(cc >> 8));
        e = __builtin_fmaf(t1, t1, e);
      }
    }
    a.err[(size_t)bh * a.N + p] = e;
  } else {
    for (int c = 0; c < D; ++c) tile[c * BLK + col] = 0;
  }
  __syncthreads();
  // 128 channel rows x 128 bytes: thread t stores row t
  uint8_t* dst = a.v8t + ((size_t)bh * D + t) * a.Npad + (size_t)blk * BLK;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(dst + 16 * i) = *reinterpret_cast<const uint4*>(tile + t * BLK + 16 * i);
}

// 4-bit residual codes (VC_V4) and the repair criterion.  The group exponents
// come from k_v_stats.  Thread t owns the key pair 2t, 2t+1 of a block, whose
// two codes share one byte of every channel row of the block's tile.  Per
// channel, gfx950's v_cvt_scalef32_pk_fp4_f32 rounds the pair's two residuals
// by their group's power of two into that byte (nearest, ties to the even code,
// saturating at 6; it keeps the sign of a zero, which is cleared after), and
// v_cvt_scalef32_pk_f32_fp4 decodes them again for the criterion: two fp32 fma
// chains (r - value)^2 over channels 0..127 (sv = 1).  The 64 lanes' bytes make
// up each 64-byte channel row, so every store is one coalesced row.  No
// cross-lane traffic.  grid (nblk, BH), 64 threads.
__global__ __launch_bounds__(64) void k_v_quant4(Args a) {
  __shared__ __align__(16) uint8_t sx[4][D];  // [group][channel] E8M0 exponents
  __shared__ __align__(16) float smu[D];
  const int blk = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  smu[t] = a.mu[((size_t)bh * a.nblk + blk) * D + t];
  smu[t + 64] = a.mu[((size_t)bh * a.nblk + blk) * D + t + 64];
  {
    // the record is [group][channel % 16][channel / 16]: transpose to channel order
    const uint8_t* rec = a.v4s + ((size_t)bh * a.nblk + blk) * V4_SREC;
    for (int q = t; q < V4_SREC; q += 64) sx[q >> 7][16 * (q & 7) + ((q >> 3) & 15)] = rec[q];
  }
  const int p0 = blk * BLK, n = min(BLK, a.N - p0);
  const int k0 = 2 * t;
  const int G = v4_group(k0);
  const int byte = 16 * G + 8 * ((k0 >> 2) & 1) + 4 * ((k0 >> 5) & 1) + 2 * ((k0 >> 4) & 1) + ((k0 >> 1) & 1);
  // a key past N reads the block's first row (finite input) and is zeroed by the
  // multiply: residual 0, code 0; every load stays unconditional
  const bool ok0 = k0 < n, ok1 = k0 + 1 < n;
  const float keep0 = ok0 ? 1.0f : 0.0f, keep1 = ok1 ? 1.0f : 0.0f;
  const int* perm = a.perm + (size_t)bh * a.N + p0;
  const uint4* src0 = reinterpret_cast<const uint4*>(a.v + ((size_t)bh * a.N + perm[ok0 ? k0 : 0]) * D);
  const uint4* src1 = reinterpret_cast<const uint4*>(a.v + ((size_t)bh * a.N + perm[ok1 ? k0 + 1 : 0]) * D);
  uint8_t* dst = a.v4t + ((size_t)bh * a.nblk + blk) * V4_TILE + byte;
  __syncthreads();
  float e0 = 0.0f, e1 = 0.0f;
  // two halves of 64 channels: each half of a row is one 128-byte line, loaded
  // in one burst and used at once; the loop is kept rolled so that no half's
  // work moves into the other
#pragma unroll 1
  for (int hh = 0; hh < 2; ++hh) {
    uint4 row0[8], row1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      row0[i] = src0[8 * hh + i];
      row1[i] = src1[8 * hh + i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cb = 64 * hh + 8 * i;  // first channel of the chunk
      float mu8[8];
      *reinterpret_cast<float4*>(mu8) = *reinterpret_cast<const float4*>(smu + cb);
      *reinterpret_cast<float4*>(mu8 + 4) = *reinterpret_cast<const float4*>(smu + cb + 4);
      const uint2 xb = *reinterpret_cast<const uint2*>(&sx[G][cb]);
      const uint32_t w0[4] = {row0[i].x, row0[i].y, row0[i].z, row0[i].w};
      const uint32_t w1[4] = {row1[i].x, row1[i].y, row1[i].z, row1[i].w};
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = cb + jj;
        const uint32_t eb = ((jj < 4 ? xb.x : xb.y) >> (8 * (jj & 3))) & 0xffu;
        const float sc = __uint_as_float(eb << 23);  // 2^X, X in [-126, 127]: normal
        const uint32_t h0 = (jj & 1) ? (w0[jj >> 1] & 0xffff0000u) : (w0[jj >> 1] << 16);
        const uint32_t h1 = (jj & 1) ? (w1[jj >> 1] & 0xffff0000u) : (w1[jj >> 1] << 16);
        const float x0 = (__uint_as_float(h0) - mu8[jj]) * keep0;
        const float x1 = (__uint_as_float(h1) - mu8[jj]) * keep1;
        uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x0, x1, sc, 0) & 0xffu;
        // clear the sign of zero magnitudes (code 8 -> 0)
        d &= 0x77u | (((d & 0x77u) + 0x77u) & 0x88u);
        dst[c * (BLK / 2)] = (uint8_t)d;
        typedef float v2f __attribute__((ext_vector_type(2)));
        const v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, sc, 0);
        const float dl0 = x0 - v[0], dl1 = x1 - v[1];
        e0 = __builtin_fmaf(dl0, dl0, e0);
        e1 = __builtin_fmaf(dl1, dl1, e1);
      }
    }
  }
  if (ok0) a.err[(size_t)bh * a.N + p0 + k0] = e0;
  if (ok1) a.err[(size_t)bh * a.N + p0 + k0 + 1] = e1;
}

// ---------------------------------------------------------------------------
// Repair set: the m positions with the largest error (ties: lower position),
// by an exact radix select on the 64-bit key (~err_bits, position), then a
// compaction in position order.  grid BH, 1024 threads.
__global__ __launch_bounds__(1024) void k_rep_select(Args a) {
  __shared__ int hist[256];
  __shared__ unsigned long long s_prefix, s_mask;
  __shared__ int s_kth, s_kth_next, s_base, s_hsel;
  __shared__ int wtot[16];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* err = a.err + (size_t)bh * a.N;
  if (t == 0) {
    s_prefix = 0ull;
    s_mask = 0ull;
    s_kth = a.m;
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (t < 256) hist[t] = 0;
    __syncthreads();
    const unsigned long long pre = s_prefix, msk = s_mask;
    for (int j = t; j < a.N; j += 1024) {
      const unsigned long long key =
          ((unsigned long long)(~__float_as_uint(err[j])) << 32) | (unsigned)j;
      if ((key & msk) == pre) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    // parallel exclusive scan of the 256 bins (threads 0..255, 4 waves); the one
    // bin where the running count crosses kth fixes the next digit
    int h = 0, incl = 0;
    if (t < 256) {
      h = hist[t];
      incl = h;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (lane == 63) wtot[w] = incl;
    }
    __syncthreads();
    if (t < 256) {
      int before = 0;
      for (int ww = 0; ww < w; ++ww) before += wtot[ww];
      const int cum = before + incl - h;  // count of smaller digits
      const int kth = s_kth;
      if (h > 0 && cum < kth && kth <= cum + h) {
        s_kth_next = kth - cum;
        s_hsel = h;
        s_prefix = pre | ((unsigned long long)t << shift);
        s_mask = msk | (255ull << shift);
      }
    }
    __syncthreads();
    if (t == 0) s_kth = s_kth_next;
    __syncthreads();
    // if every key with the digits fixed so far is taken, the lower digits
    // cannot change the selected set: any threshold with this prefix works
    if (s_hsel == s_kth) {
      if (t == 0) s_prefix |= (1ull << shift) - 1ull;
      __syncthreads();
      break;
    }
  }
  const unsigned long long thr = s_prefix;  // the m-th smallest key, or a key
                                            // above it and below the next one
  int* out = a.rep_pos + (size_t)bh * a.mpad;
  if (t == 0) s_base = 0;
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < a.N; j0 += 1024) {
    const int j = j0 + t;
    bool sel = false;
    if (j < a.N) {
      const unsigned long long key =
          ((unsigned long long)(~__float_as_uint(err[j])) << 32) | (unsigned)j;
      sel = key <= thr;
    }
    const unsigned long long b = __ballot(sel);
    if (lane == 0) wtot[w] = __popcll(b);
    __syncthreads();
    int pre = s_base;
    for (int ww = 0; ww < w; ++ww) pre += wtot[ww];
    const int slot = pre + __popcll(b & lt);
    if (sel && slot < a.mpad) out[slot] = j;  // exactly m keys are <= thr
    __syncthreads();
    if (t == 0) {
      int tot = 0;
      for (int ww = 0; ww < 16; ++ww) tot += wtot[ww];
      s_base += tot;
    }
    __syncthreads();
  }
  for (int i = a.m + t; i < a.mpad; i += 1024) out[i] = -1;
}

// Residual error (bf16; V code units, real units with VC_V4) of the repaired
// positions, channel-major with the repair-slot interleave.  grid (mpad/128, BH), 128 threads = slots.
__global__ __launch_bounds__(128) void k_rep_delta(Args a) {
  __shared__ __align__(16) uint16_t tile[D * BLK];
  const int grp = blockIdx.x, bh = blockIdx.y, s = threadIdx.x;
  const int gs = grp * BLK + s;
  const int col = rep_col(s);
  const int p = gs < a.m ? a.rep_pos[(size_t)bh * a.mpad + gs] : -1;
  if (p >= 0 && (a.flags & VC_V4)) {
    // 4-bit residual: the error of the E2M1 code under its group's power of two,
    // in real units (the code is recomputed exactly as k_v_quant4 forms it)
    const uint16_t* row = a.v + ((size_t)bh * a.N + a.perm[(size_t)bh * a.N + p]) * D;
    const float* mu = a.mu + ((size_t)bh * a.nblk + p / BLK) * D;
    const uint8_t* xr = a.v4s + ((size_t)bh * a.nblk + p / BLK) * V4_SREC + 16 * v4_group(p % BLK) * 8;
    for (int i = 0; i < D / 8; ++i) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + i * 8);
      const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = i * 8 + j;
        const int X = (int)xr[(c & 15) * 8 + (c >> 4)] - 127;
        const float x = bf2f((j & 1) ? (h[j >> 1] >> 16) : h[j >> 1]) - mu[c];
        uint32_t code;
        const float val = e2m1_round(__builtin_ldexpf(x, -X), &code);
        tile[c * BLK + col] = f2bf_rne(x - __builtin_ldexpf(val, X));
      }
    }
  } else if (p >= 0) {
    const uint16_t* row = a.v + ((size_t)bh * a.N + a.perm[(size_t)bh * a.N + p]) * D;
    const float* mu = a.mu + ((size_t)bh * a.nblk + p / BLK) * D;
    const float* inv = a.inv + (size_t)bh * D;
    for (int i = 0; i < D / 8; ++i) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + i * 8);
      const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = i * 8 + 2 * j;
        const float x0 = (bf2f(h[j]) - mu[c]) * inv[c];
        const float x1 = (bf2f(h[j] >> 16) - mu[c + 1]) * inv[c + 1];
        const uint32_t cc = e4m3x2(x0, x1);
        tile[c * BLK + col] = f2bf_rne(x0 - e4m3_val(cc & 0xff));
        tile[(c + 1) * BLK + col] = f2bf_rne(x1 - e4m3_val(cc >> 8));
      }
    }
  } else {
    for (int c = 0; c < D; ++c) tile[c * BLK + col] = 0;
  }
  __syncthreads();
  uint16_t* dst = a.rep_dt + ((size_t)bh * D + s) * a.mpad + (size_t)grp * BLK;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    *reinterpret_cast<uint4*>(dst + 8 * i) = *reinterpret_cast<const uint4*>(tile + s * BLK + 8 * i);
}

// Header: marks the clusters valid for this shape.  grid 1, 64 threads.
__global__ void k_header(Args a, uint32_t clustered) {
  if (threadIdx.x == 0) {
    a.header->magic = MAGIC;
    a.header->clustered = clustered;
    a.header->B = a.B;
    a.header->H = a.H;
    a.header->N = a.N;
    a.header->C = a.C;
  }
}

}  // namespace

hipError_t launch_prepare(const Args& a, ClusterMode mode, hipStream_t st) {
  const unsigned BH = (unsigned)a.BH;
  const bool vs = (a.flags & VC_VSMOOTH) != 0;
  if (vs && mode != ClusterMode::Reuse)
    hipLaunchKernelGGL(k_ksum<true>, dim3(a.nkc, BH), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_ksum<false>, dim3(a.nkc, BH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_kbar, dim3(BH), dim3(128), 0, st, a);
  if (vs) {
    if (mode != ClusterMode::Reuse) {
      hipLaunchKernelGGL(k_vfix, dim3((a.N + 255) / 256, BH), dim3(256), 0, st, a);
      if (mode == ClusterMode::Warm)
        hipLaunchKernelGGL(k_km_warm, dim3(BH), dim3(128), 0, st, a);
      else
        hipLaunchKernelGGL(k_km_init, dim3(BH), dim3(128), 0, st, a);
      for (int it = 0; it < a.T; ++it) {
        const dim3 kg(a.nkm, BH), kb(64 * KM_WAVES);
        const size_t sm = km_smem_bytes(a.C);
        if (a.C <= 16)
          hipLaunchKernelGGL(k_km_assign<1>, kg, kb, sm, st, a);
        else if (a.C <= 32)
          hipLaunchKernelGGL(k_km_assign<2>, kg, kb, sm, st, a);
        else if (a.C <= 48)
          hipLaunchKernelGGL(k_km_assign<3>, kg, kb, sm, st, a);
        else
          hipLaunchKernelGGL(k_km_assign<4>, kg, kb, sm, st, a);
        hipLaunchKernelGGL(k_km_update, dim3(a.C, BH), dim3(128), 0, st, a);
      }
      hipLaunchKernelGGL(k_perm, dim3(BH), dim3(1024), 0, st, a);
      hipLaunchKernelGGL(k_header, dim3(1), dim3(64), 0, st, a, 1u);
    }
  } else {
    hipLaunchKernelGGL(k_perm_identity, dim3((a.N + 255) / 256, BH), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_header, dim3(1), dim3(64), 0, st, a, 0u);
  }
  hipLaunchKernelGGL(k_qk_quant, dim3(a.nblk, BH, 2), dim3(256), 0, st, a);
  if (a.flags & VC_SMOOTH_Q)
    hipLaunchKernelGGL(k_qbias, dim3((a.nblk + 15) / 16, (a.Npad + 255) / 256, BH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_v_stats, dim3(a.nblk, BH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_v_scale, dim3(BH), dim3(128), 0, st, a);
  hipLaunchKernelGGL(k_v_mup, dim3(a.nch16, BH), dim3(128), 0, st, a);
  if (a.flags & VC_V4)
    hipLaunchKernelGGL(k_v_quant4, dim3(a.nblk, BH), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(k_v_quant, dim3(a.nblk, BH), dim3(128), 0, st, a);
  if (a.m > 0) {
    hipLaunchKernelGGL(k_rep_select, dim3(BH), dim3(1024), 0, st, a);
    hipLaunchKernelGGL(k_rep_delta, dim3(a.mpad / BLK, BH), dim3(128), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace vc
