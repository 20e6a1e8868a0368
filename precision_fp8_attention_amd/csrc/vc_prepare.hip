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

typedef int nt_v4 __attribute__((ext_vector_type(4)));  // 16-byte operand of non-temporal loads


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

// Cross-lane exchanges without LDS.  v_permlane16_swap with both operands x
// leaves rows (0, 2) of x in the first result and rows (1, 3) in the second, so
// every lane holds its own value and that of lane ^ 16, one in each result (the
// order depends on the row); v_permlane32_swap does the same for lane ^ 32.
__device__ __forceinline__ float xmax16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xmax32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
// min of x over lanes l, l ^ 16 (SHIFT 16) or l, l ^ 32 (SHIFT 32), fp64
template <int SHIFT>
__device__ __forceinline__ double xmin_f64(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  const auto pl = SHIFT == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                              : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto ph = SHIFT == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                              : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const double a = __builtin_bit_cast(double, (uint64_t)pl[0] | ((uint64_t)ph[0] << 32));
  const double c = __builtin_bit_cast(double, (uint64_t)pl[1] | ((uint64_t)ph[1] << 32));
  return __builtin_fmin(a, c);
}
// max over the wave: rotations inside each 16-lane row (DPP row_ror 8, 4, 2, 1
// leave the row's maximum in every lane), then rows by the swaps above
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false)));
  return xmax32(xmax16(x));
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

// 32-key group of key r of a block (4-bit residual): 32 consecutive positions.
__device__ __forceinline__ int v4_group(int r) { return r >> 5; }

// ---------------------------------------------------------------------------
// One of two sweeps over a chunk of KSUM_CHUNK tokens.  With WITH_K, the K
// channel sums: fixed-point partial sums over the chunk, added into the head's
// sums.  With WITH_V, max|V| of the chunk, taken into the head's maximum (the
// k-means fixed-point scale, needed only when k-means runs).
// One workgroup of 256 threads per chunk: thread = (row r = t/16, 8-channel
// group t%16); red is a 16 x 128 LDS buffer, wm four floats of LDS.
template <bool WITH_K, bool WITH_V>
__device__ __forceinline__ void ksum_chunk(const Args& a, int ch, int bh, long long (*red)[D], float* wm) {
  static_assert(WITH_K != WITH_V, "one sweep: the K sums or max|V|");
  const int t = threadIdx.x;
  const int cg = t & 15, r = t >> 4;
  const int j0 = ch * KSUM_CHUNK, j1 = min(j0 + KSUM_CHUNK, a.N);
  const uint16_t* kh = a.k + (size_t)bh * a.N * D;
  const uint16_t* vh = a.v + (size_t)bh * a.N * D;
  // a thread sums at most KSUM_CHUNK/16 = 32 rows: exact in fp64 (see fx24d)
  double s[8];
  float vm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0;
  // The rows are streamed once: non-temporal loads (measured 20 us less over
  // the cold prepare at 2x24x16544).  A thread takes its rows 8 at a time and
  // issues the 8 loads before it waits on any: rows at or past the chunk's end
  // read the chunk's last row and count as zero (which adds nothing to the sums
  // and the maximum), so no branch stands between the loads.
  for (int jb = j0 + r; jb < j1; jb += 16 * 8) {
    uint4 u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = min(jb + 16 * i, j1 - 1);
      const nt_v4 x = __builtin_nontemporal_load(
          reinterpret_cast<const nt_v4*>((WITH_K ? kh : vh) + (size_t)j * D + cg * 8));
      u[i] = make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pin_loaded(u[i]);
      if (jb + 16 * i >= j1) u[i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (WITH_K) {
        s[0] += fx24d(bf2f(u[i].x));
        s[1] += fx24d(bf2f(u[i].x >> 16));
        s[2] += fx24d(bf2f(u[i].y));
        s[3] += fx24d(bf2f(u[i].y >> 16));
        s[4] += fx24d(bf2f(u[i].z));
        s[5] += fx24d(bf2f(u[i].z >> 16));
        s[6] += fx24d(bf2f(u[i].w));
        s[7] += fx24d(bf2f(u[i].w >> 16));
      } else {
        const uint4 w = u[i];
        vm = fmaxf(vm, fmaxf(fmaxf(fabsf(bf2f(w.x)), fabsf(bf2f(w.x >> 16))),
                             fmaxf(fabsf(bf2f(w.y)), fabsf(bf2f(w.y >> 16)))));
        vm = fmaxf(vm, fmaxf(fmaxf(fabsf(bf2f(w.z)), fabsf(bf2f(w.z >> 16))),
                             fmaxf(fabsf(bf2f(w.w)), fabsf(bf2f(w.w >> 16)))));
      }
    }
  }
  if constexpr (WITH_K) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[r][cg * 8 + i] = (long long)s[i];
  }
  if constexpr (WITH_V) {
    vm = wave_max(vm);
    if ((t & 63) == 0) wm[t >> 6] = vm;
  }
  __syncthreads();
  if (WITH_K && t < D) {
    long long tot = 0;
    for (int rr = 0; rr < 16; ++rr) tot += red[rr][t];
    a.ksum[((size_t)bh * a.nkc + ch) * D + t] = tot;
    // the head's sums: integer adds, so their order cannot change them
    atomicAdd(reinterpret_cast<unsigned long long*>(a.ktot) + (size_t)bh * D + t, (unsigned long long)tot);
  }
  // max |V| >= 0, so its fp32 bits order like the values
  if (WITH_V && t == 0) atomicMax(a.vmaxh + bh, __float_as_uint(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]))));
}

// max|V| of every head alone, for the k-means scale; the K sums come later,
// beside the V block statistics.  grid (nkc, BH), 256 threads.
__global__ __launch_bounds__(256) void k_vmax(Args a) {
  __shared__ float wm[4];
  ksum_chunk<false, true>(a, blockIdx.x, blockIdx.y, nullptr, wm);
}

// Clears the per-head accumulators that later kernels add into.  grid BH, 128
// threads.
__global__ __launch_bounds__(128) void k_prep_zero(Args a) {
  const int bh = blockIdx.x, t = threadIdx.x;
  a.ktot[(size_t)bh * D + t] = 0;
  a.vamax[(size_t)bh * D + t] = 0u;
  if (t == 0) a.vmaxh[bh] = 0u;
}


// ---------------------------------------------------------------------------
// k-means on fixed-point values ("lightweight" clustering): per head every V
// value is scaled by 2^sh, the largest power of two keeping max|V| * 2^sh below
// 2^13, and rounded to an integer u; u = 128 * (u >> 7) + (u & 127) with both
// parts in int8, so u.c is exact on int8 MFMA (four products, int32 partial
// sums, combined in int64).  Distances ||c||^2 - 2 u.c are exact integers, so
// the cluster ids do not depend on the order of any accumulation.

typedef int v4i __attribute__((ext_vector_type(4)));

// Fixed-point exponent of head bh: the largest power of two 2^sh that keeps
// max|V| * 2^sh below 2^13 (0 for an all-zero head).
__device__ __forceinline__ int head_shift(const Args& a, int bh) {
  const float am = __uint_as_float(a.vmaxh[bh]);
  int e = 0;
  if (am > 0.0f) frexpf(am, &e);
  return am > 0.0f ? 13 - e : 0;
}

// Fixed-point values u = rint(v * 2^sh) (nearest, ties to even) of 16 bf16 (two
// 16-byte words, channel order) as the int8 planes hi = u >> 7 and lo = u & 127,
// so that u = 128 hi + lo.  fma(v * s1, s2, 1.5 * 2^23) with s1 * s2 = 2^sh rounds
// the exact product once to an integer and leaves u + 2^22 in the low 23 bits of
// the result (|u| < 2^13): bits 0-6 are u & 127 and bits 7-14 are (u >> 7) & 0xff.
// s1 = 2^(sh-127) and s2 = 2^127 (BIG) when 2^sh is beyond the fp32 range (heads
// with max|V| below 2^-114); otherwise s2 = 2^sh alone.
template <bool BIG>
__device__ __forceinline__ void fixed_planes16(const v4i& wa, const v4i& wb, float s1, float s2, v4i& hi, v4i& lo) {
  const uint32_t w[8] = {(uint32_t)wa[0], (uint32_t)wa[1], (uint32_t)wa[2], (uint32_t)wa[3],
                         (uint32_t)wb[0], (uint32_t)wb[1], (uint32_t)wb[2], (uint32_t)wb[3]};
  uint32_t q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float f = __uint_as_float((i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16));
    if (BIG) f *= s1;
    q[i] = __float_as_uint(__builtin_fmaf(f, s2, 0x1.8p23f));
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t h = 0u, l = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h |= ((q[4 * d + k] >> 7) & 0xffu) << (8 * k);
      l |= (q[4 * d + k] & 127u) << (8 * k);
    }
    hi[d] = (int)h;
    lo[d] = (int)l;
  }
}

// Sum of one int64 per lane over a wave (exact).
__device__ __forceinline__ long long wave_sum_i64(long long x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}


// Forgy initialisation: seeded partial Fisher-Yates over [0, N), centroid k =
// fixed-point value of token idx[k].  The draws do not depend on the swaps, so
// lane i computes draw i and then resolves, on its own, which value the swaps
// leave at position i.  grid BH, 1024 threads.
__global__ __launch_bounds__(1024) void k_km_init(Args a) {
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
  const int sh = head_shift(a, bh);
  if (t == 0) a.kmsh[bh] = sh;
  __shared__ long long part[2][MAX_CLUSTERS];
  // eight centroids at a time: thread (r, c) = (t / 128, channel t % 128), so the
  // row loads of eight centroids are in flight together
  const int c = t & 127;
#pragma unroll 2
  for (int kk = t >> 7; kk < C; kk += 8) {
    const size_t src = ((size_t)bh * a.N + idx[kk]) * D + c;
    const int u = (int)__builtin_rintf(ldexpf(bf2f(a.v[src]), sh));
    a.centfix[((size_t)bh * C + kk) * D + c] = u;
    a.cent[((size_t)bh * C + kk) * D + c] = ldexpf((float)u, -sh);
    const long long s2 = wave_sum_i64((long long)u * u);
    if ((t & 63) == 0) part[c >> 6][kk] = s2;
  }
  __syncthreads();
  if (t < C) a.kmcc[(size_t)bh * C + t] = part[0][t] + part[1][t];
  if (t < C) a.init_idx[(size_t)bh * C + t] = idx[t];
  // no member yet: the first iteration adds every token
  for (int e = t; e < C * D; e += 1024) a.kmsum[(size_t)bh * C * D + e] = 0;
  if (t < C) a.kmn[(size_t)bh * C + t] = 0;
}

// Warm start: the previous step's centroids (fp32, in the workspace) in the
// current fixed-point scale, rounded to the nearest integer (ties to even) and
// clamped to 14 bits.  grid BH, 128 threads (one per channel).
__global__ __launch_bounds__(128) void k_km_warm(Args a) {
  __shared__ long long part[2][MAX_CLUSTERS];
  const int bh = blockIdx.x, C = a.C, t = threadIdx.x;
  const int sh = head_shift(a, bh);
  if (t == 0) a.kmsh[bh] = sh;
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
  for (int e = t; e < C * D; e += 128) a.kmsum[(size_t)bh * C * D + e] = 0;
  if (t < C) a.kmn[(size_t)bh * C + t] = 0;
}

// Assignment step on int8 MFMA plus per-workgroup member sums.
// grid (nkm, BH), KM_WAVES waves (each takes every KM_WAVES-th 16-token subtile);
// the head's tokens are cut into nkm chunks of equal size (a multiple of 16, at
// most KM_CHUNK), one per workgroup, so that no workgroup is left with a short
// tail chunk while the others run full ones.  Lane (g, j) of a 16-token subtile
// loads the hi/lo bytes of channels 16g..16g+15 and 64+16g..64+16g+15 of token j
// as its MFMA B operand.  In the first iteration every token enters its cluster
// and the same registers are added to the LDS bins; later, only moved tokens
// touch the bins, through a per-wave ring that reloads their planes 16 at a time
// (a few percent of the plane bytes once most labels have settled).
constexpr int CROW = D + 16;  // padded LDS row (bytes): spreads rows over banks

constexpr int KM_WAVES = 8;  // 8 waves: twice the loads in flight of 4 (measured 13 us
                             // less per Lloyd iteration at N=16544, 48 heads)
// Member sums are kept per head (kmsum, kmn) and changed only by the tokens
// whose label changes: after the first Lloyd iteration few do, so few LDS adds
// remain.  A workgroup collects the change of its chunk in packed bins, two
// channels per 64-bit LDS add: a token entering cluster c adds u + 16384 (in
// [8192, 24575]) to c's bin, a token leaving c adds 16384 - u (in [8193, 24576]).
// A bin thus holds sum_in u - sum_out u + 16384 (n_in + n_out); every token adds
// to a cluster's bin at most once, so a half sums at most KM_CHUNK = 2048 terms
// (< 2^26) and never carries into the other; the bias is removed with the counts.
constexpr int BROW2 = D / 2 + 1;  // LDS row of the packed bins (8-byte words)
static_assert(KM_CHUNK * 24576ll < (1ll << 32), "packed member sums would carry");
// Per-wave ring of the tokens whose label changed (chunk token index, and old <<
// 8 | new label), drained 16 at a time so that the member-sum adds run on full
// waves rather than on every subtile that holds one moved token.
constexpr int KM_QUEUE = 32;
// Tokens of one cluster in a 16-lane group add to the same bin words, and those
// atomics serialise; up to 32 clusters the bins are kept twice (even and odd
// lanes), halving the collisions (the dynamic LDS stays within 64 KB for every
// cluster count).
__host__ __device__ constexpr int km_copies(int C) { return C <= 32 ? 2 : 1; }
constexpr size_t km_smem_bytes(int C) {
  return (size_t)C * (2 * CROW + 8 * BROW2 * km_copies(C) + 8) + (size_t)KM_WAVES * KM_QUEUE * 8;
}

// A token entering a cluster: adds u + 16384 to the cluster's bins, two channels
// (16 of the token's, bytes of h and l) per 64-bit word.
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

// A token moving from cluster old to cluster nw: adds u + 16384 to nw's bins and
// 16384 - u to old's, with the channel pairs formed once.
__device__ __forceinline__ void move_bins2(unsigned long long* bins, int nbase, int obase, const v4i& h,
                                           const v4i& l) {
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    const uint32_t hb = (uint32_t)h[wd] ^ 0x80808080u;
    const uint32_t lb = (uint32_t)l[wd];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const uint32_t ua = (((hb >> (16 * pr)) & 0xffu) << 7) + ((lb >> (16 * pr)) & 0xffu);
      const uint32_t ub = (((hb >> (16 * pr + 8)) & 0xffu) << 7) + ((lb >> (16 * pr + 8)) & 0xffu);
      const unsigned long long x = (unsigned long long)ua | ((unsigned long long)ub << 32);
      atomicAdd(&bins[nbase + 2 * wd + pr], x);
      // (32768 - ua) | (32768 - ub) << 32: no borrow between the halves (ua, ub < 32768)
      atomicAdd(&bins[obase + 2 * wd + pr], 0x0000800000008000ull - x);
    }
  }
}

// NT = number of 16-centroid tiles (C <= 16 NT).  Centroids beyond C get a norm
// of 2^62, so their distance never wins and no lane needs a predicate.
// Update step: the member sums and counts take the iteration's changes;
// centroid = member mean rounded to the nearest integer (ties to even; |sum| <
// 2^34 so the fp64 quotient rounds once), empty clusters stay; then the squared
// norm.  A separate launch: handing the update to the last assignment workgroup
// of each head needs a device-scope release fence in every workgroup, which
// writes back the XCD's L2 (measured 4x slower per iteration).  grid (C, BH),
// 128 threads (one per channel); the chunk loops are unrolled so that their
// loads are in flight together.
__global__ __launch_bounds__(128) void k_km_update(Args a) {
  __shared__ long long red[2];
  const int kk = blockIdx.x, bh = blockIdx.y, c = threadIdx.x, C = a.C;
  long long* sum = a.kmsum + ((size_t)bh * C + kk) * D + c;
  long long s = *sum, n = a.kmn[(size_t)bh * C + kk];
  // the chunks' changes 16 at a time, all 16 loads issued before the first wait
  // (chunks past the last read the last one and add nothing); integer adds, so
  // the order cannot change the sums
  for (int ch0 = 0; ch0 < a.nkm; ch0 += 16) {
    int dp[16], dn[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int ch = min(ch0 + k, a.nkm - 1);
      dp[k] = a.kmpart[(((size_t)bh * a.nkm + ch) * C + kk) * D + c];
      dn[k] = a.kmcnt[((size_t)bh * a.nkm + ch) * C + kk];
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      pin_loaded(dp[k]);
      if (ch0 + k < a.nkm) {
        s += dp[k];
        n += dn[k];
      }
    }
  }
  *sum = s;
  int u;
  if (n > 0) {
    u = (int)__builtin_rint((double)s / (double)n);
    a.centfix[((size_t)bh * C + kk) * D + c] = u;
    a.cent[((size_t)bh * C + kk) * D + c] = ldexpf((float)u, -a.kmsh[bh]);
  } else {
    u = a.centfix[((size_t)bh * C + kk) * D + c];
  }
  const long long sq = wave_sum_i64((long long)u * u);
  if ((c & 63) == 0) red[c >> 6] = sq;
  // every thread has read the old count before thread 0 stores the new one
  __syncthreads();
  if (c == 0) {
    a.kmn[(size_t)bh * C + kk] = n;
    a.kmcc[(size_t)bh * C + kk] = red[0] + red[1];
  }
}

// FIRST: the first iteration of this prepare call, where every token enters its
// cluster (labels from an earlier call are not read) and the fixed-point planes
// are formed from V.
template <int NT, bool FIRST>
// Up to 48 clusters two workgroups share a CU (four waves per SIMD), which the
// chunk count assumes; the first-iteration kernel for 33-48 clusters then spills
// 16 bytes per lane rather than run in two rounds.
__global__ __launch_bounds__(64 * KM_WAVES) __attribute__((amdgpu_waves_per_eu(NT <= 3 ? 4 : 2))) void k_km_assign(Args a) {
  extern __shared__ __align__(16) unsigned char km_smem[];
  const int C = a.C;
  int8_t* chi = reinterpret_cast<int8_t*>(km_smem);                       // [C][CROW]
  int8_t* clo = chi + C * CROW;                                           // [C][CROW]
  const int ncopy = km_copies(C);
  unsigned long long* bins = reinterpret_cast<unsigned long long*>(clo + C * CROW);  // [ncopy][C][BROW2]
  int* cnt = reinterpret_cast<int*>(bins + ncopy * C * BROW2);            // [2][C]: entering, leaving
  const int bh = blockIdx.y, chunk = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, g = lane >> 4, l16 = lane & 15;
  unsigned long long* mybins = bins + (ncopy == 2 ? (l16 & 1) * C * BROW2 : 0);  // this lane's copy
  int* mq = cnt + 2 * C + w * 2 * KM_QUEUE;  // this wave's ring: token indices
  int* ml = mq + KM_QUEUE;                  // old << 8 | new label
  // Every workgroup of the launch runs at once and waits for its set-up loads
  // before its first token, so the loads of the set-up (centroids, their norms
  // and the first subtile's operands) are all issued before the first wait.
  long long cc[NT][4];  // squared centroid norms (centroid C-1 stands in past C)
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int v = 0; v < 4; ++v) cc[kt][v] = a.kmcc[(size_t)bh * C + min(16 * kt + 4 * g + v, C - 1)];
  const int8_t* uhi = a.uhi + (size_t)bh * a.N * D;
  const int8_t* ulo = a.ulo + (size_t)bh * a.N * D;
  // The first iteration reads V itself, forms the fixed-point planes of each
  // token where it uses them, and stores them for the later iterations: a lane
  // loads its token's channels 16g..16g+15 (into h0, h1) and 64+16g..64+16g+15
  // (into l0, l1) as bf16, the same 64 bytes as the planes.
  const uint16_t* vh = a.v + (size_t)bh * a.N * D;
  const int sh = FIRST ? head_shift(a, bh) : 0;
  const bool big = sh > 127;  // uniform
  const float s1 = big ? ldexpf(1.0f, sh - 127) : 1.0f, s2 = ldexpf(1.0f, big ? 127 : sh);
  // wave w takes 16-token subtiles w, w+KM_WAVES, ... of the chunk; the operands
  // and previous labels of the next subtile are loaded while the current one is
  // processed (two ahead measured slower: more registers, no latency to hide)
  // chunks of equal size (a multiple of 16 tokens, at most KM_CHUNK)
  const int csz = ((a.N + a.nkm - 1) / a.nkm + 15) & ~15;
  const int first_tok = chunk * csz, last = min(first_tok + csz, a.N);
  struct Sub {
    v4i h0, h1, l0, l1;
    int old;  // the token's label from the previous iteration (-1: none)
  };
  auto load_sub = [&](int s, Sub& x) {
    int jj = first_tok + s * 16 + l16;
    const bool ok = jj < last;
    jj = ok ? jj : last - 1;  // tail lanes read a valid row, add nothing
    if constexpr (FIRST) {
      x.h0 = *reinterpret_cast<const v4i*>(vh + (size_t)jj * D + 16 * g);
      x.h1 = *reinterpret_cast<const v4i*>(vh + (size_t)jj * D + 16 * g + 8);
      x.l0 = *reinterpret_cast<const v4i*>(vh + (size_t)jj * D + 64 + 16 * g);
      x.l1 = *reinterpret_cast<const v4i*>(vh + (size_t)jj * D + 64 + 16 * g + 8);
      x.old = -1;
    } else {
      x.h0 = *reinterpret_cast<const v4i*>(uhi + (size_t)jj * D + 16 * g);
      x.h1 = *reinterpret_cast<const v4i*>(uhi + (size_t)jj * D + 64 + 16 * g);
      x.l0 = *reinterpret_cast<const v4i*>(ulo + (size_t)jj * D + 16 * g);
      x.l1 = *reinterpret_cast<const v4i*>(ulo + (size_t)jj * D + 64 + 16 * g);
      x.old = ok ? a.labels[(size_t)bh * a.N + jj] : -1;
    }
  };
  auto has = [&](int s) { return s < KM_CHUNK / 16 && first_tok + s * 16 < last; };  // uniform per wave
  // moved tokens of later iterations: lane (g, q) of a drain takes ring entry
  // qh + q, reloads channels 16g.. and 64+16g.. of that token (read by this wave
  // a few subtiles earlier, normally still in L2) and moves its bins
  int qh = 0, qn = 0;  // ring head and fill, uniform over the wave
  auto drain = [&](int count) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (l16 < count) {
      const int e = (qh + l16) & (KM_QUEUE - 1);
      const int jj = mq[e], lab = ml[e];
      const v4i h0 = *reinterpret_cast<const v4i*>(uhi + (size_t)jj * D + 16 * g);
      const v4i h1 = *reinterpret_cast<const v4i*>(uhi + (size_t)jj * D + 64 + 16 * g);
      const v4i l0 = *reinterpret_cast<const v4i*>(ulo + (size_t)jj * D + 16 * g);
      const v4i l1 = *reinterpret_cast<const v4i*>(ulo + (size_t)jj * D + 64 + 16 * g);
      const int ob = (lab >> 8) * BROW2, nb = (lab & 0xff) * BROW2;
      move_bins2(mybins, nb + 8 * g, ob + 8 * g, h0, l0);
      move_bins2(mybins, nb + 32 + 8 * g, ob + 32 + 8 * g, h1, l1);
    }
    __builtin_amdgcn_wave_barrier();
  };
  Sub nx;
  if (has(w)) load_sub(w, nx);
  // the centroids, 4 channels per thread and step
  const int* cf = a.centfix + (size_t)bh * C * D;
  {
    constexpr int STEP = 64 * KM_WAVES, MAXS = MAX_CLUSTERS * D / 4 / STEP;
    const int n4 = C * D / 4;
    uint4 cv[MAXS];
#pragma unroll
    for (int i = 0; i < MAXS; ++i) cv[i] = reinterpret_cast<const uint4*>(cf)[min(t + STEP * i, n4 - 1)];
#pragma unroll
    for (int i = 0; i < MAXS; ++i) pin_loaded(cv[i]);
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      const int e = 4 * (t + STEP * i);  // channels e .. e+3 of one centroid
      if (e < C * D) {
        const int u[4] = {(int)cv[i].x, (int)cv[i].y, (int)cv[i].z, (int)cv[i].w};
        uint32_t h = 0u, l = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h |= (uint32_t)((u[k] >> 7) & 0xff) << (8 * k);
          l |= (uint32_t)(u[k] & 127) << (8 * k);
        }
        *reinterpret_cast<uint32_t*>(chi + (e / D) * CROW + (e % D)) = h;
        *reinterpret_cast<uint32_t*>(clo + (e / D) * CROW + (e % D)) = l;
      }
    }
  }
  for (int e = t; e < ncopy * C * BROW2; e += 64 * KM_WAVES) bins[e] = 0ull;
  if (t < 2 * C) cnt[t] = 0;
  // Distances as exact fp64 keys.  For centroid k, D = ||c||^2 - 2 u.c with
  // |D| < 2^35, and key = 64 (D + 2^35) + k is an integer below 2^42, exact in
  // fp64 at every step (fp64 fma runs at the fp32 rate here, 64-bit integer
  // arithmetic takes several instructions per operation).  The smallest key
  // gives the smallest D and, among equal D, the lowest id; k is its low 6 bits.
  // This lane's base keys 64 (||c||^2 + 2^35) + k for centroids 16kt + 4g + v;
  // centroids beyond C get 2^50, above every real key.
  double kbase[NT][4];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      asm volatile("" : "+v"(cc[kt][v]));
      const int k = 16 * kt + 4 * g + v;
      kbase[kt][v] = k < C ? ((double)cc[kt][v] + 0x1p35) * 64.0 + (double)k : 0x1p50;
    }
  __syncthreads();
#pragma unroll 1
  for (int sub = w; sub < KM_CHUNK / 16; sub += KM_WAVES) {
    if (!has(sub)) break;
    const Sub cur = nx;
    if (has(sub + KM_WAVES)) load_sub(sub + KM_WAVES, nx);
    const int j = first_tok + sub * 16 + l16;
    const int old = cur.old;
    v4i bh0, bh1, bl0, bl1;
    if constexpr (FIRST) {
      if (big) {
        fixed_planes16<true>(cur.h0, cur.h1, s1, s2, bh0, bl0);
        fixed_planes16<true>(cur.l0, cur.l1, s1, s2, bh1, bl1);
      } else {
        fixed_planes16<false>(cur.h0, cur.h1, s1, s2, bh0, bl0);
        fixed_planes16<false>(cur.l0, cur.l1, s1, s2, bh1, bl1);
      }
      // Stored as whole 128-byte rows: lanes l16 and l16 ^ 8 swap one half of
      // their token's row (a DPP rotation by 8 within the 16-lane row), so each
      // store writes eight complete rows (chunk g from the lower eight lanes,
      // chunk 4 + g from the upper eight) instead of sixteen half rows.
      const bool up = l16 >= 8;
      v4i sh0, sl0, sh1, sl1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int xh = __builtin_amdgcn_mov_dpp(up ? bh0[e] : bh1[e], 0x128, 0xf, 0xf, false);
        const int xl = __builtin_amdgcn_mov_dpp(up ? bl0[e] : bl1[e], 0x128, 0xf, 0xf, false);
        sh0[e] = up ? xh : bh0[e];
        sh1[e] = up ? bh1[e] : xh;
        sl0[e] = up ? xl : bl0[e];
        sl1[e] = up ? bl1[e] : xl;
      }
      const int ra = first_tok + sub * 16 + (l16 & 7), rb = ra + 8, cb = 16 * g + (up ? 64 : 0);
      if (ra < last) {
        *reinterpret_cast<v4i*>(a.uhi + ((size_t)bh * a.N + ra) * D + cb) = sh0;
        *reinterpret_cast<v4i*>(a.ulo + ((size_t)bh * a.N + ra) * D + cb) = sl0;
      }
      if (rb < last) {
        *reinterpret_cast<v4i*>(a.uhi + ((size_t)bh * a.N + rb) * D + cb) = sh1;
        *reinterpret_cast<v4i*>(a.ulo + ((size_t)bh * a.N + rb) * D + cb) = sl1;
      }
    } else {
      bh0 = cur.h0;
      bh1 = cur.h1;
      bl0 = cur.l0;
      bl1 = cur.l1;
    }
    double bestK = 0x1p52;
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
      const int kr = 16 * kt + l16;
      const int krow = kr < C ? kr : 0;
      const v4i ah0 = *reinterpret_cast<const v4i*>(chi + krow * CROW + 16 * g);
      const v4i ah1 = *reinterpret_cast<const v4i*>(chi + krow * CROW + 64 + 16 * g);
      const v4i al0 = *reinterpret_cast<const v4i*>(clo + krow * CROW + 16 * g);
      const v4i al1 = *reinterpret_cast<const v4i*>(clo + krow * CROW + 64 + 16 * g);
      const v4i z = {0, 0, 0, 0};
      // u.c = 2^14 HH + 2^7 M + LL with M = hi.lo + lo.hi (one accumulator;
      // |M| < 2^22, |LL| < 2^21, so 2^7 M + LL fits an int32)
      v4i HH = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah0, bh0, z, 0, 0, 0);
      HH = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah1, bh1, HH, 0, 0, 0);
      v4i M = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah0, bl0, z, 0, 0, 0);
      M = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah1, bl1, M, 0, 0, 0);
      M = __builtin_amdgcn_mfma_i32_16x16x64_i8(al0, bh0, M, 0, 0, 0);
      M = __builtin_amdgcn_mfma_i32_16x16x64_i8(al1, bh1, M, 0, 0, 0);
      v4i LL = __builtin_amdgcn_mfma_i32_16x16x64_i8(al0, bl0, z, 0, 0, 0);
      LL = __builtin_amdgcn_mfma_i32_16x16x64_i8(al1, bl1, LL, 0, 0, 0);
      // lane (g, token l16) holds centroids 16kt + 4g + v:
      // key = base - 64 * 2 u.c = base - 2^21 HH - 2^7 (2^7 M + LL)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int X = M[v] * 128 + LL[v];
        const double key = __builtin_fma(-0x1p21, (double)HH[v], __builtin_fma(-128.0, (double)X, kbase[kt][v]));
        bestK = __builtin_fmin(bestK, key);
      }
    }
    // smallest key across the four lane groups
    bestK = xmin_f64<32>(xmin_f64<16>(bestK));
    const double hi = __builtin_floor(bestK * 0x1p-6);
    const int best = (int)__builtin_fma(-64.0, hi, bestK);
    // only a token whose label changes touches the bins
    const bool moved = j < last && best != old;
    if constexpr (FIRST) {
      // every token enters: the adds run on the subtile's own operands
      if (__ballot(moved) != 0ull && moved) {
        if (g == 0) {
          a.labels[(size_t)bh * a.N + j] = best;
          atomicAdd(&cnt[best], 1);
        }
        add_bins2(mybins, best * BROW2 + 8 * g, bh0, bl0);
        add_bins2(mybins, best * BROW2 + 32 + 8 * g, bh1, bl1);
      }
    } else {
      // the four lane groups of a token agree on moved: bits 0-15 are the tokens
      const uint32_t tm = (uint32_t)__ballot(moved) & 0xffffu;
      if (tm != 0u) {
        if (moved && g == 0) {
          a.labels[(size_t)bh * a.N + j] = best;
          atomicAdd(&cnt[best], 1);
          atomicAdd(&cnt[C + old], 1);
          const int e = (qh + qn + __popc(tm & ((1u << l16) - 1u))) & (KM_QUEUE - 1);
          mq[e] = j;
          ml[e] = (old << 8) | best;
        }
        qn += __popc(tm);
        if (qn >= 16) {
          drain(16);
          qh = (qh + 16) & (KM_QUEUE - 1);
          qn -= 16;
        }
      }
    }
  }
  if (!FIRST && qn > 0) drain(qn);
  __syncthreads();
  int* part = a.kmpart + ((size_t)bh * a.nkm + chunk) * C * D;
  for (int e = t; e < C * D; e += 64 * KM_WAVES) {
    const int c = e / D, ch = e % D;
    // the copies' halves each stay below 2^26, so their sum cannot carry
    unsigned long long wv = bins[c * BROW2 + (ch >> 1)];
    if (ncopy == 2) wv += bins[(C + c) * BROW2 + (ch >> 1)];
    const uint32_t half = (ch & 1) ? (uint32_t)(wv >> 32) : (uint32_t)wv;
    part[e] = (int)half - 16384 * (cnt[c] + cnt[C + c]);
  }
  if (t < C) a.kmcnt[((size_t)bh * a.nkm + chunk) * C + t] = cnt[t] - cnt[C + t];
}


// ---------------------------------------------------------------------------
// Stable counting sort of positions by cluster id.  grid BH, 1024 threads.
// Wave w owns one contiguous run of tokens: it counts its run per cluster, the
// runs' counts give every (wave, cluster) its first position, and the wave then
// walks its run again in order, ranking tokens of one cluster inside each
// 64-token step by a ballot match and keeping its running offsets in LDS of its
// own (no barrier inside the walks).
__device__ __forceinline__ void write_header(const Args& a, uint32_t clustered) {
  a.header->magic = MAGIC;
  a.header->clustered = clustered;
  a.header->B = a.B;
  a.header->H = a.H;
  a.header->N = a.N;
  a.header->C = a.C;
}

// Stable counting sort of a head's tokens by cluster id, over the k-means chunks
// (grid (chunks, BH), 16 waves): k_perm_count writes each chunk's cluster counts
// (into the k-means count buffer, free once the last update has run), then
// k_perm_scatter places every token at
//   (tokens of smaller clusters) + (same cluster, earlier chunks)
//   + (same cluster, earlier waves of its chunk) + (same cluster, lower lanes of
//   earlier steps and of its own step),
// i.e. cluster order with ties in token order.  A wave takes a contiguous run of
// its chunk 64 tokens per step; lanes with the same label find each other by a
// ballot over the label bits.
struct PermRun {
  int j0, j1;  // the wave's tokens
};
__device__ __forceinline__ PermRun perm_run(const Args& a, int ch, int w) {
  const int csz = ((a.N + a.nkm - 1) / a.nkm + 15) & ~15;  // the k-means chunks
  const int first = min(ch * csz, a.N), last = min(first + csz, a.N);
  const int per = (((csz + 15) / 16) + 63) & ~63;
  const int j0 = min(first + w * per, last);
  return {j0, min(j0 + per, last)};
}
// lanes with the same label as this lane (a lane past the run takes the sentinel
// bucket MAX_CLUSTERS)
__device__ __forceinline__ unsigned long long label_peers(int l) {
  unsigned long long peers = ~0ull;
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const unsigned long long m = __ballot((l >> b) & 1);
    peers &= ((l >> b) & 1) ? m : ~m;
  }
  return peers;
}
// per-wave cluster counts of the wave's run into wcnt[w][.] (zeroed by the caller)
__device__ __forceinline__ void perm_count_run(const int* lab, PermRun r, int lane, int* wrow) {
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int jb = r.j0; jb < r.j1; jb += 64) {
    const int j = jb + lane;
    const int l = j < r.j1 ? lab[j] : MAX_CLUSTERS;
    const unsigned long long peers = label_peers(l);
    // the lowest lane of each label adds the label's count (distinct words)
    if (l < MAX_CLUSTERS && (peers & lt) == 0ull) wrow[l] += __popcll(peers);
  }
}

__global__ __launch_bounds__(1024) void k_perm_count(Args a) {
  __shared__ int wcnt[16][MAX_CLUSTERS + 1];
  const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6, C = a.C;
  for (int e = t; e < 16 * (MAX_CLUSTERS + 1); e += 1024) (&wcnt[0][0])[e] = 0;
  __syncthreads();
  perm_count_run(a.labels + (size_t)bh * a.N, perm_run(a, ch, w), lane, wcnt[w]);
  __syncthreads();
  if (t < C) {
    int n = 0;
#pragma unroll
    for (int ww = 0; ww < 16; ++ww) n += wcnt[ww][t];
    a.kmcnt[((size_t)bh * a.nkm + ch) * C + t] = n;
  }
}

__global__ __launch_bounds__(1024) void k_perm_scatter(Args a) {
  __shared__ int wcnt[16][MAX_CLUSTERS + 1];  // per wave: count, then next position
  __shared__ int tot[MAX_CLUSTERS], pre[MAX_CLUSTERS];
  const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6, C = a.C;
  // the workspace now holds clusters for this shape (read back by later calls
  // that reuse them, after this launch has completed)
  if (bh == 0 && ch == 0 && t == 0) write_header(a, 1u);
  const int* lab = a.labels + (size_t)bh * a.N;
  int* perm = a.perm + (size_t)bh * a.N;
  int* iperm = a.iperm + (size_t)bh * a.N;
  const PermRun r = perm_run(a, ch, w);
  for (int e = t; e < 16 * (MAX_CLUSTERS + 1); e += 1024) (&wcnt[0][0])[e] = 0;
  if (t < MAX_CLUSTERS) {
    tot[t] = 0;
    pre[t] = 0;
  }
  __syncthreads();
  perm_count_run(lab, r, lane, wcnt[w]);
  // every chunk's counts: cluster totals, and this cluster's tokens in earlier
  // chunks (integer adds, any order)
  const int* cnt = a.kmcnt + (size_t)bh * a.nkm * C;
  for (int e = t; e < a.nkm * C; e += 1024) {
    const int x = cnt[e], c = e % C;
    atomicAdd(&tot[c], x);
    if (e / C < ch) atomicAdd(&pre[c], x);
  }
  __syncthreads();
  // first position of (wave, cluster)
  if (t < C) {
    int below = pre[t];
    for (int c = 0; c < t; ++c) below += tot[c];
    for (int ww = 0; ww < 16; ++ww) {
      const int n = wcnt[ww][t];
      wcnt[ww][t] = below;
      below += n;
    }
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int jb = r.j0; jb < r.j1; jb += 64) {
    const int j = jb + lane;
    const int l = j < r.j1 ? lab[j] : MAX_CLUSTERS;
    const unsigned long long peers = label_peers(l);
    if (l < MAX_CLUSTERS) {
      const int pos = wcnt[w][l] + __popcll(peers & lt);
      perm[pos] = j;
      iperm[j] = pos;
    }
    // every lane has read its offset before the lowest lane of each label moves it
    __builtin_amdgcn_wave_barrier();
    if (l < MAX_CLUSTERS && (peers & lt) == 0ull) wcnt[w][l] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

// Identity permutation (V-Smooth off).  grid (ceil(N/256), BH), 256 threads.
__global__ __launch_bounds__(256) void k_perm_identity(Args a) {
  const int j = blockIdx.x * 256 + threadIdx.x, bh = blockIdx.y;
  if (j == 0 && bh == 0) write_header(a, 0u);
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
// t/16 + 16i), so 16 threads cover one 256-byte row.  A thread keeps its 8 rows
// as raw bf16 (32 registers, not 64 floats) and converts them where they are
// used, which doubles the waves a CU holds and the rows in flight.
// One workgroup of 256 threads per (block, head, Q or K).
template <bool SMOOTH>
__device__ __forceinline__ void qk_quant_block(const Args& a, int blk, int bh, int isk) {
  __shared__ float wmax[4];
  __shared__ long long qsum[16][D];
  __shared__ float qmean[D];
  const int t = threadIdx.x;
  const int cg = t & 15, r0 = t >> 4;
  const bool follow = isk || (a.flags & VC_PERMUTE_Q);
  const bool smooth = SMOOTH && !isk;  // uniform over the workgroup
  const uint16_t* src = (isk ? a.k : a.q) + (size_t)bh * a.N * D;
  const int nrow = a.N - blk * BLK;  // rows r < nrow of the block are tokens
  // Rows are read once and codes written once: non-temporal accesses keep them
  // from displacing other lines in L2 (measured 24 us less at 2x24x16544; the
  // 16 lanes of a row make each access two whole 128-byte lines).
  // All 8 positions, then all 8 rows, are loaded before any is waited on: rows
  // past N read the last position's row and are cleared after, so no branch
  // stands between the loads (a load under a per-row branch waits for the one
  // before it).
  int j[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) j[i] = min(blk * BLK + r0 + 16 * i, a.N - 1);
  if (follow) {  // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < 8; ++i) j[i] = a.perm[(size_t)bh * a.N + j[i]];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) pin_loaded(j[i]);
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const v4i x = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + (size_t)j[i] * D + cg * 8));
    raw[i] = make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pin_loaded(raw[i]);
    if (r0 + 16 * i >= nrow) raw[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // K channel mean from the head's fixed-point sums (while the rows load); the
  // first block's workgroup also stores it
  __shared__ float skbar[D];
  if (isk) {  // uniform over the workgroup
    if (t < D) {
      const float kb = fixed_mean(a.ktot[(size_t)bh * D + t], a.N);
      skbar[t] = kb;
      if (blk == 0) a.kbar[(size_t)bh * D + t] = kb;
    }
    __syncthreads();
  }
  // value subtracted from channel e: the K channel mean, or (smoothed queries)
  // the block mean once it is known
  float sub[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sub[e] = isk ? skbar[cg * 8 + e] : 0.0f;
  // element e of row i as fp32, minus sub[e] (exact order of the reference: one
  // fp32 subtraction)
  auto val = [&](int i, int e) {
    const uint32_t w = e < 2 ? raw[i].x : e < 4 ? raw[i].y : e < 6 ? raw[i].z : raw[i].w;
    return bf2f((e & 1) ? (w >> 16) : w) - sub[e];
  };
  // Between the passes over the rows the compiler is told the raw words may have
  // changed, so it converts them again instead of keeping 64 floats live.
  auto fence = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));
  };
  if (smooth) {
    const int n = min(BLK, nrow);
    double sm[8];  // 8 rows per thread: exact in fp64 (see fx24d); rows past N hold 0
#pragma unroll
    for (int e = 0; e < 8; ++e) sm[e] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm[e] += fx24d(val(i, e));
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
    for (int e = 0; e < 8; ++e) sub[e] = qmean[cg * 8 + e];
    fence();
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (r0 + 16 * i < nrow) {
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(val(i, e)));
    }
  amax = wave_max(amax);
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float s, inv;
  scale_from_amax(amax, &s, &inv);
  fence();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + 16 * i, p = blk * BLK + r;
    uint32_t w0 = 0u, w1 = 0u;
    if (r < nrow) {
      w0 = e4m3x2(val(i, 0) * inv, val(i, 1) * inv) | (e4m3x2(val(i, 2) * inv, val(i, 3) * inv) << 16);
      w1 = e4m3x2(val(i, 4) * inv, val(i, 5) * inv) | (e4m3x2(val(i, 6) * inv, val(i, 7) * inv) << 16);
    }
    // with the 4-bit residual a K code row goes to the tile row v4_krow(r)
    const int prow = (isk && (a.flags & VC_V4)) ? blk * BLK + v4_krow(r) : p;
    uint8_t* dst = (isk ? a.k8 : a.q8) + ((size_t)bh * a.Npad + prow) * D + cg * 8;
    __builtin_nontemporal_store(((unsigned long long)w1 << 32) | w0, reinterpret_cast<unsigned long long*>(dst));
    if (isk && (a.flags & VC_EXACT_SCORES)) {
      // the K codes decoded to bf16 (E4M3 values are exact in bf16)
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wd = e < 2 ? w0 : w1;
        const uint32_t b0 = (wd >> (16 * (e & 1))) & 0xff, b1 = (wd >> (16 * (e & 1) + 8)) & 0xff;
        h[e] = (__float_as_uint(e4m3_val(b0)) >> 16) | (__float_as_uint(e4m3_val(b1)) & 0xffff0000u);
      }
      *reinterpret_cast<uint4*>(a.k16 + ((size_t)bh * a.Npad + prow) * D + cg * 8) =
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
// runs on VALU fma, register-tiled: a workgroup computes 32 query blocks x 256
// keys, each thread 8 x 4 outputs; 32 channels at a time pass through LDS
// (k - kbar channel-major, the means channel-major), and per channel a thread
// reads three float4 (two of them the same across its wave) and issues 32 fma.
// The next 32 channels of each key row are loaded while the current ones are
// used.  grid (ceil(nblk/32), ceil(Npad/256), BH), 256 threads; the block groups
// of one key tile are neighbours, so the key rows are fetched from HBM about
// once.
__global__ __launch_bounds__(256) void k_qbias(Args a) {
  constexpr int QB = 32, KT = 256, CC = 32;
  __shared__ __align__(16) float skt[CC][KT];  // k - kbar, [channel][key]
  __shared__ __align__(16) float sqm[CC][QB];  // qbar, [channel][block]
  const int bh = blockIdx.z, t = threadIdx.x;
  const int b0 = blockIdx.x * QB, nb = min(QB, a.nblk - b0);
  const int p0 = blockIdx.y * KT;
  const int bq = t >> 6, kq = t & 63;  // outputs: blocks 8bq..8bq+7, keys 4kq..4kq+3
  // loader role: key p0 + t of the tile; the next chunk of its row is loaded
  // while the current one is used
  const int pl = p0 + t;
  const bool vl = pl < a.N;
  const uint4* row = reinterpret_cast<const uint4*>(a.k + ((size_t)bh * a.N + (vl ? a.perm[(size_t)bh * a.N + pl] : 0)) * D);
  const float* kbar = a.kbar + (size_t)bh * D;
  float acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  uint4 nxt[CC / 8];
#pragma unroll
  for (int i = 0; i < CC / 8; ++i) nxt[i] = row[i];
#pragma unroll 1
  for (int c0 = 0; c0 < D; c0 += CC) {
    uint4 cur[CC / 8];
#pragma unroll
    for (int i = 0; i < CC / 8; ++i) cur[i] = nxt[i];
    if (c0 + CC < D) {
#pragma unroll
      for (int i = 0; i < CC / 8; ++i) nxt[i] = row[(c0 + CC) / 8 + i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CC / 8; ++i) {
      const uint32_t h[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
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
#pragma unroll 4
    for (int c = 0; c < CC; ++c) {
      const float4 q0 = *reinterpret_cast<const float4*>(&sqm[c][8 * bq]);
      const float4 q1 = *reinterpret_cast<const float4*>(&sqm[c][8 * bq + 4]);
      const float4 kv = *reinterpret_cast<const float4*>(&skt[c][4 * kq]);
      const float qa[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w}, ka[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(qa[i], ka[j], acc[i][j]);
    }
  }
  const int pk = p0 + 4 * kq;
  if (pk < a.Npad) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int b = 8 * bq + i;
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
// 32-key group (rows 32G .. 32G+31) and its E8M0 exponent.
// One workgroup of 256 threads per block: thread = (8-channel chunk t%16, rows
// t/16 + 16i), so rows 2G and 2G+1 of a thread lie in group G.  The block sums
// and, after them, the block maxima share the 16 KB LDS buffer sbuf; smu holds
// 128 floats of LDS.
__device__ __forceinline__ void v_stats_block(const Args& a, int blk, int bh, long long* sbuf, float* smu) {
  long long (*ssum)[D] = reinterpret_cast<long long (*)[D]>(sbuf);
  float (*smax)[8][D] = reinterpret_cast<float (*)[8][D]>(sbuf);
  const int t = threadIdx.x;
  const int cg = t & 15, r0 = t >> 4;
  const int p0 = blk * BLK, n = min(BLK, a.N - p0);
  const bool vs = (a.flags & VC_VSMOOTH) != 0;
  const uint16_t* vh = a.v + (size_t)bh * a.N * D;
  const int* perm = a.perm + (size_t)bh * a.N;
  // the thread's 8 rows as raw bf16 (32 registers); rows past N hold 0.  All
  // 8 positions, then all 8 rows, are loaded before any is waited on: rows past
  // N read the last position's row and are cleared after, so no branch stands
  // between the loads.
  int src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) src[i] = perm[min(p0 + r0 + 16 * i, a.N - 1)];
#pragma unroll
  for (int i = 0; i < 8; ++i) pin_loaded(src[i]);
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const uint4*>(vh + (size_t)src[i] * D + cg * 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pin_loaded(raw[i]);
    if (r0 + 16 * i >= n) raw[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  auto val = [&](int i, int e) {
    const uint32_t w = e < 2 ? raw[i].x : e < 4 ? raw[i].y : e < 6 ? raw[i].z : raw[i].w;
    return bf2f((e & 1) ? (w >> 16) : w);
  };
  double s[8];  // 8 rows per thread: exact in fp64 (see fx24d)
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += fx24d(val(i, e));
#pragma unroll
  for (int e = 0; e < 8; ++e) ssum[r0][cg * 8 + e] = (long long)s[e];
  __syncthreads();
  if (t < D) {
    long long tot = 0;
    for (int rr = 0; rr < 16; ++rr) tot += ssum[rr][t];
    smu[t] = vs ? fixed_mean(tot, n) : 0.0f;
  }
  __syncthreads();
  // the raw words may have changed (for the compiler): convert them again
  // rather than keep 64 floats live across the barrier
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));
  // per group: the thread's two rows, then the neighbour with r0 ^ 1 (lane
  // t ^ 16, same channels), so 8 partial maxima per group and channel remain
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = 0.0f;
#pragma unroll
    for (int i = 2 * G; i < 2 * G + 2; ++i)
      if (r0 + 16 * i < n) {
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(val(i, e) - smu[cg * 8 + e]));
      }
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = xmax16(m[e]);
    if ((r0 & 1) == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) smax[G][r0 >> 1][cg * 8 + e] = m[e];
    }
  }
  __syncthreads();
  if (t < D) {
    float gm[4];
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      float mm = 0.0f;
      for (int rr = 0; rr < 8; ++rr) mm = fmaxf(mm, smax[G][rr][t]);
      gm[G] = mm;
    }
    const size_t o = ((size_t)bh * a.nblk + blk) * D + t;
    a.mu[o] = smu[t];
    const float bm = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
    a.bamax[o] = bm;
    // the channel's maximum over the head's blocks (bm >= 0: bits order like values)
    atomicMax(a.vamax + (size_t)bh * D + t, __float_as_uint(bm));
    if (a.flags & VC_V4) {
      uint8_t* rec = a.v4s + ((size_t)bh * a.nblk + blk) * V4_SREC;
#pragma unroll
      for (int G = 0; G < 4; ++G) rec[(16 * G + (t & 15)) * 8 + (t >> 4)] = (uint8_t)(mx_exponent(gm[G]) + 127);
    }
  }
}

// The K channel sums and the V block statistics in one launch: they read
// different tensors and write different outputs, and the V statistics alone
// leave much of the memory bandwidth unused (a workgroup waits on its gathers,
// then reduces), so the K stream runs in those gaps.  grid (nkc + nblk, BH), 256
// threads: workgroups x < nkc sum K chunk x, the others take V block x - nkc;
// every head's K chunks come just before its V blocks, so the two kinds stay
// mixed over the whole launch.  Both roles share one 16.5 KB LDS buffer, so six
// workgroups fit a CU.
__global__ __launch_bounds__(256, 6) void k_ksum_v_stats(Args a) {
  __shared__ __align__(16) long long sbuf[16 * D];
  __shared__ float smu[D];
  const int x = blockIdx.x, bh = blockIdx.y;
  if (x < a.nkc)  // uniform over the workgroup
    ksum_chunk<true, false>(a, x, bh, reinterpret_cast<long long (*)[D]>(sbuf), smu);
  else
    v_stats_block(a, x - a.nkc, bh, sbuf, smu);
}

// Channel c's residual scale, set by the head's largest |V - mu| (one per
// channel: sv = max/448, inv = 448/max; 1 with the 4-bit residual), and block
// blk's mean in V code units (mu * inv).  Block 0 also stores the scales.  The
// bf16 high/low pairs of the means that the restore MFMA reads are formed from
// these by the repair selection (k_qk_quant_rep), which writes them in whole rows.
__device__ __forceinline__ void v_channel(const Args& a, int bh, int blk, int c, float* mu_out, float* s_out,
                                          float* inv_out) {
  float s, inv;
  scale_from_amax(__uint_as_float(a.vamax[(size_t)bh * D + c]), &s, &inv);
  if (a.flags & VC_V4) s = inv = 1.0f;  // the 4-bit residual carries its own powers of two
  if (blk == 0) {
    a.sv[(size_t)bh * D + c] = s;
    a.inv[(size_t)bh * D + c] = inv;
  }
  const size_t o = ((size_t)bh * a.nblk + blk) * D + c;
  const float mu = a.mu[o];
  const float x = mu * inv;
  a.mup[o] = x;
  *mu_out = mu;
  *s_out = s;
  *inv_out = inv;
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
  v_channel(a, bh, blk, t, &smu[t], &ssv[t], &sinv[t]);
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
  // 128 channel rows x 128 bytes, 8 lanes per row: each store writes 16 whole rows
  uint8_t* dst = a.v8t + (size_t)bh * D * a.Npad + (size_t)blk * BLK;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 16 * i + (t >> 3), ch = t & 7;
    *reinterpret_cast<uint4*>(dst + (size_t)c * a.Npad + 16 * ch) = *reinterpret_cast<const uint4*>(tile + c * BLK + 16 * ch);
  }
}

// 4-bit residual codes (VC_V4) and the repair criterion.  The group exponents
// come from k_ksum_v_stats.  Thread t owns the key pair 2t, 2t+1 of a block, whose
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
  {
    float sc, iv;  // 1 with the 4-bit residual
    v_channel(a, bh, blk, t, &smu[t], &sc, &iv);
    v_channel(a, bh, blk, t + 64, &smu[t + 64], &sc, &iv);
  }
  {
    // the record is [group][channel % 16][channel / 16]: transpose to channel
    // order; thread t loads bytes 8t .. 8t+7 at once
    static_assert(V4_SREC == 8 * 64, "one 8-byte load per thread covers the record");
    const uint8_t* rec = a.v4s + ((size_t)bh * a.nblk + blk) * V4_SREC;
    const uint2 rb = *reinterpret_cast<const uint2*>(rec + 8 * t);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int q = 8 * t + k;
      sx[q >> 7][16 * (q & 7) + ((q >> 3) & 15)] = (uint8_t)(((k < 4 ? rb.x : rb.y) >> (8 * (k & 3))) & 0xffu);
    }
  }
  const int p0 = blk * BLK, n = min(BLK, a.N - p0);
  const int k0 = 2 * t;
  const int G = v4_group(k0);
  const int byte = t;  // keys 2t, 2t+1: byte t of the channel row (position order)
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
// Restore operand and repair set.  First the bf16 high/low block means for the
// restore MFMA; then (m > 0) the m positions with the largest error (ties:
// lower position), by an exact radix select on the 64-bit key (~err_bits,
// position), then a compaction in position order.  grid BH, 1024 threads.
//
// Most errors share their leading digits (sign and exponent), so one shared
// 256-bin histogram would see most lanes of an LDS add hit the same word; each
// of RS_COPIES lanes of a wave counts into its own copy instead (no two lanes
// of an instruction share an address), and the copies are summed for the scan.
// The compaction gives each wave one contiguous run of positions, so it needs
// two barriers rather than four per NTH positions.  One workgroup of NTH
// threads per head; COPIES lane-private histogram copies.
__device__ __forceinline__ void rep_delta_half(const Args& a, int bh, int gs, int c0);

template <int NTH, int COPIES>
__device__ __forceinline__ void rep_select_head(const Args& a, int bh) {
  constexpr int NW = NTH / 64;
  __shared__ int hist[256][COPIES];
  __shared__ unsigned long long s_prefix, s_mask;
  __shared__ int s_kth, s_kth_next, s_hsel;
  __shared__ int wtot[NW];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  // the restore operand first: the bf16 high/low pair of every block mean in V
  // code units, [group of 16 blocks][high, low][channel][block in group], slots
  // past the last block 0.  A thread forms one (group, channel) row of 16
  // blocks and stores it whole (the quantisation workgroups, one per block,
  // would each write 2 bytes into every row).
  for (int e = t; e < a.nch16 * D; e += NTH) {
    const int grp = e / D, c = e % D;
    const float* mp = a.mup + ((size_t)bh * a.nblk + grp * 16) * D + c;
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      uint32_t h2 = 0u, l2 = 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float x = grp * 16 + j + u < a.nblk ? mp[(size_t)(j + u) * D] : 0.0f;
        const uint32_t h = f2bf_rne(x);
        const uint32_t l = f2bf_rne(x - __uint_as_float(h << 16));
        h2 |= h << (16 * u);
        l2 |= l << (16 * u);
      }
      hw[j / 2] = h2;
      lw[j / 2] = l2;
    }
    uint16_t* dst = a.mupt + (((size_t)bh * a.nch16 + grp) * 2) * D * 16 + (size_t)c * 16;
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    reinterpret_cast<uint4*>(dst + D * 16)[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    reinterpret_cast<uint4*>(dst + D * 16)[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
  }
  if (a.m == 0) return;  // no repair set (uniform)
  const int cp = lane & (COPIES - 1);
  const float* err = a.err + (size_t)bh * a.N;
  auto key_of = [&](int j, int e) { return ((unsigned long long)(~(unsigned)e) << 32) | (unsigned)j; };
  // the error bits of positions j0, j0 + step, ..., 8 at a time: all 8 loads
  // are issued before the first wait (positions at or past N read position
  // N - 1; the callers skip them)
  auto load8 = [&](int j0, int step, int (&e)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) e[u] = __float_as_int(err[min(j0 + step * u, a.N - 1)]);
#pragma unroll
    for (int u = 0; u < 8; ++u) pin_loaded(e[u]);
  };
  if (t == 0) {
    s_prefix = 0ull;
    s_mask = 0ull;
    s_kth = a.m;
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int e = t; e < 256 * COPIES; e += NTH) (&hist[0][0])[e] = 0;
    __syncthreads();
    const unsigned long long pre = s_prefix, msk = s_mask;
    for (int jb = t; jb < a.N; jb += NTH * 8) {
      int e[8];
      load8(jb, NTH, e);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = jb + NTH * u;
        const unsigned long long key = key_of(j, e[u]);
        if (j < a.N && (key & msk) == pre) atomicAdd(&hist[(key >> shift) & 255][cp], 1);
      }
    }
    __syncthreads();
    // bin totals (threads 0..255; copy i of bin t read at (i + t) mod COPIES,
    // so the lanes of a read hit distinct banks), then a parallel exclusive scan;
    // the one bin where the running count crosses kth fixes the next digit
    int h = 0, incl = 0;
    if (t < 256) {
#pragma unroll 8
      for (int i = 0; i < COPIES; ++i) h += hist[t][(i + t) & (COPIES - 1)];
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
  // wave w owns positions [j0, j1): count its selected keys, then write them
  const int per = (((a.N + NW - 1) / NW) + 63) & ~63;
  const int j0 = min(w * per, a.N), j1 = min(j0 + per, a.N);
  const unsigned long long lt = (1ull << lane) - 1ull;
  int cnt = 0;
  for (int jb = j0; jb < j1; jb += 64 * 8) {
    int e[8];
    load8(jb + lane, 64, e);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jb + 64 * u + lane;
      cnt += __popcll(__ballot(j < j1 && key_of(j, e[u]) <= thr));
    }
  }
  if (lane == 0) wtot[w] = cnt;
  __syncthreads();
  int slot = 0;
  for (int ww = 0; ww < w; ++ww) slot += wtot[ww];
  for (int jb = j0; jb < j1; jb += 64 * 8) {
    int e[8];
    load8(jb + lane, 64, e);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jb + 64 * u + lane;
      const bool sel = j < j1 && key_of(j, e[u]) <= thr;
      const unsigned long long b = __ballot(sel);
      const int s = slot + __popcll(b & lt);
      if (sel && s < a.mpad) out[s] = j;  // exactly m keys are <= thr
      slot += __popcll(b);
    }
  }
  for (int i = a.m + t; i < a.mpad; i += NTH) out[i] = -1;
  // the repair deltas of the selected slots: two threads per slot, 64 channels
  // each (the positions were stored by this workgroup before the barrier)
  static_assert(NTH % 128 == 0, "whole slots per pass");
  __syncthreads();
  for (int e = t; e < 2 * a.mpad; e += NTH) rep_delta_half(a, bh, e % a.mpad, (e / a.mpad) * (D / 2));
}

// The repair selection and the Q/K codes in one launch.  The selection runs one
// workgroup per head and leaves most of the chip idle; the code workgroups do
// not depend on it, so they fill the chip around it.  grid 1-D: workgroups
// x < BH select head x's repair set (first, so they start first); the rest are
// the code workgroups in (block, head, Q/K) order.  Seven code workgroups per
// CU (at eight the compiler spills); the selection's histogram keeps 8 copies
// (8 KB of LDS) so that it does not lower that.
template <bool SMOOTH>
__global__ __launch_bounds__(256, SMOOTH ? 4 : 7) void k_qk_quant_rep(Args a) {
  const unsigned x = blockIdx.x, BH = (unsigned)a.BH;
  if (x < BH) {  // uniform over the workgroup
    rep_select_head<256, 8>(a, (int)x);
    return;
  }
  const unsigned q = x - BH, per = (unsigned)a.nblk * BH;
  const unsigned r = q % per;
  qk_quant_block<SMOOTH>(a, (int)(r % (unsigned)a.nblk), (int)(r / (unsigned)a.nblk), (int)(q / per));
}

// Residual error (bf16; V code units, real units with VC_V4) of channels
// c0 .. c0+63 of repair slot gs of head bh, stored straight into the
// channel-major slot layout (rep_col interleave) that the forward's repair MFMA
// reads; slots past m hold 0.  The V codes are recomputed exactly as the V code
// kernels form them.
__device__ __forceinline__ void rep_delta_half(const Args& a, int bh, int gs, int c0) {
  const int grp = gs / BLK, col = rep_col(gs % BLK);
  uint16_t* dst = a.rep_dt + ((size_t)bh * D + c0) * a.mpad + (size_t)grp * BLK + col;
  const int p = gs < a.m ? a.rep_pos[(size_t)bh * a.mpad + gs] : -1;
  if (p < 0) {
#pragma unroll 8
    for (int c = 0; c < D / 2; ++c) dst[(size_t)c * a.mpad] = 0;
    return;
  }
  const uint16_t* row = a.v + ((size_t)bh * a.N + a.perm[(size_t)bh * a.N + p]) * D + c0;
  const float* mu = a.mu + ((size_t)bh * a.nblk + p / BLK) * D + c0;
  const uint8_t* xr = a.v4s + ((size_t)bh * a.nblk + p / BLK) * V4_SREC + 16 * v4_group(p % BLK) * 8;
  const float* inv = a.inv + (size_t)bh * D + c0;
  // 32 channels at a time, their row words loaded before the first wait (the
  // selection shares its launch with the Q/K codes and their register budget)
  for (int q = 0; q < 2; ++q) {
    uint4 rw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rw[i] = *reinterpret_cast<const uint4*>(row + 32 * q + i * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) pin_loaded(rw[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h[4] = {rw[i].x, rw[i].y, rw[i].z, rw[i].w};
      const int cb = 32 * q + 8 * i;  // channel c0 + cb of the chunk's first word
      if (a.flags & VC_V4) {
        // 4-bit residual: the error of the E2M1 code under its group's power
        // of two, in real units
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = c0 + cb + j;
          const int X = (int)xr[(c & 15) * 8 + (c >> 4)] - 127;
          const float x = bf2f((j & 1) ? (h[j >> 1] >> 16) : h[j >> 1]) - mu[cb + j];
          uint32_t code;
          const float val = e2m1_round(__builtin_ldexpf(x, -X), &code);
          dst[(size_t)(cb + j) * a.mpad] = f2bf_rne(x - __builtin_ldexpf(val, X));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = cb + 2 * j;
          const float x0 = (bf2f(h[j]) - mu[c]) * inv[c];
          const float x1 = (bf2f(h[j] >> 16) - mu[c + 1]) * inv[c + 1];
          const uint32_t cc = e4m3x2(x0, x1);
          dst[(size_t)c * a.mpad] = f2bf_rne(x0 - e4m3_val(cc & 0xff));
          dst[(size_t)(c + 1) * a.mpad] = f2bf_rne(x1 - e4m3_val(cc >> 8));
        }
      }
    }
  }
}

// Number of k-means chunks per head for a device with cus compute units.  The
// assignment moves every token's 256 bytes once per iteration, and a CU's
// resident workgroups share its bandwidth, so with all workgroups resident at
// once the time is set by the CU holding the most: ceil(BH * n / cus) chunks of
// ceil16(N / n) tokens.  Among the n in [nkm, 4 nkm] whose BH * n workgroups
// are all resident (two per CU up to 48 clusters, else one: registers), the
// smallest n that minimises that count; nkm itself when none fits (measured:
// letting workgroups wait for a second pass is slower than larger chunks).
int km_chunks(const Args& a, int cus) {
  const long long slots = (long long)cus * (a.C <= 48 ? 2 : 1);
  long long best = -1;
  int pick = a.nkm;
  for (int n = a.nkm; n <= 4 * a.nkm; ++n) {
    if ((long long)a.BH * n > slots) break;
    const long long per_cu = ((long long)a.BH * n + cus - 1) / cus;
    const long long csz = (((long long)a.N + n - 1) / n + 15) / 16 * 16;
    if (best < 0 || per_cu * csz < best) {
      best = per_cu * csz;
      pick = n;
    }
  }
  return pick;
}

}  // namespace

template <int NT>
void launch_assign(const Args& a, bool first, dim3 kg, dim3 kb, size_t sm, hipStream_t st) {
  if (first)
    hipLaunchKernelGGL((k_km_assign<NT, true>), kg, kb, sm, st, a);
  else
    hipLaunchKernelGGL((k_km_assign<NT, false>), kg, kb, sm, st, a);
}

hipError_t launch_prepare(const Args& a_in, ClusterMode mode, hipStream_t st) {
  Args a = a_in;
  const unsigned BH = (unsigned)a.BH;
  const bool vs = (a.flags & VC_VSMOOTH) != 0;
  const bool kmeans = vs && mode != ClusterMode::Reuse;
  if (kmeans) {
    // k-means chunks for the device the stream runs on (before any launch, so a
    // failure leaves nothing enqueued)
    hipDevice_t dev = 0;
    int cus = 0;
    if (hipStreamGetDevice(st, &dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return hipErrorInvalidDevice;
    a.nkm = km_chunks(a, cus);
  }
  hipLaunchKernelGGL(k_prep_zero, dim3(BH), dim3(128), 0, st, a);
  if (kmeans) {
    hipLaunchKernelGGL(k_vmax, dim3(a.nkc, BH), dim3(256), 0, st, a);
    if (mode == ClusterMode::Warm)
      hipLaunchKernelGGL(k_km_warm, dim3(BH), dim3(128), 0, st, a);
    else
      hipLaunchKernelGGL(k_km_init, dim3(BH), dim3(1024), 0, st, a);
    for (int it = 0; it < a.T; ++it) {
      const dim3 kg(a.nkm, BH), kb(64 * KM_WAVES);
      const size_t sm = km_smem_bytes(a.C);
      const bool first = it == 0;
      if (a.C <= 16)
        launch_assign<1>(a, first, kg, kb, sm, st);
      else if (a.C <= 32)
        launch_assign<2>(a, first, kg, kb, sm, st);
      else if (a.C <= 48)
        launch_assign<3>(a, first, kg, kb, sm, st);
      else
        launch_assign<4>(a, first, kg, kb, sm, st);
      hipLaunchKernelGGL(k_km_update, dim3(a.C, BH), dim3(128), 0, st, a);
    }
    hipLaunchKernelGGL(k_perm_count, dim3(a.nkm, BH), dim3(1024), 0, st, a);
    hipLaunchKernelGGL(k_perm_scatter, dim3(a.nkm, BH), dim3(1024), 0, st, a);
  } else if (!vs) {
    hipLaunchKernelGGL(k_perm_identity, dim3((a.N + 255) / 256, BH), dim3(256), 0, st, a);
  }
  // the K channel sums (needed by the K codes) with the V block statistics
  hipLaunchKernelGGL(k_ksum_v_stats, dim3(a.nkc + a.nblk, BH), dim3(256), 0, st, a);
  if (a.flags & VC_V4)
    hipLaunchKernelGGL(k_v_quant4, dim3(a.nblk, BH), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(k_v_quant, dim3(a.nblk, BH), dim3(128), 0, st, a);
  // the restore operand always, and the repair set with its deltas when there is
  // one (they need the V codes' criterion), beside the Q/K codes
  const unsigned nqr = BH + 2u * (unsigned)a.nblk * BH;
  if (a.flags & VC_SMOOTH_Q)
    hipLaunchKernelGGL(k_qk_quant_rep<true>, dim3(nqr), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_qk_quant_rep<false>, dim3(nqr), dim3(256), 0, st, a);
  if (a.flags & VC_SMOOTH_Q)
    hipLaunchKernelGGL(k_qbias, dim3((a.nblk + 31) / 32, (a.Npad + 255) / 256, BH), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace vc
