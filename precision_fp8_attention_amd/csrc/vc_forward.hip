// Fused VC-Attention FP8 forward kernels for gfx950.
//
// Method (noticiai.com.br VC-Attention article, sections "V-Smooth" (Restore) and
// "ExpCast-FP8"; ip73.fr article, section "Le compromis entre vitesse et
// fidelite" (repair)):
//   S_raw = Q8 . K8^T   E4M3 codes on the FP8 MFMA (or, with VC_EXACT_SCORES,
//           the exact dot product through bf16 MFMA), fp32 result
//   M     = running row maximum in ExpCast code units, moved once per 128-key
//           block (only when the block maximum exceeds it by more than tau)
//   code  = clamp(rne(fma(S_raw, alpha, 56 + 8k - M)), 0, 126)   -- the E4M3 byte
//           of P written straight from the log-domain score, no exp, no cast
//   l     = l * r + sum(decoded codes),  r = 2^((M_old - M_new)/8)
//   acc   = acc * r + l_block * mu'_block + P8 . V8       (restore + FP8 MFMA)
//   after the loop the repaired tokens add P(final M) . delta (bf16 MFMA), and
//   O = sV * acc / l, written as bf16 to the token's original row.
//
// Layout.  A workgroup of 8 waves owns two 128-row query blocks; wave w owns
// rows 32w..32w+31 as two 16-row subtiles.  Scores are computed transposed
// (S^T = K . Q^T) on 16x16 tiles, so each lane holds 32 keys of one query: key
// 16t+4g+v of the block in S[t][v], g = lane/16.  Prepare stores V8 channel-major
// with the key interleave that makes those ExpCast bytes the B operand of
// O^T = V8^T . P^T directly: P never touches LDS.  v_cvt_pk_u8_f32 rounds to
// nearest even, saturates to [0, 255] and inserts the byte, so one fma and one
// convert produce each packed code.
//
// Two kernels share that layout:
//  * k_fwd (FP8 scores, the default): QK^T on v_mfma_f32_16x16x128_f8f6f4, P.V
//    and row sums on v_mfma_scale_f32_32x32x64_f8f6f4 (one permlane16 swap per
//    dword regroups the two subtiles' bytes into the 32-query operand), restore
//    every 32 blocks, four LDS stages, two key blocks per barrier.
//  * k_fwd_exact (VC_EXACT_SCORES): QK^T from bf16 K codes on
//    v_mfma_f32_16x16x32_bf16 (every E4M3 value is exact in bf16, and its fp32
//    accumulation is accurate to the last bits), P.V on 16x16x128, restore every
//    16 blocks, two LDS stages (its K tiles are twice as big).
//
// Scores.  The FP8 score MFMA is not exact: inside each group of 8 consecutive
// channels the products are cut toward zero 13 bits below the group's largest
// exponent sum before the group sums are added, and that is the precision in
// which the ExpCast codes are decided (the CPU simulation follows the same rule).
//
// Row sums and restore.  One more MFMA per block multiplies P by a ones row:
// block b of a restore group puts its ones in A row b % (group size), so the
// group's row sums collect in one accumulator L.  At the end of each group L is
// split into bf16 high and low parts and bf16 MFMAs add sum_b l_b * mu'_b to the
// accumulator: the restore costs no per-element VALU work and no second pass
// over the keys.
//
// K tiles and V tiles are filled by direct global->LDS loads while earlier
// blocks run.
#include "vc_internal.h"

namespace vc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c) {
  // unscaled FP8 (E4M3) x FP8 (E4M3) -> fp32, 16x16x128
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16_k32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16_k16(v4s a, v4s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 32 bytes of row `row` of a 128x128 byte tile, 16-byte chunks 2g and 2g+1,
// stored with the chunk index XOR-swizzled by row_swz(row).
// Chunk swizzle of 128-byte tile rows.  ds_read_b128 on gfx950 reads a wave's
// 64 x 16 bytes in four passes; with x = (row/2) % 8 and its two low bits
// swapped, the lanes of every pass hit 16 distinct 16-byte bank groups for both
// halves of the operand (measured: full LDS rate, where x itself halves it).
__device__ __forceinline__ int row_swz(int row) {
  const int x = (row >> 1) & 7;
  return ((x & 1) << 1) | ((x >> 1) & 1) | (x & 4);
}
__device__ __forceinline__ v8i lds_row32(const uint8_t* tile, int row, int g) {
  const int sw = row_swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * 128 + (((2 * g) ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * 128 + (((2 * g + 1) ^ sw) << 4));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// 8 bf16 (16 bytes) of row `row` of a 128x128 bf16 tile: K positions
// 32kc+8g..32kc+8g+7, i.e. 16-byte chunk 4kc+g, XOR-swizzled by row%16.
__device__ __forceinline__ v8bf lds_k16(const uint8_t* tile, int row, int kc, int g) {
  const uint4 x = *reinterpret_cast<const uint4*>(tile + row * 256 + (((4 * kc + g) ^ (row & 15)) << 4));
  return __builtin_bit_cast(v8bf, x);
}

// S^T tile (16 keys x 16 queries) from bf16 K rows and the query operand.
__device__ __forceinline__ v4f score_tile(const uint8_t* Kt, int row, int g, const v8bf (&qop)[4]) {
  v4f s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) s = mfma_bf16_k32(lds_k16(Kt, row, kc, g), qop[kc], s);
  return s;
}

// S^T tile (16 keys x 16 queries) from E4M3 K rows and the query operand.
__device__ __forceinline__ v4f score_tile8(const uint8_t* Kt, int row, int g, v8i qop) {
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  return mfma_f8(lds_row32(Kt, row, g), qop, z);
}

// 16 bytes per lane from global memory into LDS at lds_dst + 16 * lane (the
// wave's 1 KB region).  Written as inline assembly: with the builtin the compiler
// cannot tell that the next tile does not alias the current one and waits for
// the copy before every LDS read of the block.  The instruction writes no
// registers; the kernel waits for it explicitly (vmcnt(0)) before the barrier
// that publishes the tile.
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t off = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(off) : "memory", "m0");
#else
  (void)src;
  (void)lds_dst;
#endif
}

// Makes the compiler complete the load of x at this point (an empty asm that
// reads it), so that no wait for it lands inside a later loop.
__device__ __forceinline__ void keep_loaded(v8i x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

__device__ __forceinline__ uint32_t expcast_byte(float s, float alpha, float beta) {
  float y = __builtin_rintf(__builtin_fmaf(s, alpha, beta));
  y = fminf(fmaxf(y, 0.0f), 126.0f);
  return (uint32_t)y;
}

__device__ __forceinline__ uint16_t f2bf_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float xmax16(float x) {  // max with lane ^ 16
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xmax32(float x) {  // max with lane ^ 32
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xsum16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xsum32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Workgroup id -> (head, query block), so that consecutive logical tiles (same
// head, sharing its K/V codes in L2) land on the same XCD: the dispatcher deals
// workgroups round-robin over the 8 XCDs.
__device__ __forceinline__ int xcd_remap(int lin, int total) {
  const int q = total / 8, r = total % 8;
  const int x = lin % 8, i = lin / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

struct RowState {
  float M;      // running maximum, code units
  float ell;    // row sum of flushed 16-block groups
  v4f L;        // row sums of the current group (lane (g,q): blocks 4g..4g+3)
  v4f acc[8];   // O^T accumulator: channel 16ct+4g+v, query q
};

// New running maximum of one subtile for one key block (no side effects): the
// block maximum in code units replaces it when it is higher by more than tau.
__device__ __forceinline__ float block_max(const v4f (&S)[8], float Mo, float alpha, float tau) {
  float mx = S[0][0];
#pragma unroll
  for (int t = 0; t < 8; ++t) mx = fmaxf(fmaxf(mx, S[t][0]), fmaxf(fmaxf(S[t][1], S[t][2]), S[t][3]));
  mx = xmax32(xmax16(mx));
  const float tmax = mx * alpha;
  return (Mo == -INFINITY || tmax - Mo > tau) ? tmax : Mo;
}
// ExpCast codes of one subtile when |M| < 2^21: |fma - (bias + tau)| then stays
// below half a code, so the saturating convert needs no upper clamp
__device__ __forceinline__ v8i codes_fast(const v4f (&S)[8], float alpha, float beta) {
  v8i pop;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][0], alpha, beta), 0, d);
    d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][1], alpha, beta), 1, d);
    d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][2], alpha, beta), 2, d);
    d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][3], alpha, beta), 3, d);
    pop[t] = (int)d;
  }
  return pop;
}
// ExpCast codes of one subtile with the full clamp (any M)
__device__ __forceinline__ v8i codes_slow(const v4f (&S)[8], float alpha, float beta) {
  v8i pop;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint32_t d = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) d |= expcast_byte(S[t][v], alpha, beta) << (8 * v);
    pop[t] = (int)d;
  }
  return pop;
}

// Softmax of one 16-query subtile for one key block (16x16 accumulator layout):
// new maximum, rescale of the running state, ExpCast codes packed as the PV B
// operand.
__device__ __forceinline__ v8i softmax_codes(v4f (&S)[8], RowState& st, float alpha, float bias,
                                             float tau) {
  const float Mo = st.M;
  const float Mn = block_max(S, Mo, alpha, tau);
  if (Mn != Mo) {
    const float r = Mo == -INFINITY ? 0.0f : exp2f((Mo - Mn) * 0.125f);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) st.acc[ct] *= r;
    st.L *= r;
    st.ell *= r;
    st.M = Mn;
  }
  const float beta = bias - Mn;
  return fabsf(Mn) < 0x1p21f ? codes_fast(S, alpha, beta) : codes_slow(S, alpha, beta);
}

// Adds sum_b L[b] * mu'[b] of a finished 16-block group (bf16 hi/lo split, three
// products) and moves the group's row sums into ell.
__device__ __forceinline__ void restore_group(RowState& st, const uint16_t* mupt_grp, int l16, int g) {
  const v4f W = st.L;
  float s4 = (W[0] + W[1]) + (W[2] + W[3]);
  s4 = xsum32(xsum16(s4));
  st.ell += s4;
  v4s bh, bl;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint16_t h = f2bf_rne(W[v]);
    bh[v] = (short)h;
    bl[v] = (short)f2bf_rne(W[v] - __uint_as_float((uint32_t)h << 16));
  }
  const uint16_t* hip = mupt_grp;
  const uint16_t* lop = mupt_grp + D * 16;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const int c = 16 * ct + l16;
    const v4s ah = *reinterpret_cast<const v4s*>(hip + c * 16 + 4 * g);
    const v4s al = *reinterpret_cast<const v4s*>(lop + c * 16 + 4 * g);
    v4f x = st.acc[ct];
    x = mfma_bf16_k16(ah, bh, x);
    x = mfma_bf16_k16(ah, bl, x);
    x = mfma_bf16_k16(al, bh, x);
    st.acc[ct] = x;
  }
  st.L = v4f{0.0f, 0.0f, 0.0f, 0.0f};
}

// Exact-score forward (VC_EXACT_SCORES): scores from bf16 K codes on the bf16
// MFMA, P.V and row sums on the 16x16x128 FP8 MFMA, 16-block restore groups.
__global__ __launch_bounds__(512, 1) void k_fwd_exact(Args a) {
  constexpr int KROW = 2 * D;  // bytes per bf16 K row in LDS
  constexpr int NST = 2;       // LDS stages: one block computed while the next lands
  __shared__ __align__(1024) uint8_t ksm[NST][BLK * KROW];   // [stage] K rows
  __shared__ __align__(1024) uint8_t vsm[NST][D * BLK];      // [stage] V^T codes
  __shared__ float alpha_s[2][BLK];

  // block scales are read-only here: constant address space -> scalar loads
  typedef __attribute__((address_space(4))) const float cfloat;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int g = lane >> 4, l16 = lane & 15;
  const int npair = (a.nblk + 1) / 2;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int wg = w >> 2;            // which of the two query blocks
  const int bh = logical / npair, qb = 2 * (logical % npair) + wg;
  const bool active = qb < a.nblk;  // the second block of an odd count is empty
  const int qbv = active ? qb : qb - 1;
  const int wq = w & 3;             // wave within its query block

  const uint8_t* q8 = a.q8 + ((size_t)bh * a.Npad + (size_t)qbv * BLK) * D;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.k16 + (size_t)bh * a.Npad * D);
  const uint8_t* v8t = a.v8t + (size_t)bh * D * a.Npad;
  const cfloat* sk = reinterpret_cast<const cfloat*>(reinterpret_cast<uintptr_t>(a.sk + (size_t)bh * a.nblk));
  const uint16_t* mupt = a.mupt + (size_t)bh * a.nch16 * 2 * D * 16;
  const float sQa = *reinterpret_cast<const cfloat*>(reinterpret_cast<uintptr_t>(a.sq + (size_t)bh * a.nblk + qbv));

  // direct global->LDS loads of one key block: K as 1 KB regions of 4 bf16 rows
  // (32 KB), V^T (16 KB) as 16 regions of 8 rows; a lane lands at byte 16*lane
  // of its region, i.e. in stored chunk lane%16 (K) or lane%8 (V) of its row,
  // which holds the source chunk XOR the row's swizzle
  auto issue = [&](int kb) {
    uint8_t* kd = ksm[kb % NST];
    uint8_t* vd = vsm[kb % NST];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + w;
      const int row = 4 * r + (lane >> 4), cc = (lane & 15) ^ (row & 15);
      dma16(kg + ((size_t)kb * BLK + row) * 256 + cc * 16, kd + r * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * i + w;
      const int row = 8 * r + (lane >> 3), cc = (lane & 7) ^ row_swz(row);
      dma16(v8t + (size_t)row * a.Npad + (size_t)kb * BLK + cc * 16, vd + r * 1024);
    }
  };

  // query operand, lane (g, q): bf16 of the codes, chunk kc holding d = 32kc+8g..+7
  v8bf qop[2][4];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const uint8_t* qrow = q8 + (size_t)(wq * 32 + qs * 16 + l16) * D;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const uint2 b = *reinterpret_cast<const uint2*>(qrow + 32 * kc + 8 * g);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t byte = ((i < 4 ? b.x : b.y) >> (8 * (i & 3))) & 0xffu;
        qop[qs][kc][i] = __builtin_bit_cast(
            __bf16, (uint16_t)(__float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)byte, 0)) >> 16));
      }
    }
  }

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  RowState rs[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    rs[qs].M = -INFINITY;
    rs[qs].ell = 0.0f;
    rs[qs].L = zero;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) rs[qs].acc[ct] = zero;
  }

  // S^T of one key block for both query subtiles
  auto qk = [&](int kb, v4f (&S)[2][8]) {
    const uint8_t* Ks = ksm[kb % NST];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      S[0][t] = zero;
      S[1][t] = zero;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const v8bf kop = lds_k16(Ks, 16 * t + l16, kc, g);
        S[0][t] = mfma_bf16_k32(kop, qop[0][kc], S[0][t]);
        S[1][t] = mfma_bf16_k32(kop, qop[1][kc], S[1][t]);
      }
    }
  };
  // masking, row maximum, rescale and ExpCast codes of one key block
  auto soft = [&](int kb, v4f (&S)[2][8], v8i (&pop)[2]) {
    const float alpha = (sQa * sk[kb]) * a.c0;
    const int nvalid = a.N - kb * BLK;
    if (nvalid < BLK) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (16 * t + 4 * g + v >= nvalid) S[qs][t][v] = -INFINITY;
    }
    pop[0] = softmax_codes(S[0], rs[0], alpha, a.bias, a.tau);
    pop[1] = softmax_codes(S[1], rs[1], alpha, a.bias, a.tau);
    if (a.pcodes) {
      // lane (g, q) holds keys 16t+4g..16t+4g+3 of query row q: one dword each
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        uint8_t* prow = a.pcodes + ((size_t)bh * a.Npad + (size_t)qb * BLK + wq * 32 + qs * 16 + l16) * a.Npad +
                        (size_t)kb * BLK + 4 * g;
        if (active) {
#pragma unroll
          for (int t = 0; t < 8; ++t) *reinterpret_cast<int*>(prow + 16 * t) = pop[qs][t];
        }
      }
    }
  };
  // row sums (ones MFMA), P.V (FP8 MFMA) and the 16-block restore of one block
  auto pv = [&](int kb, const v8i (&pop)[2]) {
    const uint8_t* Vs = vsm[kb % NST];
    // ones in A row kb%16: the block's row sum accumulates in L element v of
    // lane group g where 4g+v = kb%16
    const int onesrow = kb & 15;
    const int o = (l16 == onesrow) ? 0x38383838 : 0;
    v8i onesop;
#pragma unroll
    for (int i = 0; i < 8; ++i) onesop[i] = o;
    rs[0].L = mfma_f8(onesop, pop[0], rs[0].L);
    rs[1].L = mfma_f8(onesop, pop[1], rs[1].L);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const v8i vop = lds_row32(Vs, 16 * ct + l16, g);
      rs[0].acc[ct] = mfma_f8(vop, pop[0], rs[0].acc[ct]);
      rs[1].acc[ct] = mfma_f8(vop, pop[1], rs[1].acc[ct]);
    }
    if (onesrow == 15 || kb + 1 == a.nblk) {
      const uint16_t* grp = mupt + (size_t)(kb >> 4) * 2 * D * 16;
      restore_group(rs[0], grp, l16, g);
      restore_group(rs[1], grp, l16, g);
    }
  };

  // Every wave runs QK(kb), softmax(kb), PV(kb) per key block while the next
  // block lands in the other LDS stage.  (Offsetting half of the waves by half a
  // block, so that one wave per SIMD is on VALU work while the other feeds the
  // matrix core, measured slower on gfx950: VALU and MFMA work of one SIMD barely
  // overlap there, whichever waves issue them.)
  issue(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kb = 0; kb < a.nblk; ++kb) {
    if (kb + 1 < a.nblk) issue(kb + 1);
    v4f S[2][8];
    v8i pop[2];
    qk(kb, S);
    soft(kb, S, pop);
    pv(kb, pop);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // Repair: the selected tokens' residual error, weighted by codes formed with
  // the final row maximum and each token's own K block scale; l is unchanged.
  for (int grp = 0; grp < a.mpad / BLK; ++grp) {
    uint8_t* Ks = ksm[0];
    const int* rp = a.rep_pos + (size_t)bh * a.mpad + (size_t)grp * BLK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 512 * i, row = ch >> 4, cc = ch & 15;
      const int pos = rp[row];
      const uint4 kv = *reinterpret_cast<const uint4*>(kg + (size_t)(pos < 0 ? 0 : pos) * 256 + cc * 16);
      *reinterpret_cast<uint4*>(Ks + row * 256 + ((cc ^ (row & 15)) << 4)) = kv;
    }
    if (tid < BLK) {
      const int pos = rp[tid];
      const float sk_pos = sk[pos < 0 ? 0 : pos / BLK];
      alpha_s[0][tid] = (a.sq[(size_t)bh * a.nblk + 2 * (logical % npair)] * sk_pos) * a.c0;
      const int qb1 = min(2 * (logical % npair) + 1, a.nblk - 1);
      alpha_s[1][tid] = (a.sq[(size_t)bh * a.nblk + qb1] * sk_pos) * a.c0;
    }
    __syncthreads();
    const float* al = alpha_s[w >> 2];
    const uint16_t* dt = a.rep_dt + (size_t)bh * D * a.mpad + (size_t)grp * BLK;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const float beta = a.bias - rs[qs].M;
#pragma unroll 1
      for (int u = 0; u < 4; ++u) {
        // key tiles 2u and 2u+1 feed the 32-key chunk u of the bf16 MFMA: lane
        // group g holds slots 16(2u+t')+4g+v at K positions 8g+4t'+v
        v8bf bop;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          const int t = 2 * u + tp;
          const v4f S = score_tile(Ks, 16 * t + l16, g, qop[qs]);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t code = expcast_byte(S[v], al[16 * t + 4 * g + v], beta);
            // E4M3 values are exact in bf16
            bop[4 * tp + v] = __builtin_bit_cast(__bf16, f2bf_rne(__builtin_amdgcn_cvt_f32_fp8((int)code, 0)));
          }
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const uint4 av = *reinterpret_cast<const uint4*>(dt + (size_t)(16 * ct + l16) * a.mpad + 32 * u + 8 * g);
          rs[qs].acc[ct] = mfma_bf16_k32(__builtin_bit_cast(v8bf, av), bop, rs[qs].acc[ct]);
        }
      }
    }
    __syncthreads();
  }

  // Epilogue: O = sV * acc / l, bf16, scattered back to the original row.
  const float* sv = a.sv + (size_t)bh * D;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int p = qb * BLK + wq * 32 + qs * 16 + l16;
    if (active && p < a.N) {
      const int orig = (a.flags & VC_PERMUTE_Q) ? a.perm[(size_t)bh * a.N + p] : p;
      const float il = 1.0f / rs[qs].ell;
      uint16_t* orow = a.o + ((size_t)bh * a.N + orig) * D;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int c = 16 * ct + 4 * g;
        const float4 s4 = *reinterpret_cast<const float4*>(sv + c);
        uint2 pk;
        pk.x = (uint32_t)f2bf_rne(s4.x * rs[qs].acc[ct][0] * il) |
               ((uint32_t)f2bf_rne(s4.y * rs[qs].acc[ct][1] * il) << 16);
        pk.y = (uint32_t)f2bf_rne(s4.z * rs[qs].acc[ct][2] * il) |
               ((uint32_t)f2bf_rne(s4.w * rs[qs].acc[ct][3] * il) << 16);
        *reinterpret_cast<uint2*>(orow + c) = pk;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// FP8-score forward with P.V on 32x32x64 MFMAs.
//
// Scores, maxima and ExpCast codes come from 16x16x128 score tiles, two 16-query
// subtiles per wave, exactly as in k_fwd_exact but with E4M3 K.  One permlane16
// swap per dword then turns the two subtiles' P bytes into the B operand of the
// 32x32x64 MFMA for all 32 queries of the wave: a lane of row r (16 lanes) keeps
// the keys of its own key class r and takes class r^1 from lane ^ 16, which
// holds the same query.  K position 32h + 4t + v of key chunk c is then key
// 16t + 4(c + 2h) + v, which is what 32-byte column group c + 2h of the stored
// V^T rows holds: the V^T layout is shared with k_fwd_exact.  The 32x32 shape
// halves the MFMA issue count of P.V and leaves more room for VALU work beside
// each (64-cycle) instruction.
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32_f8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma32_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(512, 1) void k_fwd(Args a) {
  __shared__ __align__(1024) uint8_t ksm[4][BLK * D];   // [stage] K codes
  __shared__ __align__(1024) uint8_t vsm[4][D * BLK];   // [stage] V^T codes
  typedef __attribute__((address_space(4))) const float cfloat;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int h = lane >> 5, n = lane & 31;  // 32x32 coordinates: query n, K half h
  const int npair = (a.nblk + 1) / 2;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int wg = w >> 2;
  const int bh = logical / npair, qb = 2 * (logical % npair) + wg;
  const bool active = qb < a.nblk;
  const int qbv = active ? qb : qb - 1;
  const int wq = w & 3;

  const uint8_t* q8 = a.q8 + ((size_t)bh * a.Npad + (size_t)qbv * BLK) * D;
  const uint8_t* kg = a.k8 + (size_t)bh * a.Npad * D;
  const uint8_t* v8t = a.v8t + (size_t)bh * D * a.Npad;
  const cfloat* sk = reinterpret_cast<const cfloat*>(reinterpret_cast<uintptr_t>(a.sk + (size_t)bh * a.nblk));
  const uint16_t* mupt = a.mupt + (size_t)bh * a.nch16 * 2 * D * 16;
  const float sQa = *reinterpret_cast<const cfloat*>(reinterpret_cast<uintptr_t>(a.sq + (size_t)bh * a.nblk + qbv));

  auto issue = [&](int kb) {
    uint8_t* kd = ksm[kb & 3];
    uint8_t* vd = vsm[kb & 3];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * i + w;
      const int row = 8 * r + (lane >> 3), cc = (lane & 7) ^ row_swz(row);
      dma16(kg + ((size_t)kb * BLK + row) * D + cc * 16, kd + r * 1024);
      dma16(v8t + (size_t)row * a.Npad + (size_t)kb * BLK + cc * 16, vd + r * 1024);
    }
  };

  v8i qop[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
    qop[qs] = *reinterpret_cast<const v8i*>(q8 + (size_t)(wq * 32 + qs * 16 + l16) * D + 32 * g);
  keep_loaded(qop[0]);
  keep_loaded(qop[1]);

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  v16f z16;
#pragma unroll
  for (int i = 0; i < 16; ++i) z16[i] = 0.0f;
  float M[2] = {-INFINITY, -INFINITY};  // running maxima of the two subtiles (16x16 layout)
  v16f acc[4], L = z16;                 // O^T (channels 32ct+8j+4h+v, query n), row sums
  float ell = 0.0f;                     // flushed row sum of query n
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = z16;

  // adds sum_b L[b] * mu'[b] of the 32-block group G and moves L into ell
  auto restore = [&](int G) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += L[i];
    ell += xsum32(s);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ch16 = 2 * G + cc;
      if (ch16 < a.nch16) {
        v8bf bh_, bl_;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = L[8 * cc + e];
          const uint16_t hb = f2bf_rne(x);
          bh_[e] = __builtin_bit_cast(__bf16, hb);
          bl_[e] = __builtin_bit_cast(__bf16, f2bf_rne(x - __uint_as_float((uint32_t)hb << 16)));
        }
        const uint16_t* hip = mupt + (size_t)ch16 * 2 * D * 16;
        const uint16_t* lop = hip + D * 16;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int c = 32 * ct + n;
          const uint2 h0 = *reinterpret_cast<const uint2*>(hip + c * 16 + 4 * h);
          const uint2 h1 = *reinterpret_cast<const uint2*>(hip + c * 16 + 8 + 4 * h);
          const uint2 l0 = *reinterpret_cast<const uint2*>(lop + c * 16 + 4 * h);
          const uint2 l1 = *reinterpret_cast<const uint2*>(lop + c * 16 + 8 + 4 * h);
          const v8bf ah = __builtin_bit_cast(v8bf, make_uint4(h0.x, h0.y, h1.x, h1.y));
          const v8bf al = __builtin_bit_cast(v8bf, make_uint4(l0.x, l0.y, l1.x, l1.y));
          v16f x = acc[ct];
          x = mfma32_bf16(ah, bh_, x);
          x = mfma32_bf16(ah, bl_, x);
          x = mfma32_bf16(al, bh_, x);
          acc[ct] = x;
        }
      }
    }
    L = z16;
  };

  auto block = [&](int kb) {
    const uint8_t* Ks = ksm[kb & 3];
    const uint8_t* Vs = vsm[kb & 3];
    const float alpha = (sQa * sk[kb]) * a.c0;
    v4f S[2][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v8i kop = lds_row32(Ks, 16 * t + l16, g);
      S[0][t] = mfma_f8(kop, qop[0], zero);
      S[1][t] = mfma_f8(kop, qop[1], zero);
    }
    const int nvalid = a.N - kb * BLK;
    if (nvalid < BLK) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (16 * t + 4 * g + v >= nvalid) S[qs][t][v] = -INFINITY;
    }
    float Mn[2];
    v8i pop[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      Mn[qs] = block_max(S[qs], M[qs], alpha, a.tau);
      pop[qs] = codes_fast(S[qs], alpha, a.bias - Mn[qs]);
    }
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
      if (!(fabsf(Mn[qs]) < 0x1p21f)) pop[qs] = codes_slow(S[qs], alpha, a.bias - Mn[qs]);
    if (a.pcodes && active) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        uint8_t* prow = a.pcodes + ((size_t)bh * a.Npad + (size_t)qb * BLK + wq * 32 + qs * 16 + l16) * a.Npad +
                        (size_t)kb * BLK + 4 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t) *reinterpret_cast<int*>(prow + 16 * t) = pop[qs][t];
      }
    }
    // rescale the running state of every query whose maximum moved
    const bool ch0 = Mn[0] != M[0], ch1 = Mn[1] != M[1];
    if (__builtin_amdgcn_ballot_w64(ch0 || ch1)) {
      const float r0 = ch0 ? (M[0] == -INFINITY ? 0.0f : exp2f((M[0] - Mn[0]) * 0.125f)) : 1.0f;
      const float r1 = ch1 ? (M[1] == -INFINITY ? 0.0f : exp2f((M[1] - Mn[1]) * 0.125f)) : 1.0f;
      const float r = (g & 1) ? r1 : r0;  // this lane's 32x32 query is 16*(g&1) + l16
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] *= r;
      L *= r;
      ell *= r;
    }
    M[0] = Mn[0];
    M[1] = Mn[1];
    // 16x16 P bytes -> 32x32x64 B operands of the two 64-key chunks
    v8i B0, B1;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const auto sw = __builtin_amdgcn_permlane16_swap((uint32_t)pop[0][t], (uint32_t)pop[1][t], false, false);
      B0[t] = (int)sw[0];
      B1[t] = (int)sw[1];
    }
    const int o = (n == (kb & 31)) ? 0x38383838 : 0;
    v8i onesop;
#pragma unroll
    for (int i = 0; i < 8; ++i) onesop[i] = o;
    L = mfma32_f8(onesop, B0, L);
    L = mfma32_f8(onesop, B1, L);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      acc[ct] = mfma32_f8(lds_row32(Vs, 32 * ct + n, 2 * h), B0, acc[ct]);
      acc[ct] = mfma32_f8(lds_row32(Vs, 32 * ct + n, 1 + 2 * h), B1, acc[ct]);
    }
    if ((kb & 31) == 31 || kb + 1 == a.nblk) restore(kb >> 5);
  };

  issue(0);
  if (a.nblk > 1) issue(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kb = 0; kb < a.nblk; kb += 2) {
    if (kb + 2 < a.nblk) issue(kb + 2);
    if (kb + 3 < a.nblk) issue(kb + 3);
    block(kb);
    if (kb + 1 < a.nblk) block(kb + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // Repair: codes of the selected tokens with the final maxima and each token's
  // own K block scale, times their residual error (bf16, natural slot order).
  // one alpha table per query block: the two blocks have their own Q scale
  float* alpha_s = reinterpret_cast<float*>(ksm[1]) + wg * BLK;
  for (int grp = 0; grp < a.mpad / BLK; ++grp) {
    uint8_t* Ks = ksm[0];
    const int* rp = a.rep_pos + (size_t)bh * a.mpad + (size_t)grp * BLK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int chk = tid + 512 * i, row = chk >> 3, cc = chk & 7;
      const int pos = rp[row];
      const uint4 kv = *reinterpret_cast<const uint4*>(kg + (size_t)(pos < 0 ? 0 : pos) * D + cc * 16);
      *reinterpret_cast<uint4*>(Ks + row * 128 + ((cc ^ row_swz(row)) << 4)) = kv;
    }
    if ((tid & 255) < BLK) {  // waves 0-1 for query block 0, waves 4-5 for block 1
      const int j = tid & 127, pos = rp[j];
      alpha_s[j] = (sQa * a.sk[(size_t)bh * a.nblk + (pos < 0 ? 0 : pos / BLK)]) * a.c0;
    }
    __syncthreads();
    const uint16_t* dt = a.rep_dt + (size_t)bh * D * a.mpad + (size_t)grp * BLK;
#pragma unroll 1
    for (int t = 0; t < 8; ++t) {
      uint32_t bp[2][2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const v4f S = score_tile8(Ks, 16 * t + l16, g, qop[qs]);
        const float beta = a.bias - M[qs];
        uint16_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t code = expcast_byte(S[v], alpha_s[16 * t + 4 * g + v], beta);
          hv[v] = f2bf_rne(__builtin_amdgcn_cvt_f32_fp8((int)code, 0));  // exact in bf16
        }
        bp[qs][0] = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
        bp[qs][1] = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
      }
      const auto s0 = __builtin_amdgcn_permlane16_swap(bp[0][0], bp[1][0], false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(bp[0][1], bp[1][1], false, false);
      const v8bf bop = __builtin_bit_cast(v8bf, make_uint4(s0[0], s1[0], s0[1], s1[1]));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const uint4 av = *reinterpret_cast<const uint4*>(dt + (size_t)(32 * ct + n) * a.mpad + 16 * t + 8 * h);
        acc[ct] = mfma32_bf16(__builtin_bit_cast(v8bf, av), bop, acc[ct]);
      }
    }
    __syncthreads();
  }

  // Epilogue: O = sV * acc / l, bf16, scattered back to the original row.
  const float* sv = a.sv + (size_t)bh * D;
  const int p = qb * BLK + wq * 32 + n;
  if (active && p < a.N) {
    const int orig = (a.flags & VC_PERMUTE_Q) ? a.perm[(size_t)bh * a.N + p] : p;
    const float il = 1.0f / ell;
    uint16_t* orow = a.o + ((size_t)bh * a.N + orig) * D;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 32 * ct + 8 * j + 4 * h;
        const float4 s4 = *reinterpret_cast<const float4*>(sv + c);
        uint2 pk;
        pk.x = (uint32_t)f2bf_rne(s4.x * acc[ct][4 * j + 0] * il) |
               ((uint32_t)f2bf_rne(s4.y * acc[ct][4 * j + 1] * il) << 16);
        pk.y = (uint32_t)f2bf_rne(s4.z * acc[ct][4 * j + 2] * il) |
               ((uint32_t)f2bf_rne(s4.w * acc[ct][4 * j + 3] * il) << 16);
        *reinterpret_cast<uint2*>(orow + c) = pk;
      }
  }
}

}  // namespace

hipError_t launch_forward(const Args& a, hipStream_t st) {
  const unsigned tiles = (unsigned)a.BH * (unsigned)((a.nblk + 1) / 2);
  if (a.flags & VC_EXACT_SCORES)
    hipLaunchKernelGGL(k_fwd_exact, dim3(tiles), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(k_fwd, dim3(tiles), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace vc
