// Fused VC-Attention FP8 forward kernel for gfx950.
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
// Layout.  A workgroup of 8 waves owns two 128-row query blocks (a tile); wave
// w owns rows 32w..32w+31 as two 16-row subtiles.  Such a workgroup fills its
// CU, so tiles run in rounds of one per CU; the tiles past the last whole round
// run in a second launch as one-query-block workgroups of 8 waves with one
// 16-row subtile each, which halves the length of that last round.
//   Scores are computed transposed (S^T = K . Q^T) so each lane holds 32 keys
// of one query: key 16t+4g+v of the block in S[t][v], g = lane/16.  Those 32
// ExpCast bytes are exactly the lane's B operand of O^T = V8^T . P^T on
// v_mfma_f32_16x16x128_f8f6f4, because prepare
// stores V8 channel-major with the same key interleave: P never touches LDS.
// v_cvt_pk_u8_f32 rounds to nearest even, saturates to [0, 255] and inserts the
// byte, so one fma and one convert produce each packed code.
//
// Scores.  By default QK^T runs on v_mfma_f32_16x16x128_f8f6f4 like PV.  Its
// accumulation is not exact: inside each group of 8 consecutive channels the
// products are cut toward zero 13 bits below the group's largest exponent sum
// before the group sums are added, so a score can differ from the exact dot
// product in its last bits, and an ExpCast code whose exact value lies that close
// to a rounding boundary moves by one step.  With VC_EXACT_SCORES the E4M3 codes
// are multiplied as bf16 instead (every E4M3 value is exact in bf16) on
// v_mfma_f32_16x16x32_bf16, whose fp32 accumulation is accurate to the last bits,
// at twice the matrix-core time of the FP8 path; its codes are the exact
// score's.
//
// Row sums and restore.  One more MFMA per block multiplies P by a ones row:
// block b of a 16-block group puts its ones in A row b%16, so the group's row
// sums collect in a 16x16 accumulator L (lane (g, q), element v = block 4g+v).
// Every 16 blocks L is split into bf16 high and low parts and one 16x16x16 bf16
// MFMA group adds sum_b l_b * mu'_b to the accumulator: the restore costs no
// per-element VALU work and no second pass over the keys.
//
// 4-bit residual (VC_V4).  V^T is E2M1 with one E8M0 power of two per channel
// and 32-key group, and PV runs on the same instruction in its scaled form: A
// is the FP4 tile (16 bytes per lane), B the unchanged ExpCast bytes, and each
// lane's scale register carries the exponents of its channel for four channel
// tiles (op_sel picks the byte).  The FP4 operand's lane group G spans K
// indices that P's lanes fill from score rows of two P lane groups, so prepare
// stores each block's K code rows in the order v4_krow: the score row that
// reaches the K index of block position j then holds key j, each scale group is
// 32 consecutive positions, and the FP4 codes sit in position order.  P again
// never touches LDS; the masking of keys past N, the smoothed-query score terms
// and the repair gather follow the row order; the restore and the epilogue
// are unchanged (sV = 1).
//
// K tiles (E4M3 codes, 16 KB; bf16 codes, 32 KB, for exact scores) and V tiles
// (E4M3, 16 KB; E2M1, 8 KB + 512 B of exponents) are staged in LDS and filled
// by direct global->LDS loads while earlier blocks run.
#include "vc_internal.h"

#include <type_traits>

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

// E2M1 (FP4) A x E4M3 B -> fp32, 16x16x128, A scaled by 2^(s - 127) with s the
// byte `sel` of the lane's scale register (one E8M0 exponent per lane, i.e. per
// row and 32-wide K group of A); B unscaled (127).  Only a[0..3] are read.
__device__ __forceinline__ v4f mfma_fp4(v8i a, v8i b, v4f c, int scale, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, scale, 0, 127);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 1, scale, 0, 127);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 2, scale, 0, 127);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 3, scale, 0, 127);
  }
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

// Chunk swizzle of the 64-byte rows of a 4-bit value tile: lane (g, i) reads
// chunk g of row 16ct + i; XOR-ing bit 1 of the chunk with bit 2 of the row puts
// the 16 lanes of every ds_read_b128 pass on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int v4_swz(int row) { return ((row >> 2) & 1) << 1; }

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

// Block position of the key in K tile row 16t + 4g + v, minus v: the row itself,
// or with the 4-bit residual the row under v4_krow (64(t/4) + 16g + 4(t%4)).
template <bool V4>
__device__ __forceinline__ int key_pos4(int t, int g) {
  return V4 ? 64 * (t >> 2) + 16 * g + 4 * (t & 3) : 16 * t + 4 * g;
}

// K tile row of position pos (a repaired token; -1 pads to row 0).
template <bool V4>
__device__ __forceinline__ int krow_of(int pos) {
  if (pos < 0) return 0;
  return V4 ? (pos & ~(BLK - 1)) | v4_krow(pos & (BLK - 1)) : pos;
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

// Softmax of one 16-query subtile for one key block: new maximum, rescale of the
// running state, ExpCast codes packed as the PV B operand.
__device__ __forceinline__ v8i softmax_codes(v4f (&S)[8], RowState& st, float alpha, float bias,
                                             float tau) {
  float mx = S[0][0];
#pragma unroll
  for (int t = 0; t < 8; ++t) mx = fmaxf(fmaxf(mx, S[t][0]), fmaxf(fmaxf(S[t][1], S[t][2]), S[t][3]));
  mx = xmax32(xmax16(mx));
  const float tmax = mx * alpha;
  const float Mo = st.M;
  const bool first = Mo == -INFINITY;
  const float Mn = (first || tmax - Mo > tau) ? tmax : Mo;
  if (Mn != Mo) {
    const float r = first ? 0.0f : exp2f((Mo - Mn) * 0.125f);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) st.acc[ct] *= r;
    st.L *= r;
    st.ell *= r;
    st.M = Mn;
  }
  const float beta = bias - Mn;
  v8i pop;
  if (fabsf(Mn) < 0x1p21f) {
    // |fma - (bias + tau)| stays below half a code: no upper clamp needed
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t d = 0;
      d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][0], alpha, beta), 0, d);
      d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][1], alpha, beta), 1, d);
      d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][2], alpha, beta), 2, d);
      d = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(S[t][3], alpha, beta), 3, d);
      pop[t] = (int)d;
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t d = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) d |= expcast_byte(S[t][v], alpha, beta) << (8 * v);
      pop[t] = (int)d;
    }
  }
  return pop;
}

// Adds sum_b L[b] * mu'[b] of a finished 16-block group (bf16 hi/lo split, three
// products) to every subtile's accumulator and moves the group's row sums into
// ell.  The group's 16 mean operands are the same for all subtiles: they are
// loaded once, together, so the restore waits for one round trip.
template <int NS>
__device__ __forceinline__ void restore_group(RowState (&rs)[NS], const uint16_t* mupt_grp, int l16, int g) {
  const uint16_t* hip = mupt_grp;
  const uint16_t* lop = mupt_grp + D * 16;
  uint2 ah[8], al[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const int c = 16 * ct + l16;
    ah[ct] = *reinterpret_cast<const uint2*>(hip + c * 16 + 4 * g);
    al[ct] = *reinterpret_cast<const uint2*>(lop + c * 16 + 4 * g);
  }
#pragma unroll
  for (int qs = 0; qs < NS; ++qs) {
    RowState& st = rs[qs];
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
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      if (qs == 0) {
        asm volatile("" : "+v"(ah[ct].x), "+v"(ah[ct].y));
        asm volatile("" : "+v"(al[ct].x), "+v"(al[ct].y));
      }
      v4f x = st.acc[ct];
      x = mfma_bf16_k16(__builtin_bit_cast(v4s, ah[ct]), bh, x);
      x = mfma_bf16_k16(__builtin_bit_cast(v4s, ah[ct]), bl, x);
      x = mfma_bf16_k16(__builtin_bit_cast(v4s, al[ct]), bh, x);
      st.acc[ct] = x;
    }
    st.L = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
}

// Query operands of one wave: bf16 codes (exact scores) or E4M3 bytes.
template <bool EXACT, int NS> struct QOp;
template <int NS> struct QOp<true, NS> { v8bf v[NS][4]; };
template <int NS> struct QOp<false, NS> { v8i v[NS]; };

// V operands of one key block read from LDS before its softmax, so that their
// latency hides behind the VALU work and P.V issues without LDS waits: four of
// the eight E4M3 channel tiles (all eight push the kernel past 256 VGPRs and
// spill), or all eight 4-bit tiles (4 VGPRs each) with the exponents.  Not in
// exact-score mode, whose bf16 K operands leave no room for them.
constexpr int VPRE8 = 4;
template <bool V4> struct VPre;
template <> struct VPre<false> { v8i t[VPRE8]; };
template <> struct VPre<true> { uint4 t[8]; uint2 sc; };

template <bool EXACT, bool V4, bool SQ, int NS, int QB>
__global__ __launch_bounds__(64 * (8 * QB / NS), 1) void k_fwd(Args a, int tile0) {
  // NS 16-query subtiles per wave; 8 / NS waves per 128-query block and QB
  // query blocks per workgroup: two (a tile) in the main launch, one in the
  // launch that spreads the last tiles over more CUs
  constexpr int NWV = 8 * QB / NS, NWQ = 8 / NS;
  constexpr int KROW = EXACT ? 2 * D : D;                     // bytes per K row in LDS
  // LDS stages: FP8 mode holds four key blocks (two computed per barrier while
  // the next two land), exact-score mode two (its bf16 K tiles are twice as big)
  constexpr int NST = EXACT ? 2 : 4;
  constexpr int VTILE = V4 ? V4_TILE : D * BLK;              // V^T tile bytes
  constexpr int SREC = V4 ? 1024 : 16;                        // E8M0 exponents (V4)
  __shared__ __align__(1024) uint8_t ksm[NST][BLK * KROW];   // [stage] K rows
  __shared__ __align__(1024) uint8_t vsm[NST][VTILE];        // [stage] V^T codes
  __shared__ __align__(1024) uint8_t ssm[NST][SREC];         // [stage] V exponents
  __shared__ __align__(16) float sbias[SQ ? NST : 1][2][BLK];  // [stage][query block] score terms
  __shared__ float alpha_s[2][BLK];
  __shared__ float dsel_s[SQ ? 2 : 1][BLK];                   // repair: score terms of the slots

  // block scales are read-only here: constant address space -> scalar loads
  typedef __attribute__((address_space(4))) const float cfloat;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int g = lane >> 4, l16 = lane & 15;
  const int npair = (a.nblk + 1) / 2;
  // workgroup -> tile (head, pair of query blocks), or with QB = 1 -> one query
  // block of the tiles from tile0 on
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = QB == 2 ? logical : tile0 + logical / 2;
  const int wg = w / NWQ;           // which of the workgroup's query blocks
  const int bh = tile / npair;
  const int qb0 = 2 * (tile % npair) + (QB == 2 ? 0 : (logical & 1));  // first query block
  const int qb = qb0 + wg;
  const bool active = qb < a.nblk;  // the second block of an odd count is empty
  if (QB == 1 && !active) return;   // uniform over the workgroup, before any barrier
  const int qbv = active ? qb : qb - 1;
  const int wq = w % NWQ;           // wave within its query block

  const uint8_t* q8 = a.q8 + ((size_t)bh * a.Npad + (size_t)qbv * BLK) * D;
  const uint8_t* kg = EXACT ? reinterpret_cast<const uint8_t*>(a.k16 + (size_t)bh * a.Npad * D)
                            : a.k8 + (size_t)bh * a.Npad * D;
  const uint8_t* v8t = a.v8t + (size_t)bh * D * a.Npad;
  const cfloat* sk = reinterpret_cast<const cfloat*>(reinterpret_cast<uintptr_t>(a.sk + (size_t)bh * a.nblk));
  const uint16_t* mupt = a.mupt + (size_t)bh * a.nch16 * 2 * D * 16;
  const float sQa = *reinterpret_cast<const cfloat*>(reinterpret_cast<uintptr_t>(a.sq + (size_t)bh * a.nblk + qbv));

  // direct global->LDS loads of one key block: K as 1 KB regions of 4 bf16 rows
  // (exact scores, 32 KB) or 8 E4M3 rows (16 KB), V^T (16 KB) as 16 regions of 8
  // rows; a lane lands at byte 16*lane of its region, i.e. in stored chunk
  // lane%16 (bf16 K) or lane%8 (E4M3 K, V) of its row, which holds the source
  // chunk XOR the row's swizzle
  auto issue = [&](int kb) {
    uint8_t* kd = ksm[kb % NST];
    uint8_t* vd = vsm[kb % NST];
    if constexpr (EXACT) {
#pragma unroll
      for (int i = 0; i < 32 / NWV; ++i) {
        const int r = NWV * i + w;
        const int row = 4 * r + (lane >> 4), cc = (lane & 15) ^ (row & 15);
        dma16(kg + ((size_t)kb * BLK + row) * 256 + cc * 16, kd + r * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16 / NWV; ++i) {
        const int r = NWV * i + w;
        const int row = 8 * r + (lane >> 3), cc = (lane & 7) ^ row_swz(row);
        dma16(kg + ((size_t)kb * BLK + row) * D + cc * 16, kd + r * 1024);
      }
    }
    if constexpr (V4) {
      // one contiguous 8 KB tile as eight 1 KB regions of 16 rows, region r from
      // wave r mod NWV; wave 0 (8 with more than eight waves) also the block's
      // 512 exponent bytes (its 1 KB copy runs into the next record, which the
      // layout pads at the end)
      const uint8_t* vt = a.v4t + ((size_t)bh * a.nblk + kb) * V4_TILE;
#pragma unroll
      for (int i = 0; i < (8 + NWV - 1) / NWV; ++i) {
        const int r = NWV * i + w;
        if (r < 8) {
          const int row = 16 * r + (lane >> 2), cc = (lane & 3) ^ v4_swz(row);
          dma16(vt + row * (BLK / 2) + cc * 16, vd + r * 1024);
        }
      }
      if (w == (NWV > 8 ? 8 : 0)) dma16(a.v4s + ((size_t)bh * a.nblk + kb) * V4_SREC + 16 * lane, ssm[kb % NST]);
    } else {
#pragma unroll
      for (int i = 0; i < 16 / NWV; ++i) {
        const int r = NWV * i + w;
        const int row = 8 * r + (lane >> 3), cc = (lane & 7) ^ row_swz(row);
        dma16(v8t + (size_t)row * a.Npad + (size_t)kb * BLK + cc * 16, vd + r * 1024);
      }
    }
    if constexpr (SQ) {
      // smoothed queries: the block's 128 score terms of both query blocks
      // (lanes 0-31 the first, 32-63 the second), 1 KB
      if (w == (NWV > 8 ? 9 : 1)) {
        const int qsel = min(qb0 + (QB == 2 ? (lane >> 5) : 0), a.nblk - 1);
        dma16(a.qbias + ((size_t)bh * a.nblk + qsel) * a.Npad + (size_t)kb * BLK + 4 * (lane & 31), sbias[kb % NST]);
      }
    }
  };

  // query operand, lane (g, q) holding d = 32g..32g+31: E4M3 bytes, or (exact
  // scores) bf16 of the codes with chunk kc holding d = 32kc+8g..+7
  QOp<EXACT, NS> qop;
#pragma unroll
  for (int qs = 0; qs < NS; ++qs) {
    const uint8_t* qrow = q8 + (size_t)(wq * 16 * NS + qs * 16 + l16) * D;
    if constexpr (EXACT) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint2 b = *reinterpret_cast<const uint2*>(qrow + 32 * kc + 8 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t byte = ((i < 4 ? b.x : b.y) >> (8 * (i & 3))) & 0xffu;
          qop.v[qs][kc][i] = __builtin_bit_cast(
              __bf16, (uint16_t)(__float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)byte, 0)) >> 16));
        }
      }
    } else {
      qop.v[qs] = *reinterpret_cast<const v8i*>(qrow + 32 * g);
    }
  }

  // complete the query loads here, not inside the key loop
  if constexpr (!EXACT) {
#pragma unroll
    for (int qs = 0; qs < NS; ++qs) keep_loaded(qop.v[qs]);
  }

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  RowState rs[NS];
#pragma unroll
  for (int qs = 0; qs < NS; ++qs) {
    rs[qs].M = -INFINITY;
    rs[qs].ell = 0.0f;
    rs[qs].L = zero;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) rs[qs].acc[ct] = zero;
  }

  // S^T of one key block for the wave's query subtiles
  auto qk = [&](int kb, v4f (&S)[NS][8]) {
    const uint8_t* Ks = ksm[kb % NST];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if constexpr (EXACT) {
#pragma unroll
        for (int qs = 0; qs < NS; ++qs) S[qs][t] = zero;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const v8bf kop = lds_k16(Ks, 16 * t + l16, kc, g);
#pragma unroll
          for (int qs = 0; qs < NS; ++qs) S[qs][t] = mfma_bf16_k32(kop, qop.v[qs][kc], S[qs][t]);
        }
      } else {
        const v8i kop = lds_row32(Ks, 16 * t + l16, g);
#pragma unroll
        for (int qs = 0; qs < NS; ++qs) S[qs][t] = mfma_f8(kop, qop.v[qs], zero);
      }
      if constexpr (SQ) {
        // smoothed queries: scores become t = fma(S, alpha, d) in code units;
        // lane group g holds keys 16t+4g..16t+4g+3
        const float alpha = (sQa * sk[kb]) * a.c0;
        const float4 d4 = *reinterpret_cast<const float4*>(&sbias[kb % NST][wg][key_pos4<V4>(t, g)]);
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int qs = 0; qs < NS; ++qs)
#pragma unroll
          for (int v = 0; v < 4; ++v) S[qs][t][v] = __builtin_fmaf(S[qs][t][v], alpha, dv[v]);
      }
    }
  };
  // masking, row maximum, rescale and ExpCast codes of one key block
  auto soft = [&](int kb, v4f (&S)[NS][8], v8i (&pop)[NS]) {
    const float alpha = (sQa * sk[kb]) * a.c0;
    const int nvalid = a.N - kb * BLK;
    if (nvalid < BLK) {
      // the key of row 16t + 4g + v (position key_pos4 + v) is past N when its
      // g-free part reaches nvalid minus the g part: one register per lane
      // instead of 32 key indices held through the key loop
      const int lim = nvalid - (V4 ? 16 : 4) * g;
#pragma unroll
      for (int qs = 0; qs < NS; ++qs)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (key_pos4<V4>(t, 0) + v >= lim) S[qs][t][v] = -INFINITY;
    }
    // smoothed queries already hold t in code units: fma(t, 1, beta) = t + beta
#pragma unroll
    for (int qs = 0; qs < NS; ++qs) pop[qs] = softmax_codes(S[qs], rs[qs], SQ ? 1.0f : alpha, a.bias, a.tau);
    if (a.pcodes) {
      // lane (g, q) holds the keys of rows 16t+4g..16t+4g+3 of query row q (four
      // consecutive positions from key_pos4): one dword each
#pragma unroll
      for (int qs = 0; qs < NS; ++qs) {
        uint8_t* prow = a.pcodes + ((size_t)bh * a.Npad + (size_t)qb * BLK + wq * 16 * NS + qs * 16 + l16) * a.Npad +
                        (size_t)kb * BLK;
        if (active) {
#pragma unroll
          for (int t = 0; t < 8; ++t) *reinterpret_cast<int*>(prow + key_pos4<V4>(t, g)) = pop[qs][t];
        }
      }
    }
  };
  // row sums (ones MFMA), P.V (FP8 MFMA) and the 16-block restore of one block
  constexpr bool PRE = !EXACT;
  auto read_v = [&](int kb, VPre<V4>& vp) {
    const uint8_t* Vs = vsm[kb % NST];
    if constexpr (!PRE) {
      (void)Vs;
      (void)vp;
    } else if constexpr (V4) {
      // lane (g, i) holds the E8M0 exponents of channel 16ct + i, group g for
      // ct = 0..7: byte ct&3 of dword ct/4
      vp.sc = *reinterpret_cast<const uint2*>(ssm[kb % NST] + 8 * lane);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int row = 16 * ct + l16;
        vp.t[ct] = *reinterpret_cast<const uint4*>(Vs + row * (BLK / 2) + ((g ^ v4_swz(row)) << 4));
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < VPRE8; ++ct) vp.t[ct] = lds_row32(Vs, 16 * ct + l16, g);
    }
  };
  auto pv = [&](int kb, const v8i (&pop)[NS], const VPre<V4>& vp) {
    const uint8_t* Vs = vsm[kb % NST];
    // ones in A row kb%16: the block's row sum accumulates in L element v of
    // lane group g where 4g+v = kb%16
    const int onesrow = kb & 15;
    const int o = (l16 == onesrow) ? 0x38383838 : 0;
    v8i onesop;
#pragma unroll
    for (int i = 0; i < 8; ++i) onesop[i] = o;
#pragma unroll
    for (int qs = 0; qs < NS; ++qs) rs[qs].L = mfma_f8(onesop, pop[qs], rs[qs].L);
    if constexpr (V4) {
      const uint2 sc = PRE ? vp.sc : *reinterpret_cast<const uint2*>(ssm[kb % NST] + 8 * lane);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int row = 16 * ct + l16;
        const uint4 c4 = PRE ? vp.t[ct] : *reinterpret_cast<const uint4*>(Vs + row * (BLK / 2) + ((g ^ v4_swz(row)) << 4));
        v8i vop;
        vop[0] = (int)c4.x; vop[1] = (int)c4.y; vop[2] = (int)c4.z; vop[3] = (int)c4.w;
        vop[4] = 0; vop[5] = 0; vop[6] = 0; vop[7] = 0;
        const int scl = ct < 4 ? (int)sc.x : (int)sc.y;
#pragma unroll
        for (int qs = 0; qs < NS; ++qs) rs[qs].acc[ct] = mfma_fp4(vop, pop[qs], rs[qs].acc[ct], scl, ct & 3);
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const v8i vop = PRE && ct < VPRE8 ? vp.t[ct < VPRE8 ? ct : 0] : lds_row32(Vs, 16 * ct + l16, g);
#pragma unroll
        for (int qs = 0; qs < NS; ++qs) rs[qs].acc[ct] = mfma_f8(vop, pop[qs], rs[qs].acc[ct]);
      }
    }
    if (onesrow == 15 || kb + 1 == a.nblk) {
      const uint16_t* grp = mupt + (size_t)(kb >> 4) * 2 * D * 16;
      restore_group<NS>(rs, grp, l16, g);
    }
  };

  // Every wave runs QK(kb), softmax(kb), PV(kb) per key block while the next
  // blocks land in the other LDS stages.  (Offsetting half of the waves by half a
  // block, so that one wave per SIMD is on VALU work while the other feeds the
  // matrix core, measured slower on gfx950: VALU and MFMA work of one SIMD barely
  // overlap there, whichever waves issue them.)
  if constexpr (NST == 4) {
    // two key blocks per barrier (half the barrier waits of one): blocks kb,
    // kb+1 run while kb+2, kb+3 land
    issue(0);
    if (a.nblk > 1) issue(1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int kb = 0; kb < a.nblk; kb += 2) {
      if (kb + 2 < a.nblk) issue(kb + 2);
      if (kb + 3 < a.nblk) issue(kb + 3);
      {
        v4f S[NS][8];
        v8i pop[NS];
        VPre<V4> vp;
        qk(kb, S);
        read_v(kb, vp);
        soft(kb, S, pop);
        pv(kb, pop, vp);
      }
      if (kb + 1 < a.nblk) {
        v4f S[NS][8];
        v8i pop[NS];
        VPre<V4> vp;
        qk(kb + 1, S);
        read_v(kb + 1, vp);
        soft(kb + 1, S, pop);
        pv(kb + 1, pop, vp);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  } else {
    issue(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int kb = 0; kb < a.nblk; ++kb) {
      if (kb + 1 < a.nblk) issue(kb + 1);
      v4f S[NS][8];
      v8i pop[NS];
      VPre<V4> vp;
      qk(kb, S);
      read_v(kb, vp);
      soft(kb, S, pop);
      pv(kb, pop, vp);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

  // Repair: the selected tokens' residual error, weighted by codes formed with
  // the final row maximum and each token's own K block scale; l is unchanged.
  for (int grp = 0; grp < a.mpad / BLK; ++grp) {
    uint8_t* Ks = ksm[0];
    const int* rp = a.rep_pos + (size_t)bh * a.mpad + (size_t)grp * BLK;
    // The K rows of the group's tokens and their score terms.  The positions
    // are loaded together, then the rows and block scales together: two waits.
    // A K row is 16 chunks of 16 bytes (bf16, exact scores) or 8 (E4M3).
    constexpr int RSH = EXACT ? 4 : 3, NIT = BLK * (EXACT ? 256 : 128) / 16 / (64 * NWV);
    int gpos[NIT];
#pragma unroll
    for (int i = 0; i < NIT; ++i) gpos[i] = rp[(tid + 64 * NWV * i) >> RSH];
    int tpos = rp[tid & (BLK - 1)];  // threads tid < BLK use it
#pragma unroll
    for (int i = 0; i < NIT; ++i) pin_loaded(gpos[i]);
    pin_loaded(tpos);
    uint4 kv[NIT];
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int cc = (tid + 64 * NWV * i) & ((1 << RSH) - 1);
      kv[i] = *reinterpret_cast<const uint4*>(kg + (size_t)krow_of<V4>(gpos[i]) * (16 << RSH) + cc * 16);
    }
    const int qb1 = min(qb0 + 1, a.nblk - 1);
    const size_t tcol = (size_t)(tpos < 0 ? 0 : tpos);
    int skb = __float_as_int(sk[tcol / BLK]);
    int db0 = 0, db1 = 0;
    if constexpr (SQ) {
      db0 = __float_as_int(a.qbias[((size_t)bh * a.nblk + qb0) * a.Npad + tcol]);
      db1 = __float_as_int(a.qbias[((size_t)bh * a.nblk + qb1) * a.Npad + tcol]);
    }
#pragma unroll
    for (int i = 0; i < NIT; ++i) pin_loaded(kv[i]);
    pin_loaded(skb);
    if constexpr (SQ) {
      pin_loaded(db0);
      pin_loaded(db1);
    }
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int ch = tid + 64 * NWV * i, row = ch >> RSH, cc = ch & ((1 << RSH) - 1);
      if constexpr (EXACT)
        *reinterpret_cast<uint4*>(Ks + row * 256 + ((cc ^ (row & 15)) << 4)) = kv[i];
      else
        *reinterpret_cast<uint4*>(Ks + row * 128 + ((cc ^ row_swz(row)) << 4)) = kv[i];
    }
    if (tid < BLK) {
      const float sk_pos = __int_as_float(skb);
      alpha_s[0][tid] = (a.sq[(size_t)bh * a.nblk + qb0] * sk_pos) * a.c0;
      alpha_s[1][tid] = (a.sq[(size_t)bh * a.nblk + qb1] * sk_pos) * a.c0;
      if constexpr (SQ) {
        dsel_s[0][tid] = __int_as_float(db0);
        dsel_s[1][tid] = __int_as_float(db1);
      }
    }
    __syncthreads();
    const float* al = alpha_s[wg];
    const float* dsl = dsel_s[SQ ? wg : 0];
    const uint16_t* dt = a.rep_dt + (size_t)bh * D * a.mpad + (size_t)grp * BLK;
    // the A operands of chunk u (eight channel tiles), shared by the subtiles and
    // loaded together; with FP8 scores the next chunk's are loaded while this one
    // is used (the exact-score kernel has no registers to spare for them)
    auto load_dt = [&](int u, uint4 (&av)[8]) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        av[ct] = *reinterpret_cast<const uint4*>(dt + (size_t)(16 * ct + l16) * a.mpad + 32 * u + 8 * g);
    };
    uint4 avn[8];
    if constexpr (!EXACT) load_dt(0, avn);
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      uint4 av[8];
      if constexpr (EXACT) {
        load_dt(u, av);
      } else {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) av[ct] = avn[ct];
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) pin_loaded(av[ct]);
      if (!EXACT && u < 3) load_dt(u + 1, avn);
#pragma unroll
      for (int qs = 0; qs < NS; ++qs) {
        const float beta = a.bias - rs[qs].M;
        // key tiles 2u and 2u+1 feed the 32-key chunk u of the bf16 MFMA: lane
        // group g holds slots 16(2u+t')+4g+v at K positions 8g+4t'+v
        v8bf bop;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          const int t = 2 * u + tp;
          v4f S;
          if constexpr (EXACT)
            S = score_tile(Ks, 16 * t + l16, g, qop.v[qs]);
          else
            S = score_tile8(Ks, 16 * t + l16, g, qop.v[qs]);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int slot = 16 * t + 4 * g + v;
            const uint32_t code = SQ ? expcast_byte(__builtin_fmaf(S[v], al[slot], dsl[slot]), 1.0f, beta)
                                     : expcast_byte(S[v], al[slot], beta);
            // E4M3 values are exact in bf16
            bop[4 * tp + v] = __builtin_bit_cast(__bf16, f2bf_rne(__builtin_amdgcn_cvt_f32_fp8((int)code, 0)));
          }
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) rs[qs].acc[ct] = mfma_bf16_k32(__builtin_bit_cast(v8bf, av[ct]), bop, rs[qs].acc[ct]);
      }
    }
    __syncthreads();
  }

  // Epilogue: O = sV * acc / l, bf16, scattered back to the original row.  The
  // channel scales are loaded together first: a load after a store would also
  // wait for the store.
  const float* sv = a.sv + (size_t)bh * D;
  uint4 svw[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) svw[ct] = *reinterpret_cast<const uint4*>(sv + 16 * ct + 4 * g);
  int orig[NS];  // each subtile row's original position (rows past N: any valid one)
#pragma unroll
  for (int qs = 0; qs < NS; ++qs) {
    const int p = min(qb * BLK + wq * 16 * NS + qs * 16 + l16, a.N - 1);
    orig[qs] = (a.flags & VC_PERMUTE_Q) ? a.perm[(size_t)bh * a.N + p] : p;
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) pin_loaded(svw[ct]);
#pragma unroll
  for (int qs = 0; qs < NS; ++qs) pin_loaded(orig[qs]);
#pragma unroll
  for (int qs = 0; qs < NS; ++qs) {
    const int p = qb * BLK + wq * 16 * NS + qs * 16 + l16;
    if (active && p < a.N) {
      const float il = 1.0f / rs[qs].ell;
      uint16_t* orow = a.o + ((size_t)bh * a.N + orig[qs]) * D;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int c = 16 * ct + 4 * g;
        const float4 s4 = __builtin_bit_cast(float4, svw[ct]);
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

}  // namespace

// This file is compiled twice.  The plain and 4-bit-residual variants are
// built with the max-ilp machine scheduler, which measured faster for them;
// the smoothed-query and exact-score variants (VC_FWD_DEFAULT_SCHED) with the
// default scheduler, which measured faster for the smoothed-query kernel.
// variant = (exact ? 4 : 0) | (v4 ? 2 : 0) | (sq ? 1 : 0).
#if defined(VC_FWD_DEFAULT_SCHED)
#define VC_FWD_LAUNCH_PART launch_forward_default_sched
#else
#define VC_FWD_LAUNCH_PART launch_forward_ilp_sched
#endif
// two 16-query subtiles per wave (8 waves).  One subtile per wave (16 waves,
// four per SIMD) caps a wave at 128 VGPRs: it spills in the key loop, reads
// every K/V tile twice as often, and measured 8% slower.
constexpr int kSubtiles = 2;

void VC_FWD_LAUNCH_PART(int variant, unsigned full, unsigned rest, const Args& a, hipStream_t st) {
  auto go = [&](auto qb_tag, auto ns_tag, unsigned nwg) {
    constexpr int QB = decltype(qb_tag)::value, S = decltype(ns_tag)::value;
    const dim3 grid(nwg), block(64 * (8 * QB / S));
    const int tile0 = (int)full;
#if defined(VC_FWD_DEFAULT_SCHED)
    switch (variant) {
      case 1: hipLaunchKernelGGL((k_fwd<false, false, true, S, QB>), grid, block, 0, st, a, tile0); break;
      case 3: hipLaunchKernelGGL((k_fwd<false, true, true, S, QB>), grid, block, 0, st, a, tile0); break;
      case 4: hipLaunchKernelGGL((k_fwd<true, false, false, S, QB>), grid, block, 0, st, a, tile0); break;
      case 5: hipLaunchKernelGGL((k_fwd<true, false, true, S, QB>), grid, block, 0, st, a, tile0); break;
      case 6: hipLaunchKernelGGL((k_fwd<true, true, false, S, QB>), grid, block, 0, st, a, tile0); break;
      default: hipLaunchKernelGGL((k_fwd<true, true, true, S, QB>), grid, block, 0, st, a, tile0); break;
    }
#else
    if (variant == 2)
      hipLaunchKernelGGL((k_fwd<false, true, false, S, QB>), grid, block, 0, st, a, tile0);
    else
      hipLaunchKernelGGL((k_fwd<false, false, false, S, QB>), grid, block, 0, st, a, tile0);
#endif
  };
  if (full > 0) go(std::integral_constant<int, 2>{}, std::integral_constant<int, kSubtiles>{}, full);
  if (rest > 0) go(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, 2 * rest);
}

#if !defined(VC_FWD_DEFAULT_SCHED)
void launch_forward_default_sched(int variant, unsigned full, unsigned rest, const Args& a, hipStream_t st);

static bool forward_variant_ilp(int variant) { return variant == 0 || variant == 2; }

hipError_t launch_forward(const Args& a, hipStream_t st) {
  const unsigned tiles = (unsigned)a.BH * (unsigned)((a.nblk + 1) / 2);
  const bool exact = (a.flags & VC_EXACT_SCORES) != 0, v4 = (a.flags & VC_V4) != 0;
  const bool sq = (a.flags & VC_SMOOTH_Q) != 0;
  // A tile workgroup fills its CU (one per CU), so the tiles run in rounds of
  // one per CU.  Whole rounds run as tiles.  The rest run as one-query-block
  // workgroups of 8 waves with one 16-query subtile each: half the work per
  // wave, and a wave's time is set by its own MFMA -> softmax -> MFMA chain
  // more than by the other wave on its SIMD, so the last partial round takes
  // about half as long.  The per-row arithmetic is the same in both shapes.
  // Problems with fewer tiles than half the CUs run entirely in the one-block
  // shape, which spreads them over twice as many CUs.
  hipDevice_t dev = 0;  // the device the stream runs on (the current one for the null stream)
  int cus = 0;
  if (hipStreamGetDevice(st, &dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return hipErrorInvalidDevice;
  unsigned full = tiles / (unsigned)cus * (unsigned)cus;
  unsigned rest = tiles - full;
  // A round of one-block workgroups takes about 0.6 of a tile round (measured at
  // 2x24x16544: 163 against 272 us).  When the rest needs more than one such
  // round, one more round of tiles is shorter (1.0 against 1.2 or more).
  if (2 * rest > (unsigned)cus) {
    full = tiles;
    rest = 0;
  }
  const int variant = (exact ? 4 : 0) | (v4 ? 2 : 0) | (sq ? 1 : 0);
  if (forward_variant_ilp(variant))
    launch_forward_ilp_sched(variant, full, rest, a, st);
  else
    launch_forward_default_sched(variant, full, rest, a, st);
  return hipGetLastError();
}
#endif

}  // namespace vc
