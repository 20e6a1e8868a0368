// Fused VC-Attention FP8 forward kernel for gfx950.
//
// Method (noticiai.com.br VC-Attention article, sections "V-Smooth" (Restore) and
// "ExpCast-FP8"; ip73.fr article, section "Le compromis entre vitesse et
// fidelite" (repair)):
//   S_raw = Q8 . K8^T                       FP8 MFMA, fp32 accumulate
//   M     = running row maximum in ExpCast code units, moved once per 128-key
//           block (only when the block maximum exceeds it by more than tau)
//   code  = clamp(rne(fma(S_raw, alpha, 56 + 8k - M)), 0, 126)   -- the E4M3 byte
//           of P written straight from the log-domain score, no exp, no cast
//   l     = l * r + sum(decoded codes),  r = 2^((M_old - M_new)/8)
//   acc   = acc * r + l_block * mu'_block + P8 . V8       (restore + FP8 MFMA)
//   after the loop the repaired tokens add P(final M) . delta (bf16 MFMA), and
//   O = sV * acc / l, written as bf16 to the token's original row.
//
// Layout.  A workgroup of 4 waves owns one 128-row query block; wave w owns rows
// 32w..32w+31 as two 16-row subtiles.  Scores are computed transposed
// (S^T = K8 . Q8^T on v_mfma_f32_16x16x128_f8f6f4) so each lane holds 32 keys of
// one query: key 16t+4g+v of the block in S[t][v], g = lane/16.  Those 32 ExpCast
// bytes are exactly the lane's B operand of O^T = V8^T . P^T because prepare
// stores V8 channel-major with the same key interleave, so P never touches LDS.
// The row sum of the block comes from one more MFMA against a ones row.
#include "vc_internal.h"

namespace vc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c) {
  // unscaled FP8 (E4M3) x FP8 (E4M3) -> fp32, 16x16x128
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32 bytes of row `row` of a 128x128 byte tile, 16-byte chunks 2g and 2g+1,
// stored with the chunk index XOR-swizzled by row%8 (LDS bank spreading).
__device__ __forceinline__ v8i lds_row32(const uint8_t* tile, int row, int g) {
  const int sw = row & 7;
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * 128 + (((2 * g) ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * 128 + (((2 * g + 1) ^ sw) << 4));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
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

// Workgroup id -> (head, query block), so that consecutive logical tiles (same
// head, sharing its K/V codes in L2) land on the same XCD: the dispatcher deals
// workgroups round-robin over the 8 XCDs.
__device__ __forceinline__ int xcd_remap(int lin, int total) {
  const int q = total / 8, r = total % 8;
  const int x = lin % 8, i = lin / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

__global__ __launch_bounds__(256) void k_fwd(Args a) {
  __shared__ __align__(16) uint8_t Ks[BLK * D];
  __shared__ __align__(16) uint8_t Vs[D * BLK];
  __shared__ float mup_s[D];
  __shared__ float alpha_s[BLK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.nblk, qb = logical % a.nblk;

  const uint8_t* q8 = a.q8 + ((size_t)bh * a.Npad + (size_t)qb * BLK) * D;
  const uint8_t* k8 = a.k8 + (size_t)bh * a.Npad * D;
  const uint8_t* v8t = a.v8t + (size_t)bh * D * a.Npad;
  const float* sk = a.sk + (size_t)bh * a.nblk;
  const float* mup = a.mup + (size_t)bh * a.nblk * D;
  const float sQa = a.sq[(size_t)bh * a.nblk + qb];

  v8i qop[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
    qop[qs] = *reinterpret_cast<const v8i*>(q8 + (size_t)(w * 32 + qs * 16 + l16) * D + 32 * g);

  // ones in rows 0, 4, 8, 12: every lane receives its query's block row sum in
  // accumulator element 0 of the ones MFMA
  v8i ones;
  {
    const int o = (l16 & 3) == 0 ? 0x38383838 : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = o;
  }
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};

  float M[2] = {-INFINITY, -INFINITY}, ell[2] = {0.0f, 0.0f};
  v4f acc[2][8];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[qs][ct] = zero;

  for (int kb = 0; kb < a.nblk; ++kb) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 3, cc = ch & 7;
      const uint4 kv = *reinterpret_cast<const uint4*>(k8 + ((size_t)kb * BLK + row) * D + cc * 16);
      *reinterpret_cast<uint4*>(Ks + row * D + ((cc ^ (row & 7)) << 4)) = kv;
      const uint4 vv = *reinterpret_cast<const uint4*>(v8t + (size_t)row * a.Npad + (size_t)kb * BLK + cc * 16);
      *reinterpret_cast<uint4*>(Vs + row * BLK + ((cc ^ (row & 7)) << 4)) = vv;
    }
    if (tid < D) mup_s[tid] = mup[(size_t)kb * D + tid];
    __syncthreads();

    const float alpha = (sQa * sk[kb]) * a.c0;
    const int nvalid = min(BLK, a.N - kb * BLK);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      v4f S[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = mfma_f8(lds_row32(Ks, 16 * t + l16, g), qop[qs], zero);
      if (nvalid < BLK) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (16 * t + 4 * g + v >= nvalid) S[t][v] = -INFINITY;
      }
      float mx = S[0][0];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, S[t][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float tmax = mx * alpha;
      const float Mo = M[qs];
      const float Mn = (Mo == -INFINITY || tmax - Mo > a.tau) ? tmax : Mo;
      const float beta = a.bias - Mn;
      const float r = (Mo == -INFINITY) ? 0.0f : exp2f((Mo - Mn) * 0.125f);
      v8i pop;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint32_t dw = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) dw |= expcast_byte(S[t][v], alpha, beta) << (8 * v);
        pop[t] = (int)dw;
      }
      const float lb = mfma_f8(ones, pop, zero)[0];
      if (r != 1.0f) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[qs][ct] *= r;
      }
      ell[qs] = ell[qs] * r + lb;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[qs][ct][v] += lb * mup_s[16 * ct + 4 * g + v];
        acc[qs][ct] = mfma_f8(lds_row32(Vs, 16 * ct + l16, g), pop, acc[qs][ct]);
      }
      M[qs] = Mn;
    }
  }

  // Repair: the selected tokens' residual error, weighted by codes formed with
  // the final row maximum and each token's own K block scale; l is unchanged.
  for (int grp = 0; grp < a.mpad / BLK; ++grp) {
    __syncthreads();
    const int* rp = a.rep_pos + (size_t)bh * a.mpad + (size_t)grp * BLK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 3, cc = ch & 7;
      const int pos = rp[row];
      const uint4 kv = *reinterpret_cast<const uint4*>(k8 + (size_t)(pos < 0 ? 0 : pos) * D + cc * 16);
      *reinterpret_cast<uint4*>(Ks + row * D + ((cc ^ (row & 7)) << 4)) = kv;
    }
    if (tid < BLK) {
      const int pos = rp[tid];
      alpha_s[tid] = (sQa * sk[pos < 0 ? 0 : pos / BLK]) * a.c0;
    }
    __syncthreads();
    const uint16_t* dt = a.rep_dt + (size_t)bh * D * a.mpad + (size_t)grp * BLK;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      v4f S[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = mfma_f8(lds_row32(Ks, 16 * t + l16, g), qop[qs], zero);
      const float beta = a.bias - M[qs];
      uint16_t pb[8][4];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t code = expcast_byte(S[t][v], alpha_s[16 * t + 4 * g + v], beta);
          // E4M3 values are exact in bf16
          pb[t][v] = f2bf_rne(__builtin_amdgcn_cvt_f32_fp8((int)code, 0));
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v8bf bop;
#pragma unroll
        for (int i = 0; i < 8; ++i) bop[i] = __builtin_bit_cast(__bf16, pb[2 * u + (i >> 2)][i & 3]);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const uint4 av = *reinterpret_cast<const uint4*>(dt + (size_t)(16 * ct + l16) * a.mpad + 32 * u + 8 * g);
          const v8bf aop = __builtin_bit_cast(v8bf, av);
          acc[qs][ct] = mfma_bf16(aop, bop, acc[qs][ct]);
        }
      }
    }
  }

  // Epilogue: O = sV * acc / l, bf16, scattered back to the original row.
  const float* sv = a.sv + (size_t)bh * D;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int p = qb * BLK + w * 32 + qs * 16 + l16;
    if (p < a.N) {
      const int orig = (a.flags & VC_PERMUTE_Q) ? a.perm[(size_t)bh * a.N + p] : p;
      const float il = 1.0f / ell[qs];
      uint16_t* orow = a.o + ((size_t)bh * a.N + orig) * D;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int c = 16 * ct + 4 * g;
        uint2 pk;
        pk.x = (uint32_t)f2bf_rne(sv[c] * acc[qs][ct][0] * il) |
               ((uint32_t)f2bf_rne(sv[c + 1] * acc[qs][ct][1] * il) << 16);
        pk.y = (uint32_t)f2bf_rne(sv[c + 2] * acc[qs][ct][2] * il) |
               ((uint32_t)f2bf_rne(sv[c + 3] * acc[qs][ct][3] * il) << 16);
        *reinterpret_cast<uint2*>(orow + c) = pk;
      }
    }
  }
}

}  // namespace

hipError_t launch_forward(const Args& a, hipStream_t st) {
  const unsigned tiles = (unsigned)a.BH * (unsigned)a.nblk;
  hipLaunchKernelGGL(k_fwd, dim3(tiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace vc
