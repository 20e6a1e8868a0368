// Internal declarations of the VC-Attention FP8 library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "vc_attn.h"

namespace vc {

constexpr int D = 128;              // head dimension
constexpr int BLK = 128;            // quantisation block (tokens)
constexpr int KSUM_CHUNK = 512;     // tokens per partial K-sum workgroup
constexpr int KM_CHUNK = 2048;      // tokens per k-means assignment workgroup
constexpr int MAX_CLUSTERS = 64;    // centroids and bins live in LDS
constexpr int V4_TILE = D * BLK / 2;  // bytes of one block's E2M1 value tile
constexpr int V4_SREC = 512;        // bytes of one block's E8M0 exponents
constexpr uint32_t MAGIC = 0x56434154u;  // "VCAT"

// Shape derived from the public parameters.
struct Shape {
  int B, H, N, BH, nblk, Npad, C, T, m, mpad, nkc, nkm, nch16;
  bool v4;  // 4-bit value residual (VC_V4)
  bool smooth_q;  // query smoothing (VC_SMOOTH_Q)
};

// Workspace header (first 256 bytes of the workspace).
struct Header {
  uint32_t magic;
  uint32_t clustered;  // labels/perm/centroids valid for (B, H, N, C)
  int32_t B, H, N, C;
  uint32_t pad[58];
};

// Everything a kernel needs, passed by value.
struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, H, N, BH, nblk, Npad, C, T, m, mpad, nkc, nkm, nch16;
  uint32_t flags;
  uint64_t seed;
  float c0;    // 8*log2(e)*softmax scale, fp32
  float bias;  // 56 + 8k
  float tau;
  Header* header;
  float* kbar;
  long long* ksum;
  int* init_idx;
  float* cent;
  int* kmpart;        // [BH][nkm][C][128] partial sums of members (fixed point)
  int* kmcnt;         // [BH][nkm][C] member counts
  float* vmaxp;       // [BH][nkc] partial max |V|
  int* kmsh;          // [BH] fixed-point exponent of the head
  int8_t* uhi;        // [BH][N][128] high part (u >> 7) of the fixed-point V
  int8_t* ulo;        // [BH][N][128] low part (u & 127)
  int* centfix;       // [BH][C][128] fixed-point centroids
  long long* kmcc;    // [BH][C] squared norms of the fixed-point centroids
  int* labels;
  int* perm;
  int* iperm;
  uint8_t* q8;
  uint8_t* k8;
  uint16_t* k16;  // [BH][Npad][128] bf16 of the K codes
  float* sq;
  float* sk;
  float* mu;
  float* bamax;
  float* mup;
  uint16_t* mupt;  // [BH][nch16][2][128][16] bf16 hi/lo of mup
  float* sv;
  float* inv;
  uint8_t* v8t;
  uint8_t* v4t;  // [BH][nblk][128][64] E2M1 codes (VC_V4)
  uint8_t* v4s;  // [BH*nblk+1][512] E8M0 group exponents (VC_V4)
  float* qbar;   // [BH][nblk][128] query block means (VC_SMOOTH_Q)
  float* qbias;  // [BH][nblk][Npad] score term of query block b, key j (VC_SMOOTH_Q)
  float* err;
  int* rep_pos;
  uint16_t* rep_dt;
  uint8_t* pcodes;  // optional [BH][Npad][Npad] ExpCast bytes of the main loop
};

// Private extension of the public layout (partial k-means sums).
struct FullLayout {
  vc_attn_ws_layout pub;
  size_t kmpart, kmcnt, vmaxp, kmsh, uhi, ulo, centfix, kmcc;
};

bool shape_of(const vc_attn_params* p, Shape* s);
void layout_of(const Shape& s, FullLayout* out);
Args make_args(const vc_attn_params* p, const Shape& s, const FullLayout& L, void* ws);

// How prepare obtains the clusters: seeded Forgy start, start from the previous
// centroids in the workspace, or the previous labels/permutation unchanged.
enum class ClusterMode { Cold, Warm, Reuse };

hipError_t launch_prepare(const Args& a, ClusterMode mode, hipStream_t st);
hipError_t launch_forward(const Args& a, hipStream_t st);

}  // namespace vc
