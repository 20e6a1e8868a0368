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

// With the 4-bit residual, row r of a block's K code tile holds the key at block
// position v4_krow(r): bits 2-3 and 4-5 of r swapped (the map is its own
// inverse).  The score MFMA's row r = 16t + 4g + v then lands in the P operand
// at the K index of that position, so the FP4 operand's 32-wide scale groups
// are 32 consecutive positions and its codes are stored in position order.
__host__ __device__ constexpr int v4_krow(int r) { return (r & 0x43) | ((r >> 2) & 0x0c) | ((r << 2) & 0x30); }

// An empty asm that reads and writes loaded words, so that the load that made
// them is complete here and cannot be moved past this point.  The compiler
// otherwise moves a load whose value only feeds a select (row in range ? value
// : 0) under a per-row branch, and each such branch then waits for its load
// before the next one is issued; it may also delay a prefetch until just before
// its use.  With the values pinned, a thread issues all of a batch's loads first.
__device__ __forceinline__ void pin_loaded(uint4& x) { asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w)); }
__device__ __forceinline__ void pin_loaded(int& x) { asm volatile("" : "+v"(x)); }
constexpr uint32_t MAGIC = 0x56434154u;  // "VCAT"

// Shape derived from the public parameters.
struct Shape {
  // nkm: the fewest k-means chunks per head (chunks of at most KM_CHUNK tokens);
  // the workspace holds partial sums for up to 4 * nkm
  int B, H, N, BH, nblk, Npad, C, T, m, mpad, nkc, nkm, nch16;
  bool v4;  // 4-bit value residual (VC_V4)
  bool smooth_q;  // query smoothing (VC_SMOOTH_Q)
  bool exact;  // scores as the exact dot product (bf16 MFMA) rather than the FP8 MFMA
};

// Score mode of a parameter set: VC_EXACT_SCORES, VC_FP8_SCORES, or by N.
bool exact_scores(const vc_attn_params* p);

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
  uint32_t flags;  // public flags with the score mode resolved into VC_EXACT_SCORES
  uint64_t seed;
  float c0;    // 8*log2(e)*softmax scale, fp32
  float bias;  // 56 + 8k
  float tau;
  Header* header;
  float* kbar;
  long long* ksum;
  int* init_idx;
  float* cent;
  int* kmpart;        // [BH][nkm][C][128] change of the member sums (fixed point) in one
                      // Lloyd iteration, per assignment workgroup (prepare sets nkm
                      // for the device, between the shape's nkm and four times that)
  int* kmcnt;         // [BH][nkm][C] change of the member counts, likewise
  long long* kmsum;   // [BH][C][128] member sums of the current labels (fixed point)
  long long* kmn;     // [BH][C] member counts of the current labels
  long long* ktot;    // [BH][128] fixed-point channel sums of K (atomic adds of the chunks)
  unsigned* vmaxh;    // [BH] max |V| of the head as fp32 bits (atomic max; values >= 0)
  unsigned* vamax;    // [BH][128] max over blocks of |V - mu| per channel, fp32 bits
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
  size_t kmpart, kmcnt, kmsum, kmn, ktot, vmaxh, vamax, kmsh, uhi, ulo, centfix, kmcc;
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
