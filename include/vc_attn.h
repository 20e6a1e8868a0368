/*
 * vc_attn.h -- C ABI of the VC-Attention FP8 library for AMD Instinct MI355X (gfx950).
 *
 * VC-Attention is training-free low-bit non-causal self-attention for image and
 * video diffusion transformers.  It is described by the articles
 *   "VC-Attention acelera atencao em modelos de video de IA em ate 3,58x sem
 *    retreinamento" (noticiai.com.br), sections "V-Smooth: corrigindo outliers de
 *    valor" (Group / Demean / Restore) and "ExpCast-FP8: eliminando o gargalo do
 *    softmax" (an E4M3 byte read as an integer is about 8*log2(v)+56, written by
 *    one fused multiply-add from the log-domain score), and
 *   "VC-Attention et FLUX 3 accelerent la generation d'images sur Blackwell"
 *    (ip73.fr), introduction (block scales are fixed by the block maximum) and
 *    section "Le compromis entre vitesse et fidelite" (repair budget rho: the
 *    fraction of tokens with the largest quantisation error gets its residual
 *    corrected; rho = 0.005).
 *
 * The work is split in two calls on the caller's HIP stream:
 *   vc_attn_prepare  K smoothing and per-block Q/K E4M3 codes; V-Smooth (k-means
 *                    over value tokens per (batch, head), joint permutation,
 *                    128-token block demeaning, per-channel E4M3 residual codes);
 *                    selection of the repaired tokens.
 *   vc_attn_forward  one fused kernel: QK^T on FP8 MFMA, online row maximum and
 *                    row sum, ExpCast P bytes, PV on FP8 MFMA, restore of the
 *                    block means through the row sum, repair of the selected
 *                    tokens, normalisation and un-permutation of the output.
 *
 * Tensors.  Q, K, V are bf16, contiguous [B][H][N][d] with d = 128, device memory,
 * 16-byte aligned.  O is bf16 [B][H][N][d] in the ORIGINAL token order.
 *
 * Ownership.  The caller allocates Q, K, V, O and the workspace on the device and
 * keeps them alive until the stream has finished the calls.  The library never
 * allocates or frees device memory and never synchronises the stream, except
 * vc_attn_prepare with VC_REUSE_CLUSTERS or VC_WARM_START, which reads 64 bytes
 * of the workspace header back to the host (one stream synchronisation) to check
 * that clusters exist for the same shape.  The library has no global mutable state; calls on
 * different streams with different workspaces may run concurrently.  Two calls
 * that share a workspace must be ordered by the caller.
 *
 * Errors.  Every entry point checks its arguments before touching the device and
 * returns a vc_status; nothing is launched when the status is not VC_OK.  A HIP
 * launch failure returns VC_ERR_HIP (work launched earlier in the same call may
 * have run).  Inputs must be finite with |x| < 2^22 (the fixed-point means are
 * exact under that bound); this is not checked.
 */
#ifndef VC_ATTN_H
#define VC_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VC_OK = 0,
  VC_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, out-of-range parameter */
  VC_ERR_UNSUPPORTED = 2,  /* d != 128, block != 128, or VC_SMOOTH_Q with N above
                              VC_SMOOTH_Q_MAX_TOKENS */
  VC_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than required */
  VC_ERR_NOT_PREPARED = 4, /* VC_REUSE_CLUSTERS / VC_WARM_START without clusters
                              for this shape */
  VC_ERR_HIP = 5,          /* a HIP runtime call or launch failed */
  VC_ERR_INTERNAL = 6
} vc_status;

/* Flags (vc_attn_params.flags). */
enum {
  VC_VSMOOTH = 1u,       /* V-Smooth: cluster, permute, demean (else identity, no mean) */
  VC_REPAIR = 2u,        /* correct the ceil(rho*N) worst-quantised value tokens */
  VC_PERMUTE_Q = 4u,     /* queries follow the cluster permutation too (output is
                            scattered back to original order either way) */
  VC_REUSE_CLUSTERS = 8u, /* prepare skips k-means and reuses labels/permutation
                            already in the workspace (clustering runs only in the
                            early denoising steps, as the V-Smooth section says) */
  VC_WARM_START = 32u,   /* k-means starts from the centroids a previous prepare of
                            the same shape left in the workspace (a denoising step
                            close to the last one) instead of the seeded Forgy
                            draw; each is rescaled to the current fixed-point
                            exponent, rounded and clamped to 14 bits.  Needs
                            VC_VSMOOTH, excludes VC_REUSE_CLUSTERS; without
                            clusters of this shape prepare returns
                            VC_ERR_NOT_PREPARED */
  VC_EXACT_SCORES = 16u, /* QK^T as the exact dot product of the E4M3 codes: the
                            codes multiplied as bf16 (exact) on the bf16 MFMA, twice
                            the matrix-core time of the FP8 MFMA.  The article's
                            bottleneck section runs QK^T on FP8 tensor cores; their
                            accumulation is not exact (gfx950's FP8 MFMA drops the
                            low bits of products far below the largest one of each
                            8-channel group), so about 2 ExpCast codes in 10^4 land
                            one step away from the exact score's code.  One such
                            step moves O by at most 1/8 of that key's share of the
                            row sum times |V|, which for rows spread over fewer
                            than a few thousand keys can exceed 1e-2.  Set the
                            same score flag on prepare and forward */
  VC_FP8_SCORES = 256u,  /* QK^T on the FP8 MFMA whatever N is.  Without either
                            score flag the library takes FP8 scores when N >=
                            VC_FP8_SCORES_MIN_TOKENS and exact scores below;
                            setting both flags is VC_ERR_INVALID_ARG */
  VC_V4 = 64u,           /* 4-bit value residual: the article's V-Smooth section
                            offers NVFP4 instead of per-channel E4M3 for the demeaned
                            residual; here it takes the OCP MX form gfx950's scaled
                            MFMA reads.  Each 128-key block splits into four
                            groups of 32 consecutive positions (key k in group
                            k/32, the MX block of 32 elements); every
                            (block, group, channel) gets the power of two 2^X with
                            X = floor(log2 max|r|) - 2, kept in [-126, 127] (a
                            normal fp32 scale; -126 for an all-zero group), and
                            the residual r = V - mu is coded in E2M1 (round to
                            nearest, ties to the even code, saturating at 6, no
                            negative zero).  No per-channel scale (sv = inv = 1),
                            repair deltas in real units, P stays ExpCast E4M3.  Set
                            the same flag on prepare and forward */
  VC_SMOOTH_Q = 128u,    /* query smoothing, the SageAttention2-style smoothing the
                            article's section on the attention bottleneck names:
                            each 128-position query block subtracts its channel
                            mean qbar_b (exact fixed-point mean) before its codes
                            are formed, and the dropped part returns as a per-key
                            score term d_bj = fp32(c0 * delta_bj), delta_bj =
                            qbar_b . (k_j - kbar) as an fp32 fma chain over
                            channels 0..127, c0 = 8 log2(e) * softmax scale.  A
                            score is t = fma(S_raw, alpha, d_bj) in code units, the
                            block maximum is taken over t and code = clamp(rne(t +
                            56 + 8k - M), 0, 126).  Costs a prepare pass over
                            nblk x N scores and one more VALU operation per score
                            in the forward; the score terms take nblk * Npad * 4
                            bytes of workspace per (batch, head), so the flag is
                            VC_ERR_UNSUPPORTED above N = VC_SMOOTH_Q_MAX_TOKENS
                            (512 MiB per head there).  Set the same flag on
                            prepare and forward */
};

/* Token count from which the default score mode is the FP8 MFMA. */
#define VC_FP8_SCORES_MIN_TOKENS 4096
/* Largest N accepted with VC_SMOOTH_Q. */
#define VC_SMOOTH_Q_MAX_TOKENS 131072

typedef struct {
  int32_t B, H, N;       /* batch, heads, tokens; B*H >= 1, 1 <= N <= 2^20 */
  int32_t d;             /* head dimension, must be 128 */
  int32_t block;         /* quantisation block in tokens, must be 128 */
  int32_t n_clusters;    /* k-means clusters C, 1 <= C <= min(N, 64) */
  int32_t kmeans_iters;  /* Lloyd iterations T, 1 <= T <= 1000 */
  int32_t expcast_k;     /* ExpCast bias is 56 + 8k, 0 <= k <= 8 */
  uint64_t seed;         /* k-means initialisation seed */
  float rho;             /* repair budget, 0 <= rho <= 1 */
  float sm_scale;        /* softmax scale; <= 0 means 1/sqrt(d) */
  float tau;             /* row-maximum slack in code units: the maximum moves only
                            when a block maximum exceeds it by more than tau;
                            0 <= tau and 56 + 8k + tau <= 126 */
  uint32_t flags;        /* VC_* flags */
} vc_attn_params;

/* Byte offsets (from the workspace base) of the arrays prepare writes.  Each is
 * 256-byte aligned.  nblk = ceil(N/128), Npad = 128*nblk, BH = B*H,
 * m = ceil(rho*N) (0 without VC_REPAIR), mpad = 128*ceil(m/128). */
typedef struct {
  size_t total;      /* workspace bytes required                                 */
  size_t header;     /* 256 B: magic, shape, state                               */
  size_t kbar;       /* f32 [BH][128] channel mean of K                          */
  size_t ksum;       /* i64 [BH][nkc][128] fixed-point partial sums of K         */
  size_t init_idx;   /* i32 [BH][C] k-means initial token indices                */
  size_t centroids;  /* f32 [BH][C][128]                                         */
  size_t labels;     /* i32 [BH][N] cluster of each original token               */
  size_t perm;       /* i32 [BH][N] position -> original token                   */
  size_t iperm;      /* i32 [BH][N] original token -> position                   */
  size_t q8;         /* u8  [BH][Npad][128] Q codes, position order               */
  size_t k8;         /* u8  [BH][Npad][128] smoothed-K codes, position order; with
                        VC_V4 row r of a block holds the key at block position
                        r with bits 2-3 and 4-5 swapped                          */
  size_t k16;        /* bf16 [BH][Npad][128] the same codes decoded (exact in bf16),
                        operand of the exact score MFMA; 0 bytes unless the
                        scores are exact (VC_EXACT_SCORES, or neither score flag
                        and N < VC_FP8_SCORES_MIN_TOKENS)                        */
  size_t sq;         /* f32 [BH][nblk] Q block scales                            */
  size_t sk;         /* f32 [BH][nblk] K block scales                            */
  size_t mu;         /* f32 [BH][nblk][128] V block means (real units)           */
  size_t bamax;      /* f32 [BH][nblk][128] block maxima of |V - mu|             */
  size_t mup;        /* f32 [BH][nblk][128] block means in V code units          */
  size_t mupt;       /* bf16 [BH][ceil(nblk/16)][2][128][16] the same means split
                        into a high and a low bf16 part, 16 blocks per group,
                        channel-major (operand of the restore MFMA)              */
  size_t sv;         /* f32 [BH][128] per-channel V residual scale               */
  size_t inv;        /* f32 [BH][128] its inverse                                */
  size_t v8t;        /* u8  [BH][128][Npad] residual codes, channel-major; inside
                        each 128-key block key 16t+4g+v sits at column 32g+4t+v.
                        Not allocated (0 bytes) with VC_V4                       */
  size_t err;        /* f32 [BH][N] repair criterion per position                */
  size_t rep_pos;    /* i32 [BH][mpad] repaired positions ascending, padded with -1 */
  size_t rep_dt;     /* bf16 [BH][128][mpad] residual error of the repaired tokens
                        in V code units, channel-major; inside each 128-slot group
                        slot 32u+16t'+4g+v sits at column 32u+8g+4t'+v; with
                        VC_V4 in real units                                      */
  size_t v4t;        /* VC_V4 only (else 0 bytes): u8 [BH][nblk][128][64] E2M1
                        residual codes, one 8 KB tile per block, channel-major,
                        two codes per byte in position order: key k of the block
                        sits in byte k/2, low nibble for even k                  */
  size_t v4s;        /* VC_V4 only (else 0 bytes): u8 [BH*nblk + 1][4][16][8]
                        E8M0 exponents X + 127: record [(b*H+h)*nblk + block]
                        holds group G, channel 16j + i at byte [G][i][j]; the
                        last record is padding                                   */
  size_t qbar;       /* VC_SMOOTH_Q only (else 0 bytes): f32 [BH][nblk][128] query
                        block means, blocks in processing order                 */
  size_t qbias;      /* VC_SMOOTH_Q only (else 0 bytes): f32 [BH][nblk][Npad] score
                        term d of query block b and key position j (0 past N)    */
} vc_attn_ws_layout;

/* Fill *p with the defaults: d = block = 128, C = 16, T = 10, k = 8, seed 0,
 * rho = 0.005, sm_scale 0 (1/sqrt(d)), tau = 0, flags VSMOOTH|REPAIR|PERMUTE_Q.
 * B, H, N are set to 0 and must be filled in. */
void vc_attn_default_params(vc_attn_params* p);

/* Required workspace size in bytes, or 0 when the parameters are invalid. */
size_t vc_attn_workspace_size(const vc_attn_params* p);

/* Workspace layout for these parameters (host only, no device access). */
vc_status vc_attn_workspace_layout(const vc_attn_params* p, vc_attn_ws_layout* out);

/* Checks the parameters without touching the device. */
vc_status vc_attn_check_params(const vc_attn_params* p);

/* Prepare stage (see above).  q, k, v: device bf16 [B][H][N][128].  workspace:
 * device buffer of ws_bytes >= vc_attn_workspace_size(p), 256-byte aligned.
 * stream: a hipStream_t (NULL = default stream).  Asynchronous. */
vc_status vc_attn_prepare(const vc_attn_params* p, const void* q, const void* k,
                          const void* v, void* workspace, size_t ws_bytes, void* stream);

/* Forward stage: reads the prepared workspace and writes o (device bf16
 * [B][H][N][128], original token order).  p must equal the parameters of the
 * prepare call that filled the workspace.  Asynchronous. */
vc_status vc_attn_forward(const vc_attn_params* p, const void* workspace, size_t ws_bytes,
                          void* o, void* stream);

/* vc_attn_forward that also writes every ExpCast probability byte of the main
 * loop (the codes of P the article's ExpCast-FP8 section describes), for
 * checking them code by code.  pcodes: device buffer of B*H*Npad*Npad bytes,
 * [b*H+h][query position][key position], both positions in the order the kernel
 * processes them (cluster order when VC_PERMUTE_Q, else original order for the
 * queries; cluster order for the keys).  Keys >= N hold 0; rows >= N are
 * written with the codes of a padding query.  The repaired tokens' final-M
 * codes are not included.  Same errors as vc_attn_forward, plus
 * VC_ERR_INVALID_ARG for a null pcodes.  Asynchronous. */
vc_status vc_attn_forward_pcodes(const vc_attn_params* p, const void* workspace, size_t ws_bytes,
                                 void* o, void* pcodes, void* stream);

/* Size of the static device workspace of vc_attn_run_noalloc (per GPU). */
#define VC_NOALLOC_WORKSPACE_BYTES (256u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): vc_attn_prepare then
 * vc_attn_forward with the workspace in a static device array of
 * VC_NOALLOC_WORKSPACE_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The caller passes only q, k, v (device bf16
 * [B][H][N][128]) and o (device bf16, original token order); the device is the
 * stream's.  Allocates nothing.  Returns VC_ERR_WORKSPACE when
 * vc_attn_workspace_size(p) exceeds VC_NOALLOC_WORKSPACE_BYTES (about six heads
 * of 16544 tokens), otherwise the statuses of prepare and forward.  Every call
 * on one GPU uses that GPU's array, which keeps the last call's contents (so
 * VC_REUSE_CLUSTERS / VC_WARM_START see the previous call's clusters when the
 * shape matches): calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  Asynchronous. */
vc_status vc_attn_run_noalloc(const vc_attn_params* p, const void* q, const void* k,
                              const void* v, void* o, void* stream);

/* Static description of a status code. */
const char* vc_attn_status_string(vc_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t vc_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VC_ATTN_H */
