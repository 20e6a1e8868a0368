// Host side of the VC-Attention FP8 C ABI: argument checks, workspace layout,
// and the stream-ordered entry points.  No device allocation; the only global
// state is the static workspace of vc_attn_run_noalloc (per GPU) and the
// per-device addresses of it.
#include <cmath>
#include <cstring>
#include <mutex>

#include "vc_internal.h"

// Workspace of vc_attn_run_noalloc: one copy per GPU, held until the process
// ends.  In host code this name is only a stand-in for the symbol: kernels get
// the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[VC_NOALLOC_WORKSPACE_BYTES];

namespace vc {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int32_t repair_count(const vc_attn_params* p) {
  if (!(p->flags & VC_REPAIR) || !(p->rho > 0.0f)) return 0;
  double m = std::ceil((double)p->rho * (double)p->N);
  if (m > p->N) m = p->N;
  return (int32_t)m;
}

static vc_status check(const vc_attn_params* p) {
  if (!p) return VC_ERR_INVALID_ARG;
  if (p->d != D || p->block != BLK) return VC_ERR_UNSUPPORTED;
  if (p->B < 1 || p->H < 1 || p->N < 1 || p->N > (1 << 20)) return VC_ERR_INVALID_ARG;
  if ((int64_t)p->B * p->H > (1 << 24)) return VC_ERR_INVALID_ARG;
  if (p->n_clusters < 1 || p->n_clusters > MAX_CLUSTERS || p->n_clusters > p->N) return VC_ERR_INVALID_ARG;
  if (p->kmeans_iters < 1 || p->kmeans_iters > 1000) return VC_ERR_INVALID_ARG;
  if (p->expcast_k < 0 || p->expcast_k > 8) return VC_ERR_INVALID_ARG;
  if (!(p->rho >= 0.0f && p->rho <= 1.0f)) return VC_ERR_INVALID_ARG;  // also rejects NaN
  if (!std::isfinite(p->sm_scale)) return VC_ERR_INVALID_ARG;
  if (!(p->tau >= 0.0f) || 56.0f + 8.0f * p->expcast_k + p->tau > 126.0f) return VC_ERR_INVALID_ARG;
  if (p->flags & ~(uint32_t)(VC_VSMOOTH | VC_REPAIR | VC_PERMUTE_Q | VC_REUSE_CLUSTERS |
                         VC_EXACT_SCORES | VC_WARM_START | VC_V4 | VC_SMOOTH_Q | VC_FP8_SCORES))
    return VC_ERR_INVALID_ARG;
  if ((p->flags & VC_EXACT_SCORES) && (p->flags & VC_FP8_SCORES)) return VC_ERR_INVALID_ARG;
  // the smoothed-query score terms are nblk x Npad per head
  if ((p->flags & VC_SMOOTH_Q) && p->N > VC_SMOOTH_Q_MAX_TOKENS) return VC_ERR_UNSUPPORTED;
  if ((p->flags & VC_WARM_START) && (!(p->flags & VC_VSMOOTH) || (p->flags & VC_REUSE_CLUSTERS)))
    return VC_ERR_INVALID_ARG;
  return VC_OK;
}

bool shape_of(const vc_attn_params* p, Shape* s) {
  if (check(p) != VC_OK) return false;
  s->B = p->B;
  s->H = p->H;
  s->N = p->N;
  s->BH = p->B * p->H;
  s->nblk = (p->N + BLK - 1) / BLK;
  s->Npad = s->nblk * BLK;
  s->C = p->n_clusters;
  s->T = p->kmeans_iters;
  s->m = repair_count(p);
  s->mpad = ((s->m + BLK - 1) / BLK) * BLK;
  s->nkc = (p->N + KSUM_CHUNK - 1) / KSUM_CHUNK;
  s->nkm = (p->N + KM_CHUNK - 1) / KM_CHUNK;
  s->nch16 = (s->nblk + 15) / 16;
  s->v4 = (p->flags & VC_V4) != 0;
  s->smooth_q = (p->flags & VC_SMOOTH_Q) != 0;
  s->exact = exact_scores(p);
  return true;
}

bool exact_scores(const vc_attn_params* p) {
  if (p->flags & VC_EXACT_SCORES) return true;
  if (p->flags & VC_FP8_SCORES) return false;
  return p->N < VC_FP8_SCORES_MIN_TOKENS;
}

void layout_of(const Shape& s, FullLayout* out) {
  const size_t BH = (size_t)s.BH, N = (size_t)s.N, Np = (size_t)s.Npad, nb = (size_t)s.nblk;
  const size_t C = (size_t)s.C;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  vc_attn_ws_layout& L = out->pub;
  L.header = take(sizeof(Header));
  L.kbar = take(BH * D * 4);
  L.ksum = take(BH * (size_t)s.nkc * D * 8);
  L.init_idx = take(BH * C * 4);
  L.centroids = take(BH * C * D * 4);
  // prepare may cut a head into up to four times the fewest k-means chunks
  out->kmpart = take(BH * (size_t)(4 * s.nkm) * C * D * 4);
  out->kmcnt = take(BH * (size_t)(4 * s.nkm) * C * 4);
  out->kmsum = take(BH * C * D * 8);
  out->kmn = take(BH * C * 8);
  out->ktot = take(BH * D * 8);
  out->vmaxh = take(BH * 4);
  out->vamax = take(BH * D * 4);
  out->kmsh = take(BH * 4);
  out->uhi = take(BH * N * D);
  out->ulo = take(BH * N * D);
  out->centfix = take(BH * C * D * 4);
  out->kmcc = take(BH * C * 8);
  L.labels = take(BH * N * 4);
  L.perm = take(BH * N * 4);
  L.iperm = take(BH * N * 4);
  L.q8 = take(BH * Np * D);
  L.k8 = take(BH * Np * D);
  L.k16 = take(s.exact ? BH * Np * D * 2 : 0);
  L.sq = take(BH * nb * 4);
  L.sk = take(BH * nb * 4);
  L.mu = take(BH * nb * D * 4);
  L.bamax = take(BH * nb * D * 4);
  L.mup = take(BH * nb * D * 4);
  L.mupt = take(BH * (size_t)s.nch16 * 2 * D * 16 * 2);
  L.sv = take(BH * D * 4);
  L.inv = take(BH * D * 4);
  L.v8t = take(s.v4 ? 0 : BH * D * Np);
  L.err = take(BH * N * 4);
  L.rep_pos = take(BH * (size_t)s.mpad * 4);
  L.rep_dt = take(BH * D * (size_t)s.mpad * 2);
  L.v4t = take(s.v4 ? BH * nb * V4_TILE : 0);
  L.v4s = take(s.v4 ? (BH * nb + 1) * V4_SREC : 0);
  L.qbar = take(s.smooth_q ? BH * nb * D * 4 : 0);
  L.qbias = take(s.smooth_q ? BH * nb * Np * 4 : 0);
  L.total = off;
}

Args make_args(const vc_attn_params* p, const Shape& s, const FullLayout& FL, void* ws) {
  const vc_attn_ws_layout& L = FL.pub;
  uint8_t* b = static_cast<uint8_t*>(ws);
  Args a;
  std::memset(&a, 0, sizeof(a));
  a.B = s.B;
  a.H = s.H;
  a.N = s.N;
  a.BH = s.BH;
  a.nblk = s.nblk;
  a.Npad = s.Npad;
  a.C = s.C;
  a.T = s.T;
  a.m = s.m;
  a.mpad = s.mpad;
  a.nkc = s.nkc;
  a.nkm = s.nkm;
  a.nch16 = s.nch16;
  // the kernels see the score mode resolved: VC_EXACT_SCORES set or clear
  a.flags = (p->flags & ~(uint32_t)(VC_EXACT_SCORES | VC_FP8_SCORES)) | (s.exact ? VC_EXACT_SCORES : 0u);
  a.seed = p->seed;
  const float scale = p->sm_scale > 0.0f ? p->sm_scale : (float)(1.0 / std::sqrt((double)D));
  a.c0 = (float)(8.0 * 1.4426950408889634074 * (double)scale);
  a.bias = (float)(56 + 8 * p->expcast_k);
  a.tau = p->tau;
  a.header = reinterpret_cast<Header*>(b + L.header);
  a.kbar = reinterpret_cast<float*>(b + L.kbar);
  a.ksum = reinterpret_cast<long long*>(b + L.ksum);
  a.init_idx = reinterpret_cast<int*>(b + L.init_idx);
  a.cent = reinterpret_cast<float*>(b + L.centroids);
  a.kmpart = reinterpret_cast<int*>(b + FL.kmpart);
  a.kmcnt = reinterpret_cast<int*>(b + FL.kmcnt);
  a.kmsum = reinterpret_cast<long long*>(b + FL.kmsum);
  a.kmn = reinterpret_cast<long long*>(b + FL.kmn);
  a.ktot = reinterpret_cast<long long*>(b + FL.ktot);
  a.vmaxh = reinterpret_cast<unsigned*>(b + FL.vmaxh);
  a.vamax = reinterpret_cast<unsigned*>(b + FL.vamax);
  a.kmsh = reinterpret_cast<int*>(b + FL.kmsh);
  a.uhi = reinterpret_cast<int8_t*>(b + FL.uhi);
  a.ulo = reinterpret_cast<int8_t*>(b + FL.ulo);
  a.centfix = reinterpret_cast<int*>(b + FL.centfix);
  a.kmcc = reinterpret_cast<long long*>(b + FL.kmcc);
  a.labels = reinterpret_cast<int*>(b + L.labels);
  a.perm = reinterpret_cast<int*>(b + L.perm);
  a.iperm = reinterpret_cast<int*>(b + L.iperm);
  a.q8 = b + L.q8;
  a.k8 = b + L.k8;
  a.k16 = reinterpret_cast<uint16_t*>(b + L.k16);
  a.sq = reinterpret_cast<float*>(b + L.sq);
  a.sk = reinterpret_cast<float*>(b + L.sk);
  a.mu = reinterpret_cast<float*>(b + L.mu);
  a.bamax = reinterpret_cast<float*>(b + L.bamax);
  a.mup = reinterpret_cast<float*>(b + L.mup);
  a.mupt = reinterpret_cast<uint16_t*>(b + L.mupt);
  a.sv = reinterpret_cast<float*>(b + L.sv);
  a.inv = reinterpret_cast<float*>(b + L.inv);
  a.v8t = b + L.v8t;
  a.v4t = b + L.v4t;
  a.v4s = b + L.v4s;
  a.qbar = reinterpret_cast<float*>(b + L.qbar);
  a.qbias = reinterpret_cast<float*>(b + L.qbias);
  a.err = reinterpret_cast<float*>(b + L.err);
  a.rep_pos = reinterpret_cast<int*>(b + L.rep_pos);
  a.rep_dt = reinterpret_cast<uint16_t*>(b + L.rep_dt);
  return a;
}

static bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace vc

using namespace vc;

extern "C" {

void vc_attn_default_params(vc_attn_params* p) {
  if (!p) return;
  std::memset(p, 0, sizeof(*p));
  p->d = D;
  p->block = BLK;
  p->n_clusters = 16;
  p->kmeans_iters = 10;
  p->expcast_k = 8;
  p->seed = 0;
  p->rho = 0.005f;
  p->sm_scale = 0.0f;
  p->tau = 0.0f;
  p->flags = VC_VSMOOTH | VC_REPAIR | VC_PERMUTE_Q;
}

vc_status vc_attn_check_params(const vc_attn_params* p) { return check(p); }

size_t vc_attn_workspace_size(const vc_attn_params* p) {
  Shape s;
  if (!shape_of(p, &s)) return 0;
  FullLayout L;
  layout_of(s, &L);
  return L.pub.total;
}

vc_status vc_attn_workspace_layout(const vc_attn_params* p, vc_attn_ws_layout* out) {
  if (!out) return VC_ERR_INVALID_ARG;
  const vc_status st = check(p);
  if (st != VC_OK) return st;
  Shape s;
  shape_of(p, &s);
  FullLayout L;
  layout_of(s, &L);
  *out = L.pub;
  return VC_OK;
}

vc_status vc_attn_prepare(const vc_attn_params* p, const void* q, const void* k, const void* v,
                          void* workspace, size_t ws_bytes, void* stream) {
  const vc_status st = check(p);
  if (st != VC_OK) return st;
  if (!q || !k || !v || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return VC_ERR_INVALID_ARG;
  Shape s;
  shape_of(p, &s);
  FullLayout L;
  layout_of(s, &L);
  if (!workspace || !aligned(workspace, 256) || ws_bytes < L.pub.total) return VC_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool vs = (p->flags & VC_VSMOOTH) != 0;
  const bool reuse = vs && (p->flags & VC_REUSE_CLUSTERS);
  const bool warm = vs && (p->flags & VC_WARM_START);
  if (reuse || warm) {
    Header h;
    if (hipMemcpyAsync(&h, static_cast<uint8_t*>(workspace) + L.pub.header, sizeof(h),
                       hipMemcpyDeviceToHost, hs) != hipSuccess)
      return VC_ERR_HIP;
    if (hipStreamSynchronize(hs) != hipSuccess) return VC_ERR_HIP;
    if (h.magic != MAGIC || h.clustered != 1u || h.B != p->B || h.H != p->H || h.N != p->N ||
        h.C != p->n_clusters)
      return VC_ERR_NOT_PREPARED;
  }
  Args a = make_args(p, s, L, workspace);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  const ClusterMode mode = reuse ? ClusterMode::Reuse : (warm ? ClusterMode::Warm : ClusterMode::Cold);
  // the launches are checked with hipGetLastError, which also returns an error an
  // earlier runtime call of this thread (the caller's) left behind: drop it first
  (void)hipGetLastError();
  return launch_prepare(a, mode, hs) == hipSuccess ? VC_OK : VC_ERR_HIP;
}

static vc_status forward_impl(const vc_attn_params* p, const void* workspace, size_t ws_bytes,
                              void* o, uint8_t* pcodes, void* stream) {
  const vc_status st = check(p);
  if (st != VC_OK) return st;
  if (!o || !aligned(o, 16)) return VC_ERR_INVALID_ARG;
  Shape s;
  shape_of(p, &s);
  FullLayout L;
  layout_of(s, &L);
  if (!workspace || !aligned(workspace, 256) || ws_bytes < L.pub.total) return VC_ERR_WORKSPACE;
  Args a = make_args(p, s, L, const_cast<void*>(workspace));
  a.o = static_cast<uint16_t*>(o);
  a.pcodes = pcodes;
  (void)hipGetLastError();  // as in prepare: report only this call's launches
  return launch_forward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? VC_OK : VC_ERR_HIP;
}

vc_status vc_attn_forward(const vc_attn_params* p, const void* workspace, size_t ws_bytes, void* o,
                          void* stream) {
  return forward_impl(p, workspace, ws_bytes, o, nullptr, stream);
}

vc_status vc_attn_forward_pcodes(const vc_attn_params* p, const void* workspace, size_t ws_bytes,
                                 void* o, void* pcodes, void* stream) {
  if (!pcodes || !aligned(pcodes, 16)) {
    const vc_status st = check(p);
    return st != VC_OK ? st : VC_ERR_INVALID_ARG;
  }
  return forward_impl(p, workspace, ws_bytes, o, static_cast<uint8_t*>(pcodes), stream);
}

}  // extern "C"

namespace vc {

// Device address of `scratch` on the device the stream runs on, looked up once
// per device with that device current (each GPU holds its own copy of the
// array at its own address).
static vc_status scratch_of(hipStream_t st, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VC_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return VC_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return VC_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return VC_ERR_HIP;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return VC_OK;
}

}  // namespace vc

extern "C" {

vc_status vc_attn_run_noalloc(const vc_attn_params* p, const void* q, const void* k, const void* v,
                              void* o, void* stream) {
  const vc_status st = check(p);
  if (st != VC_OK) return st;
  if (!q || !k || !v || !o || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return VC_ERR_INVALID_ARG;
  if (vc_attn_workspace_size(p) > (size_t)VC_NOALLOC_WORKSPACE_BYTES) return VC_ERR_WORKSPACE;
  void* ws = nullptr;
  const vc_status sa = scratch_of(static_cast<hipStream_t>(stream), &ws);
  if (sa != VC_OK) return sa;
  // the same kernels as vc_attn_prepare + vc_attn_forward, workspace = the array
  const vc_status sp = vc_attn_prepare(p, q, k, v, ws, VC_NOALLOC_WORKSPACE_BYTES, stream);
  if (sp != VC_OK) return sp;
  return vc_attn_forward(p, ws, VC_NOALLOC_WORKSPACE_BYTES, o, stream);
}

const char* vc_attn_status_string(vc_status s) {
  switch (s) {
    case VC_OK: return "ok";
    case VC_ERR_INVALID_ARG: return "invalid argument";
    case VC_ERR_UNSUPPORTED: return "unsupported shape (d and block must be 128)";
    case VC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case VC_ERR_NOT_PREPARED: return "no clusters in the workspace for this shape";
    case VC_ERR_HIP: return "HIP runtime error";
    case VC_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

int32_t vc_attn_version(void) { return 200; }

}  // extern "C"
