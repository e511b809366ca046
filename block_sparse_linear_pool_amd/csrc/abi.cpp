// Host side of libsla2.so: argument validation, workspace plan, launch sequence.
// The declarations and conventions are in include/sla2.h.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "../../include/sla2.h"
#include "sla2_common.h"
#include "sla2_fit.h"
#include "sla2_grad.h"

using namespace sla2;

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  size_t err, qsum, ksum, mu64, mu32, Bt, At, mask, list, cnt, qc, kc, vc, sq, sk, sv, hbf, z,
      hpart, zpart, htot, ztot, ones;
  // backward only
  size_t tcnt, tlist, lse2, Dd, dht, dz, dhtot, dztot, kcol, kmean, qbf, vbf, ksb, dos, kplan,
      xoff, items, xpart;
  // stage-1 router gradient only
  size_t soft, lam, gO, gOs, gOl, ks16, v16, pk16, gmask, lossp, Arow, dA, dG, dB, total;
  int cap;
};

// Workspace regions of one entry point (256-byte aligned; regions an entry does not use are
// left at offset 0 and never touched). `kb` is the list stride of the forward entries.
Plan make_plan(const Geom& g, sla2_entry e, int kb) {
  Plan p{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up(bytes);
    return at;
  };
  const size_t BH = static_cast<size_t>(g.BH), N = g.N, nqb = g.nqb, nkb = g.nkb;
  const size_t np = (nkb + kKpPerWg - 1) / kKpPerWg;
  const bool grad = e == SLA2_ENTRY_ROUTER_GRAD;
  const bool router = e == SLA2_ENTRY_ROUTER || e == SLA2_ENTRY_ROUTER_SOFT ||
                      e == SLA2_ENTRY_FORWARD || e == SLA2_ENTRY_FORWARD_SLA1 || grad;
  const bool fwd = e == SLA2_ENTRY_FORWARD || e == SLA2_ENTRY_FORWARD_WITH_MASK ||
                   e == SLA2_ENTRY_FORWARD_SLA1 || grad;
  const bool bwd = e == SLA2_ENTRY_BACKWARD;
  p.err = take(4);                     // offset 0: the attention kernel's error word
  p.qsum = take(BH * nqb * kD * 8);    // the pool pass always writes both block sums
  p.ksum = take(BH * nkb * kD * 8);
  p.mu64 = take(BH * kD * 8);
  p.mu32 = take(BH * kD * 4);
  if (router) {
    p.Bt = take(BH * nkb * kD * 4);   // B = (Kbar - mu) Wk, fp32
    p.At = take(BH * nqb * kD * 4);   // A = Qbar Wq, fp32
  }
  if (fwd || bwd) {
    const size_t stride =
        e == SLA2_ENTRY_FORWARD || e == SLA2_ENTRY_FORWARD_SLA1 || grad ? kb : nkb;
    p.mask = take(BH * nqb * nkb);
    p.list = take(BH * nqb * stride * 4);
    p.cnt = take(BH * nqb * 4);
    p.kc = take(BH * N * kD);
    p.vc = take(BH * N * kD);
    p.sk = take(BH * nkb * 4);
    p.sv = take(BH * nkb * 4);
    p.hbf = take(BH * nkb * kD * kD * 2);
    p.htot = take(BH * kD * kD * 4);
    p.ztot = take(BH * kD * 4);
  }
  if (fwd) {
    p.qc = take(BH * N * kD);
    p.sq = take(BH * nqb * 4);
  }
  if (fwd || bwd || e == SLA2_ENTRY_LINEAR_PRECOMPUTE) {
    p.z = take(BH * nkb * kD * 4);
    p.hpart = take(BH * np * kD * kD * 4);
    p.zpart = take(BH * np * kD * 4);
  }
  if (e == SLA2_ENTRY_FORWARD_SLA1) p.ones = take(static_cast<size_t>(g.H) * nqb * 4);
  if (bwd) {
    p.tcnt = take(BH * nkb * 4);
    p.tlist = take(BH * nkb * nqb * 2);
    p.lse2 = take(BH * N * 4);
    p.Dd = take(BH * N * 4);
    p.dht = take(BH * nqb * kD * kD * 2);
    p.dz = take(BH * nqb * kD * 4);
    p.dhtot = take(BH * kD * kD * 4);
    p.dztot = take(BH * kD * 4);
    p.kcol = take(BH * nkb * kD * 4);
    p.kmean = take(BH * kD * 4);
    p.qbf = take(BH * N * kD * 2);
    p.vbf = take(BH * N * kD * 2);
    p.ksb = take(BH * N * kD * 2);
    p.dos = take(BH * N * kD * 2);
    p.cap = static_cast<int>((nkb + 1) / 2);
    p.kplan = take(BH * 2 * 4);
    p.xoff = take(BH * nkb * 4);
    p.items = take(BH * static_cast<size_t>(p.cap) * 4);
    p.xpart = take(BH * static_cast<size_t>(p.cap) * kSlot * 4);
  }
  if (grad) {
    p.soft = take(BH * nqb * nkb * 4);
    p.lam = take(BH * nqb * 4);
    p.gO = take(BH * N * kD * 4);
    p.gOs = take(BH * N * kD * 4);
    p.gOl = take(BH * N * kD * 4);
    p.ks16 = take(BH * N * kD * 2);
    p.v16 = take(BH * N * kD * 2);
    p.pk16 = take(BH * N * kD * 2);
    p.gmask = take(BH * nqb * nkb * 4);
    p.lossp = take(BH * nqb * 4);
    p.Arow = take(BH * nqb * kD * 4);
    p.dA = take(BH * nqb * kD * 4);
    p.dG = take(BH * nqb * nkb * 4);
    p.dB = take(BH * nkb * kD * 4);
  }
  p.total = o;
  return p;
}

bool entry_ok(int e) { return e >= SLA2_ENTRY_ROUTER && e <= SLA2_ENTRY_ROUTER_GRAD; }

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sla2_status check_shape(const sla2_shape* s, Geom* g) {
  if (s == nullptr) return SLA2_ERR_NULL_POINTER;
  if (s->dtype != SLA2_FP32 && s->dtype != SLA2_BF16) return SLA2_ERR_BAD_DTYPE;
  if (s->B < 1 || s->H < 1 || s->d != kD || s->N < kBQ || s->N % kBQ != 0 || s->N > kMaxN)
    return SLA2_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(s->B) * s->H > 65535) return SLA2_ERR_BAD_SHAPE;
  g->B = s->B;
  g->H = s->H;
  g->N = s->N;
  g->BH = s->B * s->H;
  g->nqb = s->N / kBQ;
  g->nkb = s->N / kBK;
  return SLA2_OK;
}

bool keep_ok(float k) { return std::isfinite(k) && k > 0.f && k <= 1.f; }

// Pointer checks: required pointers non-null; every given pointer 16-byte aligned.
struct PtrCheck {
  sla2_status st = SLA2_OK;
  void req(const void* p) {
    if (st != SLA2_OK) return;
    if (p == nullptr) st = SLA2_ERR_NULL_POINTER;
    else if (!aligned16(p)) st = SLA2_ERR_MISALIGNED;
  }
  void opt(const void* p) {
    if (st != SLA2_OK || p == nullptr) return;
    if (!aligned16(p)) st = SLA2_ERR_MISALIGNED;
  }
};

sla2_status check_workspace(const Plan& p, const void* ws, size_t bytes) {
  if (ws == nullptr) return SLA2_ERR_NULL_POINTER;
  if (!aligned16(ws)) return SLA2_ERR_MISALIGNED;
  if (bytes < p.total) return SLA2_ERR_WORKSPACE_TOO_SMALL;
  return SLA2_OK;
}

// Scratch of sla2_router_noalloc: a file-scope device array, one copy per GPU, held until the
// process ends. In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device, at that device's set-up (hipGetSymbolAddress with
// the device current), kept in g_scratch[dev], and only that pointer is ever handed to
// kernels.
static __device__ __align__(256) uint8_t scratch[SLA2_NOALLOC_SCRATCH_BYTES];

// The state the library keeps, per device, from its set-up (the first call on that device or
// sla2_init_device): whether it is a gfx950 (and the scoring kernel's LDS limit raised), and the
// device address of `scratch`.
std::atomic<int> g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other
std::atomic<void*> g_scratch[64];

sla2_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SLA2_ERR_HIP;
  if (dev < 0 || dev >= 64) return SLA2_ERR_UNSUPPORTED_DEVICE;
  int st = g_dev_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SLA2_ERR_HIP;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (st == 1) {
      if (configure_router() != hipSuccess) return SLA2_ERR_HIP;
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return SLA2_ERR_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
    g_dev_ok[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? SLA2_OK : SLA2_ERR_UNSUPPORTED_DEVICE;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("SLA2_DEBUG_SYNC");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

// Optional caller events recorded around every kernel (see sla2_taps.stage_events).
struct Rec {
  void** ev;
  int n, cap;
  explicit Rec(const sla2_taps* t)
      : ev(t ? t->stage_events : nullptr), n(0), cap(SLA2_MAX_STAGES + 1) {}
  explicit Rec(void** events, int count = SLA2_MAX_STAGES + 1) : ev(events), n(0), cap(count) {}
  hipError_t mark(hipStream_t s) {
    if (ev == nullptr || n >= cap) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(ev[n++]), s);
  }
};

// Runs a launch; records the caller's stage event; in debug mode also synchronises.
#define SLA2_LAUNCH(expr)                                                   \
  do {                                                                      \
    if ((expr) != hipSuccess) return SLA2_ERR_HIP;                          \
    if (rec.mark(stream) != hipSuccess) return SLA2_ERR_HIP;                \
    if (debug_sync() && hipStreamSynchronize(stream) != hipSuccess)         \
      return SLA2_ERR_HIP;                                                  \
  } while (0)

// The workspace's error word (set by a bounded wait of the attention kernel that gave up).
sla2_status read_error_word(const void* ws, hipStream_t stream) {
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SLA2_ERR_HIP;
  return word != 0 ? SLA2_ERR_WAIT_TIMEOUT : SLA2_OK;
}

}  // namespace

extern "C" {

int32_t sla2_blocks_kept(int32_t n_key_blocks, float keep_frac) {
  if (n_key_blocks < 1 || !keep_ok(keep_frac)) return -1;
  const double v = std::floor(static_cast<double>(keep_frac) * n_key_blocks + 1e-9);
  int64_t kb = static_cast<int64_t>(v);
  if (kb < 1) kb = 1;
  if (kb > n_key_blocks) kb = n_key_blocks;
  return static_cast<int32_t>(kb);
}

size_t sla2_workspace_bytes(const sla2_shape* shape, sla2_entry entry, float keep_frac) {
  Geom g;
  if (check_shape(shape, &g) != SLA2_OK || !entry_ok(entry)) return 0;
  int kb = g.nkb;
  if (entry == SLA2_ENTRY_FORWARD || entry == SLA2_ENTRY_FORWARD_SLA1 ||
      entry == SLA2_ENTRY_ROUTER_GRAD) {
    if (!keep_ok(keep_frac)) return 0;
    kb = sla2_blocks_kept(g.nkb, keep_frac);
  }
  return make_plan(g, entry, kb).total;
}

sla2_status sla2_workspace_status(const void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return SLA2_ERR_NULL_POINTER;
  if (!aligned16(workspace)) return SLA2_ERR_MISALIGNED;
  if (workspace_bytes < kAlign) return SLA2_ERR_WORKSPACE_TOO_SMALL;
  return read_error_word(workspace, static_cast<hipStream_t>(stream));
}

const char* sla2_status_string(sla2_status s) {
  switch (s) {
    case SLA2_OK: return "success";
    case SLA2_ERR_NULL_POINTER: return "a required pointer is NULL";
    case SLA2_ERR_BAD_SHAPE:
      return "bad shape: need d == 128, N a positive multiple of 128 up to 262144, B, H >= 1, "
             "B*H <= 65535";
    case SLA2_ERR_BAD_DTYPE: return "unsupported dtype (SLA2_FP32 or SLA2_BF16)";
    case SLA2_ERR_MISALIGNED: return "a device pointer is not 16-byte aligned";
    case SLA2_ERR_BAD_ARGUMENT:
      return "bad argument (keep_frac must lie in (0, 1]; quant must be SLA2_QUANT_NONE or "
             "SLA2_QUANT_I8_FP8; tau finite and > 0)";
    case SLA2_ERR_WORKSPACE_TOO_SMALL:
      return "workspace smaller than sla2_workspace_bytes() for this entry point (for "
             "sla2_router_noalloc: the shape needs more than SLA2_NOALLOC_SCRATCH_BYTES)";
    case SLA2_ERR_UNSUPPORTED_DEVICE: return "the current HIP device is not gfx950 (MI355X)";
    case SLA2_ERR_HIP: return "a HIP call or kernel launch failed";
    case SLA2_ERR_WAIT_TIMEOUT:
      return "a bounded wait inside the attention kernel gave up; the output is unreliable";
  }
  return "unknown status";
}

sla2_status sla2_init_device(void) { return check_device(); }

namespace {

// Checks of the router's arguments other than the workspace (both router entry points).
sla2_status check_router_args(const sla2_shape* shape, const void* Q, const void* K,
                              const float* proj_q, const float* proj_k, float keep_frac,
                              const uint8_t* mask, const int32_t* blocks, const float* scores,
                              Geom* g) {
  sla2_status st = check_shape(shape, g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(Q); pc.req(K); pc.req(proj_q); pc.req(proj_k); pc.req(blocks);
  pc.opt(mask); pc.opt(scores);
  if (pc.st != SLA2_OK) return pc.st;
  if (!keep_ok(keep_frac)) return SLA2_ERR_BAD_ARGUMENT;
  return SLA2_OK;
}

// pool -> colmean -> project -> score_topk with the router's workspace regions at `workspace`.
sla2_status run_router(const Geom& g, int dt, const void* Q, const void* K, const float* proj_q,
                       const float* proj_k, int kb, uint8_t* mask, int32_t* blocks,
                       float* scores, void* workspace, const Plan& p, hipStream_t stream) {
  Rec rec(static_cast<void**>(nullptr));
  SLA2_LAUNCH(launch_pool(g, dt, Q, K, at<double>(workspace, p.qsum), at<double>(workspace, p.ksum),
                          nullptr, nullptr, nullptr, stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(workspace, p.ksum), at<double>(workspace, p.mu64),
                             at<float>(workspace, p.mu32), nullptr, nullptr, stream));
  SLA2_LAUNCH(launch_project(g, at<double>(workspace, p.ksum), at<double>(workspace, p.mu64),
                             proj_k, at<float>(workspace, p.Bt), at<double>(workspace, p.qsum),
                             proj_q, at<float>(workspace, p.At), stream));
  SLA2_LAUNCH(launch_score_topk(g, at<float>(workspace, p.At), at<float>(workspace, p.Bt), kb,
                                mask, blocks, kb, nullptr, scores, stream));
  return SLA2_OK;
}

}  // namespace

sla2_status sla2_router(const sla2_shape* shape, const void* Q, const void* K,
                        const float* proj_q, const float* proj_k, float keep_frac,
                        uint8_t* mask, int32_t* blocks, float* scores, void* workspace,
                        size_t workspace_bytes, void* stream_) {
  Geom g;
  sla2_status st = check_router_args(shape, Q, K, proj_q, proj_k, keep_frac, mask, blocks,
                                     scores, &g);
  if (st != SLA2_OK) return st;
  const int kb = sla2_blocks_kept(g.nkb, keep_frac);
  const Plan p = make_plan(g, SLA2_ENTRY_ROUTER, kb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  return run_router(g, shape->dtype == SLA2_FP32 ? 0 : 1, Q, K, proj_q, proj_k, kb, mask,
                    blocks, scores, workspace, p, static_cast<hipStream_t>(stream_));
}

sla2_status sla2_router_noalloc(const sla2_shape* shape, const void* Q, const void* K,
                                const float* proj_q, const float* proj_k, float keep_frac,
                                uint8_t* mask, int32_t* blocks, float* scores, void* stream_) {
  Geom g;
  sla2_status st = check_router_args(shape, Q, K, proj_q, proj_k, keep_frac, mask, blocks,
                                     scores, &g);
  if (st != SLA2_OK) return st;
  const int kb = sla2_blocks_kept(g.nkb, keep_frac);
  const Plan p = make_plan(g, SLA2_ENTRY_ROUTER, kb);
  if (p.total > SLA2_NOALLOC_SCRATCH_BYTES) return SLA2_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device()) != SLA2_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SLA2_ERR_HIP;
  void* ws = g_scratch[dev].load(std::memory_order_acquire);   // set by check_device
  if (ws == nullptr) return SLA2_ERR_HIP;
  return run_router(g, shape->dtype == SLA2_FP32 ? 0 : 1, Q, K, proj_q, proj_k, kb, mask,
                    blocks, scores, ws, p, static_cast<hipStream_t>(stream_));
}

sla2_status sla2_router_soft(const sla2_shape* shape, const void* Q, const void* K,
                             const float* proj_q, const float* proj_k, float keep_frac, float tau,
                             float* soft_mask, float* lambda, void** stage_events,
                             void* workspace, size_t workspace_bytes, void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(Q); pc.req(K); pc.req(proj_q); pc.req(proj_k); pc.req(soft_mask);
  pc.opt(lambda);
  if (pc.st != SLA2_OK) return pc.st;
  if (!keep_ok(keep_frac) || !std::isfinite(tau) || !(tau > 0.f) || !std::isfinite(1.0f / tau))
    return SLA2_ERR_BAD_ARGUMENT;
  const int kb = sla2_blocks_kept(g.nkb, keep_frac);
  const Plan p = make_plan(g, SLA2_ENTRY_ROUTER_SOFT, kb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int dt = shape->dtype == SLA2_FP32 ? 0 : 1;
  Rec rec(stage_events, 5);
  if (rec.mark(stream) != hipSuccess) return SLA2_ERR_HIP;
  SLA2_LAUNCH(launch_pool(g, dt, Q, K, at<double>(workspace, p.qsum), at<double>(workspace, p.ksum),
                          nullptr, nullptr, nullptr, stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(workspace, p.ksum), at<double>(workspace, p.mu64),
                             at<float>(workspace, p.mu32), nullptr, nullptr, stream));
  SLA2_LAUNCH(launch_project(g, at<double>(workspace, p.ksum), at<double>(workspace, p.mu64),
                             proj_k, at<float>(workspace, p.Bt), at<double>(workspace, p.qsum),
                             proj_q, at<float>(workspace, p.At), stream));
  SLA2_LAUNCH(launch_score_soft(g, at<float>(workspace, p.At), at<float>(workspace, p.Bt), kb,
                                1.0f / tau, soft_mask, lambda, stream));
  return SLA2_OK;
}

sla2_status sla2_linear_precompute(const sla2_shape* shape, const void* K, const void* V,
                                   float* k_colmean, float* h, float* z, float* h_total,
                                   float* z_total, void* workspace, size_t workspace_bytes,
                                   void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(K); pc.req(V); pc.req(k_colmean); pc.req(h_total); pc.req(z_total);
  pc.opt(h); pc.opt(z);
  if (pc.st != SLA2_OK) return pc.st;
  const Plan p = make_plan(g, SLA2_ENTRY_LINEAR_PRECOMPUTE, g.nkb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int dt = shape->dtype == SLA2_FP32 ? 0 : 1;
  Rec rec(static_cast<void**>(nullptr));
  SLA2_LAUNCH(launch_pool(g, dt, nullptr, K, at<double>(workspace, p.qsum),
                          at<double>(workspace, p.ksum), nullptr, nullptr, nullptr, stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(workspace, p.ksum), at<double>(workspace, p.mu64),
                             at<float>(workspace, p.mu32), k_colmean, nullptr, stream));
  KvArgs kv{};
  kv.mu32 = at<float>(workspace, p.mu32);
  kv.h_f32 = h;
  kv.z = z ? z : at<float>(workspace, p.z);
  kv.hpart = at<float>(workspace, p.hpart);
  kv.zpart = at<float>(workspace, p.zpart);
  SLA2_LAUNCH(launch_kv_prep(g, dt, K, V, kv, stream));
  SLA2_LAUNCH(launch_linear_total(g, at<float>(workspace, p.hpart), at<float>(workspace, p.zpart),
                                  h_total, z_total, 1, stream));
  return SLA2_OK;
}

namespace {

// Everything after the block lists exist: K, V operands and the linear precompute, H_tot,
// then the attention kernel (sparse branch + linear branch + combine). Low-bit quantisation:
// Q codes come from the pool pass and the one attention kernel does everything. Without
// quantisation: the attention kernel runs its linear branch alone (O = (1 - alpha) O_l), then
// the fp32 sparse kernel adds alpha O_s.
sla2_status run_branches(const Geom& g, int dt, sla2_quant quant, const void* Q, const void* K,
                         const void* V, const float* alpha, float* O, const sla2_taps* taps,
                         void* ws, const Plan& p, int list_stride, Rec& rec, hipStream_t stream) {
  const sla2_taps none{};
  const sla2_taps& tp = taps ? *taps : none;
  const bool lowbit = quant == SLA2_QUANT_I8_FP8;
  const float* sq = lowbit && tp.s_q ? tp.s_q : at<float>(ws, p.sq);
  float* sk = lowbit && tp.s_k ? tp.s_k : at<float>(ws, p.sk);
  float* sv = lowbit && tp.s_v ? tp.s_v : at<float>(ws, p.sv);
  KvArgs kv{};
  kv.mu32 = at<float>(ws, p.mu32);
  kv.kc = at<int8_t>(ws, p.kc);
  kv.vc = at<uint8_t>(ws, p.vc);
  kv.sk = sk;
  kv.sv = sv;
  kv.k_tap = lowbit ? tp.k_codes : nullptr;
  kv.v_tap = lowbit ? tp.v_codes : nullptr;
  kv.ht_bf16 = at<uint16_t>(ws, p.hbf);
  kv.z = at<float>(ws, p.z);
  kv.hpart = at<float>(ws, p.hpart);
  kv.zpart = at<float>(ws, p.zpart);
  SLA2_LAUNCH(launch_kv_prep(g, dt, K, V, kv, stream));
  SLA2_LAUNCH(launch_linear_total(g, at<float>(ws, p.hpart), at<float>(ws, p.zpart),
                                  at<float>(ws, p.htot), at<float>(ws, p.ztot), 0, stream));
  AttnArgs x{};
  x.qc = at<int8_t>(ws, p.qc);
  x.kc = at<int8_t>(ws, p.kc);
  x.vc = at<uint8_t>(ws, p.vc);
  x.sq = sq;
  x.sk = sk;
  x.sv = sv;
  x.ht_bf16 = at<uint16_t>(ws, p.hbf);
  x.z = at<float>(ws, p.z);
  x.htot_t = at<float>(ws, p.htot);
  x.ztot = at<float>(ws, p.ztot);
  x.mask = at<uint8_t>(ws, p.mask);
  x.list = at<int32_t>(ws, p.list);
  x.list_stride = list_stride;
  x.cnt = at<int32_t>(ws, p.cnt);
  x.alpha = alpha;
  x.O = O;
  x.O_s_tap = tp.O_s;
  x.O_l_tap = tp.O_l;
  x.err = at<uint32_t>(ws, p.err);
  x.sparse = lowbit;
  SLA2_LAUNCH(launch_attn(g, dt, Q, x, stream));
  if (!lowbit) {
    ExactArgs e{};
    e.K = K;
    e.V = V;
    e.mu32 = at<float>(ws, p.mu32);
    e.list = x.list;
    e.list_stride = list_stride;
    e.cnt = x.cnt;
    e.alpha = alpha;
    e.O = O;
    e.O_s_tap = tp.O_s;
    SLA2_LAUNCH(launch_attn_exact(g, dt, Q, e, stream));
  }
  if (debug_sync()) return read_error_word(ws, stream);
  return SLA2_OK;
}

void check_taps(PtrCheck& pc, const sla2_taps* t) {
  if (!t) return;
  pc.opt(t->O_s); pc.opt(t->O_l); pc.opt(t->q_codes); pc.opt(t->k_codes); pc.opt(t->v_codes);
  pc.opt(t->s_q); pc.opt(t->s_k); pc.opt(t->s_v); pc.opt(t->k_colmean);
}

bool quant_ok(sla2_quant q) { return q == SLA2_QUANT_NONE || q == SLA2_QUANT_I8_FP8; }

}  // namespace

sla2_status sla2_forward(const sla2_shape* shape, const void* Q, const void* K, const void* V,
                         const float* proj_q, const float* proj_k, const float* alpha,
                         float keep_frac, sla2_quant quant, float* O, const sla2_taps* taps,
                         void* workspace, size_t workspace_bytes, void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(Q); pc.req(K); pc.req(V); pc.req(proj_q); pc.req(proj_k); pc.req(alpha); pc.req(O);
  check_taps(pc, taps);
  if (pc.st != SLA2_OK) return pc.st;
  if (!keep_ok(keep_frac) || !quant_ok(quant)) return SLA2_ERR_BAD_ARGUMENT;
  const int kb = sla2_blocks_kept(g.nkb, keep_frac);
  const Plan p = make_plan(g, SLA2_ENTRY_FORWARD, kb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int dt = shape->dtype == SLA2_FP32 ? 0 : 1;
  const bool lowbit = quant == SLA2_QUANT_I8_FP8;
  void* ws = workspace;
  Rec rec(taps);
  if (rec.mark(stream) != hipSuccess) return SLA2_ERR_HIP;
  SLA2_LAUNCH(launch_pool(g, dt, Q, K, at<double>(ws, p.qsum), at<double>(ws, p.ksum),
                          lowbit ? at<int8_t>(ws, p.qc) : nullptr,
                          lowbit && taps && taps->s_q ? taps->s_q : at<float>(ws, p.sq),
                          lowbit && taps ? taps->q_codes : nullptr, stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64), at<float>(ws, p.mu32),
                             taps ? taps->k_colmean : nullptr, at<uint32_t>(ws, p.err), stream));
  SLA2_LAUNCH(launch_project(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64), proj_k,
                             at<float>(ws, p.Bt), at<double>(ws, p.qsum), proj_q,
                             at<float>(ws, p.At), stream));
  SLA2_LAUNCH(launch_score_topk(g, at<float>(ws, p.At), at<float>(ws, p.Bt), kb,
                                at<uint8_t>(ws, p.mask), at<int32_t>(ws, p.list), kb,
                                at<int32_t>(ws, p.cnt), nullptr, stream));
  return run_branches(g, dt, quant, Q, K, V, alpha, O, taps, ws, p, kb, rec, stream);
}

sla2_status sla2_forward_sla1(const sla2_shape* shape, const void* Q, const void* K,
                              const void* V, const float* proj_o, float keep_frac,
                              sla2_quant quant, float* O, float* O_l, void** stage_events,
                              void* workspace, size_t workspace_bytes, void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(Q); pc.req(K); pc.req(V); pc.req(proj_o); pc.req(O); pc.req(O_l);
  if (pc.st != SLA2_OK) return pc.st;
  if (!keep_ok(keep_frac) || !quant_ok(quant)) return SLA2_ERR_BAD_ARGUMENT;
  const int kb = sla2_blocks_kept(g.nkb, keep_frac);
  const Plan p = make_plan(g, SLA2_ENTRY_FORWARD_SLA1, kb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int dt = shape->dtype == SLA2_FP32 ? 0 : 1;
  const bool lowbit = quant == SLA2_QUANT_I8_FP8;
  void* ws = workspace;
  Rec rec(stage_events);
  if (rec.mark(stream) != hipSuccess) return SLA2_ERR_HIP;
  SLA2_LAUNCH(launch_pool(g, dt, Q, K, at<double>(ws, p.qsum), at<double>(ws, p.ksum),
                          lowbit ? at<int8_t>(ws, p.qc) : nullptr, at<float>(ws, p.sq), nullptr,
                          stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64), at<float>(ws, p.mu32),
                             nullptr, at<uint32_t>(ws, p.err), stream));
  // the heuristic router: proj_q = proj_k = I (null weights select the identity mode)
  SLA2_LAUNCH(launch_project(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64), nullptr,
                             at<float>(ws, p.Bt), at<double>(ws, p.qsum), nullptr,
                             at<float>(ws, p.At), stream));
  SLA2_LAUNCH(launch_score_topk(g, at<float>(ws, p.At), at<float>(ws, p.Bt), kb,
                                at<uint8_t>(ws, p.mask), at<int32_t>(ws, p.list), kb,
                                at<int32_t>(ws, p.cnt), nullptr, stream));
  // both branches with alpha = 1 and the O_l tap: O receives O_s, O_l the linear branch
  SLA2_LAUNCH(launch_fill(at<float>(ws, p.ones), g.H * g.nqb, 1.0f, stream));
  sla2_taps tp{};
  tp.O_l = O_l;
  st = run_branches(g, dt, quant, Q, K, V, at<float>(ws, p.ones), O, &tp, ws, p, kb, rec, stream);
  if (st != SLA2_OK) return st;
  SLA2_LAUNCH(launch_sla1_mix(g, O_l, proj_o, O, stream));
  return SLA2_OK;
}

sla2_status sla2_forward_with_mask(const sla2_shape* shape, const void* Q, const void* K,
                                   const void* V, const uint8_t* mask, const float* alpha,
                                   sla2_quant quant, float* O, const sla2_taps* taps,
                                   void* workspace, size_t workspace_bytes, void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(Q); pc.req(K); pc.req(V); pc.req(mask); pc.req(alpha); pc.req(O);
  check_taps(pc, taps);
  if (pc.st != SLA2_OK) return pc.st;
  if (!quant_ok(quant)) return SLA2_ERR_BAD_ARGUMENT;
  const Plan p = make_plan(g, SLA2_ENTRY_FORWARD_WITH_MASK, g.nkb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int dt = shape->dtype == SLA2_FP32 ? 0 : 1;
  const bool lowbit = quant == SLA2_QUANT_I8_FP8;
  void* ws = workspace;
  Rec rec(taps);
  if (rec.mark(stream) != hipSuccess) return SLA2_ERR_HIP;
  SLA2_LAUNCH(launch_pool(g, dt, Q, K, at<double>(ws, p.qsum), at<double>(ws, p.ksum),
                          lowbit ? at<int8_t>(ws, p.qc) : nullptr,
                          lowbit && taps && taps->s_q ? taps->s_q : at<float>(ws, p.sq),
                          lowbit && taps ? taps->q_codes : nullptr, stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64), at<float>(ws, p.mu32),
                             taps ? taps->k_colmean : nullptr, at<uint32_t>(ws, p.err), stream));
  SLA2_LAUNCH(launch_mask_to_list(g, mask, at<uint8_t>(ws, p.mask), at<int32_t>(ws, p.list),
                                  at<int32_t>(ws, p.cnt), stream));
  return run_branches(g, dt, quant, Q, K, V, alpha, O, taps, ws, p, g.nkb, rec, stream);
}

sla2_status sla2_backward(const sla2_shape* shape, const void* Q, const void* K, const void* V,
                          const uint8_t* mask, const float* alpha, const float* dO, float* dQ,
                          float* dK, float* dV, float* dalpha, void** stage_events,
                          void* workspace, size_t workspace_bytes, void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(Q); pc.req(K); pc.req(V); pc.req(mask); pc.req(alpha); pc.req(dO);
  pc.req(dQ); pc.req(dK); pc.req(dV); pc.req(dalpha);
  if (pc.st != SLA2_OK) return pc.st;
  const Plan p = make_plan(g, SLA2_ENTRY_BACKWARD, g.nkb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int dt = shape->dtype == SLA2_FP32 ? 0 : 1;
  void* ws = workspace;
  Rec rec(stage_events, 15);
  if (rec.mark(stream) != hipSuccess) return SLA2_ERR_HIP;
  // forward pieces: colmean(K), the bf16 h_j^T, z_j and H_tot, Z_tot; the kept lists
  SLA2_LAUNCH(launch_pool(g, dt, nullptr, K, at<double>(ws, p.qsum), at<double>(ws, p.ksum),
                          nullptr, nullptr, nullptr, stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64),
                             at<float>(ws, p.mu32), nullptr, nullptr, stream));
  KvArgs kv{};
  kv.mu32 = at<float>(ws, p.mu32);
  kv.kc = at<int8_t>(ws, p.kc);
  kv.vc = at<uint8_t>(ws, p.vc);
  kv.sk = at<float>(ws, p.sk);
  kv.sv = at<float>(ws, p.sv);
  kv.ht_bf16 = at<uint16_t>(ws, p.hbf);
  kv.z = at<float>(ws, p.z);
  kv.hpart = at<float>(ws, p.hpart);
  kv.zpart = at<float>(ws, p.zpart);
  SLA2_LAUNCH(launch_kv_prep(g, dt, K, V, kv, stream));
  SLA2_LAUNCH(launch_linear_total(g, at<float>(ws, p.hpart), at<float>(ws, p.zpart),
                                  at<float>(ws, p.htot), at<float>(ws, p.ztot), 1, stream));
  SLA2_LAUNCH(launch_mask_to_list(g, mask, at<uint8_t>(ws, p.mask), at<int32_t>(ws, p.list),
                                  at<int32_t>(ws, p.cnt), stream));
  SLA2_LAUNCH(launch_key_lists(g, at<uint8_t>(ws, p.mask), at<int32_t>(ws, p.tcnt),
                               at<uint16_t>(ws, p.tlist), stream));
  SLA2_LAUNCH(launch_key_plan(g, at<int32_t>(ws, p.tcnt), at<int32_t>(ws, p.kplan),
                              at<int32_t>(ws, p.xoff), at<int32_t>(ws, p.items), p.cap, stream));
  BwdArgs b{};
  b.Q = Q; b.K = K; b.V = V;
  if (dt == 0) {   // fp32 inputs: bf16 copies of Q and V in the workspace
    b.qbf_w = at<uint16_t>(ws, p.qbf);
    b.vbf_w = at<uint16_t>(ws, p.vbf);
    b.qbf = b.qbf_w;
    b.vbf = b.vbf_w;
  } else {
    b.qbf = static_cast<const uint16_t*>(Q);
    b.vbf = static_cast<const uint16_t*>(V);
  }
  b.ksb = at<uint16_t>(ws, p.ksb);
  b.dos = at<uint16_t>(ws, p.dos);
  b.plan = at<int32_t>(ws, p.kplan);
  b.xoff = at<int32_t>(ws, p.xoff);
  b.items = at<int32_t>(ws, p.items);
  b.xpart = at<float>(ws, p.xpart);
  b.cap = p.cap;
  b.mu32 = at<float>(ws, p.mu32);
  b.dO = dO;
  b.alpha = alpha;
  b.list = at<int32_t>(ws, p.list);
  b.cnt = at<int32_t>(ws, p.cnt);
  b.hbf = at<uint16_t>(ws, p.hbf);
  b.htot = at<float>(ws, p.htot);
  b.z = at<float>(ws, p.z);
  b.ztot = at<float>(ws, p.ztot);
  b.dQ = dQ;
  b.dht = at<uint16_t>(ws, p.dht);
  b.dz = at<float>(ws, p.dz);
  b.dalpha = dalpha;
  b.dhtot = at<float>(ws, p.dhtot);
  b.dztot = at<float>(ws, p.dztot);
  b.lse2 = at<float>(ws, p.lse2);
  b.Dd = at<float>(ws, p.Dd);
  b.tcnt = at<int32_t>(ws, p.tcnt);
  b.tlist = at<uint16_t>(ws, p.tlist);
  b.dK = dK;
  b.dV = dV;
  b.kcol = at<float>(ws, p.kcol);
  b.kmean = at<float>(ws, p.kmean);
  b.H = g.H;
  b.BH = g.BH;
  b.nqb = g.nqb;
  b.nkb = g.nkb;
  SLA2_LAUNCH(launch_bwd_prep(g, dt, b, stream));
  SLA2_LAUNCH(launch_bwd_lin_q(g, dt, b, stream));
  SLA2_LAUNCH(launch_dh_total(g, b, stream));
  SLA2_LAUNCH(launch_bwd_q(g, b, stream));
  SLA2_LAUNCH(launch_bwd_kv_extra(g, b, stream));
  SLA2_LAUNCH(launch_bwd_kv(g, b, stream));
  SLA2_LAUNCH(launch_dk_center(g, b, stream));
  return SLA2_OK;
}

sla2_status sla2_fit_alpha(const sla2_shape* shape, const float* O_full, const float* O_s,
                           const float* O_l, float* alpha, void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(O_full); pc.req(O_s); pc.req(O_l); pc.req(alpha);
  if (pc.st != SLA2_OK) return pc.st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (launch_fit_alpha(g.B, g.H, g.N, O_full, O_s, O_l, alpha, stream) != hipSuccess)
    return SLA2_ERR_HIP;
  if (debug_sync() && hipStreamSynchronize(stream) != hipSuccess) return SLA2_ERR_HIP;
  return SLA2_OK;
}

sla2_status sla2_router_grad(const sla2_shape* shape, const void* Q, const void* K, const void* V,
                             const float* proj_q, const float* proj_k, const float* alpha,
                             float keep_frac, float tau, const float* O_full, float* dproj_q,
                             float* dproj_k, double* loss, float* mask_grad, void* workspace,
                             size_t workspace_bytes, void* stream_) {
  Geom g;
  sla2_status st = check_shape(shape, &g);
  if (st != SLA2_OK) return st;
  PtrCheck pc;
  pc.req(Q); pc.req(K); pc.req(V); pc.req(proj_q); pc.req(proj_k); pc.req(alpha);
  pc.req(O_full); pc.req(dproj_q); pc.req(dproj_k); pc.req(loss);
  pc.opt(mask_grad);
  if (pc.st != SLA2_OK) return pc.st;
  if (!keep_ok(keep_frac) || !std::isfinite(tau) || !(tau > 0.f) || !std::isfinite(1.0f / tau))
    return SLA2_ERR_BAD_ARGUMENT;
  const int kb = sla2_blocks_kept(g.nkb, keep_frac);
  const Plan p = make_plan(g, SLA2_ENTRY_ROUTER_GRAD, kb);
  if ((st = check_workspace(p, workspace, workspace_bytes)) != SLA2_OK) return st;
  if ((st = check_device()) != SLA2_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int dt = shape->dtype == SLA2_FP32 ? 0 : 1;
  void* ws = workspace;
  Rec rec(static_cast<void**>(nullptr));
  // the router: hard Top-k (mask and lists) and SoftTop-k (soft mask) from the same logits
  SLA2_LAUNCH(launch_pool(g, dt, Q, K, at<double>(ws, p.qsum), at<double>(ws, p.ksum), nullptr,
                          at<float>(ws, p.sq), nullptr, stream));
  SLA2_LAUNCH(launch_colmean(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64), at<float>(ws, p.mu32),
                             nullptr, at<uint32_t>(ws, p.err), stream));
  SLA2_LAUNCH(launch_project(g, at<double>(ws, p.ksum), at<double>(ws, p.mu64), proj_k,
                             at<float>(ws, p.Bt), at<double>(ws, p.qsum), proj_q,
                             at<float>(ws, p.At), stream));
  SLA2_LAUNCH(launch_score_topk(g, at<float>(ws, p.At), at<float>(ws, p.Bt), kb,
                                at<uint8_t>(ws, p.mask), at<int32_t>(ws, p.list), kb,
                                at<int32_t>(ws, p.cnt), nullptr, stream));
  SLA2_LAUNCH(launch_score_soft(g, at<float>(ws, p.At), at<float>(ws, p.Bt), kb,
                                1.0f / tau, at<float>(ws, p.soft), at<float>(ws, p.lam), stream));
  // the unquantised forward with its branch outputs kept
  sla2_taps tp{};
  tp.O_s = at<float>(ws, p.gOs);
  tp.O_l = at<float>(ws, p.gOl);
  if ((st = run_branches(g, dt, SLA2_QUANT_NONE, Q, K, V, alpha, at<float>(ws, p.gO), &tp, ws, p,
                         kb, rec, stream)) != SLA2_OK)
    return st;
  // dL/dM over every block pair, then the router's chain
  GradArgs x{};
  x.mu32 = at<float>(ws, p.mu32);
  x.ks16 = at<uint32_t>(ws, p.ks16);
  x.v16 = at<uint32_t>(ws, p.v16);
  x.pk16 = at<uint32_t>(ws, p.pk16);
  x.O = at<float>(ws, p.gO);
  x.O_full = O_full;
  x.O_s = tp.O_s;
  x.O_l = tp.O_l;
  x.z = at<float>(ws, p.z);
  x.ztot = at<float>(ws, p.ztot);
  x.mask = at<uint8_t>(ws, p.mask);
  x.list = at<int32_t>(ws, p.list);
  x.list_stride = kb;
  x.cnt = at<int32_t>(ws, p.cnt);
  x.alpha = alpha;
  x.g = mask_grad ? mask_grad : at<float>(ws, p.gmask);
  x.lossp = at<float>(ws, p.lossp);
  x.Arow = at<float>(ws, p.Arow);
  x.dA = at<float>(ws, p.dA);
  x.dG = at<float>(ws, p.dG);
  x.dB = at<float>(ws, p.dB);
  SLA2_LAUNCH(launch_grad_prep(g, dt, K, V, x, stream));
  SLA2_LAUNCH(launch_mask_grad(g, dt, Q, x, stream));
  SLA2_LAUNCH(launch_router_vjp(g, at<double>(ws, p.qsum), at<double>(ws, p.ksum),
                                at<double>(ws, p.mu64), proj_q, at<float>(ws, p.Bt),
                                at<float>(ws, p.soft), x, 1.0f / tau, dproj_q, dproj_k, loss,
                                stream));
  return SLA2_OK;
}

}  // extern "C"
