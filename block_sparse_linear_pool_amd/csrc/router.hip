// SLA2 router (step 1 of the computation flow on the summary page "SLA2: Sparse-Linear
// Attention with Learnable Routing and QAT", paper.rainbus.top; "Router" box of the §3
// flowchart of "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers"):
// mean-pool Q (128 rows) and the smoothed K (64 rows), project with proj_q / proj_k,
// score every block pair, keep the top kb key blocks of every query block.
//
// Kernels, in launch order:
//   pool        one pass over Q and K (HBM-bound): fp64 block sums of Q and K, and (in
//               the forward) the INT8 codes of Q for the sparse branch.
//   colmean     mu = colmean(K) from the key-block sums (all blocks have 64 rows), the
//               K smoothing of §7 note 1 of the second page.
//   project     B = (Kbar - mu) Wk and A = Qbar Wq in fp32 (Kbar - mu is the mean of K_s);
//               with no weights the identity (the heuristic router of the earlier SLA).
//   score_topk  per 16 query blocks: G = A B^T / sqrt(d) in fp32 (MFMA) into
//               LDS, then one wavefront per query block selects the kb largest logits
//               exactly (ties to the lower index) and writes the mask and the ascending
//               block list; in its soft mode the SoftTop-k mask sigma(P_c / tau + lambda_i)
//               of the training-time router.
//   fill        a constant into a float array (alpha = 1 for the earlier SLA mix).
// Ranking by the logit G is ranking by P_c = softmax(G): softmax is monotone per row.
#include "sla2_common.h"

namespace sla2 {

// ---------------------------------------------------------------- pool
// grid (nqb, BH), 256 threads. Thread t: 8 columns starting at 8*(t%16), rows t/16 + 16m.
// kMode 0: K only; 1: Q and K; 2: also quantise the 128-row Q block to INT8 (step 2 operands,
// §2 Q2 of the second page): inv = fl32(127 / amax), code = clamp(rne(fl32(x inv)), +-127),
// s_q = fl32(amax / 127); an all-zero block gets scale 0 and zero codes. Every load of the
// thread is issued before the first use (the mode is a template argument: a run-time test
// around the Q loads made the compiler wait for each one in turn).
template <typename T, int kMode>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ Q,
                                                   const T* __restrict__ K,
                                                   double* __restrict__ qsum,
                                                   double* __restrict__ ksum,
                                                   int8_t* __restrict__ qc,
                                                   float* __restrict__ sq,
                                                   int8_t* __restrict__ q_tap, int N) {
  constexpr bool kQ = kMode >= 1, kCodes = kMode == 2;
  __shared__ double red[3][16][kD + 2];
  __shared__ float amax_w[4];
  const int i = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int cg = t & 15, rl = t >> 4;
  const size_t base = (static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ) * kD;
  auto off_of = [&](int m) { return base + static_cast<size_t>(rl + 16 * m) * kD + 8 * cg; };
  Raw8<T> rq[8], rk[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if constexpr (kQ) rq[m] = load_raw8<T>(Q + off_of(m));
    rk[m] = load_raw8<T>(K + off_of(m));
  }
  double aq[8] = {}, ak0[8] = {}, ak1[8] = {};
  float am = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (kQ) {
        const float x = raw8_at(rq[m], c);
        aq[c] += static_cast<double>(x);
        am = fmaxf(am, fabsf(x));
      }
      const double y = static_cast<double>(raw8_at(rk[m], c));
      if (m < 4) ak0[c] += y;
      else ak1[c] += y;
    }
  }
  if constexpr (kCodes) {
    am = wave_max(am);
    if ((t & 63) == 0) amax_w[t >> 6] = am;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    red[0][rl][8 * cg + c] = aq[c];
    red[1][rl][8 * cg + c] = ak0[c];
    red[2][rl][8 * cg + c] = ak1[c];
  }
  __syncthreads();
  if constexpr (kCodes) {
    const float amb = fmaxf(fmaxf(amax_w[0], amax_w[1]), fmaxf(amax_w[2], amax_w[3]));
    const float inv = amb > 0.f ? 127.0f / amb : 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint2 w = make_uint2(
          i8_pack4(raw8_at(rq[m], 0), raw8_at(rq[m], 1), raw8_at(rq[m], 2), raw8_at(rq[m], 3), inv),
          i8_pack4(raw8_at(rq[m], 4), raw8_at(rq[m], 5), raw8_at(rq[m], 6), raw8_at(rq[m], 7), inv));
      *reinterpret_cast<uint2*>(qc + off_of(m)) = w;
      if (q_tap != nullptr) *reinterpret_cast<uint2*>(q_tap + off_of(m)) = w;
    }
    if (t == 0) sq[static_cast<size_t>(bh) * (N / kBQ) + i] = amb / 127.0f;
  }
  // threads 0..127: Q column t; 128..255: first key block column t-128; then second.
  {
    const int which = t >> 7, c = t & 127;
    double s = 0.0;
    for (int r = 0; r < 16; ++r) s += red[which][r][c];
    if (which == 0) {
      if constexpr (kQ) qsum[(static_cast<size_t>(bh) * (N / kBQ) + i) * kD + c] = s;
    } else {
      ksum[(static_cast<size_t>(bh) * (N / kBK) + 2 * i) * kD + c] = s;
    }
    if (t < 128) {
      double s2 = 0.0;
      for (int r = 0; r < 16; ++r) s2 += red[2][r][t];
      ksum[(static_cast<size_t>(bh) * (N / kBK) + 2 * i + 1) * kD + t] = s2;
    }
  }
}

template <typename T>
static void launch_pool_t(const Geom& g, const T* Q, const T* K, double* qsum, double* ksum,
                          int8_t* qc, float* sq, int8_t* q_tap, hipStream_t s) {
  dim3 grid(g.nqb, g.BH);
  if (Q == nullptr)
    hipLaunchKernelGGL((pool_kernel<T, 0>), grid, dim3(256), 0, s, Q, K, qsum, ksum, qc, sq,
                       q_tap, g.N);
  else if (qc == nullptr)
    hipLaunchKernelGGL((pool_kernel<T, 1>), grid, dim3(256), 0, s, Q, K, qsum, ksum, qc, sq,
                       q_tap, g.N);
  else
    hipLaunchKernelGGL((pool_kernel<T, 2>), grid, dim3(256), 0, s, Q, K, qsum, ksum, qc, sq,
                       q_tap, g.N);
}

hipError_t launch_pool(const Geom& g, int dtype, const void* Q, const void* K, double* qsum,
                       double* ksum, int8_t* qc, float* sq, int8_t* q_tap, hipStream_t s) {
  if (dtype == 0)
    launch_pool_t<float>(g, static_cast<const float*>(Q), static_cast<const float*>(K), qsum,
                         ksum, qc, sq, q_tap, s);
  else
    launch_pool_t<uint16_t>(g, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                            qsum, ksum, qc, sq, q_tap, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- colmean
// grid (8, BH), 1024 threads: workgroup x takes columns 16 x .. 16 x + 15 of head bh; thread t
// sums column 16 x + t % 16 over key blocks t / 16 + 64 m (eight loads in flight per round, so
// one round covers 512 key blocks); the 64 partial sums of a column are combined by a fixed
// pairwise tree in LDS (deterministic).
constexpr int kColThreads = 1024;
__global__ __launch_bounds__(kColThreads) void colmean_kernel(const double* __restrict__ ksum,
                                                              double* __restrict__ mu64,
                                                              float* __restrict__ mu32,
                                                              float* __restrict__ mu32_tap,
                                                              uint32_t* __restrict__ err, int nkb,
                                                              int N) {
  __shared__ double part[64][17];
  const int bh = blockIdx.y, t = threadIdx.x, c = 16 * blockIdx.x + (t & 15), sl = t >> 4;
  if (err != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && t == 0) *err = 0u;
  const double* p = ksum + static_cast<size_t>(bh) * nkb * kD + c;
  double a = 0.0;
  for (int j0 = sl; j0 < nkb; j0 += 512) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = j0 + 64 * u < nkb ? p[static_cast<size_t>(j0 + 64 * u) * kD] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) a += v[u];
  }
  part[sl][t & 15] = a;
  __syncthreads();
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    if (sl < h) part[sl][t & 15] += part[sl + h][t & 15];
    __syncthreads();
  }
  if (t < 16) {
    const double mu = part[0][t] / static_cast<double>(N);
    mu64[bh * kD + c] = mu;
    mu32[bh * kD + c] = static_cast<float>(mu);
    if (mu32_tap) mu32_tap[bh * kD + c] = static_cast<float>(mu);
  }
}

hipError_t launch_colmean(const Geom& g, const double* ksum, double* mu64, float* mu32,
                          float* mu32_tap, uint32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(colmean_kernel, dim3(kD / 16, g.BH), dim3(kColThreads), 0, s, ksum, mu64,
                     mu32, mu32_tap, err, g.nkb, g.N);
  return hipGetLastError();
}

// fp32 MFMA 16x16x4 operand/result layout (gfx950): lane l supplies A[l % 16][k] and
// B[k][l % 16] for the K slot k = l / 16; result register i of lane l is D[4 (l / 16) + i][l % 16].
// K step s of a 128-long dot product pairs slot k with element 32 k + s, so a lane's 32 operand
// values of one row are contiguous in memory.
__device__ inline f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- project (both sides)
// B = (Kbar - mu) Wk and A = Qbar Wq, fp32 [BH][rows][d] row-major (Kbar - mu is the mean of
// K_s; no weights: the identity, the heuristic router of the earlier SLA). grid
// (ceil(nkb / R) + ceil(nqb / R), BH), R = kProjRows, 256 threads: R key blocks (the first
// ceil(nkb / R) workgroups) or R query blocks per workgroup, wavefront w the output columns
// 32 w .. 32 w + 31 (R / 16 x 2 tiles of 16 x 16, K = 128 in 32 fp32 MFMA steps each); a
// lane's 64 weights stay in registers for all its tiles. Every load of a thread (block sums,
// means, weights) is issued before the first is used. (R = 32 halves the weight reads but
// measured no faster at 12 heads, N = 32768.)
constexpr int kXPad = kD + 4;
constexpr int kProjRows = 16;
__global__ __launch_bounds__(256) void project_kernel(const double* __restrict__ ksum,
                                                      const double* __restrict__ mu64,
                                                      const float* __restrict__ wk,
                                                      float* __restrict__ B,
                                                      const double* __restrict__ qsum,
                                                      const float* __restrict__ wq,
                                                      float* __restrict__ A, int nkb, int nqb,
                                                      int H) {
  __shared__ float xs[kProjRows][kXPad];
  const int bh = blockIdx.y, h = bh % H, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, ra = lane & 15, kq = lane >> 4;
  const int nkt = (nkb + kProjRows - 1) / kProjRows;
  const bool key_side = static_cast<int>(blockIdx.x) < nkt;
  const int r0 = kProjRows * (key_side ? blockIdx.x : blockIdx.x - nkt);
  const int nrow = key_side ? nkb : nqb;
  const double* src = key_side ? ksum + static_cast<size_t>(bh) * nkb * kD
                               : qsum + static_cast<size_t>(bh) * nqb * kD;
  const float* W = key_side ? wk : wq;
  float* out = key_side ? B + static_cast<size_t>(bh) * nkb * kD
                        : A + static_cast<size_t>(bh) * nqb * kD;
  float wv[2][32];
  if (W != nullptr) {
    const float* Wh = W + static_cast<size_t>(h) * kD * kD;
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int k = 32 * kq + s;
      wv[0][s] = Wh[k * kD + 32 * w + ra];
      wv[1][s] = Wh[k * kD + 32 * w + 16 + ra];
    }
  }
  constexpr int kPer = kProjRows * kD / 256;
  double xv[kPer];
  const double mu = key_side ? mu64[bh * kD + (t & 127)] : 0.0;   // column t % 128 throughout
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int r = (t + 256 * u) >> 7;
    xv[u] = r0 + r < nrow ? src[static_cast<size_t>(r0 + r) * kD + (t & 127)] : 0.0;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int r = (t + 256 * u) >> 7;
    xs[r][t & 127] = r0 + r >= nrow ? 0.f
                     : key_side     ? static_cast<float>(xv[u] * (1.0 / kBK) - mu)
                                    : static_cast<float>(xv[u] * (1.0 / kBQ));
  }
  __syncthreads();
  if (W == nullptr) {
    for (int e = t; e < kProjRows * kD; e += 256) {
      const int r = e >> 7, c = e & 127;
      if (r0 + r < nrow) out[static_cast<size_t>(r0 + r) * kD + c] = xs[r][c];
    }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < kProjRows / 16; ++rt) {
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const float x = xs[16 * rt + ra][32 * kq + s];
      acc[0] = mfma_f32(x, wv[0][s], acc[0]);
      acc[1] = mfma_f32(x, wv[1][s], acc[1]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 16 * rt + 4 * kq + i;
        if (r < nrow) out[static_cast<size_t>(r) * kD + 32 * w + 16 * u + ra] = acc[u][i];
      }
  }
}

hipError_t launch_project(const Geom& g, const double* ksum, const double* mu64, const float* wk,
                          float* B, const double* qsum, const float* wq, float* A,
                          hipStream_t s) {
  const int tiles = (g.nkb + kProjRows - 1) / kProjRows +
                    (A != nullptr ? (g.nqb + kProjRows - 1) / kProjRows : 0);
  hipLaunchKernelGGL(project_kernel, dim3(tiles, g.BH), dim3(256), 0, s, ksum, mu64, wk, B,
                     qsum, wq, A, g.nkb, g.nqb, g.H);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fill
__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, int n, float v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill(float* p, int n, float v, hipStream_t s) {
  hipLaunchKernelGGL(fill_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------- score + top-k
__device__ inline uint32_t order_key(float g) {
  // monotone map from finite floats to unsigned integers (larger g -> larger key)
  const uint32_t b = __float_as_uint(g);
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

__device__ inline int count_below_lane(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// Query-block rows one scoring workgroup handles (its logits stay in LDS as fp32, at most
// 128 KB): 16 (one full MFMA tile) up to 2048 key blocks, else 8.
__host__ __device__ inline int score_rows(int nkb) { return nkb <= 2048 ? 16 : 8; }
constexpr int kScoreThreads = 1024;   // 16 wavefronts: one row each in the selection

// The largest T with #{key >= T} >= kb, built bit by bit from the top (each count a sum of
// ballot popcounts over the wavefront's N keys per lane), stopping early once #{key >= T} is
// exactly kb. Either way #{key >= T} >= kb and no key above T is left out of the kb largest.
template <int N>
__device__ inline uint32_t kth_key(const uint32_t (&key)[N], int kb) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) c += __popcll(__ballot(key[e] >= cand));
    if (c >= kb) {
      T = cand;
      // exactly kb keys >= T: they are the kept set (no key equal to the boundary is left
      // out), and the selection below keeps exactly the keys >= T
      if (c == kb) break;
    }
  }
  return T;
}

constexpr int kCand = 256;   // candidate keys one wavefront compacts before its threshold search

// Kept set of one row, exact (ties to the lower index), by one wavefront. The row's keys
// sit in registers, E per lane (key j = lane + 64 e). T is a threshold from kth_key; every key
// > T is kept, plus the lowest-index keys equal to T up to kb.
// Candidate filter (kb <= 64, more than 256 keys): the kb-th largest of the 64 lane maxima,
// T0, is at most the kb-th largest key (those kb maxima are kb distinct keys >= T0), so every
// key that can be kept is >= T0. When at most kCand keys are, they are compacted into `cand`
// (this wavefront's LDS) and searched 4 per lane instead of E; a search result below T0 (an
// early stop with exactly kb candidates) is raised to T0, where #{key >= T0} is also kb.
template <int E>
__device__ void select_row(const float* g, int nkb, int kb, int lane, size_t row,
                           int32_t* __restrict__ list, int list_stride,
                           uint8_t* __restrict__ mask, uint32_t* cand) {
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    key[e] = j < nkb ? order_key(g[j]) : 0u;   // finite keys are >= 1
  }
  uint32_t T = 0;
  bool found = false;
  if (kb <= 64 && nkb > 256) {
    uint32_t mx[1] = {key[0]};
#pragma unroll
    for (int e = 1; e < E; ++e) mx[0] = max(mx[0], key[e]);
    const uint32_t T0 = kth_key<1>(mx, kb);
    int C = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) C += __popcll(__ballot(key[e] >= T0));
    if (C <= kCand) {
      int at = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool in = key[e] >= T0;
        const uint64_t m = __ballot(in);
        if (in) cand[at + count_below_lane(m)] = key[e];
        at += __popcll(m);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint32_t ck[kCand / 64];
#pragma unroll
      for (int u = 0; u < kCand / 64; ++u) ck[u] = lane + 64 * u < C ? cand[lane + 64 * u] : 0u;
      T = max(kth_key<kCand / 64>(ck, kb), T0);
      found = true;
    }
  }
  if (!found) T = kth_key<E>(key, kb);
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) gt += __popcll(__ballot(key[e] > T));
  const int need = kb - gt;   // >= 0: equal keys to keep, lowest indices first
  int eq_before = 0, sel_before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    const bool valid = j < nkb;
    const bool is_eq = valid && key[e] == T;
    const uint64_t eqm = __ballot(is_eq);
    const int eq_rank = eq_before + count_below_lane(eqm);
    const bool sel = valid && (key[e] > T || (is_eq && eq_rank < need));
    const uint64_t selm = __ballot(sel);
    if (sel) list[row * list_stride + sel_before + count_below_lane(selm)] = j;
    if (valid && mask) mask[row * nkb + j] = sel ? 1 : 0;
    eq_before += __popcll(eqm);
    sel_before += __popcll(selm);
  }
}

// SoftTop-k of one row (training-time router, §4 Eq. 17 of the second page): P_c = softmax(g)
// in fp64, x = P_c / tau in fp32, then lambda with f(lambda) = sum_j sigma(x_j + lambda) = kb.
// The root lies in the bracket [L - max x, L - min x], L = log(kb / (nkb - kb)) (every term is
// at most, resp. at least, kb / nkb at its ends). Safeguarded Newton in fp32, at most 16 steps from
// the uniform-row root L - 1 / (tau nkb): each step evaluates f and f' = sum sigma (1 - sigma),
// narrows the bracket at the current point, and takes the Newton step, or the bracket midpoint
// when that step leaves the bracket; it stops early once a step moves lambda by at most 1e-7
// relative (converged in fp32). Row sums are butterfly reductions (every lane holds the
// same value, fixed order: deterministic). kb = nkb gives ones and lambda = +inf. Writes
// soft[row][j] = sigma(x_j + lambda) and lam[row].
template <int E>
__device__ void soft_row(const float* g, int nkb, int kb, float inv_tau, int lane, size_t row,
                         float* __restrict__ soft, float* __restrict__ lam) {
  float x[E];
  {
    double ex[E];
    double mx = -1.0e300;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) mx = fmax(mx, static_cast<double>(g[j]));
    }
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    double sum = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      ex[e] = j < nkb ? exp(static_cast<double>(g[min(j, nkb - 1)]) - mx) : 0.0;
      sum += ex[e];
    }
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = static_cast<float>(ex[e] / sum * static_cast<double>(inv_tau));
  }
  float lv = INFINITY;
  if (kb < nkb) {
    const float L = logf(static_cast<float>(kb) / static_cast<float>(nkb - kb));
    float xmax = -INFINITY, xmin = INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (lane + 64 * e < nkb) {
        xmax = fmaxf(xmax, x[e]);
        xmin = fminf(xmin, x[e]);
      }
    for (int o = 32; o >= 1; o >>= 1) {
      xmax = fmaxf(xmax, __shfl_xor(xmax, o));
      xmin = fminf(xmin, __shfl_xor(xmin, o));
    }
    float lo = L - xmax, hi = L - xmin;
    lv = fminf(fmaxf(L - inv_tau / static_cast<float>(nkb), lo), hi);
    const float kbf = static_cast<float>(kb);
    for (int it = 0; it < 16; ++it) {
      float f = 0.f, df = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (lane + 64 * e < nkb) {
          const float sg = 1.0f / (1.0f + __expf(-(x[e] + lv)));
          f += sg;
          df = fmaf(sg, 1.0f - sg, df);
        }
      for (int o = 32; o >= 1; o >>= 1) {
        f += __shfl_xor(f, o);
        df += __shfl_xor(df, o);
      }
      const float fq = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(f)));
      const float dq = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(df)));
      if (fq < kbf) lo = lv;
      else hi = lv;
      const float nt = lv - (fq - kbf) / dq;
      const float nv = (nt > lo && nt < hi) ? nt : 0.5f * (lo + hi);
      // every lane holds the same lambda: the exit is uniform
      const bool done = fabsf(nv - lv) <= 1e-7f * fmaxf(1.0f, fabsf(lv));
      lv = nv;
      if (done) break;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    if (j < nkb) soft[row * nkb + j] = kb < nkb ? 1.0f / (1.0f + __expf(-(x[e] + lv))) : 1.0f;
  }
  if (lane == 0 && lam) lam[row] = lv;
}

// grid (ceil(nqb / RT), BH), kScoreThreads threads, RT = score_rows(nkb); dynamic LDS RT * nkb
// floats. Per workgroup: the logits G = A B^T / sqrt(d) of its RT query-block rows against
// every key block (fp32 MFMA, 16 x 16 tiles dealt to the 16 wavefronts, the next tile's B
// operands loaded during the current tile's products; a lane's A and B operands are 32
// contiguous floats of one row) into LDS, then one row per wavefront: the exact hard Top-k
// (kSoft = false: mask, ascending list, count and the optional fp32 P_c) or the SoftTop-k mask
// and lambda (kSoft). E = keys per lane held in registers (nkb <= 64 E).
template <int E, bool kSoft>
__global__ __launch_bounds__(kScoreThreads) void score_topk_kernel(
    const float* __restrict__ A, const float* __restrict__ B, int nqb, int nkb, int kb,
    uint8_t* __restrict__ mask, int32_t* __restrict__ list, int list_stride,
    int32_t* __restrict__ cnt, float* __restrict__ scores, float inv_tau,
    float* __restrict__ soft, float* __restrict__ lam) {
  extern __shared__ float G[];                        // [RT][nkb]
  __shared__ uint32_t cand[kScoreThreads / 64][kCand];
  const int RT = score_rows(nkb);
  const int bh = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int ra = lane & 15, kq = lane >> 4;
  const int i0 = blockIdx.x * RT;
  {
    const float inv_sqrt_d = 0.088388347648318440f;   // 1/sqrt(128)
    const float* Bh = B + static_cast<size_t>(bh) * nkb * kD;
    const int ntile = (nkb + 15) >> 4;
    f32x4 bv[8], bn[8], av[8];
    auto load_tile = [&](f32x4(&dst)[8], int ct) {
      const int col = min(16 * ct + ra, nkb - 1);
      const f32x4* bp = reinterpret_cast<const f32x4*>(Bh + static_cast<size_t>(col) * kD + 32 * kq);
#pragma unroll
      for (int u = 0; u < 8; ++u) dst[u] = bp[u];
    };
    if (w < ntile) load_tile(bv, w);
    // this lane's A operand: row i0 + ra (zero past RT or nqb), elements 32 kq .. 32 kq + 31
    const int ia = i0 + ra;
    if (ra < RT && ia < nqb) {
      const f32x4* ap = reinterpret_cast<const f32x4*>(A + (static_cast<size_t>(bh) * nqb + ia) * kD + 32 * kq);
#pragma unroll
      for (int u = 0; u < 8; ++u) av[u] = ap[u];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) av[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int ct = w; ct < ntile; ct += kScoreThreads / 64) {
      if (ct + kScoreThreads / 64 < ntile) load_tile(bn, ct + kScoreThreads / 64);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 32; ++s) acc = mfma_f32(av[s >> 2][s & 3], bv[s >> 2][s & 3], acc);
      const int col = 16 * ct + ra;
      if (col < nkb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * kq + i;
          if (r < RT) G[r * nkb + col] = acc[i] * inv_sqrt_d + 0.0f;   // +0: no -0
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) bv[u] = bn[u];
    }
  }
  __syncthreads();
  const int r = w;
  const int i = i0 + r;
  if (r >= RT || i >= nqb) return;
  const float* g = G + r * nkb;
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  if constexpr (kSoft) {
    soft_row<E>(g, nkb, kb, inv_tau, lane, row, soft, lam);
    return;
  }
  select_row<E>(g, nkb, kb, lane, row, list, list_stride, mask, cand[w]);
  if (lane == 0 && cnt) cnt[row] = kb;
  if (scores) {
    const int nE = (nkb + 63) >> 6;
    double mx = -1.0e300;
    for (int e = 0; e < nE; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) mx = fmax(mx, static_cast<double>(g[j]));
    }
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    double sum = 0.0;
    for (int e = 0; e < nE; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) sum += exp(static_cast<double>(g[j]) - mx);
    }
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    for (int e = 0; e < nE; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) scores[row * nkb + j] = static_cast<float>(exp(static_cast<double>(g[j]) - mx) / sum);
    }
  }
}

hipError_t configure_router() {
  // largest dynamic LDS: RT * nkb floats = 128 KB at the top of every RT class
  const void* fns[] = {reinterpret_cast<const void*>(&score_topk_kernel<8, false>),
                       reinterpret_cast<const void*>(&score_topk_kernel<16, false>),
                       reinterpret_cast<const void*>(&score_topk_kernel<32, false>),
                       reinterpret_cast<const void*>(&score_topk_kernel<64, false>),
                       reinterpret_cast<const void*>(&score_topk_kernel<8, true>),
                       reinterpret_cast<const void*>(&score_topk_kernel<16, true>),
                       reinterpret_cast<const void*>(&score_topk_kernel<32, true>),
                       reinterpret_cast<const void*>(&score_topk_kernel<64, true>)};
  for (const void* f : fns) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             32 * 1024 * 4);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool kSoft>
static void launch_score_t(const Geom& g, const float* A, const float* B, int kb, uint8_t* mask,
                           int32_t* list, int list_stride, int32_t* cnt, float* scores,
                           float inv_tau, float* soft, float* lam, hipStream_t s) {
  const int RT = score_rows(g.nkb);
  dim3 grid((g.nqb + RT - 1) / RT, g.BH);
  const size_t lds = static_cast<size_t>(RT) * g.nkb * sizeof(float);
  const int E = (g.nkb + 63) / 64;
#define SLA2_SCORE(EE)                                                                        \
  hipLaunchKernelGGL((score_topk_kernel<EE, kSoft>), grid, dim3(kScoreThreads), lds, s, A, B, \
                     g.nqb, g.nkb, kb, mask, list, list_stride, cnt, scores, inv_tau, soft,   \
                     lam)
  if (E <= 8) SLA2_SCORE(8);
  else if (E <= 16) SLA2_SCORE(16);
  else if (E <= 32) SLA2_SCORE(32);
  else SLA2_SCORE(64);
#undef SLA2_SCORE
}

hipError_t launch_score_topk(const Geom& g, const float* A, const float* B, int kb,
                             uint8_t* mask, int32_t* list, int list_stride, int32_t* cnt,
                             float* scores, hipStream_t s) {
  launch_score_t<false>(g, A, B, kb, mask, list, list_stride, cnt, scores, 0.f, nullptr, nullptr,
                        s);
  return hipGetLastError();
}

hipError_t launch_score_soft(const Geom& g, const float* A, const float* B, int kb,
                             float inv_tau, float* soft, float* lam, hipStream_t s) {
  launch_score_t<true>(g, A, B, kb, nullptr, nullptr, 0, nullptr, nullptr, inv_tau, soft, lam, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- external mask -> lists
// grid (nqb, BH), 64 threads: one wavefront compacts one mask row (any byte != 0 is 1).
__global__ __launch_bounds__(64) void mask_to_list_kernel(const uint8_t* __restrict__ mask_in,
                                                          uint8_t* __restrict__ mask_out,
                                                          int32_t* __restrict__ list,
                                                          int32_t* __restrict__ cnt, int nqb,
                                                          int nkb) {
  const size_t row = static_cast<size_t>(blockIdx.y) * nqb + blockIdx.x;
  const int lane = threadIdx.x;
  int before = 0;
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const int j = j0 + lane;
    const bool sel = j < nkb && mask_in[row * nkb + j] != 0;
    const uint64_t m = __ballot(sel);
    if (sel) list[row * nkb + before + count_below_lane(m)] = j;
    if (j < nkb) mask_out[row * nkb + j] = sel ? 1 : 0;
    before += __popcll(m);
  }
  if (lane == 0) cnt[row] = before;
}

hipError_t launch_mask_to_list(const Geom& g, const uint8_t* mask_in, uint8_t* mask_out,
                               int32_t* list, int32_t* cnt, hipStream_t s) {
  hipLaunchKernelGGL(mask_to_list_kernel, dim3(g.nqb, g.BH), dim3(64), 0, s, mask_in, mask_out,
                     list, cnt, g.nqb, g.nkb);
  return hipGetLastError();
}

}  // namespace sla2
