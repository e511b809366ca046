// SLA2 router (step 1 of the computation flow on the summary page "SLA2: Sparse-Linear
// Attention with Learnable Routing and QAT", paper.rainbus.top; "Router" box of the §3
// flowchart of "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers"):
// mean-pool Q (128 rows) and the smoothed K (64 rows), project with proj_q / proj_k,
// score every block pair, keep the top kb key blocks of every query block.
//
// Kernels, in launch order:
//   pool        one pass over Q and K (HBM-bound): fp64 block sums of Q and K.
//   colmean     mu = colmean(K) from the key-block sums (all blocks have 64 rows), the
//               K smoothing of §7 note 1 of the second page.
//   project     A = Qbar Wq, B = (Kbar - mu) Wk in fp64 (Kbar - mu is the mean of K_s).
//   score_topk  G = A B^T / sqrt(d) in fp64 into LDS, then one wavefront per query
//               block selects the kb largest logits exactly (ties to the lower index)
//               and writes the mask and the ascending block list.
// Ranking by the logit G is ranking by P_c = softmax(G): softmax is monotone per row.
#include "sla2_common.h"

namespace sla2 {

// ---------------------------------------------------------------- pool
// grid (nqb, BH), 256 threads. Thread t: 8 columns starting at 8*(t%16), rows t/16 + 16m.
template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ Q,
                                                   const T* __restrict__ K,
                                                   double* __restrict__ qsum,
                                                   double* __restrict__ ksum, int N) {
  __shared__ double red[3][16][kD + 2];
  const int i = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int cg = t & 15, rl = t >> 4;
  const size_t base = (static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ) * kD;
  double aq[8] = {}, ak0[8] = {}, ak1[8] = {};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const size_t off = base + static_cast<size_t>(rl + 16 * m) * kD + 8 * cg;
    float v[8];
    if (Q != nullptr) {
      load8<T>(Q + off, v);
#pragma unroll
      for (int c = 0; c < 8; ++c) aq[c] += static_cast<double>(v[c]);
    }
    load8<T>(K + off, v);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (m < 4) ak0[c] += static_cast<double>(v[c]);
      else ak1[c] += static_cast<double>(v[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    red[0][rl][8 * cg + c] = aq[c];
    red[1][rl][8 * cg + c] = ak0[c];
    red[2][rl][8 * cg + c] = ak1[c];
  }
  __syncthreads();
  // threads 0..127: Q column t; 128..255: first key block column t-128; then second.
  {
    const int which = t >> 7, c = t & 127;
    double s = 0.0;
    for (int r = 0; r < 16; ++r) s += red[which][r][c];
    if (which == 0) {
      if (Q != nullptr) qsum[(static_cast<size_t>(bh) * (N / kBQ) + i) * kD + c] = s;
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

hipError_t launch_pool(const Geom& g, int dtype, const void* Q, const void* K, double* qsum,
                       double* ksum, hipStream_t s) {
  dim3 grid(g.nqb, g.BH);
  if (dtype == 0)
    hipLaunchKernelGGL(pool_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(Q), static_cast<const float*>(K), qsum, ksum,
                       g.N);
  else
    hipLaunchKernelGGL(pool_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K), qsum,
                       ksum, g.N);
  return hipGetLastError();
}

// ---------------------------------------------------------------- colmean
// grid BH, 128 threads (one per column). Eight interleaved fp64 partial sums.
__global__ __launch_bounds__(128) void colmean_kernel(const double* __restrict__ ksum,
                                                      double* __restrict__ mu64,
                                                      float* __restrict__ mu32,
                                                      float* __restrict__ mu32_tap, int nkb,
                                                      int N) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const double* p = ksum + static_cast<size_t>(bh) * nkb * kD + c;
  double part[8] = {};
  int j = 0;
  for (; j + 8 <= nkb; j += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) part[u] += p[static_cast<size_t>(j + u) * kD];
  }
  for (; j < nkb; ++j) part[0] += p[static_cast<size_t>(j) * kD];
  double s = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
  const double mu = s / static_cast<double>(N);
  mu64[bh * kD + c] = mu;
  mu32[bh * kD + c] = static_cast<float>(mu);
  if (mu32_tap) mu32_tap[bh * kD + c] = static_cast<float>(mu);
}

hipError_t launch_colmean(const Geom& g, const double* ksum, double* mu64, float* mu32,
                          float* mu32_tap, hipStream_t s) {
  hipLaunchKernelGGL(colmean_kernel, dim3(g.BH), dim3(128), 0, s, ksum, mu64, mu32, mu32_tap,
                     g.nkb, g.N);
  return hipGetLastError();
}

// ---------------------------------------------------------------- project
// grid (ceil((nqb + nkb) / 16), BH), 128 threads (one per output column).
// Rows [0, nqb) are query blocks, [nqb, nqb + nkb) key blocks.
constexpr int kProjRows = 16;
__global__ __launch_bounds__(128) void project_kernel(
    const double* __restrict__ qsum, const double* __restrict__ ksum,
    const double* __restrict__ mu64, const float* __restrict__ wq, const float* __restrict__ wk,
    double* __restrict__ A, double* __restrict__ Bt, int nqb, int nkb, int H) {
  __shared__ double x[kProjRows][kD];
  const int bh = blockIdx.y, h = bh % H, c = threadIdx.x;
  const int r0 = blockIdx.x * kProjRows;
  const int total = nqb + nkb;
  const double mu = mu64[bh * kD + c];
  for (int r = 0; r < kProjRows; ++r) {
    const int rr = r0 + r;
    double v = 0.0;
    if (rr < nqb) v = qsum[(static_cast<size_t>(bh) * nqb + rr) * kD + c] * (1.0 / kBQ);
    else if (rr < total)
      v = ksum[(static_cast<size_t>(bh) * nkb + (rr - nqb)) * kD + c] * (1.0 / kBK) - mu;
    x[r][c] = v;
  }
  __syncthreads();
  // Two passes when the chunk straddles query and key rows: W differs.
  double acc[kProjRows];
#pragma unroll
  for (int r = 0; r < kProjRows; ++r) acc[r] = 0.0;
  const bool any_q = r0 < nqb;
  const bool any_k = r0 + kProjRows > nqb && r0 < total;
  for (int pass = 0; pass < 2; ++pass) {
    if ((pass == 0 && !any_q) || (pass == 1 && !any_k)) continue;
    const float* W = (pass == 0 ? wq : wk) + static_cast<size_t>(h) * kD * kD + c;
    double a2[kProjRows];
#pragma unroll
    for (int r = 0; r < kProjRows; ++r) a2[r] = 0.0;
    for (int k = 0; k < kD; ++k) {
      const double w = static_cast<double>(W[k * kD]);
#pragma unroll
      for (int r = 0; r < kProjRows; ++r) a2[r] = fma(x[r][k], w, a2[r]);
    }
#pragma unroll
    for (int r = 0; r < kProjRows; ++r) {
      const int rr = r0 + r;
      const bool is_q = rr < nqb;
      if ((pass == 0) == is_q) acc[r] = a2[r];
    }
  }
#pragma unroll
  for (int r = 0; r < kProjRows; ++r) {
    const int rr = r0 + r;
    if (rr < nqb) A[(static_cast<size_t>(bh) * nqb + rr) * kD + c] = acc[r];
    else if (rr < total) Bt[(static_cast<size_t>(bh) * kD + c) * nkb + (rr - nqb)] = acc[r];
  }
}

hipError_t launch_project(const Geom& g, const double* qsum, const double* ksum,
                          const double* mu64, const float* wq, const float* wk, double* A,
                          double* Bt, hipStream_t s) {
  dim3 grid((g.nqb + g.nkb + kProjRows - 1) / kProjRows, g.BH);
  hipLaunchKernelGGL(project_kernel, grid, dim3(128), 0, s, qsum, ksum, mu64, wq, wk, A, Bt,
                     g.nqb, g.nkb, g.H);
  return hipGetLastError();
}

// ---------------------------------------------------------------- score + top-k
constexpr int kScoreRows = 4;  // query blocks per workgroup, one per wavefront

__device__ inline uint64_t order_key(double g) {
  // monotone map from finite doubles to unsigned integers (larger g -> larger key)
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(g));
  return (b >> 63) ? ~b : (b | (1ull << 63));
}

__device__ inline int count_below_lane(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// grid (ceil(nqb / 4), BH), 256 threads; dynamic LDS kScoreRows * nkb doubles.
__global__ __launch_bounds__(256) void score_topk_kernel(
    const double* __restrict__ A, const double* __restrict__ Bt, int nqb, int nkb, int kb,
    uint8_t* __restrict__ mask, int32_t* __restrict__ list, int list_stride,
    int32_t* __restrict__ cnt, float* __restrict__ scores) {
  extern __shared__ double smem[];
  __shared__ double arow[kScoreRows][kD];
  double* G = smem;  // [kScoreRows][nkb]
  const int bh = blockIdx.y, t = threadIdx.x;
  const int i0 = blockIdx.x * kScoreRows;
  for (int e = t; e < kScoreRows * kD; e += 256) {
    const int r = e / kD, k = e % kD;
    const int i = i0 + r;
    arow[r][k] = i < nqb ? A[(static_cast<size_t>(bh) * nqb + i) * kD + k] : 0.0;
  }
  __syncthreads();
  const double inv_sqrt_d = 0.088388347648318440550;  // 1/sqrt(128)
  const double* bt = Bt + static_cast<size_t>(bh) * kD * nkb;
  for (int j = t; j < nkb; j += 256) {
    double acc[kScoreRows] = {};
    for (int k = 0; k < kD; ++k) {
      const double b = bt[static_cast<size_t>(k) * nkb + j];
#pragma unroll
      for (int r = 0; r < kScoreRows; ++r) acc[r] = fma(arow[r][k], b, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kScoreRows; ++r) G[r * nkb + j] = acc[r] * inv_sqrt_d + 0.0;
  }
  __syncthreads();

  const int w = t >> 6, lane = t & 63;
  const int i = i0 + w;
  if (i >= nqb) return;
  const double* g = G + w * nkb;
  const int E = (nkb + 63) >> 6;
  // kb-th largest key by bitwise construction: largest T with #{key >= T} >= kb
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = T | (1ull << bit);
    int c = 0;
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      const uint64_t key = j < nkb ? order_key(g[j]) : 0ull;
      c += __popcll(__ballot(key >= cand));
    }
    if (c >= kb) T = cand;
  }
  int gt = 0;
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    const uint64_t key = j < nkb ? order_key(g[j]) : 0ull;
    gt += __popcll(__ballot(key > T));
  }
  const int need = kb - gt;  // equal keys to take, lowest indices first
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  int eq_before = 0, sel_before = 0;
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    const uint64_t key = j < nkb ? order_key(g[j]) : 0ull;
    const uint64_t eqm = __ballot(j < nkb && key == T);
    const bool is_eq = j < nkb && key == T;
    const int eq_rank = eq_before + count_below_lane(eqm);
    const bool sel = j < nkb && (key > T || (is_eq && eq_rank < need));
    const uint64_t selm = __ballot(sel);
    if (sel) list[row * list_stride + sel_before + count_below_lane(selm)] = j;
    if (j < nkb && mask) mask[row * nkb + j] = sel ? 1 : 0;
    eq_before += __popcll(eqm);
    sel_before += __popcll(selm);
  }
  if (lane == 0 && cnt) cnt[row] = kb;
  if (scores) {
    double mx = -1.0e300;
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) mx = fmax(mx, g[j]);
    }
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    double sum = 0.0;
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) sum += exp(g[j] - mx);
    }
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) scores[row * nkb + j] = static_cast<float>(exp(g[j] - mx) / sum);
    }
  }
}

hipError_t configure_router() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&score_topk_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             kScoreRows * (kMaxN / kBK) * static_cast<int>(sizeof(double)));
}

hipError_t launch_score_topk(const Geom& g, const double* A, const double* Bt, int kb,
                             uint8_t* mask, int32_t* list, int list_stride, int32_t* cnt,
                             float* scores, hipStream_t s) {
  dim3 grid((g.nqb + kScoreRows - 1) / kScoreRows, g.BH);
  const size_t lds = static_cast<size_t>(kScoreRows) * g.nkb * sizeof(double);
  hipLaunchKernelGGL(score_topk_kernel, grid, dim3(256), lds, s, A, Bt, g.nqb, g.nkb, kb, mask,
                     list, list_stride, cnt, scores);
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
