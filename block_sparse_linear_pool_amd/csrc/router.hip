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
//   project     A = Qbar Wq, B = (Kbar - mu) Wk in fp64 (Kbar - mu is the mean of K_s); with
//               no weights the identity (the heuristic router of the earlier SLA).
//   score_topk  G = A B^T / sqrt(d) in fp64 into LDS, then one wavefront per query
//               block selects the kb largest logits exactly (ties to the lower index)
//               and writes the mask and the ascending block list; in its soft mode the
//               SoftTop-k mask sigma(P_c / tau + lambda_i) of the training-time router.
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
// grid (8, BH), 256 threads: workgroup x takes columns 16 x .. 16 x + 15 of head bh; thread t
// sums column 16 x + t % 16 over key blocks t / 16, t / 16 + 16, ... with four accumulators
// (four loads in flight); the 16 partial sums are combined in a fixed order (deterministic).
__global__ __launch_bounds__(256) void colmean_kernel(const double* __restrict__ ksum,
                                                      double* __restrict__ mu64,
                                                      float* __restrict__ mu32,
                                                      float* __restrict__ mu32_tap, int nkb,
                                                      int N) {
  __shared__ double part[16][17];
  const int bh = blockIdx.y, t = threadIdx.x, c = 16 * blockIdx.x + (t & 15), sl = t >> 4;
  const double* p = ksum + static_cast<size_t>(bh) * nkb * kD + c;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int j = sl;
  for (; j + 48 < nkb; j += 64) {
    a0 += p[static_cast<size_t>(j) * kD];
    a1 += p[static_cast<size_t>(j + 16) * kD];
    a2 += p[static_cast<size_t>(j + 32) * kD];
    a3 += p[static_cast<size_t>(j + 48) * kD];
  }
  for (; j < nkb; j += 16) a0 += p[static_cast<size_t>(j) * kD];
  part[sl][t & 15] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (t < 16) {
    double s = 0.0;
    for (int q = 0; q < 16; ++q) s += part[q][t];
    const double mu = s / static_cast<double>(N);
    mu64[bh * kD + c] = mu;
    mu32[bh * kD + c] = static_cast<float>(mu);
    if (mu32_tap) mu32_tap[bh * kD + c] = static_cast<float>(mu);
  }
}

hipError_t launch_colmean(const Geom& g, const double* ksum, double* mu64, float* mu32,
                          float* mu32_tap, hipStream_t s) {
  hipLaunchKernelGGL(colmean_kernel, dim3(kD / 16, g.BH), dim3(256), 0, s, ksum, mu64, mu32,
                     mu32_tap, g.nkb, g.N);
  return hipGetLastError();
}

// fp64 MFMA 16x16x4 operand/result layout (gfx950): lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; result register i of lane l is D[l / 16 + 4 i][l % 16].
__device__ inline f64x4 mfma_f64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- project
// grid (ceil(nqb/16) + ceil(nkb/16), BH), 256 threads. A workgroup takes 16 rows of either
// Qbar (W = proj_q) or Kbar - mu (W = proj_k); wavefront w the 16x16 fp64 MFMA output tiles
// of columns 32 w .. 32 w + 31, the two K = 128 chains interleaved, all W values of both
// tiles loaded up front.
constexpr int kXPad = kD + 1;
__global__ __launch_bounds__(256) void project_kernel(
    const double* __restrict__ qsum, const double* __restrict__ ksum,
    const double* __restrict__ mu64, const float* __restrict__ wq, const float* __restrict__ wk,
    double* __restrict__ A, double* __restrict__ Bt, int nqb, int nkb, int H, int identity) {
  __shared__ double xs[16][kXPad];
  const int bh = blockIdx.y, h = bh % H, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int qwg = (nqb + 15) / 16;
  const bool is_q = static_cast<int>(blockIdx.x) < qwg;
  const int r0 = 16 * (is_q ? blockIdx.x : blockIdx.x - qwg);
  const int nrows = is_q ? nqb : nkb;
  const double* src = is_q ? qsum + static_cast<size_t>(bh) * nqb * kD
                           : ksum + static_cast<size_t>(bh) * nkb * kD;
  const double scale = is_q ? 1.0 / kBQ : 1.0 / kBK;
  for (int e = t; e < 16 * kD; e += 256) {
    const int r = e >> 7, c = e & 127;
    double v = 0.0;
    if (r0 + r < nrows) {
      v = src[static_cast<size_t>(r0 + r) * kD + c] * scale;
      if (!is_q) v -= mu64[bh * kD + c];
    }
    xs[r][c] = v;
  }
  if (identity) {
    // proj_q = proj_k = I (the heuristic router of the earlier SLA): A = Qbar, B = Kbar - mu
    __syncthreads();
    for (int e = t; e < 16 * kD; e += 256) {
      const int r = e >> 7, c = e & 127;
      if (r0 + r >= nrows) continue;
      if (is_q) A[(static_cast<size_t>(bh) * nqb + r0 + r) * kD + c] = xs[r][c];
      else Bt[(static_cast<size_t>(bh) * kD + c) * nkb + r0 + r] = xs[r][c];
    }
    return;
  }
  const float* W = (is_q ? wq : wk) + static_cast<size_t>(h) * kD * kD;
  const int ra = lane & 15, kq = lane >> 4;
  float wv[2][32];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int s = 0; s < 32; ++s) wv[u][s] = W[(4 * s + kq) * kD + 32 * w + 16 * u + ra];
  __syncthreads();
  f64x4 acc[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const double x = xs[ra][4 * s + kq];
    acc[0] = mfma_f64(x, static_cast<double>(wv[0][s]), acc[0]);
    acc[1] = mfma_f64(x, static_cast<double>(wv[1][s]), acc[1]);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int col = 32 * w + 16 * u + ra;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + kq + 4 * i;
      if (r >= nrows) continue;
      if (is_q) A[(static_cast<size_t>(bh) * nqb + r) * kD + col] = acc[u][i];
      else Bt[(static_cast<size_t>(bh) * kD + col) * nkb + r] = acc[u][i];
    }
  }
}

hipError_t launch_project(const Geom& g, const double* qsum, const double* ksum,
                          const double* mu64, const float* wq, const float* wk, double* A,
                          double* Bt, hipStream_t s) {
  dim3 grid((g.nqb + 15) / 16 + (g.nkb + 15) / 16, g.BH);
  hipLaunchKernelGGL(project_kernel, grid, dim3(256), 0, s, qsum, ksum, mu64, wq, wk, A, Bt,
                     g.nqb, g.nkb, g.H, wq == nullptr ? 1 : 0);
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
__device__ inline uint64_t order_key(double g) {
  // monotone map from finite doubles to unsigned integers (larger g -> larger key)
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(g));
  return (b >> 63) ? ~b : (b | (1ull << 63));
}

__device__ inline int count_below_lane(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// Rows of logits one workgroup keeps in LDS (fp64), by key-block count.
// Eight rows (two per wavefront in the selection) keep enough workgroups in flight; the logit
// tiles are 16 rows tall, the other 8 zero.
__host__ __device__ inline int score_rows(int nkb) { return nkb <= 2048 ? 8 : 4; }

// Kept set of one row, exact (ties to the lower index), by one wavefront. The row's keys
// sit in registers, E per lane (key j = lane + 64 e). T is built bit by bit from the top as
// the largest T with #{key >= T} >= kb (the kb-th largest key), each count a sum of ballot
// popcounts, stopping early once #{key >= T} is exactly kb. Then every key > T is kept, plus
// the lowest-index keys equal to T up to kb.
template <int E>
__device__ void select_row(const double* g, int nkb, int kb, int lane, size_t row,
                           int32_t* __restrict__ list, int list_stride,
                           uint8_t* __restrict__ mask) {
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    key[e] = j < nkb ? order_key(g[j]) : 0ull;   // finite keys are >= 1
  }
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
    if (c >= kb) {
      T = cand;
      // exactly kb keys >= T: they are the kept set (no key equal to the boundary is left
      // out), and the code below keeps exactly the keys >= T
      if (c == kb) break;
    }
  }
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) gt += __popcll(__ballot(key[e] > T));
  const int need = kb - gt;   // >= 1: equal keys to keep, lowest indices first
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

// SoftTop-k of rows (training-time router, §4 Eq. 17 of the second page), two rows per
// wavefront at once (their reductions overlap): P_c = softmax(g) in fp64, x = P_c / tau in
// fp32, then lambda with f(lambda) = sum_j sigma(x_j + lambda) = kb. The root lies in the
// bracket [L - max x, L - min x], L = log(kb / (nkb - kb)) (every term is at most, resp. at
// least, kb / nkb at its ends). Safeguarded Newton in fp32, 16 steps from the uniform-row
// root L - 1 / (tau nkb): each step evaluates f and f' = sum sigma (1 - sigma), narrows the
// bracket at the current point, and takes the Newton step, or the bracket midpoint when that
// step leaves the bracket. Row sums are butterfly reductions (every lane holds the same
// value, fixed order: deterministic). kb = nkb gives ones and lambda = +inf. Writes
// soft[row][j] = sigma(x_j + lambda) and lam[row]; `valid[q]` false skips row q's writes.
template <int E>
__device__ void soft_rows(const double* const (&g)[2], const bool (&valid)[2], int nkb, int kb,
                          float inv_tau, int lane, const size_t (&row)[2],
                          float* __restrict__ soft, float* __restrict__ lam) {
  float x[2][E];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    double ex[E];
    double mx = -1.0e300;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb) mx = fmax(mx, g[q][j]);
    }
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    double sum = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      ex[e] = j < nkb ? exp(g[q][min(j, nkb - 1)] - mx) : 0.0;
      sum += ex[e];
    }
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
#pragma unroll
    for (int e = 0; e < E; ++e)
      x[q][e] = static_cast<float>(ex[e] / sum * static_cast<double>(inv_tau));
  }
  float lv[2] = {INFINITY, INFINITY};
  if (kb < nkb) {
    float lo[2], hi[2];
    const float L = logf(static_cast<float>(kb) / static_cast<float>(nkb - kb));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float xmax = -INFINITY, xmin = INFINITY;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (lane + 64 * e < nkb) {
          xmax = fmaxf(xmax, x[q][e]);
          xmin = fminf(xmin, x[q][e]);
        }
      for (int o = 32; o >= 1; o >>= 1) {
        xmax = fmaxf(xmax, __shfl_xor(xmax, o));
        xmin = fminf(xmin, __shfl_xor(xmin, o));
      }
      lo[q] = L - xmax;
      hi[q] = L - xmin;
      lv[q] = fminf(fmaxf(L - inv_tau / static_cast<float>(nkb), lo[q]), hi[q]);
    }
    const float kbf = static_cast<float>(kb);
    for (int it = 0; it < 16; ++it) {
      float f[2], df[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        f[q] = 0.f;
        df[q] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (lane + 64 * e < nkb) {
            const float sg = 1.0f / (1.0f + __expf(-(x[q][e] + lv[q])));
            f[q] += sg;
            df[q] = fmaf(sg, 1.0f - sg, df[q]);
          }
      }
      for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          f[q] += __shfl_xor(f[q], o);
          df[q] += __shfl_xor(df[q], o);
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float fq = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(f[q])));
        const float dq = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(df[q])));
        if (fq < kbf) lo[q] = lv[q];
        else hi[q] = lv[q];
        const float nt = lv[q] - (fq - kbf) / dq;
        lv[q] = (nt > lo[q] && nt < hi[q]) ? nt : 0.5f * (lo[q] + hi[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (!valid[q]) continue;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < nkb)
        soft[row[q] * nkb + j] = kb < nkb ? 1.0f / (1.0f + __expf(-(x[q][e] + lv[q]))) : 1.0f;
    }
    if (lane == 0 && lam) lam[row[q]] = lv[q];
  }
}

// grid (ceil(nqb / RT), BH), 256 threads, RT = score_rows(nkb); dynamic LDS RT * nkb doubles.
// E = keys per lane held in registers (nkb <= 64 E). kSoft: the SoftTop-k mask and lambda
// (soft, lam, inv_tau) instead of the hard selection.
template <int E, bool kSoft>
__global__ __launch_bounds__(256) void score_topk_kernel(
    const double* __restrict__ A, const double* __restrict__ Bt, int nqb, int nkb, int kb,
    uint8_t* __restrict__ mask, int32_t* __restrict__ list, int list_stride,
    int32_t* __restrict__ cnt, float* __restrict__ scores, float inv_tau,
    float* __restrict__ soft, float* __restrict__ lam) {
  extern __shared__ double G[];                 // [RT][nkb]
  __shared__ double as[16][kXPad];
  const int RT = score_rows(nkb);
  const int bh = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int i0 = blockIdx.x * RT;
  for (int e = t; e < 16 * kD; e += 256) {
    const int r = e >> 7, k = e & 127;
    const int i = i0 + r;
    as[r][k] = (r < RT && i < nqb) ? A[(static_cast<size_t>(bh) * nqb + i) * kD + k] : 0.0;
  }
  __syncthreads();
  // logits: 16-column fp64 MFMA tiles, round-robin over the wavefronts
  const double inv_sqrt_d = 0.088388347648318440550;  // 1/sqrt(128)
  const double* bt = Bt + static_cast<size_t>(bh) * kD * nkb;
  const int ntile = (nkb + 15) >> 4, ra = lane & 15, kq = lane >> 4;
  // This wavefront's column tiles ct = w, w + 4, ...; step q = tile q / 2, k half q % 2. The B
  // values of step q + 1 load while step q multiplies (two register buffers); loads are
  // unconditional at clamped addresses and masked in the product.
  const int nsteps = 2 * ((ntile - w + 3) / 4);
  auto bload = [&](double (&dst)[16], int q) {
    const int qc = min(q, nsteps - 1);
    const int col = min(16 * (w + 4 * (qc >> 1)) + ra, nkb - 1);
    const double* bc = bt + col + static_cast<size_t>(64 * (qc & 1) + kq) * nkb;
#pragma unroll
    for (int s = 0; s < 16; ++s) dst[s] = bc[static_cast<size_t>(4 * s) * nkb];
  };
  if (nsteps > 0) {
    double bb[2][16];
    bload(bb[0], 0);
    f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
    for (int q0 = 0; q0 < nsteps; q0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {   // u = k half of step q0 + u
        bload(bb[u ^ 1], q0 + u + 1);
        const int col = 16 * (w + 4 * (q0 >> 1)) + ra;
        const bool ok = col < nkb;
        if (u == 0) acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s = 0; s < 16; ++s)
          acc = mfma_f64(as[ra][4 * (16 * u + s) + kq], ok ? bb[u][s] : 0.0, acc);
        if (u == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = kq + 4 * i;
            if (ok && r < RT) G[r * nkb + col] = acc[i] * inv_sqrt_d + 0.0;  // +0.0: no -0
          }
        }
      }
    }
  }
  __syncthreads();
  const int nE = (nkb + 63) >> 6;
  for (int r = w; r < RT; r += 4) {
    const int i = i0 + r;
    if (i >= nqb) break;
    const double* g = G + r * nkb;
    const size_t row = static_cast<size_t>(bh) * nqb + i;
    if constexpr (kSoft) {
      // rows r and r + 4 together (the second only when it exists)
      const int r2 = r + 4;
      const bool v2 = r2 < RT && i0 + r2 < nqb;
      const double* const gq[2] = {g, G + (v2 ? r2 : r) * nkb};
      const bool vq[2] = {true, v2};
      const size_t rq[2] = {row, row + (v2 ? 4 : 0)};
      soft_rows<E>(gq, vq, nkb, kb, inv_tau, lane, rq, soft, lam);
      if (RT > 4) break;   // this wavefront's rows are done (RT <= 8)
      continue;
    }
    select_row<E>(g, nkb, kb, lane, row, list, list_stride, mask);
    if (lane == 0 && cnt) cnt[row] = kb;
    if (scores) {
      double mx = -1.0e300;
      for (int e = 0; e < nE; ++e) {
        const int j = lane + 64 * e;
        if (j < nkb) mx = fmax(mx, g[j]);
      }
      for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
      double sum = 0.0;
      for (int e = 0; e < nE; ++e) {
        const int j = lane + 64 * e;
        if (j < nkb) sum += exp(g[j] - mx);
      }
      for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
      for (int e = 0; e < nE; ++e) {
        const int j = lane + 64 * e;
        if (j < nkb) scores[row * nkb + j] = static_cast<float>(exp(g[j] - mx) / sum);
      }
    }
  }
}

hipError_t configure_router() {
  // largest dynamic LDS: RT * nkb doubles = 128 KB at the top of every RT class
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
                                             16 * 1024 * 8);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool kSoft>
static void launch_score_t(const Geom& g, const double* A, const double* Bt, int kb, uint8_t* mask,
                           int32_t* list, int list_stride, int32_t* cnt, float* scores,
                           float inv_tau, float* soft, float* lam, hipStream_t s) {
  const int RT = score_rows(g.nkb);
  dim3 grid((g.nqb + RT - 1) / RT, g.BH);
  const size_t lds = static_cast<size_t>(RT) * g.nkb * sizeof(double);
  const int E = (g.nkb + 63) / 64;
  if (E <= 8)
    hipLaunchKernelGGL((score_topk_kernel<8, kSoft>), grid, dim3(256), lds, s, A, Bt, g.nqb, g.nkb,
                       kb, mask, list, list_stride, cnt, scores, inv_tau, soft, lam);
  else if (E <= 16)
    hipLaunchKernelGGL((score_topk_kernel<16, kSoft>), grid, dim3(256), lds, s, A, Bt, g.nqb,
                       g.nkb, kb, mask, list, list_stride, cnt, scores, inv_tau, soft, lam);
  else if (E <= 32)
    hipLaunchKernelGGL((score_topk_kernel<32, kSoft>), grid, dim3(256), lds, s, A, Bt, g.nqb,
                       g.nkb, kb, mask, list, list_stride, cnt, scores, inv_tau, soft, lam);
  else
    hipLaunchKernelGGL((score_topk_kernel<64, kSoft>), grid, dim3(256), lds, s, A, Bt, g.nqb,
                       g.nkb, kb, mask, list, list_stride, cnt, scores, inv_tau, soft, lam);
}

hipError_t launch_score_topk(const Geom& g, const double* A, const double* Bt, int kb,
                             uint8_t* mask, int32_t* list, int list_stride, int32_t* cnt,
                             float* scores, hipStream_t s) {
  launch_score_t<false>(g, A, Bt, kb, mask, list, list_stride, cnt, scores, 0.f, nullptr,
                        nullptr, s);
  return hipGetLastError();
}

hipError_t launch_score_soft(const Geom& g, const double* A, const double* Bt, int kb,
                             float inv_tau, float* soft, float* lam, hipStream_t s) {
  launch_score_t<true>(g, A, Bt, kb, nullptr, nullptr, 0, nullptr, nullptr, inv_tau, soft, lam,
                       s);
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
