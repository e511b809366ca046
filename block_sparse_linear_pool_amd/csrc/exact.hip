// The unquantised sparse branch (SLA2_QUANT_NONE): softmax attention of each query block over
// the keys of its kept key blocks, with fp32 operands throughout (step 2 of the computation
// flow on the summary page "SLA2: Sparse-Linear Attention with Learnable Routing and QAT",
// without its quantisation; the masked softmax of the "Sparse Branch" box of the §3 flowchart
// of "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers", masked logits -inf, which
// makes its Eq. 9 exact). K is smoothed as in the low-bit path: K_s = fl32(K - mu32) (§7 note 1).
//
// It runs after the attention kernel has run its linear branch alone (O = (1 - alpha) O_l) and
// adds alpha O_s to O. The reference form of the branch, not the fast one: one workgroup per
// query block, fp32 MFMA 32x32x2 (exact fp32 products, fp32 accumulation).
//
// Wavefront w owns queries 32 w .. 32 w + 31 (lane: query 32 w + lane % 32). For each kept
// key block j in ascending order: the block's K_s and V rows are staged in LDS as fp32;
//   S^T = K_s Q^T / sqrt(d)      two 32 x 32 tiles (keys 0-31, 32-63), K step s pairs
//                                d = s (lanes 0-31) with d = 64 + s (lanes 32-63), so each lane
//                                keeps its query's 64 values of one half of d in registers
//   m = max(m, rowmax S), P = exp(S - m), l = l e^(m_old - m) + sum P   (log2 domain)
//   O^T = O^T e^(m_old - m) + V^T P^T   (P^T through a per-wavefront LDS tile)
// O_s = O^T / l; a query block with no kept block gets O_s = 0.
#include "sla2_common.h"

namespace sla2 {

constexpr int kExThreads = 256;
constexpr int kExPad = kD + 1;   // fp32 row stride of the staged K_s and V rows (LDS)
constexpr float kExLog2e = 1.4426950408889634f;
constexpr float kExInvSqrtD = 0.088388347648318440f;

template <typename T, bool kTap>
__global__ __launch_bounds__(kExThreads) void attn_exact_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ mu32, const int32_t* __restrict__ list, int list_stride,
    const int32_t* __restrict__ cnt, const float* __restrict__ alpha, float* __restrict__ O,
    float* __restrict__ O_s_tap, int N, int H) {
  __shared__ float kt[kBK][kExPad];         // K_s rows of the current key block
  __shared__ float vt[kBK][kExPad];         // V rows of the current key block
  __shared__ float pt[4][kBK][33];          // per wavefront: P^T [key][query]
  const int i = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, l32 = lane & 31, g = lane >> 5;
  const int nqb = N / kBQ;
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  const size_t head = static_cast<size_t>(bh) * N;
  const int n = cnt[row];
  const int32_t* L = list + row * list_stride;
  const size_t q0 = head + static_cast<size_t>(i) * kBQ + 32 * w + l32;   // this lane's query
  float q[64];
#pragma unroll
  for (int u = 0; u < 8; ++u) load8<T>(Q + q0 * kD + 64 * g + 8 * u, q + 8 * u);
  // staging: thread t copies row t / 4, columns 32 (t % 4) .. +31 of the K and V blocks
  const int sr = t >> 2, sc = 32 * (t & 3);
  float mu[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) mu[e] = mu32[static_cast<size_t>(bh) * kD + sc + e];
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float m = -INFINITY, l = 0.f;
  const float c2 = kExLog2e * kExInvSqrtD;
  for (int k = 0; k < n; ++k) {
    const int j = L[k];
    __syncthreads();   // the previous block's tiles are no longer read
    const size_t r = head + static_cast<size_t>(j) * kBK + sr;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float x[8];
      load8<T>(K + r * kD + sc + 8 * u, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) kt[sr][sc + 8 * u + e] = x[e] - mu[8 * u + e];
      load8<T>(V + r * kD + sc + 8 * u, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[sr][sc + 8 * u + e] = x[e];
    }
    __syncthreads();   // tiles staged
    // S^T tiles: register r of s[c] is key 32 c + 8 (r / 4) + 4 g + r % 4, query l32
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll 8
    for (int dd = 0; dd < 64; ++dd) {
      s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[l32][dd + 64 * g], q[dd], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[32 + l32][dd + 64 * g], q[dd], s[1], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[c][e] * c2);
    mx = fmaxf(mx, __shfl_xor(mx, 32));   // the other 32 keys of the block
    const float m_new = fmaxf(m, mx);
    const float corr = exp2f(m - m_new);  // 0 on the first block
    float ps = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(fmaf(s[c][e], c2, -m_new));
        ps += p;
        pt[w][32 * c + 8 * (e >> 2) + 4 * g + (e & 3)][l32] = p;
      }
    l = fmaf(l, corr, ps);
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] *= corr;
    __syncthreads();   // P^T visible
    // O^T[d_v][query] += V^T P^T: register r of acc[dt] is d_v = 32 dt + 8 (r / 4) + 4 g + r % 4
#pragma unroll 4
    for (int tt = 0; tt < 32; ++tt) {
      const float b = pt[w][tt + 32 * g][l32];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[tt + 32 * g][32 * dt + l32], b, acc[dt],
                                                        0, 0, 0);
    }
  }
  const float ltot = l + __shfl_xor(l, 32);
  const float inv = (n > 0 && ltot > 0.f) ? 1.0f / ltot : 0.f;
  const float a = alpha[static_cast<size_t>(bh % H) * nqb + i];
  float* orow = O + q0 * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int dv = 32 * dt + 8 * k4 + 4 * g;
      const f32x4 os = f32x4{acc[dt][4 * k4], acc[dt][4 * k4 + 1], acc[dt][4 * k4 + 2],
                             acc[dt][4 * k4 + 3]} * inv;
      f32x4* op = reinterpret_cast<f32x4*>(orow + dv);
      *op = *op + a * os;
      if (kTap) *reinterpret_cast<f32x4*>(O_s_tap + q0 * kD + dv) = os;
    }
}

template <typename T>
static void launch_exact_t(const Geom& g, const void* Q, const ExactArgs& x, hipStream_t s) {
  const dim3 grid(g.nqb, g.BH);
  const T* q = static_cast<const T*>(Q);
  const T* k = static_cast<const T*>(x.K);
  const T* v = static_cast<const T*>(x.V);
  if (x.O_s_tap)
    hipLaunchKernelGGL((attn_exact_kernel<T, true>), grid, dim3(kExThreads), 0, s, q, k, v,
                       x.mu32, x.list, x.list_stride, x.cnt, x.alpha, x.O, x.O_s_tap, g.N, g.H);
  else
    hipLaunchKernelGGL((attn_exact_kernel<T, false>), grid, dim3(kExThreads), 0, s, q, k, v,
                       x.mu32, x.list, x.list_stride, x.cnt, x.alpha, x.O, x.O_s_tap, g.N, g.H);
}

hipError_t launch_attn_exact(const Geom& g, int dtype, const void* Q, const ExactArgs& x,
                             hipStream_t s) {
  if (dtype == 0) launch_exact_t<float>(g, Q, x, s);
  else launch_exact_t<uint16_t>(g, Q, x, s);
  return hipGetLastError();
}

}  // namespace sla2
