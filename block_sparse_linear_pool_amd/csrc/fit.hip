// Stage-1 alpha fit (gfx950 / CDNA4): the alpha part of the first training stage of
// "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers" (§4 six checks item 5: alpha is
// fitted with an MSE loss against full attention and lands near the kept row mass). With the
// router fixed, O = alpha O_s + (1 - alpha) O_l is affine in alpha, so the MSE of each (head,
// query block) is a quadratic whose minimiser is <O_full - O_l, O_s - O_l> / |O_s - O_l|^2,
// kept in [0, 1] (the convex combination of §4 check 2).
//
// grid (N / 128, H), 256 threads. One pass over the three [128][d] fp32 blocks of every batch,
// 16-byte loads, fp64 accumulation; wavefront sums in a fixed order (deterministic). Bound by
// HBM bandwidth: 3 * 64 KB read per (batch, head, query block).
#include "sla2_fit.h"

#include <stddef.h>
#include <stdint.h>

namespace sla2 {

namespace {
constexpr int kD = 128, kBQ = 128;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
}  // namespace

__global__ __launch_bounds__(256) void fit_alpha_kernel(const float* __restrict__ Of,
                                                        const float* __restrict__ Os,
                                                        const float* __restrict__ Ol,
                                                        float* __restrict__ alpha, int B, int H,
                                                        int N) {
  __shared__ double red[2][4];
  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  double num = 0.0, den = 0.0;
  for (int b = 0; b < B; ++b) {
    const size_t base = ((static_cast<size_t>(b) * H + h) * N + static_cast<size_t>(i) * kBQ) * kD;
#pragma unroll 4
    for (int k = 0; k < kBQ * kD / 1024; ++k) {
      const size_t e = base + 1024 * k + 4 * t;
      const f32x4 f = *reinterpret_cast<const f32x4*>(Of + e);
      const f32x4 s = *reinterpret_cast<const f32x4*>(Os + e);
      const f32x4 l = *reinterpret_cast<const f32x4*>(Ol + e);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double dlt = static_cast<double>(s[c]) - static_cast<double>(l[c]);
        const double res = static_cast<double>(f[c]) - static_cast<double>(l[c]);
        num += res * dlt;
        den += dlt * dlt;
      }
    }
  }
  num = wave_sum_f64(num);
  den = wave_sum_f64(den);
  if (lane == 0) {
    red[0][w] = num;
    red[1][w] = den;
  }
  __syncthreads();
  if (t == 0) {
    const double n = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    const double d = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    double a = d > 0.0 ? n / d : 1.0;
    a = a < 0.0 ? 0.0 : (a > 1.0 ? 1.0 : a);
    alpha[static_cast<size_t>(h) * (N / kBQ) + i] = static_cast<float>(a);
  }
}

hipError_t launch_fit_alpha(int B, int H, int N, const float* O_full, const float* O_s,
                            const float* O_l, float* alpha, hipStream_t s) {
  hipLaunchKernelGGL(fit_alpha_kernel, dim3(N / kBQ, H), dim3(256), 0, s, O_full, O_s, O_l,
                     alpha, B, H, N);
  return hipGetLastError();
}

}  // namespace sla2
