// SLA2 linear branch, per-key-block part (step 3 of the computation flow on the summary
// page "SLA2: Sparse-Linear Attention with Learnable Routing and QAT", paper.rainbus.top;
// the "Linear Branch" box of the §3 flowchart and §7 note 2 of "SLA2: Sparse-Linear
// Attention v2 for Diffusion Transformers"; phi = softmax over the head dim per its §4
// symbol table).
//
//   linear_pre    per key block j: phi(K_s,j) (softmax of each row over d), rounded to
//                 bf16; z_j = column sums of those values; h_j^T = V_j^T phi by bf16 MFMA
//                 with fp32 accumulation, stored transposed ([d_v][d_phi]) in bf16 for
//                 the attention kernel, which gathers h_j^T rows per query block. Also
//                 fp32 partial sums over 8 key blocks.
//   linear_total  H_tot = sum_j h_j and Z_tot = sum_j z_j from the partials (fixed order).

#include "sla2_common.h"

namespace sla2 {

constexpr int kPadKP = 72;    // bf16 row stride of the transposed 128 x 64 tiles (bank spread)

__device__ inline bf16x8 lds_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// ---------------------------------------------------------------- linear_pre
// grid (ceil(nkb / 8), BH), 256 threads.
template <typename T>
__global__ __launch_bounds__(256) void linear_pre_kernel(
    const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ mu32,
    uint16_t* __restrict__ ht_bf16, float* __restrict__ h_f32, float* __restrict__ z,
    float* __restrict__ hpart, float* __restrict__ zpart, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t phit[kD][kPadKP];  // phi^T [d][row]
  __shared__ __attribute__((aligned(16))) uint16_t vt[kD][kPadKP];    // V^T   [d][row]
  const int p = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int nkb = N / kBK, np = (nkb + kKpPerWg - 1) / kKpPerWg;
  const int rr = t >> 2, cq = 32 * (t & 3);
  const float* mu = mu32 + static_cast<size_t>(bh) * kD + cq;
  f32x16 hsum[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) hsum[tb] = f32x16{};
  float zs = 0.f;
  const int j_end = min(nkb, (p + 1) * kKpPerWg);
  for (int j = p * kKpPerWg; j < j_end; ++j) {
    const size_t row_off = (static_cast<size_t>(bh) * N + static_cast<size_t>(j) * kBK + rr) * kD + cq;
    float x[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(K + row_off + 8 * u, x + 8 * u);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = x[e] - mu[e];
      mx = fmaxf(mx, x[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = __expf(x[e] - mx);
      sum += x[e];
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    const float inv = 1.0f / sum;
    __syncthreads();  // previous block's tiles are no longer read
#pragma unroll
    for (int e = 0; e < 32; ++e) phit[cq + e][rr] = f32_to_bf16_rne(x[e] * inv);
    float v[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(V + row_off + 8 * u, v + 8 * u);
#pragma unroll
    for (int e = 0; e < 32; ++e) vt[cq + e][rr] = f32_to_bf16_rne(v[e]);
    __syncthreads();
    // z_j: column sums of the bf16 phi values (fp32)
    if (t < kD) {
      float s = 0.f;
      for (int r = 0; r < kBK; ++r) s += bf16_to_f32(phit[t][r]);
      z[(static_cast<size_t>(bh) * nkb + j) * kD + t] = s;
      zs += s;
    }
    // h_j^T tiles: rows d_v = 32 tb + ..., columns d_phi = 32 w + ...
    f32x16 acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x16{};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 b = lds_bf16x8(&phit[32 * w + l32][16 * s + 8 * g]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const bf16x8 a = lds_bf16x8(&vt[32 * tb + l32][16 * s + 8 * g]);
        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[tb], 0, 0, 0);
      }
    }
    const size_t hbase = (static_cast<size_t>(bh) * nkb + j) * (kD * kD);
    const int dphi = 32 * w + l32;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dv = 32 * tb + 8 * (i >> 2) + 4 * g + (i & 3);
        const float hv = acc[tb][i];
        if (ht_bf16) ht_bf16[hbase + dv * kD + dphi] = f32_to_bf16_rne(hv);
        if (h_f32) h_f32[hbase + dphi * kD + dv] = hv;
        hsum[tb][i] += hv;
      }
    }
  }
  const size_t pbase = (static_cast<size_t>(bh) * np + p) * (kD * kD);
  const int dphi = 32 * w + l32;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dv = 32 * tb + 8 * (i >> 2) + 4 * g + (i & 3);
      hpart[pbase + dv * kD + dphi] = hsum[tb][i];
    }
  }
  if (t < kD) zpart[(static_cast<size_t>(bh) * np + p) * kD + t] = zs;
}

hipError_t launch_linear_pre(const Geom& g, int dtype, const void* K, const void* V,
                             const float* mu32, uint16_t* ht_bf16, float* h_f32, float* z,
                             float* hpart, float* zpart, hipStream_t s) {
  dim3 grid((g.nkb + kKpPerWg - 1) / kKpPerWg, g.BH);
  if (dtype == 0)
    hipLaunchKernelGGL(linear_pre_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(K), static_cast<const float*>(V), mu32, ht_bf16,
                       h_f32, z, hpart, zpart, g.N);
  else
    hipLaunchKernelGGL(linear_pre_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), mu32,
                       ht_bf16, h_f32, z, hpart, zpart, g.N);
  return hipGetLastError();
}

// ---------------------------------------------------------------- linear_total
// grid (64, BH), 256 threads: element e = 256 * blockIdx.x + t of H_tot^T (partials are
// transposed); with `standard` set the result is written as H_tot ([d_phi][d_v]).
// Block 0 also sums Z_tot.
__global__ __launch_bounds__(256) void linear_total_kernel(const float* __restrict__ hpart,
                                                           const float* __restrict__ zpart,
                                                           float* __restrict__ htot,
                                                           float* __restrict__ ztot, int np,
                                                           int standard) {
  const int bh = blockIdx.y, t = threadIdx.x;
  const int e = 256 * blockIdx.x + t;
  const float* hp = hpart + static_cast<size_t>(bh) * np * (kD * kD) + e;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;   // fixed interleaved order: deterministic
  int p = 0;
  for (; p + 4 <= np; p += 4) {
    s0 += hp[static_cast<size_t>(p) * (kD * kD)];
    s1 += hp[static_cast<size_t>(p + 1) * (kD * kD)];
    s2 += hp[static_cast<size_t>(p + 2) * (kD * kD)];
    s3 += hp[static_cast<size_t>(p + 3) * (kD * kD)];
  }
  for (; p < np; ++p) s0 += hp[static_cast<size_t>(p) * (kD * kD)];
  const int out = standard ? (e & (kD - 1)) * kD + (e >> 7) : e;
  htot[static_cast<size_t>(bh) * (kD * kD) + out] = (s0 + s1) + (s2 + s3);
  if (blockIdx.x == 0 && t < kD) {
    float zz = 0.f;
    for (int q = 0; q < np; ++q) zz += zpart[(static_cast<size_t>(bh) * np + q) * kD + t];
    ztot[static_cast<size_t>(bh) * kD + t] = zz;
  }
}

hipError_t launch_linear_total(const Geom& g, const float* hpart, const float* zpart,
                               float* htot, float* ztot, int standard, hipStream_t s) {
  const int np = (g.nkb + kKpPerWg - 1) / kKpPerWg;
  hipLaunchKernelGGL(linear_total_kernel, dim3(kD * kD / 256, g.BH), dim3(256), 0, s, hpart,
                     zpart, htot, ztot, np, standard);
  return hipGetLastError();
}

}  // namespace sla2
