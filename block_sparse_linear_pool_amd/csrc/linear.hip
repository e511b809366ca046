// SLA2 linear branch (step 3 of the computation flow on the summary page "SLA2: Sparse-
// Linear Attention with Learnable Routing and QAT", paper.rainbus.top; the "Linear
// Branch" box of the §3 flowchart and §7 note 2 of "SLA2: Sparse-Linear Attention v2 for
// Diffusion Transformers"; phi = softmax over the head dim per its §4 symbol table).
//
//   linear_pre    per key block j: phi(K_s,j) (softmax of each row over d), rounded to
//                 bf16; z_j = column sums of those values; h_j^T = V_j^T phi by bf16 MFMA
//                 with fp32 accumulation, stored transposed ([d_v][d_phi]) in bf16 for
//                 the output kernel. Also fp32 partial sums over 8 key blocks.
//   linear_total  H_tot = sum_j h_j and Z_tot = sum_j z_j from the partials (fixed order).
//   linear_out    per query block i: H_i, Z_i over the dropped blocks — as the total
//                 minus the kept blocks when those are fewer, else as a direct sum over
//                 the dropped blocks (bounds the cancellation) — then
//                 O_l = phi(Q_i) H_i / (phi(Q_i) . Z_i), with H_i split into bf16 hi + lo
//                 parts for the MFMA. A query block with no dropped block gets O_l = 0.
//
// In linear_out every wavefront owns 32 rows (d_v) of H_i^T for all 128 queries, so it
// gathers exactly the A-operand fragments of its MFMA into registers: no LDS staging of H.
// The MFMA k slots are assigned so that lane group g holds d_phi = 64 g + 8 s + [0, 8) at
// step s: each lane then reads one contiguous 128-byte run of a transposed h_j row. The
// phi(Q) B operand uses the same assignment.
#include "sla2_common.h"

namespace sla2 {

constexpr int kPadKP = 72;    // bf16 row stride of the transposed 128 x 64 tiles (bank spread)
constexpr int kPadQ = 136;    // bf16 row stride of the phi(Q) tile

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

// ---------------------------------------------------------------- linear_out
// grid (nqb, BH), 256 threads. Wavefront w: rows d_v = 32 w + (lane % 32) of H_i^T, all 128
// queries (4 query tiles of 32).
template <typename T>
__global__ __launch_bounds__(256, 2) void linear_out_kernel(
    const T* __restrict__ Q, const uint16_t* __restrict__ ht_bf16, const float* __restrict__ z,
    const float* __restrict__ htot_t, const float* __restrict__ ztot,
    const uint8_t* __restrict__ mask, const int32_t* __restrict__ list, int list_stride,
    const int32_t* __restrict__ cnt, float* __restrict__ O_l, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t phq[kBQ][kPadQ];   // phi(Q_i), bf16
  __shared__ float zsh[kD];
  __shared__ float den[kBQ];
  __shared__ uint16_t lst[kMaxN / kBK];
  const int t = threadIdx.x;
  int i, bh;
  xcd_block(N / kBQ, static_cast<int>(gridDim.y), &i, &bh);
  const int lane = t & 63, w = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int nqb = N / kBQ, nkb = N / kBK;
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  const int nsel = cnt[row];
  const int nuns = nkb - nsel;
  float* out = O_l + (static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ) * kD;
  if (nuns == 0) {
    for (int e = t; e < kBQ * kD / 4; e += 256)
      reinterpret_cast<f32x4*>(out)[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const bool sub = nsel <= nuns;  // total minus kept, else direct sum over dropped
  const int nl = sub ? nsel : nuns;
  if (sub) {
    for (int n = t; n < nsel; n += 256) lst[n] = static_cast<uint16_t>(list[row * list_stride + n]);
  } else if (w == 0) {
    int before = 0;
    for (int j0 = 0; j0 < nkb; j0 += 64) {
      const int j = j0 + lane;
      const bool take = j < nkb && mask[row * nkb + j] == 0;
      const uint64_t m = __ballot(take);
      if (take)
        lst[before + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0))] =
            static_cast<uint16_t>(j);
      before += __popcll(m);
    }
  }
  // ---- phi(Q_i) into LDS: thread t -> query t/2, d = 64 (t%2) .. +64
  {
    const int q = t >> 1, d0 = 64 * (t & 1);
    const T* qrow = Q + (static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ + q) * kD + d0;
    float x[64];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8<T>(qrow + 8 * u, x + 8 * u);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 64; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      x[e] = __expf(x[e] - mx);
      sum += x[e];
    }
    sum += __shfl_xor(sum, 1);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      i32x4 pk;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        pk[k] = static_cast<int>(static_cast<uint32_t>(f32_to_bf16_rne(x[8 * u + 2 * k] * inv)) |
                                 (static_cast<uint32_t>(f32_to_bf16_rne(x[8 * u + 2 * k + 1] * inv)) << 16));
      *reinterpret_cast<i32x4*>(&phq[q][d0 + 8 * u]) = pk;
    }
  }
  __syncthreads();   // list and phi(Q) ready
  // ---- gather this lane's part of H_i^T: row dv, d_phi = 64 g + [0, 64)
  const int dv = 32 * w + l32;
  float hacc[64];
  if (sub) {
    const float* hp = htot_t + static_cast<size_t>(bh) * (kD * kD) + dv * kD + 64 * g;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(hp + 4 * u);
      hacc[4 * u] = v[0]; hacc[4 * u + 1] = v[1]; hacc[4 * u + 2] = v[2]; hacc[4 * u + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 64; ++e) hacc[e] = 0.f;
  }
  float zacc = 0.f;
  if (t < kD) zacc = sub ? ztot[static_cast<size_t>(bh) * kD + t] : 0.f;
  const float sgn = sub ? -1.f : 1.f;
  const uint16_t* hbase = ht_bf16 + static_cast<size_t>(bh) * nkb * (kD * kD) + dv * kD + 64 * g;
  const float* zbase = z + static_cast<size_t>(bh) * nkb * kD + t;
  for (int n = 0; n < nl; ++n) {
    const int j = lst[n];
    const uint16_t* hp = hbase + static_cast<size_t>(j) * (kD * kD);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(hp + 8 * u);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t wd = static_cast<uint32_t>(v[k]);
        hacc[8 * u + 2 * k] = fmaf(sgn, __uint_as_float(wd << 16), hacc[8 * u + 2 * k]);
        hacc[8 * u + 2 * k + 1] = fmaf(sgn, __uint_as_float(wd & 0xFFFF0000u), hacc[8 * u + 2 * k + 1]);
      }
    }
    if (t < kD) zacc = fmaf(sgn, zbase[static_cast<size_t>(j) * kD], zacc);
  }
  if (t < kD) zsh[t] = zacc;
  // ---- bf16 hi + lo A operands (k slot: step s, element b -> d_phi = 64 g + 8 s + b)
  bf16x8 ahi[8], alo[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const float hv = hacc[8 * s + b];
      const uint16_t hi = f32_to_bf16_rne(hv);
      ahi[s][b] = __builtin_bit_cast(__bf16, hi);
      alo[s][b] = __builtin_bit_cast(__bf16, f32_to_bf16_rne(hv - bf16_to_f32(hi)));
    }
  }
  __syncthreads();   // Z ready
  // ---- den[q] = phi(q) . Z_i with the bf16 phi values the MFMA uses
  {
    const int q = t >> 1, d0 = 64 * (t & 1);
    float dsum = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) dsum = fmaf(bf16_to_f32(phq[q][d0 + e]), zsh[d0 + e], dsum);
    dsum += __shfl_xor(dsum, 1);
    if ((t & 1) == 0) den[q] = dsum;
  }
  __syncthreads();
  // ---- O_l^T[dv][q] = sum_dphi H^T[dv][dphi] phi(q)[dphi], 4 query tiles
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    f32x16 acc = f32x16{};
    const int q = 32 * qt + l32;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 b = lds_bf16x8(&phq[q][64 * g + 8 * s]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[s], b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[s], b, acc, 0, 0, 0);
    }
    // lane holds O_l^T[32 w + 8 (ii/4) + 4 g + (ii%4)][q]
    const float rden = 1.0f / den[q];
    float* orow = out + static_cast<size_t>(q) * kD + 32 * w + 4 * g;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
      *reinterpret_cast<f32x4*>(orow + 8 * ib) =
          f32x4{acc[4 * ib] * rden, acc[4 * ib + 1] * rden, acc[4 * ib + 2] * rden,
                acc[4 * ib + 3] * rden};
  }
}

hipError_t launch_linear_out(const Geom& g, int dtype, const void* Q, const uint16_t* ht_bf16,
                             const float* z, const float* htot_t, const float* ztot,
                             const uint8_t* mask, const int32_t* list, int list_stride,
                             const int32_t* cnt, float* O_l, hipStream_t s) {
  dim3 grid(g.nqb, g.BH);
  if (dtype == 0)
    hipLaunchKernelGGL(linear_out_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(Q), ht_bf16, z, htot_t, ztot, mask, list,
                       list_stride, cnt, O_l, g.N);
  else
    hipLaunchKernelGGL(linear_out_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(Q), ht_bf16, z, htot_t, ztot, mask, list,
                       list_stride, cnt, O_l, g.N);
  return hipGetLastError();
}

}  // namespace sla2
