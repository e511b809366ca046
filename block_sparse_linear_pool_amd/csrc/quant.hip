// Low-bit operands of the SLA2 sparse branch (step 2 of the computation flow on the
// summary page "SLA2: Sparse-Linear Attention with Learnable Routing and QAT",
// paper.rainbus.top; INT8/FP8 forward in §2 Q2 of "SLA2: Sparse-Linear Attention v2 for
// Diffusion Transformers"):
//   Q   -> INT8, one scale per 128-row query block
//   K_s -> INT8, one scale per 64-row key block, K_s = fl32(K - mu32) (§7 note 1)
//   V   -> OCP E4M3, one scale per 64-row key block
// Symmetric scales from the exact block amax; the code steps are IEEE fp32:
//   inv = fl32(127 / amax), code = clamp(rne(fl32(x * inv)), -127, 127), s = fl32(amax / 127)
//   inv = fl32(448 / amax), code = E4M3(min(fl32(v * inv), 448)),        s = fl32(amax / 448)
// An all-zero block gets scale 0 and zero codes. The hardware FP8 conversion rounds to
// nearest even but does not saturate, so the product is clamped to +-448 first.
//
// One workgroup per 128 rows (query block i = key blocks 2i, 2i+1); HBM-bound.
#include "sla2_common.h"

namespace sla2 {

__device__ inline float block_amax_256(float v, float* red, int t) {
  v = wave_max(v);
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// amax over the two halves of the workgroup (waves 0-1 and waves 2-3)
__device__ inline float half_amax_256(float v, float* red, int t) {
  v = wave_max(v);
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  const int h = t >> 7;
  const float r = fmaxf(red[2 * h], red[2 * h + 1]);
  __syncthreads();
  return r;
}

// grid (nqb, BH), 256 threads. Thread t handles row t/2 (of 128), columns 64*(t%2)..+64.
template <typename T>
__global__ __launch_bounds__(256) void quant_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ mu32, int8_t* __restrict__ qc, int8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, float* __restrict__ sq, float* __restrict__ sk,
    float* __restrict__ sv, int8_t* __restrict__ q_tap, int8_t* __restrict__ k_tap,
    uint8_t* __restrict__ v_tap, int N) {
  __shared__ float red[4];
  __shared__ uint8_t vt[2][kD][kBK];  // transposed, permuted V codes of the two key blocks
  const int i = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int r = t >> 1, c0 = 64 * (t & 1);
  const int nqb = N / kBQ, nkb = N / kBK;
  const size_t row_off = (static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ + r) * kD;
  float x[64];

  // ---- Q: INT8 per 128-row block
#pragma unroll
  for (int u = 0; u < 8; ++u) load8<T>(Q + row_off + c0 + 8 * u, x + 8 * u);
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) am = fmaxf(am, fabsf(x[e]));
  am = block_amax_256(am, red, t);
  {
    const float inv = am > 0.f ? 127.0f / am : 0.f;
    uint32_t packed[16];
#pragma unroll
    for (int e = 0; e < 64; e += 4) {
      uint32_t w = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float y = rintf(x[e + u] * inv);
        y = fminf(fmaxf(y, -127.f), 127.f);
        w |= (static_cast<uint32_t>(static_cast<int>(y)) & 0xFFu) << (8 * u);
      }
      packed[e >> 2] = w;
    }
    i32x4* dst = reinterpret_cast<i32x4*>(qc + row_off + c0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      dst[u] = i32x4{static_cast<int>(packed[4 * u]), static_cast<int>(packed[4 * u + 1]),
                     static_cast<int>(packed[4 * u + 2]), static_cast<int>(packed[4 * u + 3])};
    if (q_tap) {
      i32x4* tp = reinterpret_cast<i32x4*>(q_tap + row_off + c0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        tp[u] = i32x4{static_cast<int>(packed[4 * u]), static_cast<int>(packed[4 * u + 1]),
                      static_cast<int>(packed[4 * u + 2]), static_cast<int>(packed[4 * u + 3])};
    }
    if (t == 0) sq[static_cast<size_t>(bh) * nqb + i] = am / 127.0f;
  }

  // ---- K_s: INT8 per 64-row block (rows 0-63 -> block 2i, 64-127 -> block 2i+1)
  const int kblk = 2 * i + (r >> 6), kr = r & 63;
#pragma unroll
  for (int u = 0; u < 8; ++u) load8<T>(K + row_off + c0 + 8 * u, x + 8 * u);
  const float* mu = mu32 + static_cast<size_t>(bh) * kD + c0;
#pragma unroll
  for (int e = 0; e < 64; ++e) x[e] = x[e] - mu[e];
  am = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) am = fmaxf(am, fabsf(x[e]));
  am = half_amax_256(am, red, t);
  {
    const float inv = am > 0.f ? 127.0f / am : 0.f;
    uint32_t packed[16];
#pragma unroll
    for (int e = 0; e < 64; e += 4) {
      uint32_t w = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float y = rintf(x[e + u] * inv);
        y = fminf(fmaxf(y, -127.f), 127.f);
        w |= (static_cast<uint32_t>(static_cast<int>(y)) & 0xFFu) << (8 * u);
      }
      packed[e >> 2] = w;
    }
    int8_t* tile = kc + (static_cast<size_t>(bh) * nkb + kblk) * (kBK * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int chunk = (c0 >> 4) + u;
      *reinterpret_cast<i32x4*>(tile + kr * kD + 16 * kchunk_swz(kr, chunk)) =
          i32x4{static_cast<int>(packed[4 * u]), static_cast<int>(packed[4 * u + 1]),
                static_cast<int>(packed[4 * u + 2]), static_cast<int>(packed[4 * u + 3])};
    }
    if (k_tap) {
      i32x4* tp = reinterpret_cast<i32x4*>(k_tap + row_off + c0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        tp[u] = i32x4{static_cast<int>(packed[4 * u]), static_cast<int>(packed[4 * u + 1]),
                      static_cast<int>(packed[4 * u + 2]), static_cast<int>(packed[4 * u + 3])};
    }
    if ((t & 127) == 0) sk[static_cast<size_t>(bh) * nkb + kblk] = am / 127.0f;
  }

  // ---- V: E4M3 per 64-row block, stored transposed [d][64] in key order vkey_at
#pragma unroll
  for (int u = 0; u < 8; ++u) load8<T>(V + row_off + c0 + 8 * u, x + 8 * u);
  am = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) am = fmaxf(am, fabsf(x[e]));
  am = half_amax_256(am, red, t);
  {
    const float inv = am > 0.f ? 448.0f / am : 0.f;
    const int pos = vkey_pos(kr);
    uint32_t packed[16];
#pragma unroll
    for (int e = 0; e < 64; e += 4) {
      float y0 = fminf(fmaxf(x[e] * inv, -448.f), 448.f);
      float y1 = fminf(fmaxf(x[e + 1] * inv, -448.f), 448.f);
      float y2 = fminf(fmaxf(x[e + 2] * inv, -448.f), 448.f);
      float y3 = fminf(fmaxf(x[e + 3] * inv, -448.f), 448.f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
      packed[e >> 2] = static_cast<uint32_t>(w);
    }
#pragma unroll
    for (int e = 0; e < 64; ++e)
      vt[r >> 6][c0 + e][pos] = static_cast<uint8_t>(packed[e >> 2] >> (8 * (e & 3)));
    if (v_tap) {
      i32x4* tp = reinterpret_cast<i32x4*>(v_tap + row_off + c0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        tp[u] = i32x4{static_cast<int>(packed[4 * u]), static_cast<int>(packed[4 * u + 1]),
                      static_cast<int>(packed[4 * u + 2]), static_cast<int>(packed[4 * u + 3])};
    }
    if ((t & 127) == 0) sv[static_cast<size_t>(bh) * nkb + kblk] = am / 448.0f;
  }
  __syncthreads();
  // write both V^T tiles: 2 x 128 rows x 4 chunks = 1024 chunks of 16 B, 4 per thread
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = t + 256 * u;
    const int blk = q >> 9, d = (q >> 2) & 127, ch = q & 3;
    const i32x4 val = *reinterpret_cast<const i32x4*>(&vt[blk][d][16 * ch]);
    uint8_t* tile = vc + (static_cast<size_t>(bh) * nkb + 2 * i + blk) * (kBK * kD);
    *reinterpret_cast<i32x4*>(tile + d * kBK + 16 * vchunk_swz(d, ch)) = val;
  }
}

hipError_t launch_quant(const Geom& g, int dtype, const void* Q, const void* K, const void* V,
                        const float* mu32, int8_t* qc, int8_t* kc, uint8_t* vc, float* sq,
                        float* sk, float* sv, int8_t* q_tap, int8_t* k_tap, uint8_t* v_tap,
                        hipStream_t s) {
  dim3 grid(g.nqb, g.BH);
  if (dtype == 0)
    hipLaunchKernelGGL(quant_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(Q),
                       static_cast<const float*>(K), static_cast<const float*>(V), mu32, qc, kc,
                       vc, sq, sk, sv, q_tap, k_tap, v_tap, g.N);
  else
    hipLaunchKernelGGL(quant_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), mu32, qc, kc, vc, sq, sk, sv, q_tap,
                       k_tap, v_tap, g.N);
  return hipGetLastError();
}

}  // namespace sla2
