// SLA2 sparse branch with the combine in its epilogue (steps 2 and 4 of the computation
// flow on the summary page "SLA2: Sparse-Linear Attention with Learnable Routing and
// QAT", paper.rainbus.top; "Sparse Branch" and the mix box of the §3 flowchart of
// "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers").
//
// One workgroup per query block (128 queries, 4 wavefronts of 32 queries). For each kept
// key block j, in ascending order:
//   S^T = Khat_j Qhat_i^T                 INT8 MFMA 32x32x32, exact int32
//   S   = S_int * s_q * s_k / sqrt(d)     folded into one fp32 multiply (log2 domain)
//   m   = max(m, rowmax S)                running max, raised once per 64-key block
//   P~  = exp(S - m);  l = l e^(m_old-m) + sum P~   (l sums the unquantised P~)
//   Phat = E4M3(448 P~)                   packed from the accumulator registers
//   acc = acc e^(m_old-m) + (Phat Vhat_j) s_v / 448   FP8 MFMA 32x32x64
// then O_s = acc / l (0 for a query block with no kept block) and
//   O = alpha_i O_s + (1 - alpha_i) O_l   (step 4; alpha per query block).
// The accumulator is kept in units of the current block's V scale, so each block costs
// one multiply per accumulator element: acc' <- acc' (f s_v,prev / s_v,j) + Phat Vhat_j.
//
// Operand plumbing: with S^T (keys as MFMA rows) every lane owns one query, so row
// maxima and sums are in-lane plus one exchange with lane ^ 32, and the 32 P values a
// lane holds are exactly the B operand the FP8 product needs; V^T tiles are stored with
// the matching key order (vkey_at). K/V tiles are double-buffered in LDS and fetched
// with global_load_lds (no VGPR staging).
#include "sla2_common.h"

namespace sla2 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.8073549220576041f;  // log2(448)
constexpr float kInvSqrtD = 0.088388347648318440f;

__device__ inline void issue_tile(int8_t* lds_stage, const int8_t* kt, const uint8_t* vt, int w,
                                  int lane) {
  // 16 KB per stage = 1024 chunks of 16 B; wave w, instruction u copies chunks
  // (4u + w)*64 .. +63 (K tile for chunk < 512, V tile after).
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c0 = (4 * u + w) * 64;
    const int c = c0 + lane;
    const void* src = c < 512 ? static_cast<const void*>(kt + 16 * c)
                              : static_cast<const void*>(vt + 16 * (c - 512));
    __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                              reinterpret_cast<uintptr_t>(lds_stage + 16 * c0)),
                                     16, 0, 0);
  }
}

__global__ __launch_bounds__(256) void sparse_kernel(
    const int8_t* __restrict__ qc, const int8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    const int32_t* __restrict__ list, int list_stride, const int32_t* __restrict__ cnt,
    const float* __restrict__ alpha, const float* __restrict__ O_l, float* __restrict__ O,
    float* __restrict__ O_s_tap, int N, int H) {
  __shared__ __attribute__((aligned(16))) int8_t stage[2][2 * kBK * kD];  // [K 8 KB | V^T 8 KB]
  const int t = threadIdx.x;
  int i, bh;
  xcd_block(N / kBQ, static_cast<int>(gridDim.y), &i, &bh);
  const int lane = t & 63, w = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int nqb = N / kBQ, nkb = N / kBK;
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  const int n = cnt[row];
  const int32_t* L = list + row * list_stride;
  const int q = 32 * w + l32;
  const size_t qrow = static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ + q;

  i32x4 qf[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    qf[tt] = *reinterpret_cast<const i32x4*>(qc + qrow * kD + 32 * tt + 16 * g);
  const float cq = sq[row] * (kLog2e * kInvSqrtD);

  f32x16 acc[4];
#pragma unroll
  for (int td = 0; td < 4; ++td) acc[td] = f32x16{};
  float m2 = -INFINITY, lsum = 0.f, svcur = 0.f;
  const size_t tile0 = static_cast<size_t>(bh) * nkb;

  if (n > 0) {
    const size_t o = (tile0 + L[0]) * (kBK * kD);
    issue_tile(stage[0], kc + o, vc + o, w, lane);
  }
  for (int p = 0; p < n; ++p) {
    const int j = L[p];
    const int cur = p & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (p + 1 < n) {
      const size_t o = (tile0 + L[p + 1]) * (kBK * kD);
      issue_tile(stage[cur ^ 1], kc + o, vc + o, w, lane);
    }
    const int8_t* kt = stage[cur];
    const int8_t* vt = stage[cur] + kBK * kD;
    // ---- S^T for key tiles T = 0 (keys 0-31) and T = 1 (keys 32-63)
    i32x16 s0 = i32x16{}, s1 = i32x16{};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int r0 = l32, r1 = 32 + l32;
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(kt + r0 * kD + 16 * kchunk_swz(r0, 2 * tt + g));
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(kt + r1 * kD + 16 * kchunk_swz(r1, 2 * tt + g));
      s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qf[tt], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qf[tt], s1, 0, 0, 0);
    }
    // ---- online softmax in the log2 domain
    const float c = cq * sk[tile0 + j];
    int mx = s0[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = max(mx, s0[e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = max(mx, s1[e]);
    mx = max(mx, __shfl_xor(mx, 32));
    const float m2new = fmaxf(m2, static_cast<float>(mx) * c);
    const float f = __builtin_amdgcn_exp2f(m2 - m2new);  // 0 on the first block
    const float b0 = kLog2_448 - m2new;
    float psum = 0.f;
    i32x8 pk;
#pragma unroll
    for (int wv = 0; wv < 8; ++wv) {
      const i32x16& sT = (wv < 4) ? s0 : s1;
      const int e0 = 4 * (wv & 3);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0]), c, b0));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0 + 1]), c, b0));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0 + 2]), c, b0));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(sT[e0 + 3]), c, b0));
      psum += (p0 + p1) + (p2 + p3);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pk[wv] = word;
    }
    lsum = fmaf(lsum, f, psum);
    m2 = m2new;
    // ---- acc' <- acc' * (f * s_v,prev / s_v,j) + Phat Vhat_j. A block with s_v = 0 has
    // all-zero codes, adds nothing and keeps the current units (factor f alone).
    const float svj = sv[tile0 + j];
    const float r = svj > 0.f ? (svcur > 0.f ? f * (svcur / svj) : 0.f) : f;
    svcur = svj > 0.f ? svj : svcur;
#pragma unroll
    for (int td = 0; td < 4; ++td) {
      const int d = 32 * td + l32;
      const i32x4 v0 = *reinterpret_cast<const i32x4*>(vt + d * kBK + 16 * vchunk_swz(d, 2 * g));
      const i32x4 v1 = *reinterpret_cast<const i32x4*>(vt + d * kBK + 16 * vchunk_swz(d, 2 * g + 1));
      const i32x8 a = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      acc[td] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pk, acc[td] * r, 0, 0, 0, 127,
                                                                0, 127);
    }
  }
  // ---- epilogue: O_s = acc' s_v,last / l;  O = alpha O_s + (1 - alpha) O_l
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float os_scale = (n > 0 && ltot > 0.f) ? svcur / ltot : 0.f;
  const float a = alpha[static_cast<size_t>(bh % H) * nqb + i];
  const float* olr = O_l + qrow * kD;
  float* orow = O + qrow * kD;
#pragma unroll
  for (int td = 0; td < 4; ++td) {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int d = 32 * td + 8 * ib + 4 * g;
      const f32x4 ol = *reinterpret_cast<const f32x4*>(olr + d);
      f32x4 os;
      os[0] = acc[td][4 * ib] * os_scale;
      os[1] = acc[td][4 * ib + 1] * os_scale;
      os[2] = acc[td][4 * ib + 2] * os_scale;
      os[3] = acc[td][4 * ib + 3] * os_scale;
      f32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = fmaf(a, os[k], (1.f - a) * ol[k]);
      *reinterpret_cast<f32x4*>(orow + d) = o;
      if (O_s_tap) *reinterpret_cast<f32x4*>(O_s_tap + qrow * kD + d) = os;
    }
  }
}

hipError_t launch_sparse(const Geom& g, const int8_t* qc, const int8_t* kc, const uint8_t* vc,
                         const float* sq, const float* sk, const float* sv, const int32_t* list,
                         int list_stride, const int32_t* cnt, const float* alpha,
                         const float* O_l, float* O, float* O_s_tap, hipStream_t s) {
  hipLaunchKernelGGL(sparse_kernel, dim3(g.nqb, g.BH), dim3(256), 0, s, qc, kc, vc, sq, sk, sv,
                     list, list_stride, cnt, alpha, O_l, O, O_s_tap, g.N, g.H);
  return hipGetLastError();
}

}  // namespace sla2
