// SLA2 attention for one query block: sparse branch, linear branch and the combine in one
// kernel (steps 2-4 of the computation flow on the summary page "SLA2: Sparse-Linear
// Attention with Learnable Routing and QAT", paper.rainbus.top; "Sparse Branch", "Linear
// Branch" and the mix box of the §3 flowchart, §7 note 2, of "SLA2: Sparse-Linear
// Attention v2 for Diffusion Transformers").
//
// One workgroup per query block i (128 queries, 4 wavefronts of 32 queries).
//
// Sparse branch — for each kept key block j, in ascending order:
//   S^T = Khat_j Qhat_i^T                 INT8 MFMA 32x32x32, exact int32
//   S   = S_int * s_q * s_k / sqrt(d)     folded into one fp32 multiply (log2 domain)
//   m   = max(m, rowmax S)                running max, raised once per 64-key block
//   P~  = exp(S - m);  l = l e^(m_old-m) + sum P~   (l sums the unquantised P~)
//   Phat = E4M3(448 P~)                   packed from the accumulator registers
//   acc = acc e^(m_old-m) + (Phat Vhat_j) s_v / 448   FP8 MFMA 32x32x64
// O_s = acc / l (0 for a query block with no kept block). The accumulator is kept in units
// of the current block's V scale: acc' <- acc' (f s_v,prev / s_v,j) + Phat Vhat_j.
// With S^T (keys as MFMA rows) every lane owns one query, so row maxima and sums are in-lane
// plus one exchange with lane ^ 32, and the lane's 32 P values are exactly the B operand of
// the FP8 product; V^T tiles are stored in the matching key order (vkey_at). K/V tiles
// stream through a 3-stage LDS ring fed by global_load_lds.
//
// Linear branch — H_i, Z_i over the dropped blocks: the total minus the kept blocks when
// those are fewer (the same list the sparse loop walked), else a direct sum over the dropped
// blocks. Thread t gathers row t/2, half t%2 of H_i^T (bf16 h_j^T rows, fp32 sums) into
// registers; H_i^T is then split into bf16 hi + lo and passed through the now idle LDS ring
// in two halves of 64 rows; O_l^T = H_i^T phi(Q_i)^T by bf16 MFMA (phi = softmax over d,
// MFMA k slot (step s, lane group g, element b) = d 64 g + 8 s + b, the lane's own half of
// its query's row); den = phi(q) . Z_i with the same bf16 phi values.
//
// Combine — O = alpha O_s + (1 - alpha) O_l in registers: the sparse accumulator is scaled
// by alpha den / (1 - alpha) (in O_s units), the linear MFMA adds N_l = phi(q) H_i on top,
// and O = acc (1 - alpha) / den. alpha = 1 or no dropped block skips the linear branch.
#include "sla2_common.h"

namespace sla2 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.8073549220576041f;  // log2(448)
constexpr float kInvSqrtD = 0.088388347648318440f;
constexpr int kStages = 3;        // LDS ring depth: tiles p+1 .. p+2 are in flight while p is used
constexpr int kStage = 2 * kBK * kD;   // 16 KB: [K 8 KB | V^T 8 KB]
constexpr int kPadH = 136;        // bf16 row stride of the H^T half tiles in LDS

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

// Wait until at most `after` tiles (4 load instructions each) issued after the tile about
// to be used are still in flight (vmcnt only; the immediate must be a constant).
__device__ inline void wait_tiles_after(int after) {
  if (after <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
  else if (after == 1) __builtin_amdgcn_s_waitcnt(0x0F74);
  else __builtin_amdgcn_s_waitcnt(0x0F78);
}

__device__ inline bf16x8 lds_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// grid (nqb, BH) (remapped per XCD), 256 threads. kTaps: also write O_s and O_l (debug taps).
template <typename T, bool kTaps>
__global__ __launch_bounds__(256) void attn_kernel(
    const T* __restrict__ Q, const int8_t* __restrict__ qc, const int8_t* __restrict__ kc,
    const uint8_t* __restrict__ vc, const float* __restrict__ sq, const float* __restrict__ sk,
    const float* __restrict__ sv, const uint16_t* __restrict__ ht_bf16,
    const float* __restrict__ z, const float* __restrict__ htot_t,
    const float* __restrict__ ztot, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ list, int list_stride, const int32_t* __restrict__ cnt,
    const float* __restrict__ alpha, float* __restrict__ O, float* __restrict__ O_s_tap,
    float* __restrict__ O_l_tap, int N, int H) {
  __shared__ __attribute__((aligned(16))) int8_t smem[kStages * kStage];  // tile ring / H^T halves
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
  const float a = alpha[static_cast<size_t>(bh % H) * nqb + i];

  // =========================================================== sparse branch
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

  for (int p = 0; p < kStages - 1 && p < n; ++p) {
    const size_t o = (tile0 + L[p]) * (kBK * kD);
    issue_tile(smem + p * kStage, kc + o, vc + o, w, lane);
  }
  int cur = 0;
  for (int p = 0; p < n; ++p) {
    const int j = L[p];
    // tile p landed (this thread's part), then everyone's part and everyone done with p-1
    wait_tiles_after(min(n - 1, p + kStages - 2) - p);
    __syncthreads();
    if (p + kStages - 1 < n) {
      const int nxt = cur == 0 ? kStages - 1 : cur - 1;   // stage of tile p-1, now free
      const size_t o = (tile0 + L[p + kStages - 1]) * (kBK * kD);
      issue_tile(smem + nxt * kStage, kc + o, vc + o, w, lane);
    }
    const int8_t* kt = smem + cur * kStage;
    const int8_t* vt = kt + kBK * kD;
    cur = cur == kStages - 1 ? 0 : cur + 1;
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
      const i32x8 av = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      acc[td] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pk, acc[td] * r, 0, 0, 0,
                                                                127, 0, 127);
    }
  }
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float os_scale = (n > 0 && ltot > 0.f) ? svcur / ltot : 0.f;
  float* orow = O + qrow * kD;

  // =========================================================== linear branch
  const int nuns = nkb - n;
  if (nuns == 0 || (!kTaps && a == 1.f)) {
    // no dropped block (O_l = 0) or alpha = 1: O = alpha O_s
#pragma unroll
    for (int td = 0; td < 4; ++td) {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int d = 32 * td + 8 * ib + 4 * g;
        f32x4 os;
#pragma unroll
        for (int k = 0; k < 4; ++k) os[k] = acc[td][4 * ib + k] * os_scale;
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = (nuns == 0 ? a : 1.f) * os[k];
        *reinterpret_cast<f32x4*>(orow + d) = o;
        if (kTaps) {
          if (O_s_tap) *reinterpret_cast<f32x4*>(O_s_tap + qrow * kD + d) = os;
          if (O_l_tap) *reinterpret_cast<f32x4*>(O_l_tap + qrow * kD + d) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    return;
  }
  const bool sub = n <= nuns;   // total minus kept, else direct sum over dropped
  const int nl = sub ? n : nuns;
  // The tile ring is idle from here on: H^T half tiles at 0 (34.8 KB), the dropped-block
  // list (direct mode, < nkb / 2 entries) at 36 KB, Z_i at 40 KB.
  uint16_t* hhi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* hlo = hhi + 64 * kPadH;
  uint16_t* lst = reinterpret_cast<uint16_t*>(smem + 36864);
  float* zsh = reinterpret_cast<float*>(smem + 40960);
  __syncthreads();              // every wave is done with the tile ring
  if (!sub && w == 0) {
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
  // ---- phi(q): this lane's half d = 64 g + [0, 64) as bf16 B fragments
  bf16x8 bq[8];
  {
    const T* qp = Q + qrow * kD + 64 * g;
    float x[64];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8<T>(qp + 8 * u, x + 8 * u);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 64; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      x[e] = __expf(x[e] - mx);
      sum += x[e];
    }
    sum += __shfl_xor(sum, 32);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int b = 0; b < 8; ++b) bq[s][b] = __builtin_bit_cast(__bf16, f32_to_bf16_rne(x[8 * s + b] * inv));
  }
  __syncthreads();              // dropped-block list ready
  const float sgn = sub ? -1.f : 1.f;
  // ---- Z_i
  if (t < kD) {
    float zacc = sub ? ztot[static_cast<size_t>(bh) * kD + t] : 0.f;
    const float* zbase = z + tile0 * kD + t;
    for (int nn = 0; nn < nl; ++nn) {
      const int j = sub ? L[nn] : lst[nn];
      zacc = fmaf(sgn, zbase[static_cast<size_t>(j) * kD], zacc);
    }
    zsh[t] = zacc;
  }
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int b = 0; b < 8; ++b)
      den = fmaf(static_cast<float>(bq[s][b]), zsh[64 * g + 8 * s + b], den);
  den += __shfl_xor(den, 32);
  // ---- sparse part into the combined units (or kept aside for the taps)
  f32x16 os[kTaps ? 4 : 1];
  if (kTaps) {
#pragma unroll
    for (int td = 0; td < 4; ++td) {
      os[td] = acc[td] * os_scale;
      acc[td] = f32x16{};
    }
  } else {
    const float kappa = os_scale * a * den / (1.f - a);
#pragma unroll
    for (int td = 0; td < 4; ++td) acc[td] *= kappa;
  }
  // ---- H_i^T in two halves of 64 rows: gather (thread t: row t/4, d_phi 32 (t%4) .. +32),
  // split into bf16 hi + lo in LDS, then acc += H^T phi^T for the half's two d tiles
  const int hr = t >> 2, hc = 32 * (t & 3);
#pragma unroll   // static acc indices keep the accumulator in registers
  for (int half = 0; half < 2; ++half) {
    const int dv = 64 * half + hr;
    float hacc[32];
    if (sub) {
      const float* hp = htot_t + static_cast<size_t>(bh) * (kD * kD) + dv * kD + hc;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(hp + 4 * u);
        hacc[4 * u] = v[0]; hacc[4 * u + 1] = v[1]; hacc[4 * u + 2] = v[2]; hacc[4 * u + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) hacc[e] = 0.f;
    }
    const uint16_t* hbase = ht_bf16 + tile0 * (kD * kD) + dv * kD + hc;
    for (int nn = 0; nn < nl; ++nn) {
      const int j = sub ? L[nn] : lst[nn];
      const uint16_t* hp = hbase + static_cast<size_t>(j) * (kD * kD);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(hp + 8 * u);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wd = static_cast<uint32_t>(v[k]);
          hacc[8 * u + 2 * k] = fmaf(sgn, __uint_as_float(wd << 16), hacc[8 * u + 2 * k]);
          hacc[8 * u + 2 * k + 1] = fmaf(sgn, __uint_as_float(wd & 0xFFFF0000u), hacc[8 * u + 2 * k + 1]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      i32x4 phi4, plo4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float h0 = hacc[8 * u + 2 * k], h1 = hacc[8 * u + 2 * k + 1];
        const uint16_t x0 = f32_to_bf16_rne(h0), x1 = f32_to_bf16_rne(h1);
        const uint16_t y0 = f32_to_bf16_rne(h0 - bf16_to_f32(x0));
        const uint16_t y1 = f32_to_bf16_rne(h1 - bf16_to_f32(x1));
        phi4[k] = static_cast<int>(static_cast<uint32_t>(x0) | (static_cast<uint32_t>(x1) << 16));
        plo4[k] = static_cast<int>(static_cast<uint32_t>(y0) | (static_cast<uint32_t>(y1) << 16));
      }
      *reinterpret_cast<i32x4*>(hhi + hr * kPadH + hc + 8 * u) = phi4;
      *reinterpret_cast<i32x4*>(hlo + hr * kPadH + hc + 8 * u) = plo4;
    }
    __syncthreads();
#pragma unroll
    for (int td2 = 0; td2 < 2; ++td2) {
      const int td = 2 * half + td2;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 ahi = lds_bf16x8(hhi + (32 * td2 + l32) * kPadH + 64 * g + 8 * s);
        const bf16x8 alo = lds_bf16x8(hlo + (32 * td2 + l32) * kPadH + 64 * g + 8 * s);
        acc[td] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bq[s], acc[td], 0, 0, 0);
        acc[td] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bq[s], acc[td], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // ---- O (lane holds rows d = 32 td + 8 ib + 4 g + k of its query)
  const float rden = 1.0f / den;
  const float fin = (1.f - a) * rden;
#pragma unroll
  for (int td = 0; td < 4; ++td) {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int d = 32 * td + 8 * ib + 4 * g;
      f32x4 o;
      if (kTaps) {
        f32x4 ol, osv;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ol[k] = acc[td][4 * ib + k] * rden;
          osv[k] = os[td][4 * ib + k];
          o[k] = fmaf(a, osv[k], (1.f - a) * ol[k]);
        }
        if (O_s_tap) *reinterpret_cast<f32x4*>(O_s_tap + qrow * kD + d) = osv;
        if (O_l_tap) *reinterpret_cast<f32x4*>(O_l_tap + qrow * kD + d) = ol;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = acc[td][4 * ib + k] * fin;
      }
      *reinterpret_cast<f32x4*>(orow + d) = o;
    }
  }
}

template <typename T>
static void launch_attn_t(const Geom& g, const void* Q, const AttnArgs& x, bool taps,
                          hipStream_t s) {
  dim3 grid(g.nqb, g.BH);
  if (taps)
    hipLaunchKernelGGL((attn_kernel<T, true>), grid, dim3(256), 0, s, static_cast<const T*>(Q),
                       x.qc, x.kc, x.vc, x.sq, x.sk, x.sv, x.ht_bf16, x.z, x.htot_t, x.ztot,
                       x.mask, x.list, x.list_stride, x.cnt, x.alpha, x.O, x.O_s_tap, x.O_l_tap,
                       g.N, g.H);
  else
    hipLaunchKernelGGL((attn_kernel<T, false>), grid, dim3(256), 0, s, static_cast<const T*>(Q),
                       x.qc, x.kc, x.vc, x.sq, x.sk, x.sv, x.ht_bf16, x.z, x.htot_t, x.ztot,
                       x.mask, x.list, x.list_stride, x.cnt, x.alpha, x.O, x.O_s_tap, x.O_l_tap,
                       g.N, g.H);
}

hipError_t launch_attn(const Geom& g, int dtype, const void* Q, const AttnArgs& x,
                       hipStream_t s) {
  const bool taps = x.O_s_tap != nullptr || x.O_l_tap != nullptr;
  if (dtype == 0) launch_attn_t<float>(g, Q, x, taps, s);
  else launch_attn_t<uint16_t>(g, Q, x, taps, s);
  return hipGetLastError();
}

}  // namespace sla2
