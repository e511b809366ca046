// Stage-1 router gradient (training time): dL/dproj_q and dL/dproj_k of the loss
// L = sum (O - O_full)^2 against full attention, with the hard Top-k mask in the forward and
// its gradient passed straight through to the SoftTop-k mask ("SLA2: Sparse-Linear Attention
// with Learnable Routing and QAT", summary page, novelty paragraph: two-stage training,
// SoftTop-k during training; "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers",
// §4 Eq. 17 and §5 training table, stage 1).
//
// The forward (router, unquantised sparse branch, linear branch, combine) is the library's
// own; the kernels here take its O, O_s, O_l and work out, for every (query block i, key
// block j) of every head, the derivative of L with respect to the block mask entry M_ij under
// the relaxation that weights key block j's exponentials by M_ij in the sparse branch and its
// h_j, z_j by 1 - M_ij in the linear branch. With delta = 2 (O - O_full), and per query row q
// the kept-key sum l_q = sum_k M e^{S_qk - m_q}, den_q = phi(q) . Z_i, c_q = delta_q . O_s,q,
// c'_q = delta_q . O_l,q:
//   g_ij = alpha_i / l_q  sum_q sum_{k in j} e^{S_qk - m_q} (delta_q . V_k - c_q)
//        - (1 - alpha_i) / den_q  sum_q sum_{k in j} (phi(q) . phi(k)) (delta_q . V_k - c'_q)
// (the linear part written per key: delta_q . (phi(q) h_j) = sum_{k in j} (phi(q) . phi(k))
// (delta_q . V_k)). That is a dense pass over all key blocks of every query block: three
// 128 x 64 x 128 products per pair (S = Q K_s^T, delta V^T, phi(Q) phi(K_s)^T) in f16 with
// fp32 accumulation, reduced to one number per pair.
//
// Then, per query block row: the SoftTop-k derivative (lambda_i held to the row-sum
// constraint), the softmax derivative of P_c, and dA_i = dG_i B / sqrt(d) with A = Qbar Wq,
// B = Kbar_s Wk; per key block dB_j = sum_i dG_ij A_i / sqrt(d); per head
// dWq = sum Qbar^T dA, dWk = sum Kbar_s^T dB over the batch, and the loss.
#include "sla2_common.h"
#include "sla2_grad.h"

namespace sla2 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kGLog2e = 1.4426950408889634f;
constexpr float kGInvSqrtD = 0.088388347648318440f;

// ---------------------------------------------------------------- grad_prep
// f16 copies of K_s = fl32(K - mu32), V and phi(K_s) (softmax over d), [BH][N][d] row-major.
// One wavefront per key row, lane holding d = 2 lane, 2 lane + 1.
template <typename T>
__device__ inline void load2(const T* p, float* a, float* b);
template <>
__device__ inline void load2<float>(const float* p, float* a, float* b) {
  const f32x2 v = *reinterpret_cast<const f32x2*>(p);
  *a = v[0];
  *b = v[1];
}
template <>
__device__ inline void load2<uint16_t>(const uint16_t* p, float* a, float* b) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  *a = __uint_as_float(w << 16);
  *b = __uint_as_float(w & 0xFFFF0000u);
}
__device__ inline uint32_t pack_f16x2(float a, float b) {
  f16x2 v;
  v[0] = static_cast<_Float16>(a);
  v[1] = static_cast<_Float16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__global__ __launch_bounds__(256) void grad_prep_kernel(const T* __restrict__ K,
                                                        const T* __restrict__ V,
                                                        const float* __restrict__ mu32,
                                                        uint32_t* __restrict__ ks16,
                                                        uint32_t* __restrict__ v16,
                                                        uint32_t* __restrict__ pk16, int N,
                                                        size_t rows) {
  const size_t r = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const size_t bh = r / static_cast<size_t>(N);
  float k0, k1, v0, v1;
  load2<T>(K + r * kD + 2 * lane, &k0, &k1);
  load2<T>(V + r * kD + 2 * lane, &v0, &v1);
  const float s0 = k0 - mu32[bh * kD + 2 * lane];
  const float s1 = k1 - mu32[bh * kD + 2 * lane + 1];
  const float mx = wave_max(fmaxf(s0, s1));
  const float e0 = __expf(s0 - mx), e1 = __expf(s1 - mx);
  const float inv = 1.0f / wave_sum(e0 + e1);
  const size_t o = r * (kD / 2) + lane;
  ks16[o] = pack_f16x2(s0, s1);
  v16[o] = pack_f16x2(v0, v1);
  pk16[o] = pack_f16x2(e0 * inv, e1 * inv);
}

// ---------------------------------------------------------------- mask_grad
// One workgroup per (query block i, head), four wavefronts; wavefront w owns queries
// 32 w .. 32 w + 31 (lane: query 32 w + lane % 32, half g = lane / 32 of each key tile).
// Products are transposed (keys as MFMA rows, queries as columns), so every per-query
// constant is one value per lane: v_mfma_f32_32x32x16_f16, A = 32 key rows x 16 d from LDS
// (lane: key row lane % 32, d = 8 g .. +7 of the K step), B = the lane's query, the same d, from
// registers (Q, delta scaled by a power of two, phi(Q), all f16); register r of the
// accumulator is key 8 (r / 4) + 4 g + r % 4 of the tile, query lane % 32.
//
// Key tiles come in through global_load_lds, 32 keys at a time (K_s, V, phi(K_s): 32 rows x
// 256 B each), double buffered: 48 KB, so two workgroups share a CU and each SIMD holds two
// wavefronts (one waits on its loads or its dependent exponentials while the other issues).
// 16-byte chunk c of row r is stored at position c ^ (r % 16) of the row, so the 16 lanes of
// one LDS read phase touch 16 different bank groups.
constexpr int kGThreads = 256;
constexpr int kGTile = kBK * kD * 2;                 // 16 KB: one f16 64 x 128 tile (pass 1)
constexpr int kGHalf = 32 * kD * 2;                  // 8 KB: 32 key rows of one operand
constexpr int kGBuf = 3 * kGHalf;                    // K_s, V, phi(K_s) of 32 keys
constexpr int kGLds = 2 * kGBuf;                     // double buffered (pass 1 uses 16 KB)

// this wavefront's quarter of a key block's three tiles into LDS buffer `buf`
__device__ inline void g_issue(int8_t* buf, const uint32_t* ks, const uint32_t* vv,
                               const uint32_t* pk, size_t row0, int w, int lane,
                               bool k_only) {
  // instruction u of a tile covers its rows 4 u .. 4 u + 3: lane -> row 4 u + lane / 16,
  // position lane % 16, which holds chunk (lane % 16) ^ (row % 16)
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if (k_only && t > 0) break;
    const uint32_t* src = t == 0 ? ks : (t == 1 ? vv : pk);
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
      const int u = 4 * u4 + w;
      const int row = 4 * u + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      const uint32_t* s = src + (row0 + row) * (kD / 2) + 4 * c;   // 16 B = 4 words
      int8_t* d = buf + t * kGTile + 1024 * u;
      __builtin_amdgcn_global_load_lds(
          s, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(d)),
          16, 0, 0);
    }
  }
}
// this wavefront's quarter of 32 keys' three 8 KB tiles (rows 4 u .. 4 u + 3 for u = w, 4 + w)
__device__ inline void g_issue_half(int8_t* buf, const uint32_t* ks, const uint32_t* vv,
                                    const uint32_t* pk, size_t row0, int w, int lane) {
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const uint32_t* src = t == 0 ? ks : (t == 1 ? vv : pk);
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
      const int u = 4 * u2 + w;
      const int row = 4 * u + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      const uint32_t* s = src + (row0 + row) * (kD / 2) + 4 * c;
      int8_t* d = buf + t * kGHalf + 1024 * u;
      __builtin_amdgcn_global_load_lds(
          s, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(d)),
          16, 0, 0);
    }
  }
}
// A fragment: key row `row` (0..63) of a tile, K step s (d = 16 s + 8 g .. +7)
__device__ inline f16x8 g_frag(const int8_t* tile, int row, int s, int g) {
  const int c = 2 * s + g;
  return *reinterpret_cast<const f16x8*>(tile + row * 256 + 16 * (c ^ (row & 15)));
}

template <typename T>
__global__ __launch_bounds__(kGThreads, 2) void mask_grad_kernel(const T* __restrict__ Q,
                                                              const GradArgs x, int N, int H) {
  __shared__ __attribute__((aligned(16))) int8_t smem[kGLds];
  __shared__ float zrow[kD];
  __shared__ float red[2][4];
  __shared__ float lred[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int nqb = N / kBQ, nkb = N / kBK;
  int i, bh;
  xcd_block(nqb, gridDim.y, &i, &bh);
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  const size_t head = static_cast<size_t>(bh) * N;
  const int n = x.cnt[row];
  const int32_t* L = x.list + row * x.list_stride;
  const uint8_t* mrow = x.mask + row * nkb;
  const int nuns = nkb - n;
  const float a = x.alpha[static_cast<size_t>(bh % H) * nqb + i];

  // ---- Z_i (dropped blocks) into LDS: the total minus the kept blocks when those are fewer
  if (t < kD) {
    const float* zb = x.z + static_cast<size_t>(bh) * nkb * kD + t;
    float zs;
    if (n <= nuns) {
      zs = x.ztot[static_cast<size_t>(bh) * kD + t];
      for (int k = 0; k < n; ++k) zs -= zb[static_cast<size_t>(L[k]) * kD];
    } else {
      zs = 0.f;
      for (int j = 0; j < nkb; ++j)
        if (mrow[j] == 0) zs += zb[static_cast<size_t>(j) * kD];
    }
    zrow[t] = zs;
  }
  // ---- the lane's query: d = 16 s + 8 g + e (s = 0..7, e = 0..7)
  const size_t q = head + static_cast<size_t>(i) * kBQ + 32 * w + l32;
  float qv[64], dl[64];
  float c_s = 0.f, c_l = 0.f, lossp = 0.f, dmax = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int d0 = 16 * s + 8 * g;
    load8<T>(Q + q * kD + d0, qv + 8 * s);
    float o[8], of[8], os[8], ol[8];
    load8<float>(x.O + q * kD + d0, o);
    load8<float>(x.O_full + q * kD + d0, of);
    load8<float>(x.O_s + q * kD + d0, os);
    load8<float>(x.O_l + q * kD + d0, ol);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float r = o[e] - of[e];
      lossp = fmaf(r, r, lossp);
      const float dv = 2.f * r;
      dl[8 * s + e] = dv;
      c_s = fmaf(dv, os[e], c_s);
      c_l = fmaf(dv, ol[e], c_l);
      dmax = fmaxf(dmax, fabsf(dv));
    }
  }
  // the other half of d sits in lane ^ 32
  c_s += __shfl_xor(c_s, 32);
  c_l += __shfl_xor(c_l, 32);
  dmax = fmaxf(dmax, __shfl_xor(dmax, 32));
  // delta goes to f16 scaled by a power of two (its largest entry in [1, 2)); products with
  // delta are unscaled exactly afterwards
  const float dsc = dmax > 0.f ? __builtin_amdgcn_ldexpf(1.0f, -static_cast<int>(
                                     __builtin_amdgcn_frexp_expf(dmax)) + 1) : 1.0f;
  // phi(q): softmax over the 128 d of the query
  float qm = -INFINITY;
#pragma unroll
  for (int e = 0; e < 64; ++e) qm = fmaxf(qm, qv[e]);
  qm = fmaxf(qm, __shfl_xor(qm, 32));
  float ph[64], psum = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    ph[e] = __expf(qv[e] - qm);
    psum += ph[e];
  }
  psum += __shfl_xor(psum, 32);
  const float pinv = 1.0f / psum;
  f16x8 qB[8], dB[8], pB[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qB[s][e] = static_cast<_Float16>(qv[8 * s + e]);
      dB[s][e] = static_cast<_Float16>(dl[8 * s + e] * dsc);
      pB[s][e] = static_cast<_Float16>(ph[8 * s + e] * pinv);
    }
  // the row's loss: the four wavefronts' sums
  {
    const float wl = wave_sum(lossp);
    if (lane == 0) lred[w] = wl;
  }
  __syncthreads();   // Z_i and the loss parts visible
  if (t == 0) x.lossp[row] = (lred[0] + lred[1]) + (lred[2] + lred[3]);
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      den = fmaf(static_cast<float>(pB[s][e]), zrow[16 * s + 8 * g + e], den);   // f16 phi(q)
  den += __shfl_xor(den, 32);

  const float c2 = kGLog2e * kGInvSqrtD;
  const size_t tile0 = head;   // row of key 0 of the head in the f16 copies
  auto s_tile = [&](const int8_t* kt, int kt2) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(g_frag(kt, 32 * kt2 + l32, s, g), qB[s], acc,
                                                   0, 0, 0);
    return acc;
  };

  // ---- pass 1: running max and sum of e^{S} over the kept keys (log2 domain), per lane
  // over its half of each key tile, merged with lane ^ 32 at the end
  float m2 = -INFINITY, lsum = 0.f;
  for (int k = 0; k < n; ++k) {
    g_issue(smem, x.ks16, x.v16, x.pk16, tile0 + static_cast<size_t>(L[k]) * kBK, w, lane, true);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();                      // the tile is in LDS
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      const f32x16 sv = s_tile(smem, kt2);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[r] * c2);
      const float mn = fmaxf(m2, mx);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(fmaf(sv[r], c2, -mn));
      lsum = fmaf(lsum, __builtin_amdgcn_exp2f(m2 - mn), ps);
      m2 = mn;
    }
    __syncthreads();                      // every wavefront is done with the tile
  }
  {
    const float mo = __shfl_xor(m2, 32), lo = __shfl_xor(lsum, 32);
    const float mq = fmaxf(m2, mo);
    lsum = lsum * __builtin_amdgcn_exp2f(m2 - mq) + lo * __builtin_amdgcn_exp2f(mo - mq);
    m2 = mq;
  }
  // per-lane factors of the two parts (delta's scale undone here)
  const float ka = (n > 0 && lsum > 0.f) ? a / lsum : 0.f;
  const float kl = (nuns > 0 && den != 0.f) ? (1.f - a) / den : 0.f;
  const float undo = 1.0f / dsc;

  // ---- pass 2: every key block, 32 keys per step (two steps a block)
  float* gout = x.g + row * nkb;
  const int nh = 2 * nkb;
  g_issue_half(smem, x.ks16, x.v16, x.pk16, tile0, w, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  float a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f;
  for (int hb = 0; hb < nh; ++hb) {
    const int8_t* cur = smem + (hb & 1) * kGBuf;
    if (hb + 1 < nh)
      g_issue_half(smem + ((hb + 1) & 1) * kGBuf, x.ks16, x.v16, x.pk16,
                   tile0 + static_cast<size_t>(hb + 1) * 32, w, lane);
    if (t == 0 && (hb & 1) == 0 && hb > 0) {   // block hb / 2 - 1 (its parts are visible)
      const int jb = (hb >> 1) - 1;
      gout[jb] = (red[jb & 1][0] + red[jb & 1][1]) + (red[jb & 1][2] + red[jb & 1][3]);
    }
    f32x16 sv = f32x16{}, dp = f32x16{}, sp = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sv = __builtin_amdgcn_mfma_f32_32x32x16_f16(g_frag(cur, l32, s, g), qB[s], sv, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(g_frag(cur + kGHalf, l32, s, g), dB[s], dp, 0,
                                                  0, 0);
      sp = __builtin_amdgcn_mfma_f32_32x32x16_f16(g_frag(cur + 2 * kGHalf, l32, s, g), pB[s], sp,
                                                  0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(fmaf(sv[r], c2, -m2));
      a1 = fmaf(e, dp[r], a1);
      a2 += e;
      a3 = fmaf(sp[r], dp[r], a3);
      a4 += sp[r];
    }
    if (hb & 1) {   // the block's second half: its number
      const float gl = ka * fmaf(a1, undo, -c_s * a2) - kl * fmaf(a3, undo, -c_l * a4);
      const float ws = wave_sum(gl);
      if (lane == 0) red[(hb >> 1) & 1][w] = ws;
      a1 = a2 = a3 = a4 = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next 32 keys' tiles landed
    __syncthreads();                      // ... for every wavefront; this step's parts visible
  }
  if (t == 0)
    gout[nkb - 1] = (red[(nkb - 1) & 1][0] + red[(nkb - 1) & 1][1]) +
                    (red[(nkb - 1) & 1][2] + red[(nkb - 1) & 1][3]);
}

// ---------------------------------------------------------------- router_vjp_row
// One workgroup per (query block i, head): A_i = Qbar_i Wq, the logits row
// G_ij = A_i . B_j / sqrt(d), P_c = softmax_j(G), then
//   dP_ij = s'_ij (g_ij - sum s' g / sum s') / tau,  s' = soft (1 - soft)
//   dG_ij = P_ij (dP_ij - sum_j P dP)
//   dA_i  = sum_j dG_ij B_j / sqrt(d)
// Writes A_i, dA_i and the dG row.
constexpr int kVThreads = 256;

__device__ inline float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int t = threadIdx.x;
  __syncthreads();
  if ((t & 63) == 0) sh[t >> 6] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}
__device__ inline float block_max(float v, float* sh) {
  v = wave_max(v);
  const int t = threadIdx.x;
  __syncthreads();
  if ((t & 63) == 0) sh[t >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

__global__ __launch_bounds__(kVThreads) void router_vjp_row_kernel(
    const double* __restrict__ qsum, const float* __restrict__ wq, const float* __restrict__ B,
    const float* __restrict__ soft, const float* __restrict__ gmask, float inv_tau,
    float* __restrict__ Arow, float* __restrict__ dA, float* __restrict__ dG, int nqb, int nkb,
    int H) {
  extern __shared__ float vsh[];   // G / P row [nkb], then dG row [nkb]
  __shared__ float arow[kD];
  __shared__ float part[2][kD];
  __shared__ float sh[4];
  const int i = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  const float* W = wq + static_cast<size_t>(bh % H) * kD * kD;
  {
    // A_i = Qbar_i Wq in fp64 (two threads per output, halves of the sum)
    const int o = t & (kD - 1), hh = t >> 7;
    const double* qs = qsum + row * kD;
    double acc = 0.0;
    for (int k = 64 * hh; k < 64 * hh + 64; ++k)
      acc += (qs[k] * (1.0 / kBQ)) * static_cast<double>(W[static_cast<size_t>(k) * kD + o]);
    part[hh][o] = static_cast<float>(acc);
  }
  __syncthreads();
  if (t < kD) arow[t] = part[0][t] + part[1][t];
  __syncthreads();
  // logits: one wavefront per key block at a time, lanes over d
  const float* Bh = B + static_cast<size_t>(bh) * nkb * kD;
  const float a0 = arow[2 * lane], a1v = arow[2 * lane + 1];
  for (int j = w; j < nkb; j += 4) {
    const f32x2 b = *reinterpret_cast<const f32x2*>(Bh + static_cast<size_t>(j) * kD + 2 * lane);
    const float s = wave_sum(fmaf(a0, b[0], a1v * b[1]));
    if (lane == 0) vsh[j] = s * kGInvSqrtD;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = t; j < nkb; j += kVThreads) mx = fmaxf(mx, vsh[j]);
  mx = block_max(mx, sh);
  float se = 0.f;
  for (int j = t; j < nkb; j += kVThreads) {
    const float e = __expf(vsh[j] - mx);
    vsh[j] = e;
    se += e;
  }
  se = block_sum(se, sh);
  const float pinv = 1.0f / se;
  const float* srow = soft + row * nkb;
  const float* grow = gmask + row * nkb;
  float ssum = 0.f, sg = 0.f;
  for (int j = t; j < nkb; j += kVThreads) {
    const float s = srow[j], sp = s * (1.f - s);
    ssum += sp;
    sg = fmaf(sp, grow[j], sg);
  }
  ssum = block_sum(ssum, sh);
  sg = block_sum(sg, sh);
  const float centre = ssum > 0.f ? sg / ssum : 0.f;
  float pdp = 0.f;
  for (int j = t; j < nkb; j += kVThreads) {
    const float s = srow[j], sp = s * (1.f - s);
    const float dp = sp * (grow[j] - centre) * inv_tau;
    const float p = vsh[j] * pinv;
    pdp = fmaf(p, dp, pdp);
    vsh[nkb + j] = dp;
    vsh[j] = p;
  }
  pdp = block_sum(pdp, sh);
  float* dgrow = dG + row * nkb;
  for (int j = t; j < nkb; j += kVThreads) {
    const float v = vsh[j] * (vsh[nkb + j] - pdp);
    vsh[nkb + j] = v;
    dgrow[j] = v;
  }
  __syncthreads();
  {
    // dA_i = sum_j dG_ij B_j / sqrt(d): thread (o, hh) sums key blocks j = hh mod 2
    const int o = t & (kD - 1), hh = t >> 7;
    float acc = 0.f;
    for (int j = hh; j < nkb; j += 2) acc = fmaf(vsh[nkb + j], Bh[static_cast<size_t>(j) * kD + o], acc);
    part[hh][o] = acc;
  }
  __syncthreads();
  if (t < kD) {
    dA[row * kD + t] = (part[0][t] + part[1][t]) * kGInvSqrtD;
    Arow[row * kD + t] = arow[t];
  }
}

// ---------------------------------------------------------------- dB
// dB_j = sum_i dG_ij A_i / sqrt(d): workgroup (64 key blocks, head); thread (d = t % 128,
// half t / 128) accumulates 32 key blocks, reading dG and A through LDS in chunks of 16 rows.
__global__ __launch_bounds__(256) void router_db_kernel(const float* __restrict__ dG,
                                                        const float* __restrict__ Arow,
                                                        float* __restrict__ dB, int nqb, int nkb) {
  __shared__ float gs[16][64];
  __shared__ float as[16][kD];
  const int bh = blockIdx.y, j0 = 64 * blockIdx.x, t = threadIdx.x;
  const int o = t & (kD - 1), hh = t >> 7;
  float acc[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) acc[u] = 0.f;
  const float* G = dG + static_cast<size_t>(bh) * nqb * nkb;
  const float* A = Arow + static_cast<size_t>(bh) * nqb * kD;
  for (int i0 = 0; i0 < nqb; i0 += 16) {
    __syncthreads();
    for (int e = t; e < 16 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      gs[r][c] = (i0 + r < nqb && j0 + c < nkb) ? G[static_cast<size_t>(i0 + r) * nkb + j0 + c] : 0.f;
    }
    for (int e = t; e < 16 * kD; e += 256) {
      const int r = e >> 7, c = e & (kD - 1);
      as[r][c] = i0 + r < nqb ? A[static_cast<size_t>(i0 + r) * kD + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const float av = as[r][o];
#pragma unroll
      for (int u = 0; u < 32; ++u) acc[u] = fmaf(gs[r][32 * hh + u], av, acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const int j = j0 + 32 * hh + u;
    if (j < nkb) dB[(static_cast<size_t>(bh) * nkb + j) * kD + o] = acc[u] * kGInvSqrtD;
  }
}

// ---------------------------------------------------------------- dW and the loss
// Workgroup (head h, which = q or k, a chunk of 16 rows a): dW[a][b] = sum over the batch and
// the rows r of X[r][a] D[r][b] in fp64, X = Qbar (qsum / 128) with D = dA, or
// X = Kbar_s (ksum / 64 - mu64) with D = dB. Thread (a = 16 chunk + t / 16, b = 8 (t % 16) ..
// +7). The workgroup (h, q, 0) also sums the loss of head h over the batch and query blocks.
__global__ __launch_bounds__(256) void router_dw_kernel(
    const double* __restrict__ qsum, const double* __restrict__ ksum,
    const double* __restrict__ mu64, const float* __restrict__ dA, const float* __restrict__ dB,
    const float* __restrict__ lossp, float* __restrict__ dWq, float* __restrict__ dWk,
    double* __restrict__ loss, int B, int H, int nqb, int nkb) {
  __shared__ double xs[32][16];
  __shared__ float ds[32][kD];
  __shared__ double lsh[4];
  const int h = blockIdx.x, which = blockIdx.y / 8, ac = blockIdx.y % 8, t = threadIdx.x;
  const int al = t >> 4, b0 = 8 * (t & 15);
  const int rows = which == 0 ? nqb : nkb;
  double acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.0;
  for (int b = 0; b < B; ++b) {
    const size_t bh = static_cast<size_t>(b) * H + h;
    const double* X = (which == 0 ? qsum : ksum) + bh * rows * kD;
    const float* D = (which == 0 ? dA : dB) + bh * rows * kD;
    const double scale = which == 0 ? 1.0 / kBQ : 1.0 / kBK;
    for (int r0 = 0; r0 < rows; r0 += 32) {
      __syncthreads();
      for (int e = t; e < 32 * 16; e += 256) {
        const int r = e >> 4, c = e & 15;
        const int a = 16 * ac + c;
        double v = 0.0;
        if (r0 + r < rows) {
          v = X[static_cast<size_t>(r0 + r) * kD + a] * scale;
          if (which == 1) v -= mu64[bh * kD + a];
        }
        xs[r][c] = v;
      }
      for (int e = t; e < 32 * kD; e += 256) {
        const int r = e >> 7, c = e & (kD - 1);
        ds[r][c] = r0 + r < rows ? D[static_cast<size_t>(r0 + r) * kD + c] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < 32; ++r) {
        const double xv = xs[r][al];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = fma(xv, static_cast<double>(ds[r][b0 + u]), acc[u]);
      }
    }
  }
  float* dW = (which == 0 ? dWq : dWk) + static_cast<size_t>(h) * kD * kD;
  const int a = 16 * ac + al;
#pragma unroll
  for (int u = 0; u < 8; ++u) dW[static_cast<size_t>(a) * kD + b0 + u] = static_cast<float>(acc[u]);
  if (which == 0 && ac == 0) {
    double s = 0.0;
    for (int e = t; e < B * nqb; e += 256) {
      const int b = e / nqb, i = e % nqb;
      s += static_cast<double>(lossp[(static_cast<size_t>(b) * H + h) * nqb + i]);
    }
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if ((t & 63) == 0) lsh[t >> 6] = s;
    __syncthreads();
    if (t == 0) loss[h] = (lsh[0] + lsh[1]) + (lsh[2] + lsh[3]);
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_grad_prep(const Geom& g, int dtype, const void* K, const void* V,
                            const GradArgs& x, hipStream_t s) {
  const size_t rows = static_cast<size_t>(g.BH) * g.N;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (dtype == 0)
    hipLaunchKernelGGL(grad_prep_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(K),
                       static_cast<const float*>(V), x.mu32, x.ks16, x.v16, x.pk16, g.N, rows);
  else
    hipLaunchKernelGGL(grad_prep_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), x.mu32,
                       x.ks16, x.v16, x.pk16, g.N, rows);
  return hipGetLastError();
}

hipError_t launch_mask_grad(const Geom& g, int dtype, const void* Q, const GradArgs& x,
                            hipStream_t s) {
  const dim3 grid(g.nqb, g.BH);
  if (dtype == 0)
    hipLaunchKernelGGL(mask_grad_kernel<float>, grid, dim3(kGThreads), 0, s,
                       static_cast<const float*>(Q), x, g.N, g.H);
  else
    hipLaunchKernelGGL(mask_grad_kernel<uint16_t>, grid, dim3(kGThreads), 0, s,
                       static_cast<const uint16_t*>(Q), x, g.N, g.H);
  return hipGetLastError();
}

hipError_t launch_router_vjp(const Geom& g, const double* qsum, const double* ksum,
                             const double* mu64, const float* wq, const float* B,
                             const float* soft, const GradArgs& x, float inv_tau, float* dWq,
                             float* dWk, double* loss, hipStream_t s) {
  const size_t lds = static_cast<size_t>(2 * g.nkb) * sizeof(float);
  hipLaunchKernelGGL(router_vjp_row_kernel, dim3(g.nqb, g.BH), dim3(kVThreads), lds, s, qsum, wq,
                     B, soft, x.g, inv_tau, x.Arow, x.dA, x.dG, g.nqb, g.nkb, g.H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_db_kernel, dim3((g.nkb + 63) / 64, g.BH), dim3(256), 0, s, x.dG,
                     x.Arow, x.dB, g.nqb, g.nkb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(router_dw_kernel, dim3(g.H, 16), dim3(256), 0, s, qsum, ksum, mu64, x.dA,
                     x.dB, x.lossp, dWq, dWk, loss, g.B, g.H, g.nqb, g.nkb);
  return hipGetLastError();
}

}  // namespace sla2
