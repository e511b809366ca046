// SLA2 attention for one query block: sparse branch, linear branch and the combine in one
// kernel (steps 2-4 of the computation flow on the summary page "SLA2: Sparse-Linear
// Attention with Learnable Routing and QAT", paper.rainbus.top; "Sparse Branch", "Linear
// Branch" and the mix box of the §3 flowchart, §7 note 2, of "SLA2: Sparse-Linear
// Attention v2 for Diffusion Transformers").
//
// One workgroup per query block i (128 queries, 4 wavefronts). Wavefront w computes scores and
// softmax for queries 32 w .. 32 w + 31, and accumulates both branches' outputs for the d_v
// slice 32 w .. 32 w + 31 of all 128 queries; the P tiles and per-query factors pass through
// LDS. Accumulator acc[qt] of wavefront w holds O^T rows d_v = 32 w + 8 (i/4) + 4 g + i%4
// (register i, lane group g = lane / 32) of query 32 qt + lane % 32.
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
// plus one exchange with lane ^ 32, and the lane's 32 P values are exactly a B operand of the
// FP8 product; V^T tiles are stored in the matching key order (vkey_at). K tiles stream
// through a 3-stage and V^T tiles through a 4-stage LDS ring (global_load_lds); the loop is
// software-pipelined: iteration p issues S of block p and the P V product of block p - 1
// (whose P and rescale factors all wavefronts published before the barrier) before the
// softmax of block p.
//
// Linear branch — H_i, Z_i over the dropped blocks: the total minus the kept blocks when
// those are fewer (the same list the sparse loop walks), else a direct sum over the dropped
// blocks. Wavefront w gathers rows d_v = 32 w .. +31 of every h_j^T straight into MFMA
// accumulators: with A = +-I (one nonzero product per output, so each step is one exact fp32
// addition) and B = 16 columns of the h_j^T rows, 32x32x16 bf16 MFMAs add H tiles (rows d_phi,
// columns d_v). That accumulator layout is already the A operand (rows d_v, 8 d_phi per lane)
// of O_l^T = H_i^T phi(Q_i)^T, so H_i goes through bf16 hi + lo straight from registers; the B
// operand phi(Q_i) (phi = softmax over d) is shared through LDS with its d order permuted to
// match. den = phi(q) . Z_i with the same bf16 phi values.
//
// Combine — O = alpha O_s + (1 - alpha) O_l in registers: the sparse accumulator is scaled
// by alpha den / (1 - alpha) (in O_s units), the linear MFMA adds N_l = phi(q) H_i on top,
// and O = acc (1 - alpha) / den. alpha = 1 or no dropped block skips the linear branch.
#include "sla2_common.h"

namespace sla2 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.8073549220576041f;  // log2(448)
constexpr float kInvSqrtD = 0.088388347648318440f;
constexpr int kTile = kBK * kD;            // 8 KB: one K tile or one V^T tile
// LDS map (bytes). Sparse branch: K ring, V^T ring, P tiles (2 buffers x 2 halves of 16 B per
// lane), per-query rescale factors (2 buffers), per-query O_s scale.
constexpr int kOffK = 0;                   // 3 x 8 KB
constexpr int kOffV = 3 * kTile;           // 4 x 8 KB
constexpr int kOffP = 7 * kTile;           // 2 x 8 KB
constexpr int kOffR = 9 * kTile;           // 2 x 128 floats
constexpr int kOffS = kOffR + 1024;        // 128 floats
constexpr int kLdsBytes = kOffS + 512;     // 75264
// Linear branch, over the idle rings: phi(Q_i) (128 rows x 272 B), the dropped-block list
// (direct mode, < nkb / 2 entries), Z_i, den.
constexpr int kPadPhi = 136;               // bf16 row stride of phi(Q_i)
constexpr int kOffPhi = 0;
constexpr int kOffLst = 128 * kPadPhi * 2; // 34816
constexpr int kOffZ = kOffLst + 4096;
constexpr int kOffDen = kOffZ + 512;       // ends at 39936 < kOffP

// One key block: 512 chunks of 16 B of K and 512 of V^T. Wavefront w, instruction u copies
// chunks (2u + w / 2) * 64 .. +63 of K (u = 0, 1) or of V^T (u = 2, 3)... in LDS order: the
// destination of a wavefront's instruction is contiguous.
__device__ inline void issue_tile(int8_t* kdst, int8_t* vdst, const int8_t* kt, const uint8_t* vt,
                                  int w, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c0 = ((u & 1) * 4 + w) * 64;     // chunk of this wavefront within the tile
    const void* src = u < 2 ? static_cast<const void*>(kt + 16 * (c0 + lane))
                            : static_cast<const void*>(vt + 16 * (c0 + lane));
    int8_t* dst = (u < 2 ? kdst : vdst) + 16 * c0;
    __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                              reinterpret_cast<uintptr_t>(dst)),
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
  __shared__ __attribute__((aligned(16))) int8_t smem[kLdsBytes];
  const int t = threadIdx.x;
  int i, bh;
  xcd_block(N / kBQ, static_cast<int>(gridDim.y), &i, &bh);
  const int lane = t & 63, w = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int nqb = N / kBQ, nkb = N / kBK;
  const size_t row = static_cast<size_t>(bh) * nqb + i;
  const int n = cnt[row];
  const int32_t* L = list + row * list_stride;
  const size_t qblk = static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ;  // first query
  const float a = alpha[static_cast<size_t>(bh % H) * nqb + i];
  const size_t tile0 = static_cast<size_t>(bh) * nkb;
  const int nuns = nkb - n;
  const bool do_lin = nuns > 0 && (kTaps || a != 1.f);
  float* Rbuf = reinterpret_cast<float*>(smem + kOffR);
  float* Sbuf = reinterpret_cast<float*>(smem + kOffS);
  const int dv0 = 32 * w + 4 * g;   // first d_v of this lane's accumulator rows

  f32x16 acc[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) acc[qt] = f32x16{};

  // =========================================================== sparse branch
  {
    const int qo = 32 * w + l32;              // the query this lane scores
    i32x4 qf[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      qf[tt] = *reinterpret_cast<const i32x4*>(qc + (qblk + qo) * kD + 32 * tt + 16 * g);
    const float cq = sq[row] * (kLog2e * kInvSqrtD);
    float m2 = -INFINITY, lsum = 0.f, svcur = 0.f;
    for (int p = 0; p < 2 && p < n; ++p) {
      const size_t o = (tile0 + L[p]) * kTile;
      issue_tile(smem + kOffK + p * kTile, smem + kOffV + p * kTile, kc + o, vc + o, w, lane);
    }
    for (int p = 0; p <= n; ++p) {
      // tile p landed (this thread's part); then everyone's part, everyone done with K_{p-1},
      // V_{p-2}, and the P tiles and factors of block p - 1 published
      if (p < n) wait_tiles_after(min(n - 1, p + 1) - p);
      __syncthreads();
      if (p + 2 < n) {
        const size_t o = (tile0 + L[p + 2]) * kTile;
        issue_tile(smem + kOffK + ((p + 2) % 3) * kTile, smem + kOffV + ((p + 2) & 3) * kTile,
                   kc + o, vc + o, w, lane);
      }
      i32x16 s0, s1;   // written (and read) only when p < n
      if (p < n) {
        // ---- S^T for key tiles T = 0 (keys 0-31) and T = 1 (keys 32-63); the first step takes
        // a literal zero accumulator (the MFMA's inline constant, no register fill)
        const int8_t* kt = smem + kOffK + (p % 3) * kTile;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int r0 = l32, r1 = 32 + l32;
          const i32x4 a0 = *reinterpret_cast<const i32x4*>(kt + r0 * kD + 16 * kchunk_swz(r0, 2 * tt + g));
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(kt + r1 * kD + 16 * kchunk_swz(r1, 2 * tt + g));
          s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qf[tt], tt == 0 ? i32x16{} : s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qf[tt], tt == 0 ? i32x16{} : s1, 0, 0, 0);
        }
      }
      if (p >= 1) {
        // ---- acc[qt] <- acc[qt] r + Phat_qt Vhat (block p - 1, this wavefront's d_v rows)
        const int pb = (p - 1) & 1;
        const int8_t* vt = smem + kOffV + ((p - 1) & 3) * kTile;
        const int d = 32 * w + l32;
        const i32x4 v0 = *reinterpret_cast<const i32x4*>(vt + d * kBK + 16 * vchunk_swz(d, 2 * g));
        const i32x4 v1 = *reinterpret_cast<const i32x4*>(vt + d * kBK + 16 * vchunk_swz(d, 2 * g + 1));
        const i32x8 av = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        const int8_t* pp = smem + kOffP + pb * 8192;
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const i32x4 b0 = *reinterpret_cast<const i32x4*>(pp + (qt * 64 + lane) * 16);
          const i32x4 b1 = *reinterpret_cast<const i32x4*>(pp + 4096 + (qt * 64 + lane) * 16);
          const float r = Rbuf[pb * 128 + 32 * qt + l32];
          const i32x8 bp = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          acc[qt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bp, acc[qt] * r, 0, 0, 0,
                                                                    127, 0, 127);
        }
      }
      if (p < n) {
        // ---- online softmax of block p in the log2 domain
        const int j = L[p];
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
        // rescale of the accumulator for this block: f s_v,prev / s_v,j. A block with s_v = 0
        // has all-zero codes, adds nothing and keeps the current units (factor f alone). The
        // ratio uses the hardware reciprocal (a rescale factor; 1 ulp does not matter).
        const float svj = sv[tile0 + j];
        const float r = svj > 0.f ? (svcur > 0.f ? f * svcur * __builtin_amdgcn_rcpf(svj) : 0.f) : f;
        svcur = svj > 0.f ? svj : svcur;
        int8_t* pp = smem + kOffP + (p & 1) * 8192;
        *reinterpret_cast<i32x4*>(pp + (w * 64 + lane) * 16) = i32x4{pk[0], pk[1], pk[2], pk[3]};
        *reinterpret_cast<i32x4*>(pp + 4096 + (w * 64 + lane) * 16) = i32x4{pk[4], pk[5], pk[6], pk[7]};
        if (g == 0) Rbuf[(p & 1) * 128 + qo] = r;
      }
    }
    lsum = lsum + __shfl_xor(lsum, 32);
    if (g == 0) Sbuf[qo] = (n > 0 && lsum > 0.f) ? svcur / lsum : 0.f;
  }
  __syncthreads();   // O_s scales visible; rings idle
  float os_scale[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) os_scale[qt] = Sbuf[32 * qt + l32];

  // lane's output rows: query 32 qt + l32, d_v = dv0 + 8 k4 + (0..3)
  auto out_ptr = [&](float* base, int qt, int k4) {
    return base + (qblk + 32 * qt + l32) * kD + dv0 + 8 * k4;
  };

  if (!do_lin) {
    // no dropped block (O_l = 0) or alpha = 1: O = alpha O_s
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const float coef = (nuns == 0 ? a : 1.f) * os_scale[qt];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        *reinterpret_cast<f32x4*>(out_ptr(O, qt, k4)) =
            f32x4{acc[qt][4 * k4] * coef, acc[qt][4 * k4 + 1] * coef, acc[qt][4 * k4 + 2] * coef,
                  acc[qt][4 * k4 + 3] * coef};
        if (kTaps) {
          const float sc = os_scale[qt];
          if (O_s_tap)
            *reinterpret_cast<f32x4*>(out_ptr(O_s_tap, qt, k4)) =
                f32x4{acc[qt][4 * k4] * sc, acc[qt][4 * k4 + 1] * sc, acc[qt][4 * k4 + 2] * sc,
                      acc[qt][4 * k4 + 3] * sc};
          if (O_l_tap) *reinterpret_cast<f32x4*>(out_ptr(O_l_tap, qt, k4)) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    return;
  }

  // =========================================================== linear branch
  const bool sub = n <= nuns;   // total minus kept, else direct sum over dropped
  const int nl = sub ? n : nuns;
  const float sgn = sub ? -1.f : 1.f;
  uint16_t* phs = reinterpret_cast<uint16_t*>(smem + kOffPhi);
  uint16_t* lst = reinterpret_cast<uint16_t*>(smem + kOffLst);
  float* zsh = reinterpret_cast<float*>(smem + kOffZ);
  float* dsh = reinterpret_cast<float*>(smem + kOffDen);
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
  // phi(q) for query t/2, d = 64 (t%2) .. +63, rounded to bf16
  const int pq = t >> 1, ph = t & 1;
  uint32_t phw[32];   // bf16 pairs, d = 64 ph + 2 e, +1
  {
    const T* qp = Q + (qblk + pq) * kD + 64 * ph;
    float x[64];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8<T>(qp + 8 * u, x + 8 * u);
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
    for (int e = 0; e < 32; ++e) phw[e] = pack_bf16x2(x[2 * e] * inv, x[2 * e + 1] * inv);
  }
  __syncthreads();   // dropped-block list ready
  if (t < kD) {
    float z4[4] = {0.f, 0.f, 0.f, 0.f};
    const float* zbase = z + tile0 * kD + t;
    int nn = 0;
    for (; nn + 4 <= nl; nn += 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = sub ? L[nn + k] : lst[nn + k];
        z4[k] += zbase[static_cast<size_t>(j) * kD];
      }
    }
    for (; nn < nl; ++nn) z4[0] += zbase[static_cast<size_t>(sub ? L[nn] : lst[nn]) * kD];
    const float zt = sub ? ztot[static_cast<size_t>(bh) * kD + t] : 0.f;
    zsh[t] = fmaf(sgn, (z4[0] + z4[1]) + (z4[2] + z4[3]), zt);
  }
  __syncthreads();   // Z_i ready
  {
    // den = phi(q) . Z_i; phi(q) to LDS with d order permuted for the MFMA B operand: slot
    // 16 k + s of a row holds d = 16 k + (s with bits 2 and 3 swapped)
    float dn = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      dn = fmaf(__uint_as_float(phw[e] << 16), zsh[64 * ph + 2 * e], dn);
      dn = fmaf(__uint_as_float(phw[e] & 0xFFFF0000u), zsh[64 * ph + 2 * e + 1], dn);
    }
    dn += __shfl_xor(dn, 1);
    if (ph == 0) dsh[pq] = dn;
    uint16_t* prow = phs + pq * kPadPhi + 64 * ph;
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const uint32_t* hw = phw + 8 * G;   // d = 16 G + 0..15 of this half as 8 bf16 pairs
      *reinterpret_cast<i32x4*>(prow + 16 * G) =
          i32x4{static_cast<int>(hw[0]), static_cast<int>(hw[1]), static_cast<int>(hw[4]),
                static_cast<int>(hw[5])};
      *reinterpret_cast<i32x4*>(prow + 16 * G + 8) =
          i32x4{static_cast<int>(hw[2]), static_cast<int>(hw[3]), static_cast<int>(hw[6]),
                static_cast<int>(hw[7])};
    }
  }
  __syncthreads();   // phi(Q_i), den visible
  float den[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) den[qt] = dsh[32 * qt + l32];
  // ---- sparse part into the combined units, or (taps) O_s stored to the O_s tap, else to
  // the thread's own O elements, and read back by the same thread at the end
  float* os_park = O_s_tap ? O_s_tap : O;
  if (kTaps) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        *reinterpret_cast<f32x4*>(out_ptr(os_park, qt, k4)) =
            f32x4{acc[qt][4 * k4] * os_scale[qt], acc[qt][4 * k4 + 1] * os_scale[qt],
                  acc[qt][4 * k4 + 2] * os_scale[qt], acc[qt][4 * k4 + 3] * os_scale[qt]};
      acc[qt] = f32x16{};
    }
  } else {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) acc[qt] *= os_scale[qt] * a * den[qt] / (1.f - a);
  }
  // ---- H tiles of this wavefront's d_v rows: hacc[tl] rows d_phi = 32 tl + 8 (i/4) + 4 g + i%4,
  // column d_v = dvr = 32 w + l32
  f32x16 hacc[4];
  if (sub) {
    // fragment order: chunk (16 w + 4 tl + k4) * 64 + lane holds d_phi = 32 tl + 8 k4 + 4 g .. +3
    const float* hp = htot_t + static_cast<size_t>(bh) * (kD * kD) + (1024 * w + lane) * 4;
#pragma unroll
    for (int tl = 0; tl < 4; ++tl)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(hp + 256 * (4 * tl + k4));
        hacc[tl][4 * k4] = v[0]; hacc[tl][4 * k4 + 1] = v[1];
        hacc[tl][4 * k4 + 2] = v[2]; hacc[tl][4 * k4 + 3] = v[3];
      }
  } else {
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) hacc[tl] = f32x16{};
  }
  // A = sgn I: fragment m has lane row l32 = 16 m + 8 g + b set at element b
  bf16x8 idf[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 8; ++b) idf[m][b] = to_bf16(l32 == 16 * m + 8 * g + b ? sgn : 0.f);
  // B fragment f = 2 tl + m of block j: row d_v = dvr of h_j^T, d_phi = 32 tl + 16 m + 8 g .. +7,
  // which in fragment order is chunk (8 w + f) * 64 + lane
  const uint16_t* hb = ht_bf16 + tile0 * (kD * kD) + (512 * w + lane) * 8;
  if (nl > 0) {
    i32x4 cur[8];
    {
      const uint16_t* hp = hb + static_cast<size_t>(sub ? L[0] : lst[0]) * (kD * kD);
#pragma unroll
      for (int f = 0; f < 8; ++f) cur[f] = *reinterpret_cast<const i32x4*>(hp + 512 * f);
    }
    for (int nn = 0; nn < nl; ++nn) {
      i32x4 nxt[8];
      if (nn + 1 < nl) {
        const uint16_t* hp = hb + static_cast<size_t>(sub ? L[nn + 1] : lst[nn + 1]) * (kD * kD);
#pragma unroll
        for (int f = 0; f < 8; ++f) nxt[f] = *reinterpret_cast<const i32x4*>(hp + 512 * f);
      }
#pragma unroll
      for (int f = 0; f < 8; ++f)   // f = 2 tl + m
        hacc[f >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            idf[f & 1], __builtin_bit_cast(bf16x8, cur[f]), hacc[f >> 1], 0, 0, 0);
      if (nn + 1 < nl) {
#pragma unroll
        for (int f = 0; f < 8; ++f) cur[f] = nxt[f];
      }
    }
  }
  // ---- acc[qt] += H_i^T phi(Q_i)^T: K step ks = 2 tl + u takes registers 8 u .. 8 u + 7 of
  // hacc[tl] (d_phi = 32 tl + 16 u + 8 (b/4) + 4 g + b%4), split into bf16 hi + lo
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int tl = ks >> 1, u = ks & 1;
    bf16x8 ahi, alo;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const float h = hacc[tl][8 * u + b];
      ahi[b] = to_bf16(h);
      alo[b] = to_bf16(h - static_cast<float>(ahi[b]));
    }
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const bf16x8 bph = *reinterpret_cast<const bf16x8*>(phs + (32 * qt + l32) * kPadPhi + 16 * ks + 8 * g);
      acc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bph, acc[qt], 0, 0, 0);
      acc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bph, acc[qt], 0, 0, 0);
    }
  }
  // ---- O
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const float rden = 1.0f / den[qt];
    const float fin = (1.f - a) * rden;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      f32x4 o;
      if (kTaps) {
        f32x4 ol;
        const f32x4 osv = *reinterpret_cast<const f32x4*>(out_ptr(os_park, qt, k4));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ol[k] = acc[qt][4 * k4 + k] * rden;
          o[k] = fmaf(a, osv[k], (1.f - a) * ol[k]);
        }
        if (O_l_tap) *reinterpret_cast<f32x4*>(out_ptr(O_l_tap, qt, k4)) = ol;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = acc[qt][4 * k4 + k] * fin;
      }
      *reinterpret_cast<f32x4*>(out_ptr(O, qt, k4)) = o;
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
