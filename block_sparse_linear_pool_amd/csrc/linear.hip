// Per-key-block work of SLA2: the linear branch's precompute (step 3 of the computation flow
// on the summary page "SLA2: Sparse-Linear Attention with Learnable Routing and QAT",
// paper.rainbus.top; the "Linear Branch" box of the §3 flowchart and §7 note 2 of "SLA2:
// Sparse-Linear Attention v2 for Diffusion Transformers"; phi = softmax over the head dim per
// its §4 symbol table) and the low-bit K and V operands of the sparse branch (step 2; §2 Q2
// of the second page), in one pass over K and V.
//
//   kv_prep       per key block j (64 rows), on K_s = fl32(K - mu32) (§7 note 1):
//                   K_s -> INT8, one scale per block: inv = fl32(127 / amax),
//                          code = clamp(rne(fl32(x inv)), +-127), s_k = fl32(amax / 127)
//                   V   -> OCP E4M3, one scale per block: inv = fl32(448 / amax),
//                          code = E4M3(clamp(fl32(v inv), +-448)), s_v = fl32(amax / 448)
//                          (the hardware conversion rounds to nearest even but does not
//                          saturate, hence the clamp); an all-zero block gets scale 0
//                   phi(K_s,j) row softmax over d, rounded to bf16; z_j = column sums of
//                   those values (fp32); h_j = phi^T V_j by bf16 MFMA (fp32 accumulation),
//                   stored as h_j^T ([d_v][d_phi]) in bf16 for the attention kernel's
//                   gathers; fp32 partial sums of h_j^T and z_j over kKpPerWg blocks.
//   linear_total  H_tot = sum_j h_j and Z_tot = sum_j z_j from the partials (fixed order).

#include "sla2_common.h"

namespace sla2 {

// Transposed bf16 tiles in LDS (phi^T and V^T): 128 rows (d) of 64 keys, row stride 144 B.
// The 16-byte chunk c (keys 8c .. 8c+7) of row d sits at chunk slot c ^ ((d >> 4) & 7): the
// 8-byte transposed writes (4 keys of one d per thread) and the 16-byte MFMA operand reads
// (8 keys of 16 consecutive d) then both spread over all LDS banks.
constexpr int kRowT = 72;
__device__ inline int tslot(int d, int c) { return d * kRowT + 8 * (c ^ ((d >> 4) & 7)); }

__device__ inline bf16x8 lds_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// A 32-bit lane offset made opaque inside the loop body (an empty asm, no instruction), so
// the address stays (block-uniform 64-bit base) + (32-bit lane offset), the scalar-base
// form, instead of the offset being widened to a 64-bit register pair outside the loop.
__device__ inline uint32_t lane_off(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---------------------------------------------------------------- kv_prep
// grid (ceil(nkb / kKpPerWg), BH), 256 threads. Element work: thread t takes rows
// 4 (t/16) .. +3 and columns 8 (t%16) .. +7 of the block; a row's 16 threads share one DPP
// row, so row maxima and sums are DPP reductions. MFMA: wavefront w computes the rows
// d_phi = 32 w .. 32 w + 31 of h_j for all 128 d_v. The next block's K and V are loaded while
// the current one is processed.
template <typename T>
__global__ __launch_bounds__(256) void kv_prep_kernel(const T* __restrict__ K,
                                                      const T* __restrict__ V, KvArgs x,
                                                      int N) {
  __shared__ __attribute__((aligned(16))) uint16_t phit[kD * kRowT];
  __shared__ __attribute__((aligned(16))) uint16_t vtt[kD * kRowT];
  __shared__ __attribute__((aligned(16))) uint32_t vq[kD * 16];   // E4M3 V^T rows, 16 words each
  __shared__ float red[2][4];
  const int p = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int rg = t >> 4, cg = t & 15;
  const int nkb = N / kBK, np = (nkb + kKpPerWg - 1) / kKpPerWg;
  const bool quant = x.kc != nullptr;
  float mu[8];
  {
    const f32x4* mp = reinterpret_cast<const f32x4*>(x.mu32 + static_cast<size_t>(bh) * kD + 8 * cg);
    const f32x4 m0 = mp[0], m1 = mp[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      mu[k] = m0[k];
      mu[4 + k] = m1[k];
    }
  }
  f32x16 hsum[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) hsum[tb] = f32x16{};
  float zs = 0.f;
  const int j0 = p * kKpPerWg, j_end = min(nkb, j0 + kKpPerWg);
  const size_t head = static_cast<size_t>(bh) * N;
  // word of keys 4 rg .. 4 rg + 3 inside a V^T row (key order vkey_at)
  const int vw = 8 * (rg & 1) + 4 * (rg >> 3) + ((rg >> 1) & 3);

  // per-lane offsets are 32-bit against block-uniform base pointers (scalar-base addressing)
  const uint32_t eoff = static_cast<uint32_t>(4 * rg * kD + 8 * cg);   // element (4 rg, 8 cg)
  Raw8<T> rk[4], rv[4];
  {
    const T* kb = K + (head + static_cast<size_t>(j0) * kBK) * kD;
    const T* vb = V + (head + static_cast<size_t>(j0) * kBK) * kD;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      rk[m] = load_raw8<T>(kb + (eoff + m * kD));
      rv[m] = load_raw8<T>(vb + (eoff + m * kD));
    }
  }
  // thread-invariant LDS offsets: for d = 8 cg + e the chunk swizzle (d >> 4) & 7 and the V^T
  // word swizzle (d >> 3) & 3 do not depend on e, so row e is base + e * row stride
  const int tw_off = tslot(8 * cg, rg >> 1) + 4 * (rg & 1);
  uint32_t* vq_row = vq + 8 * cg * 16 + 4 * ((vw >> 2) ^ (cg & 3)) + (vw & 3);
  for (int j = j0; j < j_end; ++j) {
    float xk[4][8];
    Raw8<T> cv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      raw8_to_f32(rk[m], xk[m]);
      cv[m] = rv[m];
    }
    if (j + 1 < j_end) {
      const T* kb = K + (head + static_cast<size_t>(j + 1) * kBK) * kD;
      const T* vb = V + (head + static_cast<size_t>(j + 1) * kBK) * kD;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        rk[m] = load_raw8<T>(kb + (eoff + m * kD));
        rv[m] = load_raw8<T>(vb + (eoff + m * kD));
      }
    }
    const size_t blk = static_cast<size_t>(bh) * nkb + j;
    // ---- K_s, block maxima of |K_s| and |V|, row maxima of K_s
    float ak = 0.f, av = 0.f, rmax[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xk[m][e] = xk[m][e] - mu[e];
        ak = fmaxf(ak, fabsf(xk[m][e]));
        av = fmaxf(av, fabsf(raw8_at(cv[m], e)));
        mx = fmaxf(mx, xk[m][e]);
      }
      rmax[m] = row16_max(mx);
    }
    if (quant) {
      ak = wave_max(ak);
      av = wave_max(av);
      if (lane == 0) {
        red[0][w] = ak;
        red[1][w] = av;
      }
    }
    __syncthreads();   // block maxima visible; the previous block's LDS tiles are consumed
    if (quant) {
      const float akb = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
      const float avb = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
      const float ik = akb > 0.f ? 127.0f / akb : 0.f;
      int8_t* tile = x.kc + blk * (kBK * kD);
      int8_t* ktap = x.k_tap + (head + static_cast<size_t>(j) * kBK) * kD;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 4 * rg + m;
        const uint2 cw = make_uint2(i8_pack4(xk[m][0], xk[m][1], xk[m][2], xk[m][3], ik),
                                    i8_pack4(xk[m][4], xk[m][5], xk[m][6], xk[m][7], ik));
        *reinterpret_cast<uint2*>(
            tile + lane_off(static_cast<uint32_t>(r * kD + 16 * kchunk_swz(r, cg >> 1) + 8 * (cg & 1)))) = cw;
        if (x.k_tap) *reinterpret_cast<uint2*>(ktap + lane_off(eoff + m * kD)) = cw;
      }
      const float iv = avb > 0.f ? 448.0f / avb : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vq_row[16 * e] = e4m3_pack4(raw8_at(cv[0], e), raw8_at(cv[1], e), raw8_at(cv[2], e),
                                    raw8_at(cv[3], e), iv);
      if (x.v_tap) {
        uint8_t* vtap = x.v_tap + (head + static_cast<size_t>(j) * kBK) * kD;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint2 cw = make_uint2(
              e4m3_pack4(raw8_at(cv[m], 0), raw8_at(cv[m], 1), raw8_at(cv[m], 2), raw8_at(cv[m], 3), iv),
              e4m3_pack4(raw8_at(cv[m], 4), raw8_at(cv[m], 5), raw8_at(cv[m], 6), raw8_at(cv[m], 7), iv));
          *reinterpret_cast<uint2*>(vtap + lane_off(eoff + m * kD)) = cw;
        }
      }
      if (t == 0) {
        x.sk[blk] = akb / 127.0f;
        x.sv[blk] = avb / 448.0f;
      }
    }
    // ---- phi(K_s) = softmax over d of every row
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xk[m][e] = __expf(xk[m][e] - rmax[m]);
        s += xk[m][e];
      }
      const float inv = 1.0f / row16_sum(s);
#pragma unroll
      for (int e = 0; e < 8; ++e) xk[m][e] *= inv;
    }
    // ---- bf16 phi^T and V^T tiles
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      *reinterpret_cast<uint2*>(phit + tw_off + e * kRowT) =
          make_uint2(pack_bf16x2(xk[0][e], xk[1][e]), pack_bf16x2(xk[2][e], xk[3][e]));
      *reinterpret_cast<uint2*>(vtt + tw_off + e * kRowT) =
          make_uint2(raw8_bf16_pair(cv[0], cv[1], e), raw8_bf16_pair(cv[2], cv[3], e));
    }
    __syncthreads();
    // ---- z_j: thread pair (2 d, 2 d + 1) sums keys 0-31 and 32-63 of phi^T row d
    {
      const int d = t >> 1, hf = t & 1;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(phit + tslot(d, 4 * hf + c));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wd = static_cast<uint32_t>(v[k]);
          s += __uint_as_float(wd << 16);
          s += __uint_as_float(wd & 0xFFFF0000u);
        }
      }
      s += __shfl_xor(s, 1);
      if (hf == 0) {
        x.z[blk * kD + lane_off(static_cast<uint32_t>(d))] = s;
        zs += s;
      }
    }
    // ---- E4M3 V^T tile to HBM
    if (quant) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int q = t + 256 * u;
        const int d = q >> 2, ch = q & 3;
        const i32x4 val = *reinterpret_cast<const i32x4*>(vq + d * 16 + 4 * (ch ^ ((d >> 3) & 3)));
        *reinterpret_cast<i32x4*>(x.vc + blk * (kBK * kD) +
                                  lane_off(static_cast<uint32_t>(d * kBK + 16 * vchunk_swz(d, ch)))) = val;
      }
    }
    // ---- h_j = phi^T V_j, one 32 x 32 tile at a time: rows d_phi = 32 w + ..., columns
    // d_v = 32 tb + ...; lane: d_v = 32 tb + l32, register i: d_phi = 32 w + 8 (i/4) + 4 g + i%4
    uint16_t* htb = x.ht_bf16 + blk * (kD * kD);
    float* hfb = x.h_f32 + blk * (kD * kD);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 2 * s + g;
        const bf16x8 a = lds_bf16x8(phit + tslot(32 * w + l32, c));
        const bf16x8 b = lds_bf16x8(vtt + tslot(32 * tb + l32, c));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
      const int dv = 32 * tb + l32;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int dphi = 32 * w + 8 * k4 + 4 * g;
        if (x.ht_bf16)
          *reinterpret_cast<uint2*>(htb + lane_off(static_cast<uint32_t>(dv * kD + dphi))) =
              make_uint2(pack_bf16x2(acc[4 * k4], acc[4 * k4 + 1]),
                         pack_bf16x2(acc[4 * k4 + 2], acc[4 * k4 + 3]));
        if (x.h_f32) {
#pragma unroll
          for (int k = 0; k < 4; ++k) hfb[static_cast<uint32_t>((dphi + k) * kD + dv)] = acc[4 * k4 + k];
        }
      }
      hsum[tb] += acc;
    }
  }
  const size_t pbase = (static_cast<size_t>(bh) * np + p) * (kD * kD);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int dv = 32 * tb + l32;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
      *reinterpret_cast<f32x4*>(x.hpart + pbase + dv * kD + 32 * w + 8 * k4 + 4 * g) =
          f32x4{hsum[tb][4 * k4], hsum[tb][4 * k4 + 1], hsum[tb][4 * k4 + 2], hsum[tb][4 * k4 + 3]};
  }
  if ((t & 1) == 0) x.zpart[(static_cast<size_t>(bh) * np + p) * kD + (t >> 1)] = zs;
}

hipError_t launch_kv_prep(const Geom& g, int dtype, const void* K, const void* V,
                          const KvArgs& x, hipStream_t s) {
  dim3 grid((g.nkb + kKpPerWg - 1) / kKpPerWg, g.BH);
  if (dtype == 0)
    hipLaunchKernelGGL(kv_prep_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(K), static_cast<const float*>(V), x, g.N);
  else
    hipLaunchKernelGGL(kv_prep_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), x, g.N);
  return hipGetLastError();
}

// ---------------------------------------------------------------- linear_total
// grid (64, BH), 256 threads: element e = 256 * blockIdx.x + t of H_tot^T (partials are
// transposed); with `standard` set the result is written as H_tot ([d_phi][d_v]).
// Eight interleaved accumulators in a fixed order (deterministic), sixteen loads in flight.
// Block 0 also sums Z_tot.
__global__ __launch_bounds__(256) void linear_total_kernel(const float* __restrict__ hpart,
                                                           const float* __restrict__ zpart,
                                                           float* __restrict__ htot,
                                                           float* __restrict__ ztot, int np,
                                                           int standard) {
  const int bh = blockIdx.y, t = threadIdx.x;
  const int e = 256 * blockIdx.x + t;
  const float* hp = hpart + static_cast<size_t>(bh) * np * (kD * kD) + e;
  float s[8] = {};
  int p = 0;
#pragma unroll 2
  for (; p + 8 <= np; p += 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] += hp[static_cast<size_t>(p + k) * (kD * kD)];
  }
  for (; p < np; ++p) s[0] += hp[static_cast<size_t>(p) * (kD * kD)];
  const int out = standard ? (e & (kD - 1)) * kD + (e >> 7) : e;
  htot[static_cast<size_t>(bh) * (kD * kD) + out] =
      ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
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
