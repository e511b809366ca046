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
//   sla1_mix      O += O_l Wo (the earlier SLA mix, a comparison workload; §2 Q2 table of the
//                 second page).
// The bf16 h_j^T and fp32 H_tot^T for the attention kernel are stored in fragment order
// (htot_frag_index): each of its wavefront loads is then one contiguous run.

#include "sla2_common.h"

namespace sla2 {

// Transposed bf16 tiles in LDS (phi^T and V^T): 128 rows (d) of 64 keys, row stride 144 B.
// The 16-byte chunk c (keys 8c .. 8c+7) of row d sits at chunk slot c ^ ((d >> 4) & 7): the
// 8-byte transposed writes (4 keys of one d per thread) and the 16-byte MFMA operand reads
// (8 keys of 16 consecutive d) then both spread over all LDS banks.
constexpr int kRowT = 72;
constexpr int kRowH = 136;   // bf16 row stride of the staged h_j^T tile
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
// grid (ceil(nkb / kKpPerWg), BH), 512 threads (8 wavefronts, two per SIMD: latency hiding
// within one workgroup, and the fp32 running sum of h_j is 32 registers per lane).
// Element work: thread t takes rows 2 (t/16), +1 and columns 8 (t%16) .. +7 of the block; a
// row's 16 threads share one DPP row, so row maxima and sums are DPP reductions. MFMA:
// wavefront w computes rows d_phi = 32 (w%4) .. +31, columns d_v = 64 (w/4) .. +63 of h_j.
// The next block's K and V are loaded while the current one is processed. Every LDS staging
// area is double-buffered by block parity, so one barrier per block suffices: before it,
// block j's block maxima, phi^T and V^T tiles are written; after it, the codes that need the
// maxima, z_j and h_j of block j are computed, and the E4M3 V^T and bf16 h_j^T tiles of block
// j - 1 (staged in the other buffers) are copied to HBM.
// kMode: 0 forward (codes, scales, h_j^T bf16, z_j, partials), 1 forward with the optional
// row-major code taps, 2 linear precompute only (z_j, partials, optional fp32 h_j). In mode 0
// every store is unconditional (single-writer outputs are written by several lanes with the
// same value), so the wait for the prefetched block at the loop end need not wait for this
// block's stores as well.
constexpr int kKvThreads = 512;
template <typename T, int kMode>
__global__ __launch_bounds__(kKvThreads) void kv_prep_kernel(const T* __restrict__ K,
                                                             const T* __restrict__ V, KvArgs x,
                                                             int N) {
  constexpr bool quant = kMode != 2;
  constexpr int kNb = 2;   // staging buffers
  __shared__ __attribute__((aligned(16))) uint16_t phit[kNb][kD * kRowT];
  __shared__ __attribute__((aligned(16))) uint16_t vtt[kNb][kD * kRowT];
  __shared__ __attribute__((aligned(16))) uint16_t vq[quant ? kNb : 1][quant ? kD * 32 : 8];  // E4M3 V^T rows
  // h_j^T staged in bf16 for row-contiguous stores ([d_v][d_phi], row stride 272 B)
  __shared__ __attribute__((aligned(16))) uint16_t hst[quant ? kNb : 1][quant ? kD * kRowH : 8];
  __shared__ float red[kNb][2][8];
  const int p = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int rg = t >> 4, cg = t & 15;
  const int nkb = N / kBK, np = (nkb + kKpPerWg - 1) / kKpPerWg;
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
  const int ta = w & 3, tv = 2 * (w >> 2);   // MFMA tiles: d_phi tile ta, d_v tiles tv, tv + 1
  f32x16 hsum[2];
  hsum[0] = f32x16{};
  hsum[1] = f32x16{};
  float zs = 0.f;
  const int j0 = p * kKpPerWg, j_end = min(nkb, j0 + kKpPerWg);
  const size_t head = static_cast<size_t>(bh) * N;

  // per-lane offsets are 32-bit against block-uniform base pointers (scalar-base addressing)
  const uint32_t eoff = static_cast<uint32_t>(2 * rg * kD + 8 * cg);   // element (2 rg, 8 cg)
  Raw8<T> rk[2], rv[2];
  {
    const T* kb = K + (head + static_cast<size_t>(j0) * kBK) * kD;
    const T* vb = V + (head + static_cast<size_t>(j0) * kBK) * kD;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      rk[m] = load_raw8<T>(kb + (eoff + m * kD));
      rv[m] = load_raw8<T>(vb + (eoff + m * kD));
    }
  }
  // Thread-invariant LDS offsets. For d = 8 cg + e the chunk swizzles (d >> 4) & 7 of the bf16
  // tiles and (d >> 3) & 3 of the E4M3 tile do not depend on e: row e is base + e * stride.
  // Keys 2 rg, 2 rg + 1 are chunk rg / 4, elements 2 (rg % 4), +1 of the bf16 rows, and
  // byte positions vkey_pos(2 rg), +1 of the E4M3 V^T row.
  const int tw_off = tslot(8 * cg, rg >> 2) + 2 * (rg & 3);
  const int vpos = vkey_pos(2 * rg);
  const int vq_off = 8 * cg * 32 + 8 * ((vpos >> 4) ^ (cg & 3)) + ((vpos & 15) >> 1);
  // copy of the staged E4M3 V^T and bf16 h_j^T tiles of block jb (buffer b) to HBM
  auto copy_out = [&](int jb, int b) {
    const size_t blk = static_cast<size_t>(bh) * nkb + jb;
    {
      const int d = t >> 2, ch = t & 3;
      const i32x4 val = *reinterpret_cast<const i32x4*>(&vq[b][d * 32 + 8 * (ch ^ ((d >> 3) & 3))]);
      *reinterpret_cast<i32x4*>(x.vc + blk * (kBK * kD) +
                                lane_off(static_cast<uint32_t>(d * kBK + 16 * vchunk_swz(d, ch)))) = val;
    }
    // h_j^T in fragment order: chunk q holds row d_v = 32 (q / 512) + q % 32, elements
    // 8 c .. 8 c + 7 with c = (q / 32) % 16
    uint16_t* htb = x.ht_bf16 + blk * (kD * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = t + kKvThreads * u;
      const int row = 32 * (q >> 9) + (q & 31), c16 = (q >> 5) & 15;
      const i32x4 val = *reinterpret_cast<const i32x4*>(&hst[b][row * kRowH + 8 * c16]);
      *reinterpret_cast<i32x4*>(htb + lane_off(static_cast<uint32_t>(8 * q))) = val;
    }
  };
  // Drain the prologue loads (mu, first block) here: otherwise the wait for mu, which the
  // loop's first iteration needs, is placed inside the loop as a wait for every outstanding
  // load, including the prefetch of the next block.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  for (int j = j0; j < j_end; ++j) {
    const int b = (j - j0) & 1;
    float ks[2][8];
    Raw8<T> cv[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      raw8_to_f32(rk[m], ks[m]);
      cv[m] = rv[m];
    }
    if (j + 1 < j_end) {
      const T* kb = K + (head + static_cast<size_t>(j + 1) * kBK) * kD;
      const T* vb = V + (head + static_cast<size_t>(j + 1) * kBK) * kD;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        rk[m] = load_raw8<T>(kb + (eoff + m * kD));
        rv[m] = load_raw8<T>(vb + (eoff + m * kD));
      }
    }
    const size_t blk = static_cast<size_t>(bh) * nkb + j;
    // ---- K_s, block maxima of |K_s| and |V|, row maxima of K_s
    float ak = 0.f, av = 0.f, rmax[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ks[m][e] = ks[m][e] - mu[e];
        ak = fmaxf(ak, fabsf(ks[m][e]));
        av = fmaxf(av, fabsf(raw8_at(cv[m], e)));
        mx = fmaxf(mx, ks[m][e]);
      }
      rmax[m] = row16_max(mx);
    }
    if (quant) {
      ak = wave_max(ak);
      av = wave_max(av);
      if (lane == 0) {
        red[b][0][w] = ak;
        red[b][1][w] = av;
      }
    }
    // ---- phi(K_s) = softmax over d of every row, to the bf16 phi^T tile; V^T tile
    {
      float ex[2][8];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float sm = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ex[m][e] = __expf(ks[m][e] - rmax[m]);
          sm += ex[m][e];
        }
        const float inv = 1.0f / row16_sum(sm);
#pragma unroll
        for (int e = 0; e < 8; ++e) ex[m][e] *= inv;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        *reinterpret_cast<uint32_t*>(&phit[b][tw_off + e * kRowT]) = pack_bf16x2(ex[0][e], ex[1][e]);
        *reinterpret_cast<uint32_t*>(&vtt[b][tw_off + e * kRowT]) = raw8_bf16_pair(cv[0], cv[1], e);
      }
    }
    __syncthreads();   // block j's maxima and tiles visible; block j - 1's staging complete
    if (quant) {
      float akb = red[b][0][0], avb = red[b][1][0];
#pragma unroll
      for (int u = 1; u < 8; ++u) {
        akb = fmaxf(akb, red[b][0][u]);
        avb = fmaxf(avb, red[b][1][u]);
      }
      const float ik = akb > 0.f ? 127.0f / akb : 0.f;
      int8_t* tile = x.kc + blk * (kBK * kD);
      int8_t* ktap = x.k_tap + (head + static_cast<size_t>(j) * kBK) * kD;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = 2 * rg + m;
        const uint2 cw = make_uint2(i8_pack4(ks[m][0], ks[m][1], ks[m][2], ks[m][3], ik),
                                    i8_pack4(ks[m][4], ks[m][5], ks[m][6], ks[m][7], ik));
        *reinterpret_cast<uint2*>(
            tile + lane_off(static_cast<uint32_t>(r * kD + 16 * kchunk_swz(r, cg >> 1) + 8 * (cg & 1)))) = cw;
        if (kMode == 1 && x.k_tap) *reinterpret_cast<uint2*>(ktap + lane_off(eoff + m * kD)) = cw;
      }
      const float iv = avb > 0.f ? 448.0f / avb : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vq[b][vq_off + 32 * e] =
            static_cast<uint16_t>(e4m3_pack4(raw8_at(cv[0], e), raw8_at(cv[1], e), 0.f, 0.f, iv));
      if (kMode == 1 && x.v_tap) {
        uint8_t* vtap = x.v_tap + (head + static_cast<size_t>(j) * kBK) * kD;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint2 cw = make_uint2(
              e4m3_pack4(raw8_at(cv[m], 0), raw8_at(cv[m], 1), raw8_at(cv[m], 2), raw8_at(cv[m], 3), iv),
              e4m3_pack4(raw8_at(cv[m], 4), raw8_at(cv[m], 5), raw8_at(cv[m], 6), raw8_at(cv[m], 7), iv));
          *reinterpret_cast<uint2*>(vtap + lane_off(eoff + m * kD)) = cw;
        }
      }
      x.sk[blk] = akb / 127.0f;   // every lane, same value
      x.sv[blk] = avb / 448.0f;
      if (j > j0) copy_out(j - 1, b ^ 1);
    }
    // ---- z_j: four threads per d, 16 keys each
    {
      const int d = t >> 2, qq = t & 3;
      float sz = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(&phit[b][tslot(d, 2 * qq + c)]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wd = static_cast<uint32_t>(v[k]);
          sz += __uint_as_float(wd << 16);
          sz += __uint_as_float(wd & 0xFFFF0000u);
        }
      }
      sz += __shfl_xor(sz, 1);
      sz += __shfl_xor(sz, 2);   // the four lanes of d now hold the same value
      x.z[blk * kD + lane_off(static_cast<uint32_t>(d))] = sz;
      zs += sz;
    }
    // ---- h_j = phi^T V_j, one 32 x 32 tile at a time; lane: d_v = 32 tb + l32,
    // register i: d_phi = 32 ta + 8 (i/4) + 4 g + i%4
    float* hfb = x.h_f32 + blk * (kD * kD);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tb = tv + u;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 2 * s + g;
        const bf16x8 a = lds_bf16x8(&phit[b][tslot(32 * ta + l32, c)]);
        const bf16x8 bb = lds_bf16x8(&vtt[b][tslot(32 * tb + l32, c)]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
      }
      const int dv = 32 * tb + l32;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int dphi = 32 * ta + 8 * k4 + 4 * g;
        if (kMode != 2)
          *reinterpret_cast<uint2*>(&hst[b][dv * kRowH + dphi]) =
              make_uint2(pack_bf16x2(acc[4 * k4], acc[4 * k4 + 1]),
                         pack_bf16x2(acc[4 * k4 + 2], acc[4 * k4 + 3]));
        if (kMode == 2 && x.h_f32) {
#pragma unroll
          for (int k = 0; k < 4; ++k) hfb[static_cast<uint32_t>((dphi + k) * kD + dv)] = acc[4 * k4 + k];
        }
      }
      hsum[u] += acc;
    }
  }
  if (quant && j_end > j0) {
    __syncthreads();   // the last block's staging complete
    copy_out(j_end - 1, (j_end - 1 - j0) & 1);
  }
  const size_t pbase = (static_cast<size_t>(bh) * np + p) * (kD * kD);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int dv = 32 * (tv + u) + l32;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
      *reinterpret_cast<f32x4*>(x.hpart + pbase + dv * kD + 32 * ta + 8 * k4 + 4 * g) =
          f32x4{hsum[u][4 * k4], hsum[u][4 * k4 + 1], hsum[u][4 * k4 + 2], hsum[u][4 * k4 + 3]};
  }
  x.zpart[(static_cast<size_t>(bh) * np + p) * kD + (t >> 2)] = zs;   // four lanes, same value
}

template <typename T>
static void launch_kv_prep_t(dim3 grid, const T* K, const T* V, const KvArgs& x, int N,
                             hipStream_t s) {
  if (x.kc == nullptr)
    hipLaunchKernelGGL((kv_prep_kernel<T, 2>), grid, dim3(kKvThreads), 0, s, K, V, x, N);
  else if (x.k_tap != nullptr || x.v_tap != nullptr)
    hipLaunchKernelGGL((kv_prep_kernel<T, 1>), grid, dim3(kKvThreads), 0, s, K, V, x, N);
  else
    hipLaunchKernelGGL((kv_prep_kernel<T, 0>), grid, dim3(kKvThreads), 0, s, K, V, x, N);
}

hipError_t launch_kv_prep(const Geom& g, int dtype, const void* K, const void* V,
                          const KvArgs& x, hipStream_t s) {
  dim3 grid((g.nkb + kKpPerWg - 1) / kKpPerWg, g.BH);
  if (dtype == 0)
    launch_kv_prep_t<float>(grid, static_cast<const float*>(K), static_cast<const float*>(V), x,
                            g.N, s);
  else
    launch_kv_prep_t<uint16_t>(grid, static_cast<const uint16_t*>(K),
                               static_cast<const uint16_t*>(V), x, g.N, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- linear_total
// grid (kD * kD / 256 + 1, BH), 256 threads. Workgroup x < 64 reduces elements 256 x .. 256 x +
// 255 of H_tot^T (partials are transposed; written in fragment order, or with `standard` set as
// H_tot, [d_phi][d_v]), lane l the four elements 256 x + 4 l .. + 3 (one 16-byte load, a
// wavefront's load one contiguous 1 KB run); workgroup 64 reduces Z_tot (lanes 0-31). Wavefront
// w sums partials w, w + 4, ... in rounds of 16 (all sixteen loads in flight, one round for up
// to 512 key blocks); the four wavefront sums are combined in a fixed order (deterministic).
__global__ __launch_bounds__(256) void linear_total_kernel(const float* __restrict__ hpart,
                                                           const float* __restrict__ zpart,
                                                           float* __restrict__ htot,
                                                           float* __restrict__ ztot, int np,
                                                           int standard) {
  __shared__ f32x4 red[4][64];
  const int bh = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const bool is_z = blockIdx.x >= kD * kD / 256;
  const bool live = !is_z || lane < kD / 4;   // Z_tot has 128 elements: lanes 0-31
  const int e = is_z ? 4 * (lane & 31) : 256 * blockIdx.x + 4 * lane;
  const int stride = is_z ? kD : kD * kD;
  const float* src = (is_z ? zpart : hpart) + static_cast<size_t>(bh) * np * stride + e;
  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = w; p < np; p += 64) {
    f32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[k] = live && p + 4 * k < np
                 ? *reinterpret_cast<const f32x4*>(src + static_cast<size_t>(p + 4 * k) * stride)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) a += v[k];
  }
  red[w][lane] = a;
  __syncthreads();
  if (w == 0 && live) {
    const f32x4 v = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    if (is_z) {
      *reinterpret_cast<f32x4*>(ztot + static_cast<size_t>(bh) * kD + e) = v;
    } else {
      const int dv = e >> 7, dphi = e & (kD - 1);   // dphi a multiple of 4
      float* hb = htot + static_cast<size_t>(bh) * (kD * kD);
      if (standard) {
#pragma unroll
        for (int c = 0; c < 4; ++c) hb[(dphi + c) * kD + dv] = v[c];
      } else {
        // fragment order keeps dphi .. dphi + 3 of one dv together
        *reinterpret_cast<f32x4*>(hb + htot_frag_index(dv, dphi)) = v;
      }
    }
  }
}

hipError_t launch_linear_total(const Geom& g, const float* hpart, const float* zpart,
                               float* htot, float* ztot, int standard, hipStream_t s) {
  const int np = (g.nkb + kKpPerWg - 1) / kKpPerWg;
  hipLaunchKernelGGL(linear_total_kernel, dim3(kD * kD / 256 + 1, g.BH), dim3(256), 0, s, hpart,
                     zpart, htot, ztot, np, standard);
  return hipGetLastError();
}

// ---------------------------------------------------------------- the earlier SLA mix
// O += O_l Wo per (batch, head) (comparison workload: the mix O = O_s + Proj(O_l) of the
// earlier SLA formulation, §2 Q2 table of the second page; O holds O_s on entry). grid
// (N / 128, BH), 256 threads: the head's Wo staged in LDS (fp32, 64 KB: two workgroups per
// CU); wavefront w forms rows 32 w .. +31 as four 32 x 32 tiles with fp32 MFMA 32x32x2 (exact
// fp32 products, fp32 accumulation). K step s pairs k = s (lanes 0-31) with k = 64 + s (lanes
// 32-63), so each lane's 64 values of its O_l row are one contiguous 256-byte run, loaded
// straight into registers; the four tiles are four independent accumulation chains.
__global__ __launch_bounds__(256) void sla1_mix_kernel(const float* __restrict__ Ol,
                                                       const float* __restrict__ Wo,
                                                       float* __restrict__ O, int N, int H) {
  __shared__ float wo[kD][kD];
  const int bh = blockIdx.y, h = bh % H, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const size_t r0 = static_cast<size_t>(bh) * N + static_cast<size_t>(blockIdx.x) * 128 + 32 * w;
  // this lane's O_l values: row r0 + l32, k = 64 g .. 64 g + 63
  float a[64];
  const float* ap = Ol + (r0 + l32) * kD + 64 * g;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const f32x4 v = reinterpret_cast<const f32x4*>(ap)[u];
    a[4 * u] = v[0]; a[4 * u + 1] = v[1]; a[4 * u + 2] = v[2]; a[4 * u + 3] = v[3];
  }
  const float* wsrc = Wo + static_cast<size_t>(h) * kD * kD;
  for (int e = t; e < kD * kD / 4; e += 256)
    reinterpret_cast<f32x4*>(&wo[0][0])[e] = reinterpret_cast<const f32x4*>(wsrc)[e];
  __syncthreads();
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
  for (int s = 0; s < kD / 2; ++s) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], wo[s + 64 * g][32 * ct + l32], acc[ct],
                                                      0, 0, 0);
  }
  // O += acc: register i of tile ct is row 8 (i / 4) + 4 g + i % 4, column 32 ct + l32; all
  // loads of O first, then the adds and stores
  float* ob = O + r0 * kD;
  float cur[4][16];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      cur[ct][i] = ob[(8 * (i >> 2) + 4 * g + (i & 3)) * kD + 32 * ct + l32];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      ob[(8 * (i >> 2) + 4 * g + (i & 3)) * kD + 32 * ct + l32] = cur[ct][i] + acc[ct][i];
}

hipError_t launch_sla1_mix(const Geom& g, const float* Ol, const float* Wo, float* O,
                           hipStream_t s) {
  hipLaunchKernelGGL(sla1_mix_kernel, dim3(g.N / 128, g.BH), dim3(256), 0, s, Ol, Wo, O, g.N, g.H);
  return hipGetLastError();
}

}  // namespace sla2
