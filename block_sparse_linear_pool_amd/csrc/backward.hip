// SLA2 backward kernels (gfx950 / CDNA4): gradients of the sparse-linear attention with the
// block mask held fixed, in 16-bit matrix arithmetic (bf16 operands, fp32 accumulation).
//
// "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers": the sparse branch trains with
// a low-bit forward and a 16-bit backward (§3 table, §4 six checks item 4: the
// straight-through estimator), so the gradient here is that of the unquantised forward; the
// gradient is derived by hand with the linear branch's dH_i, dZ_i formed first, so that each
// (key block, query block) pair costs one matrix addition (§7 note 3).
//
// Kernels, in launch order (after pool / colmean / kv_prep / linear_total of the forward give
// colmean(K), bf16 h_j^T, z_j, H_tot, Z_tot, and mask_to_list gives the kept lists):
//   key_lists    per key block, the ascending query blocks that keep it (transposed mask)
//   key_plan     long key lists cut into work items of at most C query blocks
//   bwd_prep     bf16 copies: Q, V (fp32 inputs), K_s = K - colmean(K), dO_s = alpha dO
//   bwd_lin_q    per query block: a = phi(Q_i), H_i, Z_i; O_l, dnum, dden; writes
//                dQ = a * (da - rowsum(da a)) (the linear part), dH_i^T (bf16), dZ_i, and
//                dalpha = -sum(dO O_l)
//   dh_total     dH_tot, dZ_tot: sums over all query blocks
//   bwd_q        per query block, two passes over its kept key blocks: pass 1 rebuilds the
//                row softmax (log-sum-exp, O_s) and D = rowsum(dO_s O_s); pass 2 forms
//                dS = P (dO_s V^T - D) and adds dS K_s / sqrt(d) to dQ; dalpha += sum(dO O_s)
//   bwd_kv_extra the work items past the first of each key list: partial dK_s, dV, dH, dz
//   bwd_kv       per key block, over the query blocks that keep it: dV += P^T dO_s,
//                dK_s += dS^T Q / sqrt(d); then the linear part with
//                dh_j = dH_tot - sum of dH_i over those query blocks (the one addition per
//                pair), dz_j likewise: dV += phi(K_s,j) dh_j,
//                dK_s += phi * (dphi - rowsum(dphi phi)), dphi = V_j dh_j^T + 1 dz_j^T;
//                writes dK_s and per-key-block column sums of it
//   dk_mean      column mean of dK_s per head; dk_center: dK = dK_s - mean (K smoothing)
//
// MFMA: the sparse and linear kernels use v_mfma_f32_16x16x32_bf16 (layout at the helpers
// below). The idea, shown here for its 32x32x16 form: v_mfma_f32_32x32x16_bf16. Operand A lane (g = lane / 32,
// l = lane % 32) holds row l,
// k = 8 g .. 8 g + 7; B holds column l, the same k; the accumulator holds column l and rows
// 8 (r / 4) + 4 g + r % 4 in register r. So an accumulator C (M x N) serves directly as the B
// operand of X C or the A operand of C^T Y (both contract over M), with k taken in register
// order: registers 8 h .. 8 h + 7 are rows 16 h + 4 g .. +3 and 16 h + 8 + 4 g .. +3; the other
// operand is then read from LDS in that row order; operands that run down the columns of a
// row-major LDS tile use the transposing LDS read. All LDS tiles are bf16 [rows][136]
// (272-byte rows).
#include "sla2_common.h"

namespace sla2 {

namespace {

constexpr int kLd = 136;          // bf16 LDS row stride (elements)
constexpr int kTile = kD * kLd;   // one 128-row bf16 tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.08838834764831845f;   // 1 / sqrt(128)

__device__ inline bf16x8 ld_row8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(p));
}
// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, source lane s gives
// the address of 4 consecutive 16-bit elements and result lane l receives element l % 4 of
// source lanes l / 4, 4 + l / 4, 8 + l / 4, 12 + l / 4 (in that order). With source lane
// s = 4 k + j pointing at row r0 + k, columns c0 + 4 j .. +3, lane l so gets rows r0 .. r0 + 3
// of column c0 + l.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ inline uint2 ld_tr4(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) v4i16*>(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(uint2, v);
}
__device__ inline void st_bf16x8(uint16_t* p, const float* v) {
  const i32x4 w = {static_cast<int>(pack_bf16x2(v[0], v[1])), static_cast<int>(pack_bf16x2(v[2], v[3])),
                   static_cast<int>(pack_bf16x2(v[4], v[5])), static_cast<int>(pack_bf16x2(v[6], v[7]))};
  *reinterpret_cast<i32x4*>(p) = w;
}
__device__ inline void unpack_bf16x8(const i32x4& v, float* out) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = static_cast<uint32_t>(v[k]);
    out[2 * k] = __uint_as_float(w << 16);
    out[2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
}
__device__ inline float bf(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ inline int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// sum of src[idx(n) * kD + col] over n in [n0, n1), in n order, four loads in flight
template <typename Idx>
__device__ inline float sum_rows(const float* src, Idx idx, int n0, int n1, int col) {
  float s = 0.f;
  int n = n0;
  for (; n + 3 < n1; n += 4) {
    const float a = src[static_cast<size_t>(idx(n)) * kD + col];
    const float b = src[static_cast<size_t>(idx(n + 1)) * kD + col];
    const float c = src[static_cast<size_t>(idx(n + 2)) * kD + col];
    const float d = src[static_cast<size_t>(idx(n + 3)) * kD + col];
    s = (((s + a) + b) + c) + d;
  }
  for (; n < n1; ++n) s += src[static_cast<size_t>(idx(n)) * kD + col];
  return s;
}

// sum over n in [n0, n1) of the bf16 d x d tiles src + idx(n) d^2 (thread: chunks t + 512 u,
// u < 4), added in n order, four tiles' loads in flight
template <typename Idx>
__device__ inline void sum_tiles512(float (&acc)[4][8], const uint16_t* src, Idx idx, int n0,
                                    int n1, int t) {
  constexpr int kF = 4;
  int n = n0;
  for (; n + kF - 1 < n1; n += kF) {
    i32x4 v[kF][4];
#pragma unroll
    for (int f = 0; f < kF; ++f) {
      const uint16_t* a = src + static_cast<size_t>(idx(n + f)) * (kD * kD);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[f][u] = *reinterpret_cast<const i32x4*>(a + 8 * (t + 512 * u));
    }
#pragma unroll
    for (int f = 0; f < kF; ++f)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float fa[8];
        unpack_bf16x8(v[f][u], fa);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[u][k] += fa[k];
      }
  }
  for (; n < n1; ++n) {
    const uint16_t* a = src + static_cast<size_t>(idx(n)) * (kD * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float fa[8];
      unpack_bf16x8(*reinterpret_cast<const i32x4*>(a + 8 * (t + 512 * u)), fa);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[u][k] += fa[k];
    }
  }
}

// ---- 16x16x32 MFMA helpers (A lane (G = lane / 16, l = lane % 16): row l, k = 8 G .. +7; B:
// column l, same k; accumulator: column l, rows 4 G .. +3)
__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// two accumulator tiles (rows 0-15 and 16-31 of a 32-deep k chunk) as a bf16 operand:
// element i of lane group G is row 4 G + i (i < 4) or 16 + 4 G + i - 4
__device__ inline bf16x8 acc_op16(const f32x4& a, const f32x4& b) {
  const i32x4 v = {static_cast<int>(pack_bf16x2(a[0], a[1])), static_cast<int>(pack_bf16x2(a[2], a[3])),
                   static_cast<int>(pack_bf16x2(b[0], b[1])), static_cast<int>(pack_bf16x2(b[2], b[3]))};
  return __builtin_bit_cast(bf16x8, v);
}
// the matching operand read down the columns of a row-major tile: lane (G, l) gets column
// c0 + l, rows r0 + 4 G .. +3 and r0 + 16 + 4 G .. +3
__device__ inline bf16x8 ld_col8_16(const uint16_t* base, int c0, int r0, int G, int lane) {
  const int s = lane & 15;
  const uint16_t* p = base + (r0 + 4 * G + (s >> 2)) * kLd + c0 + 4 * (s & 3);
  const uint2 a = ld_tr4(p), b = ld_tr4(p + 16 * kLd);
  const i32x4 v = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(b.x),
                   static_cast<int>(b.y)};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ inline float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ inline float group4_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// rows k0 + 8 G .. +7 of column c0 + l (natural order; 16x16x32 operand down the columns)
__device__ inline bf16x8 ld_col8n_16(const uint16_t* base, int c0, int r0, int G, int lane) {
  const int s = lane & 15;
  const uint16_t* p = base + (r0 + 8 * G + (s >> 2)) * kLd + c0 + 4 * (s & 3);
  const uint2 a = ld_tr4(p), b = ld_tr4(p + 4 * kLd);
  const i32x4 v = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(b.x),
                   static_cast<int>(b.y)};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace

// ---------------------------------------------------------------- bwd_prep
// grid (N / 16, BH), 256 threads; thread: one 8-element chunk. bf16 operand copies for the
// backward kernels: Q and V (fp32 inputs only), K_s = K - colmean(K), dO_s = alpha dO.
template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs x) {
  const int bh = blockIdx.y;
  const int N = x.nqb * kBQ;
  const size_t loc = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 8;   // in the head
  const int row = static_cast<int>(loc / kD), c8 = static_cast<int>(loc % kD);
  const size_t e = static_cast<size_t>(bh) * N * kD + loc;
  const float al = x.alpha[static_cast<size_t>(bh % x.H) * x.nqb + row / kBQ];
  const float* mp = x.mu32 + static_cast<size_t>(bh) * kD + c8;
  float k8[8], d8[8], v[8];
  load8<T>(static_cast<const T*>(x.K) + e, k8);
  load8<float>(x.dO + e, d8);
  if (x.qbf_w != nullptr) {
    load8<T>(static_cast<const T*>(x.Q) + e, v);
    st_bf16x8(x.qbf_w + e, v);
  }
  if (x.vbf_w != nullptr) {
    load8<T>(static_cast<const T*>(x.V) + e, v);
    st_bf16x8(x.vbf_w + e, v);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    k8[k] -= mp[k];
    d8[k] *= al;
  }
  st_bf16x8(x.ksb + e, k8);
  st_bf16x8(x.dos + e, d8);
}

// ---------------------------------------------------------------- key_lists
// grid (ceil(nkb / 4), BH), 256 threads; wavefront w compacts mask column j = 4 x + w: the
// ascending query blocks whose mask row keeps key block j (mask already 0/1).
__global__ __launch_bounds__(256) void key_lists_kernel(const uint8_t* __restrict__ mask,
                                                        int32_t* __restrict__ tcnt,
                                                        uint16_t* __restrict__ tlist, int nqb,
                                                        int nkb) {
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int j = 4 * blockIdx.x + (threadIdx.x >> 6);
  if (j >= nkb) return;
  const uint8_t* m = mask + static_cast<size_t>(bh) * nqb * nkb + j;
  uint16_t* out = tlist + (static_cast<size_t>(bh) * nkb + j) * nqb;
  int before = 0;
  for (int i0 = 0; i0 < nqb; i0 += 64) {
    const int i = i0 + lane;
    const bool sel = i < nqb && m[static_cast<size_t>(i) * nkb] != 0;
    const uint64_t b = __ballot(sel);
    if (sel) out[before + lanes_below(b)] = static_cast<uint16_t>(i);
    before += __popcll(b);
  }
  if (lane == 0) tcnt[static_cast<size_t>(bh) * nkb + j] = before;
}

// ---------------------------------------------------------------- key_plan
// grid (BH), 1024 threads. Long key lists are cut into work items of at most C query blocks,
// C = max(kChunk, ceil(2 P / nkb)) for P kept pairs in the head, so the number of items past
// the first of each key block is at most P / C <= nkb / 2 (the capacity `cap`). Writes C and
// that count to plan[bh], the first extra item of every key block to xoff, and the items
// (j << 16 | chunk) in key-block order.
__global__ __launch_bounds__(1024) void key_plan_kernel(const int32_t* __restrict__ tcnt,
                                                        int32_t* __restrict__ plan,
                                                        int32_t* __restrict__ xoff,
                                                        int32_t* __restrict__ items, int nkb,
                                                        int cap) {
  __shared__ int wsum[16];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int32_t* tc = tcnt + static_cast<size_t>(bh) * nkb;
  int p = 0;
  for (int j = t; j < nkb; j += 1024) p += tc[j];
  for (int o = 32; o >= 1; o >>= 1) p += __shfl_xor(p, o);
  if (lane == 0) wsum[w] = p;
  __syncthreads();
  int P = 0;
  for (int k = 0; k < 16; ++k) P += wsum[k];
  const int C = max(kChunk, (2 * P + nkb - 1) / nkb);
  int base = 0;
  for (int j0 = 0; j0 < nkb; j0 += 1024) {
    __syncthreads();   // wsum reuse
    const int j = j0 + t;
    const int e = j < nkb ? max(0, (tc[j] + C - 1) / C - 1) : 0;
    int inc = e;   // inclusive scan within the wavefront
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int before = base;
    for (int k = 0; k < w; ++k) before += wsum[k];
    const int off = before + inc - e;
    if (j < nkb) {
      xoff[static_cast<size_t>(bh) * nkb + j] = off;
      for (int c = 1; c <= e; ++c)
        if (off + c - 1 < cap) items[static_cast<size_t>(bh) * cap + off + c - 1] = (j << 16) | c;
    }
    for (int k = 0; k < 16; ++k) base += wsum[k];
  }
  if (t == 0) {
    plan[2 * bh] = C;
    plan[2 * bh + 1] = min(base, cap);
  }
}

// ---------------------------------------------------------------- bwd_lin_q
// grid (nqb, BH) (XCD-aware order), 512 threads; MFMA 16x16x32 bf16. Wavefront w owns query
// rows 16 w .. +15 (the lane's column) for num^T = H_i^T a^T and da^T = H_i dnum^T (the query
// as column, so row sums are per lane plus the four lane groups), and o rows 16 w .. +15 of
// dH_i^T = dnum^T a. LDS (two bf16 tiles, so that two workgroups fit per CU): a = phi(Q_i)
// [q][a], and one tile that holds H_i^T [o][a], then dnum [q][o], then the dH_i^T staging.
constexpr int kLinT = 512;
template <typename T>
__global__ __launch_bounds__(kLinT) void bwd_lin_q_kernel(BwdArgs x) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kTile];   // a = phi(Q_i) [q][a]
  __shared__ __attribute__((aligned(16))) uint16_t Ht[kTile];   // H_i^T [o][a]; dnum; dH_i^T
  uint16_t* const DN = Ht;                                      // dnum [q][o]
  __shared__ float Zs[kD], ddl[kD], red[8], zq[4][kD];
  int i, bh;
  xcd_block(x.nqb, x.BH, &i, &bh);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, G = lane >> 4, l16 = lane & 15;
  const int N = x.nqb * kBQ, nkb = x.nkb;
  const size_t qb = static_cast<size_t>(bh) * x.nqb + i;
  const size_t row0 = static_cast<size_t>(bh) * N + static_cast<size_t>(i) * kBQ;
  const int ncnt = x.cnt[qb];
  const float al = x.alpha[static_cast<size_t>(bh % x.H) * x.nqb + i];
  if (ncnt == nkb) {   // nothing dropped: O_l = 0, no linear gradient
    for (int e = t; e < kBQ * kD / 4; e += kLinT)
      *reinterpret_cast<f32x4*>(x.dQ + row0 * kD + 4 * e) = f32x4{};
    for (int e = t; e < kD * kD / 8; e += kLinT)
      *reinterpret_cast<i32x4*>(x.dht + qb * (kD * kD) + 8 * e) = i32x4{};
    if (t < kD) x.dz[qb * kD + t] = 0.f;
    if (t == 0) x.dalpha[qb] = 0.f;
    return;
  }
  // ---- a = phi(Q_i): thread t takes row t / 4, columns 32 (t % 4) .. +31
  {
    const int r = t >> 2, c0 = 32 * (t & 3);
    const T* qp = static_cast<const T*>(x.Q) + (row0 + r) * kD + c0;
    float v[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(qp + 8 * u, v + 8 * u);
    float mx = v[0];
#pragma unroll
    for (int k = 1; k < 32; ++k) mx = fmaxf(mx, v[k]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      v[k] = __expf(v[k] - mx);
      sum += v[k];
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int k = 0; k < 32; ++k) v[k] *= inv;
#pragma unroll
    for (int u = 0; u < 4; ++u) st_bf16x8(&As[r * kLd + c0 + 8 * u], v + 8 * u);
  }
  // ---- H_i = H_tot - sum over kept j of h_j. h_j^T bf16 in fragment order: 16-byte chunk c
  // holds row o = 32 (c / 512) + c % 32, columns a = 8 ((c / 32) % 16) .. +7. Thread t takes
  // chunks t + 512 u.
  {
    const int32_t* lst = x.list + qb * nkb;
    float acc[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[u][k] = 0.f;
    sum_tiles512(acc, x.hbf + static_cast<size_t>(bh) * nkb * (kD * kD),
                 [&](int n) { return lst[n]; }, 0, ncnt, t);
    const float* ht = x.htot + static_cast<size_t>(bh) * (kD * kD);   // H_tot [a][o]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = t + kLinT * u;
      const int o = 32 * (c >> 9) + (c & 31), a0 = 8 * ((c >> 5) & 15);
      float hv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) hv[k] = ht[(a0 + k) * kD + o] - acc[u][k];
      st_bf16x8(&Ht[o * kLd + a0], hv);
    }
    if (t < kD) {
      const float zs = sum_rows(x.z + static_cast<size_t>(bh) * nkb * kD,
                                [&](int n) { return lst[n]; }, 0, ncnt, t);
      Zs[t] = x.ztot[static_cast<size_t>(bh) * kD + t] - zs;
    }
  }
  __syncthreads();
  // ---- num^T = H_i^T a^T: lane = query q = 16 w + l16, registers = o (tile ot: 16 ot + 4 G + r)
  const int q = 16 * w + l16;
  f32x4 num[8];
#pragma unroll
  for (int ot = 0; ot < 8; ++ot) {
    num[ot] = f32x4{};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      num[ot] = mfma16(ld_row8(&Ht[(16 * ot + l16) * kLd + 32 * c + 8 * G]),
                       ld_row8(&As[q * kLd + 32 * c + 8 * G]), num[ot]);
  }
  float den = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float f[8];
    unpack_bf16x8(*reinterpret_cast<const i32x4*>(&As[q * kLd + 32 * G + 8 * u]), f);
#pragma unroll
    for (int k = 0; k < 8; ++k) den += f[k] * Zs[32 * G + 8 * u + k];
  }
  den = group4_sum(den);
  const float oml = 1.0f - al, inv_den = 1.0f / den;
  // O_l = num / den; sum(dO O_l) per row; dnum = (1 - alpha) dO / den (in num's registers)
  float sl = 0.f;
  {
    const float* dop = x.dO + (row0 + q) * kD + 4 * G;
#pragma unroll
    for (int ot = 0; ot < 8; ++ot) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dop + 16 * ot);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sl += d4[r] * (num[ot][r] * inv_den);
        num[ot][r] = oml * d4[r] * inv_den;
      }
    }
  }
  sl = group4_sum(sl);
  const float dden = -oml * sl * inv_den;
  {
    const float ws = wave_sum(G == 0 ? sl : 0.f);
    if (lane == 0) red[w] = ws;
  }
  // ---- da^T = H_i dnum^T (+ dden Z_i): lane = q, registers = a; dQ = a (da - rowsum(da a))
  {
    f32x4 da[8];
#pragma unroll
    for (int at = 0; at < 8; ++at) {
      da[at] = f32x4{};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        da[at] = mfma16(ld_col8_16(Ht, 16 * at, 32 * c, G, lane), acc_op16(num[2 * c], num[2 * c + 1]),
                        da[at]);
    }
    float av[8][4];
    float cs = 0.f;
#pragma unroll
    for (int at = 0; at < 8; ++at) {
      const int a0 = 16 * at + 4 * G;
      const uint2 pv = *reinterpret_cast<const uint2*>(&As[q * kLd + a0]);
      av[at][0] = __uint_as_float(pv.x << 16);
      av[at][1] = __uint_as_float(pv.x & 0xFFFF0000u);
      av[at][2] = __uint_as_float(pv.y << 16);
      av[at][3] = __uint_as_float(pv.y & 0xFFFF0000u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        da[at][r] += dden * Zs[a0 + r];
        cs += da[at][r] * av[at][r];
      }
    }
    cs = group4_sum(cs);
    float* dqp = x.dQ + (row0 + q) * kD + 4 * G;
#pragma unroll
    for (int at = 0; at < 8; ++at) {
      f32x4 o4;
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = av[at][r] * (da[at][r] - cs);
      *reinterpret_cast<f32x4*>(dqp + 16 * at) = o4;
    }
  }
  // ---- dnum -> LDS [q][o] (bf16, over H_i^T once every wavefront is done with it), dden
  __syncthreads();
#pragma unroll
  for (int ot = 0; ot < 8; ++ot)
    *reinterpret_cast<uint2*>(&DN[q * kLd + 16 * ot + 4 * G]) =
        make_uint2(pack_bf16x2(num[ot][0], num[ot][1]), pack_bf16x2(num[ot][2], num[ot][3]));
  if (G == 0) ddl[q] = dden;
  __syncthreads();
  // ---- dH_i^T [o][a] = sum_q dnum[q][o] a[q][a]: wavefront w owns o = 16 w .. +15; staged as
  // bf16 over dnum once every wavefront is done with it, and stored in 16-byte pieces
  f32x4 dh[8];
#pragma unroll
  for (int at = 0; at < 8; ++at) {
    dh[at] = f32x4{};
#pragma unroll
    for (int cq = 0; cq < 4; ++cq)
      dh[at] = mfma16(ld_col8n_16(DN, 16 * w, 32 * cq, G, lane), ld_col8n_16(As, 16 * at, 32 * cq, G, lane),
                      dh[at]);
  }
  // dZ_i[a] = sum_q a[q][a] dden[q]: four threads per column, 32 query rows each
  {
    const int a = t & (kD - 1), h = t >> 7;
    float s = 0.f;
#pragma unroll 8
    for (int r = 32 * h; r < 32 * h + 32; ++r) s += bf(As[r * kLd + a]) * ddl[r];
    zq[h][a] = s;
  }
  __syncthreads();
#pragma unroll
  for (int at = 0; at < 8; ++at) {
    const int a = 16 * at + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) Ht[(16 * w + 4 * G + r) * kLd + a] = f32_to_bf16_rne(dh[at][r]);
  }
  __syncthreads();
  if (t < kD) x.dz[qb * kD + t] = (zq[0][t] + zq[1][t]) + (zq[2][t] + zq[3][t]);
  {
    uint16_t* out = x.dht + qb * (kD * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = t + kLinT * u, o = c >> 4, a0 = 8 * (c & 15);
      *reinterpret_cast<i32x4*>(out + o * kD + a0) = *reinterpret_cast<const i32x4*>(&Ht[o * kLd + a0]);
    }
  }
  if (t == 0) {
    float sdl = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) sdl += red[k];
    x.dalpha[qb] = -sdl;
  }
}

// ---------------------------------------------------------------- bwd_q
// grid (nqb, BH), plain block order, 512 threads. MFMA 16x16x32 bf16 (A lane (G = lane / 16,
// l = lane % 16): row l, k = 8 G .. +7; B: column l, same k; accumulator: column l, rows
// 4 G .. +3). Wavefront w owns query rows 16 w .. +15 and holds S^T = K_s,j Q^T with the query
// as column (lane) and the 64 keys in its four 16-row tiles, so row statistics are per lane
// plus a reduction over the four lane groups. Its Q and dO_s rows stay in registers as B
// operands. K_s and V tiles are double-buffered in LDS; the next-but-one block is loaded into
// registers while the current one is processed (one barrier per block). Logits are kept in
// base-2 units: s2 = S log2(e) / sqrt(d).
constexpr int kQThreads = 512;
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(4))) void bwd_q_kernel(BwdArgs x) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBK * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBK * kLd];
  __shared__ float red[8];
  int i, bh;
  i = blockIdx.x;
  bh = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, G = lane >> 4, l16 = lane & 15;
  const int N = x.nqb * kBQ, nkb = x.nkb;
  const size_t qb = static_cast<size_t>(bh) * x.nqb + i;
  const size_t head = static_cast<size_t>(bh) * N;
  const size_t row0 = head + static_cast<size_t>(i) * kBQ;
  const int ncnt = x.cnt[qb];
  if (ncnt == 0) {   // nothing kept: O_s = 0, no sparse gradient
    if (t < kBQ) {
      x.lse2[row0 + t] = 0.f;
      x.Dd[row0 + t] = 0.f;
    }
    return;
  }
  const float al = x.alpha[static_cast<size_t>(bh % x.H) * x.nqb + i];
  const int q = 16 * w + l16;
  bf16x8 qop[4], dop[4];   // B operands: row q, d = 32 c + 8 G .. +7 (dO_s: loaded for pass 2)
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(x.qbf + (row0 + q) * kD + 32 * c + 8 * G));
  const int32_t* lst = x.list + qb * nkb;
  const float c2 = kLog2e * kInvSqrtD;
  i32x4 pk[2], pv[2];
  auto fetch = [&](int j) {
    const size_t kr = head + static_cast<size_t>(j) * kBK;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ch = t + kQThreads * u;
      const size_t e = (kr + (ch >> 4)) * kD + 8 * (ch & 15);
      pk[u] = *reinterpret_cast<const i32x4*>(x.ksb + e);
      pv[u] = *reinterpret_cast<const i32x4*>(x.vbf + e);
    }
  };
  auto put = [&](int b) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ch = t + kQThreads * u;
      const int o = (ch >> 4) * kLd + 8 * (ch & 15);
      *reinterpret_cast<i32x4*>(&Ks[b][o]) = pk[u];
      *reinterpret_cast<i32x4*>(&Vs[b][o]) = pv[u];
    }
  };
  auto scores = [&](const uint16_t* kt, f32x4 (&sT)[4]) {
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      sT[T] = f32x4{};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sT[T] = mfma16(ld_row8(&kt[(16 * T + l16) * kLd + 32 * c + 8 * G]), qop[c], sT[T]);
    }
  };
  // ---- pass 1: running max m and sum l (per lane: its 16 keys of each block), O_s^T
  float m = -INFINITY, l = 0.f;
  f32x4 oT[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oT[dt] = f32x4{};
  fetch(lst[0]);
  put(0);
  __syncthreads();
  if (ncnt > 1) fetch(lst[1]);
  for (int n = 0; n < ncnt; ++n) {
    const int b = n & 1;
    f32x4 sT[4];
    scores(Ks[b], sT);
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sT[T][r]);
    mx = group4_max(mx);
    const float mn = fmaxf(m, mx * c2);
    const float corr = exp2f(m - mn);
    float ls = 0.f;
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(sT[T][r] * c2 - mn);
        sT[T][r] = p;
        ls += p;
      }
    l = l * corr + ls;
    m = mn;
    if (__ballot(corr != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oT[dt] *= corr;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        oT[dt] = mfma16(ld_col8_16(Vs[b], 16 * dt, 32 * cc, G, lane),
                        acc_op16(sT[2 * cc], sT[2 * cc + 1]), oT[dt]);
    if (n + 1 < ncnt) put(b ^ 1);
    __syncthreads();
    if (n + 2 < ncnt) fetch(lst[n + 2]);
  }
  fetch(lst[0]);   // pass 2 starts over; in flight during the row statistics below
  const float lt = group4_sum(l);
  const float lse = m + log2f(lt);
  const float invl = 1.0f / lt;
  float sd = 0.f;
  {
    const float* dp_ = x.dO + (row0 + q) * kD + 4 * G;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dp_ + 16 * dt);
#pragma unroll
      for (int r = 0; r < 4; ++r) sd += d4[r] * (oT[dt][r] * invl);
    }
  }
  sd = group4_sum(sd);
  const float Dq = al * sd;
  if (G == 0) {
    x.lse2[row0 + q] = lse;
    x.Dd[row0 + q] = Dq;
  }
  {
    const float ws = wave_sum(G == 0 ? sd : 0.f);
    if (lane == 0) red[w] = ws;
  }
  // ---- pass 2: P^T, dP^T = V_j dO_s^T, dS^T = P^T (dP^T - D), dQ^T += K_s,j^T dS^T
#pragma unroll
  for (int c = 0; c < 4; ++c)
    dop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(x.dos + (row0 + q) * kD + 32 * c + 8 * G));
  put(0);
  __syncthreads();
  if (ncnt > 1) fetch(lst[1]);
  f32x4 dq[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dq[dt] = f32x4{};
  for (int n = 0; n < ncnt; ++n) {
    const int b = n & 1;
    f32x4 sT[4], dp[4];
    scores(Ks[b], sT);
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      dp[T] = f32x4{};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        dp[T] = mfma16(ld_row8(&Vs[b][(16 * T + l16) * kLd + 32 * c + 8 * G]), dop[c], dp[T]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(sT[T][r] * c2 - lse);
        dp[T][r] = p * (dp[T][r] - Dq);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        dq[dt] = mfma16(ld_col8_16(Ks[b], 16 * dt, 32 * cc, G, lane),
                        acc_op16(dp[2 * cc], dp[2 * cc + 1]), dq[dt]);
    if (n + 1 < ncnt) put(b ^ 1);
    __syncthreads();
    if (n + 2 < ncnt) fetch(lst[n + 2]);
  }
  {
    float* dqp = x.dQ + (row0 + q) * kD + 4 * G;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      f32x4* p = reinterpret_cast<f32x4*>(dqp + 16 * dt);
      f32x4 v = *p;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += dq[dt][r] * kInvSqrtD;
      *p = v;
    }
  }
  if (t == 0) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += red[k];
    x.dalpha[qb] += s;
  }
}

// ---------------------------------------------------------------- bwd_kv
// One work item = one key block j and a range of its keeping query blocks; 512 threads.
// Wavefront w = (kt = w % 4, qh = w / 4): keys 16 kt .. +15 and, in the sparse loop, query rows
// 64 qh .. +63 of each query block. MFMA 16x16x32 bf16 with S = Q K_s^T and dP = dO_s V^T held
// with the key as column (lane) and the query in registers, so P and dS are directly the A
// operand of dV = P^T dO_s and dK = dS^T Q; the B operands run down the columns of the Q and
// dO_s tiles (transposing LDS read). K_s and V rows of the wavefront's keys stay in registers.
// Q and dO_s tiles are double-buffered in LDS, the next-but-one query block loaded into
// registers while the current one is processed. dK and dV accumulate as eight 16 x 16 tiles
// (lane = d, registers = keys); after the loop the two query halves are summed through LDS so
// that wavefront (kt, qh) holds the totals of d tiles 4 qh .. 4 qh + 3.
constexpr int kKvT = 512;
constexpr int kXld = kD + 4;   // fp32 row stride of the exchange tiles
// LDS (bytes): Q tiles [2] at 0, dO_s tiles [2] at 69632, lse [2][128] and D [2][128] at
// 139264; after the loop the first 122880 bytes hold the exchange tiles (fp32 [2][64][kXld]),
// phi(K_s,j) (bf16 [64][kLd]), dh_j^T (bf16 [128][kLd]), dz_j, row and column sums.
constexpr int kKvLds = 4 * kTile * 2 + 4 * kBQ * 4;
constexpr int kOffX = 0, kOffPK = 67584, kOffDH = 84992, kOffDz = 119808, kOffCrow = 120320,
              kOffKred = 120832;

struct KvState {
  f32x4 dk[8], dv[8];   // lane = d column 16 dt + l16, registers = keys 16 kt + 4 G + r
};

// The sparse loop over tl[n0 .. n1) plus the query-half exchange. On return, the wavefront's
// dk[4 qh .. 4 qh + 3] (scaled by 1 / sqrt(d)) and dv[4 qh .. 4 qh + 3] are its key block's totals
// over the range.
__device__ inline void kv_sparse(const BwdArgs& x, size_t head, const uint16_t* tl, int n0,
                                 int n1, char* smem, const bf16x8 (&kop)[4],
                                 const bf16x8 (&vop)[4], KvState& st, int t, int lane, int G,
                                 int l16, int kt, int qh) {
  uint16_t* const Q0 = reinterpret_cast<uint16_t*>(smem);   // Q tiles b = 0, 1; dO_s at + 2 kTile
  float* lse_s = reinterpret_cast<float*>(smem + 4 * kTile * 2);   // [2][128]
  float* D_s = lse_s + 2 * kBQ;                                     // [2][128]
  const float c2 = kLog2e * kInvSqrtD;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    st.dk[dt] = f32x4{};
    st.dv[dt] = f32x4{};
  }
  i32x4 pq[4], pd[4];
  float pl = 0.f, pD = 0.f;
  auto fetch = [&](int i) {
    const size_t row0 = head + static_cast<size_t>(i) * kBQ;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ch = t + kKvT * u;
      const size_t e = (row0 + (ch >> 4)) * kD + 8 * (ch & 15);
      pq[u] = *reinterpret_cast<const i32x4*>(x.qbf + e);
      pd[u] = *reinterpret_cast<const i32x4*>(x.dos + e);
    }
    if (t < kBQ) {
      pl = x.lse2[row0 + t];
      pD = x.Dd[row0 + t];
    }
  };
  auto put = [&](int b) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ch = t + kKvT * u;
      const int o = (ch >> 4) * kLd + 8 * (ch & 15);
      *reinterpret_cast<i32x4*>(&Q0[b * kTile + o]) = pq[u];
      *reinterpret_cast<i32x4*>(&Q0[(2 + b) * kTile + o]) = pd[u];
    }
    if (t < kBQ) {
      lse_s[b * kBQ + t] = pl;
      D_s[b * kBQ + t] = pD;
    }
  };
  if (n0 < n1) {
    fetch(tl[n0]);
    put(0);
    __syncthreads();
    if (n0 + 1 < n1) fetch(tl[n0 + 1]);
  }
  for (int n = n0; n < n1; ++n) {
    const int b = (n - n0) & 1;
    const uint16_t* Q = Q0 + b * kTile;
    const uint16_t* Dm = Q0 + (2 + b) * kTile;
    f32x4 s[4], ds[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int qr = 64 * qh + 16 * T;
      f32x4 sv = f32x4{}, dp = f32x4{};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sv = mfma16(ld_row8(&Q[(qr + l16) * kLd + 32 * c + 8 * G]), kop[c], sv);
        dp = mfma16(ld_row8(&Dm[(qr + l16) * kLd + 32 * c + 8 * G]), vop[c], dp);
      }
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[b * kBQ + qr + 4 * G]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&D_s[b * kBQ + qr + 4 * G]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(sv[r] * c2 - l4[r]);
        s[T][r] = p;
        ds[T][r] = p * (dp[r] - d4[r]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        st.dv[dt] = mfma16(acc_op16(s[2 * cc], s[2 * cc + 1]),
                           ld_col8_16(Dm, 16 * dt, 64 * qh + 32 * cc, G, lane), st.dv[dt]);
        st.dk[dt] = mfma16(acc_op16(ds[2 * cc], ds[2 * cc + 1]),
                           ld_col8_16(Q, 16 * dt, 64 * qh + 32 * cc, G, lane), st.dk[dt]);
      }
    if (n + 1 < n1) put(b ^ 1);
    __syncthreads();
    if (n + 2 < n1) fetch(tl[n + 2]);
  }
  // exchange: send the other half's d tiles, receive the partner's contribution to ours
  float* X = reinterpret_cast<float*>(smem + kOffX);   // [2][64][kXld]
  __syncthreads();
  // (tile indices stay compile-time constants: the wavefront's half is a uniform predicate)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    if ((dt >> 2) == qh) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kt + 4 * G + r;
      X[key * kXld + 16 * dt + l16] = st.dk[dt][r];
      X[(kBK + key) * kXld + 16 * dt + l16] = st.dv[dt][r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    if ((dt >> 2) != qh) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kt + 4 * G + r;
      st.dk[dt][r] = (st.dk[dt][r] + X[key * kXld + 16 * dt + l16]) * kInvSqrtD;
      st.dv[dt][r] += X[(kBK + key) * kXld + 16 * dt + l16];
    }
  }
  __syncthreads();   // X free again
}

__device__ inline void load_kv_ops(const BwdArgs& x, size_t krow0, int kt, int G, int l16,
                                   bf16x8 (&kop)[4], bf16x8 (&vop)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const size_t e = (krow0 + 16 * kt + l16) * kD + 32 * c + 8 * G;
    kop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(x.ksb + e));
    vop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(x.vbf + e));
  }
}

// Extra work items: grid (cap, BH); item e < plan[bh].count covers the query blocks
// [c C, min((c + 1) C, T_j)) of key block j; writes its partial dK_s, dV ([64][128] each) and
// the sums of dH_i^T and dZ_i over its query blocks into slot e.
__global__ __launch_bounds__(kKvT) void bwd_kv_extra_kernel(BwdArgs x) {
  __shared__ __attribute__((aligned(16))) char smem[kKvLds];
  const int e = blockIdx.x, bh = blockIdx.y;
  if (e >= x.plan[2 * bh + 1]) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, G = lane >> 4, l16 = lane & 15;
  const int kt = w & 3, qh = w >> 2;
  const int item = x.items[static_cast<size_t>(bh) * x.cap + e];
  const int j = item >> 16, c = item & 0xFFFF, C = x.plan[2 * bh];
  const int nqb = x.nqb, N = nqb * kBQ;
  const size_t head = static_cast<size_t>(bh) * N;
  const size_t krow0 = head + static_cast<size_t>(j) * kBK;
  const int nT = x.tcnt[static_cast<size_t>(bh) * x.nkb + j];
  const uint16_t* tl = x.tlist + (static_cast<size_t>(bh) * x.nkb + j) * nqb;
  const int n0 = c * C, n1 = min(nT, n0 + C);
  bf16x8 kop[4], vop[4];
  load_kv_ops(x, krow0, kt, G, l16, kop, vop);
  KvState st;
  kv_sparse(x, head, tl, n0, n1, smem, kop, vop, st, t, lane, G, l16, kt, qh);
  float* slot = x.xpart + (static_cast<size_t>(bh) * x.cap + e) * kSlot;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    if ((dt >> 2) != qh) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kt + 4 * G + r;
      slot[key * kD + 16 * dt + l16] = st.dk[dt][r];
      slot[kBK * kD + key * kD + 16 * dt + l16] = st.dv[dt][r];
    }
  }
  // sums of dH_i^T (chunk f = t + 512 u: 8 elements at 8 f) and dZ_i over the range
  float acc[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[u][k] = 0.f;
  sum_tiles512(acc, x.dht + static_cast<size_t>(bh) * nqb * (kD * kD), [&](int n) { return static_cast<int>(tl[n]); }, n0, n1, t);
  float* sh = slot + 2 * kBK * kD;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int f = t + kKvT * u;
    *reinterpret_cast<f32x4*>(sh + 8 * f) = f32x4{acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
    *reinterpret_cast<f32x4*>(sh + 8 * f + 4) = f32x4{acc[u][4], acc[u][5], acc[u][6], acc[u][7]};
  }
  if (t < kD)
    sh[kD * kD + t] = sum_rows(x.dz + static_cast<size_t>(bh) * nqb * kD,
                               [&](int n) { return static_cast<int>(tl[n]); }, n0, n1, t);
}

// Main work items: grid (nkb, BH), plain block order (all XCDs on the same head at a time: its
// Q and dO_s tiles, read once per keeping pair, stay in the shared cache). Key block j: its first C keeping query
// blocks, then the extra items' partials in item order, then the linear part; writes dK_s, dV
// and the column sums of dK_s.
__global__ __launch_bounds__(kKvT) void bwd_kv_kernel(BwdArgs x) {
  __shared__ __attribute__((aligned(16))) char smem[kKvLds];
  uint16_t* PK = reinterpret_cast<uint16_t*>(smem + kOffPK);   // phi(K_s,j) [64][kLd]
  uint16_t* DH = reinterpret_cast<uint16_t*>(smem + kOffDH);   // dh_j^T [o][a]
  float* dz_s = reinterpret_cast<float*>(smem + kOffDz);        // [128]
  float* crow = reinterpret_cast<float*>(smem + kOffCrow);      // [2][64]
  float* kred = reinterpret_cast<float*>(smem + kOffKred);      // [4][128]
  int j, bh;
  j = blockIdx.x;
  bh = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, G = lane >> 4, l16 = lane & 15;
  const int kt = w & 3, qh = w >> 2;
  const int nqb = x.nqb, N = nqb * kBQ;
  const size_t head = static_cast<size_t>(bh) * N;
  const size_t krow0 = head + static_cast<size_t>(j) * kBK;
  const int nT = x.tcnt[static_cast<size_t>(bh) * x.nkb + j];
  const uint16_t* tl = x.tlist + (static_cast<size_t>(bh) * x.nkb + j) * nqb;
  const int C = x.plan[2 * bh];
  const int n1 = min(nT, C);
  const int nx = nT > C ? (nT + C - 1) / C - 1 : 0;
  const float* xs = x.xpart + (static_cast<size_t>(bh) * x.cap + x.xoff[static_cast<size_t>(bh) * x.nkb + j]) * kSlot;
  bf16x8 kop[4], vop[4];
  load_kv_ops(x, krow0, kt, G, l16, kop, vop);
  KvState st;
  kv_sparse(x, head, tl, 0, n1, smem, kop, vop, st, t, lane, G, l16, kt, qh);
  // the linear part's independent loads, issued together before they are needed: the K_s
  // rows for phi (thread: row t / 8, columns 16 (t % 8) .. +15) and dH_tot^T (chunks t + 512 u)
  i32x4 kraw[2];
  f32x4 tot4[4][2];
  {
    const int r = t >> 3, c0 = 16 * (t & 7);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      kraw[u] = *reinterpret_cast<const i32x4*>(x.ksb + (krow0 + r) * kD + c0 + 8 * u);
    const float* tot = x.dhtot + static_cast<size_t>(bh) * (kD * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = t + kKvT * u;
      tot4[u][0] = *reinterpret_cast<const f32x4*>(tot + 8 * f);
      tot4[u][1] = *reinterpret_cast<const f32x4*>(tot + 8 * f + 4);
    }
  }
  // partials of the extra items (fixed order)
  for (int e = 0; e < nx; ++e) {
    const float* sl = xs + static_cast<size_t>(e) * kSlot;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if ((dt >> 2) != qh) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * kt + 4 * G + r;
        st.dk[dt][r] += sl[key * kD + 16 * dt + l16];
        st.dv[dt][r] += sl[kBK * kD + key * kD + 16 * dt + l16];
      }
    }
  }
  // ---- linear part. phi(K_s,j)
  {
    const int r = t >> 3, c0 = 16 * (t & 7);
    float v[16];
#pragma unroll
    for (int u = 0; u < 2; ++u) unpack_bf16x8(kraw[u], v + 8 * u);
    float mx = v[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) mx = fmaxf(mx, v[k]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v[k] = __expf(v[k] - mx);
      s += v[k];
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    const float inv = 1.0f / s;
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] *= inv;
#pragma unroll
    for (int u = 0; u < 2; ++u) st_bf16x8(&PK[r * kLd + c0 + 8 * u], v + 8 * u);
  }
  // dh_j^T = dH_tot^T - sum over the keeping query blocks of dH_i^T; dz_j
  {
    float acc[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[u][k] = 0.f;
    sum_tiles512(acc, x.dht + static_cast<size_t>(bh) * nqb * (kD * kD), [&](int n) { return static_cast<int>(tl[n]); }, 0, n1, t);
    for (int e = 0; e < nx; ++e) {
      const float* sh = xs + static_cast<size_t>(e) * kSlot + 2 * kBK * kD;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = t + kKvT * u;
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(sh + 8 * f);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(sh + 8 * f + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[u][k] += a0[k];
          acc[u][4 + k] += a1[k];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = t + kKvT * u, o = f >> 4, a0 = 8 * (f & 15);
      const f32x4 t0 = tot4[u][0], t1 = tot4[u][1];
      float hv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
      for (int k = 0; k < 8; ++k) hv[k] -= acc[u][k];
      st_bf16x8(&DH[o * kLd + a0], hv);
    }
    if (t < kD) {
      float s = sum_rows(x.dz + static_cast<size_t>(bh) * nqb * kD,
                         [&](int n) { return static_cast<int>(tl[n]); }, 0, n1, t);
      for (int e = 0; e < nx; ++e) s += xs[static_cast<size_t>(e) * kSlot + 2 * kBK * kD + kD * kD + t];
      dz_s[t] = x.dztot[static_cast<size_t>(bh) * kD + t] - s;
    }
  }
  __syncthreads();
  // dV += phi dh_j (o tiles 4 qh .. +3); dphi = V dh_j^T + dz_j (a tiles 4 qh .. +3)
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 dph[8];
#pragma unroll
  for (int ot = 0; ot < 8; ++ot) {
    dph[ot] = f32x4{};
    if ((ot >> 2) != qh) continue;
    f32x4 cv = f32x4{}, cp = f32x4{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      cv = mfma16(ld_row8(&PK[(16 * kt + l16) * kLd + 32 * c + 8 * G]),
                  ld_row8(&DH[(16 * ot + l16) * kLd + 32 * c + 8 * G]), cv);
      cp = mfma16(vop[c], ld_col8n_16(DH, 16 * ot, 32 * c, G, lane), cp);
    }
    st.dv[ot] += cv;
    const int a = 16 * ot + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kt + 4 * G + r;
      cp[r] += dz_s[a];
      cs[r] += cp[r] * bf(PK[key * kLd + a]);
    }
    dph[ot] = cp;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    cs[r] = row16_sum(cs[r]);
    if (l16 == 0) crow[qh * kBK + 16 * kt + 4 * G + r] = cs[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = 16 * kt + 4 * G + r;
    cs[r] = crow[key] + crow[kBK + key];
  }
#pragma unroll
  for (int at = 0; at < 8; ++at) {
    if ((at >> 2) != qh) continue;
    const int a = 16 * at + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kt + 4 * G + r;
      st.dk[at][r] += bf(PK[key * kLd + a]) * (dph[at][r] - cs[r]);
    }
  }
  // ---- write dK_s, dV; column sums of dK_s for the centring
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    if ((dt >> 2) != qh) continue;
    const int d = 16 * dt + l16;
    float cd = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t o = (krow0 + 16 * kt + 4 * G + r) * kD + d;
      x.dK[o] = st.dk[dt][r];
      x.dV[o] = st.dv[dt][r];
      cd += st.dk[dt][r];
    }
    cd += __shfl_xor(cd, 16);
    cd += __shfl_xor(cd, 32);
    if (G == 0) kred[kt * kD + d] = cd;
  }
  __syncthreads();
  if (t < kD)
    x.kcol[(static_cast<size_t>(bh) * x.nkb + j) * kD + t] =
        (kred[t] + kred[kD + t]) + (kred[2 * kD + t] + kred[3 * kD + t]);
}

// ---------------------------------------------------------------- dh_total
// grid (65, BH), 256 threads. Workgroup x < 64 sums elements 256 x .. +255 of dH_i^T over all
// query blocks: thread (chunk t % 32 of 8 elements, query-block group t / 32) sums the blocks
// i = group, group + 8, ...; the 8 group sums are added in a fixed order. Workgroup 64 sums dZ_i
// the same way (column t % 128, group t / 128).
__global__ __launch_bounds__(256) void dh_total_kernel(const uint16_t* __restrict__ dht,
                                                       const float* __restrict__ dz,
                                                       float* __restrict__ dhtot,
                                                       float* __restrict__ dztot, int nqb) {
  __shared__ float part[8][256 + 4];
  const int bh = blockIdx.y, t = threadIdx.x;
  if (blockIdx.x < 64) {
    const int ch = t & 31, grp = t >> 5;
    const size_t e = 256 * blockIdx.x + 8 * ch;
    const uint16_t* src = dht + static_cast<size_t>(bh) * nqb * (kD * kD) + e;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = grp; i < nqb; i += 8) {
      float f[8];
      unpack_bf16x8(*reinterpret_cast<const i32x4*>(src + static_cast<size_t>(i) * (kD * kD)), f);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += f[k];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) part[grp][8 * ch + k] = acc[k];
    __syncthreads();
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) v += part[q][t];
    dhtot[static_cast<size_t>(bh) * (kD * kD) + 256 * blockIdx.x + t] = v;
  } else {
    const int a = t & 127, grp = t >> 7;
    float s = 0.f;
    for (int i = grp; i < nqb; i += 2) s += dz[(static_cast<size_t>(bh) * nqb + i) * kD + a];
    part[grp][a] = s;
    __syncthreads();
    if (t < kD) dztot[static_cast<size_t>(bh) * kD + t] = part[0][t] + part[1][t];
  }
}

// ---------------------------------------------------------------- dK centring
// dk_mean: grid (BH), 1024 threads: column t % 128, key-block group t / 128 (8 groups, summed
// in a fixed order), divided by N.
__global__ __launch_bounds__(1024) void dk_mean_kernel(const float* __restrict__ kcol,
                                                       float* __restrict__ kmean, int nkb, int N) {
  __shared__ float part[8][kD];
  const int bh = blockIdx.x, t = threadIdx.x, col = t & 127, grp = t >> 7;
  const float* src = kcol + static_cast<size_t>(bh) * nkb * kD + col;
  // key blocks grp, grp + 8, ... in order; eight loads in flight
  float s = 0.f;
  int j = grp;
  for (; j + 56 < nkb; j += 64) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[static_cast<size_t>(j + 8 * u) * kD];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; j < nkb; j += 8) s += src[static_cast<size_t>(j) * kD];
  part[grp][col] = s;
  __syncthreads();
  if (t < kD) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) v += part[q][t];
    kmean[static_cast<size_t>(bh) * kD + t] = v / static_cast<float>(N);
  }
}
// dk_center: grid (N * d / 1024, BH), 256 threads: dK -= mean (four elements per thread).
__global__ __launch_bounds__(256) void dk_center_kernel(float* __restrict__ dK,
                                                        const float* __restrict__ kmean, int N) {
  const int bh = blockIdx.y;
  const size_t e = 1024 * static_cast<size_t>(blockIdx.x) + 4 * threadIdx.x;
  const f32x4 m = *reinterpret_cast<const f32x4*>(kmean + static_cast<size_t>(bh) * kD + (e & (kD - 1)));
  f32x4* p = reinterpret_cast<f32x4*>(dK + static_cast<size_t>(bh) * N * kD + e);
  *p = *p - m;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_key_lists(const Geom& g, const uint8_t* mask, int32_t* tcnt, uint16_t* tlist,
                            hipStream_t s) {
  hipLaunchKernelGGL(key_lists_kernel, dim3((g.nkb + 3) / 4, g.BH), dim3(256), 0, s, mask,
                     tcnt, tlist, g.nqb, g.nkb);
  return hipGetLastError();
}

hipError_t launch_key_plan(const Geom& g, const int32_t* tcnt, int32_t* plan, int32_t* xoff,
                           int32_t* items, int cap, hipStream_t s) {
  hipLaunchKernelGGL(key_plan_kernel, dim3(g.BH), dim3(1024), 0, s, tcnt, plan, xoff, items,
                     g.nkb, cap);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const Geom& g, int dtype, const BwdArgs& x, hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(bwd_prep_kernel<float>, dim3(g.N / 16, g.BH), dim3(256), 0, s, x);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<uint16_t>, dim3(g.N / 16, g.BH), dim3(256), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_bwd_lin_q(const Geom& g, int dtype, const BwdArgs& x, hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(bwd_lin_q_kernel<float>, dim3(g.nqb, g.BH), dim3(kLinT), 0, s, x);
  else
    hipLaunchKernelGGL(bwd_lin_q_kernel<uint16_t>, dim3(g.nqb, g.BH), dim3(kLinT), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_dh_total(const Geom& g, const BwdArgs& x, hipStream_t s) {
  hipLaunchKernelGGL(dh_total_kernel, dim3(65, g.BH), dim3(256), 0, s, x.dht, x.dz, x.dhtot,
                     x.dztot, g.nqb);
  return hipGetLastError();
}

hipError_t launch_bwd_q(const Geom& g, const BwdArgs& x, hipStream_t s) {
  hipLaunchKernelGGL(bwd_q_kernel, dim3(g.nqb, g.BH), dim3(kQThreads), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_bwd_kv_extra(const Geom& g, const BwdArgs& x, hipStream_t s) {
  hipLaunchKernelGGL(bwd_kv_extra_kernel, dim3(x.cap, g.BH), dim3(kKvT), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(const Geom& g, const BwdArgs& x, hipStream_t s) {
  hipLaunchKernelGGL(bwd_kv_kernel, dim3(g.nkb, g.BH), dim3(kKvT), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_dk_center(const Geom& g, const BwdArgs& x, hipStream_t s) {
  hipLaunchKernelGGL(dk_mean_kernel, dim3(g.BH), dim3(1024), 0, s, x.kcol, x.kmean, g.nkb, g.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dk_center_kernel, dim3(g.N * kD / 1024, g.BH), dim3(256), 0, s, x.dK,
                     x.kmean, g.N);
  return hipGetLastError();
}

}  // namespace sla2
