// Internal definitions shared by the SLA2 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sla2 {

constexpr int kD = 128;    // head dimension
constexpr int kBQ = 128;   // query block rows (b_q)
constexpr int kBK = 64;    // key block rows (b_k)
constexpr int kMaxN = 262144;
constexpr int kKpPerWg = 8;  // key blocks per workgroup in the linear precompute
constexpr int kChunk = 16;   // fewest query blocks per key-block work item of the backward
constexpr int kSlot = 2 * kBK * kD + kD * kD + kD;   // floats per extra backward work item

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Geom {
  int B, H, N, BH, nqb, nkb;
};

// ---------------------------------------------------------------- tile layouts
// INT8 K_s tiles: one 64 x 128 byte tile per key block, rows of 8 chunks of 16 B;
// chunk c of row r is stored at chunk position kchunk_swz(r, c) so that the 32
// rows one MFMA operand read touches spread over the LDS banks.
__host__ __device__ inline int kchunk_swz(int row, int chunk) {
  return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}
// E4M3 V tiles are stored transposed, [d = 128][64 keys], rows of 4 chunks of 16 B.
__host__ __device__ inline int vchunk_swz(int row, int chunk) {
  return chunk ^ (((row >> 1) & 3) ^ ((row >> 3) & 1));
}
// Key order inside a transposed V row. The 32x32 i32 accumulator of S^T = K Q^T
// gives lane group g (lanes 32g..32g+31) keys 32T + 8(i/4) + 4g + (i%4) in register i
// of key tile T. Packing those 32 values (byte b = 16T + i) as the B operand of the
// FP8 product means the A operand (V^T) must hold, in lane group g byte b, the same
// key; so position 32g + b of a V^T row holds key vkey_at(g, b).
__host__ __device__ inline int vkey_at(int g, int b) {
  return 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * g + (b & 3);
}
__host__ __device__ inline int vkey_pos(int key) {
  int T = key >> 5, r = key & 31;
  int g = (r & 7) >> 2;
  int b = 16 * T + 4 * (r >> 3) + (r & 3);
  return 32 * g + b;
}

// bf16 by the native conversion (round to nearest even)
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Load 8 consecutive input elements (fp32 or bf16) as fp32.
template <typename T>
__device__ inline void load8(const T* p, float* out);
template <>
__device__ inline void load8<float>(const float* p, float* out) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
  out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
}
template <>
__device__ inline void load8<uint16_t>(const uint16_t* p, float* out) {
  i32x4 v = *reinterpret_cast<const i32x4*>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w = static_cast<uint32_t>(v[k]);
    out[2 * k] = __uint_as_float(w << 16);
    out[2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------- XCD-aware block order
// The dispatcher hands workgroups to the 8 XCDs round-robin by linear block id. For a
// (query block, batch*head) grid this maps XCD x to the contiguous logical range
// [x * total / 8, (x + 1) * total / 8) of (bh, i) in row-major order, so query blocks of one
// head that run together share that XCD's L2 (their key tiles and h_j gathers).
__device__ inline void xcd_block(int nqb, int BH, int* i, int* bh) {
  const int total = nqb * BH;
  int L = blockIdx.x + gridDim.x * blockIdx.y;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  *i = L % nqb;
  *bh = L / nqb;
}

// Workgroup barrier for exchanges through LDS only: waits for this wavefront's LDS (and
// scalar) memory operations, lgkmcnt(0), then meets the other wavefronts. Unlike
// __syncthreads() it does not wait for outstanding global loads (vmcnt), so prefetches stay in
// flight across it; data loaded into LDS by global_load_lds must be waited for explicitly
// before it. The memory clobber keeps the compiler from moving memory accesses across it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------- wave helpers
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Reductions over the 16 lanes of one DPP row (lanes 16r .. 16r + 15); every lane of the
// row gets the result. Steps: swap neighbours, swap pairs (quad permutes), mirror each half
// row, mirror the row. Each lane combines the same two operands, so all lanes agree bitwise.
template <int kCtrl>
__device__ inline float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               kCtrl, 0xF, 0xF, false));
}
__device__ inline float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));   // row_mirror
  return v;
}
__device__ inline float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// ---------------------------------------------------------------- quantisation steps
// INT8: code = clamp(rne(fl32(x * inv)), -127, 127), inv = fl32(127 / amax) (0 if amax = 0).
// Computed as clamp first (one med3; the bounds are integers, so clamping before or after the
// rounding gives the same integer), then + 1.5 * 2^23: the fp32 add rounds to the nearest
// integer, ties to even (as rint), and leaves that integer in the low mantissa bits, whose low
// byte is the two's-complement code. i8_code returns the code in the low byte of a word whose
// other bytes are not zero; i8_pack4 keeps only the low bytes.
__device__ inline uint32_t i8_code(float x, float inv) {
  const float y = __builtin_amdgcn_fmed3f(x * inv, -127.f, 127.f);
  return __float_as_uint(y + 12582912.0f);   // 1.5 * 2^23
}
__device__ inline uint32_t i8_pack4(float a, float b, float c, float d, float inv) {
  const uint32_t ua = i8_code(a, inv) & 0xFFu, ub = i8_code(b, inv) & 0xFFu;
  const uint32_t uc = i8_code(c, inv) & 0xFFu, ud = i8_code(d, inv);
  return (ud << 24) | (uc << 16) | (ub << 8) | ua;
}
// OCP E4M3 (round to nearest even) of fl32(x * inv) saturated to +-448, four codes per word
__device__ inline uint32_t e4m3_pack4(float a, float b, float c, float d, float inv) {
  const float ya = fminf(fmaxf(a * inv, -448.f), 448.f);
  const float yb = fminf(fmaxf(b * inv, -448.f), 448.f);
  const float yc = fminf(fmaxf(c * inv, -448.f), 448.f);
  const float yd = fminf(fmaxf(d * inv, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(yc, yd, w, true);
  return static_cast<uint32_t>(w);
}

// Eight consecutive input elements as raw 16-byte words (1 for bf16, 2 for fp32), so a load
// can be issued early and converted later.
template <typename T>
struct Raw8 {
  i32x4 v[sizeof(T) / 2];
};
template <typename T>
__device__ inline Raw8<T> load_raw8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int u = 0; u < static_cast<int>(sizeof(T) / 2); ++u)
    r.v[u] = *reinterpret_cast<const i32x4*>(p + u * (16 / sizeof(T)));
  return r;
}
// element e (a compile-time constant after unrolling) as fp32
// (bit casts go through a scalar copy: __builtin_bit_cast of a vector-element lvalue reads
// element 0 with this compiler)
__device__ inline float raw8_at(const Raw8<float>& r, int e) {
  const int i = r.v[e >> 2][e & 3];
  return __int_as_float(i);
}
__device__ inline float raw8_at(const Raw8<uint16_t>& r, int e) {
  const uint32_t w = static_cast<uint32_t>(r.v[0][e >> 1]);
  return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}
// bf16 of element e of rows a (low half) and b (high half); bf16 input is moved bit-exactly
__device__ inline uint32_t raw8_bf16_pair(const Raw8<float>& a, const Raw8<float>& b, int e) {
  return pack_bf16x2(raw8_at(a, e), raw8_at(b, e));
}
__device__ inline uint32_t raw8_bf16_pair(const Raw8<uint16_t>& a, const Raw8<uint16_t>& b, int e) {
  return __builtin_amdgcn_perm(static_cast<uint32_t>(b.v[0][e >> 1]),
                               static_cast<uint32_t>(a.v[0][e >> 1]),
                               (e & 1) ? 0x07060302u : 0x05040100u);
}
__device__ inline void raw8_to_f32(const Raw8<float>& r, float* out) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i0 = r.v[0][k], i1 = r.v[1][k];
    out[k] = __int_as_float(i0);
    out[4 + k] = __int_as_float(i1);
  }
}
__device__ inline void raw8_to_f32(const Raw8<uint16_t>& r, float* out) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = static_cast<uint32_t>(r.v[0][k]);
    out[2 * k] = __uint_as_float(w << 16);
    out[2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------- launchers
// Each returns hipGetLastError() after enqueueing on `s`.
// Block sums of Q (128 rows, if Q is given) and K (64 rows) in fp64; with qc given also the
// INT8 codes of Q (row-major) and their per-block scales sq (q_tap: optional copy of codes).
hipError_t launch_pool(const Geom& g, int dtype, const void* Q, const void* K, double* qsum,
                       double* ksum, int8_t* qc, float* sq, int8_t* q_tap, hipStream_t s);
// one-time per-device set-up (dynamic LDS limit of the scoring kernel)
hipError_t configure_router();
// err (optional): the attention kernel's error word, cleared here (one launch before it)
hipError_t launch_colmean(const Geom& g, const double* ksum, double* mu64, float* mu32,
                          float* mu32_tap, uint32_t* err, hipStream_t s);
// B = (Kbar - mu) Wk, fp32 [BH][nkb][d], and (A non-null) A = Qbar Wq, fp32 [BH][nqb][d]
// (wk, wq null: the identity)
hipError_t launch_project(const Geom& g, const double* ksum, const double* mu64, const float* wk,
                          float* B, const double* qsum, const float* wq, float* A,
                          hipStream_t s);
// G = A B^T / sqrt(d), exact Top-k per row
hipError_t launch_score_topk(const Geom& g, const float* A, const float* B, int kb,
                             uint8_t* mask, int32_t* list, int list_stride, int32_t* cnt,
                             float* scores, hipStream_t s);
// p[0 .. n) = v (a kernel: no memset node in a captured graph)
hipError_t launch_fill(float* p, int n, float v, hipStream_t s);
// the earlier SLA mix: O += O_l Wo per (batch, head); wo [H, d, d] fp32
hipError_t launch_sla1_mix(const Geom& g, const float* Ol, const float* Wo, float* O,
                           hipStream_t s);
// SoftTop-k (training-time router): soft [BH, nqb, nkb] fp32, lam [BH, nqb] fp32 (or null)
hipError_t launch_score_soft(const Geom& g, const float* A, const float* B, int kb,
                             float inv_tau, float* soft, float* lam, hipStream_t s);
hipError_t launch_mask_to_list(const Geom& g, const uint8_t* mask_in, uint8_t* mask_out,
                               int32_t* list, int32_t* cnt, hipStream_t s);
// Fragment order of the d x d linear-branch matrices read by the attention kernel. Its
// wavefront w reads rows d_v = 32 w .. +31 of h_j^T and H_tot^T, lane (g = lane / 32,
// l = lane % 32) taking d_v = 32 w + l; storing the matrices in that read order makes each
// wavefront load one contiguous 1 KB run instead of 32-byte pieces of 32 rows.
//   h_j^T, bf16:   16-byte chunk (w * 8 + f) * 64 + lane holds d_phi = 16 f + 8 g .. +7
//   H_tot^T, fp32: 16-byte chunk (w * 16 + c) * 64 + lane holds d_phi = 8 c + 4 g .. +3
__host__ __device__ inline int htot_frag_index(int dv, int dphi) {
  return (((dv >> 5) * 16 + (dphi >> 3)) * 64 + 32 * ((dphi >> 2) & 1) + (dv & 31)) * 4 + (dphi & 3);
}
// Per key block: INT8 K_s tiles + sk and E4M3 V^T tiles + sv (skipped when kc is null;
// k_tap / v_tap optional row-major copies of the codes), z_j, h_j^T in bf16 (fragment order,
// optional), h_j in fp32 (standard orientation [d_phi][d_v], optional), and fp32 partial
// sums of h_j^T ([d_v][d_phi]) and z_j over kKpPerWg blocks.
struct KvArgs {
  const float* mu32;
  int8_t* kc;
  uint8_t* vc;
  float *sk, *sv;
  int8_t* k_tap;
  uint8_t* v_tap;
  uint16_t* ht_bf16;
  float* h_f32;
  float* z;
  float *hpart, *zpart;
};
hipError_t launch_kv_prep(const Geom& g, int dtype, const void* K, const void* V,
                          const KvArgs& x, hipStream_t s);
// standard = 0: H_tot^T in fragment order (for the attention kernel); 1: H_tot.
hipError_t launch_linear_total(const Geom& g, const float* hpart, const float* zpart,
                               float* htot, float* ztot, int standard, hipStream_t s);
// Operands of the fused attention kernel (sparse branch, linear branch, combine).
struct AttnArgs {
  const int8_t* qc;            // INT8 Q, row-major
  const int8_t* kc;            // INT8 K_s tiles
  const uint8_t* vc;           // E4M3 V^T tiles
  const float *sq, *sk, *sv;   // scales
  const uint16_t* ht_bf16;     // h_j^T, bf16, fragment order
  const float* z;              // z_j
  const float* htot_t;         // H_tot^T, fp32, fragment order
  const float* ztot;           // Z_tot
  const uint8_t* mask;         // 0/1 block mask
  const int32_t* list;         // kept lists
  int list_stride;
  const int32_t* cnt;          // kept count per query block
  const float* alpha;
  float* O;
  float* O_s_tap;              // optional
  float* O_l_tap;              // optional
  uint32_t* err;               // error word: set if a bounded wait gives up
  bool sparse;                 // false: the linear branch only, O = (1 - alpha) O_l
};
hipError_t launch_attn(const Geom& g, int dtype, const void* Q, const AttnArgs& x,
                       hipStream_t s);
// The unquantised sparse branch (fp32 operands): O += alpha O_s (after the attention kernel
// ran its linear branch alone); O_s_tap (optional) receives O_s.
struct ExactArgs {
  const void *K, *V;
  const float* mu32;
  const int32_t* list;
  int list_stride;
  const int32_t* cnt;
  const float* alpha;
  float* O;
  float* O_s_tap;
};
hipError_t launch_attn_exact(const Geom& g, int dtype, const void* Q, const ExactArgs& x,
                             hipStream_t s);

// Operands of the backward kernels. Layouts: Q, K, V [BH][N][d] (fp32 or bf16); dO, dQ, dK,
// dV [BH][N][d] fp32; h_j^T bf16 in fragment order; H_tot standard [a][o] fp32; dH_i^T bf16
// [BH][nqb][o][a]; dH_tot^T fp32 [BH][o][a]; lse2 = row log-sum-exp of the kept logits in
// base-2 units (S log2(e) / sqrt(d)); D = rowsum(dO_s O_s); key lists [BH][nkb][nqb] uint16.
struct BwdArgs {
  const void *Q, *K, *V;
  // bf16 operand copies: Q and V are the inputs themselves when they are bf16, else written by
  // bwd_prep (qbf_w, vbf_w non-null); K_s = K - colmean(K) and dO_s = alpha dO always written
  const uint16_t *qbf, *vbf;
  uint16_t *qbf_w, *vbf_w, *ksb, *dos;
  const int32_t* plan;       // [BH][2]: chunk size C, number of extra items
  const int32_t* xoff;       // [BH][nkb] first extra item of each key block
  const int32_t* items;      // [BH][cap] (j << 16 | chunk)
  float* xpart;              // [BH][cap][kSlot]: dK, dV [64][128], dH^T sum [128][128], dz sum
  int cap;
  const float* mu32;
  const float* dO;
  const float* alpha;
  const int32_t* list;       // kept lists, stride nkb
  const int32_t* cnt;
  const uint16_t* hbf;
  const float* htot;
  const float* z;
  const float* ztot;
  float* dQ;
  uint16_t* dht;
  float* dz;
  float* dalpha;             // [BH][nqb]
  float* dhtot;
  float* dztot;
  float* lse2;
  float* Dd;
  const int32_t* tcnt;
  const uint16_t* tlist;
  float *dK, *dV;
  float* kcol;               // [BH][nkb][d] column sums of dK_s per key block
  float* kmean;              // [BH][d]
  int H, BH, nqb, nkb;
};
hipError_t launch_key_lists(const Geom& g, const uint8_t* mask, int32_t* tcnt, uint16_t* tlist,
                            hipStream_t s);
hipError_t launch_key_plan(const Geom& g, const int32_t* tcnt, int32_t* plan, int32_t* xoff,
                           int32_t* items, int cap, hipStream_t s);
// the work items past the first of each long key list (partials into xpart)
hipError_t launch_bwd_kv_extra(const Geom& g, const BwdArgs& x, hipStream_t s);
hipError_t launch_bwd_prep(const Geom& g, int dtype, const BwdArgs& x, hipStream_t s);
hipError_t launch_bwd_lin_q(const Geom& g, int dtype, const BwdArgs& x, hipStream_t s);
hipError_t launch_dh_total(const Geom& g, const BwdArgs& x, hipStream_t s);
hipError_t launch_bwd_q(const Geom& g, const BwdArgs& x, hipStream_t s);
hipError_t launch_bwd_kv(const Geom& g, const BwdArgs& x, hipStream_t s);
// column mean of dK_s, then dK -= mean (two kernels)
hipError_t launch_dk_center(const Geom& g, const BwdArgs& x, hipStream_t s);

}  // namespace sla2
