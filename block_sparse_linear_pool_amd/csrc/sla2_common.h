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

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
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

// ---------------------------------------------------------------- launchers
// Each returns hipGetLastError() after enqueueing on `s`.
hipError_t launch_pool(const Geom& g, int dtype, const void* Q, const void* K, double* qsum,
                       double* ksum, hipStream_t s);
// one-time per-device set-up (dynamic LDS limit of the scoring kernel)
hipError_t configure_router();
hipError_t launch_colmean(const Geom& g, const double* ksum, double* mu64, float* mu32,
                          float* mu32_tap, hipStream_t s);
hipError_t launch_project(const Geom& g, const double* qsum, const double* ksum,
                          const double* mu64, const float* wq, const float* wk, double* A,
                          double* Bt, hipStream_t s);
hipError_t launch_score_topk(const Geom& g, const double* A, const double* Bt, int kb,
                             uint8_t* mask, int32_t* list, int list_stride, int32_t* cnt,
                             float* scores, hipStream_t s);
hipError_t launch_mask_to_list(const Geom& g, const uint8_t* mask_in, uint8_t* mask_out,
                               int32_t* list, int32_t* cnt, hipStream_t s);
hipError_t launch_quant(const Geom& g, int dtype, const void* Q, const void* K, const void* V,
                        const float* mu32, int8_t* qc, int8_t* kc, uint8_t* vc, float* sq,
                        float* sk, float* sv, int8_t* q_tap, int8_t* k_tap, uint8_t* v_tap,
                        hipStream_t s);
// h_j is kept transposed ([d_v][d_phi]) in bf16 for linear_out; h_f32 (optional) is the
// standard orientation [d_phi][d_v].
hipError_t launch_linear_pre(const Geom& g, int dtype, const void* K, const void* V,
                             const float* mu32, uint16_t* ht_bf16, float* h_f32, float* z,
                             float* hpart, float* zpart, hipStream_t s);
// standard = 0: H_tot^T (for linear_out); 1: H_tot.
hipError_t launch_linear_total(const Geom& g, const float* hpart, const float* zpart,
                               float* htot, float* ztot, int standard, hipStream_t s);
// Operands of the fused attention kernel (sparse branch, linear branch, combine).
struct AttnArgs {
  const int8_t* qc;            // INT8 Q, row-major
  const int8_t* kc;            // INT8 K_s tiles
  const uint8_t* vc;           // E4M3 V^T tiles
  const float *sq, *sk, *sv;   // scales
  const uint16_t* ht_bf16;     // h_j^T, bf16
  const float* z;              // z_j
  const float* htot_t;         // H_tot^T, fp32
  const float* ztot;           // Z_tot
  const uint8_t* mask;         // 0/1 block mask
  const int32_t* list;         // kept lists
  int list_stride;
  const int32_t* cnt;          // kept count per query block
  const float* alpha;
  float* O;
  float* O_s_tap;              // optional
  float* O_l_tap;              // optional
};
hipError_t launch_attn(const Geom& g, int dtype, const void* Q, const AttnArgs& x,
                       hipStream_t s);

}  // namespace sla2
