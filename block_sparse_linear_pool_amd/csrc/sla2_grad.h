// Internal: the stage-1 router-gradient kernels (grad.hip).
#pragma once

#include "sla2_common.h"

namespace sla2 {

struct GradArgs {
  const float* mu32;                     // colmean(K) in fp32 [BH][d]
  uint32_t *ks16, *v16, *pk16;           // f16 K_s, V, phi(K_s) [BH][N][d] (pairs per word)
  const float *O, *O_full, *O_s, *O_l;   // [BH][N][d]
  const float *z, *ztot;                 // z_j [BH][nkb][d], Z_tot [BH][d]
  const uint8_t* mask;                   // hard mask [BH][nqb][nkb]
  const int32_t* list;                   // kept lists
  int list_stride;
  const int32_t* cnt;
  const float* alpha;                    // [H][nqb]
  float* g;                              // dL/dM [BH][nqb][nkb]
  float* lossp;                          // per query block sum of squares [BH][nqb]
  float *Arow, *dA, *dG, *dB;            // router part: A, dA [BH][nqb][d]; dG [BH][nqb][nkb];
                                         // dB [BH][nkb][d]
};

hipError_t launch_grad_prep(const Geom& g, int dtype, const void* K, const void* V,
                            const GradArgs& x, hipStream_t s);
hipError_t launch_mask_grad(const Geom& g, int dtype, const void* Q, const GradArgs& x,
                            hipStream_t s);
// router_vjp_row, router_db, router_dw: dWq, dWk [H][d][d], loss [H]
hipError_t launch_router_vjp(const Geom& g, const double* qsum, const double* ksum,
                             const double* mu64, const float* wq, const float* B,
                             const float* soft, const GradArgs& x, float inv_tau, float* dWq,
                             float* dWk, double* loss, hipStream_t s);

}  // namespace sla2
