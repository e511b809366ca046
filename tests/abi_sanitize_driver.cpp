// Host-side validation of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
// (built by tests/test_abi_sanitize.py with the sanitizers on host code only). Every call
// below returns before any device work: bad arguments are rejected by the host checks, and
// valid ones stop at the device check (no GPU here) or are host-only functions. The program
// exits non-zero on the first unexpected status; a sanitizer finding aborts it.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/sla2.h"

extern "C" const char* __asan_default_options() { return "detect_leaks=0"; }

namespace {

int failures = 0;

void expect(const char* what, long got, long want) {
  if (got != want) {
    std::fprintf(stderr, "%s: got %ld, want %ld\n", what, got, want);
    ++failures;
  }
}

// fake, 16-byte aligned device addresses: never dereferenced
void* const A = reinterpret_cast<void*>(0x10000);
void* const MIS = reinterpret_cast<void*>(0x10008);
float* const Af = static_cast<float*>(A);
float* const MISf = static_cast<float*>(MIS);

sla2_shape shape(int B, int H, int N, int d = 128, int dtype = SLA2_BF16) {
  sla2_shape s;
  s.B = B;
  s.H = H;
  s.N = N;
  s.d = d;
  s.dtype = static_cast<sla2_dtype>(dtype);
  return s;
}

bool device_or_hip(sla2_status s) {
  return s == SLA2_ERR_UNSUPPORTED_DEVICE || s == SLA2_ERR_HIP;
}

}  // namespace

int main() {
  // host-only functions over their whole argument ranges
  for (int n = -2; n <= 4100; n += 37)
    for (float k : {-1.f, 0.f, 1e-7f, 0.03f, 0.5f, 1.f, 1.5f, NAN, INFINITY}) {
      const int32_t kb = sla2_blocks_kept(n, k);
      if (n < 1 || !(k > 0.f && k <= 1.f)) expect("blocks_kept invalid", kb, -1);
      else if (kb < 1 || kb > n) expect("blocks_kept range", kb, 1);
    }
  for (int s = -3; s < 16; ++s)
    if (sla2_status_string(static_cast<sla2_status>(s)) == nullptr) expect("status string", 0, 1);
  const int Ns[] = {0, 64, 128, 640, 1000, 32768, 262144, 262272};
  for (int e = -1; e <= 8; ++e)
    for (int N : Ns)
      for (int H : {0, 1, 12, 40, 70000}) {
        sla2_shape s = shape(1, H, N);
        const size_t b = sla2_workspace_bytes(&s, static_cast<sla2_entry>(e), 0.03f);
        const bool valid = e >= 0 && e <= 7 && H >= 1 && H <= 65535 && N >= 128 &&
                           N % 128 == 0 && N <= 262144;
        if (valid != (b > 0)) expect("workspace_bytes validity", static_cast<long>(b), valid);
      }
  expect("workspace_bytes null", static_cast<long>(sla2_workspace_bytes(nullptr, SLA2_ENTRY_FORWARD, 0.5f)), 0);
  expect("workspace_status null", sla2_workspace_status(nullptr, 1024, nullptr), SLA2_ERR_NULL_POINTER);
  expect("workspace_status misaligned", sla2_workspace_status(MIS, 1024, nullptr), SLA2_ERR_MISALIGNED);
  expect("workspace_status small", sla2_workspace_status(A, 3, nullptr), SLA2_ERR_WORKSPACE_TOO_SMALL);

  sla2_shape s = shape(1, 2, 1024);
  const size_t fw = sla2_workspace_bytes(&s, SLA2_ENTRY_FORWARD, 0.25f);
  const size_t big = sla2_workspace_bytes(&s, SLA2_ENTRY_ROUTER_GRAD, 0.25f);
  sla2_taps taps;
  std::memset(&taps, 0, sizeof(taps));
  // forward
  expect("fwd null shape", sla2_forward(nullptr, A, A, A, Af, Af, Af, 0.25f, SLA2_QUANT_I8_FP8, Af, nullptr, A, fw, nullptr), SLA2_ERR_NULL_POINTER);
  sla2_shape bad = shape(1, 2, 1000);
  expect("fwd bad N", sla2_forward(&bad, A, A, A, Af, Af, Af, 0.25f, SLA2_QUANT_I8_FP8, Af, nullptr, A, fw, nullptr), SLA2_ERR_BAD_SHAPE);
  bad = shape(1, 2, 1024, 128, 9);
  expect("fwd bad dtype", sla2_forward(&bad, A, A, A, Af, Af, Af, 0.25f, SLA2_QUANT_I8_FP8, Af, nullptr, A, fw, nullptr), SLA2_ERR_BAD_DTYPE);
  expect("fwd null q", sla2_forward(&s, nullptr, A, A, Af, Af, Af, 0.25f, SLA2_QUANT_I8_FP8, Af, nullptr, A, fw, nullptr), SLA2_ERR_NULL_POINTER);
  expect("fwd misaligned v", sla2_forward(&s, A, A, MIS, Af, Af, Af, 0.25f, SLA2_QUANT_I8_FP8, Af, nullptr, A, fw, nullptr), SLA2_ERR_MISALIGNED);
  taps.O_s = MISf;
  expect("fwd misaligned tap", sla2_forward(&s, A, A, A, Af, Af, Af, 0.25f, SLA2_QUANT_I8_FP8, Af, &taps, A, fw, nullptr), SLA2_ERR_MISALIGNED);
  taps.O_s = nullptr;
  for (float k : {0.f, -1.f, 1.5f, NAN})
    expect("fwd keep", sla2_forward(&s, A, A, A, Af, Af, Af, k, SLA2_QUANT_I8_FP8, Af, nullptr, A, fw, nullptr), SLA2_ERR_BAD_ARGUMENT);
  expect("fwd quant", sla2_forward(&s, A, A, A, Af, Af, Af, 0.25f, static_cast<sla2_quant>(5), Af, nullptr, A, fw, nullptr), SLA2_ERR_BAD_ARGUMENT);
  expect("fwd small ws", sla2_forward(&s, A, A, A, Af, Af, Af, 0.25f, SLA2_QUANT_I8_FP8, Af, nullptr, A, fw - 1, nullptr), SLA2_ERR_WORKSPACE_TOO_SMALL);
  if (!device_or_hip(sla2_forward(&s, A, A, A, Af, Af, Af, 0.25f, SLA2_QUANT_NONE, Af, &taps, A, fw, nullptr)))
    expect("fwd valid reaches the device check", 0, 1);
  // other entry points
  expect("router blocks", sla2_router(&s, A, A, Af, Af, 0.25f, nullptr, nullptr, nullptr, A, big, nullptr), SLA2_ERR_NULL_POINTER);
  expect("router keep", sla2_router(&s, A, A, Af, Af, 2.f, nullptr, static_cast<int32_t*>(A), nullptr, A, big, nullptr), SLA2_ERR_BAD_ARGUMENT);
  expect("noalloc keep", sla2_router_noalloc(&s, A, A, Af, Af, 0.f, nullptr, static_cast<int32_t*>(A), nullptr, nullptr), SLA2_ERR_BAD_ARGUMENT);
  sla2_shape huge = shape(1, 40, 75648);
  expect("noalloc too big", sla2_router_noalloc(&huge, A, A, Af, Af, 0.05f, nullptr, static_cast<int32_t*>(A), nullptr, nullptr), SLA2_ERR_WORKSPACE_TOO_SMALL);
  expect("soft tau", sla2_router_soft(&s, A, A, Af, Af, 0.25f, 0.f, Af, nullptr, nullptr, A, big, nullptr), SLA2_ERR_BAD_ARGUMENT);
  expect("soft tau tiny", sla2_router_soft(&s, A, A, Af, Af, 0.25f, 1e-45f, Af, nullptr, nullptr, A, big, nullptr), SLA2_ERR_BAD_ARGUMENT);
  expect("precompute colmean", sla2_linear_precompute(&s, A, A, nullptr, nullptr, nullptr, Af, Af, A, big, nullptr), SLA2_ERR_NULL_POINTER);
  expect("with_mask mask", sla2_forward_with_mask(&s, A, A, A, nullptr, Af, SLA2_QUANT_I8_FP8, Af, nullptr, A, big, nullptr), SLA2_ERR_NULL_POINTER);
  expect("sla1 quant", sla2_forward_sla1(&s, A, A, A, Af, 0.25f, static_cast<sla2_quant>(2), Af, Af, nullptr, A, big, nullptr), SLA2_ERR_BAD_ARGUMENT);
  expect("backward dO", sla2_backward(&s, A, A, A, static_cast<uint8_t*>(A), Af, nullptr, Af, Af, Af, Af, nullptr, A, big, nullptr), SLA2_ERR_NULL_POINTER);
  expect("fit shape", sla2_fit_alpha(&bad, Af, Af, Af, Af, nullptr), SLA2_ERR_BAD_DTYPE);
  double* const Ad = static_cast<double*>(A);
  expect("grad target", sla2_router_grad(&s, A, A, A, Af, Af, Af, 0.25f, 0.1f, nullptr, Af, Af, Ad, nullptr, A, big, nullptr), SLA2_ERR_NULL_POINTER);
  expect("grad tau", sla2_router_grad(&s, A, A, A, Af, Af, Af, 0.25f, -1.f, Af, Af, Af, Ad, nullptr, A, big, nullptr), SLA2_ERR_BAD_ARGUMENT);
  expect("grad ws", sla2_router_grad(&s, A, A, A, Af, Af, Af, 0.25f, 0.1f, Af, Af, Af, Ad, nullptr, A, big - 1, nullptr), SLA2_ERR_WORKSPACE_TOO_SMALL);
  if (!device_or_hip(sla2_router_grad(&s, A, A, A, Af, Af, Af, 0.25f, 0.1f, Af, Af, Af, Ad, Af, A, big, nullptr)))
    expect("grad valid reaches the device check", 0, 1);
  if (!device_or_hip(sla2_init_device())) expect("init_device without a GPU", 0, 1);
  std::printf("%s: %d unexpected results\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
