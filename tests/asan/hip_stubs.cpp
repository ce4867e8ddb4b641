// Host-only stand-ins for the HIP runtime calls and kernel launchers that
// csrc/api.cpp uses, so that the C ABI's argument checking, layout arithmetic
// and descriptor handling can be built with AddressSanitizer and
// UndefinedBehaviorSanitizer and exercised on a machine without a GPU.
//
// QGEMM_STUB_DEVICE selects the device the stubs report: unset or "none" (no
// device), "gfx950", or any other architecture name. Launchers do no work;
// they count their calls in qg_stub_launches and check that the arguments
// they receive describe buffers of sane sizes.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.hpp"

extern "C" {
int qg_stub_launches = 0;
int qg_stub_memsets = 0;
}

namespace {
const char* stub_arch() {
  const char* a = std::getenv("QGEMM_STUB_DEVICE");
  return (a && *a && std::strcmp(a, "none") != 0) ? a : nullptr;
}
void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub launcher: %s\n", what);
    std::abort();
  }
}
void check_gemm(const qg::GemmArgs& a) {
  require(a.M >= 1 && a.N >= 1 && a.K >= 1 && a.K <= a.K_pad && a.K_pad % 256 == 0, "GEMM sizes");
  require(a.a != nullptr && a.w != nullptr && a.out != nullptr, "GEMM pointers");
  require(a.ldo >= a.N, "GEMM ldo");
}
float g_scratch[qg::kScratchFloats];
}  // namespace

extern "C" hipError_t hipGetDevice(int* d) {
  if (!stub_arch()) return hipErrorNoDevice;
  *d = 0;
  return hipSuccess;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t* p, int dev) {
  if (!stub_arch() || dev != 0) return hipErrorInvalidDevice;
  std::memset(p, 0, sizeof(*p));
  std::snprintf(p->gcnArchName, sizeof(p->gcnArchName), "%s:sramecc+:xnack-", stub_arch());
  p->multiProcessorCount = 256;
  return hipSuccess;
}

extern "C" hipError_t hipGetLastError() { return hipSuccess; }

extern "C" hipError_t hipMemsetAsync(void* p, int, size_t n, hipStream_t) {
  require(p != nullptr && n > 0, "memset range");
  ++qg_stub_memsets;
  return hipSuccess;
}

namespace qg {
void launch_quantize_int(const float* x, int64_t rows, int64_t K, int64_t ldx, bool, bool, uint8_t* q, int64_t ldq,
                         int64_t, float* scales, int32_t*, int32_t*, float*, hipStream_t) {
  require(x && q && scales && rows >= 0 && K >= 1 && ldx >= K && ldq >= 1, "quantize_int args");
  ++qg_stub_launches;
}
void launch_rmsnorm_quantize(const float* x, int64_t rows, int64_t K, int64_t ldx, const float* gamma, float, bool,
                             uint8_t* q, int64_t ldq, float* scales, int32_t*, hipStream_t) {
  require(x && gamma && q && scales && rows >= 0 && K >= 1 && ldx >= K && ldq >= K, "rmsnorm args");
  ++qg_stub_launches;
}
void launch_quantize_mx(const float* x, int64_t rows, int64_t K, int64_t ldx, bool, uint8_t* q, int64_t ldq,
                        uint8_t* e8, int64_t lde, int64_t wblk_kpad, hipStream_t) {
  require(x && q && e8 && rows >= 0 && K % 32 == 0 && ldx >= K && lde >= K / 32, "quantize_mx args");
  require(wblk_kpad == 0 || (wblk_kpad >= K && wblk_kpad % 256 == 0), "quantize_mx blocked weights");
  (void)ldq;
  ++qg_stub_launches;
}
void launch_quantize_int4(const float* w, int64_t rows, int64_t K, int64_t ldw, int64_t K_pad, uint8_t* codes,
                          float* scales, hipStream_t) {
  require(w && codes && scales && rows >= 1 && K >= 1 && ldw >= K && K_pad >= K && K_pad % 256 == 0, "int4 args");
  ++qg_stub_launches;
}
int cu_count() { return 256; }
hipError_t scratch_buffer(float** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
bool mx_dma_eligible(const GemmArgs&, int) { return true; }
hipError_t launch_gemm_i8(const GemmArgs& a, bool, int, hipStream_t) {
  check_gemm(a);
  ++qg_stub_launches;
  return hipSuccess;
}
hipError_t launch_gemm_mx(const GemmArgs& a, int, hipStream_t) {
  check_gemm(a);
  ++qg_stub_launches;
  return hipSuccess;
}
hipError_t launch_gemm_mx_grouped(const GemmArgs& a, int, hipStream_t) {
  require(a.groups != nullptr && a.num_groups >= 1, "grouped args");
  ++qg_stub_launches;
  return hipSuccess;
}
hipError_t launch_unpack(const UnpackArgs& a, hipStream_t) {
  require(a.src != nullptr && a.out != nullptr && a.rows >= 1 && a.cols >= 1 && a.ld >= 1 && a.K_pad % 256 == 0,
          "unpack args");
  ++qg_stub_launches;
  return hipSuccess;
}
hipError_t launch_ceiling_mfma(int kind, int waves_per_simd, int64_t trips, const uint8_t* a_ops,
                               const uint8_t* b_ops, int32_t* sink, int64_t*, hipStream_t) {
  require(kind >= 0 && kind <= 3 && (waves_per_simd == 1 || waves_per_simd == 2) && trips >= 1 && a_ops && b_ops &&
              sink,
          "ceiling mfma args");
  ++qg_stub_launches;
  return hipSuccess;
}
hipError_t launch_ceiling_stream(const uint8_t* src, int64_t bytes, int64_t block_bytes, int32_t* sink, hipStream_t) {
  require(src && sink && bytes >= 16 && bytes % 16 == 0 && block_bytes % 16384 == 0, "ceiling stream args");
  ++qg_stub_launches;
  return hipSuccess;
}
hipError_t launch_gemm_w4a8(const GemmArgs& a, int, hipStream_t) {
  check_gemm(a);
  ++qg_stub_launches;
  return hipSuccess;
}
}  // namespace qg
