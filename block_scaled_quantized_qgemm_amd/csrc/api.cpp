// C ABI of the quantized linear-layer library: argument validation, the
// packed weight layout, device check and kernel dispatch. Every check runs
// before anything is launched, so an error leaves all outputs untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "../../include/qgemm.h"
#include "../../include/qgemm_ceiling.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kNPad = 256;   // packed rows are padded to this multiple
constexpr int64_t kKPad = 256;   // packed columns are padded to this multiple (an even number of 128-deep steps)
constexpr int64_t kSymKMax = 133144;   // 127*127*K < 2^31
constexpr int64_t kAsymKMax = 66311;   // 255*127*K < 2^31
constexpr int64_t kMaxRows = 0x7fffffff;
constexpr int64_t kMaxExperts = 4096;  // grouped MX GEMM: experts per call
constexpr int64_t kW4MaxRows = 16 * 65535;  // 16-row bands along the grid's second dimension
constexpr int64_t kW4MaxK = int64_t(1) << 27;  // a 16-row block's codes (8 K_pad bytes) in one 32-bit range

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

std::atomic<int> g_arch_ok[64];  // per device: 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QGEMM_E_DEVICE;
  int c = dev < 64 ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
  if (c == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QGEMM_E_DEVICE;
    c = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (dev < 64) g_arch_ok[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1 ? QGEMM_OK : QGEMM_E_DEVICE;
}

bool is_int_fmt(int f) { return f == QGEMM_FMT_INT8_SYM || f == QGEMM_FMT_UINT8_ASYM; }
bool is_mx_fmt(int f) { return f == QGEMM_FMT_MXFP8_E4M3 || f == QGEMM_FMT_MXFP4_E2M1; }
// bytes a row of K codes occupies
int64_t code_bytes(int fmt, int64_t K) { return fmt == QGEMM_FMT_MXFP4_E2M1 ? K / 2 : K; }
bool is_int_gran(int g) { return g == QGEMM_GRAN_TENSOR || g == QGEMM_GRAN_ROW; }

struct Layout {
  int64_t N_pad, K_pad, codes_off, scales_off, colsum_off, bytes;
};

bool weight_layout(int64_t N, int64_t K, int fmt, int gran, Layout* L) {
  if (N < 1 || K < 1 || N > kMaxRows || K > (int64_t)1 << 30) return false;
  if (fmt == QGEMM_FMT_INT8_SYM) {
    if (!is_int_gran(gran)) return false;
  } else if (is_mx_fmt(fmt)) {
    if (gran != QGEMM_GRAN_BLOCK32 || K % 32 != 0) return false;
  } else if (fmt == QGEMM_FMT_INT4_SYM) {
    if (gran != QGEMM_GRAN_GROUP64) return false;
  } else {
    return false;
  }
  L->N_pad = round_up(N, kNPad);
  L->K_pad = round_up(K, kKPad);
  L->codes_off = 0;
  if (fmt == QGEMM_FMT_INT4_SYM) {  // two codes per byte, one float32 scale per 64 K
    L->scales_off = round_up(L->N_pad * L->K_pad / 2, 256);
    L->colsum_off = -1;
    L->bytes = round_up(L->scales_off + 4 * L->N_pad * (L->K_pad / 64), 256);
    return true;
  }
  L->scales_off = round_up(L->N_pad * code_bytes(fmt, L->K_pad), 256);
  if (fmt == QGEMM_FMT_INT8_SYM) {
    L->colsum_off = round_up(L->scales_off + 4 * L->N_pad, 256);
    L->bytes = round_up(L->colsum_off + 4 * L->N_pad, 256);
  } else {
    L->colsum_off = -1;
    L->bytes = round_up(L->scales_off + L->N_pad * (L->K_pad / 32), 256);
  }
  return true;
}

// want_fmt < 0: any MX weight format
int check_desc(const qgemm_wdesc* d, int want_fmt) {
  if (!d) return QGEMM_E_NULL;
  if (d->magic != QGEMM_WDESC_MAGIC || d->version != QGEMM_ABI_VERSION) return QGEMM_E_DESC;
  if (want_fmt >= 0 ? d->fmt != want_fmt : !is_mx_fmt(d->fmt)) return QGEMM_E_DESC;
  Layout L;
  if (!weight_layout(d->N, d->K, d->fmt, d->gran, &L)) return QGEMM_E_DESC;
  if (L.N_pad != d->N_pad || L.K_pad != d->K_pad || L.codes_off != d->codes_off || L.scales_off != d->scales_off ||
      L.colsum_off != d->colsum_off || L.bytes != d->bytes)
    return QGEMM_E_DESC;
  return QGEMM_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launch_status() { return hipGetLastError() == hipSuccess ? QGEMM_OK : QGEMM_E_HIP; }

}  // namespace

extern "C" {

int qgemm_abi_version(void) { return QGEMM_ABI_VERSION; }

const char* qgemm_status_string(int s) {
  switch (s) {
    case QGEMM_OK: return "QGEMM_OK";
    case QGEMM_E_NULL: return "QGEMM_E_NULL: a required pointer is NULL";
    case QGEMM_E_SHAPE: return "QGEMM_E_SHAPE: a size or leading dimension is out of range";
    case QGEMM_E_MODE: return "QGEMM_E_MODE: unsupported format / granularity / output combination";
    case QGEMM_E_ALIGN: return "QGEMM_E_ALIGN: pointer or leading dimension not aligned as required";
    case QGEMM_E_OVERFLOW: return "QGEMM_E_OVERFLOW: K too large for an exact int32 accumulator";
    case QGEMM_E_DEVICE: return "QGEMM_E_DEVICE: the current device is not a gfx950";
    case QGEMM_E_DESC: return "QGEMM_E_DESC: invalid weight descriptor";
    case QGEMM_E_WORKSPACE: return "QGEMM_E_WORKSPACE: workspace missing or too small";
    case QGEMM_E_HIP: return "QGEMM_E_HIP: a HIP call or kernel launch failed";
    default: return "unknown qgemm status";
  }
}

size_t qgemm_packed_weight_bytes(int64_t N, int64_t K, int fmt, int gran) {
  Layout L;
  return weight_layout(N, K, fmt, gran, &L) ? (size_t)L.bytes : 0;
}

size_t qgemm_workspace_bytes(int64_t rows, int64_t K, int fmt, int gran) {
  (void)K;
  if (rows < 0) return 0;
  if (gran == QGEMM_GRAN_TENSOR && fmt == QGEMM_FMT_INT8_SYM) return (size_t)rows * 4;
  if (gran == QGEMM_GRAN_TENSOR && fmt == QGEMM_FMT_UINT8_ASYM) return (size_t)rows * 8;
  return 0;
}

}  // extern "C"

namespace {

// Validation shared by the two quantize entry points (everything but the
// workspace); QGEMM_OK with *empty set when M == 0.
int check_quantize_args(const float* x, int64_t M, int64_t K, int64_t ldx, int fmt, int gran, void* q, int64_t ldq,
                        float* scales, int32_t* zero_points, uint8_t* mx_scales, int64_t ld_mx, bool* empty) {
  *empty = false;
  const bool mx = is_mx_fmt(fmt);
  if (mx) {
    if (gran != QGEMM_GRAN_BLOCK32) return QGEMM_E_MODE;
  } else if (!is_int_fmt(fmt) || !is_int_gran(gran)) {
    return QGEMM_E_MODE;
  }
  if (M < 0 || M > kMaxRows || K < 1 || K > ((int64_t)1 << 30)) return QGEMM_E_SHAPE;
  if (mx && K % 32 != 0) return QGEMM_E_SHAPE;
  if (M == 0) {
    *empty = true;
    return QGEMM_OK;
  }
  if (!x || !q) return QGEMM_E_NULL;
  if (ldx < K || ldq < code_bytes(fmt, K)) return QGEMM_E_SHAPE;
  if (!aligned(x, 4) || ldq % 16 != 0 || !aligned(q, 16)) return QGEMM_E_ALIGN;
  if (mx) {
    if (!mx_scales) return QGEMM_E_NULL;
    if (ld_mx < K / 32) return QGEMM_E_SHAPE;
  } else {
    if (!scales) return QGEMM_E_NULL;
    if (fmt == QGEMM_FMT_UINT8_ASYM && !zero_points) return QGEMM_E_NULL;
    if (!aligned(scales, 4) || (zero_points && !aligned(zero_points, 4))) return QGEMM_E_ALIGN;
  }
  return QGEMM_OK;
}

void launch_quantize(const float* x, int64_t M, int64_t K, int64_t ldx, int fmt, int gran, void* q, int64_t ldq,
                     float* scales, int32_t* zero_points, uint8_t* mx_scales, int64_t ld_mx, float* ws,
                     hipStream_t st) {
  if (is_mx_fmt(fmt)) {
    qg::launch_quantize_mx(x, M, K, ldx, fmt == QGEMM_FMT_MXFP4_E2M1, (uint8_t*)q, ldq, mx_scales, ld_mx, 0, st);
  } else {
    qg::launch_quantize_int(x, M, K, ldx, fmt == QGEMM_FMT_UINT8_ASYM, gran == QGEMM_GRAN_TENSOR, (uint8_t*)q, ldq,
                            0, scales, zero_points, nullptr, ws, st);
  }
}

}  // namespace

extern "C" {

int qgemm_quantize_rows(const float* x, int64_t M, int64_t K, int64_t ldx, int fmt, int gran, void* q,
                        int64_t ldq, float* scales, int32_t* zero_points, uint8_t* mx_scales, int64_t ld_mx,
                        void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  int rc = check_quantize_args(x, M, K, ldx, fmt, gran, q, ldq, scales, zero_points, mx_scales, ld_mx, &empty);
  if (rc != QGEMM_OK || empty) return rc;
  const size_t need = qgemm_workspace_bytes(M, K, fmt, gran);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QGEMM_E_WORKSPACE;
  if (need > 0 && !aligned(workspace, 4)) return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;
  launch_quantize(x, M, K, ldx, fmt, gran, q, ldq, scales, zero_points, mx_scales, ld_mx, (float*)workspace,
                  as_stream(stream));
  return launch_status();
}

int qgemm_quantize_rows_noalloc(const float* x, int64_t M, int64_t K, int64_t ldx, int fmt, int gran, void* q,
                                int64_t ldq, float* scales, int32_t* zero_points, uint8_t* mx_scales, int64_t ld_mx,
                                void* stream) {
  bool empty = false;
  int rc = check_quantize_args(x, M, K, ldx, fmt, gran, q, ldq, scales, zero_points, mx_scales, ld_mx, &empty);
  if (rc != QGEMM_OK || empty) return rc;
  const size_t need = qgemm_workspace_bytes(M, K, fmt, gran);
  if (need > (size_t)qg::kScratchFloats * sizeof(float)) return QGEMM_E_WORKSPACE;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;
  float* ws = nullptr;
  if (need > 0 && qg::scratch_buffer(&ws) != hipSuccess) return QGEMM_E_HIP;
  launch_quantize(x, M, K, ldx, fmt, gran, q, ldq, scales, zero_points, mx_scales, ld_mx, ws, as_stream(stream));
  return launch_status();
}

int qgemm_rmsnorm_quantize_rows(const float* x, int64_t M, int64_t K, int64_t ldx, const float* gamma, float eps,
                                int fmt, int gran, void* q, int64_t ldq, float* scales, int32_t* zero_points,
                                void* stream) {
  if (!is_int_fmt(fmt) || gran != QGEMM_GRAN_ROW) return QGEMM_E_MODE;
  if (!(eps >= 0.0f) || !(eps <= 3.0e38f)) return QGEMM_E_MODE;  // also rejects NaN
  if (M < 0 || M > kMaxRows || K < 1 || K > ((int64_t)1 << 30)) return QGEMM_E_SHAPE;
  if (M == 0) return QGEMM_OK;
  if (!x || !gamma || !q || !scales || (fmt == QGEMM_FMT_UINT8_ASYM && !zero_points)) return QGEMM_E_NULL;
  if (ldx < K || ldq < K) return QGEMM_E_SHAPE;
  if (!aligned(x, 4) || !aligned(gamma, 4) || ldq % 16 != 0 || !aligned(q, 16) || !aligned(scales, 4) ||
      (zero_points && !aligned(zero_points, 4)))
    return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;
  qg::launch_rmsnorm_quantize(x, M, K, ldx, gamma, eps, fmt == QGEMM_FMT_UINT8_ASYM, (uint8_t*)q, ldq, scales,
                              zero_points, as_stream(stream));
  return launch_status();
}

int qgemm_prepack_weights(const float* w, int64_t N, int64_t K, int64_t ldw, int fmt, int gran, void* packed,
                          size_t packed_bytes, qgemm_wdesc* desc, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (fmt != QGEMM_FMT_INT8_SYM && !is_mx_fmt(fmt) && fmt != QGEMM_FMT_INT4_SYM) return QGEMM_E_MODE;
  if (fmt == QGEMM_FMT_INT8_SYM && !is_int_gran(gran)) return QGEMM_E_MODE;
  if (is_mx_fmt(fmt) && gran != QGEMM_GRAN_BLOCK32) return QGEMM_E_MODE;
  if (fmt == QGEMM_FMT_INT4_SYM && gran != QGEMM_GRAN_GROUP64) return QGEMM_E_MODE;
  Layout L;
  if (!weight_layout(N, K, fmt, gran, &L)) return QGEMM_E_SHAPE;
  if (!w || !packed || !desc) return QGEMM_E_NULL;
  if (ldw < K) return QGEMM_E_SHAPE;
  if (!aligned(w, 4) || !aligned(packed, 256)) return QGEMM_E_ALIGN;
  if (packed_bytes < (size_t)L.bytes) return QGEMM_E_SHAPE;
  const size_t need = qgemm_workspace_bytes(N, K, fmt, gran);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QGEMM_E_WORKSPACE;
  if (need > 0 && !aligned(workspace, 4)) return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;

  hipStream_t st = as_stream(stream);
  uint8_t* base = (uint8_t*)packed;
  if (hipMemsetAsync(base, 0, (size_t)L.bytes, st) != hipSuccess) return QGEMM_E_HIP;
  if (fmt == QGEMM_FMT_INT8_SYM) {
    qg::launch_quantize_int(w, N, K, ldw, false, gran == QGEMM_GRAN_TENSOR, base + L.codes_off, L.K_pad,
                            L.K_pad / 64, (float*)(base + L.scales_off), nullptr, (int32_t*)(base + L.colsum_off),
                            (float*)workspace, st);
  } else if (fmt == QGEMM_FMT_INT4_SYM) {
    qg::launch_quantize_int4(w, N, K, ldw, L.K_pad, base + L.codes_off, (float*)(base + L.scales_off), st);
  } else {
    if (hipMemsetAsync(base + L.scales_off, 127, (size_t)(L.N_pad * (L.K_pad / 32)), st) != hipSuccess)
      return QGEMM_E_HIP;
    // e4m3 codes in 1 KB blocks of 16 rows x 64 K, e2m1 codes row-major
    qg::launch_quantize_mx(w, N, K, ldw, fmt == QGEMM_FMT_MXFP4_E2M1, base + L.codes_off, code_bytes(fmt, L.K_pad),
                           base + L.scales_off, L.K_pad / 32, L.K_pad, st);
  }
  int rc = launch_status();
  if (rc != QGEMM_OK) return rc;
  desc->magic = QGEMM_WDESC_MAGIC;
  desc->version = QGEMM_ABI_VERSION;
  desc->fmt = fmt;
  desc->gran = gran;
  desc->N = N;
  desc->K = K;
  desc->N_pad = L.N_pad;
  desc->K_pad = L.K_pad;
  desc->codes_off = L.codes_off;
  desc->scales_off = L.scales_off;
  desc->colsum_off = L.colsum_off;
  desc->bytes = L.bytes;
  return QGEMM_OK;
}

int qgemm_unpack_weights(const qgemm_wdesc* desc, const void* packed, void* codes_out, int64_t ld_codes,
                         float* scales_out, int64_t ld_scales, int32_t* colsums_out, uint8_t* mx_scales_out,
                         int64_t ld_mx, void* stream) {
  if (!desc || !packed) return QGEMM_E_NULL;
  int rc = check_desc(desc, desc->fmt);
  if (rc != QGEMM_OK) return rc;
  const int fmt = desc->fmt;
  const bool i8 = fmt == QGEMM_FMT_INT8_SYM, i4 = fmt == QGEMM_FMT_INT4_SYM, mx = is_mx_fmt(fmt);
  const int64_t N = desc->N, K = desc->K;
  // what the format holds
  if ((scales_out && mx) || (colsums_out && !i8) || (mx_scales_out && !mx)) return QGEMM_E_MODE;
  const int64_t code_row = fmt == QGEMM_FMT_MXFP4_E2M1 ? K / 2 : K;  // bytes of a plain code row
  const int64_t groups = (K + 63) / 64;
  if (codes_out && ld_codes < code_row) return QGEMM_E_SHAPE;
  if (scales_out && i4 && ld_scales < groups) return QGEMM_E_SHAPE;
  if (mx_scales_out && ld_mx < K / 32) return QGEMM_E_SHAPE;
  if (!aligned(packed, 256) || (scales_out && !aligned(scales_out, 4)) || (colsums_out && !aligned(colsums_out, 4)))
    return QGEMM_E_ALIGN;
  if (!codes_out && !scales_out && !colsums_out && !mx_scales_out) return QGEMM_OK;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;

  hipStream_t st = as_stream(stream);
  const uint8_t* base = static_cast<const uint8_t*>(packed);
  const int ufmt = i8 ? qg::UNPACK_FMT_INT8
                       : i4 ? qg::UNPACK_FMT_INT4
                            : (fmt == QGEMM_FMT_MXFP8_E4M3 ? qg::UNPACK_FMT_MX8 : qg::UNPACK_FMT_MX);
  auto run = [&](int what, const uint8_t* src, int64_t src_pitch, void* out, int64_t ld, int64_t rows, int64_t cols,
                 int64_t row_bytes) {
    qg::UnpackArgs u{src, src_pitch, out, ld, rows, cols, row_bytes, desc->K_pad, what, ufmt};
    return qg::launch_unpack(u, st) == hipSuccess;
  };
  bool ok = true;
  if (codes_out)
    ok = ok && run(qg::UNPACK_CODES, base + desc->codes_off, code_bytes(fmt, desc->K_pad), codes_out, ld_codes, N,
                   (code_row + 15) / 16, code_row);
  if (scales_out && i8)
    ok = ok && run(qg::UNPACK_WORDS, base + desc->scales_off, 0, scales_out, 1,
                   desc->gran == QGEMM_GRAN_TENSOR ? 1 : N, 1, 0);
  if (scales_out && i4)
    ok = ok && run(qg::UNPACK_INT4_SCALES, base + desc->scales_off, 0, scales_out, ld_scales, N, groups, 0);
  if (colsums_out) ok = ok && run(qg::UNPACK_WORDS, base + desc->colsum_off, 0, colsums_out, 1, N, 1, 0);
  if (mx_scales_out)
    ok = ok && run(qg::UNPACK_E8M0, base + desc->scales_off, desc->K_pad / 32, mx_scales_out, ld_mx, N, K / 32, 0);
  return ok ? launch_status() : QGEMM_E_HIP;
}

int qgemm_run(const void* a_q, int64_t lda, const float* a_scales, const int32_t* a_zero, int a_fmt, int a_gran,
              int64_t M, const qgemm_wdesc* w_desc, const void* w_packed, void* out, int64_t ldo, int out_type,
              const float* bias, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!is_int_fmt(a_fmt) || !is_int_gran(a_gran)) return QGEMM_E_MODE;
  if (out_type != QGEMM_OUT_F32 && out_type != QGEMM_OUT_BF16 && out_type != QGEMM_OUT_I32) return QGEMM_E_MODE;
  if (bias && out_type == QGEMM_OUT_I32) return QGEMM_E_MODE;  // the int32 export is the exact sum C
  int rc = check_desc(w_desc, QGEMM_FMT_INT8_SYM);
  if (rc != QGEMM_OK) return rc;
  const int64_t N = w_desc->N, K = w_desc->K;
  const bool asym = a_fmt == QGEMM_FMT_UINT8_ASYM;
  if (K > (asym ? kAsymKMax : kSymKMax)) return QGEMM_E_OVERFLOW;
  if (M < 0 || M > kMaxRows) return QGEMM_E_SHAPE;
  if (M == 0) return QGEMM_OK;
  if (!a_q || !a_scales || !w_packed || !out || (asym && !a_zero)) return QGEMM_E_NULL;
  if (lda < K || ldo < N) return QGEMM_E_SHAPE;
  // the GEMM addresses one 256-row band of A with 32-bit byte offsets (the
  // decode kernel's last wave may read up to 32 KB past K_pad)
  if ((std::min<int64_t>(M, 256) - 1) * lda + w_desc->K_pad + 65536 >= (int64_t(1) << 32)) return QGEMM_E_SHAPE;
  if (lda % 16 != 0 || !aligned(a_q, 16) || ldo % 4 != 0 || !aligned(out, 16) || !aligned(w_packed, 256) ||
      !aligned(a_scales, 4) || (a_zero && !aligned(a_zero, 4)) || (bias && !aligned(bias, 4)))
    return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;

  const uint8_t* base = (const uint8_t*)w_packed;
  qg::GemmArgs g{};
  g.a = (const uint8_t*)a_q;
  g.lda = lda;
  g.sa = a_scales;
  g.za = a_zero;
  g.a_per_tensor = a_gran == QGEMM_GRAN_TENSOR;
  g.w = base + w_desc->codes_off;
  g.sw = (const float*)(base + w_desc->scales_off);
  g.colsum = (const int32_t*)(base + w_desc->colsum_off);
  g.w_per_tensor = w_desc->gran == QGEMM_GRAN_TENSOR;
  g.M = M;
  g.N = N;
  g.K = K;
  g.K_pad = w_desc->K_pad;
  g.out = out;
  g.ldo = ldo;
  g.bias = bias;
  hipError_t e = qg::launch_gemm_i8(g, asym, out_type, as_stream(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_E_HIP;
}

int qgemm_run_mx(const uint8_t* a_codes, int64_t lda, const uint8_t* a_e8m0, int64_t lda_s, int a_fmt, int64_t M,
                 const qgemm_wdesc* w_desc, const void* w_packed, float* out, int64_t ldo, int mode,
                 const float* bias, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (mode != QGEMM_MX_EXACT && mode != QGEMM_MX_SCALED_MFMA) return QGEMM_E_MODE;
  if (!is_mx_fmt(a_fmt)) return QGEMM_E_MODE;
  int rc = check_desc(w_desc, -1);
  if (rc != QGEMM_OK) return rc;
  const int64_t N = w_desc->N, K = w_desc->K;
  if (M < 0 || M > kMaxRows) return QGEMM_E_SHAPE;
  if (M == 0) return QGEMM_OK;
  if (!a_codes || !a_e8m0 || !w_packed || !out) return QGEMM_E_NULL;
  if (lda < code_bytes(a_fmt, K) || lda_s < K / 32 || ldo < N) return QGEMM_E_SHAPE;
  if (lda % 16 != 0 || !aligned(a_codes, 16) || ldo % 4 != 0 || !aligned(out, 16) || !aligned(w_packed, 256) ||
      (bias && !aligned(bias, 4)))
    return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;

  const uint8_t* base = (const uint8_t*)w_packed;
  qg::GemmArgs g{};
  g.a = a_codes;
  g.lda = lda;
  g.ea = a_e8m0;
  g.lda_s = lda_s;
  g.w = base + w_desc->codes_off;
  g.ew = base + w_desc->scales_off;
  g.a_fp4 = a_fmt == QGEMM_FMT_MXFP4_E2M1;
  g.w_fp4 = w_desc->fmt == QGEMM_FMT_MXFP4_E2M1;
  g.M = M;
  g.N = N;
  g.K = K;
  g.K_pad = w_desc->K_pad;
  g.out = out;
  g.ldo = ldo;
  g.bias = bias;
  hipError_t e = qg::launch_gemm_mx(g, mode, as_stream(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_E_HIP;
}

int qgemm_run_mx_grouped(const uint8_t* a_codes, int64_t lda, const uint8_t* a_e8m0, int64_t lda_s, int a_fmt,
                         int64_t M_total, const int64_t* offsets, int64_t E, const qgemm_wdesc* w_desc,
                         const void* w_packed, float* out, int64_t ldo, int mode, const float* bias, void* workspace,
                         size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (mode != QGEMM_MX_EXACT && mode != QGEMM_MX_SCALED_MFMA) return QGEMM_E_MODE;
  if (!is_mx_fmt(a_fmt)) return QGEMM_E_MODE;
  int rc = check_desc(w_desc, -1);
  if (rc != QGEMM_OK) return rc;
  // one kernel serves the grouped call: any pair of e4m3 / e2m1 operands in
  // either mode, in stages of 64 K (128 K for e2m1 x e2m1 in the scaled mode)
  const bool a4 = a_fmt == QGEMM_FMT_MXFP4_E2M1, w4 = w_desc->fmt == QGEMM_FMT_MXFP4_E2M1;
  const int64_t N = w_desc->N, K = w_desc->K;
  if (M_total < 0 || M_total > kMaxRows || E < 1 || E > kMaxExperts) return QGEMM_E_SHAPE;
  if (K % (a4 && w4 && mode == QGEMM_MX_SCALED_MFMA ? 128 : 64) != 0) return QGEMM_E_SHAPE;
  if (M_total == 0) return QGEMM_OK;
  if (!a_codes || !a_e8m0 || !offsets || !w_packed || !out) return QGEMM_E_NULL;
  if (lda < code_bytes(a_fmt, K) || lda_s < K / 32 || ldo < N) return QGEMM_E_SHAPE;
  if (lda % 16 != 0 || !aligned(a_codes, 16) || lda_s % 4 != 0 || !aligned(a_e8m0, 4) || ldo % 4 != 0 ||
      !aligned(out, 16) || !aligned(w_packed, 256) || !aligned(offsets, 8) || (bias && !aligned(bias, 4)))
    return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;

  const uint8_t* base = (const uint8_t*)w_packed;
  qg::GemmArgs g{};
  g.a = a_codes;
  g.lda = lda;
  g.ea = a_e8m0;
  g.lda_s = lda_s;
  g.w = base + w_desc->codes_off;
  g.ew = base + w_desc->scales_off;
  g.a_fp4 = a4;
  g.w_fp4 = w4;
  g.M = M_total;
  g.N = N;
  g.K = K;
  g.K_pad = w_desc->K_pad;
  g.out = out;
  g.ldo = ldo;
  g.bias = bias;
  g.groups = offsets;
  g.num_groups = (int)E;
  g.w_stride = w_desc->bytes;
  // the kernel addresses one 256-row band of A and one expert's weights with
  // 32-bit byte offsets
  if (!qg::mx_dma_eligible(g, mode)) return QGEMM_E_SHAPE;
  hipError_t e = qg::launch_gemm_mx_grouped(g, mode, as_stream(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_E_HIP;
}

int qgemm_run_w4a8(const int8_t* a_q, int64_t lda, const float* a_scales, int a_gran, int64_t M,
                   const qgemm_wdesc* w_desc, const void* w_packed, void* out, int64_t ldo, int out_type,
                   const float* bias, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!is_int_gran(a_gran)) return QGEMM_E_MODE;
  if (out_type != QGEMM_OUT_F32 && out_type != QGEMM_OUT_BF16) return QGEMM_E_MODE;
  int rc = check_desc(w_desc, QGEMM_FMT_INT4_SYM);
  if (rc != QGEMM_OK) return rc;
  const int64_t N = w_desc->N, K = w_desc->K;
  if (K > kW4MaxK) return QGEMM_E_SHAPE;
  if (M < 0 || M > kW4MaxRows) return QGEMM_E_SHAPE;
  if (M == 0) return QGEMM_OK;
  if (!a_q || !a_scales || !w_packed || !out) return QGEMM_E_NULL;
  if (lda < K || ldo < N) return QGEMM_E_SHAPE;
  // one 16-row band of A is addressed with 32-bit byte offsets (a wave may
  // read up to 4 KB past K_pad)
  if ((std::min<int64_t>(M, 16) - 1) * lda + w_desc->K_pad + 65536 >= (int64_t(1) << 32)) return QGEMM_E_SHAPE;
  if (lda % 16 != 0 || !aligned(a_q, 16) || ldo % 4 != 0 || !aligned(out, 16) || !aligned(w_packed, 256) ||
      !aligned(a_scales, 4) || (bias && !aligned(bias, 4)))
    return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;

  const uint8_t* base = (const uint8_t*)w_packed;
  qg::GemmArgs g{};
  g.a = (const uint8_t*)a_q;
  g.lda = lda;
  g.sa = a_scales;
  g.a_per_tensor = a_gran == QGEMM_GRAN_TENSOR;
  g.w = base + w_desc->codes_off;
  g.sw = (const float*)(base + w_desc->scales_off);
  g.M = M;
  g.N = N;
  g.K = K;
  g.K_pad = w_desc->K_pad;
  g.out = out;
  g.ldo = ldo;
  g.bias = bias;
  hipError_t e = qg::launch_gemm_w4a8(g, out_type, as_stream(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_E_HIP;
}

// ---- measured ceilings (not part of the GEMM path; qgemm_ceiling.h) ----

namespace {
constexpr int64_t kCeilMaxTrips = int64_t(1) << 24;
int check_ceiling(int kind, int waves_per_simd, int64_t trips) {
  if (kind < QGEMM_CEIL_I8 || kind > QGEMM_CEIL_BF16) return QGEMM_E_MODE;
  if (waves_per_simd < 1 || waves_per_simd > 2 || trips < 1 || trips > kCeilMaxTrips) return QGEMM_E_SHAPE;
  return QGEMM_OK;
}
}  // namespace

int qgemm_ceiling_mfma_shape(int kind, int waves_per_simd, int64_t trips, int64_t* workgroups, double* ops) {
  if (!workgroups || !ops) return QGEMM_E_NULL;
  int rc = check_ceiling(kind, waves_per_simd, trips);
  if (rc != QGEMM_OK) return rc;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;
  // 2 * M * N * K of one instruction
  const double per = kind == QGEMM_CEIL_I8 ? 2.0 * 16 * 16 * 64 : kind == QGEMM_CEIL_BF16 ? 2.0 * 32 * 32 * 16
                                                                                       : 2.0 * 32 * 32 * 64;
  const int64_t wg = qg::cu_count();
  *workgroups = wg;
  *ops = per * (double)qg::kCeilSets * (double)trips * 4.0 * waves_per_simd * (double)wg;
  return QGEMM_OK;
}

int qgemm_ceiling_mfma(int kind, int waves_per_simd, int64_t trips, const void* a_ops, const void* b_ops,
                       int32_t* sink, int64_t* clocks, void* stream) {
  if (!a_ops || !b_ops || !sink) return QGEMM_E_NULL;
  int rc = check_ceiling(kind, waves_per_simd, trips);
  if (rc != QGEMM_OK) return rc;
  if (!aligned(a_ops, 32) || !aligned(b_ops, 32) || !aligned(sink, 4) || (clocks && !aligned(clocks, 8)))
    return QGEMM_E_ALIGN;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;
  hipError_t e = qg::launch_ceiling_mfma(kind, waves_per_simd, trips, static_cast<const uint8_t*>(a_ops),
                                         static_cast<const uint8_t*>(b_ops), sink, clocks, as_stream(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_E_HIP;
}

int qgemm_ceiling_stream(const void* src, int64_t bytes, int64_t block_bytes, int32_t* sink, void* stream) {
  if (!src || !sink) return QGEMM_E_NULL;
  if (bytes < 0 || bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return QGEMM_E_SHAPE;
  if (block_bytes < 16384 || block_bytes > (int64_t(1) << 20) || block_bytes % 16384 != 0) return QGEMM_E_SHAPE;
  if ((bytes + block_bytes - 1) / block_bytes > 0x7fffffff) return QGEMM_E_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return QGEMM_E_ALIGN;
  if (bytes == 0) return QGEMM_OK;
  int dc = check_device();
  if (dc != QGEMM_OK) return dc;
  hipError_t e = qg::launch_ceiling_stream(static_cast<const uint8_t*>(src), bytes, block_bytes, sink,
                                           as_stream(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_E_HIP;
}

}  // extern "C"
