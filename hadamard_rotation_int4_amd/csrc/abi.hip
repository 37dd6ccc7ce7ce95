// extern "C" entry points of libhr.so (declared in include/hr.h): host-side
// argument validation, then a launch on the caller's stream.  A call that
// fails validation makes no HIP call at all.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "hr.h"
#include "hr_internal.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int32_t ok() { return HR_OK; }

int32_t from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HR_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}
bool valid_group(int32_t g) { return g == 32 || g == 64 || g == 128 || g == 256; }

// Shared checks of hr_rotate and hr_rotate_quant_int4; fills p.
int32_t check_rotation(const char* fn, const void* x, int32_t x_dtype, int64_t rows, int32_t n,
                       int32_t m, const int8_t* signs, const float* block, int* p_out) {
  if (rows < 0) return fail(HR_EINVAL, "%s: rows < 0", fn);
  if (!x && rows > 0) return fail(HR_EINVAL, "%s: x is NULL", fn);
  if (x_dtype != HR_BF16 && x_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: x_dtype must be HR_BF16 or HR_F32", fn);
  if (!aligned16(x) || (signs && !aligned16(signs)))
    return fail(HR_EINVAL, "%s: x and signs must be 16-byte aligned", fn);
  if (m < 1 || m > 16) return fail(HR_EUNSUPPORTED, "%s: m=%d outside [1, 16]", fn, m);
  if (n <= 0 || n % m) return fail(HR_EUNSUPPORTED, "%s: n=%d is not a multiple of m=%d", fn, n, m);
  const int p = n / m;
  if (!pow2(p) || p < 64 || p > 16384)
    return fail(HR_EUNSUPPORTED, "%s: n/m=%d is not a power of two in [64, 16384]", fn, p);
  if (n > 16384) return fail(HR_EUNSUPPORTED, "%s: n=%d > 16384", fn, n);
  if (m == 1 && block) return fail(HR_EINVAL, "%s: block must be NULL when m == 1", fn);
  if (m > 1 && !block) return fail(HR_EINVAL, "%s: block is NULL with m=%d", fn, m);
  if (block && (reinterpret_cast<uintptr_t>(block) & 3u))
    return fail(HR_EINVAL, "%s: block must be 4-byte aligned", fn);
  *p_out = p;
  return HR_OK;
}

}  // namespace

extern "C" {

int32_t hr_abi_version(void) { return HR_ABI_VERSION; }

// HR_SOURCE_HASH is defined by the build: a hash of the library's sources, so
// a binding can tell a library built from other sources.
#ifndef HR_SOURCE_HASH
#define HR_SOURCE_HASH "unknown"
#endif
const char* hr_build_id(void) { return HR_SOURCE_HASH; }

const char* hr_status_string(int32_t status) {
  switch (status) {
    case HR_OK: return "HR_OK: success";
    case HR_EINVAL: return "HR_EINVAL: invalid argument";
    case HR_EUNSUPPORTED: return "HR_EUNSUPPORTED: size or mode not supported";
    case HR_EDEVICE: return "HR_EDEVICE: kernel launch failed";
    default: return "unknown hr_status";
  }
}

const char* hr_last_error(void) { return g_last_error.c_str(); }

int32_t hr_rotate(const void* x, int32_t x_dtype, float* y, int64_t rows, int32_t n, int32_t m,
                  const int8_t* signs, const float* block, void* stream) {
  int p = 0;
  const int32_t st = check_rotation("hr_rotate", x, x_dtype, rows, n, m, signs, block, &p);
  if (st) return st;
  if (!y && rows > 0) return fail(HR_EINVAL, "hr_rotate: y is NULL");
  if (!aligned16(y)) return fail(HR_EINVAL, "hr_rotate: y must be 16-byte aligned");
  if (rows == 0) return ok();
  hr::RhtArgs a{};
  a.x = x;
  a.x_bf16 = x_dtype == HR_BF16;
  a.rows = rows;
  a.n = n;
  a.m = m;
  a.p = p;
  a.signs = signs;
  a.block = block;
  a.y = y;
  return from_hip(hr::launch_rht(a, static_cast<hipStream_t>(stream)), "hr_rotate");
}

// Shared body of hr_rotate_quant_int4 and hr_rotate_quant_int8.
static int32_t rotate_quant(const char* fn, int bits, const void* x, int32_t x_dtype, int64_t rows,
                            int32_t n, int32_t m, const int8_t* signs, const float* block,
                            int32_t group, uint8_t* codes, void* scales, int32_t scale_dtype,
                            void* stream) {
  int p = 0;
  const int32_t st = check_rotation(fn, x, x_dtype, rows, n, m, signs, block, &p);
  if (st) return st;
  if ((!codes || !scales) && rows > 0)
    return fail(HR_EINVAL, "%s: codes and scales are required", fn);
  if (!aligned16(codes) || !aligned16(scales))
    return fail(HR_EINVAL, "%s: codes and scales must be 16-byte aligned", fn);
  if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
  if (!valid_group(group)) return fail(HR_EUNSUPPORTED, "%s: group=%d not in {32,64,128,256}", fn, group);
  if (p % group) return fail(HR_EUNSUPPORTED, "%s: group=%d does not divide p=%d", fn, group, p);
  if (rows == 0) return ok();
  hr::RhtArgs a{};
  a.x = x;
  a.x_bf16 = x_dtype == HR_BF16;
  a.rows = rows;
  a.n = n;
  a.m = m;
  a.p = p;
  a.signs = signs;
  a.block = block;
  a.group = group;
  a.codes = codes;
  a.bits = bits;
  a.scales = scales;
  a.scale_f16 = scale_dtype == HR_F16;
  return from_hip(hr::launch_rht(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t hr_rotate_quant_int4(const void* x, int32_t x_dtype, int64_t rows, int32_t n, int32_t m,
                             const int8_t* signs, const float* block, int32_t group,
                             uint8_t* codes, void* scales, int32_t scale_dtype, void* stream) {
  return rotate_quant("hr_rotate_quant_int4", 4, x, x_dtype, rows, n, m, signs, block, group, codes,
                      scales, scale_dtype, stream);
}

int32_t hr_rotate_quant_int8(const void* x, int32_t x_dtype, int64_t rows, int32_t n, int32_t m,
                             const int8_t* signs, const float* block, int32_t group,
                             int8_t* codes, void* scales, int32_t scale_dtype, void* stream) {
  return rotate_quant("hr_rotate_quant_int8", 8, x, x_dtype, rows, n, m, signs, block, group,
                      reinterpret_cast<uint8_t*>(codes), scales, scale_dtype, stream);
}

// Shared body of hr_quant_int4 and hr_quant_int8.
static int32_t quant_plain(const char* fn, int bits, const void* x, int32_t x_dtype, int64_t rows,
                           int32_t n, int32_t group, uint8_t* codes, void* scales, int32_t scale_dtype,
                           void* stream) {
  if (rows < 0) return fail(HR_EINVAL, "%s: rows < 0", fn);
  if ((!x || !codes || !scales) && rows > 0)
    return fail(HR_EINVAL, "%s: x, codes and scales are required", fn);
  if (x_dtype != HR_BF16 && x_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: x_dtype must be HR_BF16 or HR_F32", fn);
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(HR_EINVAL, "%s: x, codes and scales must be 16-byte aligned", fn);
  if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
  if (!valid_group(group)) return fail(HR_EUNSUPPORTED, "%s: group=%d not in {32,64,128,256}", fn, group);
  if (n <= 0 || n % group || n > (1 << 30))
    return fail(HR_EUNSUPPORTED, "%s: n=%d must be a positive multiple of group=%d", fn, n, group);
  if (rows == 0) return ok();
  hr::QuantArgs a{};
  a.x = x;
  a.x_bf16 = x_dtype == HR_BF16;
  a.rows = rows;
  a.n = n;
  a.group = group;
  a.bits = bits;
  a.codes = codes;
  a.scales = scales;
  a.scale_f16 = scale_dtype == HR_F16;
  return from_hip(hr::launch_quant(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t hr_quant_int4(const void* x, int32_t x_dtype, int64_t rows, int32_t n, int32_t group,
                      uint8_t* codes, void* scales, int32_t scale_dtype, void* stream) {
  return quant_plain("hr_quant_int4", 4, x, x_dtype, rows, n, group, codes, scales, scale_dtype, stream);
}

int32_t hr_quant_int8(const void* x, int32_t x_dtype, int64_t rows, int32_t n, int32_t group,
                      int8_t* codes, void* scales, int32_t scale_dtype, void* stream) {
  return quant_plain("hr_quant_int8", 8, x, x_dtype, rows, n, group, reinterpret_cast<uint8_t*>(codes),
                     scales, scale_dtype, stream);
}

int32_t hr_butterfly_coeffs(const float* angles, int32_t n, int32_t precondition, float* coeffs,
                            void* stream) {
  const char* fn = "hr_butterfly_coeffs";
  if (!angles || !coeffs) return fail(HR_EINVAL, "%s: angles and coeffs are required", fn);
  if (!aligned16(angles) || !aligned16(coeffs))
    return fail(HR_EINVAL, "%s: angles and coeffs must be 16-byte aligned", fn);
  if (precondition != 0 && precondition != 1) return fail(HR_EINVAL, "%s: precondition must be 0 or 1", fn);
  if (!pow2(n) || n < 64 || n > 8192)
    return fail(HR_EUNSUPPORTED, "%s: n=%d is not a power of two in [64, 8192]", fn, n);
  return from_hip(hr::launch_butterfly_coeffs(angles, n, ilog2(n), precondition, coeffs,
                                              static_cast<hipStream_t>(stream)), fn);
}

int32_t hr_butterfly_apply(const float* x, float* y, int64_t rows, int32_t n, const float* coeffs,
                           int32_t precondition, const int32_t* perm, int32_t inverse,
                           int32_t group, uint8_t* codes, void* scales, int32_t scale_dtype,
                           void* stream) {
  const char* fn = "hr_butterfly_apply";
  if (rows < 0) return fail(HR_EINVAL, "%s: rows < 0", fn);
  if (!coeffs) return fail(HR_EINVAL, "%s: coeffs is required", fn);
  if (!x && rows > 0) return fail(HR_EINVAL, "%s: x is NULL", fn);
  if (!y && !codes && rows > 0) return fail(HR_EINVAL, "%s: y and codes are both NULL", fn);
  if (!codes && scales) return fail(HR_EINVAL, "%s: scales given without codes", fn);
  if (codes && !scales) return fail(HR_EINVAL, "%s: codes given without scales", fn);
  if (!aligned16(x) || (y && !aligned16(y)) || !aligned16(coeffs) || (perm && !aligned16(perm)) ||
      (codes && !aligned16(codes)) || (scales && !aligned16(scales)))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (precondition != 0 && precondition != 1) return fail(HR_EINVAL, "%s: precondition must be 0 or 1", fn);
  if (inverse != 0 && inverse != 1) return fail(HR_EINVAL, "%s: inverse must be 0 or 1", fn);
  if (!pow2(n) || n < 64 || n > 8192)
    return fail(HR_EUNSUPPORTED, "%s: n=%d is not a power of two in [64, 8192]", fn, n);
  if (codes) {
    if (inverse) return fail(HR_EUNSUPPORTED, "%s: quantization needs inverse == 0", fn);
    if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
      return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
    if (!valid_group(group) || n % group)
      return fail(HR_EUNSUPPORTED, "%s: group=%d invalid for n=%d", fn, group, n);
  }
  if (rows == 0) return ok();
  hr::ButterflyArgs a{};
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.n = n;
  a.log2n = ilog2(n);
  a.coeffs = coeffs;
  a.precondition = precondition;
  a.perm = perm;
  a.inverse = inverse;
  a.group = group;
  a.codes = codes;
  a.scales = scales;
  a.scale_f16 = scale_dtype == HR_F16;
  return from_hip(hr::launch_butterfly(a, static_cast<hipStream_t>(stream)), fn);
}

// Checks a HARP schedule given on the host and fills the per-stage offsets.
static int32_t harp_schedule(const char* fn, const int32_t* radices, int32_t nstages, int32_t* d_out,
                             hr::HarpSchedule* sc) {
  if (!radices) return fail(HR_EINVAL, "%s: radices is NULL", fn);
  if (nstages < 1 || nstages > hr::kHarpMaxStages)
    return fail(HR_EUNSUPPORTED, "%s: nstages=%d outside [1, %d]", fn, nstages, hr::kHarpMaxStages);
  int64_t d = 1;
  for (int t = 0; t < nstages; ++t) {
    if (radices[t] < 2 || radices[t] > hr::kHarpMaxRadix)
      return fail(HR_EUNSUPPORTED, "%s: radix %d of stage %d outside [2, %d]", fn, radices[t], t,
                  hr::kHarpMaxRadix);
    d *= radices[t];
    if (d > 16384) return fail(HR_EUNSUPPORTED, "%s: the radices multiply past 16384", fn);
  }
  if (d % 4) return fail(HR_EUNSUPPORTED, "%s: d=%lld is not a multiple of 4", fn, (long long)d);
  *sc = hr::HarpSchedule{};
  sc->nstages = nstages;
  int64_t stride = 1, nblk = 0, th = 0, fb = 0, bo = 0;
  for (int t = 0; t < nstages; ++t) {
    const int b = radices[t];
    sc->radix[t] = b;
    sc->stride[t] = (int)stride;
    sc->block_begin[t] = nblk;
    sc->theta_off[t] = th;
    sc->fallback_off[t] = fb;
    sc->blocks_off[t] = bo;
    stride *= b;
    nblk += d / b;
    th += (d / b) * (b == 2 ? 1 : b * (b - 1) / 2);
    if (!pow2(b)) fb += (int64_t)b * b;
    bo += (int64_t)4 * ((b * b + 3) / 4) * (d / b);   // quads of coefficients, the last one padded
  }
  sc->block_begin[nstages] = nblk;
  *d_out = (int32_t)d;
  return HR_OK;
}

int32_t hr_harp_blocks(const int32_t* radices, int32_t nstages, const float* theta,
                       const float* fallbacks, float* blocks, void* stream) {
  const char* fn = "hr_harp_blocks";
  hr::HarpSchedule sc;
  int32_t d = 0;
  const int32_t st = harp_schedule(fn, radices, nstages, &d, &sc);
  if (st) return st;
  bool need_fb = false;
  for (int t = 0; t < nstages; ++t) need_fb |= !pow2(radices[t]);
  if (!theta || !blocks) return fail(HR_EINVAL, "%s: theta and blocks are required", fn);
  if (need_fb && !fallbacks)
    return fail(HR_EINVAL, "%s: a radix is not a power of two but fallbacks is NULL", fn);
  if (!aligned16(theta) || !aligned16(blocks) || (fallbacks && !aligned16(fallbacks)))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  return from_hip(hr::launch_harp_blocks(sc, theta, fallbacks, blocks, static_cast<hipStream_t>(stream)),
                  fn);
}

int32_t hr_harp_apply(const float* x, float* y, int64_t rows, const int32_t* radices, int32_t nstages,
                      const float* blocks, int32_t inverse, int32_t group, uint8_t* codes,
                      void* scales, int32_t scale_dtype, void* stream) {
  const char* fn = "hr_harp_apply";
  hr::HarpSchedule sc;
  int32_t d = 0;
  const int32_t st = harp_schedule(fn, radices, nstages, &d, &sc);
  if (st) return st;
  if (rows < 0) return fail(HR_EINVAL, "%s: rows < 0", fn);
  if (!blocks) return fail(HR_EINVAL, "%s: blocks is required", fn);
  if (!x && rows > 0) return fail(HR_EINVAL, "%s: x is NULL", fn);
  if (!y && !codes && rows > 0) return fail(HR_EINVAL, "%s: y and codes are both NULL", fn);
  if (!codes && scales) return fail(HR_EINVAL, "%s: scales given without codes", fn);
  if (codes && !scales) return fail(HR_EINVAL, "%s: codes given without scales", fn);
  if (!aligned16(x) || (y && !aligned16(y)) || !aligned16(blocks) || (codes && !aligned16(codes)) ||
      (scales && !aligned16(scales)))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (inverse != 0 && inverse != 1) return fail(HR_EINVAL, "%s: inverse must be 0 or 1", fn);
  if (codes) {
    if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
      return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
    if (!valid_group(group) || d % group)
      return fail(HR_EUNSUPPORTED, "%s: group=%d invalid for d=%d", fn, group, d);
  }
  if (rows == 0) return ok();
  hr::HarpArgs a{};
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.d = d;
  a.sc = sc;
  a.blocks = blocks;
  a.inverse = inverse;
  a.group = group;
  a.codes = codes;
  a.scales = scales;
  a.scale_f16 = scale_dtype == HR_F16;
  return from_hip(hr::launch_harp_apply(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t hr_dequant_int4(const uint8_t* codes, const void* scales, int32_t scale_dtype, int64_t rows,
                        int32_t n, int32_t group, float* out, void* stream) {
  const char* fn = "hr_dequant_int4";
  if (rows < 0) return fail(HR_EINVAL, "%s: rows < 0", fn);
  if ((!codes || !scales || !out) && rows > 0)
    return fail(HR_EINVAL, "%s: codes, scales and out are required", fn);
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
  if (!valid_group(group)) return fail(HR_EUNSUPPORTED, "%s: group=%d not in {32,64,128,256}", fn, group);
  if (n <= 0 || n % group || n > (1 << 30))
    return fail(HR_EUNSUPPORTED, "%s: n=%d must be a positive multiple of group=%d", fn, n, group);
  if (rows == 0) return ok();
  return from_hip(hr::launch_dequant(codes, scales, scale_dtype == HR_F16, rows, n, group, out,
                                     static_cast<hipStream_t>(stream)), fn);
}

// Shared body of hr_w4a4_gemm, hr_w4a8_gemm and hr_w8a8_gemm.
static int32_t gemm(const char* fn, int a_int8, int w_int8, const uint8_t* a_codes, const void* a_scales,
                    const uint8_t* w_codes, const void* w_scales, int32_t scale_dtype, int64_t M,
                    int64_t N, int64_t K, int32_t group, float* c, int32_t* group_acc,
                    void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(HR_EINVAL, "%s: negative size", fn);
  if (M > 0 && N > 0 && (!a_codes || !a_scales || !w_codes || !w_scales || !c))
    return fail(HR_EINVAL, "%s: a_codes, a_scales, w_codes, w_scales and c are required", fn);
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(c) || (group_acc && !aligned16(group_acc)))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
  if (!valid_group(group)) return fail(HR_EUNSUPPORTED, "%s: group=%d not in {32,64,128,256}", fn, group);
  if (N % 64) return fail(HR_EUNSUPPORTED, "%s: N=%lld is not a multiple of 64", fn, (long long)N);
  if (K == 0 || K % 256 || K % group || K > 65536)
    return fail(HR_EUNSUPPORTED, "%s: K=%lld must be a multiple of 256 and of group, <= 65536", fn,
                (long long)K);
  if (M == 0 || N == 0) return ok();
  hr::GemmArgs a{};
  a.a = a_codes;
  a.a_int8 = a_int8;
  a.w_int8 = w_int8;
  a.sa = a_scales;
  a.w = w_codes;
  a.sw = w_scales;
  a.scale_f16 = scale_dtype == HR_F16;
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = group;
  a.c = c;
  a.group_acc = group_acc;
  return from_hip(hr::launch_gemm(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t hr_w4a4_gemm(const uint8_t* a_codes, const void* a_scales, const uint8_t* w_codes,
                     const void* w_scales, int32_t scale_dtype, int64_t M, int64_t N, int64_t K,
                     int32_t group, float* c, int32_t* group_acc, void* stream) {
  return gemm("hr_w4a4_gemm", 0, 0, a_codes, a_scales, w_codes, w_scales, scale_dtype, M, N, K, group,
              c, group_acc, stream);
}

int32_t hr_w4a8_gemm(const int8_t* a_codes, const void* a_scales, const uint8_t* w_codes,
                     const void* w_scales, int32_t scale_dtype, int64_t M, int64_t N, int64_t K,
                     int32_t group, float* c, int32_t* group_acc, void* stream) {
  return gemm("hr_w4a8_gemm", 1, 0, reinterpret_cast<const uint8_t*>(a_codes), a_scales, w_codes,
              w_scales, scale_dtype, M, N, K, group, c, group_acc, stream);
}

int32_t hr_w8a8_gemm(const int8_t* a_codes, const void* a_scales, const int8_t* w_codes,
                     const void* w_scales, int32_t scale_dtype, int64_t M, int64_t N, int64_t K,
                     int32_t group, float* c, int32_t* group_acc, void* stream) {
  return gemm("hr_w8a8_gemm", 1, 1, reinterpret_cast<const uint8_t*>(a_codes), a_scales,
              reinterpret_cast<const uint8_t*>(w_codes), w_scales, scale_dtype, M, N, K, group, c,
              group_acc, stream);
}

int32_t hr_rotate_quant_w4a4_gemm(const void* x, int32_t x_dtype, const int8_t* signs, int32_t group,
                                  const uint8_t* w_codes, const void* w_scales, int32_t scale_dtype,
                                  int64_t M, int64_t N, int64_t K, float* c, uint8_t* a_codes,
                                  void* a_scales, void* stream) {
  const char* fn = "hr_rotate_quant_w4a4_gemm";
  if (M < 0 || N < 0 || K < 0) return fail(HR_EINVAL, "%s: negative size", fn);
  if (M > 0 && N > 0 && (!x || !w_codes || !w_scales || !c))
    return fail(HR_EINVAL, "%s: x, w_codes, w_scales and c are required", fn);
  if ((a_codes == nullptr) != (a_scales == nullptr))
    return fail(HR_EINVAL, "%s: a_codes and a_scales are given together or not at all", fn);
  if (!aligned16(x) || (signs && !aligned16(signs)) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(c) || (a_codes && !aligned16(a_codes)) || (a_scales && !aligned16(a_scales)))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (x_dtype != HR_BF16) return fail(HR_EUNSUPPORTED, "%s: x_dtype must be HR_BF16", fn);
  if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
  if (!valid_group(group)) return fail(HR_EUNSUPPORTED, "%s: group=%d not in {32,64,128,256}", fn, group);
  if (M > 16) return fail(HR_EUNSUPPORTED, "%s: M=%lld > 16 (decode shapes only)", fn, (long long)M);
  if (K != 2048 && K != 4096) return fail(HR_EUNSUPPORTED, "%s: K=%lld not 2048 or 4096", fn, (long long)K);
  if (N % 64) return fail(HR_EUNSUPPORTED, "%s: N=%lld is not a multiple of 64", fn, (long long)N);
  if (M == 0 || N == 0) return ok();
  hr::FusedDecodeArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.signs = signs;
  a.norm = (float)(1.0 / sqrt((double)K));
  a.w = w_codes;
  a.sw = w_scales;
  a.scale_f16 = scale_dtype == HR_F16;
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = group;
  a.c = c;
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  return from_hip(hr::launch_rotate_quant_gemm_decode(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t hr_w4a4_to_fp6(const uint8_t* codes, const void* scales, int32_t scale_dtype, int64_t rows, int64_t K,
                       int32_t group, uint8_t* out, void* out_scales, void* stream) {
  const char* fn = "hr_w4a4_to_fp6";
  if (rows < 0 || K < 0) return fail(HR_EINVAL, "%s: negative size", fn);
  if (rows > 0 && K > 0 && (!codes || !out)) return fail(HR_EINVAL, "%s: codes and out are required", fn);
  if (!scales != !out_scales) return fail(HR_EINVAL, "%s: scales and out_scales go together", fn);
  if (!aligned16(codes) || !aligned16(out) || !aligned16(scales) || !aligned16(out_scales))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (K % 128 || K > (int64_t(1) << 30))
    return fail(HR_EUNSUPPORTED, "%s: K=%lld must be a multiple of 128", fn, (long long)K);
  if (rows > int64_t(128) * 65535)
    return fail(HR_EUNSUPPORTED, "%s: rows=%lld above 128 * 65535", fn, (long long)rows);
  if (scales) {
    if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
      return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
    if ((group != 128 && group != 256) || K % group)
      return fail(HR_EUNSUPPORTED, "%s: group=%d must be 128 or 256 and divide K", fn, group);
  }
  if (rows == 0 || K == 0) return ok();
  return from_hip(hr::launch_int4_to_fp6(codes, scales, scale_dtype == HR_F16, rows, K, group, out, out_scales,
                                         static_cast<hipStream_t>(stream)),
                  fn);
}

int32_t hr_rotate_quant_fp6(const void* x, int32_t x_dtype, const int8_t* signs, int64_t rows, int32_t n,
                            int32_t group, int32_t scale_dtype, uint8_t* tiles, void* scales, void* stream) {
  const char* fn = "hr_rotate_quant_fp6";
  if (rows < 0) return fail(HR_EINVAL, "%s: rows < 0", fn);
  if (rows > 0 && (!x || !tiles || !scales)) return fail(HR_EINVAL, "%s: x, tiles and scales are required", fn);
  if (x_dtype != HR_BF16) return fail(HR_EUNSUPPORTED, "%s: x_dtype must be HR_BF16", fn);
  if (!aligned16(x) || !aligned16(tiles) || !aligned16(scales))
    return fail(HR_EINVAL, "%s: x, tiles and scales must be 16-byte aligned", fn);
  if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
  if (n != 2048 && n != 4096) return fail(HR_EUNSUPPORTED, "%s: n=%d not 2048 or 4096", fn, n);
  if (group != 128 && group != 256) return fail(HR_EUNSUPPORTED, "%s: group=%d not in {128,256}", fn, group);
  if (rows == 0) return ok();
  hr::RhtArgs a{};
  a.x = x;
  a.x_bf16 = 1;
  a.rows = rows;
  a.n = n;
  a.m = 1;
  a.p = n;
  a.signs = signs;
  a.block = nullptr;
  a.y = nullptr;
  a.group = group;
  a.codes = tiles;
  a.bits = 6;
  a.scales = scales;
  a.scale_f16 = scale_dtype == HR_F16;
  if (!hr::launch_rotate_quant_fp6(a, static_cast<hipStream_t>(stream)))
    return fail(HR_EUNSUPPORTED, "%s: unsupported case", fn);
  return from_hip(hipGetLastError(), fn);
}

int32_t hr_w4a4_gemm_fp6(const uint8_t* a_f6, const void* a_scales, const uint8_t* w_f6, const void* w_scales,
                         int32_t scale_dtype, int64_t M, int64_t N, int64_t K, int32_t group, float* c,
                         int32_t* group_acc, void* stream) {
  const char* fn = "hr_w4a4_gemm_fp6";
  if (M < 0 || N < 0 || K < 0) return fail(HR_EINVAL, "%s: negative size", fn);
  if (M > 0 && N > 0 && (!a_f6 || !a_scales || !w_f6 || !w_scales || !c))
    return fail(HR_EINVAL, "%s: a_f6, a_scales, w_f6, w_scales and c are required", fn);
  if (!aligned16(a_f6) || !aligned16(a_scales) || !aligned16(w_f6) || !aligned16(w_scales) || !aligned16(c) ||
      (group_acc && !aligned16(group_acc)))
    return fail(HR_EINVAL, "%s: pointers must be 16-byte aligned", fn);
  if (scale_dtype != HR_F16 && scale_dtype != HR_F32)
    return fail(HR_EINVAL, "%s: scale_dtype must be HR_F16 or HR_F32", fn);
  if (group != 128 && group != 256)
    return fail(HR_EUNSUPPORTED, "%s: group=%d not in {128,256}", fn, group);
  if (N % 128) return fail(HR_EUNSUPPORTED, "%s: N=%lld is not a multiple of 128", fn, (long long)N);
  if (K == 0 || K % group || K > 65536)
    return fail(HR_EUNSUPPORTED, "%s: K=%lld must be a multiple of group, <= 65536", fn, (long long)K);
  if (M == 0 || N == 0) return ok();
  hr::GemmArgs a{};
  a.a = a_f6;
  a.sa = a_scales;
  a.w = w_f6;
  a.sw = w_scales;
  a.scale_f16 = scale_dtype == HR_F16;
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = group;
  a.c = c;
  a.group_acc = group_acc;
  return from_hip(hr::launch_gemm_fp6(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
