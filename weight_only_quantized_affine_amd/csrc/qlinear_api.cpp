// C ABI of the library (declared in include/qlinear.h): host-side validation, then dispatch
// to the gfx950 kernels.  Validation touches no device state, so every error path is testable
// without a GPU; on error nothing is launched and qlinear_last_error() names the argument.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qlinear.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

ql_status fail(ql_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
ql_status ok() {
  g_last_error.clear();
  return QL_OK;
}
ql_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QL_ERR_LAUNCH, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool is16(ql_dtype d) { return d == QL_F16 || d == QL_BF16; }
bool is_out(ql_dtype d) { return d == QL_F32 || d == QL_F16 || d == QL_BF16; }
size_t esize(ql_dtype d) { return d == QL_F32 ? 4 : 2; }

#define CHECK(cond, st, ...)          \
  do {                                \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

// Shared checks of the affine layout: bits, group size, k.
ql_status check_affine(const char* fn, int64_t n, int64_t k, int bits, int g, ql_dtype pdt) {
  CHECK(n >= 0 && k >= 0, QL_ERR_SHAPE, "%s: n=%lld and k=%lld must be >= 0", fn, (long long)n, (long long)k);
  CHECK(bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8, QL_ERR_UNSUPPORTED,
        "%s: bits=%d not supported (2, 3, 4, 5, 6 or 8)", fn, bits);
  CHECK(g == 32 || g == 64 || g == 128, QL_ERR_UNSUPPORTED, "%s: group_size=%d not supported (32, 64 or 128)", fn,
        g);
  CHECK(k % 32 == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 32", fn, (long long)k);
  CHECK(k % g == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of group_size=%d", fn, (long long)k, g);
  CHECK(is16(pdt), QL_ERR_DTYPE, "%s: param_dtype must be QL_F16 or QL_BF16", fn);
  return QL_OK;
}

ql_status check_product(const char* fn, const void* x, ql_dtype xdt, int64_t m, int64_t k, const uint32_t* packed,
                        const void* scales, const void* biases, ql_dtype pdt, int64_t n, int bits, int g,
                        const void* layer_bias, const void* y, ql_dtype ydt) {
  CHECK(m >= 0, QL_ERR_SHAPE, "%s: m=%lld must be >= 0", fn, (long long)m);
  ql_status st = check_affine(fn, n, k, bits, g, pdt);
  if (st != QL_OK) return st;
  CHECK(is16(xdt), QL_ERR_DTYPE, "%s: x_dtype must be QL_F16 or QL_BF16", fn);
  CHECK(is_out(ydt), QL_ERR_DTYPE, "%s: y_dtype must be QL_F32, QL_F16 or QL_BF16", fn);
  if (m == 0 || n == 0) return QL_OK;
  CHECK(y != nullptr, QL_ERR_NULL, "%s: y must not be NULL", fn);
  if (k > 0)
    CHECK(x && packed && scales && biases, QL_ERR_NULL, "%s: x, packed, scales and biases must not be NULL", fn);
  CHECK(aligned(x, 16), QL_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
  CHECK(aligned(packed, 16), QL_ERR_ALIGN, "%s: packed must be 16-byte aligned", fn);
  CHECK(aligned(scales, 2) && aligned(biases, 2), QL_ERR_ALIGN, "%s: scales and biases must be 2-byte aligned", fn);
  CHECK(aligned(layer_bias, 2), QL_ERR_ALIGN, "%s: layer_bias must be 2-byte aligned", fn);
  CHECK(aligned(y, esize(ydt)), QL_ERR_ALIGN, "%s: y must be aligned to its element size", fn);
  return QL_OK;
}

int dt(ql_dtype d) { return (int)d; }

}  // namespace

extern "C" {

const char* qlinear_last_error(void) { return g_last_error.c_str(); }
const char* qlinear_version(void) { return "qlinear-gfx950 0.1"; }

ql_status qlinear_quantize(const float* w, int64_t n, int64_t k, int bits, int group_size, ql_dtype param_dtype,
                           uint32_t* packed, void* scales, void* biases, void* stream) {
  const char* fn = "qlinear_quantize";
  ql_status st = check_affine(fn, n, k, bits, group_size, param_dtype);
  if (st != QL_OK) return st;
  if (n == 0 || k == 0) return ok();
  CHECK(w && packed && scales && biases, QL_ERR_NULL, "%s: w, packed, scales and biases must not be NULL", fn);
  CHECK(aligned(w, 16), QL_ERR_ALIGN, "%s: w must be 16-byte aligned", fn);
  CHECK(aligned(packed, 16), QL_ERR_ALIGN, "%s: packed must be 16-byte aligned", fn);
  CHECK(aligned(scales, 2) && aligned(biases, 2), QL_ERR_ALIGN, "%s: scales and biases must be 2-byte aligned", fn);
  return launched(ql::launch_quantize(w, n, k, bits, group_size, dt(param_dtype), packed, scales, biases,
                                      (hipStream_t)stream),
                  fn);
}

ql_status qlinear_quantize_q8_0(const float* w, int64_t rows, int64_t k, uint8_t* blocks, void* stream) {
  const char* fn = "qlinear_quantize_q8_0";
  CHECK(rows >= 0 && k >= 0, QL_ERR_SHAPE, "%s: rows and k must be >= 0", fn);
  CHECK(k % 32 == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 32", fn, (long long)k);
  if (rows == 0 || k == 0) return ok();
  CHECK(w && blocks, QL_ERR_NULL, "%s: w and blocks must not be NULL", fn);
  CHECK(aligned(w, 16), QL_ERR_ALIGN, "%s: w must be 16-byte aligned", fn);
  CHECK(aligned(blocks, 2), QL_ERR_ALIGN, "%s: blocks must be 2-byte aligned", fn);
  return launched(ql::launch_quantize_q8_0(w, rows, k, blocks, (hipStream_t)stream), fn);
}

ql_status qlinear_transcode_gptq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales,
                                 ql_dtype scale_dtype, int64_t k, int64_t n, int bits, int group_size, int v1_zeros,
                                 uint32_t* packed, void* scales_out, void* biases_out, void* stream) {
  const char* fn = "qlinear_transcode_gptq";
  CHECK(k >= 0 && n >= 0, QL_ERR_SHAPE, "%s: k and n must be >= 0", fn);
  CHECK(bits == 2 || bits == 3 || bits == 4 || bits == 8, QL_ERR_UNSUPPORTED,
        "%s: bits=%d not supported (GPTQ's continuous widths 2, 3, 4, 8)", fn, bits);
  CHECK(group_size == 32 || group_size == 64 || group_size == 128, QL_ERR_UNSUPPORTED,
        "%s: group_size=%d not supported (32, 64 or 128)", fn, group_size);
  CHECK(k % 32 == 0 && k % group_size == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 32 and of group_size", fn,
        (long long)k);
  CHECK(n * bits % 32 == 0, QL_ERR_SHAPE, "%s: n*bits (%lld) must fill whole words (qzeros rows)", fn,
        (long long)(n * bits));
  CHECK(is16(scale_dtype), QL_ERR_DTYPE, "%s: scale_dtype must be QL_F16 or QL_BF16", fn);
  if (k == 0 || n == 0) return ok();
  CHECK(qweight && qzeros && scales && packed && scales_out && biases_out, QL_ERR_NULL,
        "%s: qweight, qzeros, scales, packed, scales_out and biases_out must not be NULL", fn);
  CHECK(aligned(qweight, 4) && aligned(qzeros, 4) && aligned(packed, 4), QL_ERR_ALIGN,
        "%s: qweight, qzeros and packed must be 4-byte aligned", fn);
  CHECK(aligned(scales, 2) && aligned(scales_out, 2) && aligned(biases_out, 2), QL_ERR_ALIGN,
        "%s: scales, scales_out and biases_out must be 2-byte aligned", fn);
  CHECK(n * k * bits / 32 < (int64_t(1) << 31), QL_ERR_UNSUPPORTED, "%s: weight too large", fn);
  return launched(ql::launch_transcode_gptq(qweight, qzeros, scales, dt(scale_dtype), k, n, bits, group_size,
                                            v1_zeros ? 1 : 0, packed, scales_out, biases_out, (hipStream_t)stream),
                  fn);
}

ql_status qlinear_transcode_gptq_planar(const uint32_t* qweight, const uint32_t* qzeros, const void* scales,
                                        ql_dtype scale_dtype, int64_t k, int64_t n, int bits, int group_size,
                                        uint32_t* packed, void* scales_out, void* biases_out, void* stream) {
  const char* fn = "qlinear_transcode_gptq_planar";
  CHECK(k >= 0 && n >= 0, QL_ERR_SHAPE, "%s: k and n must be >= 0", fn);
  CHECK(bits >= 2 && bits <= 8, QL_ERR_UNSUPPORTED, "%s: bits=%d not supported (GPTQ_P widths 2 to 8)", fn, bits);
  CHECK(group_size == 32 || group_size == 64 || group_size == 128, QL_ERR_UNSUPPORTED,
        "%s: group_size=%d not supported (32, 64 or 128)", fn, group_size);
  CHECK(k % 32 == 0 && k % group_size == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 32 and of group_size", fn,
        (long long)k);
  CHECK(n % 32 == 0, QL_ERR_SHAPE, "%s: n=%lld must be a multiple of 32 (whole planar blocks of zeros)", fn,
        (long long)n);
  CHECK(is16(scale_dtype), QL_ERR_DTYPE, "%s: scale_dtype must be QL_F16 or QL_BF16", fn);
  if (k == 0 || n == 0) return ok();
  CHECK(qweight && qzeros && scales && packed && scales_out && biases_out, QL_ERR_NULL,
        "%s: qweight, qzeros, scales, packed, scales_out and biases_out must not be NULL", fn);
  CHECK(aligned(qweight, 4) && aligned(qzeros, 4) && aligned(packed, 4), QL_ERR_ALIGN,
        "%s: qweight, qzeros and packed must be 4-byte aligned", fn);
  CHECK(aligned(scales, 2) && aligned(scales_out, 2) && aligned(biases_out, 2), QL_ERR_ALIGN,
        "%s: scales, scales_out and biases_out must be 2-byte aligned", fn);
  CHECK(n * k / 32 * 8 < (int64_t(1) << 31), QL_ERR_UNSUPPORTED, "%s: weight too large", fn);
  return launched(ql::launch_transcode_gptq_planar(qweight, qzeros, scales, dt(scale_dtype), k, n, bits, group_size,
                                                   packed, scales_out, biases_out, (hipStream_t)stream),
                  fn);
}

ql_status qlinear_gptq_check_g_idx(const int32_t* g_idx, int64_t k, int group_size) {
  const char* fn = "qlinear_gptq_check_g_idx";
  CHECK(k >= 0, QL_ERR_SHAPE, "%s: k must be >= 0", fn);
  CHECK(group_size > 0, QL_ERR_UNSUPPORTED, "%s: group_size=%d must be > 0", fn, group_size);
  if (k == 0) return ok();
  CHECK(g_idx, QL_ERR_NULL, "%s: g_idx must not be NULL", fn);
  for (int64_t i = 0; i < k; ++i)
    CHECK(g_idx[i] == (int32_t)(i / group_size), QL_ERR_UNSUPPORTED,
          "%s: g_idx[%lld]=%d, not %lld: an activation-order permutation has no exact affine form", fn, (long long)i,
          (int)g_idx[i], (long long)(i / group_size));
  return ok();
}

ql_status qlinear_transcode_awq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales,
                                ql_dtype scale_dtype, int64_t k, int64_t n, int bits, int group_size, uint32_t* packed,
                                void* scales_out, void* biases_out, void* stream) {
  const char* fn = "qlinear_transcode_awq";
  CHECK(k >= 0 && n >= 0, QL_ERR_SHAPE, "%s: k and n must be >= 0", fn);
  CHECK(bits >= 2 && bits <= 8, QL_ERR_UNSUPPORTED, "%s: bits=%d not supported (AWQ GEMM widths 2 to 8)", fn, bits);
  CHECK(group_size == 32 || group_size == 64 || group_size == 128, QL_ERR_UNSUPPORTED,
        "%s: group_size=%d not supported (32, 64 or 128)", fn, group_size);
  CHECK(k % 32 == 0 && k % group_size == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 32 and of group_size", fn,
        (long long)k);
  CHECK(n % 32 == 0, QL_ERR_SHAPE, "%s: n=%lld must be a multiple of 32", fn, (long long)n);
  CHECK(is16(scale_dtype), QL_ERR_DTYPE, "%s: scale_dtype must be QL_F16 or QL_BF16", fn);
  if (k == 0 || n == 0) return ok();
  CHECK(qweight && qzeros && scales && packed && scales_out && biases_out, QL_ERR_NULL,
        "%s: qweight, qzeros, scales, packed, scales_out and biases_out must not be NULL", fn);
  CHECK(aligned(qweight, 4) && aligned(qzeros, 4) && aligned(packed, 4), QL_ERR_ALIGN,
        "%s: qweight, qzeros and packed must be 4-byte aligned", fn);
  CHECK(aligned(scales, 2) && aligned(scales_out, 2) && aligned(biases_out, 2), QL_ERR_ALIGN,
        "%s: scales, scales_out and biases_out must be 2-byte aligned", fn);
  CHECK(n * k / 32 * 8 < (int64_t(1) << 31), QL_ERR_UNSUPPORTED, "%s: weight too large", fn);
  return launched(ql::launch_transcode_awq(qweight, qzeros, scales, dt(scale_dtype), k, n, bits, group_size, packed,
                                           scales_out, biases_out, (hipStream_t)stream),
                  fn);
}

ql_status qlinear_take(const int64_t* pos, int64_t n_pos, const void* src, int64_t src_rows, int64_t row_bytes,
                       void* dst, void* stream) {
  const char* fn = "qlinear_take";
  CHECK(n_pos >= 0 && src_rows >= 0 && row_bytes >= 0, QL_ERR_SHAPE,
        "%s: n_pos, src_rows and row_bytes must be >= 0", fn);
  if (n_pos == 0 || row_bytes == 0) return ok();
  CHECK(pos && dst, QL_ERR_NULL, "%s: pos and dst must not be NULL", fn);
  CHECK(src_rows == 0 || src != nullptr, QL_ERR_NULL, "%s: src must not be NULL", fn);
  CHECK(aligned(pos, 8), QL_ERR_ALIGN, "%s: pos must be 8-byte aligned", fn);
  CHECK(n_pos * ((row_bytes + 32767) / 32768) < (int64_t(1) << 31), QL_ERR_UNSUPPORTED, "%s: output too large", fn);
  return launched(ql::launch_take(pos, n_pos, src, src_rows, row_bytes, dst, (hipStream_t)stream), fn);
}

ql_status qlinear_dequant(ql_format fmt, const void* w0, const void* w1, const void* w2, ql_dtype param_dtype,
                          int64_t rows, int64_t k, int bits, int group_size, void* out, ql_dtype out_dtype,
                          void* stream) {
  const char* fn = "qlinear_dequant";
  CHECK(is_out(out_dtype), QL_ERR_DTYPE, "%s: out_dtype must be QL_F32, QL_F16 or QL_BF16", fn);
  CHECK(rows >= 0 && k >= 0, QL_ERR_SHAPE, "%s: rows and k must be >= 0", fn);
  hipStream_t s = (hipStream_t)stream;
  if (fmt == QL_AFFINE) {
    ql_status st = check_affine(fn, rows, k, bits, group_size, param_dtype);
    if (st != QL_OK) return st;
    if (rows == 0 || k == 0) return ok();
    CHECK(w0 && w1 && w2 && out, QL_ERR_NULL, "%s: packed (w0), scales (w1), biases (w2) and out must not be NULL", fn);
    CHECK(aligned(w0, 16), QL_ERR_ALIGN, "%s: packed (w0) must be 16-byte aligned", fn);
    CHECK(aligned(w1, 2) && aligned(w2, 2), QL_ERR_ALIGN, "%s: scales and biases must be 2-byte aligned", fn);
    CHECK(aligned(out, 16), QL_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
    return launched(ql::launch_dequant_affine((const uint32_t*)w0, w1, w2, dt(param_dtype), rows, k, bits,
                                              group_size, out, dt(out_dtype), s),
                    fn);
  }
  if (fmt == QL_MXFP4_BLOCKS) {
    CHECK(k % 32 == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 32", fn, (long long)k);
    CHECK(w1 == nullptr && w2 == nullptr, QL_ERR_SHAPE, "%s: w1 and w2 must be NULL for MXFP4 blocks", fn);
    if (rows == 0 || k == 0) return ok();
    CHECK(w0 && out, QL_ERR_NULL, "%s: w0 and out must not be NULL", fn);
    CHECK(aligned(out, 16), QL_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
    return launched(ql::launch_dequant_mxfp4_blocks((const uint8_t*)w0, rows, k, out, dt(out_dtype), s), fn);
  }
  if (fmt == QL_Q4_K || fmt == QL_Q6_K) {
    CHECK(k % 256 == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 256", fn, (long long)k);
    CHECK(w1 == nullptr && w2 == nullptr, QL_ERR_SHAPE, "%s: w1 and w2 must be NULL for Q4_K / Q6_K", fn);
    if (rows == 0 || k == 0) return ok();
    CHECK(w0 && out, QL_ERR_NULL, "%s: w0 and out must not be NULL", fn);
    CHECK(aligned(w0, fmt == QL_Q4_K ? 16 : 2), QL_ERR_ALIGN, "%s: Q4_K blocks must be 16-byte aligned, Q6_K 2-byte",
          fn);
    CHECK(aligned(out, 16), QL_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
    CHECK(rows * (k / 256) * 8 < (int64_t(1) << 31), QL_ERR_UNSUPPORTED, "%s: weight too large", fn);
    return launched(ql::launch_dequant_kquant(fmt == QL_Q4_K ? 144 : 210, (const uint8_t*)w0, rows, k, out,
                                              dt(out_dtype), s),
                    fn);
  }
  if (fmt == QL_MXFP4 || fmt == QL_Q8_0) {
    CHECK(k % 32 == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of 32", fn, (long long)k);
    CHECK(w2 == nullptr, QL_ERR_SHAPE, "%s: w2 must be NULL for block formats", fn);
    if (rows == 0 || k == 0) return ok();
    CHECK(w0 && out, QL_ERR_NULL, "%s: w0 and out must not be NULL", fn);
    CHECK(aligned(out, 16), QL_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
    if (fmt == QL_MXFP4) {
      CHECK(w1 != nullptr, QL_ERR_NULL, "%s: MXFP4 scales (w1) must not be NULL", fn);
      CHECK(aligned(w0, 16), QL_ERR_ALIGN, "%s: MXFP4 codes (w0) must be 16-byte aligned", fn);
      return launched(ql::launch_dequant_mxfp4((const uint8_t*)w0, (const uint8_t*)w1, rows, k, out, dt(out_dtype), s),
                      fn);
    }
    CHECK(w1 == nullptr, QL_ERR_SHAPE, "%s: w1 must be NULL for Q8_0", fn);
    CHECK(aligned(w0, 2), QL_ERR_ALIGN, "%s: Q8_0 blocks (w0) must be 2-byte aligned", fn);
    return launched(ql::launch_dequant_q8_0((const uint8_t*)w0, rows, k, out, dt(out_dtype), s), fn);
  }
  return fail(QL_ERR_UNSUPPORTED, "%s: unknown format %d", fn, (int)fmt);
}

ql_status qlinear_gemv(const void* x, ql_dtype x_dtype, int64_t m, int64_t k, const uint32_t* packed,
                       const void* scales, const void* biases, ql_dtype param_dtype, int64_t n, int bits,
                       int group_size, const void* layer_bias, void* y, ql_dtype y_dtype, void* stream) {
  const char* fn = "qlinear_gemv";
  ql_status st = check_product(fn, x, x_dtype, m, k, packed, scales, biases, param_dtype, n, bits, group_size,
                               layer_bias, y, y_dtype);
  if (st != QL_OK) return st;
  if (m == 0 || n == 0) return ok();
  CHECK(n * k * bits / 8 < (int64_t(1) << 31), QL_ERR_UNSUPPORTED, "%s: packed weights of 2 GiB or more", fn);
  for (int64_t m0 = 0; m0 < m; m0 += 8) {
    const int64_t mm = std::min<int64_t>(8, m - m0);
    if (ql::is_stream_bits(bits) && !ql::gemv_mf_eligible(mm, k, bits, group_size, scales, biases)) {
      ql::GemvStreamArgs a{};
      a.x = (const uint8_t*)x + m0 * k * 2;
      a.m = (int)mm;
      a.k = k;
      a.packed = packed;
      a.scales = scales;
      a.biases = biases;
      a.n = n;
      a.g = group_size;
      a.layer_bias = layer_bias;
      a.y = (uint8_t*)y + m0 * n * esize(y_dtype);
      a.ydt = dt(y_dtype);
      a.bits = bits;
      a.xdt = dt(x_dtype);
      a.pdt = dt(param_dtype);
      const hipError_t e = ql::launch_gemv_stream(a, (hipStream_t)stream);
      if (e != hipSuccess) return launched(e, fn);
      continue;
    }
    ql::GemvDesc d{};
    d.x = (const uint8_t*)x + m0 * k * 2;
    d.packed = packed;
    d.scales = scales;
    d.biases = biases;
    d.layer_bias = layer_bias;
    d.y = (uint8_t*)y + m0 * n * esize(y_dtype);
    d.m = mm;
    d.n = n;
    d.k = k;
    d.bits = bits;
    d.group_size = group_size;
    hipError_t e;
    if (ql::gemv_mf_eligible(mm, k, bits, group_size, scales, biases)) {
      const int mt = ql::gemv_mt(mm);
      d.batches = ql::gemv_mf_batches(n, k, bits, group_size, mt, 1024);
      const ql::GemvMfGeom g = ql::gemv_mf_geometry(k, d.batches);
      const int64_t tiles = (n + g.rows_per_wg - 1) / g.rows_per_wg;
      e = ql::launch_gemv_mf(d, nullptr, nullptr, tiles, (int)mm, bits, group_size, dt(x_dtype), dt(param_dtype),
                             dt(y_dtype), ql::gemv_mf_lds(k, mt, group_size, d.batches, bits).bytes, (hipStream_t)stream);
    } else {
      d.batches = ql::gemv_batches(n, k, bits, 1024);
      const ql::GemvGeom g = ql::gemv_geometry(k, bits, d.batches);
      const int64_t tiles = (n + g.rows_per_wg - 1) / g.rows_per_wg;
      const ql::GemvLds lds = ql::gemv_lds(k, bits, ql::gemv_mt(mm), d.batches);
      e = ql::launch_gemv(d, nullptr, nullptr, tiles, (int)mm, bits, dt(x_dtype), dt(param_dtype), dt(y_dtype),
                          lds.bytes, lds.xlds, bits == 4 && group_size == 32, (hipStream_t)stream);
    }
    if (e != hipSuccess) return launched(e, fn);
  }
  return ok();
}

size_t qlinear_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int bits, int group_size) {
  if (m <= 0 || n <= 0 || k <= 0 || group_size <= 0 || bits <= 0) return 0;
  return ql::gemm_workspace_bytes(m, n, k, bits, group_size);
}

ql_status qlinear_gemm(const void* x, ql_dtype x_dtype, int64_t m, int64_t k, const uint32_t* packed,
                       const void* scales, const void* biases, ql_dtype param_dtype, int64_t n, int bits,
                       int group_size, const void* layer_bias, void* y, ql_dtype y_dtype, void* workspace,
                       size_t ws_bytes, void* stream) {
  const char* fn = "qlinear_gemm";
  ql_status st = check_product(fn, x, x_dtype, m, k, packed, scales, biases, param_dtype, n, bits, group_size,
                               layer_bias, y, y_dtype);
  if (st != QL_OK) return st;
  if (m == 0 || n == 0) return ok();
  if (k == 0)  // no codes to read: the GEMV path writes the bias (or zeros)
    return qlinear_gemv(x, x_dtype, m, k, packed, scales, biases, param_dtype, n, bits, group_size, layer_bias, y,
                        y_dtype, stream);
  // the kernel addresses the fp16 copy of x (rows padded to a multiple of 64) and the packed
  // words with 32-bit buffer offsets
  CHECK(m * ((k + 63) / 64 * 64) * 2 < (int64_t(1) << 31) && n * (k * bits / 8) < (int64_t(1) << 31),
        QL_ERR_UNSUPPORTED, "%s: x (%lld x %lld) and the packed words must each be smaller than 2 GiB", fn,
        (long long)m, (long long)k);
  CHECK(!ql::is_stream_bits(bits) || n * k < (int64_t(1) << 31), QL_ERR_UNSUPPORTED,
        "%s: at %d bits the codes as bytes (n * k) must be smaller than 2 GiB", fn, bits);
  const size_t need = qlinear_gemm_workspace_size(m, n, k, bits, group_size);
  CHECK(workspace != nullptr, QL_ERR_WORKSPACE, "%s: workspace must not be NULL (%zu bytes needed)", fn, need);
  CHECK(ws_bytes >= need, QL_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn, ws_bytes,
        need);
  CHECK(aligned(workspace, 16), QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return launched(ql::launch_gemm(x, dt(x_dtype), m, k, packed, scales, biases, dt(param_dtype), n, bits, group_size,
                                  layer_bias, y, dt(y_dtype), workspace, (hipStream_t)stream),
                  fn);
}

size_t qlinear_gemm_grouped_workspace_size(int64_t m, int64_t k, const ql_gemm_weight* weights, int count, int bits,
                                           int group_size) {
  if (m <= 0 || k <= 0 || count <= 0 || count > 4 || weights == nullptr || group_size <= 0 || bits <= 0) return 0;
  ql::GemmWeight w[4];
  for (int j = 0; j < count; ++j)
    w[j] = ql::GemmWeight{weights[j].packed, weights[j].scales, weights[j].biases, weights[j].layer_bias, weights[j].y,
                          weights[j].n < 0 ? 0 : weights[j].n};
  return ql::gemm_grouped_workspace_bytes(m, k, w, count, bits, group_size);
}

ql_status qlinear_gemm_grouped(const void* x, ql_dtype x_dtype, int64_t m, int64_t k, const ql_gemm_weight* weights,
                               int count, ql_dtype param_dtype, int bits, int group_size, ql_dtype y_dtype,
                               void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "qlinear_gemm_grouped";
  CHECK(count >= 0 && count <= 4, QL_ERR_SHAPE, "%s: count=%d must be in [0, 4]", fn, count);
  if (count == 0) return ok();
  CHECK(weights != nullptr, QL_ERR_NULL, "%s: weights must not be NULL", fn);
  ql::GemmWeight w[4];
  bool any = false;
  for (int j = 0; j < count; ++j) {
    const ql_gemm_weight& q = weights[j];
    char name[64];
    snprintf(name, sizeof(name), "%s: weight %d", fn, j);
    ql_status st = check_product(name, x, x_dtype, m, k, q.packed, q.scales, q.biases, param_dtype, q.n, bits,
                                 group_size, q.layer_bias, q.y, y_dtype);
    if (st != QL_OK) return st;
    CHECK(q.n * (k * bits / 8) < (int64_t(1) << 31), QL_ERR_UNSUPPORTED,
          "%s: weight %d's packed words must be smaller than 2 GiB", fn, j);
    CHECK(!ql::is_stream_bits(bits) || q.n * k < (int64_t(1) << 31), QL_ERR_UNSUPPORTED,
          "%s: at %d bits the codes of weight %d as bytes (n * k) must be smaller than 2 GiB", fn, bits, j);
    w[j] = ql::GemmWeight{q.packed, q.scales, q.biases, q.layer_bias, q.y, q.n};
    any = any || q.n > 0;
  }
  if (m == 0 || !any) return ok();
  if (k == 0) {  // no codes: each output is the layer bias (or zeros), as qlinear_gemm writes it
    for (int j = 0; j < count; ++j) {
      const ql_status st = qlinear_gemm(x, x_dtype, m, k, w[j].packed, w[j].scales, w[j].biases, param_dtype, w[j].n,
                                        bits, group_size, w[j].layer_bias, w[j].y, y_dtype, nullptr, 0, stream);
      if (st != QL_OK) return st;
    }
    return ok();
  }
  CHECK(m * ((k + 63) / 64 * 64) * 2 < (int64_t(1) << 31), QL_ERR_UNSUPPORTED,
        "%s: x (%lld x %lld) must be smaller than 2 GiB", fn, (long long)m, (long long)k);
  const size_t need = qlinear_gemm_grouped_workspace_size(m, k, weights, count, bits, group_size);
  CHECK(workspace != nullptr, QL_ERR_WORKSPACE, "%s: workspace must not be NULL (%zu bytes needed)", fn, need);
  CHECK(ws_bytes >= need, QL_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn, ws_bytes,
        need);
  CHECK(aligned(workspace, 16), QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return launched(ql::launch_gemm_grouped(x, dt(x_dtype), m, k, w, count, dt(param_dtype), bits, group_size,
                                          dt(y_dtype), workspace, (hipStream_t)stream),
                  fn);
}

#ifndef GEMV_TILES_BY_SIZE
#define GEMV_TILES_BY_SIZE 1
#endif

namespace {
// Device table of a problem list: descs (ordered by class), then the tiles of every class.
struct BatchedPlan {
  std::vector<ql::GemvDesc> descs;
  std::vector<ql::GemvTile> tiles;
  struct Cls {
    int m, bits, xlds, mf_g;  // mf_g: group size of a matrix-core class, 0 for the vector-ALU kernel
    bool g2;
    bool stream;  // bitstream widths (2, 3, 5, 6 bits)
    size_t first_tile, n_tiles, lds;
  };
  std::vector<Cls> classes;
  // problems at 2, 3, 5 or 6 bits whose k is not a positive multiple of 128: one launch each, by the
  // kernel qlinear_gemv takes for them (they need no table)
  std::vector<int> singles;
  size_t tiles_offset = 0, bytes = 0;
};

void make_plan(const ql_problem* probs, int count, BatchedPlan& plan) {
  std::vector<int> order;
  for (int i = 0; i < count; ++i) {
    if (probs[i].m <= 0 || probs[i].n <= 0) continue;
    if (ql::is_stream_bits(probs[i].bits) && (probs[i].k <= 0 || probs[i].k % 128 != 0))
      plan.singles.push_back(i);
    else
      order.push_back(i);
  }
  auto mf = [&](int i) {
    return ql::gemv_mf_eligible(probs[i].m, probs[i].k, probs[i].bits, probs[i].group_size, probs[i].scales,
                                probs[i].biases);
  };
  auto key = [&](int i) {
    if (mf(i)) return (1 << 16) + ql::gemv_mt(probs[i].m) * 4096 + probs[i].bits * 256 + probs[i].group_size;
    if (ql::is_stream_bits(probs[i].bits)) return (2 << 16) + ql::gemv_mt(probs[i].m) * 4096 + probs[i].bits * 256;
    const bool g2 = probs[i].bits == 4 && probs[i].group_size == 32;
    return ql::gemv_mt(probs[i].m) * 32 + probs[i].bits * 2 + (g2 ? 1 : 0);
  };
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return key(a) < key(b); });
  const int live = (int)order.size();
  plan.descs.resize(live);
  for (int j = 0; j < live;) {
    int e = j;
    while (e < live && key(order[e]) == key(order[j])) ++e;
    BatchedPlan::Cls c;
    c.m = 0;
    c.bits = probs[order[j]].bits;
    c.g2 = c.bits == 4 && probs[order[j]].group_size == 32;
    c.mf_g = mf(order[j]) ? probs[order[j]].group_size : 0;
    c.stream = !c.mf_g && ql::is_stream_bits(c.bits);
    c.first_tile = plan.tiles.size();
    bool fits = true;
    size_t lds_x = 0, lds_lb = 0;
    for (int q = j; q < e; ++q) {
      const ql_problem& p = probs[order[q]];
      ql::GemvDesc& d = plan.descs[q];
      d = ql::GemvDesc{};
      d.x = p.x;
      d.packed = p.packed;
      d.scales = p.scales;
      d.biases = p.biases;
      d.layer_bias = p.layer_bias;
      d.y = p.y;
      d.m = p.m;
      d.n = p.n;
      d.k = p.k;
      d.bits = p.bits;
      d.group_size = p.group_size;
      c.m = std::max<int>(c.m, (int)p.m);
      if (c.stream) {
        const int mt = ql::gemv_mt(p.m);  // the class's row-count template (part of its key)
        d.batches = ql::stream_quad_lg(p.k, mt);
        lds_x = std::max(lds_x, ql::stream_quad_lds(p.k, mt));
        const int64_t rows = ql::stream_quad_tile_rows(p.k, mt);
        const int64_t t = (p.n + rows - 1) / rows;
        for (int64_t i = 0; i < t; ++i) plan.tiles.push_back(ql::GemvTile{q, (int32_t)i});
        continue;
      }
      if (c.mf_g) {
        d.batches = ql::gemv_mf_batches(p.n, p.k, p.bits, p.group_size, ql::gemv_mt(p.m), 1);
        const ql::GemvMfGeom g = ql::gemv_mf_geometry(p.k, d.batches);
        lds_x = std::max(lds_x, ql::gemv_mf_lds(p.k, ql::gemv_mt(p.m), p.group_size, d.batches, p.bits).bytes);
        const int64_t t = (p.n + g.rows_per_wg - 1) / g.rows_per_wg;
        for (int64_t i = 0; i < t; ++i) plan.tiles.push_back(ql::GemvTile{q, (int32_t)i});
        continue;
      }
      d.batches = ql::gemv_batches(p.n, p.k, p.bits, 1);
      const ql::GemvLds need = ql::gemv_lds(p.k, p.bits, ql::gemv_mt(p.m), d.batches);
      const ql::GemvGeom g = ql::gemv_geometry(p.k, p.bits, d.batches);
      if (!need.xlds) fits = false;
      lds_x = std::max(lds_x, need.bytes);
      lds_lb = std::max(lds_lb, (size_t)g.rows_per_wg * 4);
      const int64_t t = (p.n + g.rows_per_wg - 1) / g.rows_per_wg;
      for (int64_t i = 0; i < t; ++i) plan.tiles.push_back(ql::GemvTile{q, (int32_t)i});
    }
    c.n_tiles = plan.tiles.size() - c.first_tile;
    // Largest tiles first: the workgroups that start last, and so end the launch, are short.
    if (GEMV_TILES_BY_SIZE) {
      auto tile_bytes = [&](const ql::GemvTile& t) {
        const ql::GemvDesc& d = plan.descs[t.prob];
        const int64_t rows = c.stream ? ql::stream_quad_tile_rows(d.k, ql::gemv_mt(d.m))
                             : c.mf_g ? ql::gemv_mf_geometry(d.k, d.batches).rows_per_wg
                                      : ql::gemv_geometry(d.k, d.bits, d.batches).rows_per_wg;
        return std::min<int64_t>(rows, d.n - (int64_t)t.local * rows) * (d.k * d.bits / 8);
      };
      std::stable_sort(plan.tiles.begin() + c.first_tile, plan.tiles.end(),
                       [&](const ql::GemvTile& a, const ql::GemvTile& b) { return tile_bytes(a) > tile_bytes(b); });
    }
    c.xlds = fits ? 1 : 0;
    c.lds = (fits || c.mf_g || c.stream) ? lds_x : lds_lb;
    plan.classes.push_back(c);
    j = e;
  }
  plan.tiles_offset = (plan.descs.size() * sizeof(ql::GemvDesc) + 15) & ~(size_t)15;
  plan.bytes = plan.tiles_offset + plan.tiles.size() * sizeof(ql::GemvTile);
}
}  // namespace

size_t qlinear_gemv_batched_workspace_size(const ql_problem* probs, int count) {
  if (count <= 0 || probs == nullptr) return 0;
  BatchedPlan plan;
  make_plan(probs, count, plan);
  return plan.bytes;
}

ql_status qlinear_gemv_batched(const ql_problem* probs, int count, ql_dtype x_dtype, ql_dtype param_dtype,
                               ql_dtype y_dtype, void* workspace, size_t ws_bytes, int upload, void* stream) {
  const char* fn = "qlinear_gemv_batched";
  CHECK(count >= 0, QL_ERR_SHAPE, "%s: count=%d must be >= 0", fn, count);
  if (count == 0) return ok();
  CHECK(probs != nullptr, QL_ERR_NULL, "%s: probs must not be NULL", fn);
  for (int i = 0; i < count; ++i) {
    const ql_problem& p = probs[i];
    char name[64];
    snprintf(name, sizeof(name), "%s: problem %d", fn, i);
    ql_status st = check_product(name, p.x, x_dtype, p.m, p.k, p.packed, p.scales, p.biases, param_dtype, p.n, p.bits,
                                 p.group_size, p.layer_bias, p.y, y_dtype);
    if (st != QL_OK) return st;
    CHECK(p.m <= 8, QL_ERR_UNSUPPORTED, "%s: problem %d has m=%lld > 8 (use qlinear_gemv or qlinear_gemm)", fn, i,
          (long long)p.m);
    CHECK(p.n * p.k * p.bits / 8 < (int64_t(1) << 31), QL_ERR_UNSUPPORTED,
          "%s: problem %d has packed weights of 2 GiB or more", fn, i);
  }
  BatchedPlan plan;
  make_plan(probs, count, plan);
  hipStream_t s = (hipStream_t)stream;
  for (int i : plan.singles) {
    const ql_problem& p = probs[i];
    ql::GemvStreamArgs a{};
    a.x = p.x;
    a.m = (int)p.m;
    a.k = p.k;
    a.packed = p.packed;
    a.scales = p.scales;
    a.biases = p.biases;
    a.n = p.n;
    a.g = p.group_size;
    a.layer_bias = p.layer_bias;
    a.y = p.y;
    a.ydt = dt(y_dtype);
    a.bits = p.bits;
    a.xdt = dt(x_dtype);
    a.pdt = dt(param_dtype);
    const hipError_t e = ql::launch_gemv_stream(a, s);
    if (e != hipSuccess) return launched(e, fn);
  }
  if (plan.descs.empty()) return ok();
  CHECK(workspace != nullptr, QL_ERR_WORKSPACE, "%s: workspace must not be NULL (%zu bytes needed)", fn, plan.bytes);
  CHECK(ws_bytes >= plan.bytes, QL_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
        ws_bytes, plan.bytes);
  CHECK(aligned(workspace, 16), QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  uint8_t* ws = (uint8_t*)workspace;
  if (upload) {
    std::vector<uint8_t> host(plan.bytes);
    memcpy(host.data(), plan.descs.data(), plan.descs.size() * sizeof(ql::GemvDesc));
    memcpy(host.data() + plan.tiles_offset, plan.tiles.data(), plan.tiles.size() * sizeof(ql::GemvTile));
    // through kernel arguments: asynchronous, and the host image may go when the call returns
    const hipError_t e = ql::launch_upload(host.data(), host.size(), ws, s);
    if (e != hipSuccess) return launched(e, fn);
  }
  const ql::GemvDesc* d_descs = (const ql::GemvDesc*)ws;
  const ql::GemvTile* d_tiles = (const ql::GemvTile*)(ws + plan.tiles_offset);
  for (const BatchedPlan::Cls& c : plan.classes) {
    ql::GemvDesc none{};
    hipError_t e =
        c.stream ? ql::launch_gemv_stream_table(d_descs, d_tiles + c.first_tile, (int64_t)c.n_tiles, c.m, c.bits,
                                                dt(x_dtype), dt(param_dtype), dt(y_dtype), c.lds, s)
        : c.mf_g ? ql::launch_gemv_mf(none, d_descs, d_tiles + c.first_tile, (int64_t)c.n_tiles, c.m, c.bits, c.mf_g,
                                      dt(x_dtype), dt(param_dtype), dt(y_dtype), c.lds, s)
               : ql::launch_gemv(none, d_descs, d_tiles + c.first_tile, (int64_t)c.n_tiles, c.m, c.bits,
                                 dt(x_dtype), dt(param_dtype), dt(y_dtype), c.lds, c.xlds, c.g2, s);
    if (e != hipSuccess) return launched(e, fn);
  }
  return ok();
}

ql_status qlinear_route(const int64_t* ids, int64_t n_pos, int64_t e, int32_t* offsets, int32_t* perm,
                        void* stream) {
  const char* fn = "qlinear_route";
  CHECK(n_pos >= 0 && n_pos < (int64_t(1) << 31), QL_ERR_SHAPE, "%s: n_pos=%lld must be in [0, 2^31)", fn,
        (long long)n_pos);
  CHECK(e >= 1 && e <= 4096, QL_ERR_SHAPE, "%s: e=%lld must be in [1, 4096]", fn, (long long)e);
  CHECK(offsets != nullptr, QL_ERR_NULL, "%s: offsets must not be NULL", fn);
  CHECK(n_pos == 0 || (ids && perm), QL_ERR_NULL, "%s: ids and perm must not be NULL", fn);
  CHECK(aligned(ids, 8) && aligned(offsets, 4) && aligned(perm, 4), QL_ERR_ALIGN,
        "%s: ids must be 8-byte and offsets/perm 4-byte aligned", fn);
  return launched(ql::launch_route(ids, n_pos, e, offsets, perm, (hipStream_t)stream), fn);
}

size_t qlinear_apply_experts_workspace_size(int64_t n_pos, int64_t e) {
  if (n_pos < 0 || e < 0) return 0;
  return (size_t)(((e + 1) * 4 + 15) / 16 * 16) + (size_t)((n_pos * 4 + 15) / 16 * 16) +
         (size_t)((e * 4 + 15) / 16 * 16) + (size_t)n_pos * 8;
}

ql_status qlinear_apply_experts(ql_format fmt, const void* w0, const void* w1, int64_t e, int64_t n, int64_t k,
                                const int64_t* ids, int64_t n_pos, const void* x, ql_dtype x_dtype,
                                int64_t pos_per_row, void* y, ql_dtype y_dtype, void* workspace, size_t ws_bytes,
                                void* stream) {
  const char* fn = "qlinear_apply_experts";
  const bool kq = fmt == QL_Q4_K || fmt == QL_Q6_K;
  CHECK(fmt == QL_MXFP4 || fmt == QL_Q8_0 || fmt == QL_MXFP4_BLOCKS || kq, QL_ERR_UNSUPPORTED,
        "%s: format must be QL_MXFP4, QL_MXFP4_BLOCKS, QL_Q8_0, QL_Q4_K or QL_Q6_K", fn);
  CHECK(e >= 0 && e <= 4096, QL_ERR_SHAPE, "%s: e=%lld must be in [0, 4096]", fn, (long long)e);
  CHECK(n >= 0 && k >= 0 && n_pos >= 0 && n_pos < (int64_t(1) << 31), QL_ERR_SHAPE,
        "%s: n, k must be >= 0 and n_pos in [0, 2^31)", fn);
  CHECK(k % (kq ? 256 : 32) == 0, QL_ERR_SHAPE, "%s: k=%lld must be a multiple of %d", fn, (long long)k, kq ? 256 : 32);
  CHECK(pos_per_row >= 1 && n_pos % pos_per_row == 0, QL_ERR_SHAPE,
        "%s: pos_per_row=%lld must be >= 1 and divide n_pos=%lld", fn, (long long)pos_per_row, (long long)n_pos);
  CHECK(x_dtype == QL_BF16 || x_dtype == QL_F16, QL_ERR_DTYPE, "%s: x_dtype must be QL_BF16 or QL_F16", fn);
  CHECK(is_out(y_dtype), QL_ERR_DTYPE, "%s: y_dtype must be QL_F32, QL_F16 or QL_BF16", fn);
  if (n_pos == 0 || n == 0) return ok();
  CHECK(ids && y, QL_ERR_NULL, "%s: ids and y must not be NULL", fn);
  CHECK(aligned(ids, 8), QL_ERR_ALIGN, "%s: ids must be 8-byte aligned", fn);
  CHECK(aligned(y, esize(y_dtype)), QL_ERR_ALIGN, "%s: y must be aligned to its element size", fn);
  hipStream_t s = (hipStream_t)stream;
  if (e == 0) {  // every position is out of range: zeros
    hipError_t err = ql::launch_apply_experts((int)fmt, nullptr, nullptr, 0, n, 0, ids, n_pos, nullptr, 0,
                                              pos_per_row, y, dt(y_dtype), nullptr, nullptr, nullptr, nullptr, s);
    return launched(err, fn);
  }
  CHECK(w0 && x, QL_ERR_NULL, "%s: w0 and x must not be NULL", fn);
  CHECK(aligned(x, 16), QL_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
  if (fmt == QL_MXFP4) {
    CHECK(w1 != nullptr, QL_ERR_NULL, "%s: MXFP4 scales (w1) must not be NULL", fn);
    CHECK(aligned(w0, 16), QL_ERR_ALIGN, "%s: MXFP4 codes (w0) must be 16-byte aligned", fn);
  } else {
    CHECK(w1 == nullptr, QL_ERR_SHAPE, "%s: w1 must be NULL for block formats", fn);
    CHECK(aligned(w0, fmt == QL_Q4_K ? 16 : (fmt == QL_MXFP4_BLOCKS ? 1 : 2)), QL_ERR_ALIGN,
          "%s: blocks (w0) must be 16-byte aligned (Q4_K) or 2-byte aligned (Q8_0, Q6_K)", fn);
  }
  // the kernel addresses x and the expert weights with 32-bit buffer offsets
  const int64_t wbytes = fmt == QL_MXFP4          ? e * n * (k / 2)
                         : fmt == QL_MXFP4_BLOCKS ? e * n * (k / 32) * 17
                         : fmt == QL_Q8_0         ? e * n * (k / 32) * 34
                                                  : e * n * (k / 256) * (fmt == QL_Q4_K ? 144 : 210);
  CHECK((n_pos / pos_per_row) * k * 2 < (int64_t(1) << 31) && wbytes < (int64_t(1) << 31), QL_ERR_UNSUPPORTED,
        "%s: x and the expert weights must each be smaller than 2 GiB", fn);
  const size_t need = qlinear_apply_experts_workspace_size(n_pos, e);
  CHECK(workspace != nullptr, QL_ERR_WORKSPACE, "%s: workspace must not be NULL (%zu bytes needed)", fn, need);
  CHECK(ws_bytes >= need, QL_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn, ws_bytes,
        need);
  CHECK(aligned(workspace, 16), QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  int32_t* offsets = (int32_t*)workspace;
  int32_t* perm = (int32_t*)((uint8_t*)workspace + ((e + 1) * 4 + 15) / 16 * 16);
  int32_t* order = (int32_t*)((uint8_t*)perm + (n_pos * 4 + 15) / 16 * 16);
  float* xfac = (float*)((uint8_t*)order + (e * 4 + 15) / 16 * 16);
  return launched(ql::launch_apply_experts((int)fmt, w0, w1, e, n, k, ids, n_pos, x, dt(x_dtype), pos_per_row, y,
                                           dt(y_dtype), offsets, perm, order, xfac, s),
                  fn);
}

}  // extern "C"

// ---------------------------------------------------------------- routed apply without allocation
// The routing scratch of qlinear_apply_experts_noalloc lives in this file-scope device array: one
// copy per GPU, loaded with the library's code object and held until the process ends.  Host code
// never uses the array's name as an address: the device address of this GPU's copy is queried
// once per device (hipGetSymbolAddress, with that device current) and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[QL_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; null until its first call

ql_status scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launched(e, fn);
  CHECK(dev >= 0 && dev < kMaxDevices, QL_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices supported", fn, dev,
        kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return launched(e, fn);
    CHECK(p != nullptr, QL_ERR_LAUNCH, "%s: no device address for the scratch array on device %d", fn, dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QL_OK;
}
}  // namespace

extern "C" ql_status qlinear_apply_experts_noalloc(ql_format fmt, const void* w0, const void* w1, int64_t e,
                                                   int64_t n, int64_t k, const int64_t* ids, int64_t n_pos,
                                                   const void* x, ql_dtype x_dtype, int64_t pos_per_row, void* y,
                                                   ql_dtype y_dtype, void* stream) {
  const char* fn = "qlinear_apply_experts_noalloc";
  CHECK(e >= 0 && n_pos >= 0, QL_ERR_SHAPE, "%s: e and n_pos must be >= 0", fn);
  const size_t need = qlinear_apply_experts_workspace_size(n_pos, e);
  CHECK(need <= (size_t)QL_NOALLOC_SCRATCH_BYTES, QL_ERR_UNSUPPORTED,
        "%s: n_pos=%lld and e=%lld need %zu bytes of routing scratch, more than the %u bytes of the built-in array "
        "(use qlinear_apply_experts with a workspace)",
        fn, (long long)n_pos, (long long)e, need, (unsigned)QL_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const ql_status st = scratch_for_current_device(fn, &ws);
  if (st != QL_OK) return st;
  // the routing kernel writes every scratch word the apply kernels read, so nothing is cleared
  return qlinear_apply_experts(fmt, w0, w1, e, n, k, ids, n_pos, x, x_dtype, pos_per_row, y, y_dtype, ws,
                               (size_t)QL_NOALLOC_SCRATCH_BYTES, stream);
}
