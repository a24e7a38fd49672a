// Host entry points of libtq: geometry, the host packer/unpacker, argument
// validation and dispatch to the kernel launchers.
//
// Geometry and plane layout: [ninfer-skill] §2 (format parameters), §3
// (row-split geometry and field order), §1 (256-byte plane alignment,
// 128-element K alignment).  Code semantics: [gguf-explainer] §4.3 (PQ2_0
// codes, LSB pair first, value code-1).  PTQ1_0 trit order: this library's
// radix-3 convention, stated in include/tq.h.

#include "../../include/tq.h"
#include "tq_launch.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

namespace {
thread_local std::string g_err;
}  // namespace

namespace tq {
// Record the message of a failing status for tq_last_error (shared with the
// other host sources of the library).
tq_status fail(tq_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
}  // namespace tq

namespace {
using tq::fail;

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

constexpr uint64_t kGroup = 128;
constexpr uint64_t kPlaneAlign = 256;

struct Fmt {
  uint64_t base, high;
  const char *name;
};

bool format_params(int32_t f, Fmt *out) {
  if (f == TQ_PQ2_0_G128) {
    *out = {32, 0, "PQ2_0_G128"};
    return true;
  }
  if (f == TQ_PTQ1_0_G128) {
    *out = {24, 2, "PTQ1_0_G128"};
    return true;
  }
  return false;
}

tq_status geometry(int32_t format, int64_t n, int64_t k, tq_geometry *g) {
  Fmt f;
  if (!format_params(format, &f))
    return fail(TQ_ERR_FORMAT, "unknown numeric format: %d", (int)format);
  if (n < 1 || k < 1)
    return fail(TQ_ERR_SHAPE, "shape must be rank 2 with positive dimensions "
                "(got n=%lld, k=%lld)", (long long)n, (long long)k);
  // every size below must fit 64 bits: the largest, the payload, is under
  // n * (k_pad / 128) * 28 + 512 bytes, so bound that product by 2^62
  {
    const uint64_t groups = ((uint64_t)k + kGroup - 1) / kGroup;
    uint64_t rowb = 0, all = 0;
    if (__builtin_mul_overflow(groups, (uint64_t)(f.base + f.high + 2), &rowb) ||
        __builtin_mul_overflow(rowb, (uint64_t)n, &all) || all > (uint64_t(1) << 62))
      return fail(TQ_ERR_SHAPE, "shape n=%lld, k=%lld is too large: its payload does not fit "
                  "64-bit sizes", (long long)n, (long long)k);
  }
  g->n = (uint64_t)n;
  g->k = (uint64_t)k;
  g->k_pad = align_up(g->k, kGroup);
  g->groups_per_row = g->k_pad / kGroup;
  g->base_bytes_per_group = f.base;
  g->high_bytes_per_group = f.high;
  g->base_row_bytes = g->groups_per_row * f.base;
  g->high_row_bytes = g->groups_per_row * f.high;
  g->scale_row_bytes = g->groups_per_row * 2;
  g->base_offset = 0;
  g->base_bytes = g->n * g->base_row_bytes;
  g->high_offset = align_up(g->base_bytes, kPlaneAlign);
  g->high_bytes = g->n * g->high_row_bytes;
  g->scale_offset = g->high_offset + align_up(g->high_bytes, kPlaneAlign);
  g->scale_bytes = g->n * g->scale_row_bytes;
  g->payload_bytes = g->scale_offset + g->scale_bytes;
  return TQ_OK;
}

tq_status check_payload_size(const tq_geometry &g, uint64_t payload_bytes) {
  if (payload_bytes != g.payload_bytes)
    return fail(TQ_ERR_GEOMETRY, "payload stores %llu bytes; layout requires %llu",
                (unsigned long long)payload_bytes,
                (unsigned long long)g.payload_bytes);
  return TQ_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool dtype_ok(int32_t d) { return d == TQ_F32 || d == TQ_BF16 || d == TQ_F16; }

tq_status device_status(hipError_t e, const char *what) {
  if (e != hipSuccess)
    return fail(TQ_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e,
                hipGetErrorString(e));
  return TQ_OK;
}

// Common validation of a device payload and its shape.
tq_status check_device_payload(const uint8_t *payload, uint64_t payload_bytes,
                               int32_t format, int64_t n, int64_t k,
                               tq_geometry *g, tq::Planes *p) {
  tq_status st = geometry(format, n, k, g);
  if (st != TQ_OK) return st;
  if ((st = check_payload_size(*g, payload_bytes)) != TQ_OK) return st;
  if (!payload) return fail(TQ_ERR_ARG, "payload is NULL");
  if (!aligned(payload, kPlaneAlign))
    return fail(TQ_ERR_ALIGN, "payload must be 256-byte aligned (plane alignment)");
  p->base = payload + g->base_offset;
  p->high = payload + g->high_offset;
  p->scale = reinterpret_cast<const uint16_t *>(payload + g->scale_offset);
  p->n = n;
  p->k = k;
  p->groups = (int64_t)g->groups_per_row;
  p->base_row = (int64_t)g->base_row_bytes;
  p->high_row = (int64_t)g->high_row_bytes;
  p->fmt = format;
  return TQ_OK;
}

// Grouped head order ([ninfer-skill] §5): tiles x groups heads of head_dim
// elements covering the row exactly.
tq_status check_head_order(int64_t k, int32_t tiles, int32_t groups, int32_t head_dim) {
  if (tiles < 1 || groups < 1 || head_dim < 16 || head_dim % 16)
    return fail(TQ_ERR_SHAPE, "head order needs tiles, groups >= 1 and head_dim a positive "
                "multiple of 16 (got %d, %d, %d)", (int)tiles, (int)groups, (int)head_dim);
  if ((int64_t)tiles * groups * head_dim != k)
    return fail(TQ_ERR_SHAPE, "tiles * groups * head_dim = %lld must equal k = %lld",
                (long long)tiles * groups * head_dim, (long long)k);
  return TQ_OK;
}

size_t dtype_size(int32_t d) { return d == TQ_F32 ? 4 : 2; }

tq_status check_signs(const uint16_t *signs) {
  if (!signs) return fail(TQ_ERR_ARG, "signs_bf16 is NULL");
  if (!aligned(signs, 16))
    return fail(TQ_ERR_ALIGN, "signs_bf16 must be 16-byte aligned");
  return TQ_OK;
}

}  // namespace

extern "C" {

const char *tq_last_error(void) { return g_err.c_str(); }

const char *tq_version(void) { return "0.1.0"; }

tq_status tq_geometry_get(int32_t format, int64_t n, int64_t k, tq_geometry *out) {
  if (!out) return fail(TQ_ERR_ARG, "out is NULL");
  tq_geometry g;
  tq_status st = geometry(format, n, k, &g);
  if (st == TQ_OK) *out = g;
  return st;
}

tq_status tq_pack_rowsplit(int32_t format, int64_t n, int64_t k,
                           const int8_t *trits, const uint16_t *scale_bits,
                           uint8_t *payload, uint64_t payload_bytes) {
  tq_geometry g;
  tq_status st = geometry(format, n, k, &g);
  if (st != TQ_OK) return st;
  if ((st = check_payload_size(g, payload_bytes)) != TQ_OK) return st;
  if (!trits || !scale_bits || !payload)
    return fail(TQ_ERR_ARG, "host_trits, host_scale_bits and host_payload must be non-NULL");
  const uint64_t N = g.n, K = g.k, G = g.groups_per_row;
  for (uint64_t i = 0; i < N * K; ++i) {
    int8_t t = trits[i];
    if (t < -1 || t > 1)
      return fail(TQ_ERR_DATA, "trit %d at row %llu column %llu is not in {-1,0,1}",
                  (int)t, (unsigned long long)(i / K), (unsigned long long)(i % K));
  }
  std::memset(payload, 0, payload_bytes);
  uint8_t *base = payload + g.base_offset;
  uint8_t *high = payload + g.high_offset;
  uint8_t *scale = payload + g.scale_offset;
  uint8_t u[kGroup];
  for (uint64_t r = 0; r < N; ++r) {
    const int8_t *row = trits + r * K;
    for (uint64_t gi = 0; gi < G; ++gi) {
      // digits u = trit + 1; columns past k are zero trits (u = 1)
      for (uint64_t j = 0; j < kGroup; ++j) {
        uint64_t col = gi * kGroup + j;
        u[j] = (uint8_t)(col < K ? row[col] + 1 : 1);
      }
      uint8_t *b = base + r * g.base_row_bytes + gi * g.base_bytes_per_group;
      if (format == TQ_PQ2_0_G128) {
        for (int q = 0; q < 32; ++q)
          b[q] = (uint8_t)(u[4 * q] | (u[4 * q + 1] << 2) | (u[4 * q + 2] << 4) |
                           (u[4 * q + 3] << 6));
      } else {
        for (int q = 0; q < 24; ++q) {
          const uint8_t *d = u + 5 * q;
          b[q] = (uint8_t)(d[0] + 3 * (d[1] + 3 * (d[2] + 3 * (d[3] + 3 * d[4]))));
        }
        uint8_t *h = high + r * g.high_row_bytes + gi * g.high_bytes_per_group;
        for (int q = 0; q < 2; ++q) {
          const uint8_t *d = u + 120 + 4 * q;
          h[q] = (uint8_t)(d[0] + 3 * (d[1] + 3 * (d[2] + 3 * d[3])));
        }
      }
      uint16_t s = scale_bits[r * G + gi];
      uint8_t *sp = scale + r * g.scale_row_bytes + 2 * gi;
      sp[0] = (uint8_t)(s & 0xFF);
      sp[1] = (uint8_t)(s >> 8);
    }
  }
  return TQ_OK;
}

tq_status tq_unpack_rowsplit(int32_t format, int64_t n, int64_t k,
                             const uint8_t *payload, uint64_t payload_bytes,
                             int8_t *values, uint16_t *scale_bits,
                             uint64_t *bad_codes) {
  tq_geometry g;
  tq_status st = geometry(format, n, k, &g);
  if (st != TQ_OK) return st;
  if ((st = check_payload_size(g, payload_bytes)) != TQ_OK) return st;
  if (!payload || !values || !scale_bits)
    return fail(TQ_ERR_ARG, "host_payload, host_values and host_scale_bits must be non-NULL");
  const uint64_t N = g.n, G = g.groups_per_row, KP = g.k_pad;
  const uint8_t *base = payload + g.base_offset;
  const uint8_t *high = payload + g.high_offset;
  const uint8_t *scale = payload + g.scale_offset;
  uint64_t bad = 0;
  for (uint64_t r = 0; r < N; ++r) {
    for (uint64_t gi = 0; gi < G; ++gi) {
      int8_t *out = values + r * KP + gi * kGroup;
      const uint8_t *b = base + r * g.base_row_bytes + gi * g.base_bytes_per_group;
      if (format == TQ_PQ2_0_G128) {
        for (int j = 0; j < 128; ++j) {
          int code = (b[j >> 2] >> (2 * (j & 3))) & 3;
          bad += code == 3;
          out[j] = (int8_t)(code - 1);
        }
      } else {
        for (int q = 0; q < 24; ++q) {
          int v = b[q];
          bad += v > 242;
          for (int i = 0; i < 5; ++i, v /= 3) out[5 * q + i] = (int8_t)(v % 3 - 1);
        }
        const uint8_t *h = high + r * g.high_row_bytes + gi * g.high_bytes_per_group;
        for (int q = 0; q < 2; ++q) {
          int v = h[q];
          bad += v > 80;
          for (int i = 0; i < 4; ++i, v /= 3) out[120 + 4 * q + i] = (int8_t)(v % 3 - 1);
        }
      }
      const uint8_t *sp = scale + r * g.scale_row_bytes + 2 * gi;
      scale_bits[r * G + gi] = (uint16_t)(sp[0] | (sp[1] << 8));
    }
  }
  if (bad_codes) *bad_codes = bad;
  return TQ_OK;
}

tq_status tq_hadamard_signed(const void *x, int32_t x_dtype, int64_t rows,
                             int64_t k, int64_t ldx, const uint16_t *signs,
                             int32_t inverse, void *y, int32_t y_dtype,
                             int64_t ldy, void *stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype))
    return fail(TQ_ERR_ARG, "x_dtype/y_dtype must be TQ_F32, TQ_BF16 or TQ_F16");
  if (inverse != 0 && inverse != 1) return fail(TQ_ERR_ARG, "inverse must be 0 or 1");
  if (rows < 0) return fail(TQ_ERR_SHAPE, "rows must be >= 0");
  if (k < 1 || k % 1024)
    return fail(TQ_ERR_SHAPE, "k=%lld: the transform needs a positive multiple of the "
                "1024-element Hadamard block", (long long)k);
  if (ldx < k || ldy < k) return fail(TQ_ERR_ARG, "ldx and ldy must be >= k");
  tq_status st = check_signs(signs);
  if (st != TQ_OK) return st;
  if (rows == 0) return TQ_OK;
  if (!x || !y) return fail(TQ_ERR_ARG, "x and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || ldx % 8 || ldy % 8)
    return fail(TQ_ERR_ALIGN, "x and y must be 16-byte aligned with ldx, ldy multiples of 8");
  if (x == y && (x_dtype != y_dtype || ldx != ldy))
    return fail(TQ_ERR_ARG, "in-place transform needs equal dtypes and leading dimensions");
  return device_status(tq::launch_hadamard(x, x_dtype, rows, k, ldx, signs, inverse,
                                           y, y_dtype, ldy, (hipStream_t)stream),
                       "tq_hadamard_signed");
}

tq_status tq_hadamard_signed_grouped(const void *x, int32_t x_dtype, int64_t rows, int64_t k,
                                     int64_t ldx, int32_t tiles, int32_t groups,
                                     int32_t head_dim, const uint16_t *signs, void *y,
                                     int32_t y_dtype, int64_t ldy, void *stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype))
    return fail(TQ_ERR_ARG, "x_dtype/y_dtype must be TQ_F32, TQ_BF16 or TQ_F16");
  if (rows < 0) return fail(TQ_ERR_SHAPE, "rows must be >= 0");
  if (k < 1 || k % 1024)
    return fail(TQ_ERR_SHAPE, "k=%lld: the transform needs a positive multiple of the "
                "1024-element Hadamard block", (long long)k);
  tq_status st = check_head_order(k, tiles, groups, head_dim);
  if (st != TQ_OK) return st;
  if (ldx < k || ldy < k) return fail(TQ_ERR_ARG, "ldx and ldy must be >= k");
  if ((st = check_signs(signs)) != TQ_OK) return st;
  if (rows == 0) return TQ_OK;
  if (!x || !y) return fail(TQ_ERR_ARG, "x and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || ldx % 8 || ldy % 8)
    return fail(TQ_ERR_ALIGN, "x and y must be 16-byte aligned with ldx, ldy multiples of 8");
  const char *xb = static_cast<const char *>(x), *yb = static_cast<const char *>(y);
  const int64_t xe = ((rows - 1) * ldx + k) * (int64_t)dtype_size(x_dtype);
  const int64_t ye = ((rows - 1) * ldy + k) * (int64_t)dtype_size(y_dtype);
  if (xb < yb + ye && yb < xb + xe)
    return fail(TQ_ERR_ARG, "x and y overlap (the head gather cannot run in place)");
  return device_status(tq::launch_hadamard(x, x_dtype, rows, k, ldx, signs, 0, y, y_dtype, ldy,
                                           (hipStream_t)stream, tiles, groups, head_dim),
                       "tq_hadamard_signed_grouped");
}

tq_status tq_gemv_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                           int32_t format, int64_t n, int64_t k, const void *xrot,
                           int32_t x_dtype, int64_t batch, int64_t ldx, float *y,
                           int64_t ldy, void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, &g, &p);
  if (st != TQ_OK) return st;
  if (k % 128)
    return fail(TQ_ERR_SHAPE, "k=%lld: device projections need k %% 128 == 0", (long long)k);
  if (batch < 1 || batch > 8) return fail(TQ_ERR_SHAPE, "batch=%lld must be in 1..8", (long long)batch);
  if (k > tq::gemv_max_k(format))
    return fail(TQ_ERR_SHAPE, "k=%lld exceeds the GEMV limit %lld for this format", (long long)k,
                (long long)tq::gemv_max_k(format));
  if (!dtype_ok(x_dtype)) return fail(TQ_ERR_ARG, "x_dtype must be TQ_F32, TQ_BF16 or TQ_F16");
  if (!xrot || !y) return fail(TQ_ERR_ARG, "xrot and y must be non-NULL");
  if (ldx < k || ldy < n) return fail(TQ_ERR_ARG, "ldx must be >= k and ldy >= n");
  if (!aligned(xrot, 16) || ldx % 8)
    return fail(TQ_ERR_ALIGN, "xrot must be 16-byte aligned with ldx a multiple of 8");
  if (!aligned(y, 4)) return fail(TQ_ERR_ALIGN, "y must be 4-byte aligned");
  return device_status(tq::launch_gemv(p, xrot, x_dtype, batch, ldx, y, ldy,
                                       (hipStream_t)stream),
                       "tq_gemv_rowsplit");
}

tq_status tq_rotated_gemv_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                                   int32_t format, int64_t n, int64_t k, const void *x,
                                   int32_t x_dtype, int64_t batch, int64_t ldx,
                                   const uint16_t *signs_bf16, float *y, int64_t ldy,
                                   void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, &g, &p);
  if (st != TQ_OK) return st;
  if (k % 1024)
    return fail(TQ_ERR_SHAPE, "k=%lld: the transform needs a multiple of the 1024-element block",
                (long long)k);
  if (batch < 1 || batch > 8) return fail(TQ_ERR_SHAPE, "batch=%lld must be in 1..8", (long long)batch);
  if (!dtype_ok(x_dtype)) return fail(TQ_ERR_ARG, "x_dtype must be TQ_F32, TQ_BF16 or TQ_F16");
  if (!x || !y) return fail(TQ_ERR_ARG, "x and y must be non-NULL");
  st = check_signs(signs_bf16);
  if (st != TQ_OK) return st;
  if (ldx < k || ldy < n) return fail(TQ_ERR_ARG, "ldx must be >= k and ldy >= n");
  if (!aligned(x, 16) || ldx % 8)
    return fail(TQ_ERR_ALIGN, "x must be 16-byte aligned with ldx a multiple of 8");
  if (!aligned(y, 4)) return fail(TQ_ERR_ALIGN, "y must be 4-byte aligned");
  if (!tq::rotated_gemv_fused(p, batch))
    return fail(TQ_ERR_UNSUPPORTED,
                "the fused transform + GEMV covers PQ2_0_G128, batch 1, k <= 11264; "
                "use tq_hadamard_signed then tq_gemv_rowsplit");
  return device_status(tq::launch_rotated_gemv(p, x, x_dtype, signs_bf16, y,
                                               (hipStream_t)stream),
                       "tq_rotated_gemv_rowsplit");
}

tq_status tq_rotated_gemv_rowsplit_grouped(const uint8_t *payload, uint64_t payload_bytes,
                                           int32_t format, int64_t n, int64_t k, const void *x,
                                           int32_t x_dtype, int64_t batch, int64_t ldx,
                                           int32_t tiles, int32_t groups, int32_t head_dim,
                                           const uint16_t *signs_bf16, float *y, int64_t ldy,
                                           void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, &g, &p);
  if (st != TQ_OK) return st;
  if (k % 1024)
    return fail(TQ_ERR_SHAPE, "k=%lld: the transform needs a multiple of the 1024-element block",
                (long long)k);
  if ((st = check_head_order(k, tiles, groups, head_dim)) != TQ_OK) return st;
  if (batch < 1 || batch > 8) return fail(TQ_ERR_SHAPE, "batch=%lld must be in 1..8", (long long)batch);
  if (!dtype_ok(x_dtype)) return fail(TQ_ERR_ARG, "x_dtype must be TQ_F32, TQ_BF16 or TQ_F16");
  if (!x || !y) return fail(TQ_ERR_ARG, "x and y must be non-NULL");
  if ((st = check_signs(signs_bf16)) != TQ_OK) return st;
  if (ldx < k || ldy < n) return fail(TQ_ERR_ARG, "ldx must be >= k and ldy >= n");
  if (!aligned(x, 16) || ldx % 8)
    return fail(TQ_ERR_ALIGN, "x must be 16-byte aligned with ldx a multiple of 8");
  if (!aligned(y, 4)) return fail(TQ_ERR_ALIGN, "y must be 4-byte aligned");
  if (!tq::rotated_gemv_fused(p, batch))
    return fail(TQ_ERR_UNSUPPORTED,
                "the fused transform + GEMV covers PQ2_0_G128, batch 1, k <= 11264; "
                "use tq_hadamard_signed_grouped then tq_gemv_rowsplit");
  return device_status(tq::launch_rotated_gemv(p, x, x_dtype, signs_bf16, y, (hipStream_t)stream,
                                               tiles, groups, head_dim),
                       "tq_rotated_gemv_rowsplit_grouped");
}

tq_status tq_gemm_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                           int32_t format, int64_t n, int64_t k, const void *x,
                           int32_t x_dtype, int64_t m, int64_t ldx, void *y,
                           int32_t y_dtype, int64_t ldy, void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, &g, &p);
  if (st != TQ_OK) return st;
  if (k % 128)
    return fail(TQ_ERR_SHAPE, "k=%lld: device projections need k %% 128 == 0", (long long)k);
  if (k > (int64_t(1) << 20))
    return fail(TQ_ERR_SHAPE, "k=%lld exceeds the GEMM's limit of 2^20", (long long)k);
  if (m < 0) return fail(TQ_ERR_SHAPE, "m must be >= 0");
  if (x_dtype != TQ_F16 && x_dtype != TQ_BF16)
    return fail(TQ_ERR_ARG, "x_dtype must be TQ_F16 or TQ_BF16");
  if (y_dtype != TQ_F32 && y_dtype != TQ_BF16)
    return fail(TQ_ERR_ARG, "y_dtype must be TQ_F32 or TQ_BF16");
  if (m == 0) return TQ_OK;
  if (!x || !y) return fail(TQ_ERR_ARG, "x and y must be non-NULL");
  if (ldx < k || ldy < n) return fail(TQ_ERR_ARG, "ldx must be >= k and ldy >= n");
  // 256 rows of X are addressed with 32-bit byte offsets
  if (ldx >= (int64_t(1) << 22)) return fail(TQ_ERR_ARG, "ldx must be < 2^22");
  if (!aligned(x, 16) || ldx % 8)
    return fail(TQ_ERR_ALIGN, "x must be 16-byte aligned with ldx a multiple of 8");
  if (!aligned(y, 4)) return fail(TQ_ERR_ALIGN, "y must be 4-byte aligned");
  return device_status(tq::launch_gemm(p, static_cast<const uint16_t *>(x), x_dtype, m, ldx, y,
                                       y_dtype, ldy, (hipStream_t)stream),
                       "tq_gemm_rowsplit");
}

tq_status tq_embed_rows_inverse(const uint8_t *payload, uint64_t payload_bytes,
                                int32_t format, int64_t n, int64_t k,
                                const int32_t *ids, int64_t count,
                                const uint16_t *signs, float *out, int64_t ldo,
                                int32_t *err_word, void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, &g, &p);
  if (st != TQ_OK) return st;
  if (k % 1024)
    return fail(TQ_ERR_SHAPE, "k=%lld: the inverse transform needs a multiple of the "
                "1024-element Hadamard block", (long long)k);
  if (count < 0) return fail(TQ_ERR_SHAPE, "count must be >= 0");
  if ((st = check_signs(signs)) != TQ_OK) return st;
  if (count == 0) return TQ_OK;
  if (!ids || !out) return fail(TQ_ERR_ARG, "ids and out must be non-NULL");
  if (ldo < k) return fail(TQ_ERR_ARG, "ldo must be >= k");
  if (!aligned(out, 16) || ldo % 4)
    return fail(TQ_ERR_ALIGN, "out must be 16-byte aligned with ldo a multiple of 4");
  return device_status(tq::launch_embed(p, ids, count, signs, out, ldo, err_word,
                                        (hipStream_t)stream),
                       "tq_embed_rows_inverse");
}

tq_status tq_decode_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                             int32_t format, int64_t n, int64_t k,
                             const int32_t *rows, int64_t count, int8_t *values,
                             uint16_t *scale_bits, void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, &g, &p);
  if (st != TQ_OK) return st;
  if (count < 0) return fail(TQ_ERR_SHAPE, "count must be >= 0");
  if (count == 0) return TQ_OK;
  if (!rows || !values || !scale_bits)
    return fail(TQ_ERR_ARG, "rows, values and scale_bits must be non-NULL");
  return device_status(tq::launch_decode(p, rows, count, values, scale_bits,
                                         (int64_t)g.k_pad, (hipStream_t)stream),
                       "tq_decode_rowsplit");
}

// Block stream <-> planes: shared validation, then one launch.
static tq_status transcode(const uint8_t *src, uint8_t *dst, bool to_planes, uint64_t payload_bytes,
                           uint64_t blocks_bytes, int32_t format, int64_t n, int64_t k,
                           void *stream, const char *what) {
  tq_geometry g;
  tq_status st = geometry(format, n, k, &g);
  if (st != TQ_OK) return st;
  if ((st = check_payload_size(g, payload_bytes)) != TQ_OK) return st;
  const uint64_t blk = format == TQ_PQ2_0_G128 ? 34 : 28;
  const uint64_t need = g.n * g.groups_per_row * blk;
  if (blocks_bytes != need)
    return fail(TQ_ERR_GEOMETRY, "block stream stores %llu bytes; layout requires %llu",
                (unsigned long long)blocks_bytes, (unsigned long long)need);
  if (!src || !dst) return fail(TQ_ERR_ARG, "blocks and payload must be non-NULL");
  const uint8_t *payload = to_planes ? dst : src;
  const uint8_t *blocks = to_planes ? src : dst;
  if (!aligned(payload, kPlaneAlign))
    return fail(TQ_ERR_ALIGN, "payload must be 256-byte aligned (plane alignment)");
  if (!aligned(blocks, 8)) return fail(TQ_ERR_ALIGN, "blocks must be 8-byte aligned");
  if (payload < blocks + blocks_bytes && blocks < payload + payload_bytes)
    return fail(TQ_ERR_ARG, "blocks and payload overlap");
  return device_status(tq::launch_transcode(format, to_planes, src, dst, g.base_bytes,
                                            g.high_offset, g.high_bytes, g.scale_offset,
                                            g.scale_bytes, g.payload_bytes, need,
                                            (hipStream_t)stream),
                       what);
}

tq_status tq_blocks_to_planes(const uint8_t *blocks, uint64_t blocks_bytes, int32_t format,
                              int64_t n, int64_t k, uint8_t *payload, uint64_t payload_bytes,
                              void *stream) {
  return transcode(blocks, payload, true, payload_bytes, blocks_bytes, format, n, k, stream,
                   "tq_blocks_to_planes");
}

tq_status tq_planes_to_blocks(const uint8_t *payload, uint64_t payload_bytes, int32_t format,
                              int64_t n, int64_t k, uint8_t *blocks, uint64_t blocks_bytes,
                              void *stream) {
  return transcode(payload, blocks, false, payload_bytes, blocks_bytes, format, n, k, stream,
                   "tq_planes_to_blocks");
}

}  // extern "C"

namespace {

// Validation shared by the two entry points of the one-launch head.
tq_status check_head(const uint8_t *payload, uint64_t payload_bytes, int32_t format, int64_t n,
                     int64_t k, const void *x, int32_t x_dtype, const uint16_t *norm_bf16,
                     float eps, const uint16_t *signs_bf16, const float *logits,
                     const int32_t *token, tq_geometry *g, tq::Planes *p) {
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, g, p);
  if (st != TQ_OK) return st;
  if (k % 1024) return fail(TQ_ERR_SHAPE, "k=%lld: the head step needs k %% 1024 == 0", (long long)k);
  if (n >= (int64_t(1) << 30)) return fail(TQ_ERR_SHAPE, "n=%lld must be below 2^30", (long long)n);
  if (!dtype_ok(x_dtype)) return fail(TQ_ERR_ARG, "x_dtype must be TQ_F32, TQ_BF16 or TQ_F16");
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(TQ_ERR_ARG, "eps must be finite and >= 0");
  if (!x || !norm_bf16 || !token) return fail(TQ_ERR_ARG, "x, norm_bf16 and token must be non-NULL");
  if ((st = check_signs(signs_bf16)) != TQ_OK) return st;
  if (!aligned(x, 16) || !aligned(norm_bf16, 16))
    return fail(TQ_ERR_ALIGN, "x and norm_bf16 must be 16-byte aligned");
  if (!aligned(token, 4) || (logits && !aligned(logits, 4)))
    return fail(TQ_ERR_ALIGN, "token and logits must be 4-byte aligned");
  if (format != TQ_PQ2_0_G128 || k > 11 * 1024)
    return fail(TQ_ERR_UNSUPPORTED, "the one-launch head covers PQ2_0_G128 with k <= 11264; "
                "use tq_hadamard_signed then tq_gemv_rowsplit");
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_head_argmax(const uint8_t *payload, uint64_t payload_bytes, int32_t format,
                         int64_t n, int64_t k, const void *x, int32_t x_dtype,
                         const uint16_t *norm_bf16, float eps, const uint16_t *signs_bf16,
                         float *logits, uint64_t *work, int32_t *token, void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_head(payload, payload_bytes, format, n, k, x, x_dtype, norm_bf16, eps,
                            signs_bf16, logits, token, &g, &p);
  if (st != TQ_OK) return st;
  if (!work) return fail(TQ_ERR_ARG, "work must be non-NULL");
  if (!aligned(work, 16)) return fail(TQ_ERR_ALIGN, "work must be 16-byte aligned");
  return device_status(tq::launch_head_argmax(p, x, x_dtype, norm_bf16, eps, signs_bf16, logits,
                                              reinterpret_cast<unsigned long long *>(work), token,
                                              (hipStream_t)stream),
                       "tq_head_argmax");
}

tq_status tq_head_argmax_noalloc(const uint8_t *payload, uint64_t payload_bytes, int32_t format,
                                 int64_t n, int64_t k, const void *x, int32_t x_dtype,
                                 const uint16_t *norm_bf16, float eps, const uint16_t *signs_bf16,
                                 float *logits, int32_t *token, void *stream) {
  tq_geometry g;
  tq::Planes p;
  // every request the one-launch head covers (n < 2^30, k <= 11264) needs
  // the same two work words, so check_head's limits are the scratch's too
  tq_status st = check_head(payload, payload_bytes, format, n, k, x, x_dtype, norm_bf16, eps,
                            signs_bf16, logits, token, &g, &p);
  if (st != TQ_OK) return st;
  unsigned long long *work = nullptr;
  if ((st = device_status(tq::head_scratch(&work), "tq_head_argmax_noalloc: scratch address")) != TQ_OK)
    return st;
  return device_status(tq::launch_head_argmax(p, x, x_dtype, norm_bf16, eps, signs_bf16, logits,
                                              work, token, (hipStream_t)stream),
                       "tq_head_argmax_noalloc");
}

// 2-bit G64 block stream ([tensorsharp] §4.1 expansion; block rule of
// [gguf-explainer] §4.3): n rows of k_pad/64 blocks of 18 bytes.
static uint64_t g64_bytes(const tq_geometry &g) { return g.n * (g.k_pad / 64) * 18; }

tq_status tq_g64_bytes(int64_t n, int64_t k, uint64_t *bytes) {
  if (!bytes) return fail(TQ_ERR_ARG, "bytes is NULL");
  tq_geometry g;
  tq_status st = geometry(TQ_PQ2_0_G128, n, k, &g);
  if (st != TQ_OK) return st;
  *bytes = g64_bytes(g);
  return TQ_OK;
}

tq_status tq_expand_g64(const uint8_t *payload, uint64_t payload_bytes, int32_t format,
                        int64_t n, int64_t k, uint8_t *blocks, uint64_t blocks_bytes,
                        void *stream) {
  tq_geometry g;
  tq::Planes p;
  tq_status st = check_device_payload(payload, payload_bytes, format, n, k, &g, &p);
  if (st != TQ_OK) return st;
  const uint64_t need = g64_bytes(g);
  if (blocks_bytes != need)
    return fail(TQ_ERR_GEOMETRY, "block stream stores %llu bytes; layout requires %llu",
                (unsigned long long)blocks_bytes, (unsigned long long)need);
  if (!blocks) return fail(TQ_ERR_ARG, "blocks is NULL");
  if (!aligned(blocks, 16)) return fail(TQ_ERR_ALIGN, "blocks must be 16-byte aligned");
  if (payload < blocks + blocks_bytes && blocks < payload + payload_bytes)
    return fail(TQ_ERR_ARG, "blocks and payload overlap");
  return device_status(tq::launch_expand_g64(format, p.base, p.high, p.scale, blocks,
                                             (int64_t)(g.n * g.groups_per_row),
                                             (hipStream_t)stream),
                       "tq_expand_g64");
}

tq_status tq_gemv_g64(const uint8_t *blocks, uint64_t blocks_bytes, int64_t n, int64_t k,
                      const void *xrot, int32_t x_dtype, int64_t batch, int64_t ldx, float *y,
                      int64_t ldy, void *stream) {
  tq_geometry g;
  tq_status st = geometry(TQ_PQ2_0_G128, n, k, &g);
  if (st != TQ_OK) return st;
  const uint64_t need = g64_bytes(g);
  if (blocks_bytes != need)
    return fail(TQ_ERR_GEOMETRY, "block stream stores %llu bytes; layout requires %llu",
                (unsigned long long)blocks_bytes, (unsigned long long)need);
  if (k % 1024 || k > 17 * 1024)
    return fail(TQ_ERR_SHAPE, "k=%lld: the G64 GEMV needs k %% 1024 == 0 and k <= 17408",
                (long long)k);
  if (n >= (int64_t(1) << 30)) return fail(TQ_ERR_SHAPE, "n=%lld must be below 2^30", (long long)n);
  if (batch < 1) return fail(TQ_ERR_SHAPE, "batch=%lld must be >= 1", (long long)batch);
  if (!dtype_ok(x_dtype)) return fail(TQ_ERR_ARG, "x_dtype must be TQ_F32, TQ_BF16 or TQ_F16");
  if (!blocks || !xrot || !y) return fail(TQ_ERR_ARG, "blocks, xrot and y must be non-NULL");
  if (ldx < k || ldy < n) return fail(TQ_ERR_ARG, "ldx must be >= k and ldy >= n");
  if (!aligned(blocks, 16)) return fail(TQ_ERR_ALIGN, "blocks must be 16-byte aligned");
  if (!aligned(xrot, 16) || ldx % 8)
    return fail(TQ_ERR_ALIGN, "xrot must be 16-byte aligned with ldx a multiple of 8");
  if (!aligned(y, 4)) return fail(TQ_ERR_ALIGN, "y must be 4-byte aligned");
  if (batch != 1)
    return fail(TQ_ERR_UNSUPPORTED, "the G64 GEMV covers batch 1 only (got %lld)", (long long)batch);
  return device_status(tq::launch_gemv_g64(blocks, n, k, xrot, x_dtype, y, (hipStream_t)stream),
                       "tq_gemv_g64");
}

tq_status tq_stream_read(const void *src, uint64_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink) return fail(TQ_ERR_ARG, "src and sink must be non-NULL");
  if (bytes < 16 || bytes % 16 || bytes > (uint64_t(1) << 40))
    return fail(TQ_ERR_SHAPE, "bytes=%llu must be a positive multiple of 16 below 2^40",
                (unsigned long long)bytes);
  if (!aligned(src, 16) || !aligned(sink, 4))
    return fail(TQ_ERR_ALIGN, "src must be 16-byte and sink 4-byte aligned");
  return device_status(tq::launch_stream_read(src, bytes, sink, (hipStream_t)stream),
                       "tq_stream_read");
}

}  // extern "C"
