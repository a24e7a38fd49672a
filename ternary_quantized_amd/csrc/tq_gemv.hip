// Decode GEMV over row-split ternary planes:
//   y[b][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * x'[b][j]
// [gguf-explainer] §4.3 (code semantics) and §4.4 (the dot product with an
// offset code: d * sum (q-1) x = d * (sum q x - sum x), where sum x does not
// depend on the weights and is computed once); [ninfer-skill] §3 (planes).
//
// Design (gfx950, wave64):
//  * Every thread owns one fixed K-chunk of the row ("lane chunk") and keeps
//    the matching activations in registers as binary16 pairs, so weights are
//    the only data streamed from HBM; a team of ceil(C/16)*16 threads covers
//    the C chunks of one row and a workgroup holds R teams.
//  * Codes are unpacked with the fp4 (E2M1) converter: masking the 2-bit
//    codes into the low half of each nibble turns a nibble into the fp4
//    number code/2, so v_cvt_scalef32_pk_f16_fp4 with scale 2 yields the
//    codes 0..3 as exact binary16 pairs, consumed by v_dot2_f32_f16 with fp32
//    accumulation.  The offset -1 is applied once per chunk as
//    s * (sum code*x - sum x).
//  * PTQ1_0 bytes (five radix-3 digits) go through 256-entry LDS tables whose
//    entries hold the digits as fp4 nibbles laid out for the same converter.
//  * Partial sums are reduced across 16-lane segments with lane shuffles and
//    across segments through LDS in a fixed order (no atomics: bitwise
//    reproducible).

#include "tq_device.h"
#include "tq_launch.h"

#include <type_traits>

namespace tq {

__device__ __forceinline__ half2_t cvt_codes(uint32_t v, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 3);
  }
}

__device__ __forceinline__ half2_t bits_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// The first products of the five code classes, a[c] = t[c].lo*x[c].lo +
// t[c].hi*x[c].hi, each from a zero accumulator.  They are taken in the
// three-operand form: the compiler only emits the two-operand form, whose
// accumulator is tied to the destination and would need five registers
// cleared first.  A dot product's result may be read by a different vector
// instruction only three wait states later, which the compiler cannot see
// through the asm, so the block ends with those wait states itself.
__device__ __forceinline__ void dot2_first5(const uint32_t (&t)[8], const half2_t *x, float (&a)[5]) {
  asm("v_dot2_f32_f16 %0, %5, %10, 0\n\t"
      "v_dot2_f32_f16 %1, %6, %11, 0\n\t"
      "v_dot2_f32_f16 %2, %7, %12, 0\n\t"
      "v_dot2_f32_f16 %3, %8, %13, 0\n\t"
      "v_dot2_f32_f16 %4, %9, %14, 0\n\t"
      "s_nop 2"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4])
      : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "v"(t[4]),
        "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]));
}

// The same for four classes: a[c] = t[c].lo*x[c].lo + t[c].hi*x[c].hi.
__device__ __forceinline__ void dot2_first4(const uint32_t (&t)[8], const half2_t *x, float (&a)[4]) {
  asm("v_dot2_f32_f16 %0, %4, %8, 0\n\t"
      "v_dot2_f32_f16 %1, %5, %9, 0\n\t"
      "v_dot2_f32_f16 %2, %6, %10, 0\n\t"
      "v_dot2_f32_f16 %3, %7, %11, 0\n\t"
      "s_nop 2"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]),
        "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
}

// cache policy of a streaming (read-once) buffer load
constexpr int CPOL_NT = 2;

__device__ __forceinline__ half2_t pack_h2(float a, float b) {
  half2_t r;
  r.x = (_Float16)a;
  r.y = (_Float16)b;
  return r;
}

template <int XD>
__device__ __forceinline__ float xload(const void *x, int64_t i) {
  return load_elem<XD>(x, i);
}

// Raw activation words of one lane chunk, as loaded (no conversion yet).
template <int FMT, int CW, int XD>
struct XRaw {
  // PQ2_0: CW contiguous elements; PTQ1_0: 32 gathered elements.
  static constexpr int n = FMT == FMT_PQ2 ? (XD == DT_F32 ? CW : CW / 2) : 32;
  uint32_t w[n];
};

template <int FMT, int CW, int XD>
__device__ __forceinline__ void load_x_raw(const void *x, int64_t xrow, int64_t c,
                                           XRaw<FMT, CW, XD> &r) {
  if constexpr (FMT == FMT_PQ2) {
    // CW contiguous elements starting at a multiple of 16: 16-byte loads
    const u32x4 *q;
    if constexpr (XD == DT_F32)
      q = reinterpret_cast<const u32x4 *>(static_cast<const float *>(x) + xrow + c * CW);
    else
      q = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(x) + xrow + c * CW);
#pragma unroll
    for (int i = 0; i < XRaw<FMT, CW, XD>::n / 4; ++i) {
      const u32x4 v = q[i];
      r.w[4 * i] = v[0]; r.w[4 * i + 1] = v[1]; r.w[4 * i + 2] = v[2]; r.w[4 * i + 3] = v[3];
    }
  } else {
    // chunk c = 4*g + q: trits 30q..30q+29 and 120+2q, 121+2q of group g
    const int64_t g = c >> 2;
    const int q = (int)(c & 3);
    const int64_t gk = xrow + g * 128;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int64_t e = i < 30 ? gk + 30 * q + i : gk + 120 + 2 * q + (i - 30);
      if constexpr (XD == DT_F32) r.w[i] = __float_as_uint(static_cast<const float *>(x)[e]);
      else r.w[i] = static_cast<const uint16_t *>(x)[e];
    }
  }
}

template <int XD>
__device__ __forceinline__ float x_elem(uint32_t w, int half) {
  if constexpr (XD == DT_F32) return __uint_as_float(w);
  const uint16_t b = (uint16_t)(half ? (w >> 16) : (w & 0xFFFF));
  if constexpr (XD == DT_BF16) return bf16_to_f32(b);
  else return f16_to_f32(b);
}

// Activation pairs of one lane chunk in the order the decoder produces
// weight pairs, and their fp32 sum (of the binary16-rounded values).
template <int FMT, int CW, int XD>
__device__ __forceinline__ float convert_x_chunk(const XRaw<FMT, CW, XD> &r, int64_t c,
                                                 half2_t xp[CW / 2]) {
  float v[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    if constexpr (FMT == FMT_PQ2 && XD != DT_F32) v[i] = x_elem<XD>(r.w[i >> 1], i & 1);
    else v[i] = x_elem<XD>(r.w[i], 0);
    v[i] = (float)(_Float16)v[i];
  }
  if constexpr (FMT == FMT_PQ2) {
    // dword d covers weights 16d..16d+15; pair e holds weights (e, e+8).
#pragma unroll
    for (int d = 0; d < CW / 16; ++d) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xp[8 * d + e] = pack_h2(v[16 * d + e], v[16 * d + e + 8]);
    }
  } else {
    // byte pair pp covers trits 10pp..10pp+4 (first byte) and 10pp+5..10pp+9
    // (second); digit i of both bytes forms pair 5pp+i
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
#pragma unroll
      for (int i = 0; i < 5; ++i) xp[5 * pp + i] = pack_h2(v[10 * pp + i], v[10 * pp + 5 + i]);
    xp[15] = pack_h2(v[30], v[31]);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < CW; ++i) s += v[i];
  return s;
}

// Raw plane bytes of one lane chunk of one row.
template <int FMT, int CW>
struct Raw {
  uint32_t w[FMT == FMT_PQ2 ? CW / 16 : 2];
  uint32_t h;      // PTQ1_0: the high byte this lane needs
  uint32_t s;      // scale bits (kept in a full register: a 16-bit field
                   // would make every scale load a serialising round trip)
};

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

// Plane pointers of one lane chunk in row 0 (advance by the row strides).
template <int FMT, int CW>
struct ChunkPtr {
  const uint8_t *base;    // base bytes of the chunk (PTQ1_0: 4-byte aligned window)
  const uint8_t *high;    // PTQ1_0: the group's high bytes
  const uint16_t *scale;  // the chunk's group scale
};

template <int FMT, int CW>
__device__ __forceinline__ ChunkPtr<FMT, CW> chunk_ptr(const Planes &p, int64_t c) {
  ChunkPtr<FMT, CW> r;
  if constexpr (FMT == FMT_PQ2) {
    r.base = p.base + c * (CW / 4);
    r.high = nullptr;
    r.scale = p.scale + (c * CW) / 128;
  } else {
    const int64_t g = c >> 2;
    const int q = (int)(c & 3);
    r.base = p.base + g * 24 + ((6 * q) & ~3);
    r.high = p.high + g * 2 + (q >> 1);
    r.scale = p.scale + g;
  }
  return r;
}

// Raw plane bytes of one lane chunk of row `row` (always a valid row).
template <int FMT, int CW>
__device__ __forceinline__ void load_raw(const Planes &p, const ChunkPtr<FMT, CW> &cp, int64_t row,
                                         Raw<FMT, CW> &r) {
  const uint8_t *b = cp.base + row * p.base_row;
  if constexpr (FMT == FMT_PQ2) {
    if constexpr (CW == 64) {
      u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(b));
      r.w[0] = t[0]; r.w[1] = t[1]; r.w[2] = t[2]; r.w[3] = t[3];
    } else if constexpr (CW == 32) {
      u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(b));
      r.w[0] = t[0]; r.w[1] = t[1];
    } else {
      r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(b));
    }
    r.h = 0;
  } else {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(b));
    r.w[1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(b + 4));
    r.h = cp.high[row * p.high_row];
  }
  r.s = cp.scale[row * p.groups];
}

// Loader cursor: the plane pointers of one lane chunk at row `row`,
// advanced by fixed byte strides (no 64-bit multiplies in the loop).  Rows
// past n are skipped (no memory access) and masked when reduced.
template <int FMT, int CW>
struct Cursor {
  const uint8_t *b, *h;
  const uint16_t *s;
  int64_t row;
  int64_t sb, sh, ss, srow;  // strides per step
};

template <int FMT, int CW>
__device__ __forceinline__ Cursor<FMT, CW> make_cursor(const Planes &p, const ChunkPtr<FMT, CW> &cp,
                                                      int64_t row, int64_t row_step) {
  Cursor<FMT, CW> k;
  k.row = row;
  k.b = cp.base + row * p.base_row;
  k.h = cp.high + row * p.high_row;
  k.s = cp.scale + row * p.groups;
  k.sb = row_step * p.base_row;
  k.sh = row_step * p.high_row;
  k.ss = row_step * p.groups;
  k.srow = row_step;
  return k;
}

template <int FMT, int CW>
__device__ __forceinline__ void load_next(Cursor<FMT, CW> &k, int64_t n, Raw<FMT, CW> &r) {
  // rows past n are not read at all (masked lanes make no memory access):
  // pointing them at one shared valid row would funnel every such request
  // of the grid into one L2 channel
  if (k.row < n) {
    const uint8_t *b = k.b;
    if constexpr (FMT == FMT_PQ2) {
      if constexpr (CW >= 64) {
#pragma unroll
        for (int q = 0; q < CW / 64; ++q) {
          u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(b) + q);
          r.w[4 * q] = t[0]; r.w[4 * q + 1] = t[1]; r.w[4 * q + 2] = t[2]; r.w[4 * q + 3] = t[3];
        }
      } else if constexpr (CW == 32) {
        u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(b));
        r.w[0] = t[0]; r.w[1] = t[1];
      } else {
        r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(b));
      }
      r.h = 0;
    } else {
      r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(b));
      r.w[1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(b + 4));
      r.h = *k.h;
    }
    r.s = *k.s;
  }  // else: the slot keeps stale data; that row is masked when reduced
  k.b += k.sb;
  k.h += k.sh;
  k.s += k.ss;
  k.row += k.srow;
}

// sum_j code_j * x_j over one lane chunk (codes 0..2 for ternary data).
template <int FMT, int CW, int B>
__device__ __forceinline__ void chunk_dot(const Raw<FMT, CW> &r, int64_t c,
                                          const half2_t (&xp)[B][CW / 2],
                                          const uint32_t *lut, float part[B]) {
#pragma unroll
  for (int b = 0; b < B; ++b) part[b] = 0.0f;
  if constexpr (FMT == FMT_PQ2) {
    // A code masked in place into a binary16 with zero exponent is the exact
    // subnormal code * 4^e * 2^-24 (e = its 2-bit slot, slots 0..4 of each
    // half); slots 5..7 are shifted down by 10 first.  Products are summed
    // per slot class in fp32 and rescaled by powers of two at the end.
    float a[B][5];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int e = 0; e < 5; ++e) a[b][e] = 0.0f;
#pragma unroll
    for (int d = 0; d < CW / 16; ++d) {
      const uint32_t w = r.w[d], w10 = w >> 10;
      const uint32_t t[8] = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u,
                             w & 0x00C000C0u, w & 0x03000300u, w10 & 0x00030003u,
                             w10 & 0x000C000Cu, w10 & 0x00300030u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int b = 0; b < B; ++b)
          a[b][e < 5 ? e : e - 5] = dot2(bits_h2(t[e]), xp[b][8 * d + e], a[b][e < 5 ? e : e - 5]);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b)
      part[b] = a[b][0] * 16777216.0f + a[b][1] * 4194304.0f + a[b][2] * 1048576.0f +
                a[b][3] * 262144.0f + a[b][4] * 65536.0f;
  } else {
    const int q = (int)(c & 3);
    // the lane's 6 base bytes start 0 or 2 bytes into the loaded window
    const uint64_t win = ((uint64_t)r.w[1] << 32) | r.w[0];
    const uint64_t bytes = (q & 1) ? (win >> 16) : win;
    // lut[v]: the five radix-3 digits of byte v as 2-bit codes, digit i at
    // bits 2i.  Two bytes side by side (second one shifted up 16) give, for
    // each digit i, a binary16 pair whose zero-exponent fields are the codes
    // times 4^i * 2^-24: the same subnormal-class products as PQ2_0, one
    // mask and one dot2 per two trits.
    float a[B][5];
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) {
      const uint32_t dw = lut[(bytes >> (16 * pp)) & 0xFF] |
                          (lut[(bytes >> (16 * pp + 8)) & 0xFF] << 16);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const half2_t t = bits_h2(dw & (0x00030003u << (2 * i)));
#pragma unroll
        for (int b = 0; b < B; ++b)
          a[b][i] = __builtin_amdgcn_fdot2(t, xp[b][5 * pp + i], pp == 0 ? 0.0f : a[b][i], false);
      }
    }
    // the chunk's two high trits: digits 2(q&1) and 2(q&1)+1 of its high
    // byte, placed as a class-0 pair
    const uint32_t wh = lut[r.h & 0xFF] >> (4 * (q & 1));
    const half2_t th = bits_h2((wh & 3u) | ((wh & 0xCu) << 14));
#pragma unroll
    for (int b = 0; b < B; ++b) {
      a[b][0] = dot2(th, xp[b][15], a[b][0]);
      part[b] = a[b][0] * 16777216.0f + a[b][1] * 4194304.0f + a[b][2] * 1048576.0f +
                a[b][3] * 262144.0f + a[b][4] * 65536.0f;
    }
  }
}

// Sum over aligned segments of SEG (8 or 16) lanes inside each DPP row; the
// total lands in the segment's last lane (inclusive scan with row_shr 1, 2,
// 4 (, 8): a shift never reaches past the segment start before the partial
// it pulls already covers that segment only).
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x111, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x112, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x114, 0xF, 0xF, true));
  if constexpr (SEG == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x118, 0xF, 0xF, true));
  return v;
}

// Sum over the 16 lanes of each DPP row; the total lands in lane 15 of the
// row (inclusive scan with row_shr 1, 2, 4, 8).
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x111, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x112, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x114, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                            0x118, 0xF, 0xF, true));
  return v;
}

// Persistent launch: R teams of cseg threads per workgroup (cseg = chunks
// per row rounded up to a 16-lane segment); a "pass" is R consecutive rows,
// one per team.  Workgroup w handles passes w, w + G, w + 2G, ... (G = grid
// size), so the workgroups resident at one time read one compact band of
// rows.  Each lane keeps its activation chunk in registers for the whole
// kernel and the weights of the next D passes in flight: after a pass is
// consumed its ring slot is refilled with the pass D steps ahead.  Every D
// passes the segment sums are reduced through LDS and written out.
template <int FMT, int CW, int B, int D, int XD, int LB, int SEG>
__global__ __launch_bounds__(LB) void gemv_kernel(Planes p, const void *__restrict__ x,
                                                  int64_t batch, int64_t ldx,
                                                  float *__restrict__ y, int64_t ldy,
                                                  int chunks, int cseg, int teams) {
  __shared__ uint32_t lut[FMT == FMT_PTQ1 ? 256 : 1];
  __shared__ float red[D * B * (1024 / SEG)];  // [slot][b][segment]
  // activation pairs of every chunk in decode order, plus chunk sums:
  // staged once per workgroup (teams share chunks)
  extern __shared__ uint32_t xlds[];  // [chunk][CW/2 pairs], then [chunk] sums (one batch row)

  const int t = threadIdx.x;
  const int team = t / cseg;
  const int c = t % cseg;
  const bool active = team < teams && c < chunks;
  const int64_t npass = (p.n + teams - 1) / teams;
  const int64_t G = gridDim.x;

  if constexpr (FMT == FMT_PTQ1) {
    // byte v -> its radix-3 digits floor(v / 3^i) mod 3, i < 5, as 2-bit
    // codes at bits 2i (high bytes use digits 0..3 of the same table)
    for (int v = t; v < 256; v += blockDim.x) {
      uint32_t u = (uint32_t)v, w = 0;
      for (int i = 0; i < 5; ++i) { w |= (u % 3u) << (2 * i); u /= 3u; }
      lut[v] = w;
    }
  }
  // ---- stage the activations, one batch row at a time: thread i converts
  // chunk i of row b into LDS; every lane then copies its own chunk's pairs
  // into registers
  half2_t xp[B][CW / 2];
  float xs[B];
  const int64_t cc = c < chunks ? c : 0;
  if constexpr (FMT == FMT_PTQ1) __syncthreads();  // tables ready
#pragma unroll
  for (int b = 0; b < B; ++b) {
    if (b < batch) {
      for (int i = t; i < chunks; i += blockDim.x) {
        XRaw<FMT, CW, XD> xr;
        load_x_raw<FMT, CW, XD>(x, b * ldx, i, xr);
        half2_t xp1[CW / 2];
        const float sum = convert_x_chunk<FMT, CW, XD>(xr, i, xp1);
        uint32_t *dst = xlds + (int64_t)i * (CW / 2);
#pragma unroll
        for (int k = 0; k < CW / 2; k += 4)
          *reinterpret_cast<u32x4 *>(dst + k) = (u32x4){
              __builtin_bit_cast(uint32_t, xp1[k]), __builtin_bit_cast(uint32_t, xp1[k + 1]),
              __builtin_bit_cast(uint32_t, xp1[k + 2]), __builtin_bit_cast(uint32_t, xp1[k + 3])};
        xlds[(int64_t)chunks * (CW / 2) + i] = __float_as_uint(sum);
      }
    }
    __syncthreads();
    const bool xok = active && b < batch;
    const uint32_t *src = xlds + cc * (CW / 2);
#pragma unroll
    for (int k = 0; k < CW / 2; k += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src + k);
      xp[b][k] = bits_h2(xok ? v[0] : 0u);
      xp[b][k + 1] = bits_h2(xok ? v[1] : 0u);
      xp[b][k + 2] = bits_h2(xok ? v[2] : 0u);
      xp[b][k + 3] = bits_h2(xok ? v[3] : 0u);
    }
    xs[b] = xok ? __uint_as_float(xlds[(int64_t)chunks * (CW / 2) + cc]) : 0.0f;
    __syncthreads();
  }

  // ---- weight ring: idle lanes read chunk 0 and are masked afterwards,
  // rows past n are not read; pointers advance by fixed strides
  const ChunkPtr<FMT, CW> cp = chunk_ptr<FMT, CW>(p, cc);
  const int64_t row_step = G * teams;  // rows between consecutive passes
  Cursor<FMT, CW> cur = make_cursor<FMT, CW>(p, cp, (int64_t)blockIdx.x * teams + team, row_step);
  Raw<FMT, CW> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_next<FMT, CW>(cur, p.n, ring[d]);
    __builtin_amdgcn_sched_barrier(0);
  }

  __builtin_amdgcn_sched_barrier(0);

  constexpr int NSEG = 1024 / SEG;
  const int seg = t / SEG;
  const int segs_per_team = cseg / SEG;
  int64_t row = (int64_t)blockIdx.x * teams + team;  // row of ring slot 0
  for (int64_t base = blockIdx.x; base < npass; base += D * G) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      float part[B];
      chunk_dot<FMT, CW, B>(ring[d], cc, xp, lut, part);
      const float s = f16_to_f32((uint16_t)ring[d].s);
      // refill the slot with the pass D steps ahead
      load_next<FMT, CW>(cur, p.n, ring[d]);
      const bool ok = active && row < p.n;
      row += row_step;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float v = seg_sum<SEG>(ok ? s * (part[b] - xs[b]) : 0.0f);
        if ((t & (SEG - 1)) == SEG - 1) red[(d * B + b) * NSEG + seg] = v;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    for (int o = t; o < D * teams * B; o += blockDim.x) {
      const int d = o / (teams * B);
      const int rem = o % (teams * B);
      const int tm = rem / B, b = rem % B;
      const int64_t orow = (base + d * G) * teams + tm;
      if (orow >= p.n || b >= batch) continue;
      float sum = 0.0f;
      const float *rp = red + (d * B + b) * NSEG + tm * segs_per_team;
      for (int sgi = 0; sgi < segs_per_team; ++sgi) sum += rp[sgi];
      y[b * ldy + orow] = sum;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// PQ2_0 batch-1 GEMV, one wave per row.
//
// A row of k = 1024*m weights is k/4 bytes; lane l of the wave reads, for
// each of the A = m/4 whole kilobytes of the row, the 16 bytes at
// 1024*i + 16*l (64 weights, inside group 32*i + l/2) and, for each of the
// BQ = m%4 remaining 256-byte blocks, the 4 bytes at 1024*A + 256*j + 4*l
// (16 weights, inside group 32*A + 8*j + l/8).  Every load instruction of the
// wave covers one contiguous span, the wave's partial sums are reduced with
// DPP row shifts and four lane reads, and lane 0 writes the row: waves never
// synchronise, so each is an independent persistent stream over blocks of D
// consecutive rows (W = waves in the grid) with D rows in flight.
template <int A, int BQ>
struct WRaw {
  uint32_t w[4 * A + BQ];
  uint32_t s[A + BQ];
};

__device__ __forceinline__ float wave_sum(float v) {
  v = seg_sum<16>(v);  // lanes 15, 31, 47, 63 hold their row's sum
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sums of up to 8 rows' per-lane partials v[0..D-1] over the 64 lanes of a
// wave, all at once: two swap stages halve the values per lane while pairing
// lane halves (32) and 16-lane rows, a rotate by 8 inside each 16-lane row
// merges the last two values, and three DPP row shifts finish each 8-lane
// group.  Lane 8g+7 then holds the total of row bitrev3(g); it is returned
// for that lane (other lanes return garbage) together with the row index.
template <int D>
__device__ __forceinline__ float rows8_sum(const float (&v)[D], int lane, int &row) {
  static_assert(D >= 1 && D <= 8, "at most 8 rows");
  auto bits = [](float f) { return __builtin_bit_cast(unsigned, f); };
  auto flt = [](unsigned u) { return __builtin_bit_cast(float, u); };
  float u[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) u[d] = d < D ? v[d] : 0.0f;
  // lanes 0-31 | 32-63 of s1[i] carry rows 2i | 2i+1
  float s1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(bits(u[2 * i]), bits(u[2 * i + 1]), false, false);
    s1[i] = flt(r[0]) + flt(r[1]);
  }
  // 16-lane rows R0..R3 of s2[i] carry rows 4i + (0, 2, 1, 3)
  float s2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(bits(s1[2 * i]), bits(s1[2 * i + 1]), false, false);
    s2[i] = flt(r[0]) + flt(r[1]);
  }
  // lanes 0-7 of each 16-lane row keep s2[0], lanes 8-15 s2[1]; each adds
  // the matching value of the other half-row (row_ror:8)
  const bool hi = (lane & 8) != 0;
  const float keep = hi ? s2[1] : s2[0];
  const float give = hi ? s2[0] : s2[1];
  float x = keep + flt(__builtin_amdgcn_update_dpp(0u, bits(give), 0x128, 0xF, 0xF, false));
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x111, 0xF, 0xF, true));
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x112, 0xF, 0xF, true));
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x114, 0xF, 0xF, true));
  const int g = lane >> 3;
  row = ((g & 1) << 2) | (g & 2) | ((g >> 2) & 1);
  return x;
}

// Workgroups are fat (WPG waves, one workgroup per CU) because the
// activation row is read once per workgroup: every wave reading it on its own
// sends thousands of requests to the same few L2 lines.  The first NB waves
// ("staging" waves) stage it into LDS as binary16 pairs in the order the
// decoder consumes them, lane-major so that every lane later reads its own
// pairs with conflict-free 16-byte LDS reads, together with the sum of every
// lane piece.  The other waves request their first D weight rows as soon
// as the activations have arrived, so the weight stream runs while the
// staging waves work; the staging waves request theirs once the staging is
// done (a wave whose loads fill the compute unit's memory queue stalls at
// its next load until rows arrive, which would hold up the staging).
//
// With FUSED set the kernel also performs the signed transform of its input
// ([tensorsharp] §4.2: a projection input is rotated by H(D.x)/32 per
// 1024-element block): x is then the unrotated activation row, each staging
// wave transforms its 1024-element blocks in registers and rounds them to
// binary16 exactly as the standalone transform with binary16 output does,
// so one launch covers the whole step with the same result as two.
template <int A, int BQ, int D, int XD, bool FUSED, int WPG>
__global__ __launch_bounds__(64 * WPG) void gemv_wave_kernel(Planes p, const void *__restrict__ x,
                                                             const uint16_t *__restrict__ signs,
                                                             float *__restrict__ y) {
  constexpr int NB = 4 * A + BQ;  // 1024-element blocks in a row = 16-weight dwords per lane
  constexpr int NP = A + BQ;      // pieces per lane
  // Activation pairs: dword s of lane l (16 weights, pairs (e, e+8)) is held
  // by quads (2s)*64 + l (pairs 0-3) and (2s+1)*64 + l (pairs 4-7).  Dword s
  // of lane l is natural 16-element chunk 256i + 4l + d for s = 4i + d < 4A
  // (a kilobyte piece) and 256A + 64j + l for s = 4A + j (a 256-byte piece).
  __shared__ __attribute__((aligned(16))) u32x4 xq[NB * 128];
  __shared__ float xsum[NP * 64];  // [piece][lane]: sum of the piece's binary16 activations
  __shared__ uint32_t staged;      // staging waves done
  // the transform's per-wave scratch (staging waves only)
  __shared__ __attribute__((aligned(16))) float wsc[FUSED ? (NB < WPG ? NB : WPG) : 1][1024];
  const int lane = threadIdx.x & 63;
  // the wave index is made explicitly uniform so that row offsets live in
  // scalar registers and every load is (scalar row base + lane offset)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * WPG + wave;
  const int64_t W = (int64_t)gridDim.x * WPG;
  const bool stager = wave < NB;

  // ---- rows: in pass q wave gw takes the D consecutive rows (q*W + gw)*D
  // + d, so each wave streams one contiguous span of every plane; the launch
  // picks D so that every wave has the same share.  Slot loads are
  // unconditional: a branch around them would stop the compiler from
  // counting the loads still in flight, and it would then wait for all of
  // them at every row.  A slot whose next row lies past n re-reads the row
  // it already holds (fb), so such loads stay spread over the planes; the
  // last pass requests nothing (a wave cannot end before its loads return).
  // Row numbers are 32-bit (the launch guarantees n < 2^30): the scalar
  // unit has no 64-bit ordered compare, so 64-bit row tests would run on the
  // vector unit every row.
  const int n32 = (int)p.n;
  const int q0 = lane / 2, q1 = 32 * A + lane / 8;  // scale entries
  auto load_row = [&](int row, int fb, WRaw<A, BQ> &r) {
    const int rr = row < n32 ? row : fb;
    // the row's base bytes as a buffer: the row address stays in scalar
    // registers and each load adds only the lane's offset (a streaming load
    // through a flat pointer would rebuild the 64-bit address every row)
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(p.base + (int64_t)rr * p.base_row), 0, (int)p.base_row, 0x00020000);
    const uint16_t *rs = p.scale + (int64_t)rr * p.groups;
#pragma unroll
    for (int i = 0; i < A; ++i) {
      const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane + 1024 * i, 0, CPOL_NT);
      r.w[4 * i] = t[0]; r.w[4 * i + 1] = t[1]; r.w[4 * i + 2] = t[2]; r.w[4 * i + 3] = t[3];
      r.s[i] = rs[q0 + 32 * i];
    }
#pragma unroll
    for (int j = 0; j < BQ; ++j) {
      r.w[4 * A + j] = __builtin_amdgcn_raw_buffer_load_b32(rb, 1024 * A + 4 * lane + 256 * j, 0, CPOL_NT);
      r.s[A + j] = rs[q1 + 8 * j];
    }
  };
  WRaw<A, BQ> ring[D];
  const int gw32 = (int)gw, W32 = (int)W;
  const int first = gw32 * D < n32 ? gw32 * D : n32 - 1;
  auto load_first = [&]() {
#pragma unroll
    for (int d = 0; d < D; ++d) load_row(gw32 * D + d, first, ring[d]);
  };

  // ---- 1. the staging waves load the activations, and the workgroup
  // waits for them before any weight row is requested: requested alongside
  // the rows, they would queue behind the weight stream.  Fused: wave w
  // transforms blocks w, w + WPG, ... (chunks 64*block + lane); unfused:
  // thread t converts chunks t, t + 64*WPG, ...  Items past the end re-read
  // the last block or chunk, so the loads stay unconditional.
  constexpr int NI = FUSED ? (NB + WPG - 1) / WPG : (NB * 64 + 64 * WPG - 1) / (64 * WPG);
  Raw16<XD> xraw[NI];
  u32x4 sraw[FUSED ? NI : 1][2];
  auto item = [&](int i) -> int64_t {  // first element of item i of this thread
    if constexpr (FUSED) {
      const int blk = wave + WPG * i < NB ? wave + WPG * i : NB - 1;
      return (int64_t)blk * 1024 + 16 * lane;
    } else {
      const int c = (int)threadIdx.x + 64 * WPG * i;
      return 16 * (int64_t)(c < NB * 64 ? c : NB * 64 - 1);
    }
  };
  if (threadIdx.x == 0) staged = 0;
  if (stager) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      load16_raw<XD>(x, item(i), xraw[i]);
      if constexpr (FUSED) {
        const u32x4 *sp = reinterpret_cast<const u32x4 *>(signs + item(i));
        sraw[i][0] = sp[0];
        sraw[i][1] = sp[1];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  __syncthreads();

  // ---- 2. the other waves request their first D rows now
  if (!stager) load_first();
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. staging waves: activations -> binary16 pairs in LDS
  if (stager) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool mine = FUSED ? wave + WPG * i < NB : (int)threadIdx.x + 64 * WPG * i < NB * 64;
      if (!mine) continue;
      // h[m]: binary16 elements 2m, 2m+1 of this thread's 16-element chunk
      uint32_t h[8];
      if constexpr (FUSED) {
        float v[16];
        convert16<XD>(xraw[i], v);
        const uint32_t sw[8] = {sraw[i][0][0], sraw[i][0][1], sraw[i][0][2], sraw[i][0][3],
                                sraw[i][1][0], sraw[i][1][1], sraw[i][1][2], sraw[i][1][3]};
#pragma unroll
        for (int e = 0; e < 16; ++e)
          v[e] = apply_sign(v[e], (uint16_t)(sw[e >> 1] >> (16 * (e & 1))));
        // v[4g + j] leaves the transform holding element 256g + 4*lane + j
        // of the block; the block goes back through the wave's scratch in
        // natural order, and the lane takes chunk `lane` of it
        float *sc = wsc[wave];
        wht1024_wave(v, lane, sc);
        uint16_t *nat = reinterpret_cast<uint16_t *>(sc);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lo = (uint32_t)f32_to_f16(v[4 * g] * 0.03125f) |
                              ((uint32_t)f32_to_f16(v[4 * g + 1] * 0.03125f) << 16);
          const uint32_t hi = (uint32_t)f32_to_f16(v[4 * g + 2] * 0.03125f) |
                              ((uint32_t)f32_to_f16(v[4 * g + 3] * 0.03125f) << 16);
          *reinterpret_cast<u32x2 *>(nat + 256 * g + 4 * lane) = (u32x2){lo, hi};
        }
        const u32x4 *q = reinterpret_cast<const u32x4 *>(nat + 16 * lane);
        const u32x4 a0 = q[0], a1 = q[1];
        h[0] = a0[0]; h[1] = a0[1]; h[2] = a0[2]; h[3] = a0[3];
        h[4] = a1[0]; h[5] = a1[1]; h[6] = a1[2]; h[7] = a1[3];
      } else if constexpr (XD == DT_F16) {
#pragma unroll
        for (int m = 0; m < 4; ++m) { h[m] = xraw[i].q[0][m]; h[4 + m] = xraw[i].q[1][m]; }
      } else {
        float v[16];
        convert16<XD>(xraw[i], v);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          h[m] = (uint32_t)f32_to_f16(v[2 * m]) | ((uint32_t)f32_to_f16(v[2 * m + 1]) << 16);
      }
      // pairs (e, e+8) of the chunk and their sum
      uint32_t pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pr[e] = __builtin_amdgcn_perm(h[4 + e / 2], h[e / 2], (e & 1) ? 0x07060302u : 0x05040100u);
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sum = __builtin_amdgcn_fdot2(bits_h2(pr[e]), bits_h2(0x3C003C00u), sum, false);
      const int c = FUSED ? (wave + WPG * i) * 64 + lane : (int)threadIdx.x + 64 * WPG * i;
      int s, l;
      if (c < 256 * A) {
        s = 4 * (c >> 8) + (c & 3);
        l = (c & 255) >> 2;
      } else {
        s = 4 * A + ((c - 256 * A) >> 6);
        l = (c - 256 * A) & 63;
      }
      xq[(2 * s) * 64 + l] = (u32x4){pr[0], pr[1], pr[2], pr[3]};
      xq[(2 * s + 1) * 64 + l] = (u32x4){pr[4], pr[5], pr[6], pr[7]};
      // a kilobyte piece is four consecutive chunks, held by the four lanes
      // of a DPP quad (chunk index = lane index mod 4): sum them there
      float qs = sum + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                           __builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
      qs += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                __builtin_bit_cast(int, qs), 0x4E, 0xF, 0xF, false));            // quad_perm 2,3,0,1
      if (c < 256 * A) {
        if ((c & 3) == 0) xsum[(c >> 8) * 64 + l] = qs;
      } else {
        xsum[(A + ((c - 256 * A) >> 6)) * 64 + l] = sum;
      }
    }
    // publish: the wave's LDS writes complete before the count (LDS
    // operations only: a release fence would also wait for the global loads)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (lane == 0) __hip_atomic_fetch_add(&staged, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // Every wave waits for all staging waves.  Not a workgroup barrier: the
  // other waves may still be stalled issuing their rows, and the staging
  // waves need not wait for that.  Each staging wave counts exactly once
  // on every path, so the wait ends; the bound only guards against a
  // defect turning into a hang.
  {
    constexpr uint32_t NSTG = NB < WPG ? NB : WPG;
    for (int spin = 0; spin < (1 << 22); ++spin) {
      const uint32_t done = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&staged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
      if (done >= NSTG) break;
      __builtin_amdgcn_s_sleep(1);
    }
    // the pair reads below are issued only after the count was seen, and
    // LDS executes them after the writes that preceded it
    asm volatile("" ::: "memory");
  }

  // ---- 4. the lane's activation pairs and piece sums (read before the
  // staging waves request their rows, which may stall at issue)
  half2_t xp[NB][8];
  float xs[NP];
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    const u32x4 a = xq[(2 * s) * 64 + lane], b = xq[(2 * s + 1) * 64 + lane];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xp[s][k] = bits_h2(a[k]);
      xp[s][4 + k] = bits_h2(b[k]);
    }
  }
#pragma unroll
  for (int pc = 0; pc < NP; ++pc) xs[pc] = xsum[pc * 64 + lane];
  __builtin_amdgcn_sched_barrier(0);
  if (stager) load_first();
  __builtin_amdgcn_sched_barrier(0);

  // ---- 5. passes of D rows
  auto do_pass = [&](int base, auto refill) {
    float part[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // sum over the lane's pieces of s * (sum code*x - sum x); the first
      // product of each class starts from 0 instead of a zeroed register
      float acc = 0.0f;
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        const int nd = pc < A ? 4 : 1;
        const int d0 = pc < A ? 4 * pc : 4 * A + (pc - A);
        // codes 0-3 (and 8-11) in place, codes 4-7 (and 12-15) shifted
        // down a byte: four slot classes, e and e+4 in class e
        float a[4];
#pragma unroll
        for (int q = 0; q < nd; ++q) {
          const uint32_t w = ring[d].w[d0 + q], w8 = w >> 8;
          const uint32_t t[8] = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u,
                                 w & 0x00C000C0u, w8 & 0x00030003u, w8 & 0x000C000Cu,
                                 w8 & 0x00300030u, w8 & 0x00C000C0u};
          if (q == 0) dot2_first4(t, xp[d0], a);
#pragma unroll
          for (int e = q == 0 ? 4 : 0; e < 8; ++e)
            a[e & 3] = __builtin_amdgcn_fdot2(bits_h2(t[e]), xp[d0 + q][e], a[e & 3], false);
        }
        const float cx = a[0] * 16777216.0f + a[1] * 4194304.0f + a[2] * 1048576.0f +
                         a[3] * 262144.0f;
        acc += f16_to_f32((uint16_t)ring[d].s[pc]) * (cx - xs[pc]);
      }
      part[d] = acc;
      // refill the slot with its row of the next pass
      if constexpr (decltype(refill)::value)
        load_row(base + d + D * W32, base + d < n32 ? base + d : n32 - 1, ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    int r;
    const float tot = rows8_sum<D>(part, lane, r);
    if ((lane & 7) == 7 && r < D && base + r < n32) y[base + r] = tot;
  };
  int base = gw32 * D;
  for (; base + D * W32 < n32; base += D * W32) do_pass(base, std::integral_constant<bool, true>{});
  if (base < n32) do_pass(base, std::integral_constant<bool, false>{});
}

template <int A, int BQ, int D, int XD, bool FUSED, int WPG>
static hipError_t gemv_wave_launch(const Planes &p, const void *x, const uint16_t *signs, float *y,
                                   int64_t waves, hipStream_t st) {
  const int64_t grid = (waves + WPG - 1) / WPG;
  hipLaunchKernelGGL((gemv_wave_kernel<A, BQ, D, XD, FUSED, WPG>), dim3((unsigned)grid),
                     dim3(64 * WPG), 0, st, p, x, signs, y);
  return hipGetLastError();
}

// Row split: for each ring depth D in {4, 6, 8} (D rows per wave and pass)
// take as many workgroups per CU as fit, the fewest passes that cover n, and
// then the fewest waves; keep the D whose busiest CU has the fewest rows
// (ties: the deeper ring).  Rows past n in a wave's last block re-read the
// row their slot already holds.  Workgroup size by register need: three
// waves per SIMD up to k = 5120 (WPG 12), two up to k = 7168 (WPG 8), one
// beyond (WPG 4).
template <int A, int BQ, int XD, bool FUSED>
static hipError_t gemv_wave_go(const Planes &p, const void *x, const uint16_t *signs, float *y,
                               hipStream_t st) {
  constexpr int NBK = 4 * A + BQ;
  constexpr int WPG = NBK <= 5 ? 12 : NBK <= 7 ? 8 : 4;
  const int cus = device_cus();
  const void *kerns[3] = {
      reinterpret_cast<const void *>(gemv_wave_kernel<A, BQ, 4, XD, FUSED, WPG>),
      reinterpret_cast<const void *>(gemv_wave_kernel<A, BQ, 6, XD, FUSED, WPG>),
      reinterpret_cast<const void *>(gemv_wave_kernel<A, BQ, 8, XD, FUSED, WPG>)};
  const int depth[3] = {4, 6, 8};
  int best = -1;
  int64_t best_rows = 0, best_waves = 0;
  for (int i = 0; i < 3; ++i) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kerns[i], 64 * WPG, 0) != hipSuccess ||
        per_cu < 1)
      continue;  // this depth does not fit a workgroup on a CU
    const int64_t D = depth[i];
    const int64_t slots = (int64_t)WPG * cus * per_cu;
    const int64_t passes = (p.n + slots * D - 1) / (slots * D);
    const int64_t waves = (p.n + D * passes - 1) / (D * passes);
    const int64_t wgs = (waves + WPG - 1) / WPG;
    const int64_t rows_cu = ((wgs + cus - 1) / cus) * WPG * D * passes;
    if (best < 0 || rows_cu <= best_rows) {
      best = i;
      best_rows = rows_cu;
      best_waves = waves;
    }
  }
  if (best < 0) return hipErrorInvalidConfiguration;
  if (best == 0) return gemv_wave_launch<A, BQ, 4, XD, FUSED, WPG>(p, x, signs, y, best_waves, st);
  if (best == 1) return gemv_wave_launch<A, BQ, 6, XD, FUSED, WPG>(p, x, signs, y, best_waves, st);
  return gemv_wave_launch<A, BQ, 8, XD, FUSED, WPG>(p, x, signs, y, best_waves, st);
}

template <int A, int BQ, bool FUSED>
static hipError_t gemv_wave_dt(const Planes &p, const void *x, int xd, const uint16_t *signs,
                               float *y, hipStream_t st) {
  if (xd == DT_F32) return gemv_wave_go<A, BQ, DT_F32, FUSED>(p, x, signs, y, st);
  if (xd == DT_BF16) return gemv_wave_go<A, BQ, DT_BF16, FUSED>(p, x, signs, y, st);
  return gemv_wave_go<A, BQ, DT_F16, FUSED>(p, x, signs, y, st);
}

// k = 1024*m with m <= 11: pieces A = m/4 kilobytes + BQ = m%4 blocks.
static bool gemv_wave_fits(const Planes &p) {
  return p.fmt == FMT_PQ2 && p.k % 1024 == 0 && p.k / 1024 >= 1 && p.k / 1024 <= 11 &&
         p.n < (int64_t(1) << 30);
}

template <bool FUSED>
static hipError_t gemv_wave(const Planes &p, const void *x, int xd, const uint16_t *signs, float *y,
                            hipStream_t st) {
  switch (p.k / 1024) {
    case 1: return gemv_wave_dt<0, 1, FUSED>(p, x, xd, signs, y, st);
    case 2: return gemv_wave_dt<0, 2, FUSED>(p, x, xd, signs, y, st);
    case 3: return gemv_wave_dt<0, 3, FUSED>(p, x, xd, signs, y, st);
    case 4: return gemv_wave_dt<1, 0, FUSED>(p, x, xd, signs, y, st);
    case 5: return gemv_wave_dt<1, 1, FUSED>(p, x, xd, signs, y, st);
    case 6: return gemv_wave_dt<1, 2, FUSED>(p, x, xd, signs, y, st);
    case 7: return gemv_wave_dt<1, 3, FUSED>(p, x, xd, signs, y, st);
    case 8: return gemv_wave_dt<2, 0, FUSED>(p, x, xd, signs, y, st);
    case 9: return gemv_wave_dt<2, 1, FUSED>(p, x, xd, signs, y, st);
    case 10: return gemv_wave_dt<2, 2, FUSED>(p, x, xd, signs, y, st);
    default: return gemv_wave_dt<2, 3, FUSED>(p, x, xd, signs, y, st);
  }
}

// ---------------------------------------------------------------------------
// PQ2_0 GEMV on the matrix cores (batch 1..4).
//
// v_mfma_f32_4x4x4_16b_f16 multiplies 16 independent 4x4x4 blocks; block q of
// a wave is lanes 4q..4q+3.  Here a block is one activation chunk of 64
// weights shared by 4 weight rows: lane 4q+j supplies 4 consecutive (in
// decode order) weights of row j as the B operand and the matching 4
// activations of batch row j (batch 1: the same row in all four lanes) as
// the A operand.  Output element [i][j] of a block is then
// sum_k x_i[k] * w_j[k] over the chunk; with batch 1 every i is the same
// activation row, so the element at index lane%4 is row (lane%4)'s partial
// sum whichever way the block's output is laid out over its lanes.
//
// Codes are decoded exactly to binary16 trits with full-rate integer ops:
// OR-ing a code at mantissa bits 2e (e <= 4) into the exponent of 1024
// gives 1024 + 4^e * code, and one packed fma with (1/4^e, -(1024/4^e + 1))
// turns that into code - 1 exactly; codes in bits 10..15 are shifted down
// first.  A dword of 16 codes takes 9 bit operations and 8 packed fmas.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// (d & mask) | magic in one v_and_or_b32 (magic held in a VGPR: a VOP3
// instruction takes at most one literal/SGPR operand here).
__device__ __forceinline__ uint32_t and_or(uint32_t d, uint32_t mask, uint32_t magic_v) {
  return (d & mask) | magic_v;
}

// Two masked code pairs -> 4 trits (binary16) for one MFMA B operand.
// t = 1024 + m*code (exact); fma(t, 1/m, -(1024/m + 1)) = code - 1 (exact).
__device__ __forceinline__ half4_t trit4(uint32_t ta, uint32_t tb, float inv_ma, float neg_ca,
                                         float inv_mb, float neg_cb) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t tt = {ta, tb};
  const half4_t t4 = __builtin_bit_cast(half4_t, tt);
  const half4_t m4 = {(_Float16)inv_ma, (_Float16)inv_ma, (_Float16)inv_mb, (_Float16)inv_mb};
  const half4_t c4 = {(_Float16)neg_ca, (_Float16)neg_ca, (_Float16)neg_cb, (_Float16)neg_cb};
  return __builtin_elementwise_fma(t4, m4, c4);
}

// 16 codes of dword d -> 4 MFMA B operands; operand h holds the trits of
// codes (2h, 2h+8, 2h+1, 2h+9).
__device__ __forceinline__ void decode_pq2_trit4(uint32_t d, uint32_t magic_v, half4_t w[4]) {
  const uint32_t d10 = d >> 10;
  w[0] = trit4(and_or(d, 0x00030003u, magic_v), and_or(d, 0x000C000Cu, magic_v),
               1.0f, -1025.0f, 0.25f, -257.0f);
  w[1] = trit4(and_or(d, 0x00300030u, magic_v), and_or(d, 0x00C000C0u, magic_v),
               0.0625f, -65.0f, 0.015625f, -17.0f);
  w[2] = trit4(and_or(d, 0x03000300u, magic_v), and_or(d10, 0x00030003u, magic_v),
               0.00390625f, -5.0f, 1.0f, -1025.0f);
  w[3] = trit4(and_or(d10, 0x000C000Cu, magic_v), and_or(d10, 0x00300030u, magic_v),
               0.25f, -257.0f, 0.0625f, -65.0f);
}

// Lane layout: thread t of the workgroup is lane j = t % 4 of block
// q = t / 4; blocks [team*cpad, team*cpad + chunks) hold the chunks of team
// `team`, each team covering 4 rows per pass.  cpad = chunks rounded up to a
// multiple of 4 (whole 16-lane segments).
template <int P, int XD, bool BATCHED>
__global__ __launch_bounds__(1024) void gemv_mfma_kernel(Planes p, const void *__restrict__ x,
                                                         int64_t batch, int64_t ldx,
                                                         float *__restrict__ y, int64_t ldy,
                                                         int chunks, int cpad, int teams) {
  __shared__ float red[P * (BATCHED ? 4 : 1) * 64 * 4];  // [pass][batch][segment][row j]
  const int t = threadIdx.x;
  const int j = t & 3;
  const int q = t >> 2;
  const int team = q / cpad;
  const int c = q % cpad;
  const bool active = team < teams && c < chunks;
  const int64_t rows_per_pass = 4 * (int64_t)teams;
  const int64_t row_base = (int64_t)blockIdx.x * rows_per_pass * P + 4 * team + j;

  // ---- weight loads for all P passes (16 bytes = 64 codes per lane)
  u32x4 raw[P];
  uint32_t sraw[P];
  const uint8_t *wp = p.base + row_base * p.base_row + c * 16;
  const uint16_t *sp = p.scale + row_base * p.groups + (c >> 1);
  const int64_t wstep = rows_per_pass * p.base_row, sstep = rows_per_pass * p.groups;
#pragma unroll
  for (int it = 0; it < P; ++it) {
    if (active && row_base + it * rows_per_pass < p.n) {
      raw[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wp + it * wstep));
      sraw[it] = sp[it * sstep];
    }
  }

  // ---- activations of the chunk as the A operand, in decode order:
  // dword d, pair e = (16d + e, 16d + e + 8); MFMA step (d, h) uses pairs
  // 2h, 2h+1.  Batched: lane j carries batch row j (zero beyond batch).
  half4_t xa[16];  // A operand of MFMA step (dword d, h): xa[4d + h]
  {
    const int b = BATCHED ? j : 0;
    const bool xok = active && b < batch;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float v[16];
      if (xok) {
        load16<XD>(x, b * ldx + (int64_t)c * 64 + 16 * d, v);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int e = 2 * h;
        xa[4 * d + h] = (half4_t){(_Float16)v[e], (_Float16)v[e + 8], (_Float16)v[e + 1],
                                  (_Float16)v[e + 9]};
      }
    }
  }
  uint32_t magic_v = 0x64006400u;
  asm volatile("" : "+v"(magic_v));

  const int seg = t >> 4;
#pragma unroll
  for (int it = 0; it < P; ++it) {
    const bool ok = active && row_base + it * rows_per_pass < p.n;
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float s = 0.0f;
    if (ok) {
      const uint32_t dw[4] = {raw[it][0], raw[it][1], raw[it][2], raw[it][3]};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        half4_t w[4];
        decode_pq2_trit4(dw[d], magic_v, w);
#pragma unroll
        for (int h = 0; h < 4; ++h)
          acc = __builtin_amdgcn_mfma_f32_4x4x4f16(xa[4 * d + h], w[h], acc, 0, 0, 0);
      }
      s = f16_to_f32(sraw[it]);
    }
    // batch 1: element j is row j's partial; batched: lane j of the block
    // holds its column's four batch rows (elements) -- reduced below per
    // element.
    if constexpr (!BATCHED) {
      float v = j == 0 ? acc[0] : j == 1 ? acc[1] : j == 2 ? acc[2] : acc[3];
      v *= s;
      // sum the 4 blocks of this 16-lane segment (lanes with equal j)
      v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
      v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
      if ((t & 15) >= 12) red[(it * 64 + seg) * 4 + j] = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = acc[e] * s;
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
        acc[e] = v;
      }
      // lane 12+j holds (batch e, row j) sums of its segment; stash them
      if ((t & 15) >= 12) {
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((it * 4 + e) * 64 + seg) * 4 + j] = acc[e];
      }
    }
  }
  __syncthreads();
  const int segs = cpad >> 2;
  const int nb = BATCHED ? 4 : 1;
  for (int o = t; o < P * teams * 4 * nb; o += blockDim.x) {
    const int jj = o & 3;
    const int rest = o >> 2;
    const int b = rest % nb;
    const int tm = (rest / nb) % teams;
    const int it = rest / (nb * teams);
    const int64_t row = (int64_t)blockIdx.x * rows_per_pass * P + it * rows_per_pass + 4 * tm + jj;
    if (row >= p.n || b >= batch) continue;
    const float *rp = BATCHED ? red + ((it * 4 + b) * 64 + tm * segs) * 4 + jj
                              : red + (it * 64 + tm * segs) * 4 + jj;
    float sum = 0.0f;
    for (int sgi = 0; sgi < segs; ++sgi) sum += rp[4 * sgi];
    y[b * ldy + row] = sum;
  }
}

// Teams per workgroup: fewest idle lanes, then the smallest workgroup.
// Workgroups stay within 512 lanes whenever one team fits, so the kernel
// can be compiled for a 512-lane bound (more registers per lane).
static int pick_teams(int cseg) {
  int best_r = 1;
  double best_eff = -1.0;
  const int cap = cseg <= 512 ? 512 : 1024;
  for (int r = 1; r * cseg <= cap; ++r) {
    const int threads = (r * cseg + 63) / 64 * 64;
    if (threads > cap) break;
    const double eff = (double)(r * cseg) / threads;
    if (eff > best_eff + 1e-9) { best_eff = eff; best_r = r; }
  }
  return best_r;
}

// Resident workgroups per compute unit for a kernel instance (cached).
template <typename K>
static int resident_per_cu(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}


template <int FMT, int CW, int B, int D, int XD, int LB, int SEG>
static hipError_t gemv_launch(const Planes &p, const void *x, int64_t batch, int64_t ldx, float *y,
                              int64_t ldy, int chunks, int cseg, int teams, int threads,
                              hipStream_t st) {
  auto kern = gemv_kernel<FMT, CW, B, D, XD, LB, SEG>;
  const size_t lds = (size_t)chunks * (CW / 2 + 1) * 4;
  const int64_t npass = (p.n + teams - 1) / teams;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int64_t slots = (int64_t)device_cus() * per_cu;
  const int64_t grid = npass < slots ? npass : slots;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds, st, p, x, batch, ldx, y, ldy,
                     chunks, cseg, teams);
  return hipGetLastError();
}

template <int FMT, int CW, int B, int D, int SEG = 16>
static hipError_t gemv_go(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                          float *y, int64_t ldy, hipStream_t st) {
  const int chunks = (int)(p.k / CW);
  const int cseg = (chunks + SEG - 1) / SEG * SEG;
  const int teams = pick_teams(cseg);
  const int threads = (teams * cseg + 63) / 64 * 64;
  // a 512-lane bound leaves each lane up to 256 registers
  if (threads <= 512) {
    if (xd == DT_F32)
      return gemv_launch<FMT, CW, B, D, DT_F32, 512, SEG>(p, x, batch, ldx, y, ldy, chunks, cseg,
                                                          teams, threads, st);
    if (xd == DT_BF16)
      return gemv_launch<FMT, CW, B, D, DT_BF16, 512, SEG>(p, x, batch, ldx, y, ldy, chunks, cseg,
                                                           teams, threads, st);
    return gemv_launch<FMT, CW, B, D, DT_F16, 512, SEG>(p, x, batch, ldx, y, ldy, chunks, cseg,
                                                        teams, threads, st);
  }
  if (xd == DT_F32)
    return gemv_launch<FMT, CW, B, D, DT_F32, 1024, SEG>(p, x, batch, ldx, y, ldy, chunks, cseg,
                                                         teams, threads, st);
  if (xd == DT_BF16)
    return gemv_launch<FMT, CW, B, D, DT_BF16, 1024, SEG>(p, x, batch, ldx, y, ldy, chunks, cseg,
                                                          teams, threads, st);
  return gemv_launch<FMT, CW, B, D, DT_F16, 1024, SEG>(p, x, batch, ldx, y, ldy, chunks, cseg,
                                                       teams, threads, st);
}

template <int FMT, int CW>
static hipError_t gemv_b1(const Planes &p, const void *x, int xd, int64_t ldx, float *y,
                          int64_t ldy, hipStream_t st) {
  // PQ2_0 rows whose 128-weight chunks fill whole 8-lane segments: one lane
  // streams 32 bytes per row (halves the per-row bookkeeping per weight)
  if constexpr (FMT == FMT_PQ2) {
    if ((p.k / 128) % 8 == 0 && p.k / 128 <= 512)
      return gemv_go<FMT, 128, 1, 4, 8>(p, x, xd, 1, ldx, y, ldy, st);
  }
  return gemv_go<FMT, CW, 1, 4>(p, x, xd, 1, ldx, y, ldy, st);
}

template <int P, bool BATCHED>
static hipError_t gemv_mfma_go(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                               float *y, int64_t ldy, hipStream_t st) {
  const int chunks = (int)(p.k / 64);
  const int cpad = (chunks + 3) / 4 * 4;
  const int teams = pick_teams(4 * cpad);
  const int threads = (teams * 4 * cpad + 63) / 64 * 64;
  const int64_t rows_per_wg = 4LL * teams * P;
  dim3 grid((unsigned)((p.n + rows_per_wg - 1) / rows_per_wg)), block(threads);
  if (xd == DT_F32)
    hipLaunchKernelGGL((gemv_mfma_kernel<P, DT_F32, BATCHED>), grid, block, 0, st, p, x, batch, ldx,
                       y, ldy, chunks, cpad, teams);
  else if (xd == DT_BF16)
    hipLaunchKernelGGL((gemv_mfma_kernel<P, DT_BF16, BATCHED>), grid, block, 0, st, p, x, batch, ldx,
                       y, ldy, chunks, cpad, teams);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<P, DT_F16, BATCHED>), grid, block, 0, st, p, x, batch, ldx,
                       y, ldy, chunks, cpad, teams);
  return hipGetLastError();
}

// PQ2_0 rows of up to 16384 weights run on the matrix cores (a team of
// 4 * ceil(k/256) * 4 lanes must fit a 1024-lane workgroup).
static bool gemv_mfma_fits(const Planes &p) { return p.k <= 16384; }

template <bool BATCHED>
static hipError_t gemv_mfma(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                            float *y, int64_t ldy, hipStream_t st) {
  const int cpad = ((int)(p.k / 64) + 3) / 4 * 4;
  const int64_t passes = (p.n + 4LL * pick_teams(4 * cpad) - 1) / (4LL * pick_teams(4 * cpad));
  if (passes >= 512 * 8) return gemv_mfma_go<8, BATCHED>(p, x, xd, batch, ldx, y, ldy, st);
  return gemv_mfma_go<4, BATCHED>(p, x, xd, batch, ldx, y, ldy, st);
}

// Largest supported k: a team of at most 1024 lanes must cover a row.
int64_t gemv_max_k(int fmt) { return fmt == FMT_PQ2 ? 64 * 1024 : 32 * 1024; }

// Lane chunk (CW weights), batch tile (B) and rows per thread (P) by batch:
// smaller chunks and fewer rows at larger batch keep the activation pairs
// (B * CW / 2 registers) and partial sums in registers without spilling.
hipError_t launch_gemv(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                       float *y, int64_t ldy, hipStream_t st) {
  if (p.fmt == FMT_PTQ1) {
    if (gemv_ptq1_fits(p)) return launch_gemv_ptq1(p, x, xd, batch, ldx, y, ldy, st);
    if (batch <= 1) return gemv_b1<FMT_PTQ1, 32>(p, x, xd, ldx, y, ldy, st);
    if (batch <= 2) return gemv_go<FMT_PTQ1, 32, 2, 4>(p, x, xd, batch, ldx, y, ldy, st);
    if (batch <= 4) return gemv_go<FMT_PTQ1, 32, 4, 2>(p, x, xd, batch, ldx, y, ldy, st);
    // 5..8 rows: one pass while a row's team fits a 512-lane workgroup; wider
    // rows would need a 1024-lane workgroup, whose 128-register lanes cannot
    // hold 8 rows of activation pairs, so they run as two passes of <= 4 rows
    if ((p.k / 32 + 15) / 16 * 16 <= 512)
      return gemv_go<FMT_PTQ1, 32, 8, 1>(p, x, xd, batch, ldx, y, ldy, st);
    hipError_t e = gemv_go<FMT_PTQ1, 32, 4, 2>(p, x, xd, 4, ldx, y, ldy, st);
    if (e != hipSuccess) return e;
    const int64_t esz = xd == DT_F32 ? 4 : 2;
    return gemv_go<FMT_PTQ1, 32, 4, 2>(p, static_cast<const char *>(x) + 4 * ldx * esz, xd,
                                       batch - 4, ldx, y + 4 * ldy, ldy, st);
  }
  // a chunk never spans two groups (64 | 128); wide rows need wider chunks
  const bool wide32 = p.k / 32 > 1024, wide16 = p.k / 16 > 1024;
  if (gemv_mfma_fits(p) && batch >= 2 && batch <= 4)
    return gemv_mfma<true>(p, x, xd, batch, ldx, y, ldy, st);
  if (batch <= 1 && gemv_wave_fits(p)) return gemv_wave<false>(p, x, xd, nullptr, y, st);
  if (batch <= 1 || (wide32 && batch <= 2)) {
    if (batch <= 1) return gemv_b1<FMT_PQ2, 64>(p, x, xd, ldx, y, ldy, st);
    return gemv_go<FMT_PQ2, 64, 2, 2>(p, x, xd, batch, ldx, y, ldy, st);
  }
  if (wide32) {
    if (batch <= 4) return gemv_go<FMT_PQ2, 64, 4, 1>(p, x, xd, batch, ldx, y, ldy, st);
    return gemv_go<FMT_PQ2, 64, 8, 1>(p, x, xd, batch, ldx, y, ldy, st);
  }
  if (batch <= 2) return gemv_go<FMT_PQ2, 32, 2, 4>(p, x, xd, batch, ldx, y, ldy, st);
  if (batch <= 4) return gemv_go<FMT_PQ2, 32, 4, 2>(p, x, xd, batch, ldx, y, ldy, st);
  if (wide16) return gemv_go<FMT_PQ2, 32, 8, 1>(p, x, xd, batch, ldx, y, ldy, st);
  return gemv_go<FMT_PQ2, 16, 8, 2>(p, x, xd, batch, ldx, y, ldy, st);
}

bool rotated_gemv_fused(const Planes &p, int64_t batch) {
  return batch == 1 && gemv_wave_fits(p);
}

hipError_t launch_rotated_gemv(const Planes &p, const void *x, int xd, const uint16_t *signs,
                               float *y, hipStream_t st) {
  return gemv_wave<true>(p, x, xd, signs, y, st);
}

}  // namespace tq
