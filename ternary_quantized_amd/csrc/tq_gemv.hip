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

namespace tq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t cvt_codes(uint32_t v, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 3);
  }
}

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

__device__ __forceinline__ half2_t pack_h2(float a, float b) {
  half2_t r;
  r.x = (_Float16)a;
  r.y = (_Float16)b;
  return r;
}

__device__ __forceinline__ float xload(const void *x, int xd, int64_t i) {
  if (xd == DT_F32) return static_cast<const float *>(x)[i];
  if (xd == DT_BF16) return bf16_to_f32(static_cast<const uint16_t *>(x)[i]);
  return f16_to_f32(static_cast<const uint16_t *>(x)[i]);
}

// Number of binary16 pairs a lane chunk feeds to v_dot2.
template <int FMT, int CW>
struct Chunk {
  static constexpr int pairs = CW / 2;
};

// Build the activation pairs of one lane chunk in the order the decoder
// produces weight pairs, and their fp32 sum (of the rounded values).
template <int FMT, int CW>
__device__ __forceinline__ float load_x_chunk(const void *x, int xd, int64_t xrow, int64_t c,
                                              half2_t xp[CW / 2]) {
  float v[CW];
  if constexpr (FMT == FMT_PQ2) {
    const int64_t k0 = c * CW;
#pragma unroll
    for (int i = 0; i < CW; ++i) v[i] = (float)(_Float16)xload(x, xd, xrow + k0 + i);
    // dword d covers weights 16d..16d+15; pairs (4q,4q+2) then (4q+1,4q+3).
#pragma unroll
    for (int d = 0; d < CW / 16; ++d) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xp[8 * d + 2 * q] = pack_h2(v[16 * d + 4 * q], v[16 * d + 4 * q + 2]);
        xp[8 * d + 2 * q + 1] = pack_h2(v[16 * d + 4 * q + 1], v[16 * d + 4 * q + 3]);
      }
    }
  } else {
    // chunk c = 4*g + q: base bytes 6q..6q+5 (trits 30q..30q+29 of group g)
    // and the high trits 120+2q, 121+2q.
    const int64_t g = c >> 2;
    const int q = (int)(c & 3);
    const int64_t gk = xrow + g * 128;
#pragma unroll
    for (int i = 0; i < 30; ++i) v[i] = (float)(_Float16)xload(x, xd, gk + 30 * q + i);
    v[30] = (float)(_Float16)xload(x, xd, gk + 120 + 2 * q);
    v[31] = (float)(_Float16)xload(x, xd, gk + 121 + 2 * q);
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) {
      const int b0 = 10 * pp, b1 = 10 * pp + 5;  // first trit of the byte pair
      xp[5 * pp + 0] = pack_h2(v[b0 + 0], v[b0 + 1]);
      xp[5 * pp + 1] = pack_h2(v[b0 + 2], v[b0 + 3]);
      xp[5 * pp + 2] = pack_h2(v[b1 + 0], v[b1 + 1]);
      xp[5 * pp + 3] = pack_h2(v[b1 + 2], v[b1 + 3]);
      xp[5 * pp + 4] = pack_h2(v[b0 + 4], v[b1 + 4]);
    }
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
  uint16_t s;      // scale bits
};

template <int FMT, int CW>
__device__ __forceinline__ void load_raw(const Planes &p, int64_t row, int64_t c, Raw<FMT, CW> &r) {
  if constexpr (FMT == FMT_PQ2) {
    const uint8_t *b = p.base + row * p.base_row + c * (CW / 4);
    if constexpr (CW == 64) {
      u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(b));
      r.w[0] = t[0]; r.w[1] = t[1]; r.w[2] = t[2]; r.w[3] = t[3];
    } else if constexpr (CW == 32) {
      u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(b));
      r.w[0] = t[0]; r.w[1] = t[1];
    } else {
      r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(b));
    }
    r.s = p.scale[row * p.groups + (c * CW) / 128];
    r.h = 0;
  } else {
    const int64_t g = c >> 2;
    const int q = (int)(c & 3);
    const uint8_t *gb = p.base + row * p.base_row + g * 24 + ((6 * q) & ~3);
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(gb));
    r.w[1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(gb + 4));
    const uint8_t *hb = p.high + row * p.high_row + g * 2;
    r.h = hb[q >> 1];
    r.s = p.scale[row * p.groups + g];
  }
}

// sum_j code_j * x_j over one lane chunk (codes 0..2 for ternary data).
template <int FMT, int CW, int B>
__device__ __forceinline__ void chunk_dot(const Raw<FMT, CW> &r, int64_t c,
                                          const half2_t (&xp)[B][CW / 2],
                                          const uint32_t *lut, float part[B]) {
#pragma unroll
  for (int b = 0; b < B; ++b) part[b] = 0.0f;
  if constexpr (FMT == FMT_PQ2) {
#pragma unroll
    for (int d = 0; d < CW / 16; ++d) {
      const uint32_t lo = r.w[d] & 0x33333333u;
      const uint32_t hi = (r.w[d] >> 2) & 0x33333333u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const half2_t wl = cvt_codes(lo, q);
        const half2_t wh = cvt_codes(hi, q);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          part[b] = dot2(wl, xp[b][8 * d + 2 * q], part[b]);
          part[b] = dot2(wh, xp[b][8 * d + 2 * q + 1], part[b]);
        }
      }
    }
  } else {
    const int q = (int)(c & 3);
    // the lane's 6 base bytes start 0 or 2 bytes into the loaded window
    const uint64_t win = ((uint64_t)r.w[1] << 32) | r.w[0];
    const uint64_t bytes = (q & 1) ? (win >> 16) : win;
    const uint32_t *lut_even = lut, *lut_odd = lut + 256, *lut_high = lut + 512;
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) {
      const uint32_t e0 = lut_even[(bytes >> (16 * pp)) & 0xFF];
      const uint32_t e1 = lut_odd[(bytes >> (16 * pp + 8)) & 0xFF];
      const uint32_t e4 = e0 | e1;
      const half2_t w0 = cvt_codes(e0, 0), w1 = cvt_codes(e0, 1);
      const half2_t w2 = cvt_codes(e1, 0), w3 = cvt_codes(e1, 1);
      const half2_t w4 = cvt_codes(e4, 2);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        part[b] = dot2(w0, xp[b][5 * pp + 0], part[b]);
        part[b] = dot2(w1, xp[b][5 * pp + 1], part[b]);
        part[b] = dot2(w2, xp[b][5 * pp + 2], part[b]);
        part[b] = dot2(w3, xp[b][5 * pp + 3], part[b]);
        part[b] = dot2(w4, xp[b][5 * pp + 4], part[b]);
      }
    }
    const uint32_t eh = lut_high[r.h & 0xFF];
    const half2_t wh = (q & 1) ? cvt_codes(eh, 1) : cvt_codes(eh, 0);
#pragma unroll
    for (int b = 0; b < B; ++b) part[b] = dot2(wh, xp[b][15], part[b]);
  }
}

// Launch shape: R teams of cseg threads (cseg = chunks per row rounded up to
// a 16-lane segment), each thread handling P rows of its team.
template <int FMT, int CW, int B, int P>
__global__ __launch_bounds__(1024) void gemv_kernel(Planes p, const void *__restrict__ x, int xd,
                                                    int64_t batch, int64_t ldx,
                                                    float *__restrict__ y, int64_t ldy,
                                                    int chunks, int cseg, int teams) {
  __shared__ uint32_t lut[FMT == FMT_PTQ1 ? 768 : 1];
  __shared__ float red[P * B * 64];  // [pass][b][segment], <= 64 segments

  const int t = threadIdx.x;
  const int team = t / cseg;
  const int c = t % cseg;
  const bool active = team < teams && c < chunks;

  if constexpr (FMT == FMT_PTQ1) {
    // Tables mapping a byte v to its radix-3 digits as fp4 nibbles:
    //  even/odd: digits 0..3 in nibbles 0..3, digit 4 in nibble 4 (even) or
    //  nibble 5 (odd), so OR-ing an even and an odd entry pairs the two
    //  fifth digits in byte 2; high: digits 0..3 in nibbles 0..3.
    for (int v = t; v < 256; v += blockDim.x) {
      uint32_t d[5], u = (uint32_t)v;
      for (int i = 0; i < 5; ++i) { d[i] = u % 3u; u /= 3u; }
      const uint32_t low = d[0] | (d[1] << 4) | (d[2] << 8) | (d[3] << 12);
      lut[v] = low | (d[4] << 16);
      lut[256 + v] = low | (d[4] << 20);
      lut[512 + v] = low;
    }
    __syncthreads();
  }

  half2_t xp[B][CW / 2];
  float xs[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    if (active && b < batch) {
      xs[b] = load_x_chunk<FMT, CW>(x, xd, b * ldx, c, xp[b]);
    } else {
      xs[b] = 0.0f;
#pragma unroll
      for (int i = 0; i < CW / 2; ++i) xp[b][i] = pack_h2(0.0f, 0.0f);
    }
  }

  const int64_t row0 = (int64_t)blockIdx.x * teams * P;
  Raw<FMT, CW> raw[P];
#pragma unroll
  for (int pi = 0; pi < P; ++pi) {
    const int64_t row = row0 + (int64_t)pi * teams + team;
    if (active && row < p.n) load_raw<FMT, CW>(p, row, c, raw[pi]);
  }
  float acc[P][B];
#pragma unroll
  for (int pi = 0; pi < P; ++pi) {
    const int64_t row = row0 + (int64_t)pi * teams + team;
    float part[B];
    if (active && row < p.n) {
      chunk_dot<FMT, CW, B>(raw[pi], c, xp, lut, part);
      const float s = f16_to_f32(raw[pi].s);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[pi][b] = s * (part[b] - xs[b]);
    } else {
#pragma unroll
      for (int b = 0; b < B; ++b) acc[pi][b] = 0.0f;
    }
  }

  // Reduce within 16-lane segments, then across the team's segments.
  const int seg = t >> 4;
#pragma unroll
  for (int pi = 0; pi < P; ++pi) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = acc[pi][b];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 1, 64);
      if ((t & 15) == 0) red[(pi * B + b) * 64 + seg] = v;
    }
  }
  __syncthreads();
  const int segs_per_team = cseg >> 4;
  for (int o = t; o < P * teams * B; o += blockDim.x) {
    const int pi = o / (teams * B);
    const int rem = o % (teams * B);
    const int tm = rem / B, b = rem % B;
    const int64_t row = row0 + (int64_t)pi * teams + tm;
    if (row >= p.n || b >= batch) continue;
    float sum = 0.0f;
    const float *rp = red + (pi * B + b) * 64 + tm * segs_per_team;
    for (int sgi = 0; sgi < segs_per_team; ++sgi) sum += rp[sgi];
    y[b * ldy + row] = sum;
  }
}

template <int FMT, int CW, int B, int P>
static hipError_t gemv_go(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                          float *y, int64_t ldy, hipStream_t st) {
  const int chunks = (int)(p.k / CW);
  const int cseg = (chunks + 15) / 16 * 16;
  // teams per workgroup: fewest idle lanes, then the smallest workgroup
  int best_r = 1;
  double best_eff = -1.0;
  for (int r = 1; r * cseg <= 1024; ++r) {
    const int threads = (r * cseg + 63) / 64 * 64;
    const double eff = (double)(r * cseg) / threads;
    if (eff > best_eff + 1e-9) { best_eff = eff; best_r = r; }
    if (r * cseg >= 640) break;
  }
  const int threads = (best_r * cseg + 63) / 64 * 64;
  const int64_t rows_per_wg = (int64_t)best_r * P;
  dim3 grid((unsigned)((p.n + rows_per_wg - 1) / rows_per_wg)), block(threads);
  hipLaunchKernelGGL((gemv_kernel<FMT, CW, B, P>), grid, block, 0, st, p, x, xd, batch, ldx, y,
                     ldy, chunks, cseg, best_r);
  return hipGetLastError();
}

// Largest supported k: a team of at most 1024 lanes must cover a row.
int64_t gemv_max_k(int fmt) { return fmt == FMT_PQ2 ? 64 * 1024 : 32 * 1024; }

// Lane chunk (CW weights), batch tile (B) and rows per thread (P) by batch:
// smaller chunks and fewer rows at larger batch keep the activation pairs
// (B * CW / 2 registers) and partial sums in registers without spilling.
hipError_t launch_gemv(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                       float *y, int64_t ldy, hipStream_t st) {
  if (p.fmt == FMT_PTQ1) {
    if (batch <= 1) return gemv_go<FMT_PTQ1, 32, 1, 4>(p, x, xd, batch, ldx, y, ldy, st);
    if (batch <= 2) return gemv_go<FMT_PTQ1, 32, 2, 4>(p, x, xd, batch, ldx, y, ldy, st);
    if (batch <= 4) return gemv_go<FMT_PTQ1, 32, 4, 2>(p, x, xd, batch, ldx, y, ldy, st);
    return gemv_go<FMT_PTQ1, 32, 8, 1>(p, x, xd, batch, ldx, y, ldy, st);
  }
  // a chunk never spans two groups (64 | 128); wide rows need wider chunks
  const bool wide32 = p.k / 32 > 1024, wide16 = p.k / 16 > 1024;
  if (batch <= 1 || (wide32 && batch <= 2))
    return gemv_go<FMT_PQ2, 64, 1, 4>(p, x, xd, batch, ldx, y, ldy, st) ;
  if (wide32) {
    if (batch <= 2) return gemv_go<FMT_PQ2, 64, 2, 2>(p, x, xd, batch, ldx, y, ldy, st);
    if (batch <= 4) return gemv_go<FMT_PQ2, 64, 4, 1>(p, x, xd, batch, ldx, y, ldy, st);
    return gemv_go<FMT_PQ2, 64, 8, 1>(p, x, xd, batch, ldx, y, ldy, st);
  }
  if (batch <= 2) return gemv_go<FMT_PQ2, 32, 2, 4>(p, x, xd, batch, ldx, y, ldy, st);
  if (batch <= 4) return gemv_go<FMT_PQ2, 32, 4, 2>(p, x, xd, batch, ldx, y, ldy, st);
  if (wide16) return gemv_go<FMT_PQ2, 32, 8, 1>(p, x, xd, batch, ldx, y, ldy, st);
  return gemv_go<FMT_PQ2, 16, 8, 2>(p, x, xd, batch, ldx, y, ldy, st);
}

}  // namespace tq
