// Decode GEMV over row-split ternary planes:
//   y[b][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * x'[b][j]
// [gguf-explainer] §4.3 (code semantics: value = (code - 1) * d with one
// scale per group); [ninfer-skill] §3 (planes).  This file holds the
// persistent team kernel that serves the shapes the batch-1 wave kernel and
// the row-quad kernel do not (rows longer than they hold), and the dispatch
// of tq_gemv_rowsplit among the three.
//
// Design of the team kernel (gfx950, wave64):
//  * Every thread owns one fixed K-chunk of the row ("lane chunk") and keeps
//    the matching activations in registers as binary16 pairs, so weights are
//    the only data streamed from HBM; a team of ceil(C/16)*16 threads covers
//    the C chunks of one row and a workgroup holds R teams.
//  * Codes become exact binary16 trits: a code ORed into the mantissa of
//    1024 and one packed fma give code - 1 (trit_pair), consumed by
//    v_dot2_f32_f16 with fp32 accumulation.  Zero weights contribute exact
//    zeros, so the rounding error follows sum |w x'| alone.
//  * PTQ1_0 bytes (five radix-3 digits) go through a 256-entry LDS table
//    whose entries hold the digits as 2-bit codes, decoded the same way.
//  * Partial sums are reduced across 16-lane segments with lane shuffles and
//    across segments through LDS in a fixed order (no atomics: bitwise
//    reproducible).

#include "tq_device.h"
#include "tq_gemv_f4.h"
#include "tq_gemv_wave.h"
#include "tq_launch.h"

namespace tq {

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

__device__ __forceinline__ half2_t pack_h2(float a, float b) {
  half2_t r;
  r.x = (_Float16)a;
  r.y = (_Float16)b;
  return r;
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
// weight pairs (binary16-rounded).
template <int FMT, int CW, int XD>
__device__ __forceinline__ void convert_x_chunk(const XRaw<FMT, CW, XD> &r, int64_t c,
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

// sum_j t_j * x_j over one lane chunk, with the trits t = code - 1 made
// exact binary16 values first (trit_pair), so that zero weights add nothing.
template <int FMT, int CW, int B>
__device__ __forceinline__ void chunk_dot(const Raw<FMT, CW> &r, int64_t c,
                                          const half2_t (&xp)[B][CW / 2],
                                          const uint32_t *lut, float part[B]) {
  const uint32_t magic = 0x64006400u;  // 1024.0 in each half
  float a[B][4];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) a[b][e] = 0.0f;
  if constexpr (FMT == FMT_PQ2) {
    // codes 0..4 of each half in place (slots 0..4), codes 5..7 shifted
    // down by 10 (slots 0..2): pair e holds the codes (e, e+8) of the dword
#pragma unroll
    for (int d = 0; d < CW / 16; ++d) {
      const uint32_t w = r.w[d], w10 = w >> 10;
      const uint32_t t[8] = {trit_pair<0>(w, magic), trit_pair<1>(w, magic), trit_pair<2>(w, magic),
                             trit_pair<3>(w, magic), trit_pair<4>(w, magic), trit_pair<0>(w10, magic),
                             trit_pair<1>(w10, magic), trit_pair<2>(w10, magic)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int b = 0; b < B; ++b)
          a[b][e & 3] = dot2(bits_h2(t[e]), xp[b][8 * d + e], a[b][e & 3]);
      }
    }
  } else {
    const int q = (int)(c & 3);
    // the lane's 6 base bytes start 0 or 2 bytes into the loaded window
    const uint64_t win = ((uint64_t)r.w[1] << 32) | r.w[0];
    const uint64_t bytes = (q & 1) ? (win >> 16) : win;
    // lut[v]: the five radix-3 digits of byte v as 2-bit codes, digit i at
    // bits 2i.  Two bytes side by side (second one shifted up 16) give, for
    // each digit i, a pair of codes in slot i: one trit pair per two trits.
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) {
      const uint32_t dw = lut[(bytes >> (16 * pp)) & 0xFF] |
                          (lut[(bytes >> (16 * pp + 8)) & 0xFF] << 16);
      const uint32_t t[5] = {trit_pair<0>(dw, magic), trit_pair<1>(dw, magic), trit_pair<2>(dw, magic),
                             trit_pair<3>(dw, magic), trit_pair<4>(dw, magic)};
#pragma unroll
      for (int i = 0; i < 5; ++i) {
#pragma unroll
        for (int b = 0; b < B; ++b)
          a[b][(5 * pp + i) & 3] = dot2(bits_h2(t[i]), xp[b][5 * pp + i], a[b][(5 * pp + i) & 3]);
      }
    }
    // the chunk's two high trits: digits 2(q&1) and 2(q&1)+1 of its high
    // byte, placed as a slot-0 pair
    const uint32_t wh = lut[r.h & 0xFF] >> (4 * (q & 1));
    const uint32_t th = trit_pair<0>((wh & 3u) | ((wh & 0xCu) << 14), magic);
#pragma unroll
    for (int b = 0; b < B; ++b) a[b][3] = dot2(bits_h2(th), xp[b][15], a[b][3]);
  }
#pragma unroll
  for (int b = 0; b < B; ++b) part[b] = (a[b][0] + a[b][1]) + (a[b][2] + a[b][3]);
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
  // activation pairs of every chunk in decode order: staged once per
  // workgroup (teams share chunks)
  extern __shared__ uint32_t xlds[];  // [chunk][CW/2 pairs] (one batch row)

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
  const int64_t cc = c < chunks ? c : 0;
  if constexpr (FMT == FMT_PTQ1) __syncthreads();  // tables ready
#pragma unroll
  for (int b = 0; b < B; ++b) {
    if (b < batch) {
      for (int i = t; i < chunks; i += blockDim.x) {
        XRaw<FMT, CW, XD> xr;
        load_x_raw<FMT, CW, XD>(x, b * ldx, i, xr);
        half2_t xp1[CW / 2];
        convert_x_chunk<FMT, CW, XD>(xr, i, xp1);
        uint32_t *dst = xlds + (int64_t)i * (CW / 2);
#pragma unroll
        for (int k = 0; k < CW / 2; k += 4)
          *reinterpret_cast<u32x4 *>(dst + k) = (u32x4){
              __builtin_bit_cast(uint32_t, xp1[k]), __builtin_bit_cast(uint32_t, xp1[k + 1]),
              __builtin_bit_cast(uint32_t, xp1[k + 2]), __builtin_bit_cast(uint32_t, xp1[k + 3])};
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
        const float v = seg_sum<SEG>(ok ? s * part[b] : 0.0f);
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

template <int A, int BQ, bool FUSED>
static hipError_t gemv_wave_dt(const Planes &p, const void *x, int xd, const uint16_t *signs,
                               float *y, hipStream_t st, const StepArgs &sa) {
  if (xd == DT_F32) return gemv_wave_go<LAY_PLANES, A, BQ, DT_F32, FUSED>(p, x, signs, y, st, sa);
  if (xd == DT_BF16) return gemv_wave_go<LAY_PLANES, A, BQ, DT_BF16, FUSED>(p, x, signs, y, st, sa);
  return gemv_wave_go<LAY_PLANES, A, BQ, DT_F16, FUSED>(p, x, signs, y, st, sa);
}

template <bool FUSED>
static hipError_t gemv_wave(const Planes &p, const void *x, int xd, const uint16_t *signs, float *y,
                            hipStream_t st, const StepArgs &sa = StepArgs{}) {
  switch (p.k / 1024) {
    case 1: return gemv_wave_dt<0, 1, FUSED>(p, x, xd, signs, y, st, sa);
    case 2: return gemv_wave_dt<0, 2, FUSED>(p, x, xd, signs, y, st, sa);
    case 3: return gemv_wave_dt<0, 3, FUSED>(p, x, xd, signs, y, st, sa);
    case 4: return gemv_wave_dt<1, 0, FUSED>(p, x, xd, signs, y, st, sa);
    case 5: return gemv_wave_dt<1, 1, FUSED>(p, x, xd, signs, y, st, sa);
    case 6: return gemv_wave_dt<1, 2, FUSED>(p, x, xd, signs, y, st, sa);
    case 7: return gemv_wave_dt<1, 3, FUSED>(p, x, xd, signs, y, st, sa);
    case 8: return gemv_wave_dt<2, 0, FUSED>(p, x, xd, signs, y, st, sa);
    case 9: return gemv_wave_dt<2, 1, FUSED>(p, x, xd, signs, y, st, sa);
    case 10: return gemv_wave_dt<2, 2, FUSED>(p, x, xd, signs, y, st, sa);
    case 11: return gemv_wave_dt<2, 3, FUSED>(p, x, xd, signs, y, st, sa);
    default: break;
  }
  if constexpr (!FUSED) {
    switch (p.k / 1024) {
      case 12: return gemv_wave_dt<3, 0, false>(p, x, xd, signs, y, st, sa);
      case 13: return gemv_wave_dt<3, 1, false>(p, x, xd, signs, y, st, sa);
      case 14: return gemv_wave_dt<3, 2, false>(p, x, xd, signs, y, st, sa);
      case 15: return gemv_wave_dt<3, 3, false>(p, x, xd, signs, y, st, sa);
      case 16: return gemv_wave_dt<4, 0, false>(p, x, xd, signs, y, st, sa);
      default: return gemv_wave_dt<4, 1, false>(p, x, xd, signs, y, st, sa);
    }
  }
  return hipErrorInvalidValue;  // not reached: the fused step is checked for m <= 11
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
  const size_t lds = (size_t)chunks * (CW / 2) * 4;
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

// Lane chunk (CW weights), batch tile (B) and rows per thread (P) by batch:
// smaller chunks and fewer rows at larger batch keep the activation pairs
// (B * CW / 2 registers) and partial sums in registers without spilling.
hipError_t launch_gemv(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                       float *y, int64_t ldy, hipStream_t st) {
  if (p.fmt == FMT_PTQ1) {
    if (gemv_quads_fits(p)) return launch_gemv_quads(p, x, xd, batch, ldx, y, ldy, st);
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
  if (batch >= 2 && gemv_quads_fits(p)) return launch_gemv_quads(p, x, xd, batch, ldx, y, ldy, st);
  if (batch <= 1 && gemv_f4_fits(p)) return launch_gemv_f4(p, x, xd, nullptr, y, MODE_GEMV, StepArgs{}, st);
  if (batch <= 1 && gemv_wave_fits(p, false)) return gemv_wave<false>(p, x, xd, nullptr, y, st);
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

hipError_t launch_rotated_gemv(const Planes &p, const void *x, int xd, const uint16_t *signs,
                               float *y, hipStream_t st, int tiles, int groups, int head_dim) {
  StepArgs sa;
  sa.tiles = tiles;
  sa.groups = groups;
  sa.head_dim = head_dim;
  if (gemv_f4_fits(p)) return launch_gemv_f4(p, x, xd, signs, y, MODE_ROT, sa, st);
  return gemv_wave<true>(p, x, xd, signs, y, st, sa);
}

}  // namespace tq
