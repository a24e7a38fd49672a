// The batch-1 decode GEMV on the matrix cores (gfx950): PQ2_0 codes go to the
// fp8 x fp4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) as they are, and the
// activation row goes in as eight exact base-16 digits in fp8.
//
// Codes.  Masked with 0x33333333, every nibble of a code dword holds one
// 2-bit code in its low bits, which read as an fp4 (E2M1) number is code/2;
// shifted down two bits first, the same mask gives the other half of the
// dword's codes.  Two bit operations per 16 weights turn the weight stream
// into an MFMA operand; no conversion instruction touches it.
//
// Activations.  The instruction sums each block of 8 products in fixed point
// aligned to the block's largest product, keeping 13 bits below it, so a
// small product beside a large one loses its low bits.  The activation row
// x' (binary16) is therefore written as x' = U * sum_p 16^-p q_p with
// integer digits q_p in [-8, 8] (q_0 = rint(x'/U), each next digit the
// rounded remainder times 16) and a power of two U with max|x'| < 8U.
// Every digit is an exact fp8 (E4M3) value, every product code/2 * q a
// multiple of 1/2 below 12 in size, so each block sum is exact; eight
// digits carry 32 bits below 8U, which holds every binary16 element within
// 2^21 of the row maximum exactly (smaller ones to 2^-29 U).  The weight
// 2 U 16^-p of digit p travels in the instruction's per-row E8M0 scale.
//
// Layout of one MFMA (measured on gfx950 for fp8 A, fp4 B).  D[i][j] =
// sum_k A[i][k] B[k][j]; lane l of D holds rows 4(l/16)..+3 of column l%16.
// B column j is weight row j: lane (j, g = l/16) holds 32 codes of its row.
// A row i is (group side, digit): rows 0-3 and 8-11 are digits 0-3 and 4-7
// of the even group, rows 4-7 and 12-15 those of the odd group.  A lane
// (i, gA) byte r multiplies B lane group 2(r/16) + gA/2, nibble
// r%16 + 16(gA%2); so the even group's digits sit in A lanes gA = 0, 1, the
// odd group's in gA = 2, 3, and the other half of every A lane is zero.
// Per 512-weight line u of a row (groups 4u..4u+3) lane (j, g) takes two
// 16-byte pieces L = 0, 1 of row j: bytes 64L + 32(g%2) + 16(g/2), i.e.
// half g/2 of group 4u + 2L + g%2, and each piece feeds a chain of two MFMAs
// (m = 0, 1: code dwords 2m, 2m+1, as fp4 dwords even(2m), odd(2m),
// even(2m+1), odd(2m+1) -- even/odd: the dword's codes 4b, 4b+2 or 4b+1,
// 4b+3).  D lane group g then holds four digits of the group its own piece
// came from, so it folds the chain with that group's scale:
// acc += s * sum_v (D[v] - X[v]), where X is the chain's value on all-ones
// codes (every weight 0), computed once per launch by the same MFMAs on the
// same A operands ([gguf-explainer] §4.4 offset form).  The chain starts
// from -X instead of 0: every sum the instruction forms is exact, so it ends
// at D - X exactly, an all-zero group adds exactly 0 and an all-zero row is
// exactly 0.

// Work split.  A wave owns blocks of 16T consecutive rows (T tiles of 16);
// per line u it reads the A operands once from LDS and runs T tiles with
// them.  Its loads (two code loads per tile and line, one scale load per
// round of UD lines) run one round (DEP = UD*T slots) ahead in a ring that
// continues into the wave's next block, so the stream never drains between
// blocks.

#pragma once

#include "tq_device.h"
#include "tq_gemv_wave.h"
#include "tq_launch.h"

namespace tq {

typedef int i32x8_f4 __attribute__((ext_vector_type(8)));
typedef float f32x4_f4 __attribute__((ext_vector_type(4)));

// LDS table of A operands: per line u, blocks (L, m, c) of 32 lane slots of
// 16 bytes (slot gA*8 + digit, at byte 16 + 16 slot) between two zero slots
// read by the lanes whose half is empty.  A 16-byte LDS read serves 16
// lanes (one lane group) per pass from 64 four-byte banks: the active lanes
// of group gA read slots 8gA..8gA+7, banks 32(gA%2)+4..+35 of the block, so
// the even groups' empty lanes read the zero slot at byte 0 (banks 0-3) and
// the odd groups' the one at byte 528 (banks 4-7), away from their data.
constexpr int F4_BLOCK = 34 * 16;
constexpr int F4_UNIT = 8 * F4_BLOCK;

__device__ __forceinline__ f32x4_f4 mfma_f4(const i32x8_f4 &a, const i32x8_f4 &b, const f32x4_f4 &c,
                                            int scale_a) {
  // A fp8 (E4M3), B fp4 (E2M1); A scaled per row by 2^(scale_a - 127), B by 1
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, scale_a, 0, 127);
}

// the two B operands of one 16-byte code load (see the layout above)
__device__ __forceinline__ void f4_codes(const u32x4 &w, i32x8_f4 &b0, i32x8_f4 &b1) {
  const uint32_t m = 0x33333333u;
  b0 = (i32x8_f4){(int)(w[0] & m), (int)((w[0] >> 2) & m), (int)(w[1] & m), (int)((w[1] >> 2) & m), 0, 0, 0, 0};
  b1 = (i32x8_f4){(int)(w[2] & m), (int)((w[2] >> 2) & m), (int)(w[3] & m), (int)((w[3] >> 2) & m), 0, 0, 0, 0};
}

// Per wave, used in the main loop only (so it shares its space with the
// binary16 activations of the prologue):
//  - the code tile: one 64-byte half of a slot's 16 rows, chunk q of row r
//    at 64r + 16(q ^ (r/4 % 4)), so that the quad writes (rows 4a..4a+3 per
//    pass) and the MFMA-layout reads (rows 0..15 of one chunk per pass)
//    both meet 16 distinct bank quadruples;
//  - the scale tile of the block being consumed: its rows' scale bytes as
//    they lie in the scale plane (16T rows of k/64 bytes), at most 3 KiB.
constexpr int F4_STAGE_CODES = 16 * 64;
constexpr int F4_STAGE_SCALES = 3 * 1024;
constexpr int F4_STAGE = F4_STAGE_CODES + F4_STAGE_SCALES;

// LDS bytes of the kernel for rows of k weights
inline size_t gemv_f4_lds(int64_t k, int wpg) {
  const int64_t nu = k / 512;
  const int64_t stage = (int64_t)F4_STAGE * wpg;
  return (size_t)(nu * F4_UNIT + nu * 8 * 16 + 16 * wpg + (stage > 2 * k ? stage : 2 * k));
}

// An empty statement that reads and rewrites v: the loads that produce v
// stay ahead of it in program order (with a conditional use only, the
// compiler may move them into the branch, behind later loads, so that
// waiting for them also waits for those).
__device__ __forceinline__ void f4_keep(u32x4 &v) { asm volatile("" : "+v"(v)); }

// Lane reductions with DPP row operations and lane reads (the generic
// shuffle goes through LDS and waits for it at every step).
template <int CTRL>
__device__ __forceinline__ float f4_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float f4_lane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// the wave's maximum / sum, in every lane
__device__ __forceinline__ float f4_wave_max(float v) {
  v = __builtin_fmaxf(v, f4_dpp<0xB1>(v));
  v = __builtin_fmaxf(v, f4_dpp<0x4E>(v));
  v = __builtin_fmaxf(v, f4_dpp<0x104>(v));
  v = __builtin_fmaxf(v, f4_dpp<0x108>(v));  // row_shl:8
  return __builtin_fmaxf(__builtin_fmaxf(f4_lane(v, 0), f4_lane(v, 16)), __builtin_fmaxf(f4_lane(v, 32), f4_lane(v, 48)));
}
__device__ __forceinline__ float f4_wave_sum(float v) {
  v += f4_dpp<0xB1>(v);
  v += f4_dpp<0x4E>(v);
  v += f4_dpp<0x104>(v);
  v += f4_dpp<0x108>(v);
  return (f4_lane(v, 0) + f4_lane(v, 16)) + (f4_lane(v, 32) + f4_lane(v, 48));
}

struct F4Slot {
  u32x4 c0, c1;  // code loads L = 0, 1
};

template <int XD, int MODE, int T, int UD, int WPG>
__global__ __launch_bounds__(64 * WPG) void gemv_f4_kernel(Planes p, const void *__restrict__ x,
                                                           const uint16_t *__restrict__ signs,
                                                           float *__restrict__ y, StepArgs hd) {
  constexpr bool FUSED = MODE != MODE_GEMV;
  constexpr bool HEAD = MODE == MODE_HEAD;
  constexpr int DEP = UD * T;
  constexpr int RB = 16 * T;  // rows per block
  extern __shared__ __attribute__((aligned(16))) uint8_t f4_lds[];
  const int NU = (int)(p.k >> 9);
  const int NB = (int)(p.k >> 10);
  uint8_t *tab = f4_lds;
  f32x4_f4 *xt = reinterpret_cast<f32x4_f4 *>(f4_lds + NU * F4_UNIT);
  float *red = reinterpret_cast<float *>(xt + NU * 8);
  unsigned long long *wbest = reinterpret_cast<unsigned long long *>(red + 2 * WPG);
  uint8_t *stage = reinterpret_cast<uint8_t *>(wbest + WPG);
  uint16_t *xh = reinterpret_cast<uint16_t *>(stage);
  static_assert(UD == 2, "the scale tile of a round is 16 bytes per row");
  static_assert(T <= 4, "one scale load per round covers at most 64 rows");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  u32x4 *st = reinterpret_cast<u32x4 *>(stage + F4_STAGE * wave);                   // code tile
  uint8_t *sct = stage + F4_STAGE * wave + F4_STAGE_CODES;                          // scale tile

  // ---- the wave's rows and its load ring
  const int n32 = (int)p.n;
  const int nblk = (n32 + RB - 1) / RB;
  const int W = (int)gridDim.x * WPG;
  const int gw = (int)blockIdx.x * WPG + wave;
  const int NR = NU / UD;  // rounds per block
  const int gbytes = 2 * (int)p.groups;
  // buffer resources of a block: rows past n read as zero and cost no traffic
  auto code_rsrc = [&](int blk) {
    const int rows = blk < nblk ? (n32 - blk * RB < RB ? n32 - blk * RB : RB) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.base + (int64_t)blk * RB * p.base_row), 0,
                                             rows * (int)p.base_row, 0x00020000);
  };
  auto scale_rsrc = [&](int blk) {
    const int rows = blk < nblk ? (n32 - blk * RB < RB ? n32 - blk * RB : RB) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.scale + (int64_t)blk * RB * p.groups), 0, rows * gbytes, 0x00020000);
  };
  // ---- 1. x' as binary16 in LDS, natural order.  The activation loads go
  // out first and the ring's first loads right after them, so the weights
  // stream while the activations are staged, and waiting for the
  // activations does not wait for the weights.
  const int tid = threadIdx.x;
  F4Slot ring[DEP];
  // Code loads run in quads: lane 4r + q reads 16-byte chunk q of the
  // 64-byte half of row r, so every four lanes read one contiguous 64-byte
  // piece (a lane per row, in the MFMA layout, would split each load into 64
  // scattered pieces).  The wave then moves the chunks through its LDS tile
  // into the MFMA layout (lane (j, g) takes chunk 2(g%2) + g/2 of row j).
  const int ld_row = lane >> 2, ld_q = lane & 3;
  auto load_slot = [&](F4Slot &s, __amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int u, int t) {
    const int vo = (16 * t + ld_row) * (int)p.base_row + 16 * ld_q;
    s.c0 = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, 128 * u, 0);
    s.c1 = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, 128 * u + 64, 0);
  };
  // A block's scale tile (16T rows of k/64 bytes, contiguous in the scale
  // plane) in three contiguous kilobyte loads, issued with the refills of
  // the round before the block's first and kept in registers until that
  // round.  Every round issues the three loads so that the count of loads
  // in flight is the same in every round; in the other rounds they point
  // past the buffer's end, which returns zero and fetches nothing.
  u32x4 stl[3];
  auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, bool real) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
      stl[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, real ? 16 * lane + 1024 * i : 0x7FFFFFF0, 0, 0);
  };
  // h[m]: binary16 elements 2m, 2m+1 of the thread's chunk x'[16c..16c+15]
  // (c = thread index; k <= 16 * 64 * WPG)
  const int c = tid;
  const bool mine = c < (int)(p.k >> 4);
  uint32_t h[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if constexpr (!FUSED) {
    Raw16<XD> xr;
    load16_raw<XD>(x, 16 * (int64_t)(mine ? c : 0), xr);
    __builtin_amdgcn_sched_barrier(0);
    {
      const auto rc = code_rsrc(gw), rs = scale_rsrc(gw);
#pragma unroll
      for (int d = 0; d < DEP; ++d) {
        load_slot(ring[d], rc, rs, d / T, d % T);
        if (d == 0) load_tile(rs, true);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int q = 0; q < (XD == DT_F32 ? 4 : 2); ++q) f4_keep(xr.q[q]);
    if constexpr (XD == DT_F16) {
#pragma unroll
      for (int m = 0; m < 4; ++m) { h[m] = xr.q[0][m]; h[4 + m] = xr.q[1][m]; }
    } else {
      float v[16];
      convert16<XD>(xr, v);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        h[m] = (uint32_t)f32_to_f16(v[2 * m]) | ((uint32_t)f32_to_f16(v[2 * m + 1]) << 16);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) h[m] = mine ? h[m] : 0u;
  } else {
    // the signed transform of one 1024-element block per wave (k <= 1024 *
    // WPG), as the wave kernel does it, the wave's scratch in the table's
    // space; x' goes through LDS to the threads that own its chunks
    const int blk1 = wave;
    const bool tw = blk1 < NB;
    const int64_t e = (int64_t)(tw ? blk1 : 0) * 1024 + 16 * lane;
    Raw16<XD> xr;
    if constexpr (MODE == MODE_ROT)
      load16_raw<XD>(x, hd.tiles ? (int64_t)head_src((int)e, hd.tiles, hd.groups, hd.head_dim) : e, xr);
    else
      load16_raw<XD>(x, e, xr);
    const u32x4 *sp = reinterpret_cast<const u32x4 *>(signs + e);
    u32x4 s0 = sp[0], s1 = sp[1];
    u32x4 g0 = {0u, 0u, 0u, 0u}, g1 = {0u, 0u, 0u, 0u};
    if constexpr (HEAD) {
      const u32x4 *gp = reinterpret_cast<const u32x4 *>(hd.g + e);
      g0 = gp[0];
      g1 = gp[1];
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      const auto rc = code_rsrc(gw), rs = scale_rsrc(gw);
#pragma unroll
      for (int d = 0; d < DEP; ++d) {
        load_slot(ring[d], rc, rs, d / T, d % T);
        if (d == 0) load_tile(rs, true);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int q = 0; q < (XD == DT_F32 ? 4 : 2); ++q) f4_keep(xr.q[q]);
    f4_keep(s0);
    f4_keep(s1);
    if constexpr (HEAD) {
      f4_keep(g0);
      f4_keep(g1);
    }
    float v[16];
    float sq = 0.0f;
    convert16<XD>(xr, v);
    if constexpr (HEAD) {
#pragma unroll
      for (int q = 0; q < 16; ++q) sq = __builtin_fmaf(v[q], v[q], sq);
      sq = tw ? sq : 0.0f;
      const uint32_t gw8[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] *= bf16_to_f32((uint16_t)(gw8[q >> 1] >> (16 * (q & 1))));
    }
    {
      const uint32_t sw[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = apply_sign(v[q], (uint16_t)(sw[q >> 1] >> (16 * (q & 1))));
    }
    if (tw) wht1024_wave(v, lane, reinterpret_cast<float *>(tab) + WHT_SCRATCH * wave);
    float post = 0.03125f;
    if constexpr (HEAD) {
      sq = f4_wave_sum(sq);
      if (lane == 0) red[wave] = sq;
      __syncthreads();
      float tot = 0.0f;
      const int nst = NB < WPG ? NB : WPG;
      for (int w = 0; w < nst; ++w) tot += red[w];
      post = 0.03125f / __builtin_sqrtf(tot / (float)(NB * 1024) + hd.eps);
    }
    // x' as binary16 to LDS, and the block's largest finite |x'| (the
    // barrier that publishes x' publishes the maxima too)
    float mxl = 0.0f;
    if (tw) {
      uint16_t *o = xh + blk1 * 1024;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint16_t e4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          e4[e] = f32_to_f16(v[4 * q + e] * post);
          const float a = __builtin_fabsf(f16_to_f32(e4[e]));
          mxl = (a <= 65504.0f && a > mxl) ? a : mxl;
        }
        *reinterpret_cast<u32x2 *>(o + 256 * q + 4 * lane) =
            (u32x2){(uint32_t)e4[0] | ((uint32_t)e4[1] << 16), (uint32_t)e4[2] | ((uint32_t)e4[3] << 16)};
      }
    }
    mxl = f4_wave_max(mxl);
    if (lane == 0) red[WPG + wave] = mxl;
    __syncthreads();
    if (mine) {
      const u32x4 *q = reinterpret_cast<const u32x4 *>(xh + 16 * c);
      const u32x4 a0 = q[0], a1 = q[1];
#pragma unroll
      for (int m = 0; m < 4; ++m) { h[m] = a0[m]; h[4 + m] = a1[m]; }
    }
  }

  // ---- 2. U: the power of two with max|x'| < 8U over the finite elements
  // (the fused modes found their maxima with the transform)
  if constexpr (!FUSED) {
    float mx = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float a = __builtin_fabsf(f16_to_f32((uint16_t)h[m]));
      const float b = __builtin_fabsf(f16_to_f32((uint16_t)(h[m] >> 16)));
      mx = (a <= 65504.0f && a > mx) ? a : mx;
      mx = (b <= 65504.0f && b > mx) ? b : mx;
    }
    mx = f4_wave_max(mx);
    if (lane == 0) red[WPG + wave] = mx;
    __syncthreads();
  }
  float mx = 0.0f;
#pragma unroll
  for (int w = 0; w < WPG; ++w) mx = __builtin_fmaxf(mx, red[WPG + w]);
  // max < 2^E (E from the float's exponent); U = 2^(E-3)
  const int E = mx > 0.0f ? (int)((__float_as_uint(mx) >> 23) & 0xFF) - 126 : 0;
  const float inv_u = __builtin_ldexpf(1.0f, 3 - E);

  // ---- 3. the digit table.  Thread c's 16 elements form chunk (u, L, m,
  // half, gA) = (c/32, c/16 % 2, c/2 % 2, c/4 % 2, 2(c/8 % 2) + c % 2) of
  // the table: byte b of a slot holds element 16c + 2(b % 8) + b/8 (the
  // order f4_codes gives the codes).
  {
    float r[16];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float lo = f16_to_f32((uint16_t)h[m]), hi = f16_to_f32((uint16_t)(h[m] >> 16));
      r[m] = __builtin_fabsf(lo) <= 65504.0f ? lo * inv_u : __builtin_nanf("");
      r[8 + m] = __builtin_fabsf(hi) <= 65504.0f ? hi * inv_u : __builtin_nanf("");
    }
    const int grp = c >> 3;
    const int gA = 2 * (grp & 1) + (c & 1);
    uint8_t *blk = tab + (c >> 5) * F4_UNIT + ((((c >> 4) & 1) * 2 + ((c >> 1) & 1)) * 2 + ((c >> 2) & 1)) * F4_BLOCK +
                   16 + gA * 8 * 16;
    if (mine) {
      // one digit per pass (unrolled, the passes would hold every digit's
      // temporaries at once and cost the main loop its occupancy)
#pragma unroll 1
      for (int d = 0; d < 8; ++d) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float qq[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qq[e] = __builtin_rintf(r[4 * q + e]);
            r[4 * q + e] = (r[4 * q + e] - qq[e]) * 16.0f;
          }
          int pk = __builtin_amdgcn_cvt_pk_fp8_f32(qq[0], qq[1], 0, false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(qq[2], qq[3], pk, true);
          w[q] = (uint32_t)pk;
        }
        *reinterpret_cast<u32x4 *>(blk + d * 16) = (u32x4){w[0], w[1], w[2], w[3]};
      }
    }
  }
  // zero slots
  for (int z = tid; z < NU * 16; z += 64 * WPG)
    *reinterpret_cast<u32x4 *>(tab + (z >> 4) * F4_UNIT + ((z >> 1) & 7) * F4_BLOCK + (z & 1) * 33 * 16) =
        (u32x4){0u, 0u, 0u, 0u};
  __syncthreads();

  // ---- 4. the lane's A slot and its row's digit scale
  const bool act = ((j >> 2) & 1) == (g >> 1);
  const int a_off = act ? 16 + (g * 8 + (j & 3) + 4 * (j >> 3)) * 16 : (g & 1) * 33 * 16;
  const int sa = 127 + E - 2 - 4 * ((j & 3) + 4 * (j >> 3));
  auto read_a = [&](int u, int L, int m) -> i32x8_f4 {
    const uint8_t *b = tab + u * F4_UNIT + (L * 2 + m) * 2 * F4_BLOCK + a_off;
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(b);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(b + F4_BLOCK);
    return (i32x8_f4){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  // ---- the all-ones sums X: per line u and piece L, the chain of its two
  // MFMAs on all-ones codes (every weight 0).  It is the main loop's chain on
  // the main loop's operands, kept negated as the main loop's starting
  // value; lane (0, g) keeps digits 4(g/2)..+3 of group 4u + 2L + g%2.
  {
    const i32x8_f4 ones = {0x11111111, 0x11111111, 0x11111111, 0x11111111, 0, 0, 0, 0};
    const f32x4_f4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int pr = wave; pr < 2 * NU; pr += WPG) {
      const int u = pr >> 1, L = pr & 1;
      f32x4_f4 d = mfma_f4(read_a(u, L, 0), ones, z4, sa);
      d = mfma_f4(read_a(u, L, 1), ones, d, sa);
      if (j == 0) xt[(4 * u + 2 * L + (g & 1)) * 2 + (g >> 1)] = -d;
    }
  }
  __syncthreads();

  // ---- 5. the blocks, as one flat sequence of rounds: round q of the wave
  // is line group r = q % NR of its block gw + (q / NR) W, and the ring's
  // refills during round q load round q + 1
  const int ssh = 16 * (g & 1);
  const int rd_q = 2 * (g & 1) + (g >> 1);
  // results: a buffer over y, so that the rows past n of the last block are
  // dropped by the store itself and every block issues the same stores
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc(y, 0, (HEAD && y == nullptr) ? 0 : 4 * n32, 0x00020000);
  unsigned long long best = 0;
  const int nmine = gw < nblk ? (nblk - 1 - gw) / W + 1 : 0;
  const int rounds = nmine * NR;
  int blk = gw, r = 0;       // the round being consumed
  int tb = gw, tr = 0;       // the round the refills load
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
  for (int q = 0; q < rounds; ++q) {
    tr = tr + 1 == NR ? 0 : tr + 1;
    tb = tr == 0 ? tb + W : tb;
    const auto rc = code_rsrc(tb), rs = scale_rsrc(tb);
    // a block's first round: its scale tile, loaded with the previous
    // round, to LDS
    if (r == 0) {
      u32x4 *o = reinterpret_cast<u32x4 *>(sct);
#pragma unroll
      for (int i = 0; i < 3; ++i) o[64 * i + lane] = stl[i];
    }
#pragma unroll
    for (int ud = 0; ud < UD; ++ud) {
      const int u = r * UD + ud;
      const i32x8_f4 a00 = read_a(u, 0, 0), a01 = read_a(u, 0, 1);
      const i32x8_f4 a10 = read_a(u, 1, 0), a11 = read_a(u, 1, 1);
      // -X of the lane's group (4u + 2L + g%2) and digits: the chains'
      // starting values
      const f32x4_f4 x0 = xt[(4 * u + (g & 1)) * 2 + (g >> 1)], x1 = xt[(4 * u + 2 + (g & 1)) * 2 + (g >> 1)];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        F4Slot &s = ring[ud * T + t];
        i32x8_f4 b00, b01, b10, b11;
        // the two halves through the code tile, one after the other
        st[ld_row * 4 + (ld_q ^ ((ld_row >> 2) & 3))] = s.c0;
        const u32x4 c0 = st[j * 4 + (rd_q ^ (j >> 2))];
        st[ld_row * 4 + (ld_q ^ ((ld_row >> 2) & 3))] = s.c1;
        const u32x4 c1 = st[j * 4 + (rd_q ^ (j >> 2))];
        f4_codes(c0, b00, b01);
        f4_codes(c1, b10, b11);
        const u32x2 sv = *reinterpret_cast<const u32x2 *>(sct + (16 * t + j) * gbytes + 8 * u);
        const uint32_t s0 = sv[0], s1 = sv[1];
        f32x4_f4 d0 = mfma_f4(a00, b00, x0, sa);
        f32x4_f4 d1 = mfma_f4(a10, b10, x1, sa);
        d0 = mfma_f4(a01, b01, d0, sa);
        d1 = mfma_f4(a11, b11, d1, sa);
        const float z0 = (d0[0] + d0[1]) + (d0[2] + d0[3]);
        const float z1 = (d1[0] + d1[1]) + (d1[2] + d1[3]);
        acc[t] = __builtin_fmaf(f16_to_f32((uint16_t)(s0 >> ssh)), z0, acc[t]);
        acc[t] = __builtin_fmaf(f16_to_f32((uint16_t)(s1 >> ssh)), z1, acc[t]);
        // refill the slot only once all its registers are consumed, and
        // keep the refill here: a load into registers still in use, or
        // refills moved down together, make the next round wait for every
        // load in flight
        __builtin_amdgcn_sched_barrier(0);
        load_slot(s, rc, rs, tr * UD + ud, t);
        if (ud == 0 && t == 0) load_tile(rs, tr == 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (r + 1 == NR) {
      // rows of the block: lanes j, j+16, j+32, j+48 hold parts of row j;
      // after the two swaps all four hold its sum and store it
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float v = acc[t];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        const int row = blk * RB + 16 * t + j;
        if constexpr (HEAD) {
          if (row < n32) {
            const unsigned long long key = greedy_key(v, (uint32_t)row);
            best = key > best ? key : best;
          }
        }
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yr, 4 * row, 0, 0);
        acc[t] = 0.0f;
      }
      blk += W;
      r = 0;
    } else {
      ++r;
    }
  }

  if constexpr (HEAD) {
    uint32_t hi = (uint32_t)(best >> 32), lo = (uint32_t)best;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t ohi = (uint32_t)__shfl_xor((int)hi, o), olo = (uint32_t)__shfl_xor((int)lo, o);
      const bool take = ohi > hi || (ohi == hi && olo > lo);
      hi = take ? ohi : hi;
      lo = take ? olo : lo;
    }
    if (lane == 0) wbest[wave] = ((unsigned long long)hi << 32) | lo;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long m = 0;
#pragma unroll
      for (int w = 0; w < WPG; ++w) m = wbest[w] > m ? wbest[w] : m;
      head_finish(m, hd.work, hd.token);
    }
  }
}

}  // namespace tq

namespace tq {

// Whether the matrix-core GEMV takes a batch-1 request: PQ2_0 rows of a
// multiple of 1024 weights, at most 1024 per wave of a workgroup (the
// staging gives each wave one 1024-element block and each thread one
// 16-element chunk), whose LDS fits a compute unit, in a matrix of at
// least 2^29 weights.
bool gemv_f4_fits(const Planes &p);

// The batch-1 GEMV (mode MODE_GEMV), the fused signed transform + GEMV
// (MODE_ROT) or the output head with its greedy token (MODE_HEAD).
hipError_t launch_gemv_f4(const Planes &p, const void *x, int xd, const uint16_t *signs, float *y, int mode,
                          const StepArgs &hd, hipStream_t st);

}  // namespace tq
