// Decode GEMV on the matrix cores over row-quads, batch 1..8 per launch
// pass (PTQ1_0_G128 at every batch, PQ2_0_G128 at batch 2..8):
//   y[b][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * x'[b][j]
// [ninfer-skill] §2-§3 (row-split planes; PTQ1_0: 24 base bytes + 2 high
// bytes + one fp16 scale per 128 weights, PQ2_0: 32 base bytes + the
// scale); [gguf-explainer] §4.3 (PQ2_0 codes: weight j at byte j/4, bits
// 2*(j%4), value code-1).  The PTQ1_0 trit packing inside the bytes is this
// library's convention (five radix-3 digits per base byte, four per high
// byte, least significant digit first), stated in tq.h.
//
// Work split (gfx950, wave64).  A row of k weights is cut into 32-weight
// chunks: quarter q of group g holds, for PTQ1_0, base bytes 6q..6q+5
// (trits 30q..30q+29 of the group) and digits 2(q&1), 2(q&1)+1 of high byte
// q>>1 (trits 120+2q, 121+2q); for PQ2_0, base bytes 8q..8q+7 (weights
// 32q..32q+31).  A workgroup owns RQ consecutive row-quads (4 rows each)
// over the whole of k, so every CU gets the same number of rows and no
// result leaves the workgroup unfinished.  Its W waves split the chunks:
// lane l of wave w is lane j = l%4 of 4x4x4 MFMA block b = l/4 and owns
// chunks (w*S + s)*16 + b, s < S, for the whole kernel; chunk counts that
// do not fill W*S*16 slots leave "phantom" chunks with zero activations.
// The lane keeps the binary16 activations of its chunks for batch row j (and
// 4 + j when eight rows are in flight) in registers and streams, for each
// row-quad, the chunk bytes of weight row 4*rq + j.
//
// Decode: PTQ1_0 -- a 256-entry LDS table turns a byte into its five
// radix-3 digits as 2-bit codes at bits 2i; two bytes side by side give,
// per digit i, a pair of codes.  PQ2_0 -- a dword of 16 codes holds codes e
// and e+8 at bits 2e of its two halves (e <= 4; codes 5..7 and 13..15 after
// a shift by 10).  Either way one and-or places a code pair into the
// mantissa of binary16 1024 (1024 + 4^i * code) and one packed fma turns it
// into the trit pair code - 1 exactly.  v_mfma_f32_4x4x4_16b_f16 then multiplies block b's four batch
// rows (A, activations) by its four weight rows (B, trits) over 4 weights;
// eight MFMAs cover a chunk, after which the chunk's group scale is
// applied in fp32.  With eight batch rows a second set of eight MFMAs
// reuses the same decoded trits for rows 4..7: the decode (vector ALU) is
// what bounds the loop, so the second set costs little.  Partial sums are reduced over blocks with lane swaps
// and DPP, over waves through LDS in a fixed order (no atomics: bitwise
// reproducible).

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// One lane's view of a chunk as loaded: the 8-byte window holding its six
// base bytes, its group's high byte and scale bits.
struct ChunkRaw {
  uint32_t w0, w1, h, s;
};

// Sums of v[0..3] over the 16 blocks of a wave (lanes with equal l%4): two
// swap stages halve the values per lane while summing lane bits 5 and 4,
// two DPP rotates sum lane bits 3 and 2.  Lane l then holds the total for
// block lane j = l%4 and value index [0, 2, 1, 3][l >> 4].
__device__ __forceinline__ float blocks_sum4(const float (&v)[4]) {
  auto bits = [](float f) { return __builtin_bit_cast(unsigned, f); };
  auto flt = [](unsigned u) { return __builtin_bit_cast(float, u); };
  const auto a = __builtin_amdgcn_permlane32_swap(bits(v[0]), bits(v[1]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(bits(v[2]), bits(v[3]), false, false);
  const float s0 = flt(a[0]) + flt(a[1]);
  const float s1 = flt(b[0]) + flt(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(bits(s0), bits(s1), false, false);
  float x = flt(c[0]) + flt(c[1]);
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x124, 0xF, 0xF, false));  // row_ror:4
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x128, 0xF, 0xF, false));  // row_ror:8
  return x;
}

constexpr int RQMAX = 30;  // row-quads per workgroup

// Launch-time shape of one pass.
struct Ptq1Shape {
  int chunks;  // k / 32
  int rq;      // row-quads per workgroup (a multiple of RR)
};

template <int FMT, int S, int RR, int W, int XD, int BT>
__global__ __launch_bounds__(64 * W) void gemv_quads_kernel(Planes p, const void *__restrict__ x,
                                                           int64_t batch, int64_t ldx,
                                                           float *__restrict__ y, int64_t ldy,
                                                           Ptq1Shape sh) {
  constexpr int U = S * RR;  // steps per round (one ring of loads)
  constexpr int NG = BT == 8 ? 2 : 1;     // groups of four batch rows in flight
  constexpr int SB = BT == 1 ? 1 : 4;     // batch rows staged at a time
  __shared__ uint32_t lut[256];
  // per-wave activation staging (prologue), then the per-wave partial sums
  // [row-quad][wave][g*16 + j*4 + e] (epilogue)
  // Activation staging: per wave SB rows of XROW words, a row being the
  // slot's 512 activations as four groups of 64 words (128 activations),
  // group g at word XGRP*g.  PTQ1_0 pads the groups to 80 words and the rows
  // to 324 (4 mod 64), so that the 64 lanes' chunk reads (words 15q + t and
  // 60 + q of a group, for their row j, group and quarter q) meet 64
  // different banks; unpadded, the 16 lanes of one quarter share a bank.
  constexpr int XGRP = FMT == FMT_PTQ1 ? 80 : 64;
  constexpr int XROW = FMT == FMT_PTQ1 ? 324 : 256;
  constexpr int XST = W * SB * XROW * 4, RED = RQMAX * W * 16 * NG * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[XST > RED ? XST : RED];
  uint32_t *xst = reinterpret_cast<uint32_t *>(lds);
  float *red = reinterpret_cast<float *>(lds);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, blk = lane >> 2;
  const int n32 = (int)p.n;
  const int k32 = (int)p.k;
  const int rowq0 = (int)blockIdx.x * sh.rq;  // first row-quad of the workgroup

  // ---- the lane's chunks: byte offsets inside the row-quad's planes
  // (row j of the quad), fixed for the kernel
  int ob[S], oh[S], os[S];
  bool real[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c0 = (wave * S + s) * 16 + blk;
    real[s] = c0 < sh.chunks;
    const int c = real[s] ? c0 : 0;
    const int g = c >> 2, q = c & 3;
    if constexpr (FMT == FMT_PTQ1) {
      ob[s] = j * (int)p.base_row + g * 24 + ((6 * q) & ~3);
      oh[s] = j * (int)p.high_row + g * 2 + (q >> 1);
    } else {
      ob[s] = j * (int)p.base_row + g * 32 + 8 * q;
      oh[s] = 0;
    }
    os[s] = (j * (int)p.groups + g) * 2;
  }
  const int q = blk & 3;  // every chunk of this lane has the same quarter (16 | chunk stride)
  const int bshift = (q & 1) ? 16 : 0;  // six base bytes start 0 or 2 bytes into the window
  const int hshift = 4 * (q & 1);       // the chunk's two high digits

  // Buffers over the planes from a row-quad on: the base address and size
  // are uniform, the lane adds only its fixed offset, and rows past n fall
  // outside the buffer and read as zero (their results are never written).
  struct Rsrc { __amdgpu_buffer_rsrc_t b, h, s; };
  auto rsrc_at = [&](int rq) {
    const int row = (rowq0 + rq) * 4;
    const int left = rq < sh.rq && n32 > row ? n32 - row : 0;
    Rsrc r;
    r.b = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.base + (int64_t)row * p.base_row), 0,
                                            left * (int)p.base_row, 0x00020000);
    r.h = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.high + (int64_t)row * p.high_row), 0,
                                            left * (int)p.high_row, 0x00020000);
    r.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.scale + (int64_t)row * p.groups), 0,
                                            left * (int)p.groups * 2, 0x00020000);
    return r;
  };
  auto load_step = [&](const Rsrc &r, int s, ChunkRaw &c) {
    c.w0 = __builtin_amdgcn_raw_buffer_load_b32(r.b, ob[s], 0, 2);
    c.w1 = __builtin_amdgcn_raw_buffer_load_b32(r.b, ob[s] + 4, 0, 2);
    if constexpr (FMT == FMT_PTQ1) c.h = __builtin_amdgcn_raw_buffer_load_b8(r.h, oh[s], 0, 2);
    else c.h = 0;
    c.s = __builtin_amdgcn_raw_buffer_load_b16(r.s, os[s], 0, 0);
  };

  // ---- activations of the lane's chunks for batch row j, binary16 pairs
  // in decode order: pair 5p + i = trits (10p + i, 10p + 5 + i) of the
  // chunk (digit i of base bytes 2p and 2p+1), pair 15 = the two high
  // trits.  Each wave stages its 512 activations of a slot (16 chunks) per
  // batch row through its own LDS with coalesced loads; lanes then pick
  // their chunk out of it.  Activations past k and batch rows past `batch`
  // are zero.
  u32x2 xp[NG][S][8];
  // activation loads first: a wave's loads complete in order, so loads
  // issued after the weight rows would wait for them
  // (BT batch rows are loaded: 1 for a single row, else 4 or 8)
  u32x4 xraw[S][BT][XD == DT_F32 ? 2 : 1];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e0 = (wave * S + s) * 512 + 8 * lane;  // 8 consecutive activations per lane
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      // unconditional loads from a valid address, zeroed afterwards: a
      // branch around a load makes the compiler wait for every load in
      // flight where the paths join
      const int64_t i0 = (int64_t)(b < batch ? b : 0) * ldx + (e0 < k32 ? e0 : 0);
      if constexpr (XD == DT_F32) {
        const u32x4 *pf = reinterpret_cast<const u32x4 *>(static_cast<const float *>(x) + i0);
        xraw[s][b][0] = pf[0];
        xraw[s][b][1] = pf[1];
      } else {
        xraw[s][b][0] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(x) + i0);
      }
    }
  }
  // ---- weight loads of the first row-quad, in flight while the
  // activations are staged; the rest of the first round after that
  ChunkRaw ring[U];
  {
    const Rsrc rr = rsrc_at(0);
#pragma unroll
    for (int s = 0; s < S; ++s) load_step(rr, s, ring[s]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- the digit table (PTQ1_0), built while the loads are in flight
  for (int v = threadIdx.x; v < (FMT == FMT_PTQ1 ? 256 : 0); v += blockDim.x) {
    uint32_t a = (uint32_t)v, w = 0;
    for (int i = 0; i < 5; ++i) { w |= (a % 3u) << (2 * i); a /= 3u; }
    lut[v] = w;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e0 = (wave * S + s) * 512 + 8 * lane;
    // a wave's LDS operations complete in order: the reads of the previous
    // group are done before this group's writes reuse the staging rows
#pragma unroll
    for (int bb = 0; bb < SB; ++bb) {
      const int b = g * 4 + bb;
      const bool ok = b < batch && e0 < k32;
      uint32_t h[4];
      if constexpr (XD == DT_F16) {
#pragma unroll
        for (int t = 0; t < 4; ++t) h[t] = ok ? xraw[s][b][0][t] : 0u;
      } else {
        float v[8];
        if constexpr (XD == DT_F32) {
#pragma unroll
          for (int t = 0; t < 8; ++t) v[t] = __uint_as_float(xraw[s][b][t >> 2][t & 3]);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[2 * t] = bf16_to_f32((uint16_t)(xraw[s][b][0][t] & 0xFFFF));
            v[2 * t + 1] = bf16_to_f32((uint16_t)(xraw[s][b][0][t] >> 16));
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          h[t] = ok ? (uint32_t)f32_to_f16(v[2 * t]) | ((uint32_t)f32_to_f16(v[2 * t + 1]) << 16)
                    : 0u;
      }
      *reinterpret_cast<u32x4 *>(xst + (wave * SB + bb) * XROW + (lane >> 4) * XGRP + 4 * (lane & 15)) =
          (u32x4){h[0], h[1], h[2], h[3]};
    }
    // this lane's chunk blk of batch row 4g + j.  PTQ1_0: 30 base trits at
    // 128*(blk/4) + 30*(blk%4), 2 high trits at 128*(blk/4) + 120 + 2*(blk%4);
    // PQ2_0: 32 consecutive weights at 32*blk
    const uint32_t *src = xst + (wave * SB + (BT == 1 ? 0 : j)) * XROW + (blk >> 2) * XGRP;
    uint32_t w[16];
    if constexpr (FMT == FMT_PTQ1) {
#pragma unroll
      for (int t = 0; t < 15; ++t) w[t] = src[15 * q + t];
      w[15] = src[60 + q];
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) w[t] = src[16 * q + t];
    }
    // w[t] holds weights 2t, 2t+1 of the chunk (PTQ1_0: t < 15, then the
    // high pair)
    auto el = [&](int i) -> uint32_t {  // trit i (< 30) of the chunk, binary16 bits
      return (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
    };
    uint32_t pr[16];
    if constexpr (FMT == FMT_PTQ1) {
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int i = 0; i < 5; ++i) pr[5 * pp + i] = el(10 * pp + i) | (el(10 * pp + 5 + i) << 16);
      pr[15] = w[15];
    } else {
      // pair 8d + e = weights (16d + e, 16d + e + 8) of the chunk
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[8 * d + e] = el(16 * d + e) | (el(16 * d + e + 8) << 16);
    }
    // (one staged row: lanes of batch rows 1..3 multiply by zero)
    const bool use = BT > 1 || j == 0;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      xp[g][s][m] = use ? (u32x2){pr[2 * m], pr[2 * m + 1]} : (u32x2){0u, 0u};
  }

#pragma unroll
  for (int r = 1; r < RR; ++r) {
    const Rsrc rr = rsrc_at(r);
#pragma unroll
    for (int s = 0; s < S; ++s) load_step(rr, s, ring[r * S + s]);
  }

  __syncthreads();  // the digit table and every wave's staging are written

  uint32_t magic_v = 0x64006400u;
  asm volatile("" : "+v"(magic_v));
  const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
  const half2_t neg2 = {(_Float16)-1025.0f, (_Float16)-1025.0f};

  auto do_round = [&](int rq0, auto refill, int valid) {
    float yacc[NG][RR][4];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) yacc[g][r][e] = 0.0f;
    Rsrc next;
    if constexpr (decltype(refill)::value) next = rsrc_at(rq0 + RR);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = u % S, r = u / S;
      if (r >= valid) break;  // last round: row-quads past the workgroup's share
      const ChunkRaw c = ring[u];
      if constexpr (decltype(refill)::value) {
        if (u % S == 0 && u > 0) next = rsrc_at(rq0 + RR + r);
        load_step(next, s, ring[u]);
      }
      const float sc = real[s] ? f16_to_f32((uint16_t)c.s) : 0.0f;
      u32x2 T[8];
      if constexpr (FMT == FMT_PTQ1) {
        // the six base bytes and the high byte through the digit table
        const uint64_t win = (((uint64_t)c.w1 << 32) | c.w0) >> bshift;
        const uint32_t lo = (uint32_t)win, hi = (uint32_t)(win >> 32);
        const uint32_t P0 = lut[lo & 0xFF] | (lut[(lo >> 8) & 0xFF] << 16);
        const uint32_t P1 = lut[(lo >> 16) & 0xFF] | (lut[lo >> 24] << 16);
        const uint32_t P2 = lut[hi & 0xFF] | (lut[(hi >> 8) & 0xFF] << 16);
        const uint32_t L = lut[c.h & 0xFF] >> hshift;
        const uint32_t PH = (L & 3u) | ((L & 0xCu) << 14);
        T[0] = (u32x2){trit_pair<0>(P0, magic_v), trit_pair<1>(P0, magic_v)};
        T[1] = (u32x2){trit_pair<2>(P0, magic_v), trit_pair<3>(P0, magic_v)};
        T[2] = (u32x2){trit_pair<4>(P0, magic_v), trit_pair<0>(P1, magic_v)};
        T[3] = (u32x2){trit_pair<1>(P1, magic_v), trit_pair<2>(P1, magic_v)};
        T[4] = (u32x2){trit_pair<3>(P1, magic_v), trit_pair<4>(P1, magic_v)};
        T[5] = (u32x2){trit_pair<0>(P2, magic_v), trit_pair<1>(P2, magic_v)};
        T[6] = (u32x2){trit_pair<2>(P2, magic_v), trit_pair<3>(P2, magic_v)};
        T[7] = (u32x2){trit_pair<4>(P2, magic_v),
                       u32(__builtin_elementwise_fma(h2(PH | magic_v), one2, neg2))};
      } else {
        // codes e and e+8 of each dword: in place for e <= 4, after a shift
        // by 10 for e = 5..7
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t v = d ? c.w1 : c.w0, v10 = v >> 10;
          T[4 * d + 0] = (u32x2){trit_pair<0>(v, magic_v), trit_pair<1>(v, magic_v)};
          T[4 * d + 1] = (u32x2){trit_pair<2>(v, magic_v), trit_pair<3>(v, magic_v)};
          T[4 * d + 2] = (u32x2){trit_pair<4>(v, magic_v), trit_pair<0>(v10, magic_v)};
          T[4 * d + 3] = (u32x2){trit_pair<1>(v10, magic_v), trit_pair<2>(v10, magic_v)};
        }
      }
      if constexpr (NG == 1) {
        // two independent accumulation chains
        floatx4 a0 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, xp[0][s][0]),
                                                        __builtin_bit_cast(half4_t, T[0]),
                                                        (floatx4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        floatx4 a1 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, xp[0][s][1]),
                                                        __builtin_bit_cast(half4_t, T[1]),
                                                        (floatx4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
        for (int m = 2; m < 8; m += 2) {
          a0 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, xp[0][s][m]),
                                                  __builtin_bit_cast(half4_t, T[m]), a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, xp[0][s][m + 1]),
                                                  __builtin_bit_cast(half4_t, T[m + 1]), a1, 0, 0, 0);
        }
        // (one batch row: only row 0 of the 4x4 products is not zero)
#pragma unroll
        for (int e = 0; e < (BT == 1 ? 1 : 4); ++e) yacc[0][r][e] += sc * (a0[e] + a1[e]);
      } else {
        // one chain per group of four batch rows (registers are short)
        floatx4 a[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g)
          a[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, xp[g][s][0]),
                                                    __builtin_bit_cast(half4_t, T[0]),
                                                    (floatx4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
        for (int m = 1; m < 8; ++m)
#pragma unroll
          for (int g = 0; g < NG; ++g)
            a[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, xp[g][s][m]),
                                                      __builtin_bit_cast(half4_t, T[m]), a[g], 0, 0, 0);
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) yacc[g][r][e] += sc * a[g][e];
      }
      // the step's refill stays here; arithmetic, matrix and LDS work may
      // move across steps (mask: everything but the global loads)
      __builtin_amdgcn_sched_barrier(0x18F);
    }
    // per row-quad: sum over the wave's blocks, stash per wave
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      if (r >= valid) break;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float tot = blocks_sum4(yacc[g][r]);
        if ((lane & 12) == 0) {
          const int e = (0x3120 >> (4 * (lane >> 4))) & 3;  // [0, 2, 1, 3][lane >> 4]
          red[((rq0 + r) * W + wave) * (16 * NG) + g * 16 + j * 4 + e] = tot;
        }
      }
    }
  };
  int rq0 = 0;
  for (; rq0 + RR < sh.rq; rq0 += RR) do_round(rq0, std::integral_constant<bool, true>{}, RR);
  // (the red buffer shares LDS with the activation staging, which every
  // wave finished reading before the barrier after the staging)
  do_round(rq0, std::integral_constant<bool, false>{}, sh.rq - rq0);
  __syncthreads();

  // ---- totals over waves, in wave order
  for (int o = threadIdx.x; o < sh.rq * 16 * NG; o += blockDim.x) {
    const int rq = o / (16 * NG), g = (o >> 4) % NG, jj = (o >> 2) & 3, e = o & 3;
    const int row = (rowq0 + rq) * 4 + jj;
    const int b = 4 * g + e;  // batch row
    if (row >= n32 || b >= batch) continue;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) sum += red[(rq * W + w) * (16 * NG) + g * 16 + jj * 4 + e];
    y[(int64_t)b * ldy + row] = sum;
  }
}

template <int FMT, int S, int RR, int W, int XD>
hipError_t quads_go(const Planes &p, const void *x, int64_t batch, int64_t ldx, float *y,
                   int64_t ldy, int rq, int grid, hipStream_t st) {
  Ptq1Shape sh;
  sh.chunks = (int)(p.k / 32);
  sh.rq = rq;
  if (batch <= 1)
    hipLaunchKernelGGL((gemv_quads_kernel<FMT, S, RR, W, XD, 1>), dim3((unsigned)grid), dim3(64 * W), 0,
                       st, p, x, batch, ldx, y, ldy, sh);
  else if (batch <= 4)
    hipLaunchKernelGGL((gemv_quads_kernel<FMT, S, RR, W, XD, 4>), dim3((unsigned)grid), dim3(64 * W), 0,
                       st, p, x, batch, ldx, y, ldy, sh);
  else if constexpr (S <= 3 && XD != DT_F32)
    // eight rows: their activations take the registers of a deeper ring
    hipLaunchKernelGGL((gemv_quads_kernel<FMT, S, 1, W, XD, 8>), dim3((unsigned)grid), dim3(64 * W), 0,
                       st, p, x, batch, ldx, y, ldy, sh);
  else
    return hipErrorInvalidValue;  // not reached: such passes hold at most four rows
  return hipGetLastError();
}

template <int FMT, int S, int RR, int W>
hipError_t quads_dt(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx, float *y,
                    int64_t ldy, int rq, int grid, hipStream_t st) {
  if (xd == DT_F32) return quads_go<FMT, S, RR, W, DT_F32>(p, x, batch, ldx, y, ldy, rq, grid, st);
  if (xd == DT_BF16) return quads_go<FMT, S, RR, W, DT_BF16>(p, x, batch, ldx, y, ldy, rq, grid, st);
  return quads_go<FMT, S, RR, W, DT_F16>(p, x, batch, ldx, y, ldy, rq, grid, st);
}

template <int S, int RR, int W>
hipError_t quads_fmt(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx, float *y,
                     int64_t ldy, int rq, int grid, hipStream_t st) {
  if (p.fmt == FMT_PTQ1) return quads_dt<FMT_PTQ1, S, RR, W>(p, x, xd, batch, ldx, y, ldy, rq, grid, st);
  return quads_dt<FMT_PQ2, S, RR, W>(p, x, xd, batch, ldx, y, ldy, rq, grid, st);
}

// Waves per workgroup (up to twelve, fewer for short rows: a wave covers 16
// chunks a slot) and slots per lane for k/32 chunks.
void quads_split(int chunks, int &W, int &S) {
  const int cw = (chunks + 15) / 16;
  W = cw <= 4 ? 4 : cw <= 8 ? 8 : 12;
  S = (chunks + 16 * W - 1) / (16 * W);
}

// Batch rows one pass can hold: eight where the activations of eight rows
// fit the registers (up to three slots, 16-bit activations), else four.
int quads_pass_rows(const Planes &p, int xd) {
  int W, S;
  quads_split((int)(p.k / 32), W, S);
  return S <= 3 && xd != DT_F32 ? 8 : 4;
}

// One pass of up to quads_pass_rows batch rows.
hipError_t quads_pass(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx, float *y,
                     int64_t ldy, hipStream_t st) {
  const int chunks = (int)(p.k / 32);
  int W, S;
  quads_split(chunks, W, S);
  // row-quads per workgroup: an equal share per compute unit, at most RQMAX
  const int cus = device_cus();
  const int64_t nq = (p.n + 3) / 4;
  int64_t rq = (nq + cus - 1) / cus;
  if (rq > RQMAX) rq = RQMAX;
  const int64_t grid = (nq + rq - 1) / rq;
  // row-quads of loads in flight: S*RR steps (a last partial round skips
  // the row-quads past the workgroup's share)
#define TQ_QUADS_W(WW)                                                                         \
  switch (S) {                                                                                \
    case 1: return quads_fmt<1, 5, WW>(p, x, xd, batch, ldx, y, ldy, (int)rq, (int)grid, st);   \
    case 2: return quads_fmt<2, 3, WW>(p, x, xd, batch, ldx, y, ldy, (int)rq, (int)grid, st);   \
    case 3: return quads_fmt<3, 2, WW>(p, x, xd, batch, ldx, y, ldy, (int)rq, (int)grid, st);   \
    default: return quads_fmt<4, 1, WW>(p, x, xd, batch, ldx, y, ldy, (int)rq, (int)grid, st);  \
  }
  switch (W) {
    case 4: TQ_QUADS_W(4)
    case 8: TQ_QUADS_W(8)
    default: TQ_QUADS_W(12)
  }
#undef TQ_QUADS_W
}

}  // namespace

// k up to 12 waves x 4 slots x 16 chunks x 32 weights.
bool gemv_quads_fits(const Planes &p) {
  return (p.fmt == FMT_PTQ1 || p.fmt == FMT_PQ2) && p.k % 128 == 0 && p.k / 32 <= 12 * 4 * 16 &&
         p.n * p.base_row < (int64_t(1) << 31);
}

hipError_t launch_gemv_quads(const Planes &p, const void *x, int xd, int64_t batch, int64_t ldx,
                            float *y, int64_t ldy, hipStream_t st) {
  const int64_t esz = xd == DT_F32 ? 4 : 2;
  const int64_t step = quads_pass_rows(p, xd);
  for (int64_t b0 = 0; b0 < batch; b0 += step) {
    const int64_t nb = batch - b0 < step ? batch - b0 : step;
    hipError_t e = quads_pass(p, static_cast<const char *>(x) + b0 * ldx * esz, xd, nb, ldx,
                             y + b0 * ldy, ldy, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
