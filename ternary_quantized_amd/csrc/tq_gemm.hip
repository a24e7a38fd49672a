// Prefill GEMM over row-split ternary planes:
//   Y[m][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * X[m][j]
// [ninfer-skill] §3 (planes), [gguf-explainer] §4.3 (codes), [tensorsharp]
// §4.4 (every low-bit projection multiplies the rotated activations).
//
// This is a genuinely dense contraction, so it runs on the matrix cores
// (v_mfma_f32_32x32x16_f16, fp32 accumulation).  The workgroup stages its X
// tile in LDS as binary16 and decodes its weight tile into LDS as the
// binary16 values t*s.  That value is exact -- s is itself a binary16 and t
// is -1, 0 or +1 -- so folding the group scale into the decoded weight loses
// nothing, and the only rounding before the fp32 accumulation is that of X
// to binary16.  Output tiles are dealt XCD-aware: the workgroups of one XCD
// hold a block of tiles two M bands tall, so that its X rows and weight
// columns are shared in that XCD's L2.

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Pipelined prefill GEMM: 512-thread workgroups (8 waves), 64-deep K steps
// through two LDS stages, one barrier per step.  PQ2_0 planes hold the 2-bit
// codes; PTQ1_0 planes are turned into the same 2-bit code words on the way
// in (below), so both formats share the decode and everything after it.
//
// Stage layout: X rows and decoded weight rows of [64 k + 8 pad] binary16.
// Inside every 16-wide k block both are stored in the k order
// (0,8,1,9,...,7,15): one dword of 16 codes decodes into the pairs (e, e+8),
// and X is permuted to match, so an MFMA k slot holds the same k in both
// operands.  Weights are decoded exactly with full-rate integer ops: the
// code ORed into the exponent field of 1024 gives 1024 + 4^e*code, one fma
// turns it into code - 1, and the product with the group scale is exactly 0
// or +-s.
//
// Register ring: while step s is multiplied, X register set (s+1)&1 holds
// step s+1, which is stored into the other stage between step s's MFMA
// slices; each half of the set is refilled with step s+3 as soon as its two
// pieces are stored, so every X load has two steps to land (X misses the
// L2 often enough that one step is not enough).  The codes are fetched four
// steps ahead; they are plain (cached) loads: one 128-byte line of a weight
// row serves 8 consecutive steps.
//
// Two tile shapes share the kernel: 256 x 256 tiles (waves 2 x 4 of 128 x
// 64) for the bulk, and 128 x 64 sub-tiles (waves 4 x 2 of 32 x 32) for the
// tiles of a last, partial round, which is split 8 ways so it fills the
// chip instead of a fraction of it.
//
// PTQ1_0: a K step covers half a group, and a weight thread's 32 weights
// are one 64-bit word of the group's 2-bit code string (code = radix-3
// digit = trit + 1, weight j at bits 2j): word w = 2*(step & 1) + half.  A
// 256-entry LDS table gives a byte's five digits as a 10-bit field, and the
// word is assembled from the fields of the base bytes (and high bytes) it
// overlaps, each at a fixed shift.  The thread loads the 12 base bytes that
// hold them (bytes 0-11, 4-15, 12-23, 12-23 for words 0-3) and the group's two
// high bytes.  The half is chosen per wave, so the word is uniform in a wave.
constexpr int G2K = 64, G2ROW = G2K + 8;

// Word w of a PTQ1_0 group's code string from its base window b[3] (bytes
// 0-11, 4-15 or 12-23 of the group for w = 0, 1, 2-3) and high bytes h.
__device__ __forceinline__ uint64_t ptq1_code_word(const uint32_t (&b)[3], uint32_t h, int w,
                                                   const uint16_t *lut) {
  auto byte = [&](int i) -> uint32_t { return (b[i >> 2] >> (8 * (i & 3))) & 0xFFu; };
  auto field = [&](int i) -> uint64_t { return lut[byte(i)]; };
  uint64_t acc = 0;
  // field of group byte j sits at bit 10j - 64w of the word
  switch (w) {
    case 0:  // group bytes 0..6 = window bytes 0..6
#pragma unroll
      for (int j = 0; j <= 6; ++j) acc |= field(j) << (10 * j);
      break;
    case 1:  // group bytes 6..12 = window bytes 2..8
      acc = field(2) >> 4;
#pragma unroll
      for (int j = 7; j <= 12; ++j) acc |= field(j - 4) << (10 * j - 64);
      break;
    case 2:  // group bytes 12..19 = window bytes 0..7
      acc = field(0) >> 8;
#pragma unroll
      for (int j = 13; j <= 19; ++j) acc |= field(j - 12) << (10 * j - 128);
      break;
    default:  // group bytes 19..23 = window bytes 7..11, then the high bytes
      acc = field(7) >> 2;
#pragma unroll
      for (int j = 20; j <= 23; ++j) acc |= field(j - 12) << (10 * j - 192);
      acc |= (uint64_t)(lut[h & 0xFFu] & 0xFFu) << 48;
      acc |= (uint64_t)(lut[(h >> 8) & 0xFFu] & 0xFFu) << 56;
      break;
  }
  return acc;
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t trit_pair_scaled(uint32_t t, float inv_m, float neg_c,
                                                     half2_t s2) {
  half2_t a = __builtin_bit_cast(half2_t, t), m, c;
  m.x = m.y = (_Float16)inv_m;
  c.x = c.y = (_Float16)neg_c;
  const half2_t trit = __builtin_elementwise_fma(a, m, c);  // exactly code - 1
  return __builtin_bit_cast(uint32_t, trit * s2);            // exactly 0 or +-s
}

// Half of a dword of 16 codes -> 4 binary16 pairs of t*s: part 0 gives the
// pairs (code e, code e+8) for e = 0..3, part 1 for e = 4..7.
template <int PART>
__device__ __forceinline__ void decode_pq2_ts4(uint32_t d, uint32_t magic, half2_t s2,
                                               uint32_t o[4]) {
  if constexpr (PART == 0) {
    o[0] = trit_pair_scaled((d & 0x00030003u) | magic, 1.0f, -1025.0f, s2);
    o[1] = trit_pair_scaled((d & 0x000C000Cu) | magic, 0.25f, -257.0f, s2);
    o[2] = trit_pair_scaled((d & 0x00300030u) | magic, 0.0625f, -65.0f, s2);
    o[3] = trit_pair_scaled((d & 0x00C000C0u) | magic, 0.015625f, -17.0f, s2);
  } else {
    const uint32_t d10 = d >> 10;
    o[0] = trit_pair_scaled((d & 0x03000300u) | magic, 0.00390625f, -5.0f, s2);
    o[1] = trit_pair_scaled((d10 & 0x00030003u) | magic, 1.0f, -1025.0f, s2);
    o[2] = trit_pair_scaled((d10 & 0x000C000Cu) | magic, 0.25f, -257.0f, s2);
    o[3] = trit_pair_scaled((d10 & 0x00300030u) | magic, 0.0625f, -65.0f, s2);
  }
}

template <int XD>
__device__ __forceinline__ uint32_t x_pair_f16(uint32_t v) {
  if constexpr (XD == DT_BF16) {
    const uint32_t lo = f32_to_f16(bf16_to_f32((uint16_t)(v & 0xFFFF)));
    const uint32_t hi = f32_to_f16(bf16_to_f32((uint16_t)(v >> 16)));
    return lo | (hi << 16);
  } else {
    return v;
  }
}

// One output tile of TM x TN at (m0, n0): waves WAVES_M x (8 / WAVES_M),
// each 32*FM x 32*FN.
template <int FMT, int XD, int YD, int TM, int TN, int FM, int FN, int WAVES_M>
__device__ __forceinline__ void gemm_planes_tile(const Planes &p, const uint16_t *__restrict__ X,
                                              int64_t M, int64_t ldx, void *__restrict__ Y,
                                              int64_t ldy, int64_t m0, int64_t n0,
                                              _Float16 *lds2, const uint16_t *lut) {
  constexpr int WAVES_N = 8 / WAVES_M;
  static_assert(WAVES_M * 32 * FM == TM && WAVES_N * 32 * FN == TN, "wave grid must cover the tile");
  constexpr int TPR = 512 / TM;       // threads per X row
  constexpr int HX = G2K / TPR;       // halves of X per thread and step
  constexpr int XQ = HX / 8;          // 16-byte X loads (and LDS writes) per thread and step
  static_assert(HX % 16 == 0 && XQ <= 4, "X share must be whole 16-wide k blocks");
  constexpr int STAGE = (TM + TN) * G2ROW;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = (wave / WAVES_N) * 32 * FM, wn = (wave % WAVES_N) * 32 * FN;
  const int nsteps = (int)(p.k / G2K);  // even: k is a multiple of 128

  // X loads: row xr, halves [HX*xq, HX*xq + HX) of a step
  const int xr = t / TPR, xq = t % TPR;
  // a buffer over the tile's rows of X: rows past M read as zero, so no
  // select zeroes them (the compiler would place such a select right after
  // the load and wait for it there)
  const int64_t xrows = M - m0 < TM ? M - m0 : TM;
  const __amdgpu_buffer_rsrc_t xbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(X + m0 * ldx), 0, (int)(xrows * ldx * 2), 0x00020000);
  const int xoff = (int)((xr * ldx + HX * xq) * 2);
  // code loads (threads below 2*TN): row wr, codes [32*wh, 32*wh + 32) of a
  // step (8 bytes) and that row's group scale
  // (every thread loads codes when the tile is 256 wide: no branch, so the
  // compiler keeps counting the loads in flight instead of waiting for all
  // of them where a branch around a load would rejoin)
  const bool wthread = 2 * TN >= 512 || t < 2 * TN;
  // PQ2_0: neighbouring lanes take the two halves of a row; PTQ1_0: the half
  // is the wave's (its code word must be uniform in a wave)
  const int wr = !wthread ? 0 : FMT == FMT_PQ2 ? t >> 1 : (((t >> 7) << 6) | (t & 63));
  const int wh = FMT == FMT_PQ2 ? (t & 1) : __builtin_amdgcn_readfirstlane((t >> 6) & 1);
  // buffers over the tile's weight rows: rows past n read as zero codes and
  // zero scales, so their decoded weights are 0 without a select
  const int wrows = __builtin_amdgcn_readfirstlane((int)(p.n - n0 < TN ? p.n - n0 : TN));
  const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(p.base + n0 * p.base_row), 0, wrows * (int)p.base_row, 0x00020000);
  const __amdgpu_buffer_rsrc_t hbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(p.high + n0 * p.high_row), 0, wrows * (int)p.high_row, 0x00020000);
  const __amdgpu_buffer_rsrc_t sbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.scale + n0 * p.groups), 0, wrows * (int)p.groups * 2, 0x00020000);
  const int woff = wr * (int)p.base_row + (FMT == FMT_PQ2 ? 8 * wh : 0);
  const int hoff = wr * (int)p.high_row, soff = wr * (int)p.groups * 2;

  constexpr int WW = FMT == FMT_PQ2 ? 2 : 3;  // code (PQ2_0) or base (PTQ1_0) dwords per step
  uint32_t xreg[2][HX / 2], wreg[4][WW], hreg[4], sreg[4];
  auto clamp = [&](int st) { return st < nsteps ? st : nsteps - 1; };  // past the end: a harmless re-read
  // loads 2h and 2h+1 of step st's X share into set `set` (the two that
  // store pieces 2h and 2h+1 read)
  auto load_x_half = [&](int set, int st, int h) {
    const int kb = clamp(st) * G2K * 2;
#pragma unroll
    for (int i = 2 * h; i < 2 * h + 2 && i < XQ; ++i) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xbuf, xoff + 16 * i, kb, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) xreg[set][4 * i + c] = v[c];
    }
  };
  auto load_x = [&](int set, int st) {
    load_x_half(set, st, 0);
    load_x_half(set, st, 1);
  };
  auto load_w = [&](int set, int st) {
    if (wthread) {
      const int g = clamp(st) * G2K / 128;  // the step's group
      if constexpr (FMT == FMT_PQ2) {
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(wbuf, woff, clamp(st) * G2K / 4, 0);
        wreg[set][0] = w[0];
        wreg[set][1] = w[1];
      } else {
        // group g, window at byte 0, 4 or 12 of its 24 base bytes
        const int word = 2 * (clamp(st) & 1) + wh;
        const int off = word == 0 ? 0 : word == 1 ? 4 : 12;
#pragma unroll
        for (int i = 0; i < 3; ++i)
          wreg[set][i] = __builtin_amdgcn_raw_buffer_load_b32(wbuf, woff + 4 * i, g * 24 + off, 0);
        hreg[set] = __builtin_amdgcn_raw_buffer_load_b16(hbuf, hoff, 2 * g, 0);
      }
      sreg[set] = __builtin_amdgcn_raw_buffer_load_b16(sbuf, soff, 2 * g, 0);
    }
  };
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  // PTQ1_0: the code word of code set `wset` (built at q = 0, used by q = 0..3)
  uint32_t cw[2] = {0u, 0u};
  // quarter q of X set `set` and code set `wset` into an LDS stage: one
  // 16-byte write of permuted X (while q < XQ) and one of 8 decoded weights;
  // par = parity of the step being stored
  auto store_piece = [&](int set, int wset, int buf, int q, int par) {
    _Float16 *As = lds2 + buf * STAGE;
    _Float16 *Bs = As + TM * G2ROW;
    if (q < XQ) {
      const uint32_t *xv = xreg[set] + 8 * (q >> 1) + 2 * (q & 1);
      uint32_t lo[2], hi[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        lo[c] = x_pair_f16<XD>(xv[c]);
        hi[c] = x_pair_f16<XD>(xv[4 + c]);
      }
      u32x4_t xo;
      xo[0] = __builtin_amdgcn_perm(hi[0], lo[0], 0x05040100u);
      xo[1] = __builtin_amdgcn_perm(hi[0], lo[0], 0x07060302u);
      xo[2] = __builtin_amdgcn_perm(hi[1], lo[1], 0x05040100u);
      xo[3] = __builtin_amdgcn_perm(hi[1], lo[1], 0x07060302u);
      *reinterpret_cast<u32x4_t *>(As + xr * G2ROW + HX * xq + 8 * q) = xo;
    }
    if (wthread) {
      const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sreg[wset]);
      half2_t s2;
      s2.x = s2.y = sh;
      uint32_t o[4];
      uint32_t d;
      if constexpr (FMT == FMT_PQ2) {
        d = wreg[wset][q >> 1];
      } else {
        if (q == 0) {
          const uint64_t c = ptq1_code_word(wreg[wset], hreg[wset], 2 * par + wh, lut);
          cw[0] = (uint32_t)c;
          cw[1] = (uint32_t)(c >> 32);
        }
        d = cw[q >> 1];
      }
      if (q & 1)
        decode_pq2_ts4<1>(d, magic, s2, o);
      else
        decode_pq2_ts4<0>(d, magic, s2, o);
      *reinterpret_cast<u32x4_t *>(Bs + wr * G2ROW + 32 * wh + 8 * q) =
          (u32x4_t){o[0], o[1], o[2], o[3]};
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // step s: code set s&3 (already stored) is refilled with step s+4, stage
  // s&1 is multiplied, and between its four 16-deep k slices step s+1 (X
  // set (s+1)&1, code set (s+1)&3) is stored into the other stage, each X
  // half refilled with step s+3 right after its last piece.
  auto step = [&](int s, int ph) {  // ph = s & 3
    load_w(ph, s + 4);
    const int buf = ph & 1;
    const _Float16 *As = lds2 + buf * STAGE;
    const _Float16 *Bs = As + TM * G2ROW;
    // operand fragments of slice ks+1 are read while slice ks is multiplied
    half8_t a[2][FM], bf[2][FN];
    auto frags = [&](int ks, int set) {
      const int kb = ks * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[set][i] = *reinterpret_cast<const half8_t *>(As + (wm + 32 * i + (lane & 31)) * G2ROW + kb);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[set][j] = *reinterpret_cast<const half8_t *>(Bs + (wn + 32 * j + (lane & 31)) * G2ROW + kb);
    };
    frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < G2K / 16; ++ks) {
      if (ks + 1 < G2K / 16) frags(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks & 1][i], bf[ks & 1][j], acc[i][j],
                                                             0, 0, 0);
      store_piece((ph + 1) & 1, (ph + 1) & 3, buf ^ 1, ks, (ph + 1) & 1);
      // pieces ks-1 and ks have left the X registers they share: refill
      // them at once with step s+3, which they hold next
      if (ks & 1) load_x_half((ph + 1) & 1, s + 3, ks >> 1);
    }
    __syncthreads();
  };

  load_x(0, 0);
  load_w(0, 0);
  load_x(1, 1);
#pragma unroll
  for (int i = 1; i < 4; ++i) load_w(i, i);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    store_piece(0, 0, 0, q, 0);
    if (q & 1) load_x_half(0, 2, q >> 1);
  }
  __syncthreads();
  // whole groups of four steps, then the two left over when nsteps % 4 ==
  // 2 (nsteps is even): the loop's back edge then always leaves the same
  // loads in flight, so the count the compiler waits for at its head is
  // exact rather than zero
  int s = 0;
  for (; s + 4 <= nsteps; s += 4) {
    step(s, 0);
    step(s + 1, 1);
    step(s + 2, 2);
    step(s + 3, 3);
  }
  if (s < nsteps) {
    step(s, 0);
    step(s + 1, 1);
  }

  // epilogue: D[i][j] of a 32x32 block is in lane j + 32*((i/4) % 2),
  // element 4*(i/8) + i%4
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < M && col < p.n) {
          if constexpr (YD == DT_F32)
            static_cast<float *>(Y)[row * ldy + col] = acc[i][j][v];
          else
            static_cast<uint16_t *>(Y)[row * ldy + col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
}

// Work split of one launch over 256 x 256 tiles: workgroups [0, nbig) take
// whole tiles, the rest take 128 x 64 sub-tiles (8 per tile) of the tiles
// left over.  Tiles are numbered in groups of GEMM_GM 256-row bands: within
// a group the number runs down the bands first, then along N, so that
// consecutive tiles share their activation rows in pairs and their weight
// columns in runs.  With `xcd` set, XCD x (the workgroups b with b % 8 ==
// x) owns the contiguous tiles [x*per, (x+1)*per), the first big_per of
// them whole; otherwise tiles go in plain order.  The tiles one XCD holds
// at a time then span two bands and half as many weight columns as a
// single band would, which is fewer bytes through its L2 per round.
constexpr int GEMM_GM = 2;
struct GemmSplit {
  int tiles_m;  // 256-row bands along M
  int tiles_n;  // 256-wide tiles along N
  int per;      // tiles per XCD
  int big_per;  // whole tiles per XCD
  int nbig;     // workgroups on whole tiles
  int xcd;
};

template <int FMT, int XD, int YD>
__global__ __launch_bounds__(512) void gemm_planes_kernel(Planes p, const uint16_t *__restrict__ X,
                                                       int64_t M, int64_t ldx,
                                                       void *__restrict__ Y, int64_t ldy,
                                                       GemmSplit sp) {
  extern __shared__ __attribute__((aligned(16))) _Float16 lds2[];
  // PTQ1_0: digit i of byte v as the 2-bit field i (the first stage's
  // barrier orders these writes before any use)
  __shared__ uint16_t lut[FMT == FMT_PTQ1 ? 256 : 1];
  if constexpr (FMT == FMT_PTQ1) {
    if (threadIdx.x < 256) {
      uint32_t v = threadIdx.x, f = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        f |= (v % 3u) << (2 * i);
        v /= 3u;
      }
      lut[threadIdx.x] = (uint16_t)f;
    }
    __syncthreads();
  }
  const int b = blockIdx.x;
  int tile, sub = -1;
  if (b < sp.nbig) {
    tile = sp.xcd ? (b % 8) * sp.per + b / 8 : b;
  } else {
    const int r = b - sp.nbig;
    if (sp.xcd) {
      const int s2 = r / 8;  // nbig is a multiple of 8, so r % 8 == b % 8
      tile = (r % 8) * sp.per + sp.big_per + s2 / 8;
      sub = s2 % 8;
    } else {
      tile = sp.nbig + r / 8;
      sub = r % 8;
    }
  }
  // tile number -> (band, column tile): groups of GEMM_GM bands (the last
  // group may hold fewer), band-minor inside a group
  const int gsz = GEMM_GM * sp.tiles_n;
  const int grp = tile / gsz, rest = tile - grp * gsz;
  const int gm = sp.tiles_m - grp * GEMM_GM < GEMM_GM ? sp.tiles_m - grp * GEMM_GM : GEMM_GM;
  const int64_t m0 = (int64_t)(grp * GEMM_GM + rest % gm) * 256, n0 = (int64_t)(rest / gm) * 256;
  if (sub < 0)
    gemm_planes_tile<FMT, XD, YD, 256, 256, 4, 2, 2>(p, X, M, ldx, Y, ldy, m0, n0, lds2, lut);
  else
    gemm_planes_tile<FMT, XD, YD, 128, 64, 1, 1, 4>(p, X, M, ldx, Y, ldy, m0 + 128 * (sub >> 2),
                                                 n0 + 64 * (sub & 3), lds2, lut);
}

template <int FMT, int XD, int YD>
static hipError_t gemm_planes_go(const Planes &p, const uint16_t *x, int64_t m, int64_t ldx, void *y,
                              int64_t ldy, hipStream_t st) {
  GemmSplit sp;
  sp.tiles_n = (int)((p.n + 255) / 256);
  sp.tiles_m = (int)((m + 255) / 256);
  const int total = sp.tiles_n * sp.tiles_m;
  const int cus = device_cus();
  // a last round that would occupy at most 1/8 of the CUs is split 8 ways
  const int left = total % cus;
  const bool split = total > cus && left > 0 && 8 * left <= cus;
  sp.xcd = total % 8 == 0 && (!split || left % 8 == 0);
  if (sp.xcd) {
    sp.per = total / 8;
    sp.big_per = split ? sp.per - left / 8 : sp.per;
    sp.nbig = 8 * sp.big_per;
  } else {
    sp.per = sp.big_per = 0;
    sp.nbig = split ? total - left : total;
  }
  const int grid = sp.nbig + 8 * (total - sp.nbig);
  const size_t lds = (size_t)2 * (256 + 256) * G2ROW * sizeof(_Float16);
  auto kern = gemm_planes_kernel<FMT, XD, YD>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, p, x, m, ldx, y, ldy, sp);
  return hipGetLastError();
}

hipError_t launch_gemm(const Planes &p, const uint16_t *x, int xd, int64_t m, int64_t ldx, void *y,
                       int yd, int64_t ldy, hipStream_t st) {
  // k is a multiple of 128 (checked by the entry point): whole 64-deep steps
  if (p.fmt == FMT_PQ2) {
    if (xd == DT_F16)
      return yd == DT_F32 ? gemm_planes_go<FMT_PQ2, DT_F16, DT_F32>(p, x, m, ldx, y, ldy, st)
                          : gemm_planes_go<FMT_PQ2, DT_F16, DT_BF16>(p, x, m, ldx, y, ldy, st);
    return yd == DT_F32 ? gemm_planes_go<FMT_PQ2, DT_BF16, DT_F32>(p, x, m, ldx, y, ldy, st)
                        : gemm_planes_go<FMT_PQ2, DT_BF16, DT_BF16>(p, x, m, ldx, y, ldy, st);
  }
  if (xd == DT_F16)
    return yd == DT_F32 ? gemm_planes_go<FMT_PTQ1, DT_F16, DT_F32>(p, x, m, ldx, y, ldy, st)
                        : gemm_planes_go<FMT_PTQ1, DT_F16, DT_BF16>(p, x, m, ldx, y, ldy, st);
  return yd == DT_F32 ? gemm_planes_go<FMT_PTQ1, DT_BF16, DT_F32>(p, x, m, ldx, y, ldy, st)
                      : gemm_planes_go<FMT_PTQ1, DT_BF16, DT_BF16>(p, x, m, ldx, y, ldy, st);
}

}  // namespace tq
