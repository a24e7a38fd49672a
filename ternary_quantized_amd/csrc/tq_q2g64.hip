// Lossless expansion of the ternary row-split planes into 2-bit G64 blocks,
// and the decode GEMV over the expanded stream.
//
// [tensorsharp] §4.1: a runtime without the private ternary types expands
// their blocks, without requantising, into the upstream 2-bit block type and
// pays for it in memory (about +6% over PQ2_0, +29% over PTQ1_0).  The block
// is [binary16 d][16 code bytes] for 64 weights; weight j sits at code byte
// j/4, bits 2*(j%4), value (code - 1) * d ([gguf-explainer] §4.3 Q2_0
// dequantisation; [ninfer-v3] §6.1 q2_g64_fp16).  Group g of a row (128
// weights, one scale) becomes blocks 2g and 2g+1, both with that scale.
//
// Expansion (HBM-bound byte reshuffle): one thread per group reads the
// group's code bytes and scale and builds its two blocks (36 bytes) in LDS;
// a workgroup gathers a tile of GT consecutive groups there and writes the
// tile's 36 * GT output bytes as 16-byte chunks, lane after lane (a 36-byte
// stride per lane would scatter every store instruction over many lines).  PQ2_0
// code bytes are already the 2-bit codes, in the same order.  A PTQ1_0 digit
// is trit + 1, which is the 2-bit code: a 256-entry LDS table gives the five
// digits of a base byte as five 2-bit fields (the four of a high byte are its
// low eight bits), and the fields are laid end to end, 10 bits per base byte
// and 8 per high byte, which is exactly the 2-bit code string of the group.

#include "tq_device.h"
#include "tq_gemv_wave.h"
#include "tq_launch.h"

namespace tq {

namespace {

constexpr int GT = 1024;  // groups per expansion tile

// Two blocks of one group from its 32 code bytes c[0..7] (little-endian
// dwords) and its scale bits s: 9 dwords, [s | c0 c1], [c2..c5], ..,
// [c14 c15 | s], [c16..c19], .., [c28..c31].
__device__ __forceinline__ void store_two_blocks(uint32_t *o, const uint32_t (&c)[8], uint32_t s) {
  o[0] = s | (c[0] << 16);
  o[1] = __builtin_amdgcn_perm(c[1], c[0], 0x05040302u);
  o[2] = __builtin_amdgcn_perm(c[2], c[1], 0x05040302u);
  o[3] = __builtin_amdgcn_perm(c[3], c[2], 0x05040302u);
  o[4] = (c[3] >> 16) | (s << 16);
  o[5] = c[4];
  o[6] = c[5];
  o[7] = c[6];
  o[8] = c[7];
}

template <int FMT>
__global__ __launch_bounds__(256) void expand_g64_kernel(const uint8_t *__restrict__ base,
                                                         const uint8_t *__restrict__ high,
                                                         const uint16_t *__restrict__ scale,
                                                         uint8_t *__restrict__ out, int64_t groups) {
  // digit i of byte v = (v / 3^i) % 3, as the 2-bit field i
  __shared__ uint16_t lut[FMT == FMT_PTQ1 ? 256 : 1];
  if constexpr (FMT == FMT_PTQ1) {
    const int t = threadIdx.x;
    uint32_t v = (uint32_t)t, f = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      f |= (v % 3u) << (2 * i);
      v /= 3u;
    }
    lut[t] = (uint16_t)f;
    __syncthreads();
  }
  __shared__ __attribute__((aligned(16))) uint32_t tile_out[9 * GT];
  const int t = threadIdx.x;
  const int64_t tiles = (groups + GT - 1) / GT;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t g0 = tile * GT;
    const int R = (int)(groups - g0 < GT ? groups - g0 : GT);  // groups in this tile
#pragma unroll
    for (int j = 0; j < GT / 256; ++j) {
      const int gl = t + 256 * j;
      if (gl >= R) continue;
      const int64_t g = g0 + gl;
      uint32_t c[8];
      if constexpr (FMT == FMT_PQ2) {
        const u32x4 *b = reinterpret_cast<const u32x4 *>(base + 32 * g);
        const u32x4 lo = b[0], hi = b[1];
        c[0] = lo[0]; c[1] = lo[1]; c[2] = lo[2]; c[3] = lo[3];
        c[4] = hi[0]; c[5] = hi[1]; c[6] = hi[2]; c[7] = hi[3];
      } else {
        const u32x2 *b = reinterpret_cast<const u32x2 *>(base + 24 * g);
        const u32x2 b0 = b[0], b1 = b[1], b2 = b[2];
        const uint32_t bw[6] = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1]};
        const uint32_t hw = reinterpret_cast<const uint16_t *>(high)[g];
        uint64_t acc[4] = {0, 0, 0, 0};
#pragma unroll
        for (int bi = 0; bi < 24; ++bi) {
          const uint64_t f = lut[(bw[bi >> 2] >> (8 * (bi & 3))) & 0xFFu];
          const int pos = 10 * bi;  // trits 5bi.. -> code bits 10bi..
          acc[pos >> 6] |= f << (pos & 63);
          if ((pos & 63) > 54) acc[(pos >> 6) + 1] |= f >> (64 - (pos & 63));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // trits 120+4h.. -> code bits 240+8h..
          const uint64_t f = lut[(hw >> (8 * h)) & 0xFFu] & 0xFFu;
          acc[3] |= f << (48 + 8 * h);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[2 * i] = (uint32_t)acc[i];
          c[2 * i + 1] = (uint32_t)(acc[i] >> 32);
        }
      }
      store_two_blocks(tile_out + 9 * gl, c, scale[g]);
    }
    __syncthreads();
    uint8_t *o = out + 36 * g0;
    if (R == GT) {
#pragma unroll
      for (int j = 0; j < 9 * GT / 4 / 256; ++j)
        reinterpret_cast<u32x4 *>(o)[t + 256 * j] = reinterpret_cast<const u32x4 *>(tile_out)[t + 256 * j];
    } else {
      for (int i = t; i < 9 * R; i += 256) reinterpret_cast<uint32_t *>(o)[i] = tile_out[i];
    }
    __syncthreads();  // the tile is written out before the next one is built
  }
}

template <int XD>
hipError_t gemv_g64_dt(const Planes &p, const void *x, float *y, hipStream_t st) {
  switch (p.k / 1024) {
    case 1: return gemv_wave_go<LAY_G64, 0, 1, XD, false>(p, x, nullptr, y, st);
    case 2: return gemv_wave_go<LAY_G64, 0, 2, XD, false>(p, x, nullptr, y, st);
    case 3: return gemv_wave_go<LAY_G64, 0, 3, XD, false>(p, x, nullptr, y, st);
    case 4: return gemv_wave_go<LAY_G64, 1, 0, XD, false>(p, x, nullptr, y, st);
    case 5: return gemv_wave_go<LAY_G64, 1, 1, XD, false>(p, x, nullptr, y, st);
    case 6: return gemv_wave_go<LAY_G64, 1, 2, XD, false>(p, x, nullptr, y, st);
    case 7: return gemv_wave_go<LAY_G64, 1, 3, XD, false>(p, x, nullptr, y, st);
    case 8: return gemv_wave_go<LAY_G64, 2, 0, XD, false>(p, x, nullptr, y, st);
    case 9: return gemv_wave_go<LAY_G64, 2, 1, XD, false>(p, x, nullptr, y, st);
    case 10: return gemv_wave_go<LAY_G64, 2, 2, XD, false>(p, x, nullptr, y, st);
    case 11: return gemv_wave_go<LAY_G64, 2, 3, XD, false>(p, x, nullptr, y, st);
    case 12: return gemv_wave_go<LAY_G64, 3, 0, XD, false>(p, x, nullptr, y, st);
    case 13: return gemv_wave_go<LAY_G64, 3, 1, XD, false>(p, x, nullptr, y, st);
    case 14: return gemv_wave_go<LAY_G64, 3, 2, XD, false>(p, x, nullptr, y, st);
    case 15: return gemv_wave_go<LAY_G64, 3, 3, XD, false>(p, x, nullptr, y, st);
    case 16: return gemv_wave_go<LAY_G64, 4, 0, XD, false>(p, x, nullptr, y, st);
    default: return gemv_wave_go<LAY_G64, 4, 1, XD, false>(p, x, nullptr, y, st);
  }
}

}  // namespace

hipError_t launch_expand_g64(int fmt, const uint8_t *base, const uint8_t *high,
                             const uint16_t *scale, uint8_t *out, int64_t groups,
                             hipStream_t st) {
  if (groups <= 0) return hipSuccess;
  const int64_t want = (groups + GT - 1) / GT;
  const int64_t cap = (int64_t)device_cus() * 64;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  if (fmt == FMT_PQ2)
    hipLaunchKernelGGL(expand_g64_kernel<FMT_PQ2>, dim3(grid), dim3(256), 0, st, base, high, scale,
                       out, groups);
  else
    hipLaunchKernelGGL(expand_g64_kernel<FMT_PTQ1>, dim3(grid), dim3(256), 0, st, base, high,
                       scale, out, groups);
  return hipGetLastError();
}

hipError_t launch_gemv_g64(const uint8_t *blocks, int64_t n, int64_t k, const void *x, int x_dtype,
                           float *y, hipStream_t st) {
  Planes p{};
  p.base = blocks;
  p.n = n;
  p.k = k;
  p.groups = k / 128;
  p.base_row = 18 * (k / 64);
  p.fmt = FMT_PQ2;
  if (x_dtype == DT_F32) return gemv_g64_dt<DT_F32>(p, x, y, st);
  if (x_dtype == DT_BF16) return gemv_g64_dt<DT_BF16>(p, x, y, st);
  return gemv_g64_dt<DT_F16>(p, x, y, st);
}

}  // namespace tq
