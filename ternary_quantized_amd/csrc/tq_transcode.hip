// GGUF block stream <-> row-split planes ([ninfer-skill] §3-§4).
// A block is one (row, group) of 128 weights: PQ2_0_G128 stores
// [scale 2][base 32] (34 bytes), PTQ1_0_G128 [base 24][high 2][scale 2]
// (28 bytes); blocks follow each other row-major over (row, group).  The
// planes hold the same bytes plane by plane (base, high, scale), each plane
// row-major over (row, group), at the offsets of the row-split geometry, so
// block b owns bytes [b*base, (b+1)*base) of the base plane and the b-th
// entry of the high and scale planes.
//
// A workgroup moves a tile of TILE = 1024 consecutive blocks through LDS, so
// that both sides stay contiguous across lanes: the tile's span of the block
// stream is read (or written) as 8-byte words, lane after lane, and its
// spans of the three planes as 16-byte chunks (base) and 4-byte words (high,
// scale), lane after lane.  Every source byte is read once and every
// destination byte written once (HBM-bound: algorithmic bytes = block stream
// + payload).  In LDS the tile sits in block-stream order; a plane chunk is
// gathered from (or scattered to) it at the block's offsets.  PQ2_0 blocks
// are 34 bytes, so an even block's codes start 2 bytes past a dword boundary
// and are realigned with byte shifts; PTQ1_0 blocks are 7 whole dwords.  The
// last, partial tile moves its block-stream span 2 bytes at a time (34 * R
// bytes need not fill whole words) and writes a lone last half-pair of the
// 2-byte planes alone.  The padding between planes (less than 256 bytes
// before each plane) is written as zero by the first workgroup.

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

constexpr int TILE = 1024;  // blocks per tile
constexpr int TPB = 256;    // threads per workgroup

struct PlaneOffsets {
  uint64_t base_bytes, high_offset, high_bytes, scale_offset, scale_bytes, payload_bytes, blocks_bytes;
};

template <int FMT>
struct BlockShape {
  static constexpr int BYTES = FMT == FMT_PQ2 ? 34 : 28;  // block stream bytes per block
  static constexpr int BASE = FMT == FMT_PQ2 ? 32 : 24;   // base plane bytes per block
  static constexpr int TBYTES = BYTES * TILE;             // a tile of the block stream
};

// LDS byte offset of the b-th block's base byte 0 inside the tile
template <int FMT>
__device__ __forceinline__ int base_at(int b) {
  return FMT == FMT_PQ2 ? 34 * b + 2 : 28 * b;
}

template <int FMT, bool TO_PLANES>
__global__ __launch_bounds__(TPB) void transcode_kernel(const uint8_t *__restrict__ src,
                                                        uint8_t *__restrict__ dst, PlaneOffsets g) {
  using S = BlockShape<FMT>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[S::TBYTES / 4 + 4];
  uint16_t *lds16 = reinterpret_cast<uint16_t *>(lds);
  const int t = threadIdx.x;
  const uint64_t blocks = g.blocks_bytes / S::BYTES;
  const uint64_t tiles = (blocks + TILE - 1) / TILE;

  if (TO_PLANES && blockIdx.x == 0) {
    // zero the padding between the planes
    const uint64_t pad1 = g.high_offset - g.base_bytes;
    const uint64_t hend = g.high_offset + g.high_bytes;
    const uint64_t pad2 = g.scale_offset - hend;
    for (uint64_t i = t; i < pad1 + pad2; i += TPB) dst[i < pad1 ? g.base_bytes + i : hend + (i - pad1)] = 0;
  }

  // the tile's stretches: block stream, base plane, and the 2-byte planes
  // (high for PTQ1_0, scale for both)
  const uint8_t *blk_src = TO_PLANES ? src : nullptr;
  uint8_t *blk_dst = TO_PLANES ? nullptr : dst;
  const uint8_t *pay_src = TO_PLANES ? nullptr : src;
  uint8_t *pay_dst = TO_PLANES ? dst : nullptr;

  for (uint64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const uint64_t b0 = tile * TILE;
    const int R = (int)(blocks - b0 < (uint64_t)TILE ? blocks - b0 : (uint64_t)TILE);  // blocks here
    const bool full = R == TILE;
    const uint64_t bs_off = b0 * S::BYTES, base_off = b0 * S::BASE;
    // words of 2 bytes per block: u covers blocks 2u, 2u+1
    auto two_byte_planes = [&](auto fn) {
      for (int u = t; 2 * u < R; u += TPB) fn(u, 2 * u + 1 < R);
    };

    if constexpr (TO_PLANES) {
      // ---- block stream -> LDS
      if (full) {
        const u32x2 *s8 = reinterpret_cast<const u32x2 *>(blk_src + bs_off);
        u32x2 *l8 = reinterpret_cast<u32x2 *>(lds);
#pragma unroll
        for (int j = 0; j < S::TBYTES / 8 / TPB; ++j) l8[t + TPB * j] = s8[t + TPB * j];
      } else {
        const uint16_t *s2 = reinterpret_cast<const uint16_t *>(blk_src + bs_off);
        for (int i = t; i < R * S::BYTES / 2; i += TPB) lds16[i] = s2[i];
      }
      __syncthreads();
      // ---- base plane: 16-byte chunks c (a partial last chunk as 8 bytes)
      const int base_len = R * S::BASE;
      u32x4 *pb = reinterpret_cast<u32x4 *>(pay_dst + base_off);
      for (int c = t; 16 * c < base_len; c += TPB) {
        uint32_t w[4];
        if constexpr (FMT == FMT_PQ2) {
          const int off = base_at<FMT>(c >> 1) + 16 * (c & 1);
          const int a = off >> 2, sh = off & 3;  // sh is 0 or 2
          const uint32_t d0 = lds[a], d1 = lds[a + 1], d2 = lds[a + 2], d3 = lds[a + 3], d4 = lds[a + 4];
          w[0] = __builtin_amdgcn_alignbyte(d1, d0, sh);
          w[1] = __builtin_amdgcn_alignbyte(d2, d1, sh);
          w[2] = __builtin_amdgcn_alignbyte(d3, d2, sh);
          w[3] = __builtin_amdgcn_alignbyte(d4, d3, sh);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 16 * c + 4 * j;  // base byte of the tile, a multiple of 4
            w[j] = lds[7 * (i / 24) + (i % 24) / 4];
          }
        }
        if (16 * c + 16 <= base_len)
          pb[c] = (u32x4){w[0], w[1], w[2], w[3]};
        else
          *reinterpret_cast<u32x2 *>(pb + c) = (u32x2){w[0], w[1]};
      }
      // ---- 2-byte planes
      uint32_t *ps = reinterpret_cast<uint32_t *>(pay_dst + g.scale_offset + 2 * b0);
      uint32_t *ph = reinterpret_cast<uint32_t *>(pay_dst + g.high_offset + 2 * b0);
      two_byte_planes([&](int u, bool pair) {
        uint32_t sc, hi = 0;
        if constexpr (FMT == FMT_PQ2) {
          // scales at bytes 34b: the low half of dword 17u, the high half of 17u + 8
          sc = (lds[17 * u] & 0xFFFFu) | (lds[17 * u + 8] & 0xFFFF0000u);
        } else {
          const uint32_t e0 = lds[14 * u + 6], e1 = lds[14 * u + 13];  // [high | scale] of 2u, 2u+1
          hi = (e0 & 0xFFFFu) | (e1 << 16);
          sc = (e0 >> 16) | (e1 & 0xFFFF0000u);
        }
        if (pair) {
          ps[u] = sc;
          if constexpr (FMT == FMT_PTQ1) ph[u] = hi;
        } else {
          reinterpret_cast<uint16_t *>(ps)[2 * u] = (uint16_t)sc;
          if constexpr (FMT == FMT_PTQ1) reinterpret_cast<uint16_t *>(ph)[2 * u] = (uint16_t)hi;
        }
      });
    } else {
      // ---- base plane -> LDS
      const int base_len = R * S::BASE;
      const u32x4 *pb = reinterpret_cast<const u32x4 *>(pay_src + base_off);
      for (int c = t; 16 * c < base_len; c += TPB) {
        u32x4 v;
        if (16 * c + 16 <= base_len) {
          v = pb[c];
        } else {
          const u32x2 h = *reinterpret_cast<const u32x2 *>(pb + c);
          v = (u32x4){h[0], h[1], 0u, 0u};
        }
        const int nw = 16 * c + 16 <= base_len ? 4 : 2;
        if constexpr (FMT == FMT_PQ2) {
          const int off = base_at<FMT>(c >> 1) + 16 * (c & 1);
          if ((off & 3) == 0) {
            for (int j = 0; j < nw; ++j) lds[(off >> 2) + j] = v[j];
          } else {
            // 2 bytes past a dword boundary: a half word, whole realigned
            // words, and a closing half word
            lds16[off >> 1] = (uint16_t)v[0];
            for (int j = 0; j + 1 < nw; ++j) lds[(off + 2) / 4 + j] = (v[j] >> 16) | (v[j + 1] << 16);
            lds16[(off >> 1) + 2 * nw - 1] = (uint16_t)(v[nw - 1] >> 16);
          }
        } else {
          for (int j = 0; j < nw; ++j) {
            const int i = 16 * c + 4 * j;
            lds[7 * (i / 24) + (i % 24) / 4] = v[j];
          }
        }
      }
      const uint32_t *ps = reinterpret_cast<const uint32_t *>(pay_src + g.scale_offset + 2 * b0);
      const uint32_t *ph = reinterpret_cast<const uint32_t *>(pay_src + g.high_offset + 2 * b0);
      two_byte_planes([&](int u, bool pair) {
        const uint16_t *ps2 = reinterpret_cast<const uint16_t *>(ps);
        const uint16_t *ph2 = reinterpret_cast<const uint16_t *>(ph);
        const uint32_t sc = pair ? ps[u] : ps2[2 * u];
        if constexpr (FMT == FMT_PQ2) {
          lds16[17 * (2 * u)] = (uint16_t)sc;  // byte 34b, b = 2u
          if (pair) lds16[17 * (2 * u + 1)] = (uint16_t)(sc >> 16);
        } else {
          const uint32_t hi = pair ? ph[u] : ph2[2 * u];
          lds[14 * u + 6] = (hi & 0xFFFFu) | (sc << 16);
          if (pair) lds[14 * u + 13] = (hi >> 16) | (sc & 0xFFFF0000u);
        }
      });
      __syncthreads();
      // ---- LDS -> block stream
      if (full) {
        u32x2 *d8 = reinterpret_cast<u32x2 *>(blk_dst + bs_off);
        const u32x2 *l8 = reinterpret_cast<const u32x2 *>(lds);
#pragma unroll
        for (int j = 0; j < S::TBYTES / 8 / TPB; ++j) d8[t + TPB * j] = l8[t + TPB * j];
      } else {
        uint16_t *d2 = reinterpret_cast<uint16_t *>(blk_dst + bs_off);
        for (int i = t; i < R * S::BYTES / 2; i += TPB) d2[i] = lds16[i];
      }
    }
    __syncthreads();  // the tile's LDS is read before the next tile overwrites it
  }
}

template <bool TO_PLANES>
hipError_t transcode_go(int fmt, const uint8_t *src, uint8_t *dst, const PlaneOffsets &g,
                        hipStream_t st) {
  const uint64_t blocks = g.blocks_bytes / (fmt == FMT_PQ2 ? 34 : 28);
  uint64_t wgs = (blocks + TILE - 1) / TILE;
  const uint64_t cap = (uint64_t)device_cus() * 64;  // a grid-stride loop over tiles beyond that
  if (wgs > cap) wgs = cap;
  if (wgs == 0) wgs = 1;  // (the padding is still written)
  if (fmt == FMT_PQ2)
    hipLaunchKernelGGL((transcode_kernel<FMT_PQ2, TO_PLANES>), dim3((unsigned)wgs), dim3(TPB), 0, st,
                       src, dst, g);
  else
    hipLaunchKernelGGL((transcode_kernel<FMT_PTQ1, TO_PLANES>), dim3((unsigned)wgs), dim3(TPB), 0,
                       st, src, dst, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transcode(int fmt, bool to_planes, const uint8_t *src, uint8_t *dst,
                            uint64_t base_bytes, uint64_t high_offset, uint64_t high_bytes,
                            uint64_t scale_offset, uint64_t scale_bytes, uint64_t payload_bytes,
                            uint64_t blocks_bytes, hipStream_t st) {
  PlaneOffsets g{base_bytes, high_offset, high_bytes, scale_offset, scale_bytes, payload_bytes,
                 blocks_bytes};
  return to_planes ? transcode_go<true>(fmt, src, dst, g, st) : transcode_go<false>(fmt, src, dst, g, st);
}

}  // namespace tq
