// GGUF block stream <-> row-split planes ([ninfer-skill] §3-§4).
// A block is one (row, group) of 128 weights: PQ2_0_G128 stores
// [scale 2][base 32] (34 bytes), PTQ1_0_G128 [base 24][high 2][scale 2]
// (28 bytes); blocks follow each other row-major over (row, group).  The
// planes hold the same bytes plane by plane (base, high, scale), each plane
// row-major over (row, group), at the offsets of the row-split geometry.
// Because both sides are row-major over (row, group), block index =
// plane byte / bytes-per-group in every plane.
//
// Each thread produces eight consecutive output bytes and gathers them in
// 2-byte units from the other side; the padding between planes is written
// as zero.  Memory-bound; the gathers hit the caches.

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

template <int FMT>
struct BlockShape;
template <>
struct BlockShape<FMT_PQ2> {
  static constexpr int BLK = 34, BASE = 32, BASE_AT = 2, SCALE_AT = 0, HIGH = 0, HIGH_AT = 0;
};
template <>
struct BlockShape<FMT_PTQ1> {
  static constexpr int BLK = 28, BASE = 24, BASE_AT = 0, SCALE_AT = 26, HIGH = 2, HIGH_AT = 24;
};

struct PlaneOffsets {
  uint64_t base_bytes, high_offset, high_bytes, scale_offset, scale_bytes, payload_bytes, blocks_bytes;
};

// block-stream byte of payload byte o, or -1 for inter-plane padding
template <int FMT>
__device__ __forceinline__ int64_t block_byte_of_plane(uint64_t o, const PlaneOffsets &g) {
  using B = BlockShape<FMT>;
  if (o < g.base_bytes) return (int64_t)((o / B::BASE) * B::BLK + B::BASE_AT + o % B::BASE);
  if (B::HIGH > 0 && o >= g.high_offset && o < g.high_offset + g.high_bytes) {
    const uint64_t r = o - g.high_offset;
    return (int64_t)((r / B::HIGH) * B::BLK + B::HIGH_AT + r % B::HIGH);
  }
  if (o >= g.scale_offset && o < g.scale_offset + g.scale_bytes) {
    const uint64_t r = o - g.scale_offset;
    return (int64_t)((r / 2) * B::BLK + B::SCALE_AT + r % 2);
  }
  return -1;
}

// payload byte of block-stream byte o
template <int FMT>
__device__ __forceinline__ uint64_t plane_byte_of_block(uint64_t o, const PlaneOffsets &g) {
  using B = BlockShape<FMT>;
  const uint64_t idx = o / B::BLK;
  const int off = (int)(o % B::BLK);
  if (off >= B::BASE_AT && off < B::BASE_AT + B::BASE) return idx * B::BASE + (off - B::BASE_AT);
  if (B::HIGH > 0 && off >= B::HIGH_AT && off < B::HIGH_AT + B::HIGH)
    return g.high_offset + idx * B::HIGH + (off - B::HIGH_AT);
  return g.scale_offset + idx * 2 + (off - B::SCALE_AT);
}

// Every field of both layouts starts on an even byte and has even length
// (blocks of 34 or 28 bytes, planes 256-aligned), so the gathers are of
// 2-byte units: each thread produces eight output bytes from four of them.
template <int FMT, bool TO_PLANES>
__global__ __launch_bounds__(256) void transcode_kernel(const uint8_t *__restrict__ src,
                                                        uint8_t *__restrict__ dst, PlaneOffsets g) {
  const uint64_t out_bytes = TO_PLANES ? g.payload_bytes : g.blocks_bytes;  // even
  const uint64_t units = out_bytes / 2;
  const uint16_t *s16 = reinterpret_cast<const uint16_t *>(src);
  for (uint64_t u0 = 4 * ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x); u0 < units;
       u0 += 4 * (uint64_t)gridDim.x * blockDim.x) {
    uint32_t h[4] = {0u, 0u, 0u, 0u};
    const int nu = units - u0 < 4 ? (int)(units - u0) : 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nu) {
        if constexpr (TO_PLANES) {
          const int64_t sb = block_byte_of_plane<FMT>(2 * (u0 + i), g);
          if (sb >= 0) h[i] = s16[sb / 2];
        } else {
          h[i] = s16[plane_byte_of_block<FMT>(2 * (u0 + i), g) / 2];
        }
      }
    }
    if (nu == 4 && (2 * u0) % 8 == 0) {
      *reinterpret_cast<u32x2 *>(dst + 2 * u0) = (u32x2){h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    } else {
      uint16_t *d16 = reinterpret_cast<uint16_t *>(dst);
      for (int i = 0; i < nu; ++i) d16[u0 + i] = (uint16_t)h[i];
    }
  }
}

template <bool TO_PLANES>
hipError_t transcode_go(int fmt, const uint8_t *src, uint8_t *dst, const PlaneOffsets &g,
                        hipStream_t st) {
  const uint64_t out = TO_PLANES ? g.payload_bytes : g.blocks_bytes;
  const uint64_t quads = (out / 2 + 3) / 4;  // four 2-byte units per thread
  uint64_t wgs = (quads + 255) / 256;
  const uint64_t cap = (uint64_t)device_cus() * 16;  // a grid-stride loop beyond that
  if (wgs > cap) wgs = cap;
  if (wgs == 0) return hipSuccess;
  if (fmt == FMT_PQ2)
    hipLaunchKernelGGL((transcode_kernel<FMT_PQ2, TO_PLANES>), dim3((unsigned)wgs), dim3(256), 0, st,
                       src, dst, g);
  else
    hipLaunchKernelGGL((transcode_kernel<FMT_PTQ1, TO_PLANES>), dim3((unsigned)wgs), dim3(256), 0,
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
