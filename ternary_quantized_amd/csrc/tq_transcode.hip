// GGUF block stream <-> row-split planes ([ninfer-skill] §3-§4).
// A block is one (row, group) of 128 weights: PQ2_0_G128 stores
// [scale 2][base 32] (34 bytes), PTQ1_0_G128 [base 24][high 2][scale 2]
// (28 bytes); blocks follow each other row-major over (row, group).  The
// planes hold the same bytes plane by plane (base, high, scale), each plane
// row-major over (row, group), at the offsets of the row-split geometry, so
// block b owns bytes [b*base, (b+1)*base) of the base plane and the b-th
// entry of the high and scale planes.
//
// Each thread moves whole blocks, reading every source byte once and
// writing every destination byte once (HBM-bound: algorithmic bytes =
// block stream + payload).  PTQ1_0 blocks are 28 bytes, so one block is
// seven aligned dwords.  PQ2_0 blocks are 34 bytes, so a thread takes a pair
// (68 bytes = 17 aligned dwords): the first block's 32 base bytes sit 2
// bytes past a dword boundary and are realigned with byte permutes, the
// second block's lie on dword boundaries.  An odd last PQ2_0 block is moved
// by one thread on its own.  The padding between planes (less than 256
// bytes before each plane) is written as zero by the first workgroup.

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {
namespace {

struct PlaneOffsets {
  uint64_t base_bytes, high_offset, high_bytes, scale_offset, scale_bytes, payload_bytes, blocks_bytes;
};

// bytes 2..5 of the pair (lo, hi): a dword that starts 2 bytes into lo
__device__ __forceinline__ uint32_t shift2(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x05040302u);
}

template <int FMT, bool TO_PLANES>
__global__ __launch_bounds__(256) void transcode_kernel(const uint8_t *__restrict__ src,
                                                        uint8_t *__restrict__ dst, PlaneOffsets g) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (TO_PLANES && blockIdx.x == 0) {
    // zero the padding between the planes
    const uint64_t pad1 = g.high_offset - g.base_bytes;
    const uint64_t hend = g.high_offset + g.high_bytes;
    const uint64_t pad2 = g.scale_offset - hend;
    for (uint64_t i = threadIdx.x; i < pad1 + pad2; i += blockDim.x)
      dst[i < pad1 ? g.base_bytes + i : hend + (i - pad1)] = 0;
  }
  if constexpr (FMT == FMT_PTQ1) {
    const uint64_t blocks = g.blocks_bytes / 28;
    for (uint64_t b = tid; b < blocks; b += stride) {
      uint32_t *bw = reinterpret_cast<uint32_t *>(TO_PLANES ? nullptr : dst + 28 * b);
      u32x2 *pb = reinterpret_cast<u32x2 *>((TO_PLANES ? dst : const_cast<uint8_t *>(src)) + 24 * b);
      uint16_t *ph = reinterpret_cast<uint16_t *>((TO_PLANES ? dst : const_cast<uint8_t *>(src)) +
                                                  g.high_offset + 2 * b);
      uint16_t *ps = reinterpret_cast<uint16_t *>((TO_PLANES ? dst : const_cast<uint8_t *>(src)) +
                                                  g.scale_offset + 2 * b);
      if constexpr (TO_PLANES) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(src + 28 * b);
        uint32_t v[7];
#pragma unroll
        for (int i = 0; i < 7; ++i) v[i] = w[i];
        pb[0] = (u32x2){v[0], v[1]};
        pb[1] = (u32x2){v[2], v[3]};
        pb[2] = (u32x2){v[4], v[5]};
        *ph = (uint16_t)v[6];
        *ps = (uint16_t)(v[6] >> 16);
      } else {
        const u32x2 a = pb[0], c = pb[1], d = pb[2];
        const uint32_t hs = (uint32_t)*ph | ((uint32_t)*ps << 16);
        const uint32_t v[7] = {a[0], a[1], c[0], c[1], d[0], d[1], hs};
#pragma unroll
        for (int i = 0; i < 7; ++i) bw[i] = v[i];
      }
    }
  } else {
    const uint64_t blocks = g.blocks_bytes / 34, pairs = blocks / 2;
    for (uint64_t p = tid; p < pairs; p += stride) {
      uint32_t *pbase = reinterpret_cast<uint32_t *>((TO_PLANES ? dst : const_cast<uint8_t *>(src)) + 64 * p);
      uint32_t *pscale = reinterpret_cast<uint32_t *>((TO_PLANES ? dst : const_cast<uint8_t *>(src)) +
                                                      g.scale_offset + 4 * p);
      if constexpr (TO_PLANES) {
        // w[0] = [s0 | c0 c1], w[1..7], w[8] = [c30 c31 | s1], w[9..16] = block 2p+1's codes
        const uint32_t *s = reinterpret_cast<const uint32_t *>(src + 68 * p);
        uint32_t w[17];
#pragma unroll
        for (int i = 0; i < 17; ++i) w[i] = s[i];
        u32x4 *ob = reinterpret_cast<u32x4 *>(pbase);
        ob[0] = (u32x4){shift2(w[0], w[1]), shift2(w[1], w[2]), shift2(w[2], w[3]), shift2(w[3], w[4])};
        ob[1] = (u32x4){shift2(w[4], w[5]), shift2(w[5], w[6]), shift2(w[6], w[7]), shift2(w[7], w[8])};
        ob[2] = (u32x4){w[9], w[10], w[11], w[12]};
        ob[3] = (u32x4){w[13], w[14], w[15], w[16]};
        *pscale = (w[0] & 0xFFFFu) | (w[8] & 0xFFFF0000u);
      } else {
        const u32x4 *ib = reinterpret_cast<const u32x4 *>(pbase);
        const u32x4 q0 = ib[0], q1 = ib[1], q2 = ib[2], q3 = ib[3];
        const uint32_t c[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        const uint32_t sc = *pscale;
        uint32_t *o = reinterpret_cast<uint32_t *>(dst + 68 * p);
        o[0] = (sc & 0xFFFFu) | (c[0] << 16);
#pragma unroll
        for (int i = 1; i < 8; ++i) o[i] = shift2(c[i - 1], c[i]);
        o[8] = (c[7] >> 16) | (sc & 0xFFFF0000u);
        o[9] = q2[0]; o[10] = q2[1]; o[11] = q2[2]; o[12] = q2[3];
        o[13] = q3[0]; o[14] = q3[1]; o[15] = q3[2]; o[16] = q3[3];
      }
    }
    // an odd last block, 34 bytes from a dword boundary (its index is even)
    if ((blocks & 1) && tid == pairs % stride) {
      const uint64_t b = blocks - 1;
      const uint16_t *s16 = reinterpret_cast<const uint16_t *>(src);
      uint16_t *d16 = reinterpret_cast<uint16_t *>(dst);
      if constexpr (TO_PLANES) {
        for (int i = 0; i < 16; ++i) d16[(32 * b) / 2 + i] = s16[(34 * b) / 2 + 1 + i];
        d16[(g.scale_offset + 2 * b) / 2] = s16[(34 * b) / 2];
      } else {
        d16[(34 * b) / 2] = s16[(g.scale_offset + 2 * b) / 2];
        for (int i = 0; i < 16; ++i) d16[(34 * b) / 2 + 1 + i] = s16[(32 * b) / 2 + i];
      }
    }
  }
}

template <bool TO_PLANES>
hipError_t transcode_go(int fmt, const uint8_t *src, uint8_t *dst, const PlaneOffsets &g,
                        hipStream_t st) {
  const uint64_t items = fmt == FMT_PQ2 ? (g.blocks_bytes / 34 + 1) / 2 : g.blocks_bytes / 28;
  uint64_t wgs = (items + 255) / 256;
  const uint64_t cap = (uint64_t)device_cus() * 16;  // a grid-stride loop beyond that
  if (wgs > cap) wgs = cap;
  if (wgs == 0) wgs = 1;  // (the padding is still written)
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
