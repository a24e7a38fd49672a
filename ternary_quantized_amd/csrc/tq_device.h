// Device helpers shared by the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
enum { FMT_PQ2 = 142, FMT_PTQ1 = 143 };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> binary16 bits (hardware conversion, round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// A pair of 2-bit codes -> the pair of binary16 trits code - 1, exactly:
// (p & mask_i) | 0x6400_6400 holds 1024 + 4^i * code in each half (i is the
// code's 2-bit slot, 0..4), and fma(v, 4^-i, -(1024 * 4^-i + 1)) = code - 1.
// Every value involved is a normal binary16.
template <int I>
__device__ __forceinline__ uint32_t trit_pair(uint32_t p, uint32_t magic_v) {
  constexpr uint32_t mask = 0x00030003u << (2 * I);
  constexpr float inv = I == 0 ? 1.0f : I == 1 ? 0.25f : I == 2 ? 0.0625f : I == 3 ? 0.015625f
                                                                                   : 0.00390625f;
  constexpr float neg = I == 0 ? -1025.0f : I == 1 ? -257.0f : I == 2 ? -65.0f : I == 3 ? -17.0f
                                                                                        : -5.0f;
  const half2_t t = __builtin_bit_cast(half2_t, (p & mask) | magic_v);
  const half2_t m = {(_Float16)inv, (_Float16)inv};
  const half2_t c = {(_Float16)neg, (_Float16)neg};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(t, m, c));
}

template <int DT>
__device__ __forceinline__ float load_elem(const void *p, int64_t i) {
  if constexpr (DT == DT_F32) return static_cast<const float *>(p)[i];
  else if constexpr (DT == DT_BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return f16_to_f32(static_cast<const uint16_t *>(p)[i]);
}

// Load 16 consecutive elements starting at element i (16-byte aligned).
template <int DT>
__device__ __forceinline__ void load16(const void *p, int64_t i, float v[16]) {
  if constexpr (DT == DT_F32) {
    const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 t = q[j];
      v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
    }
  } else {
    const uint4 *q = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 t = q[j];
      uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint16_t lo = (uint16_t)(w[e] & 0xFFFF), hi = (uint16_t)(w[e] >> 16);
        if constexpr (DT == DT_BF16) {
          v[8 * j + 2 * e] = bf16_to_f32(lo);
          v[8 * j + 2 * e + 1] = bf16_to_f32(hi);
        } else {
          v[8 * j + 2 * e] = f16_to_f32(lo);
          v[8 * j + 2 * e + 1] = f16_to_f32(hi);
        }
      }
    }
  }
}

// Store 16 consecutive elements at element i (16-byte aligned).
// load16 split in two: the raw 16-byte vectors of 16 elements (issue), and
// their conversion to fp32 (use), so that other loads can be issued between.
template <int DT>
struct Raw16 {
  u32x4 q[DT == DT_F32 ? 4 : 2];
};

template <int DT>
__device__ __forceinline__ void load16_raw(const void *p, int64_t i, Raw16<DT> &r) {
  const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p) +
                                                    i * (DT == DT_F32 ? 4 : 2));
#pragma unroll
  for (int j = 0; j < (DT == DT_F32 ? 4 : 2); ++j) r.q[j] = q[j];
}

template <int DT>
__device__ __forceinline__ void convert16(const Raw16<DT> &r, float v[16]) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = __uint_as_float(r.q[j][e]);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t lo = (uint16_t)(r.q[j][e] & 0xFFFF), hi = (uint16_t)(r.q[j][e] >> 16);
        if constexpr (DT == DT_BF16) {
          v[8 * j + 2 * e] = bf16_to_f32(lo);
          v[8 * j + 2 * e + 1] = bf16_to_f32(hi);
        } else {
          v[8 * j + 2 * e] = f16_to_f32(lo);
          v[8 * j + 2 * e + 1] = f16_to_f32(hi);
        }
      }
  }
}

template <int DT>
__device__ __forceinline__ void store16(void *p, int64_t i, const float v[16]) {
  if constexpr (DT == DT_F32) {
    float4 *q = reinterpret_cast<float4 *>(static_cast<float *>(p) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  } else {
    uint4 *q = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p) + i);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo, hi;
        if constexpr (DT == DT_BF16) {
          lo = f32_to_bf16(v[8 * j + 2 * e]);
          hi = f32_to_bf16(v[8 * j + 2 * e + 1]);
        } else {
          lo = f32_to_f16(v[8 * j + 2 * e]);
          hi = f32_to_f16(v[8 * j + 2 * e + 1]);
        }
        w[e] = lo | (hi << 16);
      }
      q[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Flip the sign of v where the bf16 sign entry has its sign bit set (exact).
__device__ __forceinline__ float apply_sign(float v, uint16_t s) {
  return __uint_as_float(__float_as_uint(v) ^ ((uint32_t)(s & 0x8000u) << 16));
}

// In-wave Walsh-Hadamard butterfly of one 1024-element block (unnormalised
// Sylvester transform, natural order).  On entry lane l holds elements
// 16l + i in v[i]; on return v[i] holds element wht_out_index(l, i) =
// (i & 3) + 4l + 256(i >> 2).  All butterflies run inside registers, in the
// order of the index bits 0, 1, ..., 9 (each a + b for the lower element and
// a - b for the upper one), with two transposes through the wave's private
// scratch `sc` (1024 floats in LDS) in between:
//   bits 0-3: v[i] = element 16l + i
//   bits 4-7: after the first transpose, v[i] = element (l & 15) + 16i + 256(l >> 4)
//   bits 8-9: after the second, v[i] = element (i & 3) + 4l + 256(i >> 2)
// A wave's LDS operations complete in order, so no barrier is needed.
__device__ __forceinline__ int wht_out_index(int lane, int i) {
  return (i & 3) + 4 * lane + 256 * (i >> 2);
}

template <int HFIRST, int HLAST>
__device__ __forceinline__ void wht_regs(float v[16]) {
#pragma unroll
  for (int h = HFIRST; h <= HLAST; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// The wave's scratch holds the block as four quarters of 256 floats, each
// followed by 16 words of padding: in the strided transpose the lanes l,
// l+16, l+32 and l+48 read and write element 16i + l%16 of quarter l/16,
// which without the padding fall on one bank.
constexpr int WHT_SCRATCH = 1024 + 3 * 16;

__device__ __forceinline__ void wht1024_wave(float v[16], int lane, float *sc) {
  const int qp = 16 * (lane >> 4);  // the padding before the lane's quarter
  wht_regs<1, 8>(v);
  {
    u32x4 *w = reinterpret_cast<u32x4 *>(sc + 16 * lane + qp);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (u32x4){__float_as_uint(v[4 * j]), __float_as_uint(v[4 * j + 1]),
                     __float_as_uint(v[4 * j + 2]), __float_as_uint(v[4 * j + 3])};
  }
  const int t1 = (lane & 15) + 256 * (lane >> 4) + qp;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = sc[t1 + 16 * i];
  wht_regs<1, 8>(v);
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[t1 + 16 * i] = v[i];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const u32x4 r = *reinterpret_cast<const u32x4 *>(sc + 4 * lane + 272 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * g + j] = __uint_as_float(r[j]);
  }
  wht_regs<4, 8>(v);
}

// 4 consecutive elements (as fp32) to/from memory of type DT.
template <int DT>
__device__ __forceinline__ void store4(void *p, int64_t i, const float v[4]) {
  if constexpr (DT == DT_F32) {
    *reinterpret_cast<float4 *>(static_cast<float *>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint32_t w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint32_t lo, hi;
      if constexpr (DT == DT_BF16) {
        lo = f32_to_bf16(v[2 * e]);
        hi = f32_to_bf16(v[2 * e + 1]);
      } else {
        lo = f32_to_f16(v[2 * e]);
        hi = f32_to_f16(v[2 * e + 1]);
      }
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p) + i) = (u32x2){w[0], w[1]};
  }
}

}  // namespace tq
