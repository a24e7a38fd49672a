// Signed blockwise Walsh-Hadamard transform and the embedding-row gather.
//
// [tensorsharp] §4.2: a projection input gets H(D.x)/sqrt(1024) per block, an
// embedding row gets D.(H.x)/sqrt(1024); [ninfer-v3] §8 hadamard_signs:
// 1024-element blocks, signs stored as bf16 +-1, normalised Sylvester
// Walsh-Hadamard transform.  [tensorsharp] §4.4: the embedding row is looked
// up, dequantised and inverse-transformed.
//
// One wave transforms one 1024-element block: each lane loads 16 consecutive
// elements (one 64-byte fp32 / 32-byte 16-bit vector load per lane, so a
// wave reads the block as one contiguous span); every butterfly runs in
// registers, with two transposes through the wave's own LDS scratch (see
// wht1024_wave), and each lane writes its results as four runs of four
// consecutive elements.  The 1/32 normalisation and the sign flips are exact.

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {

// Forward transforms may read their input in the grouped head order
// ([ninfer-skill] §5 perm_row; [tensorsharp] §4.2: the GatedDeltaNet output
// is reordered into the publisher's head order before its transform): with
// tiles > 0, element j of the transform input is x[src(j)], j = h*head_dim +
// i taken from head (h % tiles)*groups + h/tiles.  head_dim is a multiple of
// 16, so a lane's 16 elements stay one contiguous load.
template <int XD, int YD>
__global__ __launch_bounds__(256) void hadamard_kernel(
    const void *x, int64_t ldx, int64_t rows, int64_t nblocks,
    const uint16_t *__restrict__ signs, int inverse, void *y, int64_t ldy,
    int tiles, int groups, int head_dim) {
  __shared__ __attribute__((aligned(16))) float scratch[4][WHT_SCRATCH];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  if (item >= rows * nblocks) return;
  const int64_t row = item / nblocks;
  const int64_t blk = (item % nblocks) * 1024;
  const int64_t col = blk + 16 * lane;

  int64_t src = col;
  if (tiles > 0) {
    const int h = (int)col / head_dim;
    src = (int64_t)((h % tiles) * groups + h / tiles) * head_dim + (col - (int64_t)h * head_dim);
  }
  float v[16];
  load16<XD>(x, row * ldx + src, v);
  if (!inverse) {
    const uint4 *sp = reinterpret_cast<const uint4 *>(signs + col);
    uint4 a = sp[0], b = sp[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = apply_sign(v[i], (uint16_t)(w[i >> 1] >> (16 * (i & 1))));
  }
  wht1024_wave(v, lane, scratch[wave]);
  // v[4g + j] now holds element blk + 256g + 4*lane + j
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t c = blk + 256 * g + 4 * lane;
    float o[4];
    if (inverse) {
      const u32x2 sw = *reinterpret_cast<const u32x2 *>(signs + c);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = apply_sign(v[4 * g + j] * 0.03125f, (uint16_t)(sw[j >> 1] >> (16 * (j & 1))));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = v[4 * g + j] * 0.03125f;
    }
    store4<YD>(y, row * ldy + c, o);
  }
}

template <int XD>
static hipError_t launch_h2(const void *x, int64_t rows, int64_t k, int64_t ldx,
                            const uint16_t *signs, int inverse, void *y, int yd,
                            int64_t ldy, hipStream_t st, int tiles, int groups, int head_dim) {
  const int64_t nblocks = k / 1024;
  const int64_t items = rows * nblocks;
  dim3 grid((unsigned)((items + 3) / 4)), block(256);
  switch (yd) {
    case DT_F32:
      hipLaunchKernelGGL((hadamard_kernel<XD, DT_F32>), grid, block, 0, st, x, ldx,
                         rows, nblocks, signs, inverse, y, ldy, tiles, groups, head_dim);
      break;
    case DT_BF16:
      hipLaunchKernelGGL((hadamard_kernel<XD, DT_BF16>), grid, block, 0, st, x, ldx,
                         rows, nblocks, signs, inverse, y, ldy, tiles, groups, head_dim);
      break;
    default:
      hipLaunchKernelGGL((hadamard_kernel<XD, DT_F16>), grid, block, 0, st, x, ldx,
                         rows, nblocks, signs, inverse, y, ldy, tiles, groups, head_dim);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_hadamard(const void *x, int xd, int64_t rows, int64_t k,
                           int64_t ldx, const uint16_t *signs, int inverse,
                           void *y, int yd, int64_t ldy, hipStream_t st, int tiles,
                           int groups, int head_dim) {
  switch (xd) {
    case DT_F32:
      return launch_h2<DT_F32>(x, rows, k, ldx, signs, inverse, y, yd, ldy, st, tiles, groups, head_dim);
    case DT_BF16:
      return launch_h2<DT_BF16>(x, rows, k, ldx, signs, inverse, y, yd, ldy, st, tiles, groups, head_dim);
    default:
      return launch_h2<DT_F16>(x, rows, k, ldx, signs, inverse, y, yd, ldy, st, tiles, groups, head_dim);
  }
}

// ------------------------------------------------------------ embedding ---
// Decode 16 consecutive weights (columns col..col+15, inside one 128-group)
// of row `row` to fp32 values code*scale.
template <int FMT>
__device__ __forceinline__ void decode16(const Planes &p, int64_t row, int64_t col,
                                         float w[16]) {
  const int64_t g = col >> 7;
  const float s = f16_to_f32(p.scale[row * p.groups + g]);
  const int j0 = (int)(col & 127);
  if constexpr (FMT == FMT_PQ2) {
    // [gguf-explainer] §4.3: weight j at byte j/4, bits 2*(j%4), value code-1.
    const uint32_t d = *reinterpret_cast<const uint32_t *>(
        p.base + row * p.base_row + g * 32 + (j0 >> 2));
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = (float)((int)((d >> (2 * i)) & 3u) - 1) * s;
  } else {
    const uint8_t *b = p.base + row * p.base_row + g * 24;
    const uint8_t *h = p.high + row * p.high_row + g * 2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + i;
      uint32_t v, dig;
      if (j < 120) { v = b[j / 5]; dig = (uint32_t)(j % 5); }
      else { v = h[(j - 120) >> 2]; dig = (uint32_t)((j - 120) & 3); }
      for (uint32_t q = 0; q < dig; ++q) v /= 3u;
      w[i] = (float)((int)(v % 3u) - 1) * s;
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void embed_kernel(Planes p, const int32_t *__restrict__ ids,
                                                    int64_t count,
                                                    const uint16_t *__restrict__ signs,
                                                    float *__restrict__ out, int64_t ldo,
                                                    int32_t *err_word) {
  __shared__ __attribute__((aligned(16))) float scratch[4][WHT_SCRATCH];
  const int lane = threadIdx.x & 63;
  const int64_t nblocks = p.k / 1024;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= count * nblocks) return;
  const int64_t i = item / nblocks;
  const int64_t blk = (item % nblocks) * 1024;
  const int64_t col = blk + 16 * lane;
  const int32_t id = ids[i];
  float v[16];
  if (id < 0 || (int64_t)id >= p.n) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0.0f;
    if (err_word && lane == 0) *err_word = 1;
    store16<DT_F32>(out, i * ldo + col, v);
    return;
  }
  decode16<FMT>(p, id, col, v);
  wht1024_wave(v, lane, scratch[threadIdx.x >> 6]);
  // v[4g + j] now holds element blk + 256g + 4*lane + j
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t c = blk + 256 * g + 4 * lane;
    const u32x2 sw = *reinterpret_cast<const u32x2 *>(signs + c);
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = apply_sign(v[4 * g + j] * 0.03125f, (uint16_t)(sw[j >> 1] >> (16 * (j & 1))));
    store4<DT_F32>(out, i * ldo + c, o);
  }
}

hipError_t launch_embed(const Planes &p, const int32_t *ids, int64_t count,
                        const uint16_t *signs, float *out, int64_t ldo,
                        int32_t *err_word, hipStream_t st) {
  const int64_t items = count * (p.k / 1024);
  dim3 grid((unsigned)((items + 3) / 4)), block(256);
  if (p.fmt == FMT_PQ2)
    hipLaunchKernelGGL(embed_kernel<FMT_PQ2>, grid, block, 0, st, p, ids, count, signs,
                       out, ldo, err_word);
  else
    hipLaunchKernelGGL(embed_kernel<FMT_PTQ1>, grid, block, 0, st, p, ids, count, signs,
                       out, ldo, err_word);
  return hipGetLastError();
}

// --------------------------------------------------------- decode hook ---
// One thread per (requested row, group): writes the group's 128 decoded
// values (code-1 / digit-1) and its scale bits.
template <int FMT>
__global__ __launch_bounds__(256) void decode_kernel(Planes p, const int32_t *__restrict__ rows,
                                                     int64_t count, int8_t *__restrict__ values,
                                                     uint16_t *__restrict__ scale_bits,
                                                     int64_t k_pad) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= count * p.groups) return;
  const int64_t i = t / p.groups, g = t % p.groups;
  const int32_t r = rows[i];
  int8_t *o = values + i * k_pad + g * 128;
  if (r < 0 || (int64_t)r >= p.n) {
    for (int j = 0; j < 128; ++j) o[j] = 0;
    scale_bits[i * p.groups + g] = 0;
    return;
  }
  if constexpr (FMT == FMT_PQ2) {
    const uint8_t *b = p.base + r * p.base_row + g * 32;
    for (int j = 0; j < 128; ++j) o[j] = (int8_t)((int)((b[j >> 2] >> (2 * (j & 3))) & 3) - 1);
  } else {
    const uint8_t *b = p.base + r * p.base_row + g * 24;
    const uint8_t *h = p.high + r * p.high_row + g * 2;
    for (int q = 0; q < 24; ++q) {
      uint32_t v = b[q];
      for (int e = 0; e < 5; ++e, v /= 3u) o[5 * q + e] = (int8_t)((int)(v % 3u) - 1);
    }
    for (int q = 0; q < 2; ++q) {
      uint32_t v = h[q];
      for (int e = 0; e < 4; ++e, v /= 3u) o[120 + 4 * q + e] = (int8_t)((int)(v % 3u) - 1);
    }
  }
  scale_bits[i * p.groups + g] = p.scale[(int64_t)r * p.groups + g];
}

hipError_t launch_decode(const Planes &p, const int32_t *rows, int64_t count,
                         int8_t *values, uint16_t *scale_bits, int64_t k_pad,
                         hipStream_t st) {
  const int64_t items = count * p.groups;
  dim3 grid((unsigned)((items + 255) / 256)), block(256);
  if (p.fmt == FMT_PQ2)
    hipLaunchKernelGGL(decode_kernel<FMT_PQ2>, grid, block, 0, st, p, rows, count, values,
                       scale_bits, k_pad);
  else
    hipLaunchKernelGGL(decode_kernel<FMT_PTQ1>, grid, block, 0, st, p, rows, count, values,
                       scale_bits, k_pad);
  return hipGetLastError();
}

}  // namespace tq
