// Internal interface between the host entry points (tq_host.cpp) and the
// kernel launchers (*.hip).  Launchers assume fully validated arguments and
// only enqueue work; they return the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// Plane geometry in the form the kernels consume (byte offsets into the
// payload and per-row strides).
struct Planes {
  const uint8_t *base;    // payload + base_offset
  const uint8_t *high;    // payload + high_offset (may be empty)
  const uint16_t *scale;  // payload + scale_offset, [n][groups]
  int64_t n, k, groups;
  int64_t base_row, high_row;  // bytes per row
  int fmt;                     // 142 or 143
};

hipError_t launch_hadamard(const void *x, int x_dtype, int64_t rows, int64_t k,
                           int64_t ldx, const uint16_t *signs, int inverse,
                           void *y, int y_dtype, int64_t ldy,
                           hipStream_t stream, int tiles = 0, int groups = 0,
                           int head_dim = 0);

hipError_t launch_gemv(const Planes &p, const void *x, int x_dtype,
                       int64_t batch, int64_t ldx, float *y, int64_t ldy,
                       hipStream_t stream);

hipError_t launch_gemm(const Planes &p, const uint16_t *x, int x_dtype,
                       int64_t m, int64_t ldx, void *y, int y_dtype,
                       int64_t ldy, hipStream_t stream);

// Longest rows the decode GEMV accepts (the team kernel's reach).
inline int64_t gemv_max_k(int fmt) { return fmt == 142 ? 64 * 1024 : 32 * 1024; }

// Shapes of the batch-1 wave kernel: PQ2_0, k = 1024*m with m <= 17 for the
// GEMV alone and m <= 11 with the transform fused in, n < 2^30.
inline bool gemv_wave_fits(const Planes &p, bool fused) {
  return p.fmt == 142 && p.k % 1024 == 0 && p.k / 1024 >= 1 &&
         p.k / 1024 <= (fused ? 11 : 17) && p.n < (int64_t(1) << 30);
}

// GEMV on the matrix cores over row-quads (either format, any batch, in
// passes of up to eight rows): shapes it covers, and the launch.
bool gemv_quads_fits(const Planes &p);
hipError_t launch_gemv_quads(const Planes &p, const void *x, int x_dtype, int64_t batch,
                             int64_t ldx, float *y, int64_t ldy, hipStream_t stream);

// Signed transform fused into the GEMV (one launch): supported shapes, and
// the launch itself (x unrotated, signs bf16 +-1; tiles > 0 gathers x into
// the grouped head order of tiles x groups heads of head_dim first).
inline bool rotated_gemv_fused(const Planes &p, int64_t batch) {
  return batch == 1 && gemv_wave_fits(p, true);
}
hipError_t launch_rotated_gemv(const Planes &p, const void *x, int x_dtype,
                               const uint16_t *signs, float *y, hipStream_t st,
                               int tiles = 0, int groups = 0, int head_dim = 0);

// compute units of the current device (cached per device)
int device_cus();

hipError_t launch_embed(const Planes &p, const int32_t *ids, int64_t count,
                        const uint16_t *signs, float *out, int64_t ldo,
                        int32_t *err_word, hipStream_t stream);

// Block stream <-> planes (to_planes: src = blocks, dst = payload).
hipError_t launch_transcode(int fmt, bool to_planes, const uint8_t *src, uint8_t *dst,
                            uint64_t base_bytes, uint64_t high_offset, uint64_t high_bytes,
                            uint64_t scale_offset, uint64_t scale_bytes, uint64_t payload_bytes,
                            uint64_t blocks_bytes, hipStream_t stream);

// Planes -> 2-bit G64 block stream (one thread per 128-weight group; the
// plane pointers are at their offsets, `groups` = n * groups_per_row).
hipError_t launch_expand_g64(int fmt, const uint8_t *base, const uint8_t *high,
                             const uint16_t *scale, uint8_t *out, int64_t groups,
                             hipStream_t st);

// Batch-1 GEMV over the G64 block stream ([n][k/64] blocks of 18 bytes),
// k = 1024*m with 1 <= m <= 17, n < 2^30.
hipError_t launch_gemv_g64(const uint8_t *blocks, int64_t n, int64_t k, const void *x, int x_dtype,
                           float *y, hipStream_t st);

// Output head in one launch (PQ2_0 planes, k = 1024*m with 1 <= m <= 11,
// batch 1): RMSNorm (bf16 weight g, eps), signed transform, head GEMV into
// logits (may be null) and the greedy token; work = two zeroed 64-bit words.
hipError_t launch_head_argmax(const Planes &p, const void *x, int x_dtype, const uint16_t *g,
                              float eps, const uint16_t *signs, float *logits,
                              unsigned long long *work, int32_t *token, hipStream_t st);

// tq_head_argmax_noalloc: the head's work words live in a device global of
// HEAD_SCRATCH_WORDS 64-bit words per GPU (tq_head.hip); head_scratch gives
// its address on the current device (looked up once per device).
constexpr int HEAD_SCRATCH_WORDS = 2;
hipError_t head_scratch(unsigned long long **out);

// Plain streaming read of `bytes` (a multiple of 16) from src: the
// bandwidth reference the GEMVs are measured beside.
hipError_t launch_stream_read(const void *src, uint64_t bytes, uint32_t *sink, hipStream_t st);

hipError_t launch_decode(const Planes &p, const int32_t *rows, int64_t count,
                         int8_t *values, uint16_t *scale_bits, int64_t k_pad,
                         hipStream_t stream);

}  // namespace tq
