// A plain streaming read of device memory: the bandwidth reference beside
// which the decode GEMVs are measured.  It does what the GEMVs' weight
// stream does (read every byte once, in 16-byte non-temporal loads, from a
// one-shot grid) and nothing else, so its rate at a given size is what a
// read of that many bytes reaches on this chip.
//
// Each thread reads U consecutive 16-byte words of its workgroup's span
// (the span of a workgroup is contiguous, lane after lane), folds them into
// one word, and stores it only if it equals `magic`: the loads cannot be
// dropped, and in practice nothing is written.

#include "tq_launch.h"

namespace tq {

typedef uint32_t u32x4_m __attribute__((ext_vector_type(4)));

constexpr int READ_TPB = 256;
constexpr int READ_U = 4;  // 16-byte words per thread

__global__ __launch_bounds__(READ_TPB) void stream_read_kernel(const u32x4_m *__restrict__ src,
                                                               int64_t words, uint32_t *sink,
                                                               uint32_t magic) {
  const int64_t base = (int64_t)blockIdx.x * (READ_TPB * READ_U) + threadIdx.x;
  uint32_t acc = 0;
  if (base + (int64_t)(READ_U - 1) * READ_TPB < words) {
    u32x4_m v[READ_U];
#pragma unroll
    for (int u = 0; u < READ_U; ++u) v[u] = __builtin_nontemporal_load(src + base + u * READ_TPB);
#pragma unroll
    for (int u = 0; u < READ_U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  } else {
    for (int u = 0; u < READ_U; ++u) {
      const int64_t i = base + u * READ_TPB;
      if (i < words) {
        const u32x4_m t = __builtin_nontemporal_load(src + i);
        acc ^= t[0] ^ t[1] ^ t[2] ^ t[3];
      }
    }
  }
  if (acc == magic) sink[0] = acc;
}

hipError_t launch_stream_read(const void *src, uint64_t bytes, uint32_t *sink, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 16);
  const int64_t per = (int64_t)READ_TPB * READ_U;
  const int64_t grid = (words + per - 1) / per;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(READ_TPB), 0, st,
                     static_cast<const u32x4_m *>(src), words, sink, 0x9E3779B9u);
  return hipGetLastError();
}

}  // namespace tq
