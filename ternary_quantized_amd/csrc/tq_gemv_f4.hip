// Launch of the matrix-core batch-1 GEMV (tq_gemv_f4.h).

#include "tq_gemv_f4.h"

#ifndef TQ_F4_T
#define TQ_F4_T 2
#endif
#ifndef TQ_F4_WPG
#define TQ_F4_WPG 8
#endif
#ifndef TQ_F4_UD
#define TQ_F4_UD 2
#endif

namespace tq {

// tiles per block, lines per ring round, waves per workgroup
constexpr int F4_T = TQ_F4_T;
constexpr int F4_UD = TQ_F4_UD;
constexpr int F4_WPG = TQ_F4_WPG;

// LDS of one compute unit
constexpr size_t F4_LDS_MAX = 160 * 1024;

bool gemv_f4_fits(const Planes &p) {
  // the digit table and the all-ones sums cost each workgroup a few
  // microseconds before its first product: below about 2^29 weights the
  // dot-product kernels finish first
  if (p.n * p.k < (int64_t(1) << 29)) return false;
  return p.fmt == FMT_PQ2 && p.k >= 1024 && p.k % 1024 == 0 && p.k % (512 * F4_UD) == 0 && p.k <= 1024 * F4_WPG && p.n >= 1 &&
         p.n < (int64_t(1) << 30) && gemv_f4_lds(p.k, F4_WPG) <= F4_LDS_MAX &&
         16 * F4_T * (p.k / 64) <= F4_STAGE_SCALES;
}

template <int XD, int MODE>
static hipError_t f4_go(const Planes &p, const void *x, const uint16_t *signs, float *y, const StepArgs &hd,
                        hipStream_t st) {
  auto kern = gemv_f4_kernel<XD, MODE, F4_T, F4_UD, F4_WPG>;
  const size_t lds = gemv_f4_lds(p.k, F4_WPG);
  // more than 64 KiB of dynamic LDS must be allowed per kernel, once
  static const hipError_t allowed = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                                        (int)F4_LDS_MAX);
  if (allowed != hipSuccess) return allowed;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * F4_WPG, lds) != hipSuccess || per_cu < 1)
    return hipErrorInvalidConfiguration;
  // blocks of 16T rows.  Either the fewest passes over the resident waves,
  // then the fewest waves with that many passes (every wave the same share),
  // or every resident workgroup (some waves one block fewer), whichever
  // leaves fewer compute units with one workgroup: such a unit streams its
  // share at about half the rate.  The first is kept while it fills at
  // least 90% of the slots.
  const int64_t nblk = (p.n + 16 * F4_T - 1) / (16 * F4_T);
  const int64_t wgs = (int64_t)device_cus() * per_cu;
  const int64_t slots = wgs * F4_WPG;
  const int64_t passes = (nblk + slots - 1) / slots;
  const int64_t waves = (nblk + passes - 1) / passes;
  const int64_t even = (waves + F4_WPG - 1) / F4_WPG;
  const int64_t need = (nblk + F4_WPG - 1) / F4_WPG;
  const int64_t full = need < wgs ? need : wgs;
  const int64_t grid = 10 * even >= 9 * full ? even : full;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * F4_WPG), lds, st, p, x, signs, y, hd);
  return hipGetLastError();
}

template <int MODE>
static hipError_t f4_dt(const Planes &p, const void *x, int xd, const uint16_t *signs, float *y,
                        const StepArgs &hd, hipStream_t st) {
  if (xd == DT_F32) return f4_go<DT_F32, MODE>(p, x, signs, y, hd, st);
  if (xd == DT_BF16) return f4_go<DT_BF16, MODE>(p, x, signs, y, hd, st);
  return f4_go<DT_F16, MODE>(p, x, signs, y, hd, st);
}

hipError_t launch_gemv_f4(const Planes &p, const void *x, int xd, const uint16_t *signs, float *y, int mode,
                          const StepArgs &hd, hipStream_t st) {
  if (!gemv_f4_fits(p)) return hipErrorInvalidValue;
  if (mode == MODE_ROT) return f4_dt<MODE_ROT>(p, x, xd, signs, y, hd, st);
  if (mode == MODE_HEAD) return f4_dt<MODE_HEAD>(p, x, xd, signs, y, hd, st);
  return f4_dt<MODE_GEMV>(p, x, xd, signs, y, hd, st);
}

}  // namespace tq
