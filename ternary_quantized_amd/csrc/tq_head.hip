// The output head of a decode step in one launch ([tensorsharp] §4.4: after
// the last layer, RMSNorm, the signed Hadamard transform and the low-bit
// output head give the logits): the batch-1 wave GEMV over PQ2_0 planes in
// its head mode, which also normalises and rotates the hidden row and
// reduces the logits to the greedy token (largest logit, lowest index).

#include "tq_device.h"
#include "tq_gemv_f4.h"
#include "tq_gemv_wave.h"
#include "tq_launch.h"

#include <mutex>

namespace tq {

// The head's two work words (running maximum key, finished-workgroup count)
// for tq_head_argmax_noalloc, whose callers cannot allocate device memory:
// one copy per GPU, held until the process ends.  Device globals start at
// zero when the code object is loaded, and every launch's last workgroup
// writes them back to zero, so each call finds them zero.  Calls on one GPU
// share them: calls that overlap on one GPU race.
static __device__ __align__(256) unsigned long long scratch[HEAD_SCRATCH_WORDS];

namespace {

template <int A, int BQ>
hipError_t head_dt(const Planes &p, const void *x, int xd, const uint16_t *signs, float *logits,
                   const StepArgs &hd, hipStream_t st) {
  if (xd == DT_F32) return gemv_wave_go<LAY_PLANES, A, BQ, DT_F32, MODE_HEAD>(p, x, signs, logits, st, hd);
  if (xd == DT_BF16) return gemv_wave_go<LAY_PLANES, A, BQ, DT_BF16, MODE_HEAD>(p, x, signs, logits, st, hd);
  return gemv_wave_go<LAY_PLANES, A, BQ, DT_F16, MODE_HEAD>(p, x, signs, logits, st, hd);
}

}  // namespace

hipError_t launch_head_argmax(const Planes &p, const void *x, int x_dtype, const uint16_t *g,
                              float eps, const uint16_t *signs, float *logits,
                              unsigned long long *work, int32_t *token, hipStream_t st) {
  StepArgs hd;
  hd.g = g;
  hd.eps = eps;
  hd.work = work;
  hd.token = token;
  if (gemv_f4_fits(p)) return launch_gemv_f4(p, x, x_dtype, signs, logits, MODE_HEAD, hd, st);
  switch (p.k / 1024) {
    case 1: return head_dt<0, 1>(p, x, x_dtype, signs, logits, hd, st);
    case 2: return head_dt<0, 2>(p, x, x_dtype, signs, logits, hd, st);
    case 3: return head_dt<0, 3>(p, x, x_dtype, signs, logits, hd, st);
    case 4: return head_dt<1, 0>(p, x, x_dtype, signs, logits, hd, st);
    case 5: return head_dt<1, 1>(p, x, x_dtype, signs, logits, hd, st);
    case 6: return head_dt<1, 2>(p, x, x_dtype, signs, logits, hd, st);
    case 7: return head_dt<1, 3>(p, x, x_dtype, signs, logits, hd, st);
    case 8: return head_dt<2, 0>(p, x, x_dtype, signs, logits, hd, st);
    case 9: return head_dt<2, 1>(p, x, x_dtype, signs, logits, hd, st);
    case 10: return head_dt<2, 2>(p, x, x_dtype, signs, logits, hd, st);
    default: return head_dt<2, 3>(p, x, x_dtype, signs, logits, hd, st);
  }
}

// Device address of `scratch` on the current device.  In host code the
// array's name is only a host-side handle, so its device address is looked
// up once per device (with that device current) and kept.
hipError_t head_scratch(unsigned long long **out) {
  constexpr int MAXDEV = 64;
  static std::mutex mu;
  static unsigned long long *addr[MAXDEV] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<unsigned long long *>(ptr);
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace tq
