// The output head of a decode step in one launch ([tensorsharp] §4.4: after
// the last layer, RMSNorm, the signed Hadamard transform and the low-bit
// output head give the logits): the batch-1 wave GEMV over PQ2_0 planes in
// its head mode, which also normalises and rotates the hidden row and
// reduces the logits to the greedy token (largest logit, lowest index).

#include "tq_device.h"
#include "tq_gemv_wave.h"
#include "tq_launch.h"

namespace tq {

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

}  // namespace tq
