// Device launchers of the host-only build of the C ABI (the build that runs
// the host code under AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU).  It links tq_host.cpp and tq_container.cpp as they
// are with these definitions in place of the kernels: every launch reports
// that no device code is present, so a call that passes validation returns
// TQ_ERR_DEVICE.  Validation, geometry, packing and container parsing run
// unchanged.

#include "../../include/tq.h"
#include "tq_launch.h"

namespace tq {

static hipError_t none() { return hipErrorNoBinaryForGpu; }

hipError_t launch_hadamard(const void *, int, int64_t, int64_t, int64_t, const uint16_t *, int,
                           void *, int, int64_t, hipStream_t, int, int, int) { return none(); }
hipError_t launch_gemv(const Planes &, const void *, int, int64_t, int64_t, float *, int64_t,
                       hipStream_t) { return none(); }
hipError_t launch_gemm(const Planes &, const uint16_t *, int, int64_t, int64_t, void *, int,
                       int64_t, hipStream_t) { return none(); }
hipError_t launch_rotated_gemv(const Planes &, const void *, int, const uint16_t *, float *,
                               hipStream_t, int, int, int) { return none(); }
hipError_t launch_embed(const Planes &, const int32_t *, int64_t, const uint16_t *, float *,
                        int64_t, int32_t *, hipStream_t) { return none(); }
hipError_t launch_transcode(int, bool, const uint8_t *, uint8_t *, uint64_t, uint64_t, uint64_t,
                            uint64_t, uint64_t, uint64_t, uint64_t, hipStream_t) { return none(); }
hipError_t launch_expand_g64(int, const uint8_t *, const uint8_t *, const uint16_t *, uint8_t *,
                             int64_t, hipStream_t) { return none(); }
hipError_t launch_gemv_g64(const uint8_t *, int64_t, int64_t, const void *, int, float *,
                           hipStream_t) { return none(); }
hipError_t launch_head_argmax(const Planes &, const void *, int, const uint16_t *, float,
                              const uint16_t *, float *, unsigned long long *, int32_t *,
                              hipStream_t) { return none(); }
hipError_t head_scratch(unsigned long long **) { return none(); }
hipError_t launch_stream_read(const void *, uint64_t, uint32_t *, hipStream_t) { return none(); }
hipError_t launch_decode(const Planes &, const int32_t *, int64_t, int8_t *, uint16_t *, int64_t,
                         hipStream_t) { return none(); }

}  // namespace tq
