// Stand-ins for the HIP runtime and the kernel launchers, so that the host part of the KDA
// library (kda_pool.cpp, kda_plan.cpp: slot pool, idle/pending state machine, argument
// validation, prefill planning) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven by the CPU ABI tests. Test infrastructure only: no
// launch does any work, every HIP call succeeds except the device query (no GPU), and the
// device error word reads as zero.
#include <hip/hip_runtime_api.h>

#include <cstring>

#include "kda_internal.h"

extern "C" {
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void*, size_t n, hipMemcpyKind, hipStream_t) {
  std::memset(dst, 0, n);
  return hipSuccess;
}
}

namespace kda {
hipError_t launch_decode(const PoolView&, const StepTensors&, int32_t, const int32_t*, const int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_verify(const PoolView&, const StepTensors&, int32_t, int32_t, const int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_commit(const PoolView&, int32_t, const int32_t*, const int32_t*, const int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_rollback(const PoolView&, int32_t, const int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_verify_direct(const PoolView&, const StepTensors&, int32_t, int32_t, const int32_t*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_commit_direct(const PoolView&, int32_t, const int32_t*, const int32_t*, const float*, int32_t, hipStream_t) { return hipSuccess; }
hipError_t launch_slot_reset(const PoolView&, int32_t, hipStream_t) { return hipSuccess; }
hipError_t launch_slot_copy(const PoolView&, int32_t, int32_t, hipStream_t) { return hipSuccess; }
hipError_t launch_clear_word(uint32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_prefill(const PoolView&, const PrefillLaunch&, hipStream_t) { return hipSuccess; }
hipError_t prefill_scratch(void**) { return hipErrorNoDevice; }
}  // namespace kda
