// Chunked prefill dispatch (placeholder until the MFMA chunked kernel lands).
#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace kda {

hipError_t launch_prefill(const PoolView& p, const PrefillLaunch& a, hipStream_t s) {
  return launch_prefill_recurrent(p, a, s);
}

}  // namespace kda
