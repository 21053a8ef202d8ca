// Device-side stand-ins for the sanitizer build of the library's host half
// (host.cpp + plan.cpp compiled with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer, no HIP runtime, no GPU): every launch reports
// that no device is available, so each entry point runs its whole host-side
// validation and then returns TQ_E_HIP.
#include "tq_internal.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "no device in the host sanitizer build"; }

namespace tq {

hipError_t launch_quantize(const Spec&, const Tables*, int, const void*, const QSeq* seqs, int64_t n_seq, int64_t,
                           int64_t, int64_t, const tq_cache&, const PageMap&, hipStream_t) {
  // touch the host-side sequence table the way a launch reads it
  int64_t sum = 0;
  for (int64_t i = 0; i < n_seq; ++i) sum += seqs[i].n_tok + seqs[i].tok0 + seqs[i].x_off;
  return sum >= 0 ? hipErrorNoDevice : hipErrorInvalidValue;
}

hipError_t launch_ip_scores(const Spec&, const Tables*, const tq_cache&, int64_t, int64_t, const float*, int, float*,
                            int64_t, void*, hipStream_t) {
  return hipErrorNoDevice;
}

hipError_t launch_attend(const Spec&, const Tables*, const tq_cache&, const Spec&, const Tables*, const tq_cache&,
                         const tq_attn&, const AttendPlan& plan, const float*, const uint16_t*, const uint16_t*,
                         const int32_t*, float*, void*, hipStream_t, const int32_t*, int, int) {
  return plan.n_split > 0 ? hipErrorNoDevice : hipErrorInvalidValue;
}

}  // namespace tq
