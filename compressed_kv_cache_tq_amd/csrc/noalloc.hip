// tq_attend_decode_noalloc: the decode step with the split partials in a
// static device array instead of a caller's workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation).
//
// The array is a file-scope __device__ object, so every GPU that loads the
// library holds its own copy for the life of the process.  Host code never
// uses the array's name as an address: the first call on a device looks up
// that device's copy with hipGetSymbolAddress (with the device current) and
// keeps the pointer; the kernels receive it like any workspace.  Nothing in
// the array needs to start at zero: the split kernel writes every partial
// before the merge reads it.  All calls on one GPU share its copy, so calls
// that overlap on one GPU (other streams, other threads) race.
#include <mutex>

#include "tq_internal.h"

namespace {

constexpr size_t SCRATCH_BYTES = TQ_NOALLOC_SCRATCH_BYTES;  // per device
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch[MAX_DEVICES] = {};

// This device's copy of the array (looked up once per device).
tq_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tq::set_error(TQ_E_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return tq::set_error(TQ_E_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      return tq::set_error(TQ_E_HIP, e != hipSuccess ? hipGetErrorString(e) : "no address for the scratch array");
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_attend_decode_noalloc(const tq_spec* ks, const void* ktables, const tq_cache* kc,
                                   const tq_spec* vs, const void* vtables, const tq_cache* vc,
                                   const tq_attn* attn, const float* q, const uint16_t* sink_k,
                                   const uint16_t* sink_v, const int32_t* seq_lens, float* out, void* stream) {
  if (!attn) return tq::set_error(TQ_E_ARG, "attn must be non-NULL");
  const size_t need = tq_attend_workspace_bytes(attn);
  if (need > SCRATCH_BYTES) {
    return tq::set_error(TQ_E_UNSUPPORTED,
                         "tq_attend_workspace_bytes of this problem exceeds TQ_NOALLOC_SCRATCH_BYTES, the "
                         "static scratch of tq_attend_decode_noalloc; use tq_attend_decode with a workspace");
  }
  void* ws = nullptr;
  if (tq_status st = scratch_of_current_device(&ws); st != TQ_OK) return st;
  return tq::attend_checked(ks, ktables, kc, vs, vtables, vc, attn, q, sink_k, sink_v, seq_lens, nullptr, 0, 0, out,
                            ws, SCRATCH_BYTES, stream, "tq_attend_decode_noalloc launch");
}

}  // extern "C"
