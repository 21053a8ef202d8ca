// Split-kernel instances for 8-bit keys (noze.it page, section "Cosa
// aggiunge turboquant-mlx": the K8/V3 default): values of 2 or 3 bits,
// uniform, no sketch.  Two 64 KiB LUTs (8-bit keys with 4-bit values) would
// leave no LDS for the query prologue.
#include "attend_split.h"

namespace tq {

hipError_t split_k88(int vkey, bool qjl, const SplitArgs& f) {
  if (qjl) return hipErrorInvalidValue;
  switch (vkey) {
    case 22: return launch_split<8, 8, 2, 2, false>(f);
    case 33: return launch_split<8, 8, 3, 3, false>(f);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
