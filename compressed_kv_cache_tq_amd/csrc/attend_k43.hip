// Split-kernel instances for keys of widths 4 / 3 bits (all value widths,
// with and without the sketch).
#include "attend_split.h"

namespace tq {

hipError_t split_k43(int vkey, bool qjl, const SplitArgs& f) { return dispatch_v<4, 3>(vkey, qjl, f); }

}  // namespace tq
