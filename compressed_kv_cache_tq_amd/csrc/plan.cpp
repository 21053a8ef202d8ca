// Host-only planning shared by the entry points: the split plan of the decode
// and the search workspace size (no device code, so the host half of the
// library can also be built and checked on its own).
#include "tq_internal.h"

namespace tq {

AttendPlan plan_attend(const tq_attn& a) {
  AttendPlan p{};
  const int64_t streams = static_cast<int64_t>(a.batch) * a.hkv;
  const int64_t comp = a.max_len > a.sink ? a.max_len - a.sink : 0;
  const int64_t tiles = (comp + TILE - 1) / TILE;
  // about one 8-wave workgroup per CU, no split longer than 32768 tokens,
  // at most MAX_SPLIT.  Once there are more streams than CUs, longer splits
  // win: every workgroup pays a prologue, a merge and a dispatch gap, and a
  // ragged batch then runs each stream whole.
  int64_t ns = streams > 0 ? (256 + streams - 1) / streams : 1;
  const int64_t by_len = (comp + 32767) / 32768;
  if (ns < by_len) ns = by_len;
  const int64_t cap_ns = (tiles + SW - 1) / SW;  // at least one tile per wave
  if (ns > cap_ns) ns = cap_ns;
  if (ns > MAX_SPLIT) ns = MAX_SPLIT;
  if (ns < 1) ns = 1;
  int64_t chunk_tiles = (tiles + ns - 1) / ns;
  if (chunk_tiles < 1) chunk_tiles = 1;
  ns = (tiles + chunk_tiles - 1) / chunk_tiles;
  if (ns < 1) ns = 1;
  p.n_split = static_cast<int>(ns);
  p.n_slot = p.n_split + (a.sink > 0 ? 1 : 0);
  p.chunk = chunk_tiles * TILE;
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  p.ws_bytes = static_cast<size_t>(heads) * static_cast<int64_t>(p.n_slot) * PART * sizeof(float);
  return p;
}

size_t ip_workspace_bytes() { return IP_WORK_BYTES; }

}  // namespace tq
