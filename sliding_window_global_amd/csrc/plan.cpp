// Host-side planning of the split-K decode: key ranges per (sequence, KV head) and the
// workspace they need. Plain C++ (no device code), so the host validation and planning can
// also be built and checked on the CPU alone.
#include <cstddef>

#include "kernels.h"

namespace plamo {

namespace {
constexpr long long kTile = 64;       // keys per decode tile
constexpr long long kMaxSplit = 256;  // key ranges per (sequence, KV head), at most
}  // namespace

DecodePlan plan_decode(int B, int Hkv, long long S, bool ragged, long long min_chunk) {
  // Aim for ~512 blocks (2 per CU, one wave per SIMD each) with at least min_chunk keys
  // each and at most kMaxSplit ranges per (sequence, KV head). A ragged batch only knows
  // its longest sequence here; its ranges are cut finer (~8 blocks per slot at the
  // longest length) so that short and long sequences even out over the CUs.
  const long long pairs = static_cast<long long>(B) * Hkv;
  const long long target_blocks = ragged ? 8 * 512 : 512;
  long long n = (target_blocks + pairs - 1) / pairs;
  const long long by_min_chunk = (S + min_chunk - 1) / min_chunk;
  if (n > by_min_chunk) n = by_min_chunk;
  if (n > kMaxSplit) n = kMaxSplit;
  if (n < 1) n = 1;
  long long chunk = (S + n - 1) / n;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  DecodePlan p;
  p.chunk = chunk;
  p.n_split = static_cast<int>((S + chunk - 1) / chunk);  // <= n (chunk >= S / n)
  // n never decreases as S grows; n_split can (the chunk is rounded up to whole tiles), so the
  // workspace is sized by n
  p.max_split = static_cast<int>(n);
  return p;
}

size_t decode_workspace_bytes(int B, int Hq, int d, const DecodePlan& plan) {
  // one split writes the output directly; a split's partial state is acc[d], m, l (sized
  // for max_split ranges, at least n_split)
  if (plan.max_split == 1) return 0;
  return static_cast<size_t>(B) * Hq * plan.max_split * (d + 2) * sizeof(float);
}

size_t decode_step_tickets_bytes(int B, int Hkv) {
  return (static_cast<size_t>(B) * Hkv * sizeof(unsigned) + 255) / 256 * 256;
}

size_t decode_step_workspace_bytes(int B, int Hq, int Hkv, int d, const DecodePlan& plan) {
  // the tickets first (the same place whatever the plan), then the partial states
  if (plan.max_split == 1) return 0;
  return decode_step_tickets_bytes(B, Hkv) + decode_workspace_bytes(B, Hq, d, plan);
}

}  // namespace plamo
