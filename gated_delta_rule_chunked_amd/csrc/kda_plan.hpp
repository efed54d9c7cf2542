// kda_plan.hpp -- which state scan the forward runs (host only).
//
// The 16-column serial scan (kda_inter.hip) keeps one workgroup per (sequence, value
// head, 16 value columns) for a sequence's whole length; the 64-column scan
// (kda_scan.hip) streams each chunk record once per 64 columns and cuts sequences into
// segments joined through the scan's affine dependence on its start state.  The
// thresholds below come from sweeps of the whole forward call over forced segment
// lengths on MI355X (K = V = 128).
#pragma once

#include <stdint.h>

#include <algorithm>

namespace kda {

struct ScanPlan {
  bool seg_path;   // the 64-column scan
  int64_t seg_L;   // its segment length in chunks (clamped to the chunk count by the caller)
};

// nt: chunks per sequence (fixed length) or of the packed sequences (varlen);
// n_seq, hv, v: sequences, value heads, value width; cus: compute units;
// forced: the caller's segment length, or 0.
inline ScanPlan choose_scan(int64_t nt, bool varlen, int64_t n_seq, int64_t hv, int64_t v, int64_t cus,
                            int64_t forced) {
  if (forced > 0) return {true, forced};
  const int64_t units16 = n_seq * hv * (v / 16);           // 16-column workgroups
  const int64_t units64 = std::max<int64_t>(1, n_seq * hv * ((v + 63) / 64));   // per segment round
  // chunks per sequence (the mean for varlen, where the lengths stay on the device)
  const int64_t per_seq = varlen ? nt / std::max<int64_t>(n_seq, 1) : nt;
  if (units64 >= cus)   // 64-column workgroups alone fill the device: one segment each
    return {true, std::max<int64_t>(nt, 1)};
  if (per_seq >= 96) {
    // long sequences: as many segments per sequence (2 to 8) as one round of the full
    // pass's 64-column workgroups allows; at or ahead of the serial scan from 16 to 64
    // heads at 6,144 to 32,768 tokens (at 4,096 tokens the two are even)
    const int64_t S = std::min<int64_t>(8, std::max<int64_t>(2, cus / units64));
    return {true, (per_seq + S - 1) / S};
  }
  // few workgroups and at least 32 chunks: segments of nt / 8 chunks (at least 4); at
  // 2 x 2,048 tokens with 4 heads 54.5 us per forward against 62.7 for the serial scan
  // (and 23 against 20 us at 256 tokens, one head, where the serial scan stays)
  return {units16 * 2 < cus && nt >= 32, std::max<int64_t>(4, (nt + 7) / 8)};
}

}  // namespace kda
