// Stage 1 of the exact top-k: every 64-token unit of a row (one wave of the
// indexer) sends its m best keys, in token order, and a floor. Shared by the
// indexer epilogue and the standalone top-k kernel.
//
// Ranking inside a wave uses a 32-bit packed key per token: the score's
// order-preserving bits with the low 6 bits replaced by (63 - lane). Packed keys
// are distinct within the wave and ordered like the scores up to those 6 bits. The
// wave's m largest packed keys are sent with their full 64-bit composite keys; the
// floor bounds the composite key of every token not sent:
// ((packed key of rank m) | 63) << 32 | 0xFFFFFFFF, or 0 when the unit sent all of
// its valid tokens. The sort runs on DPP / permlane exchanges: no LDS, no barrier.
#pragma once

#include "common.h"
#include "internal.h"

namespace dsa {

// Keys a 64-token unit sends for a row of length ctx: the largest power of two
// (at most 16) that keeps the row within kCandRowCap; 0 when the row is short
// enough for the select stage to read every score.
__device__ __forceinline__ int cand_per_unit(int ctx) {
  if (ctx <= kTopkFullRow) return 0;
  const int nu = (ctx + kCandUnit - 1) / kCandUnit;
  int m = kCandPerUnitMax;
  while (m > 1 && nu * m > kCandRowCap) m >>= 1;
  return m;
}

// Called by a whole wave; lane l carries token unit_base + l.
__device__ __forceinline__ void wave_send_candidates(float score, bool valid, int ctx, int unit_base, int row,
                                                     int unit, const TopkWs& tw) {
  const int m = cand_per_unit(ctx);
  if (m == 0) return;  // uniform over the row
  const int lane = threadIdx.x & 63;
  const uint32_t packed = valid ? ((float_key(score) & ~63u) | (63u - (uint32_t)lane)) : 0u;
  const uint32_t sorted = wave_sort_desc_u32(packed, lane);
  const uint32_t thr = (uint32_t)__builtin_amdgcn_readlane((int)sorted, m - 1);
  const bool sent = packed != 0u && packed >= thr;
  const uint64_t bal = __ballot(sent);
  const uint32_t nsent = (uint32_t)__popcll(bal);
  const uint32_t pos = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
  uint64_t* dst = tw.cand + (int64_t)row * kCandRowCap + (int64_t)unit * m;
  if (sent) dst[pos] = composite_key(score, unit_base + lane);
  if ((uint32_t)lane >= nsent && lane < m) dst[lane] = 0ull;  // unused slots of a short unit
  int valid_n = ctx - unit_base;
  valid_n = valid_n > kCandUnit ? kCandUnit : valid_n;
  const uint32_t next = (uint32_t)__builtin_amdgcn_readlane((int)sorted, m < kCandUnit ? m : kCandUnit - 1);
  if (lane == 0)
    tw.floors[(int64_t)row * tw.nunits + unit] = valid_n > m ? (((uint64_t)(next | 63u) << 32) | 0xFFFFFFFFull) : 0ull;
}

}  // namespace dsa
