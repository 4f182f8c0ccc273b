// Stage 1 of the exact top-k: every unit of a row (a run of consecutive tokens)
// sends its m best keys, in token order, and a floor. Shared by the indexer
// epilogue and the standalone top-k kernel, which both hand it one workgroup of
// 4 waves covering 256 consecutive tokens (wave w: tokens 64 w .. 64 w + 63, lane =
// token).
//
// Unit size and m depend only on the row length (see cand_plan): 64-token units
// (one wave, m = 16) up to 65,536 tokens, 256-token units (the workgroup, m = 16, 8
// or 4) above. A unit of 256 tokens holds on average 2 of the top 2048 of a
// 262,144-token row, so 16 sent keys leave it short only when it holds 17 or more.
//
// Ranking uses a 32-bit packed key per token: the score's order-preserving bits with
// the low 8 bits replaced by (255 - position in the workgroup). Packed keys are
// distinct within the workgroup and ordered like the scores up to those 8 bits. The
// m largest packed keys of a unit are sent with their full 64-bit composite keys
// (score word and token word, in two arrays) at slot cand_slot(q, u, m), q = rank in
// token order, u = unit: slot row i = q + m (u / 1024), lane u % 1024, at
// i * 1024 + u % 1024. The select's thread t then reads slots i * 1024 + t for
// i < 16, addresses that do not depend on the row length. The floor is a score word f such that every unsent token's composite key is below
// (f << 32) | 0xFFFFFFFF, so an unsent key can reach a threshold c only if
// f >= c >> 32; f = 0 when the unit sent all of its valid tokens. Sorting uses DPP /
// permlane exchanges inside a wave; 256-token units merge the four waves' best 16
// through LDS with one barrier (a bitonic merge of the four sorted lists).
#pragma once

#include "common.h"
#include "internal.h"

namespace dsa {

struct CandPlan {
  int unit;  // tokens per unit: 64 or 256
  int m;     // keys sent per unit
  int nu;    // units of the row
};

// Every row of a launch whose row-length bound exceeds kTopkFullRow sends; launches
// with a smaller bound send nothing (their select reads the rows whole).
__host__ __device__ inline CandPlan cand_plan(int ctx) {
  CandPlan p{0, 0, 0};
  if (ctx <= 4 * kTopkFullRow) {
    p.unit = 64;
    p.m = kCandPerUnitMax;
  } else {
    p.unit = 256;
    // largest power of two m <= 16 with nu * m <= kCandRowCap
    const int nu = (ctx + 255) / 256;
    p.m = nu <= 1024 ? 16 : nu <= 2048 ? 8 : nu <= 4096 ? 4 : nu <= 8192 ? 2 : 1;
  }
  p.nu = (ctx + p.unit - 1) / p.unit;
  return p;
}
static_assert(kCandPerUnitMax == 16 && kCandRowCap == 16 * 1024, "candidate slot layout");

// Position of rank q of unit u in a row's candidate array (m keys per unit).
__host__ __device__ inline int cand_slot(int q, int u, int m) { return (q + m * (u >> 10)) * 1024 + (u & 1023); }

// Called by all 256 threads of a workgroup (no thread may have returned): thread
// 64 w + l holds the score of token base + 64 w + l. `lds` is 68 words of LDS.
__device__ __forceinline__ void send_candidates(float score, bool valid, int ctx, int base, int row,
                                                const TopkWs& tw, uint32_t* lds) {
  const CandPlan p = cand_plan(ctx);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pos = threadIdx.x;  // position in the workgroup
  const uint32_t packed = valid ? ((float_key(score) & ~255u) | (255u - (uint32_t)pos)) : 0u;
  const uint32_t sorted = wave_sort_desc_u32(packed, lane);
  uint32_t* cand_hi = tw.cand_hi + (int64_t)row * kCandRowCap;
  uint32_t* cand_lo = tw.cand_lo + (int64_t)row * kCandRowCap;
  uint32_t* floors = tw.floors + (int64_t)row * kFloorRowCap;
  const uint64_t key = valid ? composite_key(score, base + pos) : 0ull;

  if (p.unit == 64) {
    // one unit per wave
    const int u = (base >> 6) + wid;
    if (u >= p.nu) return;  // wave-uniform, past the row
    const uint32_t thr = (uint32_t)__builtin_amdgcn_readlane((int)sorted, p.m - 1);
    const uint32_t nxt = (uint32_t)__builtin_amdgcn_readlane((int)sorted, p.m);
    const bool sent = packed != 0u && packed >= thr;
    const uint64_t bal = __ballot(sent);
    const uint32_t nsent = (uint32_t)__popcll(bal);
    const uint32_t q = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (sent) {
      cand_hi[cand_slot((int)q, u, p.m)] = (uint32_t)(key >> 32);
      cand_lo[cand_slot((int)q, u, p.m)] = (uint32_t)key;
    }
    if ((uint32_t)lane >= nsent && lane < p.m) cand_hi[cand_slot(lane, u, p.m)] = 0u;  // unused ranks
    if (lane == 0) floors[u] = nxt != 0u ? (nxt | 255u) : 0u;
    return;
  }

  // one unit per workgroup: merge the waves' best 16 (and each wave's 17th) in LDS.
  // Odd waves store theirs reversed, so lanes [0, 32) and [32, 64) each hold a bitonic
  // sequence and the last two phases of a bitonic sort (11 steps) order all 64.
  if (lane < 16) lds[wid * 16 + ((wid & 1) ? 15 - lane : lane)] = sorted;
  if (lane == 16) lds[64 + wid] = sorted;
  __syncthreads();
  const uint32_t all = lds[lane];
  const uint32_t w17 = max(max(lds[64], lds[65]), max(lds[66], lds[67]));
  uint32_t msort = all;
  msort = bitonic_desc_step<32, 16>(msort, lane);
  msort = bitonic_desc_step<32, 8>(msort, lane);
  msort = bitonic_desc_step<32, 4>(msort, lane);
  msort = bitonic_desc_step<32, 2>(msort, lane);
  msort = bitonic_desc_step<32, 1>(msort, lane);
  msort = bitonic_desc_step<64, 32>(msort, lane);
  msort = bitonic_desc_step<64, 16>(msort, lane);
  msort = bitonic_desc_step<64, 8>(msort, lane);
  msort = bitonic_desc_step<64, 4>(msort, lane);
  msort = bitonic_desc_step<64, 2>(msort, lane);
  msort = bitonic_desc_step<64, 1>(msort, lane);
  const uint32_t thr = (uint32_t)__builtin_amdgcn_readlane((int)msort, p.m - 1);
  const uint32_t nxt = max((uint32_t)__builtin_amdgcn_readlane((int)msort, p.m), w17);
  // keys this wave sends, and how many lower waves send (all within their best 16)
  const bool sent = packed != 0u && packed >= thr;
  const uint64_t bal = __ballot(sent);
  const uint32_t before = (uint32_t)__popcll(__ballot(all != 0u && all >= thr && lane < 16 * wid));
  const uint32_t q = before + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
  const int u = base >> 8;
  if (sent) {
    cand_hi[cand_slot((int)q, u, p.m)] = (uint32_t)(key >> 32);
    cand_lo[cand_slot((int)q, u, p.m)] = (uint32_t)key;
  }
  const uint32_t ntot = (uint32_t)__popcll(__ballot(all != 0u && all >= thr));
  if (wid == 0 && (uint32_t)lane >= ntot && lane < p.m) cand_hi[cand_slot(lane, u, p.m)] = 0u;  // unused ranks
  if (wid == 0 && lane == 0) floors[u] = nxt != 0u ? (nxt | 255u) : 0u;
}

}  // namespace dsa
