// Stage 1 of the exact top-k: every unit of a row (a run of consecutive tokens)
// sends its m best keys, in token order, and a floor. Shared by the indexer
// epilogues and the standalone send kernel, which hand it one workgroup of NT = 256
// or 512 threads covering NT consecutive tokens (wave w: tokens 64 w .. 64 w + 63,
// lane = token).
//
// Plan (cand_plan, a function of the row length and of the largest unit the producer
// supports, umax = NT): rows of at most kTopkFullRow tokens send nothing (the select
// reads their scores whole). With 512-token workgroups (the per-row indexers and the
// standalone send) a unit is one wave's 64 tokens up to 65,536 tokens, 256 tokens (four
// waves) up to 131,072 and 512 (eight waves) above. The row-group indexers (256-token
// workgroups, one send per row and wave) keep one-wave units up to 262,144 tokens: no
// barrier and no cross-wave merge per row, at the price of m = 4 above 131,072 tokens,
// where a unit that holds 5 of the top 2048 (a few per row) is rescanned by the select. The expected number of the row's top 2048
// in one unit is lam = 2048 / nu (nu = units of the row); a unit sends m >= lam +
// 4 sqrt(lam) + 2 keys (m = 8, 16 or 32), so that a unit holding more of the top k than
// it sent is rare (the select then rescans it; exactness never depends on m). With
// 512-token units a 262,144-token row sends 512 x 16 = 8,192 candidates.
//
// Layout: unit u's m keys sit at slots [u m, u m + m) of the row's candidate arrays
// (score words in cand_hi, token words in cand_lo), ranks in token order; rank slots the
// unit does not fill hold score word 0. Every token order is slot order. floors[u] is a
// score word f such that every key the unit did not send has a composite key below
// (f << 32) | 0xFFFFFFFF (f = 0 when it sent all of its tokens).
//
// Ranking inside a unit uses a 32-bit packed key per token: the score's order-preserving
// bits with the low LB bits (NT = 2^LB) replaced by (NT - 1 - position in the
// workgroup). Packed keys are distinct within the workgroup and ordered like the scores
// up to those bits; the floor ORs them back in. A wave sorts its 64 packed keys (DPP /
// permlane bitonic network); units of 4 or 8 waves merge the waves' best 16 or 8 through
// LDS with one barrier (each wave of the unit repeats the merge, so no second barrier is
// needed); the best key a wave kept back joins the floor (a 64-token wave of a row longer
// than 65,536 tokens holds 17 of its top 2048 practically never, nor 9 above 131,072
// tokens, and if it does the rescan covers it). Units of 8 waves that send at most 16 keys
// first take a cheaper exact route: a threshold from each wave's second-best key, the keys
// reaching it gathered in LDS and sorted once by one wave (described at the code).
#pragma once

#include "common.h"
#include "internal.h"

namespace dsa {

struct CandPlan {
  int unit;  // tokens per unit: 64, 256 or 512; 0 = the row sends nothing
  int m;     // keys sent per unit
  int nu;    // units of the row
  int per;   // keys per select thread: 8 (at most 8,192 candidates) or 16
  int lu;    // log2 of unit
  int lm;    // log2 of m
};

__host__ __device__ inline CandPlan cand_plan(int ctx, int umax) {
  CandPlan p{0, 0, 0, 16, 0, 0};
  if (ctx <= kTopkFullRow) {
    p.per = ctx <= kCandRowCap / 2 ? 8 : 16;
    return p;
  }
  if (umax >= 512)
    p.lu = ctx <= 4 * kTopkFullRow ? 6 : (ctx > 8 * kTopkFullRow ? 9 : 8);
  else  // row-group producers: one-wave units up to the floor capacity (4,096 units)
    p.lu = ctx <= 16 * kTopkFullRow ? 6 : 8;
  p.unit = 1 << p.lu;
  p.nu = (ctx + p.unit - 1) >> p.lu;
  // lam = 2048 / nu: nu < 410 <=> lam > 5 (m = 32 covers lam <= 14); nu < 1517 <=> lam > 1.35
  p.lm = p.nu < 410 ? 5 : p.nu < 1517 ? 4 : 3;
  while ((p.nu << p.lm) > kCandRowCap) --p.lm;
  p.m = 1 << p.lm;
  p.per = p.nu * p.m <= kCandRowCap / 2 ? 8 : 16;
  return p;
}

// Called by all NT threads of a workgroup (no thread may have returned): thread
// 64 w + l holds the score of token base + 64 w + l. `lds` is send_lds_words<NT>() words.
template <int NT>
constexpr int send_lds_words() { return 17 * (NT / 64); }

template <int NT>
__device__ __forceinline__ void send_candidates(float score, bool valid, int ctx, int base, int row,
                                                const TopkWs& tw, uint32_t* lds) {
  static_assert(NT == 256 || NT == 512, "workgroup of 4 or 8 waves");
  constexpr int LB = NT == 256 ? 8 : 9;
  constexpr uint32_t LM = (1u << LB) - 1u;
  constexpr int NWG = NT / 64;
  const CandPlan p = cand_plan(ctx, NT);
  if (p.unit == 0) return;  // uniform: the row sends nothing
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pos = threadIdx.x;  // position in the workgroup
  const uint32_t packed = valid ? ((float_key(score) & ~LM) | (LM - (uint32_t)pos)) : 0u;
  uint32_t* cand_hi = tw.cand_hi + (int64_t)row * kCandRowCap;
  uint32_t* cand_lo = tw.cand_lo + (int64_t)row * kCandRowCap;
  uint32_t* floors = tw.floors + (int64_t)row * kFloorRowCap;
  const uint64_t key = valid ? composite_key(score, base + pos) : 0ull;

  if (p.unit == 64) {
    // one unit per wave
    const int u = (base >> 6) + wid;
    if (u >= p.nu) return;  // wave-uniform, past the row
    uint32_t thr, nxt;
    if (p.m == 4) {  // uniform: the 4 best packed keys and the next one by repeated maxima
      uint32_t v = packed, mx[5];
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        mx[q] = wave_max_u32_last(v);
        v = v == mx[q] ? 0u : v;  // packed keys are distinct: one lane leaves the race
      }
      thr = mx[3];
      nxt = mx[4];
    } else {
      const uint32_t sorted = wave_sort_desc_u32(packed, lane);
      thr = (uint32_t)__builtin_amdgcn_readlane((int)sorted, p.m - 1);
      nxt = (uint32_t)__builtin_amdgcn_readlane((int)sorted, p.m);
    }
    const bool sent = packed != 0u && packed >= thr;
    const uint64_t bal = __ballot(sent);
    const uint32_t nsent = (uint32_t)__popcll(bal);
    const uint32_t q = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    const int s0 = u * p.m;
    if (sent) {
      cand_hi[s0 + (int)q] = (uint32_t)(key >> 32);
      cand_lo[s0 + (int)q] = (uint32_t)key;
    }
    if ((uint32_t)lane >= nsent && lane < p.m) cand_hi[s0 + lane] = 0u;  // unused ranks
    if (lane == 0) floors[u] = nxt != 0u ? (nxt | LM) : 0u;
    return;
  }

  // Eight-wave units sending m <= 16 keys (rows of more than 209,408 tokens: m = 16, and
  // m = 8 above 776,192). A key threshold tau first: each wave's
  // second-best packed key goes to LDS and tau is the least of the eight, so at least 16
  // keys of the unit reach it and the unit's best m are among them. The keys >= tau (about
  // 34 for independent scores) are appended to a 64-entry LDS list that wave 0 sorts: its
  // m-th entry is the send threshold, its (m+1)-th the best key kept back (when m or fewer
  // keys reach tau, all of them are sent and tau - 1 bounds the rest). Wave 0 also counts
  // each wave's sent keys from the sorted list, so that every wave places its own in token
  // order after one more barrier. Two wave maxima per wave and one sort per unit replace a
  // sort per wave and a merge in every wave, and the unit sends its best m keys outright
  // (the general path below takes the best m among each wave's best 8). More than 64 keys
  // at tau (about one unit in a hundred, or many tied scores) take the general path.
  if (NT == 512 && p.unit == 512 && p.m <= 16) {
    uint32_t* le = lds;       // [64] keys >= tau
    uint32_t* lc = lds + 64;  // [8] each wave's second-best key
    uint32_t* lo = lds + 72;  // [8] sent keys of the waves below each wave
    uint32_t* lv = lds + 80;  // [0] list length, [1] send threshold
    static_assert(send_lds_words<512>() >= 82, "send LDS");
    if (threadIdx.x == 0) lv[0] = 0u;
    uint32_t v = packed;
    const uint32_t b1 = wave_max_u32_last(v);
    v = v == b1 ? 0u : v;  // packed keys are distinct: one lane leaves the race
    const uint32_t b2 = wave_max_u32_last(v);
    if (lane == 0) lc[wid] = b2;
    __syncthreads();
    uint32_t tau = lc[0];
#pragma unroll
    for (int w = 1; w < 8; ++w) tau = min(tau, lc[w]);
    const bool in = packed != 0u && packed >= tau;
    const uint64_t bin = __ballot(in);
    uint32_t wb = 0u;
    if (lane == 0 && bin != 0ull) wb = atomicAdd(&lv[0], (uint32_t)__popcll(bin));
    wb = (uint32_t)__builtin_amdgcn_readfirstlane((int)wb);
    const uint32_t at = wb + (uint32_t)__popcll(bin & ((1ull << lane) - 1ull));
    if (in && at < 64u) le[at] = packed;
    __syncthreads();
    const uint32_t ne = lv[0];
    if (ne <= 64u) {  // uniform
      const int u = base / p.unit;
      const int s0 = u * p.m;
      if (wid == 0) {
        const uint32_t srt = wave_sort_desc_u32((uint32_t)lane < ne ? le[lane] : 0u, lane);
        const uint32_t thr = (uint32_t)__builtin_amdgcn_readlane((int)srt, p.m - 1);
        const uint32_t nx = (uint32_t)__builtin_amdgcn_readlane((int)srt, p.m);
        const uint32_t nxt = ne > (uint32_t)p.m ? nx : (tau != 0u ? tau - 1u : 0u);
        // sorted entry -> its wave (position in the workgroup from the packed low bits)
        const bool s = lane < p.m && srt != 0u;
        const uint32_t pw = (LM - (srt & LM)) >> 6;
        uint32_t below = 0u;  // lane w: sent keys of the waves below w
#pragma unroll
        for (int w = 0; w < 7; ++w) {
          const uint32_t c = (uint32_t)__popcll(__ballot(s && pw == (uint32_t)w));
          below += lane > w ? c : 0u;
        }
        if (lane < 8) lo[lane] = below;
        if (lane == 0) lv[1] = thr;
        const uint32_t ntot = (uint32_t)__popcll(__ballot(s));
        if (u < p.nu) {
          if ((uint32_t)lane >= ntot && lane < p.m) cand_hi[s0 + lane] = 0u;  // unused ranks
          if (lane == 0) floors[u] = nxt != 0u ? (nxt | LM) : 0u;
        }
      }
      __syncthreads();
      if (u >= p.nu) return;  // uniform: the unit lies past the row
      // with fewer than m entries the sorted threshold is 0 and tau selects them all
      const uint32_t thr = max(lv[1], tau);
      const bool sent = packed != 0u && packed >= thr;
      const uint64_t bal = __ballot(sent);
      const uint32_t q = lo[wid] + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
      if (sent) {
        cand_hi[s0 + (int)q] = (uint32_t)(key >> 32);
        cand_lo[s0 + (int)q] = (uint32_t)key;
      }
      return;
    }
    __syncthreads();  // every wave has read the list length before the general path reuses the LDS
  }

  // Units of W = unit / 64 waves. Every wave puts its best cw = 64 / W keys (16 of a
  // 4-wave unit, 8 of an 8-wave one) into the unit's 64-entry LDS region, odd waves
  // reversed so that each pair of waves forms a bitonic sequence, and its (cw + 1)-th
  // into wnx[]; after one barrier every wave of the unit sorts the 64 entries. (An
  // 8-wave unit belongs to a row of more than 131,072 tokens, where a 64-token wave
  // holds on average at most one of the top 2048: nine or more are practically never.)
  const uint32_t sorted = wave_sort_desc_u32(packed, lane);
  const int W = p.unit >> 6;                 // 4 or 8 (uniform)
  const int cw = 64 / W;                     // keys each wave contributes: 16 or 8
  const int wi = W == 8 ? wid : (wid & 3);   // wave index inside the unit
  const int ub = wid - wi;                   // first wave of the unit
  uint32_t* reg = lds + 16 * ub;             // the unit's 64 entries
  uint32_t* wnx = lds + 16 * NWG;            // one per wave of the workgroup
  if (lane < cw) reg[cw * wi + ((wi & 1) ? cw - 1 - lane : lane)] = sorted;
  if (lane == cw) wnx[wid] = sorted;
  __syncthreads();
  uint32_t ra = reg[lane];
  uint32_t wmax = 0u;
  for (int j = 0; j < W; ++j) wmax = max(wmax, wnx[ub + j]);
  // remaining phases of a bitonic sort of the 64 entries: runs of cw = 8 first merge into
  // sorted 16-runs of alternating direction (4 steps), then 32-runs (5), then all 64 (6)
  uint32_t msort = ra;
  if (W == 8) {
    msort = bitonic_desc_step<16, 8>(msort, lane);
    msort = bitonic_desc_step<16, 4>(msort, lane);
    msort = bitonic_desc_step<16, 2>(msort, lane);
    msort = bitonic_desc_step<16, 1>(msort, lane);
  }
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
  const uint32_t nxt = max((uint32_t)__builtin_amdgcn_readlane((int)msort, p.m), wmax);
  // a key is sent when it is among its wave's best cw and reaches the m-th of the merge
  const uint32_t wcw = (uint32_t)__builtin_amdgcn_readlane((int)sorted, cw - 1);
  const bool sent = packed != 0u && packed >= thr && packed >= wcw;
  const uint64_t bal = __ballot(sent);
  // sent keys of the unit's lower waves (LDS entry e belongs to wave e / cw)
  const uint32_t before = (uint32_t)__popcll(__ballot(ra != 0u && ra >= thr && lane < cw * wi));
  const uint32_t q = before + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
  const int u = (base + 64 * ub) / p.unit;
  if (u >= p.nu) return;  // wave-uniform: the unit lies past the row
  const int s0 = u * p.m;
  if (sent) {
    cand_hi[s0 + (int)q] = (uint32_t)(key >> 32);
    cand_lo[s0 + (int)q] = (uint32_t)key;
  }
  if (wi == 0) {
    const uint32_t ntot = (uint32_t)__popcll(__ballot(ra != 0u && ra >= thr));
    if ((uint32_t)lane >= ntot && lane < p.m) cand_hi[s0 + lane] = 0u;  // unused ranks
    if (lane == 0) floors[u] = nxt != 0u ? (nxt | LM) : 0u;
  }
}

}  // namespace dsa
