// Exact per-row top-k over fp32 scores (ties -> lower token index): the select (stage 2)
// as device code, shared by the standalone select kernel and the fused select +
// sparse-attention kernel.
//
// vLLM "Day-0 support for Kimi K3.1 Pro": the fused decode path ends the indexer
// with an exact top-k selection that emits the rows attention reads; the
// zero-mismatch RL section wants top-k to be batch invariant; and the DCP
// section's exact one-round merge sends only a bounded number of best candidates
// per shard, detects when a shard held more of the true top-k than it sent, and
// has that shard resend. The same scheme runs here between the 64-token units of
// one row instead of between GPUs.
//
// Every (score, token) pair maps to a 64-bit composite key
//   (order-preserving bits of the score) << 32 | (0xFFFFFFFF - token)
// so "larger score, then lower index" is plain integer order, the keys of a row
// are distinct, and the selection is the k largest keys. Key 0 never comes from a
// real token and marks an empty slot.
//
// Stage 1 (topk_send.h: the indexer epilogue or topk_send_kernel): every unit
// sends its m best keys plus a floor bounding the keys it kept.
// Stage 2 (topk_select_kernel, one 1024-thread workgroup per row). Every thread
// holds up to 16 keys in registers:
//   ctx <= k      every token;
//   rows of at most 16384 tokens: the row's own keys, tokens [16 t, 16 t + 16) on
//                 thread t (in a launch with longer rows, after a first search over
//                 the candidates, which the kernel starts on before it knows the
//                 row's length);
//   longer rows   the candidates of units t + 1024 j (j < units per thread), read
//                 slot-major so that each load instruction covers 64 consecutive
//                 units and no address depends on the row length (the loads start
//                 with the kernel). c_u = their k-th largest key. A unit whose floor
//                 reaches c_u may hold unsent keys >= c_u: waves rescan such units'
//                 scores (the "resend") into a compact LDS list, the unit's
//                 candidates leave the register set, and the k-th largest of the
//                 union is the answer.
// The k-th largest key: the score words of the live keys share their bits above
// the highest bit in which they differ; an 11-bit digit histogram over the next
// bits (4 copies, lane l adding into copy l % 4, so at most 16 lanes of one
// instruction hit one LDS word; 8 copies measured 0.45 us slower per step, their
// clearing and summing costing more than the atomics they spread) fixes the bucket of
// the k-th key. A bucket of at
// most 64 keys is gathered into LDS and ranked (64-bit keys, so equal scores order by
// token; every wave ranks four of them with ballots); a larger one takes another pass
// over lower bits. The
// selection is written in token order: per-unit counts and one block prefix sum over
// units place every selected token in an LDS list, which one coalesced pass then
// writes out with the tokens' page slots (block-table row staged in LDS).
#pragma once

#include "common.h"
#include "internal.h"
#include "topk_send.h"

namespace dsa {

namespace {

constexpr int SEL_NT = 1024;
constexpr int NW = SEL_NT / 64;
constexpr int PER = 16;              // keys per thread
constexpr int HBITS = 11;            // digit width of one histogram pass
constexpr int NBIN = 1 << HBITS;     // two bins per thread
constexpr int NREP = 4;              // histogram copies
constexpr int XPER = 8;              // rescanned keys per thread
constexpr int ECAP = XPER * SEL_NT;  // rescanned keys a row may hold in LDS
constexpr int FCAP = 512;            // rescanned units a row may hold in LDS
constexpr int BTCAP = 4096;          // block-table entries of a row staged in LDS (16 KB)
static_assert(PER * SEL_NT == kCandRowCap && PER * SEL_NT == kTopkFullRow, "register tiling");
static_assert(NBIN == 2 * SEL_NT, "two histogram bins per thread");

// Row length clamped to [0, max_ctx]; a clamp from above is reported in `st`.
__device__ __forceinline__ int clamp_ctx(const int32_t* row_ctx, int r, int max_ctx, uint32_t* st) {
  int c = row_ctx[r];
  c = c < 0 ? 0 : c;
  if (c > max_ctx) {
    raise_status(st, kStCtxClamped);
    c = max_ctx;
  }
  return c;
}

struct SelShared {
  union {
    struct {
      uint32_t hist[NBIN * NREP];  // bin b, copy c at b * NREP + c
      uint64_t ext[ECAP];          // keys >= c_u of the rescanned units, one segment per unit
    } a;
    struct {
      uint32_t hist[NW * 256];  // whole-row fallback: per-wave 8-bit histograms
      uint32_t sel[kMaxK];      // whole-row fallback: selection before its sort
    } g;
  };
  uint32_t funit[FCAP];   // rescanned unit of each slot, in unit order
  uint32_t fstart[FCAP];  // its segment in ext
  uint32_t flen[FCAP];    // the segment's length, then the selected ext keys before it
  uint32_t fcnt[FCAP];    // selected keys of the segment
  uint32_t foff[FCAP];    // their first output position
  uint16_t fmap[kFloorRowCap];  // rescanned unit -> its slot
  uint64_t bucket[64];    // keys of the last histogram bucket
  uint64_t res64;
  uint32_t r32[2][2][NW];  // block min / max partials, double buffered
  uint32_t scan[2][NW];    // block prefix partials, double buffered
  uint32_t scan4[4][NW];   // per-wave totals of four prefix sums
  uint32_t res[4];
  uint32_t ecount, bcount;
  uint32_t nsel;  // length of the selection list left in a.hist (token order)
  uint32_t btl;   // 1: bt holds the row's block-table entries
  int32_t bt[BTCAP];  // the row's block-table entries (clamped into the pool) when they fit
};

// Wave minimum / maximum, complete in lane 63: shifts of 1, 2, 4, 8 inside each 16-lane
// row, then the row broadcasts (lanes without a source keep their own value).
__device__ __forceinline__ uint32_t wave_min_u32_in63(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32_in63(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// Combines the NW per-wave totals p[0..NW) (LDS): lane w of every wave reads p[w], a
// 16-lane DPP scan runs over them, and two lane reads give the sum over the waves
// below this one (`before`) and the total.
__device__ __forceinline__ uint32_t wave_totals(const uint32_t* p, uint32_t& before) {
  const int lane = threadIdx.x & 63;
  uint32_t x = lane < NW ? p[lane] : 0u;
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  before = wid > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)x, wid - 1) : 0u;
  return (uint32_t)__builtin_amdgcn_readlane((int)x, NW - 1);
}

// Exclusive prefix sum over the threads in thread order; `total` gets the sum.
__device__ __forceinline__ uint32_t excl_scan(uint32_t v, uint32_t& total, SelShared& S, int& par) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) S.scan[par][wid] = inc;
  __syncthreads();
  uint32_t before;
  total = wave_totals(S.scan[par], before);
  par ^= 1;
  return before + inc - v;
}

// Four exclusive prefix sums over the threads at once (one barrier). The caller
// keeps a barrier between two calls.
__device__ __forceinline__ void excl_scan4(const uint32_t (&v)[4], uint32_t (&off)[4], uint32_t (&total)[4], int nj,
                                           SelShared& S) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t inc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < nj) inc[j] = wave_incl_scan(v[j]);  // nj is block-uniform
    if (lane == 63) S.scan4[j][wid] = inc[j];
  }
  __syncthreads();
  // one 16-lane row per sum: lane 16 j + w reads wave w's total of sum j, a scan down
  // each row, and lane reads give this wave's offsets and the totals
  uint32_t x = (lane & 15) < NW && (lane >> 4) < nj ? S.scan4[lane >> 4][lane & 15] : 0u;
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int w = __builtin_amdgcn_readfirstlane(wid);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t before = w > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)x, 16 * j + w - 1) : 0u;
    off[j] = before + inc[j] - v[j];
    total[j] = (uint32_t)__builtin_amdgcn_readlane((int)x, 16 * j + NW - 1);
  }
}

// Block-wide min and max of 32-bit values.
__device__ __forceinline__ void block_minmax32(uint32_t& lo, uint32_t& hi, SelShared& S, int& par) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  lo = wave_min_u32_in63(lo);
  hi = wave_max_u32_in63(hi);
  if (lane == 63) {
    S.r32[par][0][wid] = lo;
    S.r32[par][1][wid] = hi;
  }
  __syncthreads();
  // lanes 0..NW-1 take the waves' minima, lanes 16..16+NW-1 the complements of their
  // maxima; one min-scan down each 16-lane row leaves both results in lanes 15 and 31
  uint32_t x = 0xFFFFFFFFu;
  if (lane < NW) x = S.r32[par][0][lane];
  else if (lane >= 16 && lane < 16 + NW) x = ~S.r32[par][1][lane - 16];
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x118, 0xF, 0xF, false));  // row_shr:8
  lo = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  hi = ~(uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  par ^= 1;
}

// The need-th largest (1 <= need <= number of live keys) of the nonzero keys in
// kh[0, N)/kl[0, N) and, with EXTRA, in xs[0, nx) (LDS, thread t reading xs[t + SEL_NT j]),
// held across the workgroup. Keys are distinct.
__device__ __forceinline__ void clear_hist(SelShared& S) {
  constexpr int Q = (NBIN * NREP / 4 + SEL_NT - 1) / SEL_NT;  // 16-byte stores per thread
  v4i* hz = reinterpret_cast<v4i*>(S.a.hist);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = (int)threadIdx.x + SEL_NT * q;
    if (i < NBIN * NREP / 4) hz[i] = v4i{0, 0, 0, 0};
  }
}
// Thread t's two bins summed over their copies: h0 = bin NBIN-1-2t (upper), h1 = bin
// NBIN-2-2t, so that thread order is descending digit order.
__device__ __forceinline__ void bin_pair(const SelShared& S, int tid, uint32_t& h0, uint32_t& h1) {
  const uint32_t* hb = S.a.hist + (NBIN - 2 - 2 * tid) * NREP;
  h0 = 0u;
  h1 = 0u;
#pragma unroll
  for (int q = 0; q < NREP; ++q) {
    h1 += hb[q];
    h0 += hb[NREP + q];
  }
}

// Register keys come as score words kh[] and token words kl[] (key = kh << 32 | kl;
// kh == 0 marks an empty slot: no finite score maps to 0). The passes read only the
// score words, so the token words may still be in flight until the bucket stage:
// `late()` runs once, after the first histogram pass (or before the bucket stage when
// no pass runs), where the caller issues the loads that only later stages need (the
// token words among them): they then neither compete with the score words for the
// workgroup's load bandwidth nor stall the min / max and histogram phases, and arrive
// while the digit scan runs. PRECLEARED: the caller has already zeroed the histogram
// and the bucket count (before its first barrier).
template <int N, bool EXTRA, bool PRECLEARED = false, typename Late>
__device__ __forceinline__ uint64_t kth_largest(const uint32_t (&kh)[PER], const uint32_t (&kl)[PER], const uint64_t* xs,
                                                uint32_t nx, uint32_t need, SelShared& S, int& par, Late&& late) {
  const int tid = threadIdx.x, lane = tid & 63;
  // fn(score word, token word) over the register keys, then (only when the LDS list
  // is not empty, a uniform branch) over xs[tid + SEL_NT x], x < XPER
  auto for_keys = [&](auto&& fn) {
#pragma unroll
    for (int i = 0; i < N; ++i) fn(kh[i], kl[i]);
    if (EXTRA && nx > 0) {
#pragma unroll
      for (int x = 0; x < XPER; ++x) {
        const uint32_t p = (uint32_t)tid + (uint32_t)x * SEL_NT;
        const uint64_t v = p < nx ? xs[p] : 0ull;
        fn((uint32_t)(v >> 32), (uint32_t)v);
      }
    }
  };
  if (!PRECLEARED) {
    if (tid == 0) S.bcount = 0u;  // the bucket gather is ordered after this by the barriers below
    clear_hist(S);                // ordered before the first pass by the min / max barrier
  }
  // the least live score word via min(w - 1) (an empty slot, w = 0, wraps to the
  // identity), the largest via max(w) (0 changes nothing)
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for_keys([&](uint32_t w, uint32_t) {
    lo = min(lo, w - 1u);
    hi = max(hi, w);
  });
  block_minmax32(lo, hi, S, par);
  lo += 1u;
  // score-word bits fixed so far: (w & mask) == prefix
  // bits above `top` are common to every live score word; (w & mask) == prefix
  // selects the keys still in play. 64-bit shifts keep every shift count defined.
  int top = -1;  // -1: every live key has the same score word
  if (lo != hi) top = 31 - __clz(lo ^ hi);
  uint32_t mask = (uint32_t)(~0ull << (top + 1));
  uint32_t prefix = hi & mask;
  uint32_t cnt = 0;
  bool first = true;
  while (top >= 0) {
    const int width = top + 1 < HBITS ? top + 1 : HBITS;
    const int sh = top + 1 - width;
    const uint32_t dm = (1u << width) - 1u;
    const bool pass0 = first;
    if (!first) {
      clear_hist(S);
      __syncthreads();
    }
    first = false;
    const uint32_t rep = (uint32_t)tid & (NREP - 1);
    if (pass0) {  // every live key lies in [lo, hi], so it shares the bits above top
      for_keys([&](uint32_t w, uint32_t) {
        if (w != 0u) atomicAdd(&S.a.hist[((w >> sh) & dm) * NREP + rep], 1u);
      });
    } else {
      for_keys([&](uint32_t w, uint32_t) {
        if (w != 0u && (w & mask) == prefix) atomicAdd(&S.a.hist[((w >> sh) & dm) * NREP + rep], 1u);
      });
    }
    __syncthreads();
    if (pass0) late();
    // thread t holds bins NBIN-1-2t (upper) and NBIN-2-2t: thread order = descending digits
    uint32_t h0, h1;
    {
      bin_pair(S, tid, h0, h1);
    }
    uint32_t tot;
    const uint32_t above = excl_scan(h0 + h1, tot, S, par);
    if (above < need && above + h0 + h1 >= need) {
      if (above + h0 >= need) {
        S.res[0] = NBIN - 1 - 2 * tid;
        S.res[1] = above;
        S.res[2] = h0;
      } else {
        S.res[0] = NBIN - 2 - 2 * tid;
        S.res[1] = above + h0;
        S.res[2] = h1;
      }
    }
    __syncthreads();
    const uint32_t d = S.res[0], ab = S.res[1];
    cnt = S.res[2];
    need -= ab;
    prefix |= d << sh;
    mask |= dm << sh;
    top = sh - 1;
    if (cnt <= 64u) break;
  }
  if (first) late();  // no histogram pass ran
  // the bucket: live keys whose score word matches; need-th largest among them
  if (top < 0 && cnt == 0u) {
    // no pass ran (one score word): count the bucket
    uint32_t c = 0;
    for_keys([&](uint32_t w, uint32_t) { c += w != 0u ? 1u : 0u; });
    uint32_t unused;
    excl_scan(c, unused, S, par);
    cnt = unused;
  }
  if (cnt <= 64u) {
    for_keys([&](uint32_t w, uint32_t l) {
      if (w != 0u && (w & mask) == prefix) S.bucket[atomicAdd(&S.bcount, 1u) & 63u] = ((uint64_t)w << 32) | l;
    });
    __syncthreads();
    // The bucket's keys are distinct, so the need-th largest is the one with exactly
    // need - 1 larger keys. Wave w ranks bucket keys 4 w .. 4 w + 3 (one compare per
    // lane against every bucket key and a ballot each), all waves at once.
    {
      const int wid = tid >> 6;
      const uint64_t v = (uint32_t)lane < cnt ? S.bucket[lane] : 0ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t j = 4u * (uint32_t)wid + (uint32_t)q;
        if (j < cnt) {  // uniform
          const uint64_t pj = S.bucket[j];
          const uint32_t rank = (uint32_t)__popcll(__ballot(v > pj));
          if (rank == need - 1u && lane == 0) S.res64 = pj;
        }
      }
    }
    __syncthreads();
    return S.res64;
  }
  // more than 64 keys share the whole score word: resolve the token bits by radix
  uint32_t lmask = 0u, lprefix = 0u;
  for (int sh = 32 - HBITS; sh > -HBITS; sh -= HBITS) {
    const int s0 = sh < 0 ? 0 : sh;
    const int width = sh < 0 ? HBITS + sh : HBITS;
    const uint32_t dm = (1u << width) - 1u;
    clear_hist(S);
    __syncthreads();
    const uint32_t rep = (uint32_t)tid & (NREP - 1);
    for_keys([&](uint32_t w, uint32_t lw) {
      if (w != 0u && (w & mask) == prefix && (lw & lmask) == lprefix)
        atomicAdd(&S.a.hist[((lw >> s0) & dm) * NREP + rep], 1u);
    });
    __syncthreads();
    uint32_t h0, h1;
    {
      bin_pair(S, tid, h0, h1);
    }
    uint32_t tot;
    const uint32_t above = excl_scan(h0 + h1, tot, S, par);
    if (above < need && above + h0 + h1 >= need) {
      if (above + h0 >= need) {
        S.res[0] = NBIN - 1 - 2 * tid;
        S.res[1] = above;
      } else {
        S.res[0] = NBIN - 2 - 2 * tid;
        S.res[1] = above + h0;
      }
    }
    __syncthreads();
    need -= S.res[1];
    lprefix |= S.res[0] << s0;
    lmask |= dm << s0;
    __syncthreads();
  }
  return ((uint64_t)prefix << 32) | lprefix;
}

__device__ __forceinline__ int32_t page_slot(const CacheView& cv, const RowMap& rm, int seq, int t) {
  return (int32_t)(token_block(cv, rm, seq, t) * cv.block_size + (t & (cv.block_size - 1)));
}

__device__ __forceinline__ int key_token(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }

// Exact selection over the whole row straight from global memory (8-bit digits,
// per-wave LDS histograms), then a sort of the k tokens. Only reached when the
// rescans outgrow LDS (e.g. scores tied across far more than k tokens). Like every
// path of the select it leaves the selection as the LDS list (a.hist, nsel).
__device__ __forceinline__ void select_row_global(const float* __restrict__ srow, int ctx, int k, SelShared& S,
                                               int32_t* __restrict__ orow, int32_t* __restrict__ prow, CacheView cv,
                                               RowMap rm, int seq) {
  const int tid = threadIdx.x, wid = tid >> 6;
  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)k;
  __syncthreads();
  for (int sh = 56; sh >= 0; sh -= 8) {
    for (int i = tid; i < NW * 256; i += SEL_NT) S.g.hist[i] = 0u;
    __syncthreads();
    for (int t = tid; t < ctx; t += SEL_NT) {
      const uint64_t c = composite_key(srow[t], t);
      if ((c & mask) == prefix) atomicAdd(&S.g.hist[wid * 256 + ((c >> sh) & 0xFF)], 1u);
    }
    __syncthreads();
    uint32_t v = 0;
    if (tid < 256)
      for (int w = 0; w < NW; ++w) v += S.g.hist[w * 256 + tid];
    __syncthreads();
    if (tid < 256) S.g.hist[tid] = v;
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      for (int d = 255; d >= 0; --d) {
        const uint32_t x = S.g.hist[d];
        if (above + x >= need) {
          S.res[0] = (uint32_t)d;
          S.res[1] = above;
          break;
        }
        above += x;
      }
    }
    __syncthreads();
    const uint32_t dig = S.res[0], above = S.res[1];
    __syncthreads();
    need -= above;
    prefix |= (uint64_t)dig << sh;
    mask |= 0xFFull << sh;
  }
  if (tid == 0) S.ecount = 0;
  __syncthreads();
  for (int t = tid; t < ctx; t += SEL_NT)
    if (composite_key(srow[t], t) >= prefix) {
      const uint32_t pos = atomicAdd(&S.ecount, 1u);
      if (pos < (uint32_t)kMaxK) S.g.sel[pos] = (uint32_t)t;
    }
  __syncthreads();
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = k + tid; i < P; i += SEL_NT) S.g.sel[i] = 0xFFFFFFFFu;
  __syncthreads();
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += SEL_NT) {
        const int p = i ^ j;
        if (p > i) {
          const uint32_t a = S.g.sel[i], b = S.g.sel[p];
          if ((a > b) == ((i & kk) == 0)) {
            S.g.sel[i] = b;
            S.g.sel[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // the selection also stays in LDS as the list (a.hist, which lies below g.sel)
  for (int i = tid; i < k; i += SEL_NT) {
    const int t = (int)S.g.sel[i];
    if (orow) orow[i] = t;
    if (prow) prow[i] = page_slot(cv, rm, seq, t);
    S.a.hist[i] = (uint32_t)t;
  }
  if (tid == 0) S.nsel = (uint32_t)k;
  __syncthreads();
}


// Register i of thread t holds slot (candidate rows) or token (own-key rows)
// 8 t + i for i < 8 ("run A") and 8192 + 8 t + (i - 8) for i >= 8 ("run B"): thread
// order is slot order inside each run, and run A precedes run B.
__device__ __forceinline__ int reg_slot(int i) {
  return (i < 8 ? 0 : kCandRowCap / 2 - 8) + 8 * (int)threadIdx.x + i;
}

// Eight consecutive words at p (16-byte aligned) into v[0..8).
template <typename T>
__device__ __forceinline__ void load8(const T* p, T* v) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
  v[0] = __builtin_bit_cast(T, a.x); v[1] = __builtin_bit_cast(T, a.y);
  v[2] = __builtin_bit_cast(T, a.z); v[3] = __builtin_bit_cast(T, a.w);
  v[4] = __builtin_bit_cast(T, b.x); v[5] = __builtin_bit_cast(T, b.y);
  v[6] = __builtin_bit_cast(T, b.z); v[7] = __builtin_bit_cast(T, b.w);
}

// Everything the per-row body needs besides the register keys.
struct SelRow {
  int ctx, k, seq;
  const float* srow;
  const uint32_t* clo;   // the row's candidate token words
  const uint32_t* flr;   // the row's unit floors
  int32_t* orow;  // index output row, or nullptr (the selection stays in LDS only)
  int32_t* prow;  // page-slot output row, or nullptr
  bool stage_bt;  // stage the block-table row in LDS even without page-slot output
  CacheView cv;
  RowMap rm;
};

// Page slot of token t from the row's block-table entries staged in LDS (btl) or read.
__device__ __forceinline__ int32_t out_slot(const SelShared& S, bool btl, const SelRow& R, int t) {
  return btl ? S.bt[t >> R.cv.log2_bs] * R.cv.block_size + (t & (R.cv.block_size - 1))
             : page_slot(R.cv, R.rm, R.seq, t);
}

// The row's block-table entries go to LDS for the output's page slots when they fit.
struct BtStage {
  bool btl;
  int nblk;
  int32_t bv[BTCAP / SEL_NT];
  __device__ __forceinline__ void load(const SelRow& R) {
    nblk = (R.ctx + R.cv.block_size - 1) >> R.cv.log2_bs;
    btl = (R.prow != nullptr || R.stage_bt) && nblk <= BTCAP;
    if (!btl) return;
    const int32_t* btr = R.rm.block_table + (int64_t)R.seq * R.rm.bt_stride;
#pragma unroll
    for (int q = 0; q < BTCAP / SEL_NT; ++q) {
      const int i = (int)threadIdx.x + SEL_NT * q;
      bv[q] = i < nblk ? btr[i] : 0;
    }
  }
  __device__ __forceinline__ void stage(const SelRow& R, SelShared& S) {
    if (threadIdx.x == 0) S.btl = btl ? 1u : 0u;
    if (!btl) return;
    const uint32_t nb = R.cv.num_blocks < 0x7FFFFFFF ? (uint32_t)R.cv.num_blocks : 0x7FFFFFFFu;
#pragma unroll
    for (int q = 0; q < BTCAP / SEL_NT; ++q) {
      const int i = (int)threadIdx.x + SEL_NT * q;
      int32_t b = bv[q];
      if (i < nblk && (uint32_t)b >= nb) {  // negative entries too
        raise_status(R.cv.status, kStBlockClamped);
        b = b < 0 ? 0 : (int32_t)nb - 1;
      }
      if (i < nblk) S.bt[i] = b;
    }
  }
};

// Second half of the output: S.a.hist (free once the search is done) holds the `total`
// selected tokens in output order; every thread writes positions tid and tid + 1024 of
// the index row (and of the page-slot row), -1 past the selection. The list stays in
// LDS (length in nsel) for a consumer in the same workgroup.
__device__ __forceinline__ void flush_list(uint32_t total, const SelRow& R, const BtStage& B, SelShared& S) {
  const uint32_t nout = total < (uint32_t)R.k ? total : (uint32_t)R.k;
  if (threadIdx.x == 0) S.nsel = nout;
  if (R.orow == nullptr && R.prow == nullptr) return;
#pragma unroll
  for (int q = 0; q < kMaxK / SEL_NT; ++q) {
    const int i = (int)threadIdx.x + SEL_NT * q;
    if (i < R.k) {
      const int t = (uint32_t)i < nout ? (int)S.a.hist[i] : -1;
      if (R.orow) R.orow[i] = t;
      if (R.prow) R.prow[i] = t >= 0 ? out_slot(S, B.btl, R, t) : -1;
    }
  }
}

// Rows whose own scores are held (at most 16384 tokens): N = 8 or 16 tokens per thread.
template <int N>
__device__ __forceinline__ void select_own(SelShared& S, uint32_t (&kh)[PER], uint32_t (&kl)[PER], const SelRow& R,
                                           int& par) {
  BtStage B;
  B.load(R);
  // the row's keys: tokens reg_slot(i) < ctx
  {
    const int t0 = 8 * (int)threadIdx.x;
    const bool al = (reinterpret_cast<uintptr_t>(R.srow) & 15u) == 0;
#pragma unroll
    for (int h = 0; h < N / 8; ++h) {
      const int b0 = t0 + h * (kCandRowCap / 2);
      float f[8];
      if (al && b0 + 8 <= R.ctx) {
        load8(R.srow + b0, f);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = b0 + i < R.ctx ? R.srow[b0 + i] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = b0 + i;
        const uint64_t key = t < R.ctx ? composite_key(f[i], t) : 0ull;
        kh[8 * h + i] = (uint32_t)(key >> 32);
        kl[8 * h + i] = (uint32_t)key;
      }
    }
  }
  const uint64_t cstar = kth_largest<N, false>(kh, kl, nullptr, 0u, (uint32_t)R.k, S, par, [] {});
  B.stage(R, S);
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if ((((uint64_t)kh[i] << 32) | kl[i]) >= cstar) bits |= 1u << i;
  uint32_t v[4] = {(uint32_t)__popc(bits & 0xFFu), (uint32_t)__popc(bits >> 8), 0u, 0u}, off[4], tot[4];
  excl_scan4(v, off, tot, N / 8, S);
  const uint32_t base[2] = {off[0], tot[0] + off[1]};
  uint32_t* list = S.a.hist;  // free since the search
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t o = base[i >> 3] + (uint32_t)__popc(bits & (0xFFu << (i & ~7)) & ((1u << i) - 1u));
    if (((bits >> i) & 1u) && o < (uint32_t)R.k) list[o] = 0xFFFFFFFFu - kl[i];
  }
  __syncthreads();
  flush_list(tot[0] + (N > 8 ? tot[1] : 0u), R, B, S);
}

// The resend: the keys >= cu of the flagged units S.funit[0, nflag) go to S.a.ext, each
// unit's as one segment in token order (S.fstart, S.flen), segments in any order;
// S.ecount gets the total. Wave w takes units w, w + NW, ...; it issues the score loads
// of up to UPR of its units (CPU 64-token chunks each) before it ranks any of them, so
// that one round of loads covers up to 16 UPR units (32 of 512 tokens).
constexpr int RS_CPW = 16;  // 64-token chunks a wave loads per round
template <int CPU>
__device__ __forceinline__ void rescan_units(SelShared& S, const SelRow& R, uint32_t nflag, uint64_t cu) {
  constexpr int UPR = RS_CPW / CPU < 8 ? RS_CPW / CPU : 8;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (uint32_t q0 = (uint32_t)wid; q0 < nflag; q0 += NW * UPR) {  // wave-uniform
    float f[UPR * CPU];
    int t0[UPR];
#pragma unroll
    for (int u = 0; u < UPR; ++u) {
      const uint32_t q = q0 + (uint32_t)(NW * u);
      t0[u] = __builtin_amdgcn_readfirstlane(q < nflag ? (int)S.funit[q] * (64 * CPU) : -1);
#pragma unroll
      for (int c = 0; c < CPU; ++c) {
        const int t = t0[u] + 64 * c + lane;
        f[u * CPU + c] = (t0[u] >= 0 && t < R.ctx) ? R.srow[t] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < UPR; ++u) {
      const uint32_t q = q0 + (uint32_t)(NW * u);
      if (q >= nflag) break;  // uniform
      uint64_t bal[CPU];
      uint32_t tot = 0;
#pragma unroll
      for (int c = 0; c < CPU; ++c) {
        const int t = t0[u] + 64 * c + lane;
        bal[c] = __ballot(t < R.ctx && composite_key(f[u * CPU + c], t) >= cu);
        tot += (uint32_t)__popcll(bal[c]);
      }
      uint32_t st = 0;
      if (lane == 0) st = atomicAdd(&S.ecount, tot);
      st = (uint32_t)__shfl((int)st, 0, 64);
      uint32_t run = st;
#pragma unroll
      for (int c = 0; c < CPU; ++c) {
        const int t = t0[u] + 64 * c + lane;
        const uint32_t pos = run + (uint32_t)__popcll(bal[c] & ((1ull << lane) - 1ull));
        if (((bal[c] >> lane) & 1ull) && pos < (uint32_t)ECAP) S.a.ext[pos] = composite_key(f[u * CPU + c], t);
        run += (uint32_t)__popcll(bal[c]);
      }
      if (lane == 0) {
        S.fstart[q] = st;
        S.flen[q] = tot;
      }
    }
  }
}

// Candidate rows: register slots hold the units' sent keys (plan p, N = p.per).
// Segment j of a thread's registers: m >= 8 -> j = 0 (registers 0..7) and j = 2
// (8..15), one unit each; m = 4 -> j = 0..3, registers [4 j, 4 j + 4), one unit each.
template <int N>
__device__ __forceinline__ void select_cand(SelShared& S, uint32_t (&kh)[PER], uint32_t (&kl)[PER], const SelRow& R,
                                            const CandPlan& p, int& par) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nslot = p.nu << p.lm;
  const bool quarter = p.m < 8;  // m = 4: four one-unit segments of four registers
  const uint32_t segmask[4] = {quarter ? 0x000Fu : 0x00FFu, quarter ? 0x00F0u : 0u,
                               quarter ? 0x0F00u : (N > 8 ? 0xFF00u : 0u), quarter ? 0xF000u : 0u};
  int segu[4];  // unit of each segment (-1: none)
  bool segfirst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s0 = (j < 2 ? 0 : kCandRowCap / 2) + 8 * tid + (quarter ? 4 * (j & 1) : 0);
    const bool has = segmask[j] != 0u && s0 < nslot && (j < 2 || N > 8);
    segu[j] = has ? s0 >> p.lm : -1;
    segfirst[j] = has && (s0 & (p.m - 1)) == 0;
  }
  // slots past the row's units hold no candidate
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (reg_slot(i) >= nslot) kh[i] = 0u;

  BtStage B;
  uint32_t fl[4] = {0u, 0u, 0u, 0u};
  auto late = [&]() {
#pragma unroll
    for (int h = 0; h < N / 8; ++h) load8(R.clo + 8 * tid + h * (kCandRowCap / 2), kl + 8 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (segu[j] >= 0) fl[j] = R.flr[segu[j]];
    B.load(R);
  };
  // the search's histogram and bucket count were cleared by the caller
  const uint64_t cu = kth_largest<N, false, true>(kh, kl, nullptr, 0u, (uint32_t)R.k, S, par, late);
  B.stage(R, S);
  const uint32_t cu_hi = (uint32_t)(cu >> 32);
  uint32_t fmask = 0;  // flagged segments: their unit may hold unsent keys >= cu
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (segu[j] >= 0 && fl[j] != 0u && fl[j] >= cu_hi) fmask |= 1u << j;
  // Common case first: one scan gives the number of flagged units and, were there none,
  // every register key's output offset.
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if ((((uint64_t)kh[i] << 32) | kl[i]) >= cu) bits |= 1u << i;  // an empty slot (kh = 0) is below
  uint32_t nfl[2] = {0u, 0u};  // flagged units this thread registers, runs A and B
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (((fmask >> j) & 1u) && segfirst[j]) nfl[j >> 1]++;
  {
    // one prefix sum per run, packed: selected keys in the low half-word (at most 8,192
    // per run), flagged units in the high one
    uint32_t v[4] = {(uint32_t)__popc(bits & 0xFFu) | (nfl[0] << 16), (uint32_t)__popc(bits >> 8) | (nfl[1] << 16), 0u,
                     0u},
             pk[4], pt[4];
    excl_scan4(v, pk, pt, N > 8 ? 2 : 1, S);
    const uint32_t off[2] = {pk[0] >> 16, pk[1] >> 16}, tot[2] = {pt[0] >> 16, N > 8 ? pt[1] >> 16 : 0u};
    const uint32_t nflag = tot[0] + tot[1];
    if (nflag == 0) {
      const uint32_t totA = pt[0] & 0xFFFFu;
      const uint32_t base[2] = {pk[0] & 0xFFFFu, totA + (pk[1] & 0xFFFFu)};
      uint32_t* list = S.a.hist;  // free since the search
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const uint32_t o = base[i >> 3] + (uint32_t)__popc(bits & (0xFFu << (i & ~7)) & ((1u << i) - 1u));
        if (((bits >> i) & 1u) && o < (uint32_t)R.k) list[o] = 0xFFFFFFFFu - kl[i];
      }
      __syncthreads();
      flush_list(totA + (N > 8 ? pt[1] & 0xFFFFu : 0u), R, B, S);
      return;
    }
    if (nflag > (uint32_t)FCAP) {
      select_row_global(R.srow, R.ctx, R.k, S, R.orow, R.prow, R.cv, R.rm, R.seq);
      return;
    }
    // ---- resend: the flagged units' keys >= cu are rescanned from the scores ----
    uint32_t sl[2] = {off[0], tot[0] + off[1]};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (((fmask >> j) & 1u) && segfirst[j]) {
        const uint32_t q = sl[j >> 1]++;
        S.funit[q] = (uint32_t)segu[j];
        S.fmap[segu[j]] = (uint16_t)q;
      }
    if (tid == 0) S.ecount = 0u;
    __syncthreads();
    if (p.unit == 512)
      rescan_units<8>(S, R, nflag, cu);
    else if (p.unit == 256)
      rescan_units<4>(S, R, nflag, cu);
    else
      rescan_units<1>(S, R, nflag, cu);
    __syncthreads();
    const uint32_t ne = S.ecount;
    if (ne > (uint32_t)ECAP) {
      select_row_global(R.srow, R.ctx, R.k, S, R.orow, R.prow, R.cv, R.rm, R.seq);
      return;
    }
    // union: unflagged candidates >= cu in registers, rescanned keys from LDS
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = quarter ? (i >> 2) : ((i >> 3) << 1);
      if (((fmask >> j) & 1u) || (((uint64_t)kh[i] << 32) | kl[i]) < cu) kh[i] = 0u;
    }
    const uint64_t cstar = kth_largest<N, true>(kh, kl, S.a.ext, ne, (uint32_t)R.k, S, par, [] {});
    // ---- selected rescanned keys: thread t takes ext entries [XPER t, XPER t + XPER);
    // one block scan counts the selected entries before each thread's, and one thread per
    // segment turns its ends into the segment's count and the selected entries before it
    static_assert(XPER == 8 && XPER * SEL_NT == ECAP, "eight ext entries per thread");
    uint32_t xb = 0;
#pragma unroll
    for (int x = 0; x < XPER; ++x) {
      const uint32_t pe = (uint32_t)(XPER * tid + x);
      const uint64_t c = pe < ne ? S.a.ext[pe] : 0ull;
      if (c != 0ull && c >= cstar) xb |= 1u << x;
    }
    uint32_t xtot;
    const uint32_t xbefore = excl_scan((uint32_t)__popc(xb), xtot, S, par);
    uint32_t* xw = S.a.hist + 4096;  // per thread: selected entries before its own, its bits
    xw[tid] = (xbefore << 8) | xb;
    __syncthreads();
    auto sel_before = [&](uint32_t pe) -> uint32_t {  // selected ext entries below entry pe
      if (pe >= ne) return xtot;
      const uint32_t w = xw[pe >> 3];
      return (w >> 8) + (uint32_t)__popc(w & 0xFFu & ((1u << (pe & 7u)) - 1u));
    };
    for (uint32_t q = (uint32_t)tid; q < nflag; q += SEL_NT) {
      const uint32_t st = S.fstart[q], e0 = sel_before(st);
      S.fcnt[q] = sel_before(st + S.flen[q]) - e0;
      S.flen[q] = e0;
    }
    __syncthreads();
    // ---- ordered write: segment counts in token order, one scan per run ----
    bits = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((((uint64_t)kh[i] << 32) | kl[i]) >= cstar) bits |= 1u << i;
    uint32_t segc[4];
    uint32_t fsl[2] = {off[0], tot[0] + off[1]};  // this thread's first registered slot per run
    int fslot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fslot[j] = -1;
      if ((fmask >> j) & 1u) {
        if (segfirst[j]) {
          fslot[j] = (int)fsl[j >> 1]++;
          segc[j] = S.fcnt[fslot[j]];
        } else {
          segc[j] = 0u;
        }
      } else {
        segc[j] = (uint32_t)__popc(bits & segmask[j]);
      }
    }
    uint32_t v2[4] = {segc[0] + segc[1], segc[2] + segc[3], 0u, 0u}, off2[4], tot2[4];
    excl_scan4(v2, off2, tot2, N > 8 ? 2 : 1, S);
    uint32_t segoff[4];
    segoff[0] = off2[0];
    segoff[1] = off2[0] + segc[0];
    segoff[2] = tot2[0] + off2[1];
    segoff[3] = segoff[2] + segc[2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (fslot[j] >= 0) S.foff[fslot[j]] = segoff[j];
    uint32_t* list = S.a.hist;  // below xw
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = quarter ? (i >> 2) : ((i >> 3) << 1);
      const uint32_t o = segoff[j] + (uint32_t)__popc(bits & segmask[j] & ((1u << i) - 1u));
      if (((bits >> i) & 1u) && o < (uint32_t)R.k) list[o] = 0xFFFFFFFFu - kl[i];
    }
    __syncthreads();
    // a selected ext entry goes to its segment's first position plus its rank there
    const int lu = p.lu;
#pragma unroll
    for (int x = 0; x < XPER; ++x)
      if ((xb >> x) & 1u) {
        const uint64_t c = S.a.ext[XPER * tid + x];
        const int t = key_token(c);
        const uint32_t q = S.fmap[t >> lu];
        const uint32_t pos = S.foff[q] + xbefore + (uint32_t)__popc(xb & ((1u << x) - 1u)) - S.flen[q];
        if (pos < (uint32_t)R.k) list[pos] = (uint32_t)t;
      }
    __syncthreads();
    flush_list(tot2[0] + (N > 8 ? tot2[1] : 0u), R, B, S);
  }
}


// The select for row r, by all SEL_NT threads of a workgroup (none may have returned).
// CAND: rows may be longer than kTopkFullRow, so candidates were sent by producers whose
// units are at most `umax` tokens. load_b: the host's plan for max_ctx uses 16 keys per
// thread, so run B's score words are loaded with run A's as the select starts. `early()`
// runs right after the candidate loads are issued (a caller's own loads go out behind
// them). idx / phys may be nullptr; on return (after a barrier) the selection is the LDS
// list S.a.hist[0, S.nsel) in token order, and S.btl tells whether S.bt holds the row's
// block-table entries.
template <bool CAND, typename Early>
__device__ __forceinline__ void select_row(const uint32_t* __restrict__ cand_hi, const uint32_t* __restrict__ cand_lo,
                                           const uint32_t* __restrict__ floors, const float* __restrict__ scores,
                                           int64_t ld, const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                           int umax, int load_b, int32_t* __restrict__ idx,
                                           int32_t* __restrict__ phys, bool stage_bt, const CacheView& cv,
                                           const RowMap& rm, int r, SelShared& S, Early&& early) {
  const int tid = threadIdx.x;
  // The candidates' score words load first: their addresses need only the kernel
  // arguments, so they go out with the row's length; the first search needs nothing
  // else. Token words, unit floors and block-table entries follow after the search's
  // first histogram pass.
  uint32_t kh[PER], kl[PER];
  const uint32_t* ch = cand_hi + (int64_t)r * kCandRowCap;
  if (CAND) {
    load8(ch + 8 * tid, kh);
    if (load_b) load8(ch + kCandRowCap / 2 + 8 * tid, kh + 8);
  }
  early();
  SelRow R;
  R.ctx = __builtin_amdgcn_readfirstlane(clamp_ctx(row_ctx, r, max_ctx, cv.status));  // uniform: scalar plan
  R.k = k;
  R.seq = __builtin_amdgcn_readfirstlane(rm.row_seq[r]);  // row_seq is row_ctx when there are no page slots
  R.srow = scores + (int64_t)r * ld;
  R.clo = cand_lo + (int64_t)r * kCandRowCap;
  R.flr = floors + (int64_t)r * kFloorRowCap;
  R.orow = idx ? idx + (int64_t)r * k : nullptr;
  R.prow = phys ? phys + (int64_t)r * k : nullptr;
  R.stage_bt = stage_bt;
  R.cv = cv;
  R.rm = rm;
  if (tid == 0) S.btl = 0u;  // ordered before any staging by the barriers below
  if (CAND) {
    // the search's histogram and bucket count are cleared while the score words are in
    // flight (ordered before the first pass by the search's first barrier)
    if (tid == 0) S.bcount = 0u;
    clear_hist(S);
  }
  __builtin_amdgcn_sched_barrier(0);
  int par = 0;
  if (R.ctx <= k) {  // every token, in order
    for (int i = tid; i < k; i += SEL_NT) {
      if (R.orow) R.orow[i] = i < R.ctx ? i : -1;
      if (R.prow) R.prow[i] = i < R.ctx ? page_slot(cv, rm, R.seq, i) : -1;
      if (i < R.ctx) S.a.hist[i] = (uint32_t)i;
    }
    if (tid == 0) S.nsel = (uint32_t)R.ctx;
    __syncthreads();
    return;
  }
  const CandPlan p = cand_plan(R.ctx, umax);
  if (!CAND || p.unit == 0) {
    __syncthreads();  // the clear above (if any) is done before the search clears again
    if (R.ctx <= kCandRowCap / 2)
      select_own<8>(S, kh, kl, R, par);
    else
      select_own<16>(S, kh, kl, R, par);
  } else if (p.per == 16) {
    if (!load_b) load8(ch + kCandRowCap / 2 + 8 * tid, kh + 8);
    select_cand<16>(S, kh, kl, R, p, par);
  } else {
    select_cand<8>(S, kh, kl, R, p, par);
  }
  __syncthreads();  // the list and nsel are visible to the whole workgroup
}

}  // namespace

}  // namespace dsa
