// Exact per-row top-k over fp32 scores (ties -> lower token index).
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
  uint32_t flen[FCAP];
  uint32_t fcnt[FCAP];    // selected keys of the segment
  uint32_t foff[FCAP];    // their first output position
  uint64_t bucket[64];    // keys of the last histogram bucket
  uint64_t res64;
  uint32_t r32[2][2][NW];  // block min / max partials, double buffered
  uint32_t scan[2][NW];    // block prefix partials, double buffered
  uint32_t scan4[4][NW];   // per-wave totals of four prefix sums
  uint32_t res[4];
  uint32_t ecount, bcount;
  int32_t bt[BTCAP];  // the row's block-table entries (clamped into the pool) when they fit
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, xshfl<1>(v));
  v = min(v, xshfl<2>(v));
  v = min(v, xshfl<4>(v));
  v = min(v, xshfl<8>(v));
  v = min(v, xshfl<16>(v));
  v = min(v, xshfl<32>(v));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, xshfl<1>(v));
  v = max(v, xshfl<2>(v));
  v = max(v, xshfl<4>(v));
  v = max(v, xshfl<8>(v));
  v = max(v, xshfl<16>(v));
  v = max(v, xshfl<32>(v));
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
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t before = 0, tot = 0;
    if (j < nj) tot = wave_totals(S.scan4[j], before);
    off[j] = before + inc[j] - v[j];
    total[j] = tot;
  }
}

// Block-wide min and max of 32-bit values.
__device__ __forceinline__ void block_minmax32(uint32_t& lo, uint32_t& hi, SelShared& S, int& par) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    S.r32[par][0][wid] = lo;
    S.r32[par][1][wid] = hi;
  }
  __syncthreads();
  lo = 0xFFFFFFFFu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, S.r32[par][0][w]);
    hi = max(hi, S.r32[par][1][w]);
  }
  par ^= 1;
}

// The need-th largest (1 <= need <= number of live keys) of the nonzero keys in
// kh[]/kl[] and, with EXTRA, in xs[0, nx) (LDS, thread t reading xs[t + SEL_NT j]), held
// across the workgroup. Keys are distinct.
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
__device__ __forceinline__ uint64_t kth_largest(const uint32_t (&kh)[N], const uint32_t (&kl)[N], const uint64_t* xs,
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
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for_keys([&](uint32_t w, uint32_t) {
    if (w != 0u) {
      lo = min(lo, w);
      hi = max(hi, w);
    }
  });
  block_minmax32(lo, hi, S, par);
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
    for_keys([&](uint32_t w, uint32_t) {
      if (w != 0u && (w & mask) == prefix) atomicAdd(&S.a.hist[((w >> sh) & dm) * NREP + rep], 1u);
    });
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

// Page slot of token t, from the staged block-table row when `btl`.
__device__ __forceinline__ int32_t slot_of(const SelShared& S, bool btl, const CacheView& cv, const RowMap& rm, int seq,
                                           int t) {
  if (btl) return S.bt[t >> cv.log2_bs] * cv.block_size + (t & (cv.block_size - 1));
  return page_slot(cv, rm, seq, t);
}

// Second half of the output write: S.a.hist (free once the search is done) holds the
// `total` selected tokens in output order; every thread writes positions tid and
// tid + 1024 of the index row (and of the page-slot row), -1 past the selection.
__device__ __forceinline__ void flush_selection(uint32_t total, int k, int32_t* __restrict__ orow,
                                                int32_t* __restrict__ prow, const CacheView& cv, const RowMap& rm,
                                                int seq, bool btl, const SelShared& S) {
  const uint32_t nout = total < (uint32_t)k ? total : (uint32_t)k;
#pragma unroll
  for (int q = 0; q < kMaxK / SEL_NT; ++q) {
    const int i = (int)threadIdx.x + SEL_NT * q;
    if (i < k) {
      const int t = (uint32_t)i < nout ? (int)S.a.hist[i] : -1;
      orow[i] = t;
      if (prow) prow[i] = t >= 0 ? slot_of(S, btl, cv, rm, seq, t) : -1;
    }
  }
}

// Exact selection over the whole row straight from global memory (8-bit digits,
// per-wave LDS histograms), then a sort of the k tokens. Only reached when the
// rescans outgrow LDS (e.g. scores tied across far more than k tokens).
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
  for (int i = tid; i < k; i += SEL_NT) {
    const int t = (int)S.g.sel[i];
    orow[i] = t;
    if (prow) prow[i] = page_slot(cv, rm, seq, t);
  }
}

}  // namespace

// Stage 1 over an existing score array (the standalone top-k entry point): one
// workgroup per 256 tokens of a row, all threads reaching the send.
__global__ __launch_bounds__(256) void topk_send_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_ctx, int max_ctx,
                                                        TopkWs ws) {
  __shared__ uint32_t send_lds[68];
  const int r = blockIdx.y;
  const int ctx = clamp_ctx(row_ctx, r, max_ctx, nullptr);  // the select reports it
  const int base = blockIdx.x * 256;
  if (base >= ctx) return;  // whole workgroup
  const int t = base + threadIdx.x;
  const bool valid = t < ctx;
  const float s = valid ? scores[(int64_t)r * ld + t] : 0.f;
  send_candidates(s, valid, ctx, base, r, ws, send_lds);
}

// CAND: rows may be longer than kTopkFullRow, so candidates were sent.
template <bool CAND>
// The candidate arrays lead the argument list so that their addresses arrive preloaded in
// scalar registers (kernel-argument preloading covers leading scalar and pointer
// arguments, not structures) and the candidate loads start with the kernel.
__global__ __launch_bounds__(SEL_NT) void topk_select_kernel(const uint32_t* __restrict__ cand_hi,
                                                             const uint32_t* __restrict__ cand_lo,
                                                             const uint32_t* __restrict__ floors,
                                                             const float* __restrict__ scores, int64_t ld,
                                                             const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                                             int32_t* __restrict__ idx, int32_t* __restrict__ phys,
                                                             CacheView cv, RowMap rm) {
  const TopkWs ws{const_cast<uint32_t*>(cand_hi), const_cast<uint32_t*>(cand_lo), const_cast<uint32_t*>(floors)};
  __shared__ SelShared S;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // The candidates' score words load first, alone: their addresses need only the kernel
  // arguments, so they go out with the row's length (slots the row's plan does not use
  // are cleared once the length is known), and the first search needs nothing else. The
  // token words, unit floors and block-table entries are issued after the search's first
  // histogram pass, so that one workgroup's load bandwidth goes to the score words first.
  uint32_t kh[PER], kl[PER];
  uint32_t fl[4] = {0u, 0u, 0u, 0u};
  if (CAND) {
    const uint32_t* ch = ws.cand_hi + (int64_t)r * kCandRowCap;
#pragma unroll
    for (int i = 0; i < PER; ++i) kh[i] = ch[i * SEL_NT + tid];
  }
  const int ctx = clamp_ctx(row_ctx, r, max_ctx, cv.status);
  const int seq = rm.row_seq[r];  // the launch points row_seq at row_ctx when there are no page slots
  int32_t* orow = idx + (int64_t)r * k;
  int32_t* prow = phys ? phys + (int64_t)r * k : nullptr;
  const float* srow = scores + (int64_t)r * ld;
  int par = 0;
  auto write_all = [&]() {  // ctx <= k: every token, in order
    for (int i = tid; i < k; i += SEL_NT) {
      orow[i] = i < ctx ? i : -1;
      if (prow) prow[i] = i < ctx ? page_slot(cv, rm, seq, i) : -1;
    }
  };
  if (!CAND && ctx <= k) {
    write_all();
    return;
  }

  // the row's block-table entries for the page slots of the output, staged in LDS;
  // one dependent global load per written token would otherwise sit on the write path
  const int nblk = (ctx + cv.block_size - 1) >> cv.log2_bs;
  const bool btl = prow != nullptr && nblk <= BTCAP;
  int32_t bv[BTCAP / SEL_NT];
  auto load_bt = [&]() {
    if (!btl) return;
    const int32_t* btr = rm.block_table + (int64_t)seq * rm.bt_stride;
#pragma unroll
    for (int q = 0; q < BTCAP / SEL_NT; ++q) {
      const int i = tid + SEL_NT * q;
      bv[q] = i < nblk ? btr[i] : 0;
    }
  };
  if (!CAND) load_bt();
  // The entries reach LDS after the first search: they sit one scalar round trip
  // further down the load chain than the candidates, and a store waiting for them
  // ahead of the search's first barrier would hold every wave.
  auto stage_bt = [&]() {
    if (!btl) return;
    const int64_t nb = cv.num_blocks;
#pragma unroll
    for (int q = 0; q < BTCAP / SEL_NT; ++q) {
      const int i = tid + SEL_NT * q;
      int64_t b = bv[q];
      if (i < nblk && (uint64_t)b >= (uint64_t)nb) {
        raise_status(cv.status, kStBlockClamped);
        b = b < 0 ? 0 : nb - 1;
      }
      if (i < nblk) S.bt[i] = (int32_t)b;
    }
  };

  // The row's own keys (rows of at most kTopkFullRow tokens): thread t holds tokens
  // [16 t, 16 t + 16), one 16-key unit per thread.
  auto load_own = [&]() {
    const int t0 = tid * PER;
    float f[PER];
    if ((reinterpret_cast<uintptr_t>(srow) & 15u) == 0 && t0 + PER <= ctx) {
      const float4* p4 = reinterpret_cast<const float4*>(srow + t0);
#pragma unroll
      for (int x = 0; x < PER / 4; ++x) {
        const float4 v = p4[x];
        f[4 * x] = v.x;
        f[4 * x + 1] = v.y;
        f[4 * x + 2] = v.z;
        f[4 * x + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) f[i] = t0 + i < ctx ? srow[t0 + i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = t0 + i;
      const uint64_t key = t < ctx ? composite_key(f[i], t) : 0ull;
      kh[i] = (uint32_t)(key >> 32);
      kl[i] = (uint32_t)key;
    }
  };

  // Unit layout of the register keys: thread t holds units t + 1024 j (j < upt) with m
  // keys each, unit j in slots [m j, m j + m). Candidates: slot q + m j = rank q of unit
  // t + 1024 j. Own keys: m = 16, upt = 1.
  int m = PER, lm = 4, upt = 1;
  uint32_t fmask = 0, fbase = 0, nflag = 0;
  uint64_t cstar;
  if (!CAND) {
    load_own();
    cstar = kth_largest<PER, false>(kh, kl, nullptr, 0u, (uint32_t)k, S, par, [] {});
    stage_bt();
  } else {
    const CandPlan p = cand_plan(ctx);
    m = p.m;
    lm = 31 - __clz(m);
    upt = (p.nu + SEL_NT - 1) / SEL_NT;  // 1, 2 or 4; upt * m <= 16
    uint32_t umine = 0;                  // this thread's units that exist
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < upt && tid + SEL_NT * j < p.nu) umine |= 1u << j;
    // the search's histogram and bucket count are cleared while the score words are in
    // flight (ordered before the first pass by the search's first barrier)
    if (tid == 0) S.bcount = 0u;
    clear_hist(S);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (!((umine >> (i >> lm)) & 1u)) kh[i] = 0u;
    auto late = [&]() {
      const uint32_t* cl = ws.cand_lo + (int64_t)r * kCandRowCap;
#pragma unroll
      for (int i = 0; i < PER; ++i) kl[i] = cl[i * SEL_NT + tid];
      const uint32_t* rf = ws.floors + (int64_t)r * kFloorRowCap;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < upt) fl[j] = rf[tid + SEL_NT * j];
      load_bt();
    };
    // The first search comes before the short-row exits so that nothing between the
    // kernel's start and the first use of the candidates is a branch (a branch lets
    // the compiler sink the loads behind the row-length round trip).
    const uint64_t c1 = kth_largest<PER, false, true>(kh, kl, nullptr, 0u, (uint32_t)k, S, par, late);
    if (ctx <= k) {
      write_all();
      return;
    }
    if (ctx <= kTopkFullRow) {
      // A short row in a launch with longer rows: its own scores, read whole, take one
      // search. (Its 64-token units sent a quarter of their tokens, which can be fewer
      // than k, and every unit would need a rescan.)
      load_own();
      cstar = kth_largest<PER, false>(kh, kl, nullptr, 0u, (uint32_t)k, S, par, [] {});
      stage_bt();
      m = PER;
      lm = 4;
      upt = 1;
    } else {
      stage_bt();
      // Rows longer than kTopkFullRow sent at least 4096 >= k candidates (a 64-token unit
      // sends a quarter of its tokens, a 256-token unit m with nu * m >= 4096).
      const uint64_t cu = c1;
      const uint32_t cu_hi = (uint32_t)(cu >> 32);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (((umine >> j) & 1u) && fl[j] != 0u && fl[j] >= cu_hi) fmask |= 1u << j;
      cstar = c1;
      if (upt < 4) {
        // Common case first: one block scan gives both the number of flagged units and,
        // were there none, every unit's output offset, so with no flagged unit the
        // selection is written without a second scan.
        uint32_t bits = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (kh[i] != 0u && (((uint64_t)kh[i] << 32) | kl[i]) >= c1) bits |= 1u << i;
        const uint32_t umask = m >= 16 ? 0xFFFFu : ((1u << m) - 1u);
        uint32_t v[4] = {(uint32_t)__popc(fmask), 0u, 0u, 0u}, off[4], tot[4];
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < upt) v[1 + j] = (uint32_t)__popc(bits & ((umask << (m * j)) & 0xFFFFu));
        excl_scan4(v, off, tot, upt + 1, S);
        nflag = tot[0];
        fbase = off[0];
        if (nflag == 0) {
          uint32_t base = 0, uoff[3];
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            uoff[j] = base + off[1 + j];
            base += j < upt ? tot[1 + j] : 0u;
          }
          const uint32_t total = base;
          uint32_t* list = S.a.hist;  // free since the search
#pragma unroll
          for (int i = 0; i < PER; ++i) {
            const int j = i >> lm;
            const uint32_t oj = j == 0 ? uoff[0] : j == 1 ? uoff[1] : uoff[2];
            const uint32_t o = oj + (uint32_t)__popc(bits & (umask << (m * j)) & ((1u << i) - 1u));
            if (((bits >> i) & 1u) && o < (uint32_t)k) list[o] = 0xFFFFFFFFu - kl[i];
          }
          __syncthreads();
          flush_selection(total, k, orow, prow, cv, rm, seq, btl, S);
          return;
        }
        __syncthreads();  // the write path below runs its own scan4
      } else {
        fbase = excl_scan((uint32_t)__popc(fmask), nflag, S, par);
      }
      if (nflag > 0) {
        if (nflag > (uint32_t)FCAP) {
          select_row_global(srow, ctx, k, S, orow, prow, cv, rm, seq);
          return;
        }
        // ---- resend: each flagged unit's keys >= c_u, rescanned by one wave per unit ----
        {
          uint32_t fm = fmask, sl = fbase;
          while (fm) {
            const int j = __ffs(fm) - 1;
            fm &= fm - 1u;
            S.funit[sl++] = (uint32_t)(tid + SEL_NT * j);
          }
        }
        if (tid == 0) S.ecount = 0u;
        __syncthreads();
        const int chunks = p.unit >> 6;  // 64-token chunks per unit: 1 or 4
        for (uint32_t sl = wid; sl < nflag; sl += NW) {
          const int t0 = (int)S.funit[sl] * p.unit;
          float f[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int t = t0 + 64 * c + lane;
            f[c] = (c < chunks && t < ctx) ? srow[t] : 0.f;
          }
          uint64_t bal[4];
          uint32_t tot = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int t = t0 + 64 * c + lane;
            const bool keep = c < chunks && t < ctx && composite_key(f[c], t) >= cu;
            bal[c] = __ballot(keep);
            tot += (uint32_t)__popcll(bal[c]);
          }
          uint32_t st = 0;
          if (lane == 0) st = atomicAdd(&S.ecount, tot);
          st = (uint32_t)__shfl((int)st, 0, 64);
          uint32_t run = st;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int t = t0 + 64 * c + lane;
            const uint32_t pos = run + (uint32_t)__popcll(bal[c] & ((1ull << lane) - 1ull));
            if (((bal[c] >> lane) & 1ull) && pos < (uint32_t)ECAP) S.a.ext[pos] = composite_key(f[c], t);
            run += (uint32_t)__popcll(bal[c]);
          }
          if (lane == 0) {
            S.fstart[sl] = st;
            S.flen[sl] = tot;
          }
        }
        __syncthreads();
        const uint32_t ne = S.ecount;
        if (ne > (uint32_t)ECAP) {
          select_row_global(srow, ctx, k, S, orow, prow, cv, rm, seq);
          return;
        }
        // union: unflagged candidates >= c_u in registers, rescanned keys from LDS
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const bool flagged = (fmask >> (i >> lm)) & 1u;
          if (flagged || (((uint64_t)kh[i] << 32) | kl[i]) < cu) kh[i] = 0u;
        }
        cstar = kth_largest<PER, true>(kh, kl, S.a.ext, ne, (uint32_t)k, S, par, [] {});
        // selected keys of each rescanned unit
        for (uint32_t sl = wid; sl < nflag; sl += NW) {
          const uint32_t st = S.fstart[sl], len = S.flen[sl];
          uint32_t c = 0;
          for (uint32_t q0 = 0; q0 < len; q0 += 64) {
            const bool sel = q0 + (uint32_t)lane < len && S.a.ext[st + q0 + lane] >= cstar;
            c += (uint32_t)__popcll(__ballot(sel));
          }
          if (lane == 0) S.fcnt[sl] = c;
        }
        __syncthreads();
      }
    }  // rows longer than kTopkFullRow
  }

  // ---- ordered write: unit counts, prefix sums over units (unit u = tid + 1024 j) ----
  uint32_t bits = 0;  // selected register keys
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (kh[i] != 0u && (((uint64_t)kh[i] << 32) | kl[i]) >= cstar) bits |= 1u << i;
  const uint32_t umask = m >= 16 ? 0xFFFFu : ((1u << m) - 1u);  // keys of one unit
  uint32_t cnt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t mj = j < upt ? (umask << (m * j)) & 0xFFFFu : 0u;
    cnt[j] = (fmask >> j) & 1u ? S.fcnt[fbase + (uint32_t)__popc(fmask & ((1u << j) - 1u))]
                               : (uint32_t)__popc(bits & mj);
  }
  uint32_t off[4], tot[4];
  excl_scan4(cnt, off, tot, upt, S);
  uint32_t base = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    off[j] += base;
    base += tot[j];
  }
  const uint32_t total = base;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if ((fmask >> j) & 1u) S.foff[fbase + (uint32_t)__popc(fmask & ((1u << j) - 1u))] = off[j];
  // selected tokens go to their output positions in an LDS list first (the histogram
  // is free now), then one coalesced pass writes the index and page-slot rows
  uint32_t* list = S.a.hist;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = i >> lm;
    const uint32_t oj = j == 0 ? off[0] : j == 1 ? off[1] : j == 2 ? off[2] : off[3];
    const uint32_t o = oj + (uint32_t)__popc(bits & (umask << (m * j)) & ((1u << i) - 1u));
    if (((bits >> i) & 1u) && o < (uint32_t)k) list[o] = 0xFFFFFFFFu - kl[i];
  }
  if (nflag > 0) {
    __syncthreads();
    for (uint32_t sl = wid; sl < nflag; sl += NW) {
      const uint32_t st = S.fstart[sl], len = S.flen[sl];
      uint32_t o = S.foff[sl];
      for (uint32_t q0 = 0; q0 < len; q0 += 64) {
        const uint64_t c = q0 + (uint32_t)lane < len ? S.a.ext[st + q0 + lane] : 0ull;
        const bool sel = c != 0ull && c >= cstar;
        const uint64_t bal = __ballot(sel);
        const uint32_t pos = o + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        if (sel && pos < (uint32_t)k) list[pos] = (uint32_t)key_token(c);
        o += (uint32_t)__popcll(bal);
      }
    }
  }
  __syncthreads();
  flush_selection(total, k, orow, prow, cv, rm, seq, btl, S);
}

hipError_t launch_topk_send(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx,
                            const TopkWs& ws, hipStream_t stream) {
  if (R <= 0 || max_ctx <= kTopkFullRow) return hipSuccess;
  dim3 grid((max_ctx + 255) / 256, R);
  hipLaunchKernelGGL(topk_send_kernel, grid, dim3(256), 0, stream, scores, ld, row_ctx, max_ctx, ws);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                              int32_t* idx, const TopkWs& ws, int32_t* phys, const CacheView* cv, const RowMap* rm,
                              hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  CacheView c{};
  RowMap m{};
  if (cv) c = *cv;  // without page slots only its status word is used
  if (phys) m = *rm;
  if (!phys) m.row_seq = row_ctx;  // read, never used
  if (max_ctx > kTopkFullRow)
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3(R), dim3(SEL_NT), 0, stream, ws.cand_hi, ws.cand_lo, ws.floors,
                       scores, ld, row_ctx, max_ctx, k, idx, phys, c, m);
  else
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3(R), dim3(SEL_NT), 0, stream, ws.cand_hi, ws.cand_lo, ws.floors,
                       scores, ld, row_ctx, max_ctx, k, idx, phys, c, m);
  return hipGetLastError();
}

}  // namespace dsa
