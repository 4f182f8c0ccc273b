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
// sends its m best keys in token order plus a floor bounding the keys it kept.
// Stage 2 (topk_select_kernel, one 1024-thread workgroup per row). Every thread
// holds 16 keys in registers, a contiguous run in token order:
//   ctx <= k      every token;
//   ctx <= 16384  the row's own keys;
//   otherwise     the candidates (whole units per thread); c_u = their k-th
//                 largest key; a unit whose floor reaches c_u may hold unsent keys
//                 >= c_u and is rescanned from the scores (the "resend"), giving a
//                 set U in token order whose k largest keys are the row's top k.
// The k-th largest key is found two bits at a time over 32-bit words (score bits,
// then token bits for exact ties), counting with ballots; the result is written by
// an ordered compaction, ascending, with no sort.
#include "common.h"
#include "internal.h"
#include "topk_send.h"

namespace dsa {

namespace {

constexpr int SEL_NT = 1024;
constexpr int NW = SEL_NT / 64;
constexpr int PER = 16;  // keys per thread
static_assert(PER * SEL_NT == kCandRowCap && PER * SEL_NT == kTopkFullRow, "register tiling");

__device__ __forceinline__ int clamp_ctx(const int32_t* row_ctx, int r, int max_ctx) {
  int c = row_ctx[r];
  c = c < 0 ? 0 : c;
  return c > max_ctx ? max_ctx : c;
}

struct SelShared {
  uint64_t buf[kCandRowCap];  // U on the resend path
  union {
    uint32_t hist[NW * 256];  // whole-row fallback histograms
    uint32_t sel[kMaxK];      // whole-row fallback selection before its sort
  };
  uint32_t red[2][NW][4];     // per-wave partial results, double buffered
  uint64_t mred[NW];
  uint32_t scan[NW + 1];
  uint32_t res[4];
  uint32_t cnt[2];
};

__device__ __forceinline__ uint64_t block_min64(uint64_t v, SelShared& S) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_min_u64(v);
  __syncthreads();
  if (lane == 0) S.mred[wid] = v;
  __syncthreads();
  uint64_t t = ~0ull;
#pragma unroll
  for (int w = 0; w < NW; ++w) t = S.mred[w] < t ? S.mred[w] : t;
  return t;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  uint32_t o;
  o = xshfl<1>(v); v = o < v ? o : v;
  o = xshfl<2>(v); v = o < v ? o : v;
  o = xshfl<4>(v); v = o < v ? o : v;
  o = xshfl<8>(v); v = o < v ? o : v;
  o = xshfl<16>(v); v = o < v ? o : v;
  o = xshfl<32>(v); v = o < v ? o : v;
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t o;
  o = xshfl<1>(v); v = o > v ? o : v;
  o = xshfl<2>(v); v = o > v ? o : v;
  o = xshfl<4>(v); v = o > v ? o : v;
  o = xshfl<8>(v); v = o > v ? o : v;
  o = xshfl<16>(v); v = o > v ? o : v;
  o = xshfl<32>(v); v = o > v ? o : v;
  return v;
}

// need-th largest (1 <= need <= number of valid keys) of the nonzero 64-bit keys e[].
// Resolves the 32-bit score word, then (only if scores tie at the threshold) the
// token word, 8 bits per pass with one LDS histogram per wave; the leading bits all
// live words share are skipped, and a pass ends the search once every key left in
// the current bucket is selected.
__device__ uint64_t select_kth(const uint64_t (&e)[PER], uint32_t need, SelShared& S) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int parity = 0;
  uint32_t wv[PER];
  bool live[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    wv[i] = (uint32_t)(e[i] >> 32);
    live[i] = e[i] != 0;
  }
  uint32_t* wh = S.hist + wid * 256;
  for (int word = 0; word < 2; ++word) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0, n = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (live[i]) {
        lo = wv[i] < lo ? wv[i] : lo;
        hi = wv[i] > hi ? wv[i] : hi;
        ++n;
      }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    n = wave_sum_u32(n);
    if (lane == 0) { S.red[parity][wid][0] = lo; S.red[parity][wid][1] = hi; S.red[parity][wid][2] = n; }
    __syncthreads();
    lo = 0xFFFFFFFFu; hi = 0; n = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lo = S.red[parity][w][0] < lo ? S.red[parity][w][0] : lo;
      hi = S.red[parity][w][1] > hi ? S.red[parity][w][1] : hi;
      n += S.red[parity][w][2];
    }
    parity ^= 1;
    uint32_t bucket = n;
    bool done = need == bucket;
    uint32_t prefix = hi, mask = 0xFFFFFFFFu;
    if (!done && lo != hi) {
      const int common = __clz(lo ^ hi);
      mask = common ? (0xFFFFFFFFu << (32 - common)) : 0u;
      prefix = hi & mask;
      int top = 31 - common;  // highest unresolved bit
      while (top >= 0) {
        const int width = top >= 7 ? 8 : top + 1;
        const int sh = top + 1 - width;
        const uint32_t dm = (1u << width) - 1u;
#pragma unroll
        for (int j = 0; j < 4; ++j) wh[lane + 64 * j] = 0u;
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (live[i] && (wv[i] & mask) == prefix) atomicAdd(&wh[(wv[i] >> sh) & dm], 1u);
        __syncthreads();
        // digit d (thread 255 - d) total, suffix position from the top
        uint32_t v = 0;
        if (tid < 256) {
#pragma unroll
          for (int w = 0; w < NW; ++w) v += S.hist[w * 256 + 255 - tid];
        }
        const uint32_t inc = wave_incl_scan(v);
        if (wid < 4 && lane == 63) S.red[parity][wid][3] = inc;
        __syncthreads();
        if (tid < 256) {
          uint32_t before = 0;
          for (int w = 0; w < wid; ++w) before += S.red[parity][w][3];
          const uint32_t above = before + inc - v;
          if (above < need && above + v >= need) { S.res[0] = 255u - tid; S.res[1] = above; S.res[2] = v; }
        }
        __syncthreads();
        const uint32_t dig = S.res[0], above = S.res[1], cnt = S.res[2];
        parity ^= 1;
        need -= above;
        prefix |= dig << sh;
        mask |= dm << sh;
        bucket = cnt;
        top = sh - 1;
        if (need == bucket) { done = true; break; }
      }
    }
    if (done || word == 1) {
      // the need keys left in the bucket are selected: the threshold is the smallest
      uint64_t m = ~0ull;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (live[i] && (wv[i] & mask) == prefix && e[i] < m) m = e[i];
      return block_min64(m, S);
    }
    // scores tie at the threshold: continue on the token word of the tied keys
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      live[i] = live[i] && wv[i] == prefix;
      wv[i] = (uint32_t)e[i];
    }
  }
  return 0;  // not reached
}

__device__ __forceinline__ int32_t page_slot(const CacheView& cv, const RowMap& rm, int seq, int t) {
  return (int32_t)(token_block(cv, rm, seq, t) * cv.block_size + (t & (cv.block_size - 1)));
}

// Writes, in element order (token order), the tokens whose key is >= cstar, then
// -1 up to k. `slot` holds the page slots of the elements when `prow` is set.
__device__ void ordered_write(const uint64_t (&e)[PER], const int32_t (&slot)[PER], uint64_t cstar, int k,
                              int32_t* __restrict__ orow, int32_t* __restrict__ prow, SelShared& S) {
  uint32_t bits = 0, cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (e[i] != 0 && e[i] >= cstar) { bits |= 1u << i; ++cnt; }
  uint32_t total;
  uint32_t off = block_excl_scan<SEL_NT>(cnt, S.scan, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if ((bits >> i) & 1u) {
      if (off < (uint32_t)k) {
        orow[off] = (int32_t)(0xFFFFFFFFu - (uint32_t)e[i]);
        if (prow) prow[off] = slot[i];
      }
      ++off;
    }
  }
  for (int i = (int)total + threadIdx.x; i < k; i += SEL_NT) {
    orow[i] = -1;
    if (prow) prow[i] = -1;
  }
}

// Exact selection over the whole row straight from global memory (8-bit digits,
// per-wave LDS histograms), then a sort of the k tokens. Only reached when a
// resend set outgrows LDS (e.g. scores tied across far more than k tokens).
__device__ void select_row_global(const float* __restrict__ srow, int ctx, int k, SelShared& S,
                                  int32_t* __restrict__ orow, int32_t* __restrict__ prow, const CacheView& cv,
                                  const RowMap& rm, int seq) {
  const int tid = threadIdx.x, wid = tid >> 6;
  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)k;
  for (int sh = 56; sh >= 0; sh -= 8) {
    for (int i = tid; i < NW * 256; i += SEL_NT) S.hist[i] = 0u;
    __syncthreads();
    for (int t = tid; t < ctx; t += SEL_NT) {
      const uint64_t c = composite_key(srow[t], t);
      if ((c & mask) == prefix) atomicAdd(&S.hist[wid * 256 + ((c >> sh) & 0xFF)], 1u);
    }
    __syncthreads();
    uint32_t v = 0;
    if (tid < 256)
      for (int w = 0; w < NW; ++w) v += S.hist[w * 256 + tid];
    __syncthreads();
    if (tid < 256) S.hist[tid] = v;
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      for (int d = 255; d >= 0; --d) {
        const uint32_t x = S.hist[d];
        if (above + x >= need) { S.res[0] = (uint32_t)d; S.res[1] = above; break; }
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
  if (tid == 0) S.cnt[0] = 0;
  __syncthreads();
  for (int t = tid; t < ctx; t += SEL_NT)
    if (composite_key(srow[t], t) >= prefix) {
      const uint32_t pos = atomicAdd(&S.cnt[0], 1u);
      if (pos < (uint32_t)kMaxK) S.sel[pos] = (uint32_t)t;
    }
  __syncthreads();
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = k + tid; i < P; i += SEL_NT) S.sel[i] = 0xFFFFFFFFu;
  __syncthreads();
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += SEL_NT) {
        const int p = i ^ j;
        if (p > i) {
          const uint32_t a = S.sel[i], b = S.sel[p];
          if ((a > b) == ((i & kk) == 0)) { S.sel[i] = b; S.sel[p] = a; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += SEL_NT) {
    const int t = (int)S.sel[i];
    orow[i] = t;
    if (prow) prow[i] = page_slot(cv, rm, seq, t);
  }
}

}  // namespace

// Stage 1 over an existing score array (the standalone top-k entry point).
__global__ __launch_bounds__(256) void topk_send_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_ctx, int max_ctx,
                                                        TopkWs ws) {
  const int r = blockIdx.y;
  const int ctx = clamp_ctx(row_ctx, r, max_ctx);
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int base = unit * kCandUnit;
  if (base >= ctx || cand_per_unit(ctx) == 0) return;  // wave-uniform
  const int t = base + (threadIdx.x & 63);
  const bool valid = t < ctx;
  const float s = valid ? scores[(int64_t)r * ld + t] : 0.f;
  wave_send_candidates(s, valid, ctx, base, r, unit, ws);
}

__global__ __launch_bounds__(SEL_NT) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
                                                             const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                                             TopkWs ws, int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ phys, CacheView cv, RowMap rm) {
  __shared__ SelShared S;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int ctx = clamp_ctx(row_ctx, r, max_ctx);
  int32_t* orow = idx + (int64_t)r * k;
  int32_t* prow = phys ? phys + (int64_t)r * k : nullptr;
  const int seq = phys ? rm.row_seq[r] : 0;
  const float* srow = scores + (int64_t)r * ld;

  if (ctx <= k) {
    for (int i = tid; i < k; i += SEL_NT) {
      orow[i] = i < ctx ? i : -1;
      if (prow) prow[i] = i < ctx ? page_slot(cv, rm, seq, i) : -1;
    }
    return;
  }

  uint64_t e[PER];
  int32_t slot[PER];
  if (ctx <= kTopkFullRow) {
    // ---- the row's own keys: thread owns tokens [16 tid, 16 tid + 16) ----
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = tid * PER + i;
      e[i] = t < ctx ? composite_key(srow[t], t) : 0ull;
      slot[i] = (prow && t < ctx) ? page_slot(cv, rm, seq, t) : -1;
    }
    const uint64_t cstar = select_kth(e, (uint32_t)k, S);
    ordered_write(e, slot, cstar, k, orow, prow, S);
    return;
  }

  // ---- candidates: thread owns candidates [16 tid, 16 tid + 16), whole units ----
  const int nu = (ctx + kCandUnit - 1) / kCandUnit;
  const int m = cand_per_unit(ctx);
  const int n = nu * m;
  {
    const v4i* src = reinterpret_cast<const v4i*>(ws.cand + (int64_t)r * kCandRowCap + tid * PER);
    v4i raw[PER / 2];
#pragma unroll
    for (int q = 0; q < PER / 2; ++q) raw[q] = src[q];
#pragma unroll
    for (int q = 0; q < PER / 2; ++q) {
      e[2 * q] = ((uint64_t)(uint32_t)raw[q][1] << 32) | (uint32_t)raw[q][0];
      e[2 * q + 1] = ((uint64_t)(uint32_t)raw[q][3] << 32) | (uint32_t)raw[q][2];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (tid * PER + i >= n) e[i] = 0ull;
    // block-table lookups issued now, consumed after the search
#pragma unroll
    for (int i = 0; i < PER; ++i)
      slot[i] = (prow && e[i] != 0) ? page_slot(cv, rm, seq, (int)(0xFFFFFFFFu - (uint32_t)e[i])) : -1;
  }
  const uint64_t cu = select_kth(e, (uint32_t)k, S);

  // units (whole ones per thread) whose kept-back keys may reach cu
  const int upt = PER / m;                 // units per thread
  const int u0 = tid * upt;
  const uint64_t* rf = ws.floors + (int64_t)r * ws.nunits;
  uint32_t fmask = 0;
  for (int j = 0; j < upt; ++j)
    if (u0 + j < nu && rf[u0 + j] >= cu) fmask |= 1u << j;
  const uint32_t nflag = wave_sum_u32((uint32_t)__popc(fmask));
  if (tid % 64 == 0) S.red[0][tid >> 6][3] = nflag;
  __syncthreads();
  uint32_t nflag_all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) nflag_all += S.red[0][w][3];
  if (nflag_all == 0) {
    ordered_write(e, slot, cu, k, orow, prow, S);
    return;
  }

  // ---- resend: U in token order = per unit, (flagged ? its keys >= cu : its candidates >= cu) ----
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(srow) & 15u) == 0);
  auto unit_keys = [&](int u, auto&& fn) {
    // visits the keys of unit u's tokens in token order, 16 at a time
    const int tb = u * kCandUnit;
#pragma unroll 1
    for (int q = 0; q < kCandUnit / 16; ++q) {
      float f[16];
      const int t0 = tb + q * 16;
      if (vec_ok && t0 + 16 <= ctx) {
        const float4* p4 = reinterpret_cast<const float4*>(srow + t0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float4 v = p4[x];
          f[4 * x] = v.x; f[4 * x + 1] = v.y; f[4 * x + 2] = v.z; f[4 * x + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int x = 0; x < 16; ++x) f[x] = (t0 + x < ctx) ? srow[t0 + x] : 0.f;
      }
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (t0 + x < ctx) fn(composite_key(f[x], t0 + x));
    }
  };
  uint32_t cnt = 0;
  for (int j = 0; j < upt; ++j) {
    if ((fmask >> j) & 1u) {
      unit_keys(u0 + j, [&](uint64_t c) { cnt += c >= cu ? 1u : 0u; });
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i / m == j && e[i] != 0 && e[i] >= cu) ++cnt;
    }
  }
  uint32_t nuall;
  uint32_t off = block_excl_scan<SEL_NT>(cnt, S.scan, &nuall);
  if (nuall > (uint32_t)kCandRowCap) {
    select_row_global(srow, ctx, k, S, orow, prow, cv, rm, seq);
    return;
  }
  for (int j = 0; j < upt; ++j) {
    if ((fmask >> j) & 1u) {
      unit_keys(u0 + j, [&](uint64_t c) { if (c >= cu) S.buf[off++] = c; });
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i / m == j && e[i] != 0 && e[i] >= cu) S.buf[off++] = e[i];
    }
  }
  __syncthreads();
  uint64_t u[PER];
  int32_t uslot[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    u[i] = (uint32_t)(tid * PER + i) < nuall ? S.buf[tid * PER + i] : 0ull;
    uslot[i] = (prow && u[i] != 0) ? page_slot(cv, rm, seq, (int)(0xFFFFFFFFu - (uint32_t)u[i])) : -1;
  }
  const uint64_t cstar = select_kth(u, (uint32_t)k, S);
  ordered_write(u, uslot, cstar, k, orow, prow, S);
}

hipError_t launch_topk_send(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx,
                            const TopkWs& ws, hipStream_t stream) {
  if (R <= 0 || max_ctx <= kTopkFullRow) return hipSuccess;
  dim3 grid((cand_units(max_ctx) + 3) / 4, R);
  hipLaunchKernelGGL(topk_send_kernel, grid, dim3(256), 0, stream, scores, ld, row_ctx, max_ctx, ws);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                              int32_t* idx, const TopkWs& ws, int32_t* phys, float* pscale, const CacheView* cv,
                              const RowMap* rm, hipStream_t stream) {
  (void)pscale;
  if (R <= 0) return hipSuccess;
  CacheView c{};
  RowMap m{};
  if (phys) {
    c = *cv;
    m = *rm;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3(R), dim3(SEL_NT), 0, stream, scores, ld, row_ctx, max_ctx, k, ws, idx,
                     phys, c, m);
  return hipGetLastError();
}

}  // namespace dsa
