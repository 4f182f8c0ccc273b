// Exact per-row top-k over fp32 scores (ties -> lower token index).
//
// vLLM "Day-0 support for Kimi K3.1 Pro": the fused decode path ends the indexer
// with an exact top-k selection that emits the rows attention reads, and the
// zero-mismatch RL section wants top-k to be batch invariant. Here each row's
// selection is a pure function of that row's scores.
//
// Every (score, token) pair maps to a 64-bit composite key
//   (order-preserving bits of the score) << 32 | (0xFFFFFFFF - token)
// so "larger score, then lower index" is plain integer order and all composites
// are distinct. The k selected tokens are exactly those whose composite is >= c*,
// the k-th largest composite. Three passes over the row, each split over
// workgroups of 4096 tokens:
//   1. histogram of the top 12 key bits; the last workgroup of the row finds the
//      bin b1 holding the k-th element and how many of that bin are still needed;
//   2. tokens of bin b1 are appended to a candidate list and tokens above it are
//      counted per chunk; the last workgroup resolves c* with 8-bit radix digits
//      over the remaining 52 composite bits (reading the candidate list, or the
//      scores again if the list overflowed) and turns per-chunk counts into
//      output offsets;
//   3. each workgroup writes its chunk's selected tokens in ascending order.
#include "common.h"
#include "internal.h"

namespace dsa {

namespace {

constexpr int NT = 256;
constexpr int PER_T = kTopkChunk / NT;  // 16 tokens per thread per pass

__device__ __forceinline__ int clamp_ctx(const int32_t* row_ctx, int r, int max_ctx) {
  int c = row_ctx[r];
  c = c < 0 ? 0 : c;
  return c > max_ctx ? max_ctx : c;
}

__device__ __forceinline__ uint32_t ld_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in every thread of the workgroup that arrives last for this row.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (prev == expected - 1) ? 1 : 0;
  }
  __syncthreads();
  bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

}  // namespace

__global__ __launch_bounds__(NT) void topk_clear_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < words; i += (size_t)gridDim.x * NT) p[i] = 0u;
}

__global__ __launch_bounds__(NT) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                                       TopkWs ws) {
  const int r = blockIdx.y, ch = blockIdx.x;
  const int ctx = clamp_ctx(row_ctx, r, max_ctx);
  if (ctx <= k) return;
  const int nchr = (ctx + kTopkChunk - 1) / kTopkChunk;
  if (ch >= nchr) return;

  __shared__ uint32_t lh[kTopkBins];
  __shared__ uint32_t tmp[NT / 64 + 1];
  __shared__ int flag;
  for (int b = threadIdx.x; b < kTopkBins; b += NT) lh[b] = 0u;
  __syncthreads();
  const float* srow = scores + (int64_t)r * ld;
#pragma unroll 4
  for (int i = 0; i < PER_T; ++i) {
    int t = ch * kTopkChunk + i * NT + threadIdx.x;
    if (t < ctx) atomicAdd(&lh[float_key(srow[t]) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* gh = ws.hist + (int64_t)r * kTopkBins;
  for (int b = threadIdx.x; b < kTopkBins; b += NT) {
    uint32_t c = lh[b];
    if (c) atomicAdd(&gh[b], c);
  }
  uint32_t* ctrl = ws.ctrl + (int64_t)r * kTopkCtrl;
  if (!arrive_last(&ctrl[CT_DONE1], (uint32_t)nchr, &flag)) return;

  // Thread i owns bins [16*(255-i), 16*(255-i)+16): exclusive scan = count above its segment.
  const int seg = NT - 1 - threadIdx.x;
  uint32_t c[16];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    c[j] = ld_acquire(&gh[seg * 16 + j]);
    sum += c[j];
  }
  uint32_t total;
  uint32_t above = block_excl_scan<NT>(sum, tmp, &total);
  if (above < (uint32_t)k && above + sum >= (uint32_t)k) {
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      if (above + c[j] >= (uint32_t)k) {
        ctrl[CT_B1] = (uint32_t)(seg * 16 + j);
        ctrl[CT_NEED1] = (uint32_t)k - above;
        ctrl[CT_NEQ] = c[j];
        break;
      }
      above += c[j];
    }
  }
}

// Resolve c*: the need-th largest composite among elements whose top 12 key bits
// equal b1. Elements are read from the candidate list when it holds them all,
// otherwise by rescanning the row's scores.
__device__ uint64_t refine_threshold(const float* __restrict__ srow, int ctx, const uint32_t* __restrict__ cand,
                                     bool use_cand, uint32_t n_src, uint32_t b1, uint32_t need,
                                     uint32_t* dh /*256*/, uint32_t* tmp, uint64_t* s_min, uint32_t* s_res) {
  uint64_t prefix = (uint64_t)b1 << 52;
  uint64_t mask = 0xFFFull << 52;
  const int shifts[7] = {44, 36, 28, 20, 12, 4, 0};
  const int widths[7] = {8, 8, 8, 8, 8, 8, 4};
  for (int p = 0; p < 7; ++p) {
    const int sh = shifts[p];
    const uint64_t dm = (1ull << widths[p]) - 1;
    dh[threadIdx.x] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n_src; i += NT) {
      int t = use_cand ? (int)cand[i] : (int)i;
      if (t >= ctx) continue;
      uint64_t cc = composite_key(srow[t], t);
      if ((cc & mask) == prefix) atomicAdd(&dh[(cc >> sh) & dm], 1u);
    }
    __syncthreads();
    const int d = NT - 1 - threadIdx.x;
    uint32_t v = dh[d];
    uint32_t tot;
    uint32_t above = block_excl_scan<NT>(v, tmp, &tot);
    if (above < need && above + v >= need) {
      s_res[0] = (uint32_t)d;
      s_res[1] = above;
      s_res[2] = v;
    }
    __syncthreads();
    const uint32_t dig = s_res[0], ab = s_res[1], cnt = s_res[2];
    __syncthreads();
    need -= ab;
    prefix |= (uint64_t)dig << sh;
    mask |= dm << sh;
    if (need == cnt) {
      // every remaining match is selected: c* is the smallest of them
      if (threadIdx.x == 0) *s_min = ~0ull;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < n_src; i += NT) {
        int t = use_cand ? (int)cand[i] : (int)i;
        if (t >= ctx) continue;
        uint64_t cc = composite_key(srow[t], t);
        if ((cc & mask) == prefix) atomicMin(reinterpret_cast<unsigned long long*>(s_min), (unsigned long long)cc);
      }
      __syncthreads();
      uint64_t m = *s_min;
      __syncthreads();
      return m;
    }
  }
  return prefix;
}

__global__ __launch_bounds__(NT) void topk_cand_kernel(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                                       TopkWs ws) {
  const int r = blockIdx.y, ch = blockIdx.x;
  const int ctx = clamp_ctx(row_ctx, r, max_ctx);
  if (ctx <= k) return;
  const int nchr = (ctx + kTopkChunk - 1) / kTopkChunk;
  if (ch >= nchr) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;

  __shared__ uint32_t tmp[NT / 64 + 1];
  __shared__ uint32_t dh[256];
  __shared__ uint64_t s_min;
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t cnt[kMaxCtx / kTopkChunk];
  __shared__ int flag;

  uint32_t* ctrl = ws.ctrl + (int64_t)r * kTopkCtrl;
  const uint32_t b1 = ctrl[CT_B1];
  const float* srow = scores + (int64_t)r * ld;
  uint32_t* cand = ws.cand + (int64_t)r * kCandCap;
  uint32_t gt = 0;
#pragma unroll 4
  for (int i = 0; i < PER_T; ++i) {
    int t = ch * kTopkChunk + i * NT + threadIdx.x;
    bool eq = false;
    if (t < ctx) {
      uint32_t bin = float_key(srow[t]) >> 20;
      gt += bin > b1 ? 1u : 0u;
      eq = bin == b1;
    }
    uint64_t m = __ballot(eq);
    if (m) {
      int leader = __ffsll((unsigned long long)m) - 1;
      uint32_t basep = 0;
      if (lane == leader) basep = atomicAdd(&ctrl[CT_NCAND], (uint32_t)__popcll(m));
      basep = __shfl(basep, leader, 64);
      uint32_t pos = basep + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      if (eq && pos < (uint32_t)kCandCap) cand[pos] = (uint32_t)t;
    }
  }
  gt = wave_sum(gt);
  if (lane == 0) tmp[wid] = gt;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int i = 0; i < NT / 64; ++i) s += tmp[i];
    ws.gtc[(int64_t)r * ws.nch + ch] = s;
  }
  if (!arrive_last(&ctrl[CT_DONE2], (uint32_t)nchr, &flag)) return;

  const uint32_t n_eq = ctrl[CT_NEQ];
  const uint32_t need1 = ctrl[CT_NEED1];
  const bool use_cand = n_eq <= (uint32_t)kCandCap;
  const uint32_t n_src = use_cand ? n_eq : (uint32_t)ctx;
  const uint64_t cstar = refine_threshold(srow, ctx, cand, use_cand, n_src, b1, need1, dh, tmp, &s_min, s_res);

  // Per-chunk selected counts -> exclusive offsets.
  for (int c = threadIdx.x; c < nchr; c += NT) cnt[c] = ws.gtc[(int64_t)r * ws.nch + c];
  __syncthreads();
  const uint64_t bin_mask = 0xFFFull << 52, bin_val = (uint64_t)b1 << 52;
  for (uint32_t i = threadIdx.x; i < n_src; i += NT) {
    int t = use_cand ? (int)cand[i] : (int)i;
    if (t >= ctx) continue;
    uint64_t cc = composite_key(srow[t], t);
    if ((cc & bin_mask) == bin_val && cc >= cstar) atomicAdd(&cnt[t / kTopkChunk], 1u);
  }
  __syncthreads();
  constexpr int PER = (kMaxCtx / kTopkChunk + NT - 1) / NT;
  uint32_t loc[PER];
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int c = threadIdx.x * PER + j;
    loc[j] = c < nchr ? cnt[c] : 0u;
    s += loc[j];
  }
  uint32_t tot;
  uint32_t off = block_excl_scan<NT>(s, tmp, &tot);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int c = threadIdx.x * PER + j;
    if (c < nchr) ws.base[(int64_t)r * ws.nch + c] = off;
    off += loc[j];
  }
  if (threadIdx.x == 0) {
    ctrl[CT_CSTAR_HI] = (uint32_t)(cstar >> 32);
    ctrl[CT_CSTAR_LO] = (uint32_t)cstar;
  }
}

__global__ __launch_bounds__(NT) void topk_write_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                                        TopkWs ws, int32_t* __restrict__ idx) {
  const int r = blockIdx.y, ch = blockIdx.x;
  const int ctx = clamp_ctx(row_ctx, r, max_ctx);
  const int total = ctx < k ? ctx : k;
  int32_t* orow = idx + (int64_t)r * k;
  if (ch == 0)
    for (int j = total + threadIdx.x; j < k; j += NT) orow[j] = -1;
  const int nchr = (ctx + kTopkChunk - 1) / kTopkChunk;
  if (ch >= nchr) return;
  const bool all = ctx <= k;
  const uint32_t* ctrl = ws.ctrl + (int64_t)r * kTopkCtrl;
  const uint64_t cstar = all ? 0ull : (((uint64_t)ctrl[CT_CSTAR_HI] << 32) | ctrl[CT_CSTAR_LO]);
  const uint32_t basech = all ? (uint32_t)(ch * kTopkChunk) : ws.base[(int64_t)r * ws.nch + ch];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const float* srow = scores + (int64_t)r * ld;

  __shared__ uint32_t wc[PER_T][NT / 64];
  uint64_t masks[PER_T];
#pragma unroll
  for (int i = 0; i < PER_T; ++i) {
    int t = ch * kTopkChunk + i * NT + threadIdx.x;
    bool sel = false;
    if (t < ctx) sel = all || composite_key(srow[t], t) >= cstar;
    masks[i] = __ballot(sel);
    if (lane == 0) wc[i][wid] = (uint32_t)__popcll(masks[i]);
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t run = basech;
#pragma unroll
  for (int i = 0; i < PER_T; ++i) {
    uint32_t off = run, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      uint32_t x = wc[i][w];
      off += w < wid ? x : 0u;
      tot += x;
    }
    if ((masks[i] >> lane) & 1ull) {
      uint32_t pos = off + (uint32_t)__popcll(masks[i] & lt);
      if (pos < (uint32_t)k) orow[pos] = ch * kTopkChunk + i * NT + threadIdx.x;
    }
    run += tot;
  }
}

hipError_t launch_clear(uint32_t* p, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + NT - 1) / NT;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(topk_clear_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, p, words);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                       int32_t* idx, const TopkWs& ws, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  dim3 grid(ws.nch, R);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(NT), 0, stream, scores, ld, row_ctx, max_ctx, k, ws);
  hipLaunchKernelGGL(topk_cand_kernel, grid, dim3(NT), 0, stream, scores, ld, row_ctx, max_ctx, k, ws);
  hipLaunchKernelGGL(topk_write_kernel, grid, dim3(NT), 0, stream, scores, ld, row_ctx, max_ctx, k, ws, idx);
  return hipGetLastError();
}

}  // namespace dsa
