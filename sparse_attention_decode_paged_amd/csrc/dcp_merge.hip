// Exact top-k across token-strided shards, emulated on one GPU (vLLM "Day-0 support for
// Kimi K3.1 Pro", long-context section on decode context parallelism with the sparse
// indexer, and its sub-section on the exact top-k merge with ten times less traffic).
//
// Under decode context parallelism GPU s of W holds the tokens t = s (mod W) and can rank
// only those; before attention the shards must agree on the global top-k of every row.
// Each shard sends only its best M = ceil(1.5 k / W) candidates, one 32-bit word each:
// the score rounded to BF16, as an order-preserving 16-bit key, above a 16-bit slot that
// names the candidate in the sender's list. A radix select over the gathered words gives
// T, the key of the k-th best word. A shard whose list was full (it holds more tokens than
// it sent) and whose weakest sent key still reaches T may hold top-k tokens it did not
// send: it resends its whole local top-k. The exact top-k (fp32 scores, ties to the lower
// token) is then taken over the sent candidates whose key reaches T and the resent lists.
// Why nothing is lost: a top-k token x has key(x) >= T (otherwise k words would carry keys
// above key(x), i.e. k tokens with larger scores); if its shard did not send x, every word
// that shard sent beats x, so its weakest key reaches key(x) >= T and the shard resends.
//
// On one GPU the W shards are rows of a scratch array: a split kernel deals each row's
// scores out token-strided, the two-stage select ranks every shard row twice (best M, best
// k), and one workgroup per query row runs the exchange: words, threshold, resend decisions,
// union and the final selection (keys in HBM scratch, bins in LDS).
#include "common.h"
#include "internal.h"

namespace dsa {

namespace {
constexpr int kNT = 1024;  // merge workgroup
constexpr int kNW = kNT / 64;
constexpr uint32_t kNoWord = 0xFFFFFFFFu;  // no candidate at this slot (a real slot is < 0xFFFF)

// BF16 key: fp32 rounded to the nearest BF16 value (ties to even), then mapped so that a
// larger value has a larger key; -0 and +0 share a key.
__device__ __forceinline__ uint32_t bf16_order_key(float x) {
  const uint64_t u = __float_as_uint(x);
  const uint32_t b = (uint32_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16) & 0xFFFFu;
  if (b == 0x8000u) return 0x8000u;  // -0 rounds to the key of +0
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

struct MergeShared {
  uint32_t word[kDcpWordCap];  // word of shard i / M, slot i % M (kNoWord: none)
  int32_t tok[kDcpWordCap];    // its token
  int32_t sel[kMaxK];          // selected tokens, sorted in place
  uint32_t hist[256];
  uint32_t minkey[kDcpShardMax];
  uint32_t nsent[kDcpShardMax];
  uint32_t resend[kDcpShardMax];
  uint32_t scan[kNW + 1];
  uint32_t bin, above, count, nsel;
};

// Wave 0: the bin b of 256 (largest first) in which the need-th largest entry lies, and
// the number of entries in bins above b. Needs 1 <= need <= the histogram's total.
__device__ __forceinline__ void find_bin(MergeShared& S, uint32_t need) {
  const int lane = threadIdx.x & 63;
  const int top = 255 - 4 * lane;  // lane 0 owns the largest bins
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = S.hist[top - i];
  const uint32_t c = h[0] + h[1] + h[2] + h[3];
  const uint32_t inc = wave_incl_scan(c);
  const uint64_t hit = __ballot(inc >= need);
  if (lane == (int)__builtin_ctzll(hit)) {
    uint32_t above = inc - c;
    int b = top - 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (above + h[i] >= need) {
        b = top - i;
        break;
      }
      above += h[i];
    }
    S.bin = (uint32_t)b;
    S.above = above;
  }
}

// Appends v at the next free place of list[] for every lane with `take` (one LDS atomic
// per wave); places at or past cap are dropped. All lanes of the wave must call it.
template <typename T>
__device__ __forceinline__ void wave_append(bool take, T v, T* list, uint32_t* counter, uint32_t cap) {
  const uint64_t bal = __ballot(take);
  if (bal == 0) return;
  uint32_t base = 0;
  if ((threadIdx.x & 63) == 0) base = atomicAdd(counter, (uint32_t)__popcll(bal));
  base = __shfl(base, 0, 64);
  const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
  if (take && pos < cap) list[pos] = v;
}
}  // namespace

// Deals row r's scores out to its W shard rows: token t goes to row r W + t mod W, place
// t / W. Also writes every shard row's length.
__global__ __launch_bounds__(256) void dcp_split_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_ctx, int max_ctx, int W,
                                                        float* __restrict__ shard, int64_t ls,
                                                        int32_t* __restrict__ shard_ctx) {
  const int r = blockIdx.y;
  int ctx = row_ctx[r];
  ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
  if (blockIdx.x == 0 && (int)threadIdx.x < W) {
    const int s = threadIdx.x;
    shard_ctx[r * W + s] = ctx > s ? (ctx - s + W - 1) / W : 0;
  }
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < ctx) shard[((int64_t)r * W + t % W) * ls + t / W] = scores[(int64_t)r * ld + t];
}

// One workgroup per query row. idx_m: [R W][M] best-M lists of the shard rows, idx_k:
// [R W][k] best-k lists (shard-local places, ascending, -1 padded); ukeys: [R][ucap]
// scratch for the received candidates.
__global__ __launch_bounds__(kNT) void dcp_merge_kernel(const float* __restrict__ scores, int64_t ld, int W, int M,
                                                        int k, const int32_t* __restrict__ shard_ctx,
                                                        const int32_t* __restrict__ idx_m,
                                                        const int32_t* __restrict__ idx_k, uint64_t* __restrict__ ukeys,
                                                        int64_t ucap, int32_t* __restrict__ idx,
                                                        uint32_t* __restrict__ resend_mask,
                                                        uint32_t* __restrict__ words_out) {
  __shared__ MergeShared S;
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* srow = scores + (int64_t)r * ld;
  const int nw = W * M;
  if (tid < kDcpShardMax) {
    S.minkey[tid] = kNoWord;
    S.nsent[tid] = 0;
  }
  if (tid < 256) S.hist[tid] = 0;
  if (tid == 0) S.count = 0;
  __syncthreads();

  // 1. the words each shard sends
  uint32_t mine = 0;
  for (int i = tid; i < nw; i += kNT) {
    const int s = i / M, j = i - s * M;
    const int loc = idx_m[((int64_t)r * W + s) * M + j];
    uint32_t word = kNoWord;
    int t = -1;
    if (loc >= 0) {
      t = s + W * loc;
      const uint32_t key = bf16_order_key(srow[t]);
      word = (key << 16) | (uint32_t)j;
      atomicMin(&S.minkey[s], key);
      atomicAdd(&S.nsent[s], 1u);
      ++mine;
    }
    S.word[i] = word;
    S.tok[i] = t;
    if (words_out) words_out[(int64_t)r * nw + i] = word;
  }
  uint32_t nwords;
  block_excl_scan<kNT>(mine, S.scan, &nwords);  // also orders the LDS writes above

  // 2. T: the key of the k-th largest word (0 when fewer than k words were sent)
  uint32_t T = 0;
  if (nwords >= (uint32_t)k) {
    for (int i = tid; i < nw; i += kNT)
      if (S.word[i] != kNoWord) atomicAdd(&S.hist[S.word[i] >> 24], 1u);
    __syncthreads();
    if (tid < 64) find_bin(S, (uint32_t)k);
    __syncthreads();
    const uint32_t hi = S.bin, need = (uint32_t)k - S.above;
    if (tid < 256) S.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nw; i += kNT)
      if (S.word[i] != kNoWord && (S.word[i] >> 24) == hi) atomicAdd(&S.hist[(S.word[i] >> 16) & 255u], 1u);
    __syncthreads();
    if (tid < 64) find_bin(S, need);
    __syncthreads();
    T = (hi << 8) | S.bin;
  }

  // 3. resend decisions: a full list whose weakest key reaches T
  if (tid < W) {
    const uint32_t n = S.nsent[tid];
    S.resend[tid] = ((uint32_t)shard_ctx[r * W + tid] > n && n > 0 && S.minkey[tid] >= T) ? 1u : 0u;
  }
  __syncthreads();
  if (tid == 0 && resend_mask) {
    uint32_t m = 0;
    for (int s = 0; s < W; ++s) m |= S.resend[s] << s;
    resend_mask[r] = m;
  }

  // 4. what the shards receive: sent words with key >= T from shards that do not resend,
  // and the full local top-k of those that do (distinct tokens: shards are disjoint)
  uint64_t* u = ukeys + (int64_t)r * ucap;
  for (int i0 = 0; i0 < nw; i0 += kNT) {
    const int i = i0 + tid;
    bool take = false;
    int t = 0;
    if (i < nw && S.word[i] != kNoWord) {
      take = S.resend[i / M] == 0u && (S.word[i] >> 16) >= T;
      t = S.tok[i];
    }
    wave_append<uint64_t>(take, take ? composite_key(srow[t], t) : 0ull, u, &S.count, (uint32_t)ucap);
  }
  const int nk = W * k;
  for (int i0 = 0; i0 < nk; i0 += kNT) {
    const int i = i0 + tid;
    bool take = false;
    int t = 0;
    if (i < nk) {
      const int s = i / k;
      if (S.resend[s]) {
        const int loc = idx_k[((int64_t)r * W + s) * k + (i - s * k)];
        take = loc >= 0;
        t = s + W * loc;
      }
    }
    wave_append<uint64_t>(take, take ? composite_key(srow[t], t) : 0ull, u, &S.count, (uint32_t)ucap);
  }
  __syncthreads();
  const uint32_t U = S.count < (uint32_t)ucap ? S.count : (uint32_t)ucap;

  // 5. exact top-k of the received keys: MSB-first radix select, 8 bits a pass, until every
  // key left under the prefix is selected; then keys >= thr are exactly the top-k
  uint64_t thr = 0;
  if (U > (uint32_t)k) {
    uint32_t need = (uint32_t)k;
    uint64_t prefix = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (tid < 256) S.hist[tid] = 0;
      __syncthreads();
      const uint64_t hmask = shift == 56 ? 0ull : (~0ull << (shift + 8));
      for (uint32_t i = tid; i < U; i += kNT) {
        const uint64_t key = u[i];
        if ((key & hmask) == prefix) atomicAdd(&S.hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) find_bin(S, need);
      __syncthreads();
      need -= S.above;
      prefix |= (uint64_t)S.bin << shift;
      const bool done = S.hist[S.bin] == need;
      __syncthreads();  // hist and bin are rewritten by the next pass
      if (done) break;
    }
    thr = prefix;
  }

  // 6. selected tokens in ascending order, -1 padding
  if (tid == 0) S.nsel = 0;
  for (int j = tid; j < kMaxK; j += kNT) S.sel[j] = 0x7FFFFFFF;
  __syncthreads();
  for (uint32_t i0 = 0; i0 < U; i0 += kNT) {
    const uint32_t i = i0 + tid;
    const uint64_t key = i < U ? u[i] : 0ull;
    const bool take = i < U && key >= thr;
    wave_append<int32_t>(take, (int32_t)(0xFFFFFFFFu - (uint32_t)key), S.sel, &S.nsel, (uint32_t)kMaxK);
  }
  __syncthreads();
  const uint32_t nsel = S.nsel < (uint32_t)k ? S.nsel : (uint32_t)k;
  // Bitonic sort, one pair per thread. A stage of stride <= 64 keeps every element inside
  // the 128-element block of one wave (wave w: [128 w, 128 w + 128)), and one wave's LDS
  // operations execute in order, so two consecutive such stages need no workgroup
  // barrier; a stage of stride >= 128 crosses waves and is fenced on both sides.
  static_assert(kNT * 2 == kMaxK, "one pair per thread");
  for (int size = 2; size <= kMaxK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int lo = 2 * stride * (tid / stride) + (tid % stride), hi = lo + stride;
      const bool asc = (lo & size) == 0;
      const int32_t a = S.sel[lo], b = S.sel[hi];
      if ((a > b) == asc) {
        S.sel[lo] = b;
        S.sel[hi] = a;
      }
      const int next = stride > 1 ? stride >> 1 : size;  // the next stage's stride
      if (stride >= 128 || next >= 128 || (stride == 1 && size == kMaxK)) {
        __syncthreads();
      } else {
        // wave-scope release / acquire around the wave barrier: the exchange goes
        // through LDS between lanes of one wave, so the stores must be ordered
        // before the partner lanes' loads (free at this scope)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }
  for (int j = tid; j < k; j += kNT) idx[(int64_t)r * k + j] = j < (int)nsel ? S.sel[j] : -1;
}

hipError_t launch_topk_dcp(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k, int W,
                           int32_t* idx, uint32_t* resend_mask, uint32_t* words, void* ws, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const DcpWs d = dcp_ws_carve(ws, R, max_ctx, k, W);
  const int M = dcp_send_count(k, W);
  const int lmax = dcp_shard_len(max_ctx, W);
  dim3 g1((max_ctx + 255) / 256 > 0 ? (max_ctx + 255) / 256 : 1, R);
  hipLaunchKernelGGL(dcp_split_kernel, g1, dim3(256), 0, stream, scores, ld, row_ctx, max_ctx, W, d.shard, d.ls,
                     d.shard_ctx);
  hipError_t e = hipGetLastError();
  const int RW = R * W;
  if (e == hipSuccess) e = launch_topk_send(d.shard, d.ls, d.shard_ctx, RW, lmax, d.tw, stream);
  if (e == hipSuccess)
    e = launch_topk_select(d.shard, d.ls, d.shard_ctx, RW, lmax, M, 512, d.idx_m, d.tw, nullptr, nullptr, nullptr,
                           stream);
  if (e == hipSuccess)
    e = launch_topk_select(d.shard, d.ls, d.shard_ctx, RW, lmax, k, 512, d.idx_k, d.tw, nullptr, nullptr, nullptr,
                           stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dcp_merge_kernel, dim3(R), dim3(kNT), 0, stream, scores, ld, W, M, k, d.shard_ctx, d.idx_m,
                     d.idx_k, d.ukeys, d.ucap, idx, resend_mask, words);
  return hipGetLastError();
}

}  // namespace dsa
