// Lightning-indexer scoring for several query rows of one sequence (FP8 keys).
//
// Prefill-append (vLLM "Day-0 support for Kimi K3.1 Pro": a 2K-token append on a
// 150K prefix, every appended token a query row that sees the cache up to itself) and
// speculative verification (the AMD section: several verify tokens per sequence whose
// queries share one key scan) put many rows on the same keys. The per-row kernel would
// read and convert every key once per row; here a workgroup covers 256 tokens of up
// to G consecutive rows, loads and converts each key tile once, and runs it against
// every row's query (per row: 8 bf16 MFMAs per 32-token tile, the ReLU-weighted head
// sum and the key scale, exactly as the per-row kernel computes it).
//
// Rows of a workgroup are expected to share the sequence. A row whose block-table row
// differs from the previous row's reloads the keys, so any grouping gives the same
// result; grouping only decides how often keys are read.
#include "common.h"
#include "internal.h"
#include "topk_send.h"

namespace dsa {

namespace {
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kDIdx;  // 4 KB

// 16-byte chunk c of tile token tn sits at LDS byte tn*128 + 16*(c ^ (tn & 7)).
__device__ __forceinline__ int swz(int tn, int c) { return tn * kDIdx + 16 * (c ^ (tn & 7)); }
}  // namespace

// One workgroup = 4 waves = 256 consecutive tokens of rows [blockIdx.y * G, + G); wave w
// owns tokens [64w, 64w + 64) as two 32-token tiles. PAGED32: block size >= 32.
// SEND: also run stage 1 of the top-k for every row.
template <bool PAGED32, bool SEND>
__global__ __launch_bounds__(256, 3) void indexer_fp8_rows_kernel(CacheView cv, RowMap rm, const uint8_t* __restrict__ q_idx,
                                                               const float* __restrict__ q_scale,
                                                               const float* __restrict__ w, float* __restrict__ scores,
                                                               int64_t ld, TopkWs tw, int R, int G) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][kTileBytes];
  __shared__ uint32_t send_lds[2][send_lds_words<256>()];  // double-buffered over the rows that take the 256-token send
  __shared__ float wf_s[kRowsPerGroupMax * kHIdx];  // folded head weights w * q_scale of the group's rows
  // the current and the next row's query codes as bf16: 16-byte chunk c (dims 8c .. 8c + 7)
  // of head h at byte 256 h + 16 (c ^ (h & 15)), so the operand reads are conflict free
  __shared__ __attribute__((aligned(16))) uint8_t qs_l[2][kHIdx * kDIdx * 2];
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = blockIdx.y * G;
  const int r1 = r0 + G < R ? r0 + G : R;
  // the group's rows, lane i holding row r0 + i's length and sequence (G <= 16); the
  // longest row decides which tiles exist
  int rl_v = 0, rs_v = -1;
  if (lane < r1 - r0) {
    rl_v = row_len(rm, r0 + lane, cv.status);
    rs_v = rm.row_seq[r0 + lane];
  }
  int gmax = 0;
  for (int r = r0; r < r1; ++r) {
    const int c = __builtin_amdgcn_readlane(rl_v, r - r0);
    gmax = c > gmax ? c : gmax;
  }
  if (blockIdx.x * 256 >= gmax) return;  // whole workgroup
  const int tok0 = blockIdx.x * 256 + wid * 64;
  const int bs_mask = cv.block_size - 1;
  const int wpos = swz(lane >> 3, lane & 7);

  v8bf kb[2][8];  // B operands of both tiles (keys of the current sequence, as bf16)
  float ksc = 0.f;  // key scale of token tok0 + lane
  // Keys of sequence `seq` for the run of rows that starts at row r and shares it: tile
  // starts are clamped into the run's longest row (smax >= 1), so no block-table entry
  // past that sequence's own tokens is read.
  auto load_keys = [&](int seq, int smax) {
    const int last_tile = (smax - 1) & ~(kTileTok - 1);
    const int tb1 = tok0 + kTileTok < last_tile ? tok0 + kTileTok : last_tile;
    const int tb0 = tok0 < last_tile ? tok0 : last_tile;
    v4i kv[2][4];
    int64_t toff[2];
    if (PAGED32) {
      const int32_t* btrow = rm.block_table + (int64_t)seq * rm.bt_stride;
      const uint32_t e0 = (uint32_t)btrow[tb0 >> cv.log2_bs], e1 = (uint32_t)btrow[tb1 >> cv.log2_bs];
      const uint32_t nb = (uint32_t)cv.num_blocks;
      const uint32_t b0 = e0 < nb ? e0 : ((int32_t)e0 < 0 ? 0u : nb - 1u);
      const uint32_t b1 = e1 < nb ? e1 : ((int32_t)e1 < 0 ? 0u : nb - 1u);
      if (e0 >= nb || e1 >= nb) raise_status(cv.status, kStBlockClamped);
      toff[0] = (int64_t)b0 * cv.row_bytes + cv.idx_off;
      toff[1] = (int64_t)b1 * cv.row_bytes + cv.idx_off;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tb = j ? tb1 : tb0;
      if (PAGED32) {
        const uint8_t* tile = cv.pool + toff[j] + (int64_t)(tb & bs_mask) * kDIdx;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          kv[j][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(tile + 1024 * i + 16 * lane));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int t = tb + 8 * i + (lane >> 3);
          t = t < smax ? t : smax - 1;
          const uint8_t* key = row_base(cv, token_block(cv, rm, seq, t)) + cv.idx_off + (int64_t)(t & bs_mask) * kDIdx;
          kv[j][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(key + 16 * (lane & 7)));
        }
      }
    }
    {
      int t = tok0 + lane;
      t = t < smax ? t : smax - 1;
      const int64_t off = PAGED32 ? ((t & ~(kTileTok - 1)) == tb1 ? toff[1] : toff[0])
                                  : token_block(cv, rm, seq, t) * cv.row_bytes + cv.idx_off;
      ksc = *reinterpret_cast<const float*>(cv.pool + off + (int64_t)cv.block_size * kDIdx + (int64_t)(t & bs_mask) * 4);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(&lds[wid][1024 * i + wpos]) = kv[j][i];
      v4i kr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = *reinterpret_cast<const v4i*>(&lds[wid][swz(n, 4 * g + i)]);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        kb[j][kk] = e4m3x8_to_bf16((uint32_t)kr[kk >> 1][(kk & 1) * 2], (uint32_t)kr[kk >> 1][(kk & 1) * 2 + 1]);
    }
  };

  // The group's folded head weights go to LDS once. Each row's query is converted to
  // bf16 once per workgroup (each thread converts 16 of its 4,096 codes) into one of two
  // LDS buffers; the next row's codes are loaded while the current row runs.
  for (int i = threadIdx.x; i < (r1 - r0) * kHIdx; i += 256)
    wf_s[i] = w[(int64_t)r0 * kHIdx + i] * q_scale[(int64_t)r0 * kHIdx + i];
  auto q_load = [&](int rr) -> v4i {
    return *reinterpret_cast<const v4i*>(q_idx + (int64_t)rr * kHIdx * kDIdx + 16 * threadIdx.x);
  };
  auto q_store = [&](v4i v, int buf) {
    const int h = threadIdx.x >> 3, c = 2 * (threadIdx.x & 7);
    *reinterpret_cast<v8bf*>(&qs_l[buf][h * 256 + 16 * (c ^ (h & 15))]) =
        e4m3x8_to_bf16((uint32_t)v[0], (uint32_t)v[1]);
    *reinterpret_cast<v8bf*>(&qs_l[buf][h * 256 + 16 * ((c + 1) ^ (h & 15))]) =
        e4m3x8_to_bf16((uint32_t)v[2], (uint32_t)v[3]);
  };
  q_store(q_load(r0), 0);
  __syncthreads();

  int seq_cur = -1;
  // Send buffers alternate between rows that take the 256-token send (the only form
  // that uses LDS, and it ends its writes with a workgroup barrier): counting those rows
  // rather than all rows keeps a wave from reusing a buffer that a slower wave may
  // still read, also when shorter rows without that barrier sit in between.
  int nsend256 = 0;
  for (int r = r0; r < r1; ++r) {
    v4i qnext = {};
    if (r + 1 < r1) qnext = q_load(r + 1);  // uniform
    const int qb = (r - r0) & 1;
    const int seq = __builtin_amdgcn_readlane(rs_v, r - r0);
    const int ctx = __builtin_amdgcn_readlane(rl_v, r - r0);
    if (seq != seq_cur) {  // uniform
      int smax = ctx;  // longest row of the run of rows on this sequence
      for (int q = r + 1; q < r1 && __builtin_amdgcn_readlane(rs_v, q - r0) == seq; ++q) {
        const int c = __builtin_amdgcn_readlane(rl_v, q - r0);
        smax = c > smax ? c : smax;
      }
      if (smax > 0) load_keys(seq, smax);  // an empty run stores and sends nothing
      seq_cur = seq;
    }
    // A operands: head n, dims 64 g + 8 kk .. + 8 (chunk 8 g + kk)
    v8bf qa[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qa[kk] = *reinterpret_cast<const v8bf*>(&qs_l[qb][n * 256 + 16 * ((8 * g + kk) ^ (n & 15))]);
    // accumulator element rr of lane (n, g) is head 8 (rr >> 2) + 4 g + (rr & 3)
    float wq[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(&wf_s[(r - r0) * kHIdx + 8 * j + 4 * g]);
      wq[4 * j] = v.x;
      wq[4 * j + 1] = v.y;
      wq[4 * j + 2] = v.z;
      wq[4 * j + 3] = v.w;
    }
    float res[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v16f acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], kb[j][kk], acc, 0, 0, 0);
      float s = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s = fmaf(wq[rr], relu_bits(acc[rr]), s);
      s += xshflf<32>(s);
      res[j] = s;
    }
    // lane l owns token tok0 + l: tile 0 on lanes 0..31, tile 1 on lanes 32..63
    const int t = tok0 + lane;
    const float sc = (g ? res[1] : res[0]) * ksc;
    if (t < ctx) scores[(int64_t)r * ld + t] = sc;
    // the workgroup's span must reach into the row, or its unit would lie past the row
    if (SEND && blockIdx.x * 256 < ctx) {  // uniform
      send_candidates<256>(sc, t < ctx, ctx, blockIdx.x * 256, r, tw, send_lds[nsend256 & 1]);
      nsend256 += cand_plan(ctx, 256).unit == 256 ? 1 : 0;
    }
    // the other buffer was last read in the previous row, which every wave has left
    if (r + 1 < r1) q_store(qnext, qb ^ 1);  // uniform
    __syncthreads();
  }
}

hipError_t launch_indexer_fp8_rows(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const float* q_scale,
                                   const float* w, int R, int G, float* scores, int64_t ld, const TopkWs* ws,
                                   hipStream_t stream) {
  int nx = (rm.max_ctx + 255) / 256;
  if (nx < 1) nx = 1;
  TopkWs tw = ws ? *ws : TopkWs{nullptr, nullptr, nullptr};
  const int send = (ws != nullptr && rm.max_ctx > kTopkFullRow) ? 1 : 0;
  dim3 grid(nx, (R + G - 1) / G);
  const bool p32 = cv.block_size >= kTileTok;
  if (send && p32)
    hipLaunchKernelGGL((indexer_fp8_rows_kernel<true, true>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_scale, w,
                       scores, ld, tw, R, G);
  else if (send)
    hipLaunchKernelGGL((indexer_fp8_rows_kernel<false, true>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_scale, w,
                       scores, ld, tw, R, G);
  else if (p32)
    hipLaunchKernelGGL((indexer_fp8_rows_kernel<true, false>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_scale, w,
                       scores, ld, tw, R, G);
  else
    hipLaunchKernelGGL((indexer_fp8_rows_kernel<false, false>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_scale, w,
                       scores, ld, tw, R, G);
  return hipGetLastError();
}

}  // namespace dsa
