// Lightning-indexer scoring over the packed paged cache (FP8 index keys).
//
// score[r][t] = sum_h w[r][h] * ReLU(q_h . k_t) with q_h = sq[r][h] * e4m3 codes and
// k_t = sk[t] * e4m3 codes (vLLM "Day-0 support for Kimi K3.1 Pro", section
// "Sparse attention in K3.1 Pro": 32 light heads score every earlier token; page 3
// model table: 32 heads x 128 dims, FP8 keys with one scale, 132 B per token).
//
// Both scales are positive, so the kernel computes
//   score = sk[t] * sum_h (w[h] * sq[h]) * max(0, codes_q[h] . codes_k[t])
// The code dot products are a [32 heads x 128] x [128 x 32 tokens] contraction per
// tile, done on the matrix cores with bf16 inputs: every e4m3 code converts to bf16
// exactly, products of two codes are exact in fp32 and the accumulation is fp32.
// (gfx950's fp8 matrix instructions keep fewer bits than fp32 in their internal
// sum, measured ~1e-5 of |dot|, too coarse for exact top-k; the bf16 form is not.)
//
// Work split: one workgroup (4 waves) covers 256 consecutive tokens of one query
// row; each wave owns two 32-token tiles, issues all their key loads first, then
// runs the MFMAs. Lane (n, g) of a wave handles token n of a tile and bytes
// [64g, 64g+64) of its key (16-byte loads), which is also the K slice it feeds to
// the MFMA; the query fragment uses the same byte permutation.
//
// Epilogue for the exact top-k: each wave (a 64-token unit) sorts its keys across
// lanes and sends its best m keys (in token order) plus a floor (topk_send.h).
#include "common.h"
#include "internal.h"
#include "topk_send.h"

namespace dsa {

// One workgroup = 4 waves = 256 consecutive tokens of one row; each wave owns two
// 32-token tiles (one 64-token page at block size 64).
__global__ __launch_bounds__(256) void indexer_fp8_kernel(CacheView cv, RowMap rm, const uint8_t* __restrict__ q_idx,
                                                          const float* __restrict__ q_scale,
                                                          const float* __restrict__ w, float* __restrict__ scores,
                                                          int64_t ld, TopkWs tw, int send) {
  constexpr int TPW = 2;
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 5, n = lane & 31;

  const int ctx = row_len(rm, r);
  const int block_base = blockIdx.x * (4 * TPW * 32);
  if (block_base >= ctx) return;  // whole workgroup
  const int tok0 = block_base + wid * (TPW * 32);
  const bool active = tok0 < ctx;  // wave-uniform
  const int seq = rm.row_seq[r];
  const int bs_mask = cv.block_size - 1;

  // Key loads for both tiles first (token clamped into the row so every load is valid).
  v4i kraw[TPW][4];
  float ksc[TPW];
  if (active) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      int t = tok0 + j * 32 + n;
      int tc = t < ctx ? t : ctx - 1;
      int64_t blk = token_block(cv, rm, seq, tc);
      int slot = tc & bs_mask;
      const uint8_t* page = row_base(cv, blk) + cv.idx_off;
      const v4i* kp = reinterpret_cast<const v4i*>(page + slot * kDIdx + 64 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) kraw[j][i] = kp[i];
      ksc[j] = *reinterpret_cast<const float*>(page + (int64_t)cv.block_size * kDIdx + slot * 4);
    }
  }

  // Query fragment: head n, bytes [64g, 64g+64) -> 8 x v8bf.
  const v4i* qp = reinterpret_cast<const v4i*>(q_idx + ((int64_t)r * kHIdx + n) * kDIdx + 64 * g);
  v8bf qa[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v4i q = qp[i];
    qa[2 * i] = e4m3x8_to_bf16((uint32_t)q[0], (uint32_t)q[1]);
    qa[2 * i + 1] = e4m3x8_to_bf16((uint32_t)q[2], (uint32_t)q[3]);
  }
  // Folded head weights for the 16 heads this lane's accumulators hold.
  float wq[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    int m = 8 * (rr >> 2) + 4 * g + (rr & 3);
    wq[rr] = w[r * kHIdx + m] * q_scale[r * kHIdx + m];
  }

  float* srow = scores + (int64_t)r * ld;
  float sc[TPW] = {0.f, 0.f};
  if (active) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      v16f acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        v8bf b = e4m3x8_to_bf16((uint32_t)kraw[j][kk >> 1][(kk & 1) * 2],
                                (uint32_t)kraw[j][kk >> 1][(kk & 1) * 2 + 1]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], b, acc, 0, 0, 0);
      }
      float s = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s = fmaf(wq[rr], fmaxf(acc[rr], 0.f), s);
      s += xshflf<32>(s);
      s *= ksc[j];
      sc[j] = s;
      int t = tok0 + j * 32 + n;
      if (g == 0 && t < ctx) srow[t] = s;
    }
  }
  if (send && active) {
    // lane n + 32g of the wave owns token tok0 + 32g + n: the wave is one 64-token unit
    const int t = tok0 + 32 * g + n;
    wave_send_candidates(g ? sc[1] : sc[0], t < ctx, ctx, tok0, r, blockIdx.x * 4 + wid, tw);
  }
}

hipError_t launch_indexer_fp8(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const float* q_scale,
                              const float* w, int R, float* scores, int64_t ld, const TopkWs* ws,
                              hipStream_t stream) {
  int nx = (rm.max_ctx + 4 * kCandUnit - 1) / (4 * kCandUnit);
  if (nx < 1) nx = 1;
  TopkWs tw = ws ? *ws : TopkWs{nullptr, nullptr, 1};
  const int send = (ws != nullptr && rm.max_ctx > kTopkFullRow) ? 1 : 0;
  dim3 grid(nx, R);
  hipLaunchKernelGGL(indexer_fp8_kernel, grid, dim3(256), 0, stream, cv, rm, q_idx, q_scale, w, scores, ld, tw, send);
  return hipGetLastError();
}

}  // namespace dsa
