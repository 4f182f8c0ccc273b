// Host-side internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

// ---- top-k workspace -------------------------------------------------------------
constexpr int kTopkFullRow = 16384;   // rows up to this length are selected from all their scores
constexpr int kCandRowCap = 16384;    // candidate keys a row sends in total (select stage registers)
constexpr int kMaxCtx = 1 << 20;      // largest supported context
constexpr int kFloorRowCap = kMaxCtx / 256;  // units of a row, at most

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// A candidate key is kept as two words at the same slot of two arrays, so that the
// select can load the score words (all its search passes need) ahead of the tokens.
struct TopkWs {
  uint32_t* cand_hi;  // [R][kCandRowCap]: score word of rank q of unit u at slot u m + q; 0 = empty
  uint32_t* cand_lo;  // [R][kCandRowCap]: its token word (0xFFFFFFFF - token)
  uint32_t* floors;   // [R][kFloorRowCap]: score word bounding the keys a unit did not send (0: sent all)
};

// Rows of at most kTopkFullRow tokens send no candidates: no candidate space then.
inline size_t topk_ws_bytes(int R, int max_ctx) {
  if (max_ctx <= kTopkFullRow) return 256;
  return 2 * align_up((size_t)R * kCandRowCap * 4, 256) + align_up((size_t)R * kFloorRowCap * 4, 256);
}

inline TopkWs topk_ws_carve(void* ws, int R, int max_ctx) {
  TopkWs t{nullptr, nullptr, nullptr};
  if (max_ctx <= kTopkFullRow) return t;
  uint8_t* p = static_cast<uint8_t*>(ws);
  t.cand_hi = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)R * kCandRowCap * 4, 256);
  t.cand_lo = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)R * kCandRowCap * 4, 256);
  t.floors = reinterpret_cast<uint32_t*>(p);
  return t;
}

// ---- sparse MLA workspace -------------------------------------------------------------
constexpr int kMlaChunk = 64;   // tokens per inner iteration
// Latent-query heads per sparse-MLA workgroup: 16 for batches of up to 4 rows (a row's
// work spreads over twice as many CUs), 32 above (each gathered latent serves twice as
// many heads).
inline int mla_group(int R) { return R <= 4 ? 16 : 32; }

// Splits of a row's k tokens for sparse MLA, and which kernel runs them. An eight-wave
// workgroup (one per CU: its registers allow no second) takes whole 64-token chunks;
// R rows x 3 head groups (6 of 16 heads for up to 4 rows) x s splits run in rounds of
// kMlaSlots workgroups, at an estimated rounds x (chunks per split + a prologue worth
// 1.5 chunks), plus one chunk's worth for the merge kernel when s > 1; ties go to fewer
// splits. When that choice needs more than one round and the latents are FP8, the
// four-wave 32-head kernel runs instead, with its own split count: a CU holds
// ceil(workgroups / kMlaSlots) of its workgroups and runs them two at a time, a pair
// taking about 2.95 + 1.87 x (chunks per split) of those chunk times and an odd last
// one alone 1.27 + 1.37 x (chunks per split), plus the merge's chunk when s > 1 (fitted
// to measured batches of 16 to 64 rows; with one round or less the eight-wave kernel
// was as fast or faster).
constexpr int kMlaSlots = 256;  // CUs of the device
struct MlaPlan {
  int nsplit;
  bool four_wave;
};
inline MlaPlan mla_plan(int R, int k, bool fp8_latents) {
  MlaPlan p8{1, false}, p4{0, true};
  if (R <= 0) return p8;
  const int nch = (k + kMlaChunk - 1) / kMlaChunk;
  double c8_best = 0.0, c4_best = 0.0;
  int64_t wgs8 = 0;
  for (int s = 1; s <= nch; ++s) {
    const int cps = (nch + s - 1) / s;  // chunks per split
    if ((nch + cps - 1) / cps != s) continue;  // s is not reached by whole chunks
    const int64_t wgs = (int64_t)R * (kHQ / mla_group(R)) * s;
    const int64_t per_cu = (wgs + kMlaSlots - 1) / kMlaSlots;
    const double merge = s > 1 ? 1.0 : 0.0;
    const double c8 = (double)per_cu * (cps + 1.5) + merge;
    if (s == 1 || c8 < c8_best) {
      p8 = MlaPlan{s, false};
      c8_best = c8;
      wgs8 = wgs;
    }
    if (per_cu > 1) {
      const double c4 = (double)(per_cu / 2) * (2.95 + 1.87 * cps) + (double)(per_cu % 2) * (1.27 + 1.37 * cps) + merge;
      if (p4.nsplit == 0 || c4 < c4_best) {
        p4.nsplit = s;
        c4_best = c4;
      }
    }
  }
  const bool w4 = fp8_latents && mla_group(R) == 32 && wgs8 > kMlaSlots && p4.nsplit > 0;
  return w4 ? p4 : p8;
}
inline int mla_split_tokens(int k, int nsplit) {
  int ts = (k + nsplit - 1) / nsplit;
  return (ts + kMlaChunk - 1) / kMlaChunk * kMlaChunk;
}
// The workspace does not depend on the latent format: it covers both plans.
inline size_t mla_ws_bytes(int R, int k) {
  const int s8 = mla_plan(R, k, false).nsplit, s4 = mla_plan(R, k, true).nsplit;
  const int s = s8 > s4 ? s8 : s4;
  if (s <= 1) return 256;
  return align_up((size_t)R * s * kHQ * kDV * 2, 256) + align_up((size_t)R * s * kHQ * 2 * 4, 256);
}

// ---- context-parallel merge emulation workspace -------------------------------------
constexpr int kDcpShardMax = 32;                       // shards (bits of the resend mask)
constexpr int kDcpWordCap = 3 * kMaxK / 2 + kDcpShardMax;  // W * ceil(1.5 k / W) < 1.5 k + W

inline int dcp_send_count(int k, int W) { return (3 * k + 2 * W - 1) / (2 * W); }  // ceil(1.5 k / W)
inline int dcp_shard_len(int max_ctx, int W) { return (max_ctx + W - 1) / W; }
inline int64_t dcp_shard_ld(int max_ctx, int W) {
  const int l = dcp_shard_len(max_ctx, W);
  return (int64_t)align_up((size_t)(l > 0 ? l : 1), 64);
}

struct DcpWs {
  float* shard;        // [R W][ls] scores dealt out token-strided
  int64_t ls;
  int32_t* shard_ctx;  // [R W]
  int32_t* idx_m;      // [R W][M] best-M lists (shard-local places)
  int32_t* idx_k;      // [R W][k] best-k lists
  uint64_t* ukeys;     // [R][ucap] received candidates (composite keys)
  int64_t ucap;
  TopkWs tw;           // two-stage select over the shard rows
};

inline size_t dcp_ws_bytes(int R, int max_ctx, int k, int W) {
  const size_t RW = (size_t)R * W, M = (size_t)dcp_send_count(k, W);
  const size_t ucap = (size_t)W * M + (size_t)W * k;
  return align_up(RW * dcp_shard_ld(max_ctx, W) * 4, 256) + align_up(RW * 4, 256) + align_up(RW * M * 4, 256) +
         align_up(RW * k * 4, 256) + align_up((size_t)R * ucap * 8, 256) + topk_ws_bytes((int)RW, dcp_shard_len(max_ctx, W));
}

inline DcpWs dcp_ws_carve(void* ws, int R, int max_ctx, int k, int W) {
  DcpWs d;
  const size_t RW = (size_t)R * W, M = (size_t)dcp_send_count(k, W);
  uint8_t* p = static_cast<uint8_t*>(ws);
  d.ls = dcp_shard_ld(max_ctx, W);
  d.ucap = (int64_t)(W * M + (size_t)W * k);
  d.shard = reinterpret_cast<float*>(p);
  p += align_up(RW * d.ls * 4, 256);
  d.shard_ctx = reinterpret_cast<int32_t*>(p);
  p += align_up(RW * 4, 256);
  d.idx_m = reinterpret_cast<int32_t*>(p);
  p += align_up(RW * M * 4, 256);
  d.idx_k = reinterpret_cast<int32_t*>(p);
  p += align_up(RW * k * 4, 256);
  d.ukeys = reinterpret_cast<uint64_t*>(p);
  p += align_up((size_t)R * d.ucap * 8, 256);
  d.tw = topk_ws_carve(p, (int)RW, dcp_shard_len(max_ctx, W));
  return d;
}

// ---- launches -------------------------------------------------------------------------
// Indexer; when `ws` is non-null the epilogue also sends each block's top-k candidates.
hipError_t launch_indexer_fp8(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const float* q_scale,
                              const float* w, int R, float* scores, int64_t ld, const TopkWs* ws,
                              hipStream_t stream);

// Indexer for G consecutive rows per workgroup that share one sequence (FP8 keys): each
// key tile is read and converted once for all of them.
hipError_t launch_indexer_fp8_rows(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const float* q_scale,
                                   const float* w, int R, int G, float* scores, int64_t ld, const TopkWs* ws,
                                   hipStream_t stream);
constexpr int kRowsPerGroupMax = 16;  // rows one workgroup of the row-group indexer covers, at most

// New-token cache append (quantise and write index key and latent of one token per row).
hipError_t launch_cache_append(const CacheView& cv, int32_t index_fmt, const int32_t* block_table, int32_t bt_stride,
                               const int32_t* row_seq, const int32_t* pos, const float* idx_key,
                               const float* latent, int R, hipStream_t stream);

// Row-group indexer over MXFP4 keys (G consecutive rows per workgroup share each key tile).
hipError_t launch_indexer_mxfp4_rows(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx,
                                     const uint8_t* q_e8, const float* w, int R, int G, float* scores, int64_t ld,
                                     const TopkWs* ws, hipStream_t stream);

// Indexer over MXFP4 keys (q_idx: R x 32 x 64 packed e2m1, q_e8: R x 32 x 4 E8M0).
hipError_t launch_indexer_mxfp4(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const uint8_t* q_e8,
                                const float* w, int R, float* scores, int64_t ld, const TopkWs* ws,
                                hipStream_t stream);

// Candidate sending over an existing score array (standalone top-k).
hipError_t launch_topk_send(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx,
                            const TopkWs& ws, hipStream_t stream);
// Selection; when `phys` is non-null it also receives, per selected token, its page
// slot (physical block * block_size + slot) for the attention kernel (cv and rm are
// then required; without page slots cv may carry just the status word, or be null).
// umax: the largest unit (tokens) of the candidate producer, its workgroup size (256 or
// 512), which fixes every row's candidate plan.
hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                              int umax, int32_t* idx, const TopkWs& ws, int32_t* phys, const CacheView* cv,
                              const RowMap* rm, hipStream_t stream);
// Workgroup size of the candidate producer the decode step uses for a row grouping (the
// per-row indexers and the standalone send run 512 threads, the row-group indexers 256).
inline int send_umax(int32_t rows_per_seq) { return rows_per_seq <= 1 ? 512 : 256; }

// Sparse MLA over idx; when `phys` (page slots from the selection) is non-null it
// replaces the block-table lookups.
// parts: 1 = the attention kernel, 2 = the split merge (a kernel of its own when the
// rows are split), 3 = both.
hipError_t launch_sparse_mla(const CacheView& cv, const RowMap& rm, const uint16_t* q_lat, const int32_t* idx,
                             const int32_t* phys, int R, int k, float sm_scale, float* out, float* lse, void* ws,
                             int parts, hipStream_t stream);

// The select and the sparse-MLA attention as one launch (the merge stays a launch of its
// own): every attention workgroup runs its row's select and keeps the list on chip. For
// FP8 latents and grids of at most kSelMlaMaxGroups workgroups (one per CU of the
// 256-CU part); select_mla_fused tells whether the decode step takes it. Writes idx
// (not the page slots) and the same out / lse / partials as the two launches.
constexpr int kSelMlaMaxGroups = 256;
bool select_mla_fused(const CacheView& cv, int R, int k);
hipError_t launch_select_mla(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                             int umax, int32_t* idx, const TopkWs& tw, const CacheView& cv, const RowMap& rm,
                             const uint16_t* q_lat, float sm_scale, float* out, float* lse, void* ws,
                             hipStream_t stream);

// Exact top-k merge of decode context parallelism over W token-strided shards, emulated
// on one GPU (ws: dcp_ws_bytes). resend_mask / words may be null.
hipError_t launch_topk_dcp(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k, int W,
                           int32_t* idx, uint32_t* resend_mask, uint32_t* words, void* ws, hipStream_t stream);

// One streaming read of [p, p + bytes) (bytes a multiple of 16) by `grid` workgroups.
hipError_t launch_hbm_read(const void* p, size_t bytes, uint32_t* sink, int grid, hipStream_t stream);

}  // namespace dsa
