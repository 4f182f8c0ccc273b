// Host-side internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

// ---- top-k workspace -------------------------------------------------------------
constexpr int kTopkChunk = 4096;    // tokens per workgroup in the select passes
constexpr int kTopkBins = 4096;     // first-level histogram: top 12 bits of the score key
constexpr int kTopkCtrl = 16;       // control words per row
constexpr int kCandCap = 16384;     // per-row candidate list (beyond it, passes rescan scores)
constexpr int kMaxCtx = 1 << 22;    // largest supported context

// control word indices
enum : int { CT_DONE1 = 0, CT_DONE2 = 1, CT_NCAND = 2, CT_B1 = 3, CT_NEED1 = 4, CT_NEQ = 5,
             CT_CSTAR_HI = 6, CT_CSTAR_LO = 7 };

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int topk_chunks(int max_ctx) { int c = (max_ctx + kTopkChunk - 1) / kTopkChunk; return c < 1 ? 1 : c; }

struct TopkWs {
  uint32_t* hist;   // [R][kTopkBins]   (cleared before each call)
  uint32_t* ctrl;   // [R][kTopkCtrl]   (cleared before each call, contiguous after hist)
  uint32_t* gtc;    // [R][nch]
  uint32_t* base;   // [R][nch]
  uint32_t* cand;   // [R][kCandCap]
  int nch;
  size_t clear_words;  // words from hist to the end of ctrl
};

inline size_t topk_ws_bytes(int R, int max_ctx) {
  size_t nch = (size_t)topk_chunks(max_ctx);
  size_t b = 0;
  b += align_up((size_t)R * kTopkBins * 4, 256);
  b += align_up((size_t)R * kTopkCtrl * 4, 256);
  b += align_up((size_t)R * nch * 4, 256);
  b += align_up((size_t)R * nch * 4, 256);
  b += align_up((size_t)R * kCandCap * 4, 256);
  return b;
}

inline TopkWs topk_ws_carve(void* ws, int R, int max_ctx) {
  TopkWs t;
  uint8_t* p = static_cast<uint8_t*>(ws);
  t.nch = topk_chunks(max_ctx);
  t.hist = reinterpret_cast<uint32_t*>(p);
  size_t hb = (size_t)R * kTopkBins * 4;
  // ctrl directly after hist so that one clear covers both
  t.ctrl = reinterpret_cast<uint32_t*>(p + hb);
  t.clear_words = (size_t)R * (kTopkBins + kTopkCtrl);
  p += align_up(hb, 256) + align_up((size_t)R * kTopkCtrl * 4, 256);
  // hb is a multiple of 256 (kTopkBins * 4 = 16 KiB per row), so ctrl sits right after hist
  t.gtc = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)R * t.nch * 4, 256);
  t.base = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)R * t.nch * 4, 256);
  t.cand = reinterpret_cast<uint32_t*>(p);
  return t;
}

// ---- sparse MLA workspace -------------------------------------------------------------
constexpr int kMlaChunk = 64;   // tokens per inner iteration
constexpr int kMlaGroup = 32;   // latent-query heads per workgroup

inline int mla_splits(int R, int k) {
  if (R <= 0) return 1;
  int maxs = (k + kMlaChunk - 1) / kMlaChunk;
  int want = (512 + 3 * R - 1) / (3 * R);
  int s = want < 1 ? 1 : (want > maxs ? maxs : want);
  int ts = (k + s - 1) / s;
  ts = (ts + kMlaChunk - 1) / kMlaChunk * kMlaChunk;
  s = (k + ts - 1) / ts;
  return s < 1 ? 1 : s;
}
inline int mla_split_tokens(int k, int nsplit) {
  int ts = (k + nsplit - 1) / nsplit;
  return (ts + kMlaChunk - 1) / kMlaChunk * kMlaChunk;
}
inline size_t mla_ws_bytes(int R, int k) {
  int s = mla_splits(R, k);
  if (s <= 1) return 256;
  return align_up((size_t)R * s * kHQ * kDV * 4, 256) + align_up((size_t)R * s * kHQ * 2 * 4, 256);
}

// ---- launches -------------------------------------------------------------------------
hipError_t launch_indexer_fp8(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const float* q_scale,
                              const float* w, int R, float* scores, int64_t ld, uint32_t* clear_ptr,
                              int64_t clear_words, hipStream_t stream);

hipError_t launch_clear(uint32_t* p, size_t words, hipStream_t stream);

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                       int32_t* idx, const TopkWs& ws, hipStream_t stream);

hipError_t launch_sparse_mla(const CacheView& cv, const RowMap& rm, const uint16_t* q_lat, const int32_t* idx,
                             int R, int k, float sm_scale, float* out, float* lse, void* ws, hipStream_t stream);

}  // namespace dsa
