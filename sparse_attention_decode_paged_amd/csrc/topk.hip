// Exact per-row top-k kernels: stage 1 over an existing score array (the standalone
// top-k entry point; the indexers run the same stage in their epilogue) and stage 2, the
// select, one workgroup per row. The method (vLLM "Day-0 support for Kimi K3.1 Pro":
// the fused decode path's exact top-k, the zero-mismatch RL section's batch-invariant
// top-k and the DCP section's exact one-round merge) is described in topk_select.h.
#include "topk_select.h"

namespace dsa {

// Stage 1 over an existing score array (the standalone top-k entry point): one
// workgroup of 512 threads per 512 tokens of a row, all threads reaching the send.
__global__ __launch_bounds__(512) void topk_send_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_ctx, int max_ctx,
                                                        TopkWs ws) {
  __shared__ uint32_t send_lds[send_lds_words<512>()];
  const int r = blockIdx.y;
  const int ctx = clamp_ctx(row_ctx, r, max_ctx, nullptr);  // the select reports it
  const int base = blockIdx.x * 512;
  if (base >= ctx) return;  // whole workgroup
  const int t = base + threadIdx.x;
  const bool valid = t < ctx;
  const float s = valid ? scores[(int64_t)r * ld + t] : 0.f;
  send_candidates<512>(s, valid, ctx, base, r, ws, send_lds);
}


// One workgroup per row (the select's description is in topk_select.h). The candidate
// arrays lead the argument list so that their addresses arrive preloaded in scalar
// registers (kernel-argument preloading covers leading scalar and pointer arguments, not
// structures) and the candidate loads start with the kernel.
template <bool CAND>
__global__ __launch_bounds__(SEL_NT) void topk_select_kernel(const uint32_t* __restrict__ cand_hi,
                                                             const uint32_t* __restrict__ cand_lo,
                                                             const uint32_t* __restrict__ floors,
                                                             const float* __restrict__ scores, int64_t ld,
                                                             const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                                             int umax, int load_b, int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ phys, CacheView cv, RowMap rm) {
  __shared__ SelShared S;
  select_row<CAND>(cand_hi, cand_lo, floors, scores, ld, row_ctx, max_ctx, k, umax, load_b, idx, phys, false, cv, rm,
                   (int)blockIdx.x, S, [] {});
}

hipError_t launch_topk_send(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx,
                            const TopkWs& ws, hipStream_t stream) {
  if (R <= 0 || max_ctx <= kTopkFullRow) return hipSuccess;
  dim3 grid((max_ctx + 511) / 512, R);
  hipLaunchKernelGGL(topk_send_kernel, grid, dim3(512), 0, stream, scores, ld, row_ctx, max_ctx, ws);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                              int umax, int32_t* idx, const TopkWs& ws, int32_t* phys, const CacheView* cv,
                              const RowMap* rm, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  CacheView c{};
  RowMap m{};
  if (cv) c = *cv;  // without page slots only its status word is used
  if (phys) m = *rm;
  if (!phys) m.row_seq = row_ctx;  // read, never used
  const int load_b = cand_plan(max_ctx, umax).per == 16 ? 1 : 0;
  if (max_ctx > kTopkFullRow)
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3(R), dim3(SEL_NT), 0, stream, ws.cand_hi, ws.cand_lo, ws.floors,
                       scores, ld, row_ctx, max_ctx, k, umax, load_b, idx, phys, c, m);
  else
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3(R), dim3(SEL_NT), 0, stream, ws.cand_hi, ws.cand_lo, ws.floors,
                       scores, ld, row_ctx, max_ctx, k, umax, 0, idx, phys, c, m);
  return hipGetLastError();
}

}  // namespace dsa

