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
// Memory path. One wave scores 64 consecutive tokens of one row as two 32-token
// tiles; a tile's keys are 4 KB, contiguous inside a page when the block size is at
// least 32. Each of the wave's four 16-byte loads per tile reads 1 KB of whole
// 128-byte lines (lane l takes byte 16 l of the kilobyte), which keeps the number
// of vector memory instructions and cache-line requests per byte minimal; per-lane
// gathers of one token's half key measured 2.3x slower at 256K tokens. Key loads
// are nontemporal: the keys are read once per step. The tile
// then passes through a wave-private LDS buffer, written with an XOR swizzle of the
// 16-byte chunks so that the MFMA operand reads (lane = token, 64 bytes of its key)
// are bank-conflict free. Block-table entries, head weights and query scales are
// uniform loads; key scales come with one load and scores leave with one store per
// 64 tokens.
//
// Epilogue for the exact top-k: each unit of 64, 256 or 512 tokens sends its best m
// keys (in token order) plus a floor (topk_send.h). Workgroups of 512 tokens let rows
// longer than 131,072 tokens use 512-token units, which halves the candidates the
// select searches at 262,144 tokens (8,192 instead of 16,384).
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "topk_send.h"

namespace dsa {

namespace {
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kDIdx;  // 4 KB
constexpr int NTI = 512;                      // threads (and tokens) of a workgroup
constexpr int NWI = NTI / 64;

// 16-byte chunk c of tile token tn sits at LDS byte tn*128 + 16*(c ^ (tn & 7)).
__device__ __forceinline__ int swz(int tn, int c) { return tn * kDIdx + 16 * (c ^ (tn & 7)); }
}  // namespace

// One workgroup = 8 waves = 512 consecutive tokens of one row; wave w owns tokens
// [64w, 64w + 64) of it. PAGED32: block size >= 32, so a tile lies inside one page.
// Waves past the row's end stay to the epilogue, whose 256- and 512-token units take a
// workgroup barrier. SEND: also run stage 1 of the top-k on the fresh scores.
// EARLY (launches of several rows): workgroups past their row's end leave before
// loading keys.
// The three row-map pointers lead the argument list so that they arrive preloaded in
// scalar registers (kernel-argument preloading covers leading scalar and pointer
// arguments, not structures): the first loads of the dependent chain row -> block
// table -> keys need no kernel-argument fetch before them.
template <bool PAGED32, bool SEND, bool EARLY>
__global__ __launch_bounds__(NTI) void indexer_fp8_kernel(const int32_t* __restrict__ row_seq,
                                                          const int32_t* __restrict__ row_ctx,
                                                          const int32_t* __restrict__ block_table, CacheView cv,
                                                          RowMap rm, const uint8_t* __restrict__ q_idx,
                                                          const float* __restrict__ q_scale,
                                                          const float* __restrict__ w, float* __restrict__ scores,
                                                          int64_t ld, TopkWs tw) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[NWI][kTileBytes];
  __shared__ uint32_t send_lds[send_lds_words<NTI>()];
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the row's length and block-table row are read together. A workgroup past the
  // row's end leaves as soon as the length is in when the launch has several rows
  // (EARLY: rows of mixed lengths leave many such workgroups); with one row it still
  // issues its clamped, valid loads and leaves after them, which keeps a branch out of
  // the key stream's issue.
  const int seq = row_seq[r];
  int ctx = row_ctx[r];
  if (ctx > rm.max_ctx) {
    raise_status(cv.status, kStCtxClamped);
    ctx = rm.max_ctx;
  }
  ctx = ctx < 0 ? 0 : ctx;
  const bool past = blockIdx.x * NTI >= ctx;  // whole workgroup
  if (EARLY && past) return;                  // no barrier reached
  ctx = ctx > 0 ? ctx : 1;
  const int tok0 = blockIdx.x * NTI + wid * 64;
  const int bs_mask = cv.block_size - 1;

  // ---- query fragment (head n, bytes [64g, 64g + 64)), issued ahead of the key stream:
  // vector loads return in issue order, so the first tile's contraction then waits only
  // for its own keys and overlaps the second tile's arrival ----
  v4i qr[4];
  {
    const v4i* qp = reinterpret_cast<const v4i*>(q_idx + ((int64_t)r * kHIdx + n) * kDIdx + 64 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) qr[i] = qp[i];
  }
  // ---- key loads for both tiles: 4 x 1 KB of whole lines each. No branches: a tile
  // start past the row's end is clamped to the row's last tile, so every load reads
  // valid keys; results for tokens >= ctx are never stored ----
  v4i kv[2][4];
  int64_t toff[2];  // byte offset of each tile's index page in the pool (PAGED32)
  const int last_tile = (ctx - 1) & ~(kTileTok - 1);
  const int tb1 = tok0 + kTileTok < last_tile ? tok0 + kTileTok : last_tile;
  const int tb0 = tok0 < last_tile ? tok0 : last_tile;
  if (PAGED32) {  // both block-table entries are loaded before either is used
    const int32_t* btrow = block_table + (int64_t)seq * rm.bt_stride;
    // read as unsigned (no sign extension between the two loads), so both are in
    // flight together; ids outside [0, num_blocks) are clamped like token_block does
    const uint32_t e0 = (uint32_t)btrow[tb0 >> cv.log2_bs], e1 = (uint32_t)btrow[tb1 >> cv.log2_bs];
    __builtin_amdgcn_sched_barrier(0);
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
        t = t < ctx ? t : ctx - 1;
        const uint8_t* key = row_base(cv, token_block(cv, rm, seq, t)) + cv.idx_off + (int64_t)(t & bs_mask) * kDIdx;
        kv[j][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(key + 16 * (lane & 7)));
      }
    }
  }
  // key scale of token tok0 + lane (clamped into the row); with PAGED32 the token's
  // page is one of the two tiles' pages (uniform addresses), so the load does not
  // wait behind the key loads
  float ksc;
  {
    int t = tok0 + lane;
    t = t < ctx ? t : ctx - 1;
    const int64_t off = PAGED32 ? ((t & ~(kTileTok - 1)) == tb1 ? toff[1] : toff[0])
                                : token_block(cv, rm, seq, t) * cv.row_bytes + cv.idx_off;
    ksc = *reinterpret_cast<const float*>(cv.pool + off + (int64_t)cv.block_size * kDIdx + (int64_t)(t & bs_mask) * 4);
  }

  // folded head weights (uniform: scalar loads, kept in scalar registers)
  float W[kHIdx];
#pragma unroll
  for (int h = 0; h < kHIdx; ++h)
    W[h] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w[r * kHIdx + h] * q_scale[r * kHIdx + h])));

  // every load of the wave is in flight before anything waits on one
  __builtin_amdgcn_sched_barrier(0);
  if (!EARLY && past) return;  // whole workgroup, no barrier reached

  v8bf qa[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qa[2 * i] = e4m3x8_to_bf16((uint32_t)qr[i][0], (uint32_t)qr[i][1]);
    qa[2 * i + 1] = e4m3x8_to_bf16((uint32_t)qr[i][2], (uint32_t)qr[i][3]);
  }
  // accumulator element rr of lane (n, g) is head 8 (rr >> 2) + 4 g + (rr & 3)
  float wq[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) wq[rr] = g ? W[8 * (rr >> 2) + 4 + (rr & 3)] : W[8 * (rr >> 2) + (rr & 3)];

  // ---- per tile: swizzled LDS transpose, 8 bf16 MFMAs, ReLU + weighted head sum ----
  const int wpos = swz(lane >> 3, lane & 7);  // where this lane's chunk of each kilobyte goes
  float res[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(&lds[wid][1024 * i + wpos]) = kv[j][i];
    v4i kr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = *reinterpret_cast<const v4i*>(&lds[wid][swz(n, 4 * g + i)]);
    v16f acc = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const v8bf b = e4m3x8_to_bf16((uint32_t)kr[kk >> 1][(kk & 1) * 2], (uint32_t)kr[kk >> 1][(kk & 1) * 2 + 1]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], b, acc, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s = fmaf(wq[rr], relu_bits(acc[rr]), s);
    s += xshflf<32>(s);
    res[j] = s;
  }
  // lane l now owns token tok0 + l: tile 0 on lanes 0..31, tile 1 on lanes 32..63
  const int t = tok0 + lane;
  const float sc = (g ? res[1] : res[0]) * ksc;
  if (t < ctx) scores[(int64_t)r * ld + t] = sc;
  if (SEND) send_candidates<NTI>(sc, t < ctx, ctx, blockIdx.x * NTI, r, tw, send_lds);
}

hipError_t launch_indexer_fp8(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const float* q_scale,
                              const float* w, int R, float* scores, int64_t ld, const TopkWs* ws,
                              hipStream_t stream) {
  int nx = (rm.max_ctx + NTI - 1) / NTI;
  if (nx < 1) nx = 1;
  TopkWs tw = ws ? *ws : TopkWs{nullptr, nullptr, nullptr};
  const int send = (ws != nullptr && rm.max_ctx > kTopkFullRow) ? 1 : 0;
  dim3 grid(nx, R);
  const bool p32 = cv.block_size >= kTileTok;
  auto go = [&](auto early) {
    constexpr bool E = decltype(early)::value;
    if (send && p32)
      hipLaunchKernelGGL((indexer_fp8_kernel<true, true, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx, rm.block_table, cv,
                         rm, q_idx, q_scale, w, scores, ld, tw);
    else if (send)
      hipLaunchKernelGGL((indexer_fp8_kernel<false, true, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx, rm.block_table, cv,
                         rm, q_idx, q_scale, w, scores, ld, tw);
    else if (p32)
      hipLaunchKernelGGL((indexer_fp8_kernel<true, false, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx, rm.block_table, cv,
                         rm, q_idx, q_scale, w, scores, ld, tw);
    else
      hipLaunchKernelGGL((indexer_fp8_kernel<false, false, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx, rm.block_table, cv,
                         rm, q_idx, q_scale, w, scores, ld, tw);
  };
  if (R > 1)
    go(std::true_type{});
  else
    go(std::false_type{});
  return hipGetLastError();
}

}  // namespace dsa
