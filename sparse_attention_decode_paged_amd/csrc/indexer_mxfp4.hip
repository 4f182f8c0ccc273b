// Lightning-indexer scoring over the packed paged cache with MXFP4 index keys.
//
// Same score as the FP8 indexer, score[r][t] = sum_h w[r][h] * ReLU(q_h . k_t), with
// query and key in MXFP4 (vLLM "Day-0 support for Kimi K3.1 Pro", AMD section: MXFP4
// index keys scored with FP4 matrix instructions and fp32 accumulation; 68 B per
// token: 64 B of e2m1 codes, element 2i in the low nibble of byte i, and one E8M0
// exponent per 32 elements).
//
// The contraction runs on gfx950's native FP4 matrix instruction: one 32x32x64
// scaled MFMA (f8f6f4 in FP4 format) per 64 dims, e2m1 codes of query and key as the
// operands and each 32-group's E8M0 exponent as the lane's operand scale, fp32
// accumulation. With FP4 operands and power-of-two scales the instruction is exact (a
// measurement over 2.1M indexer-shaped dot products found no difference from float64),
// so the scores are the same as from exact products summed in fp32; two instructions
// cover a 32-head x 32-token x 128-dim tile, and no operand is converted.
//
// Operand layout: for step s (dims [64 s, 64 s + 64)) lane l holds row l % 32 (query
// head or key token) and dims [64 s + 32 (l / 32), +32), i.e. bytes
// [32 s + 16 (l / 32), +16) of the row's 64 code bytes, under the E8M0 of group
// 2 s + l / 32. Query and key use the same assignment, so every product pairs the same
// dim.
//
// Memory path as in the FP8 kernel: one wave scores 64 consecutive tokens as two
// 32-token tiles; a tile's 2 KB of codes is read as two 1 KB runs of whole 128-byte
// lines (lane l takes byte 16 l), nontemporal, and goes through a wave-private LDS
// buffer with the 16-byte chunks XOR-swizzled by token. E8M0 exponents come with one
// dword load per lane (its token's four).
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "topk_send.h"

namespace dsa {

namespace {
constexpr int kTileTok = 32;
constexpr int kKeyBytes = kDIdx / 2;             // 64 B of e2m1 codes per key
constexpr int kTileBytes = kTileTok * kKeyBytes;  // 2 KB
constexpr int NTI = 512;                          // threads (and tokens) of a per-row workgroup
constexpr int NWI = NTI / 64;

// 16-byte chunk c (of 4) of tile token tn sits at LDS byte tn*64 + 16*(c ^ (tn & 3)).
__device__ __forceinline__ int swz4(int tn, int c) { return tn * kKeyBytes + 16 * (c ^ (tn & 3)); }

// One 32 x 32 x 64 step on FP4 operands (16 code bytes per lane, e2m1 pairs) with
// per-lane E8M0 scales (the exponent byte, bias 127).
__device__ __forceinline__ v16f mfma_fp4(v4i a, v4i b, int ea, int eb, v16f acc) {
  const v8i av = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i bv = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, ea, 0, eb);
}
}  // namespace

// One workgroup = 8 waves = 512 consecutive tokens of one row (so that rows longer than
// 131,072 tokens send 512-token top-k units); wave w owns tokens [64w, 64w + 64). PAGED32: block size >= 32, so a tile lies inside one page.
// SEND: also run stage 1 of the top-k on the fresh scores. EARLY: as for the FP8 kernel.
template <bool PAGED32, bool SEND, bool EARLY>
// Row-map pointers lead the argument list (preloaded in scalar registers), as for the
// FP8 kernel.
__global__ __launch_bounds__(NTI) void indexer_mxfp4_kernel(const int32_t* __restrict__ row_seq,
                                                            const int32_t* __restrict__ row_ctx,
                                                            const int32_t* __restrict__ block_table, CacheView cv,
                                                            RowMap rm, const uint8_t* __restrict__ q_idx,
                                                            const uint8_t* __restrict__ q_e8,
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
  const int64_t sc_off = (int64_t)cv.block_size * kKeyBytes;  // E8M0 bytes follow the codes in a page

  // ---- query operands (head n, code bytes [16 g, +16) and [32 + 16 g, +16)) with their
  // E8M0 exponents, issued ahead of the key stream: vector loads return in issue order,
  // so the first tile's MFMAs wait only for its own keys ----
  v4i qr[2];
  {
    const uint8_t* qp = q_idx + ((int64_t)r * kHIdx + n) * kKeyBytes + 16 * g;
    qr[0] = *reinterpret_cast<const v4i*>(qp);
    qr[1] = *reinterpret_cast<const v4i*>(qp + 32);
  }
  const uint32_t qe = *reinterpret_cast<const uint32_t*>(q_e8 + ((int64_t)r * kHIdx + n) * 4);

  // ---- code loads for both tiles (2 x 1 KB of whole lines each), branch-free: a tile
  // start past the row's end is clamped to the row's last tile ----
  v4i kv[2][2];
  uint32_t es[2];   // the four E8M0 exponents of tile token n
  int64_t toff[2];  // byte offset of each tile's index page in the pool (PAGED32)
  const int last_tile = (ctx - 1) & ~(kTileTok - 1);
  const int tb1 = tok0 + kTileTok < last_tile ? tok0 + kTileTok : last_tile;
  const int tb0 = tok0 < last_tile ? tok0 : last_tile;
  if (PAGED32) {
    // read as unsigned (no sign extension between the two loads), so both are in
    // flight together; ids outside [0, num_blocks) are clamped like token_block does
    const int32_t* btrow = block_table + (int64_t)seq * rm.bt_stride;
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
      const uint8_t* page = cv.pool + toff[j];
      const uint8_t* tile = page + (int64_t)(tb & bs_mask) * kKeyBytes;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        kv[j][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(tile + 1024 * i + 16 * lane));
      // token tb + n lies in the tile, hence in this page (past the row's end too)
      es[j] = *reinterpret_cast<const uint32_t*>(page + sc_off + (int64_t)((tb + n) & bs_mask) * 4);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int t = tb + 16 * i + (lane >> 2);
        t = t < ctx ? t : ctx - 1;
        const uint8_t* key = row_base(cv, token_block(cv, rm, seq, t)) + cv.idx_off + (int64_t)(t & bs_mask) * kKeyBytes;
        kv[j][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(key + 16 * (lane & 3)));
      }
      int t = tb + n;
      t = t < ctx ? t : ctx - 1;
      es[j] = *reinterpret_cast<const uint32_t*>(row_base(cv, token_block(cv, rm, seq, t)) + cv.idx_off + sc_off +
                                                  (int64_t)(t & bs_mask) * 4);
    }
  }

  // head weights (uniform: scalar loads)
  float W[kHIdx];
#pragma unroll
  for (int h = 0; h < kHIdx; ++h) W[h] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w[r * kHIdx + h])));

  // every load of the wave is in flight before anything waits on one
  __builtin_amdgcn_sched_barrier(0);
  if (!EARLY && past) return;  // whole workgroup, no barrier reached

  const int qe0 = (int)((qe >> (8 * g)) & 255u), qe1 = (int)((qe >> (8 * (2 + g))) & 255u);  // groups g, 2 + g
  // accumulator element rr of lane (n, g) is head 8 (rr >> 2) + 4 g + (rr & 3)
  float wq[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) wq[rr] = g ? W[8 * (rr >> 2) + 4 + (rr & 3)] : W[8 * (rr >> 2) + (rr & 3)];

  // ---- per tile: swizzled LDS transpose, 2 FP4 MFMAs, ReLU + weighted head sum ----
  const int wpos = swz4(lane >> 2, lane & 3);  // this lane's chunk of each kilobyte (16 tokens)
  float res[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<v4i*>(&lds[wid][1024 * i + wpos]) = kv[j][i];
    // token n: code chunks g and 2 + g (bytes [16 g, +16) and [32 + 16 g, +16))
    const v4i k0 = *reinterpret_cast<const v4i*>(&lds[wid][swz4(n, g)]);
    const v4i k1 = *reinterpret_cast<const v4i*>(&lds[wid][swz4(n, 2 + g)]);
    const int ke0 = (int)((es[j] >> (8 * g)) & 255u), ke1 = (int)((es[j] >> (8 * (2 + g))) & 255u);
    v16f acc = {};
    acc = mfma_fp4(qr[0], k0, qe0, ke0, acc);
    acc = mfma_fp4(qr[1], k1, qe1, ke1, acc);
    float s = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s = fmaf(wq[rr], relu_bits(acc[rr]), s);
    s += xshflf<32>(s);
    res[j] = s;
  }
  // lane l now owns token tok0 + l: tile 0 on lanes 0..31, tile 1 on lanes 32..63
  const int t = tok0 + lane;
  const float sc = g ? res[1] : res[0];
  if (t < ctx) scores[(int64_t)r * ld + t] = sc;
  if (SEND) send_candidates<NTI>(sc, t < ctx, ctx, blockIdx.x * NTI, r, tw, send_lds);
}

// Several query rows of one sequence (speculative verification, prefill-append), as the
// FP8 row-group kernel: a workgroup covers 256 tokens of up to G consecutive rows, loads
// each key tile (codes through the swizzled LDS transpose, and the E8M0 exponents) once,
// and runs every row's query against it: per row two FP4 MFMAs per tile (the query
// needs no conversion), then the ReLU-weighted head sum, exactly as the per-row kernel
// computes it. A row whose sequence differs from the previous row's reloads the keys,
// so results never depend on the grouping.
template <bool PAGED32, bool SEND>
__global__ __launch_bounds__(256) void indexer_mxfp4_rows_kernel(CacheView cv, RowMap rm,
                                                                 const uint8_t* __restrict__ q_idx,
                                                                 const uint8_t* __restrict__ q_e8,
                                                                 const float* __restrict__ w,
                                                                 float* __restrict__ scores, int64_t ld, TopkWs tw,
                                                                 int R, int G) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][kTileBytes];
  __shared__ uint32_t send_lds[2][send_lds_words<256>()];  // double-buffered over the rows that take the 256-token send
  __shared__ __attribute__((aligned(16))) float w_s[kRowsPerGroupMax * kHIdx];  // head weights of the group's rows
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
  const int64_t sc_off = (int64_t)cv.block_size * kKeyBytes;
  const int wpos = swz4(lane >> 2, lane & 3);

  v4i kb[2][2];     // B operands of both tiles: token n's code chunks g and 2 + g
  int ke[2][2];     // and their E8M0 exponents
  // Keys of sequence `seq` for the run of rows that starts here (tile starts clamped into
  // the run's longest row, smax >= 1, so no block-table entry past that sequence's own
  // tokens is read).
  auto load_keys = [&](int seq, int smax) {
    const int last_tile = (smax - 1) & ~(kTileTok - 1);
    const int tb1 = tok0 + kTileTok < last_tile ? tok0 + kTileTok : last_tile;
    const int tb0 = tok0 < last_tile ? tok0 : last_tile;
    v4i kv[2][2];
    uint32_t es[2];
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
        const uint8_t* page = cv.pool + toff[j];
        const uint8_t* tile = page + (int64_t)(tb & bs_mask) * kKeyBytes;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          kv[j][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(tile + 1024 * i + 16 * lane));
        es[j] = *reinterpret_cast<const uint32_t*>(page + sc_off + (int64_t)((tb + n) & bs_mask) * 4);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          int t = tb + 16 * i + (lane >> 2);
          t = t < smax ? t : smax - 1;
          const uint8_t* key =
              row_base(cv, token_block(cv, rm, seq, t)) + cv.idx_off + (int64_t)(t & bs_mask) * kKeyBytes;
          kv[j][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(key + 16 * (lane & 3)));
        }
        int t = tb + n;
        t = t < smax ? t : smax - 1;
        es[j] = *reinterpret_cast<const uint32_t*>(row_base(cv, token_block(cv, rm, seq, t)) + cv.idx_off + sc_off +
                                                    (int64_t)(t & bs_mask) * 4);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 2; ++i) *reinterpret_cast<v4i*>(&lds[wid][1024 * i + wpos]) = kv[j][i];
      kb[j][0] = *reinterpret_cast<const v4i*>(&lds[wid][swz4(n, g)]);
      kb[j][1] = *reinterpret_cast<const v4i*>(&lds[wid][swz4(n, 2 + g)]);
      ke[j][0] = (int)((es[j] >> (8 * g)) & 255u);
      ke[j][1] = (int)((es[j] >> (8 * (2 + g))) & 255u);
    }
  };

  for (int i = threadIdx.x; i < (r1 - r0) * kHIdx; i += 256) w_s[i] = w[(int64_t)r0 * kHIdx + i];
  __syncthreads();

  int seq_cur = -1;
  int nsend256 = 0;  // rows that took the barrier-ended 256-token send (buffer parity)
  for (int r = r0; r < r1; ++r) {
    // query operands of the row: head n, code chunks g and 2 + g, and their exponents
    const uint8_t* qp = q_idx + ((int64_t)r * kHIdx + n) * kKeyBytes + 16 * g;
    const v4i q0 = *reinterpret_cast<const v4i*>(qp);
    const v4i q1 = *reinterpret_cast<const v4i*>(qp + 32);
    const uint32_t qe = *reinterpret_cast<const uint32_t*>(q_e8 + ((int64_t)r * kHIdx + n) * 4);
    const int seq = __builtin_amdgcn_readlane(rs_v, r - r0);
    const int ctx = __builtin_amdgcn_readlane(rl_v, r - r0);
    if (seq != seq_cur) {  // uniform
      int smax = ctx;
      for (int q = r + 1; q < r1 && __builtin_amdgcn_readlane(rs_v, q - r0) == seq; ++q) {
        const int c = __builtin_amdgcn_readlane(rl_v, q - r0);
        smax = c > smax ? c : smax;
      }
      if (smax > 0) load_keys(seq, smax);  // an empty run stores and sends nothing
      seq_cur = seq;
    }
    const int qe0 = (int)((qe >> (8 * g)) & 255u), qe1 = (int)((qe >> (8 * (2 + g))) & 255u);
    float wq[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(&w_s[(r - r0) * kHIdx + 8 * j + 4 * g]);
      wq[4 * j] = v.x;
      wq[4 * j + 1] = v.y;
      wq[4 * j + 2] = v.z;
      wq[4 * j + 3] = v.w;
    }
    float res[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v16f acc = {};
      acc = mfma_fp4(q0, kb[j][0], qe0, ke[j][0], acc);
      acc = mfma_fp4(q1, kb[j][1], qe1, ke[j][1], acc);
      float s = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s = fmaf(wq[rr], relu_bits(acc[rr]), s);
      s += xshflf<32>(s);
      res[j] = s;
    }
    const int t = tok0 + lane;
    const float sc = g ? res[1] : res[0];
    if (t < ctx) scores[(int64_t)r * ld + t] = sc;
    if (SEND && blockIdx.x * 256 < ctx) {  // uniform
      send_candidates<256>(sc, t < ctx, ctx, blockIdx.x * 256, r, tw, send_lds[nsend256 & 1]);
      nsend256 += cand_plan(ctx, 256).unit == 256 ? 1 : 0;
    }
  }
}

hipError_t launch_indexer_mxfp4_rows(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx,
                                     const uint8_t* q_e8, const float* w, int R, int G, float* scores, int64_t ld,
                                     const TopkWs* ws, hipStream_t stream) {
  int nx = (rm.max_ctx + 255) / 256;
  if (nx < 1) nx = 1;
  TopkWs tw = ws ? *ws : TopkWs{nullptr, nullptr, nullptr};
  const int send = (ws != nullptr && rm.max_ctx > kTopkFullRow) ? 1 : 0;
  dim3 grid(nx, (R + G - 1) / G);
  const bool p32 = cv.block_size >= kTileTok;
  if (send && p32)
    hipLaunchKernelGGL((indexer_mxfp4_rows_kernel<true, true>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_e8, w,
                       scores, ld, tw, R, G);
  else if (send)
    hipLaunchKernelGGL((indexer_mxfp4_rows_kernel<false, true>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_e8, w,
                       scores, ld, tw, R, G);
  else if (p32)
    hipLaunchKernelGGL((indexer_mxfp4_rows_kernel<true, false>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_e8, w,
                       scores, ld, tw, R, G);
  else
    hipLaunchKernelGGL((indexer_mxfp4_rows_kernel<false, false>), grid, dim3(256), 0, stream, cv, rm, q_idx, q_e8, w,
                       scores, ld, tw, R, G);
  return hipGetLastError();
}

hipError_t launch_indexer_mxfp4(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const uint8_t* q_e8,
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
      hipLaunchKernelGGL((indexer_mxfp4_kernel<true, true, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx,
                         rm.block_table, cv, rm, q_idx, q_e8, w, scores,
                         ld, tw);
    else if (send)
      hipLaunchKernelGGL((indexer_mxfp4_kernel<false, true, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx,
                         rm.block_table, cv, rm, q_idx, q_e8, w, scores,
                         ld, tw);
    else if (p32)
      hipLaunchKernelGGL((indexer_mxfp4_kernel<true, false, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx,
                         rm.block_table, cv, rm, q_idx, q_e8, w, scores,
                         ld, tw);
    else
      hipLaunchKernelGGL((indexer_mxfp4_kernel<false, false, E>), grid, dim3(NTI), 0, stream, rm.row_seq, rm.row_ctx,
                         rm.block_table, cv, rm, q_idx, q_e8, w, scores,
                         ld, tw);
  };
  if (R > 1)
    go(std::true_type{});
  else
    go(std::false_type{});
  return hipGetLastError();
}

}  // namespace dsa
