// Lightning-indexer scoring over the packed paged cache with MXFP4 index keys.
//
// Same score as the FP8 indexer, score[r][t] = sum_h w[r][h] * ReLU(q_h . k_t), with
// query and key in MXFP4 (vLLM "Day-0 support for Kimi K3.1 Pro", AMD section: MXFP4
// index keys scored with FP4 matrix instructions and fp32 accumulation; 68 B per
// token: 64 B of e2m1 codes, element 2i in the low nibble of byte i, and one E8M0
// exponent per 32 elements).
//
// Every value is e2m1 * 2^(E - 127); it converts exactly to bf16 with its block scale
// applied (v_cvt_scalef32_pk_bf16_fp4: a 2-bit mantissa times a power of two), so the
// per-block scales need no separate pass and the contraction runs on the same bf16
// MFMA chain as the FP8 path: products exact in fp32, fp32 accumulation. (The scaled
// FP4 MFMA would do the same work in one instruction, but gfx950's low-precision
// matrix instructions keep fewer bits in their internal sum than fp32.)
//
// The dot product's order of dims is free as long as query and key share it: in the
// 32x32x16 MFMA chain, step kk on wave half g covers dims [64 g + 8 kk, 64 g + 8 kk + 8),
// so each lane needs one contiguous 32-byte half of a key (two 16-byte LDS reads).
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

// 16-byte chunk c (of 4) of tile token tn sits at LDS byte tn*64 + 16*(c ^ (tn & 3)).
__device__ __forceinline__ int swz4(int tn, int c) { return tn * kKeyBytes + 16 * (c ^ (tn & 3)); }

// E8M0 exponent -> 2^(e - 127) as fp32 (e = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// Eight e2m1 codes (one dword, element 2i in the low nibble of byte i) times `scale`,
// exactly, as bf16.
__device__ __forceinline__ v8bf e2m1x8_to_bf16(uint32_t v, float scale) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
}  // namespace

// One workgroup = 4 waves = 256 consecutive tokens of one row; wave w owns tokens
// [64w, 64w + 64). PAGED32: block size >= 32, so a tile lies inside one page.
// SEND: also run stage 1 of the top-k on the fresh scores. EARLY: as for the FP8 kernel.
template <bool PAGED32, bool SEND, bool EARLY>
// Row-map pointers lead the argument list (preloaded in scalar registers), as for the
// FP8 kernel.
__global__ __launch_bounds__(256) void indexer_mxfp4_kernel(const int32_t* __restrict__ row_seq,
                                                            const int32_t* __restrict__ row_ctx,
                                                            const int32_t* __restrict__ block_table, CacheView cv,
                                                            RowMap rm, const uint8_t* __restrict__ q_idx,
                                                            const uint8_t* __restrict__ q_e8,
                                                            const float* __restrict__ w, float* __restrict__ scores,
                                                            int64_t ld, TopkWs tw) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][kTileBytes];
  __shared__ uint32_t send_lds[send_lds_words<256>()];
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
  const bool past = blockIdx.x * 256 >= ctx;  // whole workgroup
  if (EARLY && past) return;                  // no barrier reached
  ctx = ctx > 0 ? ctx : 1;
  const int tok0 = blockIdx.x * 256 + wid * 64;
  const int bs_mask = cv.block_size - 1;
  const int64_t sc_off = (int64_t)cv.block_size * kKeyBytes;  // E8M0 bytes follow the codes in a page

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

  // ---- query half (head n, dims [64 g, 64 g + 64)) with its two E8M0 exponents, and
  // the head weights (uniform: scalar loads), behind the key stream ----
  v4i qr[2];
  {
    const v4i* qp = reinterpret_cast<const v4i*>(q_idx + ((int64_t)r * kHIdx + n) * kKeyBytes + 32 * g);
    qr[0] = qp[0];
    qr[1] = qp[1];
  }
  const uint32_t qe = *reinterpret_cast<const uint32_t*>(q_e8 + ((int64_t)r * kHIdx + n) * 4);
  float W[kHIdx];
#pragma unroll
  for (int h = 0; h < kHIdx; ++h) W[h] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w[r * kHIdx + h])));

  // every load of the wave is in flight before anything waits on one
  __builtin_amdgcn_sched_barrier(0);
  if (!EARLY && past) return;  // whole workgroup, no barrier reached

  // step kk covers dims 64 g + 8 kk ..: dword kk of the lane's half, block 2 g + kk / 4
  v8bf qa[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qa[kk] = e2m1x8_to_bf16((uint32_t)qr[kk >> 2][kk & 3], e8m0_scale((qe >> (8 * (2 * g + (kk >> 2)))) & 255u));
  // accumulator element rr of lane (n, g) is head 8 (rr >> 2) + 4 g + (rr & 3)
  float wq[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) wq[rr] = g ? W[8 * (rr >> 2) + 4 + (rr & 3)] : W[8 * (rr >> 2) + (rr & 3)];

  // ---- per tile: swizzled LDS transpose, 8 bf16 MFMAs, ReLU + weighted head sum ----
  const int wpos = swz4(lane >> 2, lane & 3);  // this lane's chunk of each kilobyte (16 tokens)
  float res[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<v4i*>(&lds[wid][1024 * i + wpos]) = kv[j][i];
    v4i kr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) kr[i] = *reinterpret_cast<const v4i*>(&lds[wid][swz4(n, 2 * g + i)]);
    const float ks0 = e8m0_scale((es[j] >> (16 * g)) & 255u);      // block 2 g
    const float ks1 = e8m0_scale((es[j] >> (16 * g + 8)) & 255u);  // block 2 g + 1
    v16f acc = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const v8bf b = e2m1x8_to_bf16((uint32_t)kr[kk >> 2][kk & 3], kk < 4 ? ks0 : ks1);
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
  const float sc = g ? res[1] : res[0];
  if (t < ctx) scores[(int64_t)r * ld + t] = sc;
  if (SEND) send_candidates<256>(sc, t < ctx, ctx, blockIdx.x * 256, r, tw, send_lds);
}

hipError_t launch_indexer_mxfp4(const CacheView& cv, const RowMap& rm, const uint8_t* q_idx, const uint8_t* q_e8,
                                const float* w, int R, float* scores, int64_t ld, const TopkWs* ws,
                                hipStream_t stream) {
  int nx = (rm.max_ctx + 255) / 256;
  if (nx < 1) nx = 1;
  TopkWs tw = ws ? *ws : TopkWs{nullptr, nullptr, nullptr};
  const int send = (ws != nullptr && rm.max_ctx > kTopkFullRow) ? 1 : 0;
  dim3 grid(nx, R);
  const bool p32 = cv.block_size >= kTileTok;
  auto go = [&](auto early) {
    constexpr bool E = decltype(early)::value;
    if (send && p32)
      hipLaunchKernelGGL((indexer_mxfp4_kernel<true, true, E>), grid, dim3(256), 0, stream, rm.row_seq, rm.row_ctx,
                         rm.block_table, cv, rm, q_idx, q_e8, w, scores,
                         ld, tw);
    else if (send)
      hipLaunchKernelGGL((indexer_mxfp4_kernel<false, true, E>), grid, dim3(256), 0, stream, rm.row_seq, rm.row_ctx,
                         rm.block_table, cv, rm, q_idx, q_e8, w, scores,
                         ld, tw);
    else if (p32)
      hipLaunchKernelGGL((indexer_mxfp4_kernel<true, false, E>), grid, dim3(256), 0, stream, rm.row_seq, rm.row_ctx,
                         rm.block_table, cv, rm, q_idx, q_e8, w, scores,
                         ld, tw);
    else
      hipLaunchKernelGGL((indexer_mxfp4_kernel<false, false, E>), grid, dim3(256), 0, stream, rm.row_seq, rm.row_ctx,
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
