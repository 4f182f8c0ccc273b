// Sparse MLA: exact attention of 96 latent-query heads over the selected tokens,
// reading each selected token's FP8 latent straight from the packed paged cache.
//
// vLLM "Day-0 support for Kimi K3.1 Pro", section "Sparse attention in K3.1 Pro":
// MLA runs exactly, but only over the kept tokens; the AMD section's sparse MLA
// reads selected tokens directly from the FP8 KV cache and, for small batches,
// adds parallelism inside a query row. Absorbed queries live in the 576-wide
// latent space (keys = all 576 dims, values = first 512; page 3 model table: NoPE).
//
// Grid (split, row, head group of G = 16 or 32 heads). A workgroup walks its split's
// slice of the row's index list 64 tokens at a time (the steps below are for G = 16;
// G = 32 computes two blocks of 16 heads from each converted latent fragment, and
// takes 4 heads per wave in the softmax and 32x32x16 MFMAs for O):
//   the chunk's token ids / page slots are the head of a load chain (ids -> latent
//   rows), so they are fetched first; the 64 latents (576 e4m3 bytes each) of chunk
//   c + 1 are loaded into registers while chunk c is computed (the ids of c + 2
//   behind them) and go to LDS once chunk c is done with it;
//   S = Q . C^T on 16x16x32 bf16 MFMAs (8 waves, each 16 tokens x 16 heads over one
//   half of the 576 dims, so a wave holds 9 query fragments), the two halves' scaled
//   logits (log2 domain) to LDS;
//   the online softmax of the chunk adds the halves and is split across the waves
//   (each owns 2 heads and keeps their running max / sum), and P'' and the heads'
//   rescale factors pass through LDS to every wave;
//   P'' = p * scale_t / (largest scale in the chunk), in [0, 1], as fp16 straight
//   into the MFMA operand registers;
//   O += P'' . codes on 16x16x32 fp16 MFMAs (each wave: 64 of the 512 value
//   columns); e4m3 codes are exact in fp16, and fp16 P keeps 11 significant bits
//   (bf16's 8 were visibly too few on rows dominated by a handful of tokens).
//   The chunk's scale factor joins the per-head softmax rescale.
// e4m3 codes convert to bf16 exactly; the per-token scale is applied to the
// logit and folded into P'. With one split the workgroup writes out / lse; with
// several it writes its split's softmax average O / l in fp16 and (m, l) in fp32,
// which the merge kernel combines by log-sum-exp.
// Sixteen heads per workgroup spread a row over twice as many CUs and keep the FP8
// kernel at 128 registers (two workgroups per CU): the choice for batches of up to 4
// rows. Larger batches fill the GPU anyway and take 32, which gathers each latent and
// reads the value tile once per 32 heads instead of once per 16.
//
// NVFP4 latents (page 1, KV-cache section: 352 B per token; the record holds the 512
// value dims as e2m1 codes with one e4m3 scale per 16 dims and the last 64 dims as
// e4m3 codes). The gather dequantises each record to fp16 on its way to LDS: the
// e2m1 pair conversion applies the power-of-two part of the block scale, one packed
// fp16 multiply its 4-bit significand; e2m1 times an e4m3 scale has at most 6
// significant bits and stays inside fp16's normal range, so the tile is exact. QK
// then runs on fp16 MFMAs too: each head's query is scaled by a power of two that
// puts its largest element in [2^14, 2^15) and rounded to fp16, exact for every
// element within 2^28 of that largest one (8-bit bf16 significands fit fp16's 11);
// the power of two returns in the logit. (Values below 2^-14 of the head's largest after
// the scaling would be fp16 subnormals; the pkrtz conversion truncates those, an error
// under 2^-38 of the largest element.) P . V reads 16-bit columns of the tile with
// the transposing LDS read (ds_read_b64_tr_b16). The tile's 16-byte chunks are
// XOR-swizzled within each token row (nv_col) so that the gather's writes do not
// collide in the LDS banks.
#include <type_traits>

#include "dsa.h"
#include "common.h"
#include "internal.h"
#include "topk_select.h"

namespace dsa {

namespace {
using v8h = v8hf;
constexpr int NT = 64;    // merge workgroup: one wave
constexpr int kMergeCols = 2;                         // adjacent value columns per merge lane
constexpr int kMergeParts = kDV / (kMergeCols * NT);  // merge workgroups per head
constexpr int NTM = 512;  // attention workgroup: 8 waves, two per SIMD
constexpr int NWM = NTM / 64;
constexpr int CH = kMlaChunk;           // 64 tokens per iteration
constexpr int PIECES = kDLat / 16;      // 36 16-byte pieces per latent
constexpr int QROW = kDLat + 8;         // Q staging row (bf16 elements), padded like the tiles
// LDS row of one token in the latent tile: FP8 codes (576 B) or, for NVFP4 records,
// dequantised fp16 (1,152 B); both padded by 16 B so that the 16 rows an MFMA fragment
// reads fall in distinct banks.
template <bool NV>
struct Tile {
  static constexpr int ROW = NV ? 2 * kDLat + 16 : kDLat + 16;
  static constexpr int BYTES = CH * ROW;  // Q passes through the same bytes first
  static_assert(32 * QROW * 2 <= BYTES, "Q staging (up to 32 heads) fits the latent tile");
};
constexpr int XROW = CH + 16;           // logit rows: the four 16-lane groups of a store hit distinct banks
constexpr int PROW = CH + 8;            // P'' rows (fp16), padded so the fragment reads spread over the banks
constexpr float kNegInf = -__builtin_huge_valf();

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Eight e2m1 codes (nibbles of d, element 2i in the low nibble of byte i) times a block
// scale p * m -> fp16, exact: the conversion applies the power of two p (it uses only
// the exponent of its scale operand), the packed multiply the significand m (m2 = {m, m};
// m = 0 for a zero scale).
__device__ __forceinline__ v8h e2m1x8_scaled_f16(uint32_t d, float p, v2h m2) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p, 0) * m2;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p, 1) * m2;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p, 2) * m2;
  const v2h e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, p, 3) * m2;
  v8h o;
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
  o[4] = c[0]; o[5] = c[1]; o[6] = e[0]; o[7] = e[1];
  return o;
}

// NVFP4 tile: byte offset of fp16 column `col` (a multiple of 4) in a token row. The
// 16-byte chunk index is XORed with its bits 3..5, so that the eight gather threads of
// a token, which write chunks 8 q8 + j for the same j, hit eight different bank groups;
// chunks 64.. (the tail dims) stay in place.
__device__ __forceinline__ int nv_col(int col) {
  const int c = col >> 3;
  return 16 * (c ^ ((c >> 3) & 7)) + 2 * (col & 7);
}

}  // namespace

// Where a workgroup reads the token ids and page slots of its split: the index and
// page-slot rows in global memory, or an LDS copy of the split's (token, page slot)
// entries (the fused select + attention kernel).
struct MlaIds {
  const int32_t* irow;  // index row (global), used when lds == nullptr
  const int32_t* prow;  // page-slot row (global) or nullptr
  const int2* lds;      // entries of list positions j0.. (LDS) or nullptr
  int j0;
  __device__ __forceinline__ bool slots() const { return lds != nullptr || prow != nullptr; }
  __device__ __forceinline__ void get(int j, int& t, int& ps) const {
    if (lds != nullptr) {
      const int2 e = lds[j - j0];
      t = e.x;
      ps = e.y;
    } else {
      t = irow[j];
      if (prow != nullptr) ps = prow[j];
    }
  }
};

constexpr int a16(int x) { return (x + 15) & ~15; }
// The attention workgroup's LDS, carved from one raw buffer (the fused kernel lays the
// select's LDS over the same bytes): the latent tile (Q passes through it first), the
// scaled logits (head-major, one array per half of the dims), the chunk's token
// scales, the NVFP4 query powers of two, the chunk's P'' (head-major), each head's
// rescale factor and running (max, sum), and the chunk's "some head's max moved" flag.
template <bool NV, int G>
struct MlaLds {
  static constexpr int LAT = 0;
  static constexpr int X = a16(LAT + Tile<NV>::BYTES);
  static constexpr int SC = a16(X + 2 * G * XROW * 4);
  static constexpr int QE = a16(SC + CH * 4);
  static constexpr int P = a16(QE + G * 4);
  static constexpr int AL = a16(P + G * PROW * 2);
  static constexpr int ML = a16(AL + G * 4);
  static constexpr int FL = a16(ML + G * 8);
  static constexpr int BYTES = a16(FL + 4);
};

constexpr int mla_qn(int G) { return (G * (kDLat / 8) + NTM - 1) / NTM; }  // 16-byte Q pieces per thread

// Q is read from HBM coalesced (rows of this head group are contiguous): thread tid
// takes pieces tid + NTM q of the group's G x 72 16-byte pieces.
template <int G>
__device__ __forceinline__ void mla_load_q(const uint16_t* __restrict__ q_lat, int r, int hg, v4i (&qv)[mla_qn(G)]) {
  constexpr int QALL = G * (kDLat / 8);
  const int tid = threadIdx.x;
  const v4i* qg = reinterpret_cast<const v4i*>(q_lat + ((int64_t)r * kHQ + hg * G) * kDLat);
#pragma unroll
  for (int q = 0; q < mla_qn(G); ++q)
    if (tid + NTM * q < QALL) qv[q] = qg[tid + NTM * q];
}

// One workgroup of NTM threads (the first NTM of a larger one in the fused kernel):
// split `split` (list positions [j0, j1)) of row r for head group hg. (t_n, ps_n) is
// the first chunk's gather token of this thread, already fetched from `src`; qv its Q
// pieces (mla_load_q).
template <bool NV, int G>
__device__ __forceinline__ void mla_body(const MlaIds& src, int t_n, int ps_n, const v4i (&qv)[mla_qn(G)], int j0,
                                         int j1, float c2, const CacheView& cv, const RowMap& rm, int r, int hg,
                                         int split, float* __restrict__ out, float* __restrict__ lse,
                                         _Float16* __restrict__ part_o, float* __restrict__ part_ml, int nsplit,
                                         uint8_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  using L = MlaLds<NV, G>;
  constexpr int LROW = Tile<NV>::ROW;
  uint8_t* lat_s = smem + L::LAT;
  float* x_s = reinterpret_cast<float*>(smem + L::X);
  float* sc_s = reinterpret_cast<float*>(smem + L::SC);
  float* qe_s = reinterpret_cast<float*>(smem + L::QE);
  _Float16* p_s = reinterpret_cast<_Float16*>(smem + L::P);
  float* al_s = reinterpret_cast<float*>(smem + L::AL);
  float2* ml_s = reinterpret_cast<float2*>(smem + L::ML);
  uint32_t* fl_s = reinterpret_cast<uint32_t*>(smem + L::FL);
  // gather: 8 threads per token. FP8: 16-byte pieces q8 + 8 q (q < 5) of 36. NVFP4: code
  // bytes [32 q8, +32) (dims [64 q8, +64)), their 4 block scales and, for q8 < 4, tail
  // bytes [16 q8, +16) (dims 512 + 16 q8 ..)
  const int tt_g = tid >> 3, q8 = tid & 7;
  // Q stays in registers for the whole workgroup: wave w holds the MFMA A fragments of
  // heads [16 (w >> 2), +16) over all 576 dims (lane: head lane & 15, dims 32 kk +
  // 8 (lane >> 4) ..+8). Q passes through the latent tile's LDS bytes, which the first
  // chunk's latents overwrite after a barrier.
  const int hrow = lane & 15, kq = 8 * (lane >> 4);
  // QK tile of this wave: tokens 16 tg.., all heads (G = 32: two blocks of 16), dims
  // 288 wq ..; each latent fragment is converted once and feeds every head block
  const int tg = wid & 3, wq = wid >> 2;
  constexpr int KH = kDLat / 64;  // steps of 32 dims per half
  constexpr int KQ = G / 16 * KH;  // query fragments: head block kk / KH, step kk % KH
  constexpr int QP = kDLat / 8;           // 72 16-byte pieces per head row
  constexpr int QALL = G * QP;
  constexpr int QN = mla_qn(G);
  // The row's block-table row is needed only without page slots.
  const int seq = src.slots() ? 0 : rm.row_seq[r];
  const int bs_mask = cv.block_size - 1;
  v8bf qa[KQ];
  v8h qh[KQ];  // NVFP4: the same fragments in fp16, scaled by a power of two per head

  // running softmax state of the head this lane's wave owns (G = 16: head
  // 2 wid + (lane >> 5); G = 32: head 4 wid + (lane >> 4))
  float m_run = kNegInf, l_run = 0.f;
  if (tid < G) ml_s[tid] = float2{kNegInf, 0.f};  // ordered by the staging barriers below
  // O accumulators. G = 16: value columns 64 wid + 16 cb + (lane & 15), heads
  // 4 (lane >> 4) + i. G = 32: columns 64 wid + 32 c + (lane & 31), row rr = head
  // 8 (rr >> 2) + 4 (lane >> 5) + (rr & 3).
  v4f acc[4];
  v16f accw[2];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 2; ++c) accw[c] = v16f{};
  // acc holds O / s_run: the token scales are folded into P'' relative to s_run, the
  // largest token scale so far (1 before the first chunk), so that acc needs rescaling only
  // in the chunks where that maximum or some head's running logit maximum moves
  float s_run = 1.f;
  float s_max = 0.f;

  // ---- gather, software-pipelined: the latents of chunk c + 1 are loaded into
  // registers (each thread up to 5 of its token's 36 16-byte pieces, and the scale)
  // while chunk c is computed, and the ids of chunk c + 2 behind them ----
  constexpr int PN = (PIECES + 7) / 8;  // 5 pieces per thread, the last on q8 < 4
  v4i v[PN];
  uint32_t nbs = 0;  // NVFP4: the four block-scale codes of this thread's dims
  float sv = 0.f;
  bool tv = false;  // the gathered slot holds a token
  auto issue = [&]() {
    if (t_n >= rm.max_ctx) raise_status(cv.status, kStIndexRange);
    const int t = t_n < rm.max_ctx ? t_n : -1;
    const int tc = t >= 0 ? t : 0;  // every load below stays in the pool; empty slots are masked
    int64_t blk;
    int slot;
    if (src.slots()) {
      const int ps = ps_n >= 0 ? ps_n : 0;
      blk = (int64_t)ps >> cv.log2_bs;
      blk = blk < cv.num_blocks ? blk : cv.num_blocks - 1;
      slot = ps & bs_mask;
    } else {
      blk = token_block(cv, rm, seq, tc);
      slot = tc & bs_mask;
    }
    const uint8_t* page = cv.pool + blk * cv.row_bytes + cv.lat_off;
    if constexpr (NV) {
      const uint8_t* rec = page + (int64_t)slot * kNvRec;
      if (q8 == 0) sv = *reinterpret_cast<const float*>(page + (int64_t)cv.block_size * kNvRec + (int64_t)slot * 4);
      v[0] = *reinterpret_cast<const v4i*>(rec + 32 * q8);
      v[1] = *reinterpret_cast<const v4i*>(rec + 32 * q8 + 16);
      nbs = *reinterpret_cast<const uint32_t*>(rec + kDV / 2 + 4 * q8);
      if (q8 < 4) v[2] = *reinterpret_cast<const v4i*>(rec + kDV / 2 + kDV / 16 + 16 * q8);
    } else {
      const uint8_t* lrow = page + (int64_t)slot * kDLat;
      if (q8 == 0) sv = *reinterpret_cast<const float*>(page + (int64_t)cv.block_size * kDLat + (int64_t)slot * 4);
#pragma unroll
      for (int q = 0; q < PN; ++q)
        if (q8 + 8 * q < PIECES) v[q] = *reinterpret_cast<const v4i*>(lrow + 16 * (q8 + 8 * q));
    }
    tv = t >= 0;
  };
  auto fetch_ids = [&](int c0) {
    const int j = c0 + tt_g;
    t_n = -1;
    if (j < j1) src.get(j, t_n, ps_n);
  };
  issue();
  fetch_ids(j0 + CH);
  {
    uint16_t* q_s = reinterpret_cast<uint16_t*>(lat_s);
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int i = tid + NTM * q, h = i / QP, pc = i - h * QP;
      if (i < QALL) *reinterpret_cast<v4i*>(q_s + h * QROW + pc * 8) = qv[q];
    }
    __syncthreads();
    if constexpr (NV) {
      // 16 threads per head (one wave holds 4 heads; the first 16 G threads):
      // each takes 36 consecutive dims of its head row, the 16 agree on the head's
      // largest magnitude, and each rewrites its 36 values in place as fp16 scaled by
      // the head's power of two
      const int h = tid >> 4, part = tid & 15;
      if (tid < 16 * G) {  // whole waves
      uint16_t* qp = q_s + h * QROW + 36 * part;
      uint2 raw[9];
#pragma unroll
      for (int i = 0; i < 9; ++i) raw[i] = *reinterpret_cast<const uint2*>(qp + 4 * i);
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        mx = fmaxf(mx, fabsf(__uint_as_float(raw[i].x << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(raw[i].x & 0xFFFF0000u)));
        mx = fmaxf(mx, fabsf(__uint_as_float(raw[i].y << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(raw[i].y & 0xFFFF0000u)));
      }
      mx = fmaxf(mx, xshflf<1>(mx));
      mx = fmaxf(mx, xshflf<2>(mx));
      mx = fmaxf(mx, xshflf<4>(mx));
      mx = fmaxf(mx, xshflf<8>(mx));
      int ex = mx > 0.f ? (int)((__float_as_uint(mx) >> 23) & 255u) - 127 - 14 : 0;
      ex = ex < -100 ? -100 : ex;
      const float down = __uint_as_float((uint32_t)(127 - ex) << 23);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        const v2h lo = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(raw[i].x << 16) * down,
                                                                         __uint_as_float(raw[i].x & 0xFFFF0000u) * down));
        const v2h hi = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(raw[i].y << 16) * down,
                                                                         __uint_as_float(raw[i].y & 0xFFFF0000u) * down));
        *reinterpret_cast<uint2*>(qp + 4 * i) = uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
      if (part == 0) qe_s[h] = __uint_as_float((uint32_t)(127 + ex) << 23);
      }
      __syncthreads();
      const uint16_t* qrow = q_s + hrow * QROW + kq + (kDLat / 2) * wq;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) qh[kk] = *reinterpret_cast<const v8h*>(qrow + 16 * (kk / KH) * QROW + 32 * (kk % KH));
    } else {
      const uint16_t* qrow = q_s + hrow * QROW + kq + (kDLat / 2) * wq;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) qa[kk] = *reinterpret_cast<const v8bf*>(qrow + 16 * (kk / KH) * QROW + 32 * (kk % KH));
    }
    __syncthreads();  // every wave holds its fragments before the latents overwrite them
  }

  for (int c0 = j0; c0 < j1; c0 += CH) {
    // LDS is free here: the previous chunk ended with a barrier
    if constexpr (NV) {
      uint8_t* trow = lat_s + tt_g * LROW;
      const v2f s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(nbs, 1.0f, false);
      const v2f s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(nbs, 1.0f, true);
      const float bsc[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          // block scale = p * m: p its power of two, m in [1, 2) its significand (0 if zero)
          const uint32_t sb = __float_as_uint(bsc[2 * i + hb]);
          const float p = sb ? __uint_as_float(sb & 0x7F800000u) : 1.f;
          const _Float16 m = sb ? (_Float16)__uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u) : (_Float16)0.f;
          const v2h m2 = {m, m};
#pragma unroll
          for (int w2 = 0; w2 < 2; ++w2) {
            const int w4 = 2 * hb + w2;
            const v8h o = tv ? e2m1x8_scaled_f16((uint32_t)v[i][w4], p, m2) : v8h{};
            *reinterpret_cast<v8h*>(trow + nv_col(64 * q8 + 32 * i + 8 * w4)) = o;
          }
        }
      if (q8 < 4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v8h o = tv ? e4m3x8_to_f16((uint32_t)v[2][2 * h], (uint32_t)v[2][2 * h + 1]) : v8h{};
          *reinterpret_cast<v8h*>(trow + nv_col(kDV + 16 * q8 + 8 * h)) = o;
        }
      }
    } else if (__ballot(!tv) == 0ull) {  // uniform: every slot of this wave holds a token
#pragma unroll
      for (int q = 0; q < PN; ++q)
        if (q8 + 8 * q < PIECES) *reinterpret_cast<v4i*>(lat_s + tt_g * LROW + 16 * (q8 + 8 * q)) = v[q];
    } else {  // an empty slot's codes (read at a clamped address) are zeroed: no NaN code reaches PV
#pragma unroll
      for (int q = 0; q < PN; ++q)
        if (q8 + 8 * q < PIECES)
          *reinterpret_cast<v4i*>(lat_s + tt_g * LROW + 16 * (q8 + 8 * q)) = tv ? v[q] : v4i{0, 0, 0, 0};
    }
    if (q8 == 0) sc_s[tt_g] = tv ? sv : kNegInf;  // -inf marks an empty slot
    if (tid == 0) *fl_s = 0u;  // the previous chunk's PV read it before its closing barrier
    __syncthreads();
    if (c0 + CH < j1) {  // uniform
      issue();
      fetch_ids(c0 + 2 * CH);
    }
    // largest token scale so far (this chunk's by every wave, then the running maximum;
    // token scales are non-negative, -inf marks an empty slot)
    float smax;
    {
      float v = sc_s[lane];
      v = fmaxf(v, xshflf<1>(v));
      v = fmaxf(v, xshflf<2>(v));
      v = fmaxf(v, xshflf<4>(v));
      v = fmaxf(v, xshflf<8>(v));
      v = fmaxf(v, xshflf<16>(v));
      v = fmaxf(v, xshflf<32>(v));
      s_max = fmaxf(s_max, v);
      smax = s_max > 0.f ? s_max : 1.f;
    }

    // ---- S = Q . C^T : wave w -> tokens [16 (w & 3), +16), all heads, dims
    // [288 (w >> 2), +288); each half's scaled logits (log2 domain) go to LDS and the
    // softmax adds the two ----
    {
      constexpr int NB = G / 16;  // head blocks
      v4f s0[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) s0[b] = v4f{0.f, 0.f, 0.f, 0.f};
      if constexpr (NV) {
        const uint8_t* lrow = lat_s + (16 * tg + hrow) * LROW;
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) {
          const v8h b = *reinterpret_cast<const v8h*>(lrow + nv_col(kq + (kDLat / 2) * wq + 32 * kk));
#pragma unroll
          for (int hb2 = 0; hb2 < NB; ++hb2)
            s0[hb2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[KH * hb2 + kk], b, s0[hb2], 0, 0, 0);
        }
      } else {
        const uint8_t* lrow = lat_s + (16 * tg + hrow) * LROW + kq + (kDLat / 2) * wq;
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) {
          uint2 raw = *reinterpret_cast<const uint2*>(lrow + 32 * kk);
          v8bf b = e4m3x8_to_bf16(raw.x, raw.y);
#pragma unroll
          for (int hb2 = 0; hb2 < NB; ++hb2)
            s0[hb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[KH * hb2 + kk], b, s0[hb2], 0, 0, 0);
        }
      }
      const int tt = 16 * tg + hrow;
      const float sct = sc_s[tt];
      const bool ok = sct != kNegInf;
      float* xh = x_s + wq * G * XROW;
#pragma unroll
      for (int hb2 = 0; hb2 < NB; ++hb2) {
        const int hb = 16 * hb2 + 4 * (lane >> 4);
        if constexpr (NV) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xh[(hb + i) * XROW + tt] = ok ? s0[hb2][i] * qe_s[hb + i] * (sct * c2) : kNegInf;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) xh[(hb + i) * XROW + tt] = ok ? s0[hb2][i] * (sct * c2) : kNegInf;
        }
      }
    }
    __syncthreads();

    if constexpr (G == 16) {
    // ---- softmax over the chunk, split across the waves: wave w owns heads 2w, 2w+1,
    // lane l head 2w + (l >> 5) and tokens 2 (l & 31) .. +2. P'' = p * scale_t / smax
    // (fp16, in [0, 1]) and each head's rescale factor go to LDS for every wave ----
    {
      const int h = 2 * wid + (lane >> 5), t2 = 2 * (lane & 31);
      const float2 xa = *reinterpret_cast<const float2*>(x_s + h * XROW + t2);
      const float2 xb = *reinterpret_cast<const float2*>(x_s + (G + h) * XROW + t2);
      const float2 s2 = *reinterpret_cast<const float2*>(sc_s + t2);
      const float xv[2] = {xa.x + xb.x, xa.y + xb.y};  // -inf for an empty slot in both halves
      const float sv[2] = {s2.x, s2.y};
      float cm = fmaxf(xv[0], xv[1]);
      cm = fmaxf(cm, xshflf<1>(cm));
      cm = fmaxf(cm, xshflf<2>(cm));
      cm = fmaxf(cm, xshflf<4>(cm));
      cm = fmaxf(cm, xshflf<8>(cm));
      cm = fmaxf(cm, xshflf<16>(cm));
      const float mn = fmaxf(m_run, cm);
      // 2^x by the hardware instruction (2^-inf = 0); mb keeps x from being -inf - -inf
      const float mb = mn == kNegInf ? 0.f : mn;
      const float alpha = mn == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - mb);
      const float inv_smax = __builtin_amdgcn_rcpf(smax);
      float psum = 0.f;
      v2h ph;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float p = __builtin_amdgcn_exp2f(xv[e] - mb);  // 0 for an empty slot
        psum += p;
        ph[e] = (_Float16)(p * (fmaxf(sv[e], 0.f) * inv_smax));
      }
      psum += xshflf<1>(psum);
      psum += xshflf<2>(psum);
      psum += xshflf<4>(psum);
      psum += xshflf<8>(psum);
      psum += xshflf<16>(psum);
      l_run = l_run * alpha + psum;
      m_run = mn;
      *reinterpret_cast<v2h*>(p_s + h * PROW + t2) = ph;
      if ((lane & 31) == 0) {
        al_s[h] = alpha;
        ml_s[h] = float2{m_run, l_run};
      }
    }
    } else {
    // ---- softmax over the chunk, split across the waves: wave w owns heads 4w .. 4w+3,
    // lane l head 4w + (l >> 4) and tokens 4 (l & 15) .. +4 ----
    {
      const int h = 4 * wid + (lane >> 4), t4 = 4 * (lane & 15);
      const float4 xa = *reinterpret_cast<const float4*>(x_s + h * XROW + t4);
      const float4 xb = *reinterpret_cast<const float4*>(x_s + (G + h) * XROW + t4);
      const float4 s4 = *reinterpret_cast<const float4*>(sc_s + t4);
      const float xv[4] = {xa.x + xb.x, xa.y + xb.y, xa.z + xb.z, xa.w + xb.w};  // -inf for an empty slot
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
      float cm = fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3]));
      cm = fmaxf(cm, xshflf<1>(cm));
      cm = fmaxf(cm, xshflf<2>(cm));
      cm = fmaxf(cm, xshflf<4>(cm));
      cm = fmaxf(cm, xshflf<8>(cm));
      const float mn = fmaxf(m_run, cm);
      const float mb = mn == kNegInf ? 0.f : mn;
      const float alpha = mn == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - mb);
      const float inv_smax = __builtin_amdgcn_rcpf(smax);
      float psum = 0.f;
      v4h ph;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(xv[e] - mb);  // 0 for an empty slot
        psum += p;
        ph[e] = (_Float16)(p * (fmaxf(sv[e], 0.f) * inv_smax));
      }
      psum += xshflf<1>(psum);
      psum += xshflf<2>(psum);
      psum += xshflf<4>(psum);
      psum += xshflf<8>(psum);
      l_run = l_run * alpha + psum;
      m_run = mn;
      *reinterpret_cast<v4h*>(p_s + h * PROW + t4) = ph;
      if ((lane & 15) == 0) {
        al_s[h] = alpha;
        ml_s[h] = float2{m_run, l_run};
        if (alpha != 1.f) *fl_s = 1u;
      }
    }
    }
    __syncthreads();
    // P'' fragments. G = 16 (16x16x32 A operand): row = head lane & 15, k = tokens
    // 32 ks + 8 (lane >> 4) .. +8. G = 32 (32x32x16): row = head lane & 31, k = tokens
    // 16 ks + 8 (lane >> 5) .. +8.
    v8h pa[G == 16 ? 2 : 4];
#pragma unroll
    for (int ks = 0; ks < (G == 16 ? 2 : 4); ++ks)
      pa[ks] = G == 16 ? *reinterpret_cast<const v8h*>(p_s + (lane & 15) * PROW + 32 * ks + 8 * (lane >> 4))
                       : *reinterpret_cast<const v8h*>(p_s + (lane & 31) * PROW + 16 * ks + 8 * (lane >> 5));

    // ---- acc = acc * alpha * (s_run / smax) + P'' . codes : wave w -> columns [64w, 64w+64) ----
    // G = 32 (long splits at batch): the multiplies only in chunks where some head's max or
    // the largest token scale moved, the factors being 1 exactly otherwise. (G = 16 runs few
    // chunks per split and is held to 128 registers, which the branch would exceed.)
    const float rescale = smax == s_run ? 1.f : s_run * __builtin_amdgcn_rcpf(smax);
    s_run = smax;
    const bool moved = G == 16 || __builtin_amdgcn_readfirstlane((int)*fl_s) != 0 ||
                       __builtin_amdgcn_readfirstlane(__float_as_int(rescale)) != __float_as_int(1.f);
    if (!moved) {
    } else if constexpr (G == 16) {
      const float4 a4 = *reinterpret_cast<const float4*>(&al_s[4 * (lane >> 4)]);
      const float a[4] = {a4.x * rescale, a4.y * rescale, a4.z * rescale, a4.w * rescale};
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[cb][i] *= a[i];
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 a4 = *reinterpret_cast<const float4*>(&al_s[8 * jj + 4 * (lane >> 5)]);
        const float a[4] = {a4.x * rescale, a4.y * rescale, a4.z * rescale, a4.w * rescale};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 2; ++c) accw[c][4 * jj + i] *= a[i];
      }
    }
    // B operand (16x16x32: codes of tokens 32 ks + 8 (lane >> 4) .. +8 at value column
    // 64 w + 16 cb + (lane & 15)) by one transposing LDS read: within each 16-lane group,
    // lane 8 a + c' receives byte c' of the 8-byte rows that lanes 2 j + a point at,
    // j = 0..7 (in token order). So lane l points at token row 8 (l >> 4) + ((l & 15) >> 1),
    // columns 8 (l & 1).
    // NVFP4 (fp16 tile): the 16-bit transposing read gives 4 values per lane: within each
    // 16-lane group, lane 4 a + c' receives element c' of the 8-byte rows that lanes
    // a + 4 j point at, j = 0..3 (in token order). So lane l points at token row
    // 8 (l >> 4) + ((l & 15) >> 2) (+4 for the second read), columns 4 (l & 3).
    if constexpr (G == 16) {
      if constexpr (NV) {
        const int tr_row = (8 * (lane >> 4) + ((lane & 15) >> 2)) * LROW;
        const int tr_col = 4 * (lane & 3);
  #pragma unroll
        for (int ks = 0; ks < CH / 32; ++ks) {
  #pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const uint8_t* vp = lat_s + 32 * ks * LROW + tr_row + nv_col(64 * wid + 16 * cb + tr_col);
            const v4h t0 = __builtin_bit_cast(
                v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vp)));
            const v4h t1 = __builtin_bit_cast(
                v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vp + 4 * LROW)));
            const v8h b = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[ks], b, acc[cb], 0, 0, 0);
          }
        }
      } else {
        const int tr_off = (8 * (lane >> 4) + ((lane & 15) >> 1)) * LROW + 8 * (lane & 1);
  #pragma unroll
        for (int ks = 0; ks < CH / 32; ++ks) {
  #pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const uint8_t* vp = lat_s + 32 * ks * LROW + 64 * wid + 16 * cb + tr_off;
            const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(vp));
            const v8h b = e4m3x8_to_f16((uint32_t)t.x, (uint32_t)t.y);
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[ks], b, acc[cb], 0, 0, 0);
          }
        }
      }
    } else {
      if constexpr (NV) {
        const int tr_row = (8 * (lane >> 5) + ((lane & 15) >> 2)) * LROW;
        const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  #pragma unroll
        for (int ks = 0; ks < CH / 16; ++ks) {
  #pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint8_t* vp = lat_s + 16 * ks * LROW + tr_row + nv_col(64 * wid + 32 * c + tr_col);
            const v4h t0 = __builtin_bit_cast(
                v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vp)));
            const v4h t1 = __builtin_bit_cast(
                v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vp + 4 * LROW)));
            const v8h b = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
            accw[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[ks], b, accw[c], 0, 0, 0);
          }
        }
      } else {
        const int tr_off = (8 * (lane >> 5) + ((lane & 15) >> 1)) * LROW + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  #pragma unroll
        for (int ks = 0; ks < CH / 16; ++ks) {
  #pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint8_t* vp = lat_s + 16 * ks * LROW + 64 * wid + 32 * c + tr_off;
            const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(vp));
            v8h b = e4m3x8_to_f16((uint32_t)t.x, (uint32_t)t.y);
            accw[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[ks], b, accw[c], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();  // lat_s, x_s, sc_s, p_s and al_s are rewritten by the next chunk
  }

  // ---- epilogue ----
  // (the loop's last barrier, or the staging barriers for a split with no tokens, has
  // ordered every head's final (max, sum) in ml_s)
  if (nsplit == 1) {
    if constexpr (G == 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * (lane >> 4) + i;
        const float lv = ml_s[h].y;
        const float f = lv > 0.f ? s_run / lv : 0.f;
        float* orow = out + ((int64_t)r * kHQ + hg * G + h) * kDV + 64 * wid + (lane & 15);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) orow[16 * cb] = acc[cb][i] * f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float lv = ml_s[h].y;
        const float f = lv > 0.f ? s_run / lv : 0.f;
        float* orow = out + ((int64_t)r * kHQ + hg * G + h) * kDV + 64 * wid + (lane & 31);
#pragma unroll
        for (int c = 0; c < 2; ++c) orow[32 * c] = accw[c][i] * f;
      }
    }
    if (lse != nullptr && tid < G) {
      const float2 ml = ml_s[tid];
      lse[(int64_t)r * kHQ + hg * G + tid] = ml.y > 0.f ? (ml.x + log2f(ml.y)) * 0.69314718055994531f : kNegInf;
    }
  } else {
    // The split's own softmax average O / l (bounded by the latents' magnitude) in fp16:
    // half the bytes of fp32 partials, 11 significant bits; (m, l) stay fp32.
    const int64_t pbase = ((int64_t)r * nsplit + split) * kHQ + hg * G;
    if constexpr (G == 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * (lane >> 4) + i;
        const float lv = ml_s[h].y;
        const float f = lv > 0.f ? s_run / lv : 0.f;
        _Float16* orow = part_o + (pbase + h) * kDV + 64 * wid + (lane & 15);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) __builtin_nontemporal_store((_Float16)(acc[cb][i] * f), orow + 16 * cb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float lv = ml_s[h].y;
        const float f = lv > 0.f ? s_run / lv : 0.f;
        _Float16* orow = part_o + (pbase + h) * kDV + 64 * wid + (lane & 31);
#pragma unroll
        for (int c = 0; c < 2; ++c) __builtin_nontemporal_store((_Float16)(accw[c][i] * f), orow + 32 * c);
      }
    }
    if (tid < G) {
      const float2 ml = ml_s[tid];
      part_ml[(pbase + tid) * 2 + 0] = ml.x;
      part_ml[(pbase + tid) * 2 + 1] = ml.y;
    }
  }
}

// The index list, page slots and queries lead the argument list so that their
// addresses arrive preloaded in scalar registers (kernel-argument preloading covers
// leading scalar and pointer arguments, not structures): the head of the load chain
// needs no kernel-argument fetch before it.
template <bool NV, int G>
__global__ __launch_bounds__(NTM) void sparse_mla_kernel(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ phys,
                                                        const uint16_t* __restrict__ q_lat, int k, int ts, float c2,
                                                        CacheView cv, RowMap rm,
                                                        float* __restrict__ out, float* __restrict__ lse,
                                                        _Float16* __restrict__ part_o, float* __restrict__ part_ml,
                                                        int nsplit) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MlaLds<NV, G>::BYTES];
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int j0 = split * ts;
  const int j1 = (j0 + ts < k) ? j0 + ts : k;
  const MlaIds src{idx + (int64_t)r * k, phys != nullptr ? phys + (int64_t)r * k : nullptr, nullptr, j0};
  // token id and page slot of this thread's gather token: the head of the load chain,
  // issued before anything else
  int t_n = -1, ps_n = 0;
  {
    const int j = j0 + ((int)threadIdx.x >> 3);
    if (j < j1) src.get(j, t_n, ps_n);
  }
  v4i qv[mla_qn(G)];
  mla_load_q<G>(q_lat, r, hg, qv);
  // only now the loads that need the structure arguments (fetched from memory, unlike
  // the leading pointers): the id and query loads above go out without waiting for them
  __builtin_amdgcn_sched_barrier(0);
  mla_body<NV, G>(src, t_n, ps_n, qv, j0, j1, c2, cv, rm, r, hg, split, out, lse, part_o, part_ml, nsplit, smem);
}

// The select and the attention in one launch (batches of up to 4 rows, FP8 latents,
// 16 heads per workgroup). Every workgroup of a row runs the row's select itself on
// all SEL_NT threads (the same exact computation as the select kernel, so all of them
// reach the same list), keeps the selection in LDS, and its first NTM threads attend
// over their split of it: the list and the page slots never leave the CU, and the
// select's launch and the attention's id loads drop out of the step. The workgroups of
// head group 0 write the row's index output, each its split's positions. The select's
// LDS and the attention's share the same bytes; the split's (token, page slot) entries
// sit apart.
template <bool CAND>
__global__ __launch_bounds__(SEL_NT) void select_mla_kernel(const uint32_t* __restrict__ cand_hi,
                                                            const uint32_t* __restrict__ cand_lo,
                                                            const uint32_t* __restrict__ floors,
                                                            const float* __restrict__ scores, int64_t ld,
                                                            const int32_t* __restrict__ row_ctx, int max_ctx, int k,
                                                            int umax, int load_b, int32_t* __restrict__ idx,
                                                            const uint16_t* __restrict__ q_lat, int ts, float c2,
                                                            CacheView cv, RowMap rm, float* __restrict__ out,
                                                            float* __restrict__ lse, _Float16* __restrict__ part_o,
                                                            float* __restrict__ part_ml, int nsplit) {
  constexpr int G = 16;
  constexpr int SB = sizeof(SelShared) > (size_t)MlaLds<false, G>::BYTES ? (int)sizeof(SelShared)
                                                                          : MlaLds<false, G>::BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SB];
  __shared__ int2 ids_s[kMaxK];
  SelShared& S = *reinterpret_cast<SelShared*>(smem);
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x;
  v4i qv[mla_qn(G)];
  const int j0 = split * ts;
  const int j1 = (j0 + ts < k) ? j0 + ts : k;
  // the query goes out right behind the select's candidate loads
  select_row<CAND>(cand_hi, cand_lo, floors, scores, ld, row_ctx, max_ctx, k, umax, load_b, nullptr, nullptr, true, cv,
                   rm, r, S, [&] {
                     if (tid < NTM) mla_load_q<G>(q_lat, r, hg, qv);
                   });
  {
    // the split's list entries with their page slots (the block-table row staged by the
    // select when it fits, else read), -1 past the selection
    const uint32_t nsel = S.nsel;
    const bool btl = S.btl != 0u;
    const int seq = rm.row_seq[r];
    for (int j = j0 + tid; j < j1; j += SEL_NT) {
      const int t = (uint32_t)j < nsel ? (int)S.a.hist[j] : -1;
      int ps = -1;
      if (t >= 0)
        ps = btl ? S.bt[t >> cv.log2_bs] * cv.block_size + (t & (cv.block_size - 1)) : page_slot(cv, rm, seq, t);
      ids_s[j - j0] = int2{t, ps};
    }
    __syncthreads();  // the entries are in; the select's LDS is free for the attention
  }
  // the row's index output, each split's positions written by its head-group-0 workgroup
  if (hg == 0)
    for (int j = j0 + tid; j < j1; j += SEL_NT) idx[(int64_t)r * k + j] = ids_s[j - j0].x;
  if (tid >= NTM) return;  // whole waves: the attention runs on the first NTM threads
  const MlaIds src{nullptr, nullptr, ids_s, j0};
  int t_n = -1, ps_n = 0;
  {
    const int j = j0 + (tid >> 3);
    if (j < j1) src.get(j, t_n, ps_n);
  }
  mla_body<false, G>(src, t_n, ps_n, qv, j0, j1, c2, cv, rm, r, hg, split, out, lse, part_o, part_ml, nsplit, smem);
}

// out[r][h] = sum_s w_s A_s / sum_s w_s with w_s = 2^(m_s - M) l_s and A_s = O_s / l_s
// (the fp16 split averages); empty splits (m = -inf) weigh 0. One wave per (row, head,
// 128 value columns), so that the partials spread over several times as many CUs as
// heads: lane s reads split s's (m, l); each lane then loads its two adjacent columns of
// every split at once (one 32-bit word per split; splits past nsplit repeat the last one
// with weight 0), so the whole merge is one round of loads.
// MS: a power of two >= nsplit (the loads are unrolled over MS splits).
template <int MS>
__global__ __launch_bounds__(NT) void mla_merge_kernel(const _Float16* __restrict__ part_o,
                                                       const float* __restrict__ part_ml, int nsplit,
                                                       float* __restrict__ out, float* __restrict__ lse) {
  static_assert(MS <= 64 && MS <= kMaxK / kMlaChunk, "one split per lane");
  const int h = blockIdx.x / kMergeParts, q = blockIdx.x % kMergeParts, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + (int64_t)r * nsplit * kHQ + h;
  const float2 e = lane < nsplit ? ml[(int64_t)lane * kHQ] : float2{kNegInf, 0.f};
  const _Float16* po = part_o + ((int64_t)r * nsplit * kHQ + h) * kDV + kMergeCols * NT * q + kMergeCols * tid;
  v2h x[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const int sc = s < nsplit ? s : nsplit - 1;
    x[s] = *reinterpret_cast<const v2h*>(po + (int64_t)sc * kHQ * kDV);
  }
  float M = e.x;
  M = fmaxf(M, xshflf<1>(M));
  M = fmaxf(M, xshflf<2>(M));
  M = fmaxf(M, xshflf<4>(M));
  M = fmaxf(M, xshflf<8>(M));
  M = fmaxf(M, xshflf<16>(M));
  M = fmaxf(M, xshflf<32>(M));
  const float wgt = (e.x == kNegInf) ? 0.f : exp2f(e.x - M) * e.y;
  float L = wgt;
  L += xshflf<1>(L);
  L += xshflf<2>(L);
  L += xshflf<4>(L);
  L += xshflf<8>(L);
  L += xshflf<16>(L);
  L += xshflf<32>(L);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), s));
    o0 = fmaf(ws, (float)x[s][0], o0);
    o1 = fmaf(ws, (float)x[s][1], o1);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float2* orow = reinterpret_cast<float2*>(out + ((int64_t)r * kHQ + h) * kDV + kMergeCols * NT * q) + tid;
  *orow = float2{o0 * inv, o1 * inv};
  if (lse != nullptr && q == 0 && tid == 0)
    lse[(int64_t)r * kHQ + h] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : kNegInf;
}

// ---- 32 heads on four waves: grids of more workgroups than CUs, FP8 latents ----
// The body above keeps one 512-thread workgroup per CU (its 32-head registers), and its
// four barrier-separated phases per chunk (latents in, QK, softmax, PV) leave both waves
// of a SIMD in the same phase, so the matrix cores and the vector ALUs rarely work at
// once. Here a workgroup is four waves (one per SIMD) over 32-token chunks, held to 256
// registers, so that two workgroups share each CU and drift apart: one's softmax and
// format conversions overlap the other's MFMAs. Per chunk: 8 threads gather each of the 32
// latents; wave w computes S for tokens [16 (w & 1), +16) over dims [288 (w >> 1), +288)
// for both blocks of 16 heads; the softmax gives wave w heads 8w .. 8w + 7 (lane: head
// 8w + (lane >> 3), 4 tokens); PV gives wave w value columns [128 w, +128). The numerics
// are those of the 512-thread body (bf16 QK, fp16 P'' relative to the running largest
// token scale, fp16 PV on e4m3 codes, fp16 split averages). It pays where the grid holds
// more than one workgroup per CU (2,048 rows of a prefill-append: attention 1.82 -> 1.55
// ms; 32 to 128 decode rows with its own split count: 5 to 12 % less); where the
// 512-thread body's grid fits one round (up to about 28 rows) that body is faster, since a
// four-wave workgroup alone on a CU has one wave per SIMD. The split-count plan
// chooses between the two.
namespace {
constexpr int NT4 = 256;
constexpr int C2 = 32;             // tokens per chunk
constexpr int XROW2 = C2 + 16;     // logit rows
constexpr int PROW2 = C2 + 8;      // P'' rows (fp16)
constexpr int LROW4 = kDLat + 16;  // latent tile row (e4m3 codes, padded)
constexpr int QN4 = (32 * (kDLat / 8) + NT4 - 1) / NT4;  // 16-byte Q pieces per thread
struct MlaLds4 {
  static constexpr int LAT = 0;    // the latent tile; Q passes through it first
  static constexpr int LATB = C2 * LROW4 > 32 * QROW * 2 ? C2 * LROW4 : 32 * QROW * 2;
  static constexpr int X = a16(LAT + LATB);
  static constexpr int SC = a16(X + 2 * 32 * XROW2 * 4);
  static constexpr int P = a16(SC + C2 * 4);
  static constexpr int AL = a16(P + 32 * PROW2 * 2);
  static constexpr int ML = a16(AL + 32 * 4);
  static constexpr int FL = a16(ML + 32 * 8);
  static constexpr int BYTES = a16(FL + 4);
};
}  // namespace

__device__ __forceinline__ void mla_body_w4(const MlaIds& src, int t_n, int ps_n, const v4i (&qv)[QN4], int j0,
                                            int j1, float c2, const CacheView& cv, const RowMap& rm, int r, int hg,
                                            int split, float* __restrict__ out, float* __restrict__ lse,
                                            _Float16* __restrict__ part_o, float* __restrict__ part_ml, int nsplit,
                                            uint8_t* smem) {
  constexpr int G = 32;
  using L = MlaLds4;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint8_t* lat_s = smem + L::LAT;
  float* x_s = reinterpret_cast<float*>(smem + L::X);
  float* sc_s = reinterpret_cast<float*>(smem + L::SC);
  _Float16* p_s = reinterpret_cast<_Float16*>(smem + L::P);
  float* al_s = reinterpret_cast<float*>(smem + L::AL);
  float2* ml_s = reinterpret_cast<float2*>(smem + L::ML);
  uint32_t* fl_s = reinterpret_cast<uint32_t*>(smem + L::FL);
  const int tt_g = tid >> 3, q8 = tid & 7;  // gather: token tt_g, 16-byte pieces q8 + 8 q
  const int hrow = lane & 15, kq = 8 * (lane >> 4);
  const int tg = wid & 1, wq = wid >> 1;    // QK: tokens [16 tg, +16), dims [288 wq, +288)
  constexpr int KH = kDLat / 64;
  constexpr int KQ = 2 * KH;
  constexpr int QP = kDLat / 8;
  const int seq = src.slots() ? 0 : rm.row_seq[r];
  const int bs_mask = cv.block_size - 1;
  v8bf qa[KQ];
  float m_run = kNegInf, l_run = 0.f;  // softmax state of head 8 wid + (lane >> 3)
  if (tid < G) ml_s[tid] = float2{kNegInf, 0.f};
  // O: value columns 128 wid + 32 c + (lane & 31), row rr = head 8 (rr >> 2) + 4 (lane >> 5) + (rr & 3)
  v16f accw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) accw[c] = v16f{};
  float s_run = 1.f, s_max = 0.f;  // acc holds O / s_run; s_max: largest token scale so far

  constexpr int PN = (PIECES + 7) / 8;
  v4i v[PN];
  float sv = 0.f;
  bool tv = false;
  auto issue = [&]() {
    if (t_n >= rm.max_ctx) raise_status(cv.status, kStIndexRange);
    const int t = t_n < rm.max_ctx ? t_n : -1;
    const int tc = t >= 0 ? t : 0;  // every load stays in the pool; empty slots are masked
    int64_t blk;
    int slot;
    if (src.slots()) {
      const int ps = ps_n >= 0 ? ps_n : 0;
      blk = (int64_t)ps >> cv.log2_bs;
      blk = blk < cv.num_blocks ? blk : cv.num_blocks - 1;
      slot = ps & bs_mask;
    } else {
      blk = token_block(cv, rm, seq, tc);
      slot = tc & bs_mask;
    }
    const uint8_t* page = cv.pool + blk * cv.row_bytes + cv.lat_off;
    const uint8_t* lrow = page + (int64_t)slot * kDLat;
    if (q8 == 0) sv = *reinterpret_cast<const float*>(page + (int64_t)cv.block_size * kDLat + (int64_t)slot * 4);
#pragma unroll
    for (int q = 0; q < PN; ++q)
      if (q8 + 8 * q < PIECES) v[q] = *reinterpret_cast<const v4i*>(lrow + 16 * (q8 + 8 * q));
    tv = t >= 0;
  };
  auto fetch_ids = [&](int c0) {
    const int j = c0 + tt_g;
    t_n = -1;
    if (j < j1) src.get(j, t_n, ps_n);
  };
  issue();
  fetch_ids(j0 + C2);
  {
    uint16_t* q_s = reinterpret_cast<uint16_t*>(lat_s);
#pragma unroll
    for (int q = 0; q < QN4; ++q) {
      const int i = tid + NT4 * q, h = i / QP, pc = i - h * QP;
      if (i < G * QP) *reinterpret_cast<v4i*>(q_s + h * QROW + pc * 8) = qv[q];
    }
    __syncthreads();
    const uint16_t* qrow = q_s + hrow * QROW + kq + (kDLat / 2) * wq;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) qa[kk] = *reinterpret_cast<const v8bf*>(qrow + 16 * (kk / KH) * QROW + 32 * (kk % KH));
    __syncthreads();  // every wave holds its fragments before the latents overwrite them
  }

  for (int c0 = j0; c0 < j1; c0 += C2) {
    if (__ballot(!tv) == 0ull) {  // uniform: every slot of this wave holds a token
#pragma unroll
      for (int q = 0; q < PN; ++q)
        if (q8 + 8 * q < PIECES) *reinterpret_cast<v4i*>(lat_s + tt_g * LROW4 + 16 * (q8 + 8 * q)) = v[q];
    } else {  // an empty slot's codes (read at a clamped address) are zeroed
#pragma unroll
      for (int q = 0; q < PN; ++q)
        if (q8 + 8 * q < PIECES)
          *reinterpret_cast<v4i*>(lat_s + tt_g * LROW4 + 16 * (q8 + 8 * q)) = tv ? v[q] : v4i{0, 0, 0, 0};
    }
    if (q8 == 0) sc_s[tt_g] = tv ? sv : kNegInf;  // -inf marks an empty slot
    if (tid == 0) *fl_s = 0u;
    __syncthreads();
    if (c0 + C2 < j1) {  // uniform
      issue();
      fetch_ids(c0 + 2 * C2);
    }
    float smax;
    {
      float x = lane < C2 ? sc_s[lane] : kNegInf;
      x = fmaxf(x, xshflf<1>(x));
      x = fmaxf(x, xshflf<2>(x));
      x = fmaxf(x, xshflf<4>(x));
      x = fmaxf(x, xshflf<8>(x));
      x = fmaxf(x, xshflf<16>(x));
      x = fmaxf(x, xshflf<32>(x));
      s_max = fmaxf(s_max, x);
      smax = s_max > 0.f ? s_max : 1.f;
    }
    // ---- S = Q . C^T (both head blocks from each converted latent fragment) ----
    {
      v4f s0[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
      const uint8_t* lrow = lat_s + (16 * tg + hrow) * LROW4 + kq + (kDLat / 2) * wq;
#pragma unroll
      for (int kk = 0; kk < KH; ++kk) {
        const uint2 raw = *reinterpret_cast<const uint2*>(lrow + 32 * kk);
        const v8bf b = e4m3x8_to_bf16(raw.x, raw.y);
#pragma unroll
        for (int hb2 = 0; hb2 < 2; ++hb2)
          s0[hb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[KH * hb2 + kk], b, s0[hb2], 0, 0, 0);
      }
      const int tt = 16 * tg + hrow;
      const float sct = sc_s[tt];
      const bool ok = sct != kNegInf;
      float* xh = x_s + wq * G * XROW2;
#pragma unroll
      for (int hb2 = 0; hb2 < 2; ++hb2) {
        const int hb = 16 * hb2 + 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) xh[(hb + i) * XROW2 + tt] = ok ? s0[hb2][i] * (sct * c2) : kNegInf;
      }
    }
    __syncthreads();
    // ---- softmax: wave w owns heads 8w .. 8w + 7, lane l head 8w + (l >> 3), tokens 4 (l & 7) .. +4 ----
    {
      const int h = 8 * wid + (lane >> 3), t4 = 4 * (lane & 7);
      const float4 xa = *reinterpret_cast<const float4*>(x_s + h * XROW2 + t4);
      const float4 xb = *reinterpret_cast<const float4*>(x_s + (G + h) * XROW2 + t4);
      const float4 s4 = *reinterpret_cast<const float4*>(sc_s + t4);
      const float xv[4] = {xa.x + xb.x, xa.y + xb.y, xa.z + xb.z, xa.w + xb.w};  // -inf for an empty slot
      const float svv[4] = {s4.x, s4.y, s4.z, s4.w};
      float cm = fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3]));
      cm = fmaxf(cm, xshflf<1>(cm));
      cm = fmaxf(cm, xshflf<2>(cm));
      cm = fmaxf(cm, xshflf<4>(cm));
      const float mn = fmaxf(m_run, cm);
      const float mb = mn == kNegInf ? 0.f : mn;
      const float alpha = mn == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - mb);
      const float inv_smax = __builtin_amdgcn_rcpf(smax);
      float psum = 0.f;
      v4h ph;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(xv[e] - mb);  // 0 for an empty slot
        psum += p;
        ph[e] = (_Float16)(p * (fmaxf(svv[e], 0.f) * inv_smax));
      }
      psum += xshflf<1>(psum);
      psum += xshflf<2>(psum);
      psum += xshflf<4>(psum);
      l_run = l_run * alpha + psum;
      m_run = mn;
      *reinterpret_cast<v4h*>(p_s + h * PROW2 + t4) = ph;
      if ((lane & 7) == 0) {
        al_s[h] = alpha;
        ml_s[h] = float2{m_run, l_run};
        if (alpha != 1.f) *fl_s = 1u;
      }
    }
    __syncthreads();
    // P'' fragments (32x32x16 A operand): row = head lane & 31, k = tokens 16 ks + 8 (lane >> 5) .. +8
    v8h pa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pa[ks] = *reinterpret_cast<const v8h*>(p_s + (lane & 31) * PROW2 + 16 * ks + 8 * (lane >> 5));
    // acc *= alpha * (s_run / smax) only in chunks where some head's max or the largest scale moved
    const float rescale = smax == s_run ? 1.f : s_run * __builtin_amdgcn_rcpf(smax);
    s_run = smax;
    const bool moved = __builtin_amdgcn_readfirstlane((int)*fl_s) != 0 ||
                       __builtin_amdgcn_readfirstlane(__float_as_int(rescale)) != __float_as_int(1.f);
    if (moved) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 a4 = *reinterpret_cast<const float4*>(&al_s[8 * jj + 4 * (lane >> 5)]);
        const float a[4] = {a4.x * rescale, a4.y * rescale, a4.z * rescale, a4.w * rescale};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) accw[c][4 * jj + i] *= a[i];
      }
    }
    // ---- O += P'' . codes: wave w -> value columns [128 w, +128); B operands by the
    // transposing LDS read (as in the 512-thread body) ----
    {
      const int tr_off = (8 * (lane >> 5) + ((lane & 15) >> 1)) * LROW4 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint8_t* vp = lat_s + 16 * ks * LROW4 + 128 * wid + 32 * c + tr_off;
          const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(vp));
          const v8h b = e4m3x8_to_f16((uint32_t)t.x, (uint32_t)t.y);
          accw[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[ks], b, accw[c], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // lat_s, x_s, sc_s, p_s, al_s and fl_s are rewritten by the next chunk
  }

  // ---- epilogue (the last barrier, or the staging barriers of an empty split, has ordered
  // every head's final (max, sum) in ml_s) ----
  if (nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      const float lv = ml_s[h].y;
      const float f = lv > 0.f ? s_run / lv : 0.f;
      float* orow = out + ((int64_t)r * kHQ + hg * G + h) * kDV + 128 * wid + (lane & 31);
#pragma unroll
      for (int c = 0; c < 4; ++c) orow[32 * c] = accw[c][i] * f;
    }
    if (lse != nullptr && tid < G) {
      const float2 ml = ml_s[tid];
      lse[(int64_t)r * kHQ + hg * G + tid] = ml.y > 0.f ? (ml.x + log2f(ml.y)) * 0.69314718055994531f : kNegInf;
    }
  } else {
    const int64_t pbase = ((int64_t)r * nsplit + split) * kHQ + hg * G;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      const float lv = ml_s[h].y;
      const float f = lv > 0.f ? s_run / lv : 0.f;
      _Float16* orow = part_o + (pbase + h) * kDV + 128 * wid + (lane & 31);
#pragma unroll
      for (int c = 0; c < 4; ++c) __builtin_nontemporal_store((_Float16)(accw[c][i] * f), orow + 32 * c);
    }
    if (tid < G) {
      const float2 ml = ml_s[tid];
      part_ml[(pbase + tid) * 2 + 0] = ml.x;
      part_ml[(pbase + tid) * 2 + 1] = ml.y;
    }
  }
}

// The 32-head, four-wave attention kernel (grid: split, row, head group of 32). Two
// workgroups per CU: at most 256 registers per lane.
__global__ __launch_bounds__(NT4, 2) void sparse_mla32_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ phys,
                                                            const uint16_t* __restrict__ q_lat, int k, int ts,
                                                            float c2, CacheView cv, RowMap rm, float* __restrict__ out,
                                                            float* __restrict__ lse, _Float16* __restrict__ part_o,
                                                            float* __restrict__ part_ml, int nsplit) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MlaLds4::BYTES];
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int j0 = split * ts;
  const int j1 = (j0 + ts < k) ? j0 + ts : k;
  const MlaIds src{idx + (int64_t)r * k, phys != nullptr ? phys + (int64_t)r * k : nullptr, nullptr, j0};
  int t_n = -1, ps_n = 0;
  {
    const int j = j0 + ((int)threadIdx.x >> 3);
    if (j < j1) src.get(j, t_n, ps_n);
  }
  v4i qv[QN4];
  {
    const int tid = threadIdx.x;
    const v4i* qg = reinterpret_cast<const v4i*>(q_lat + ((int64_t)r * kHQ + hg * 32) * kDLat);
#pragma unroll
    for (int q = 0; q < QN4; ++q)
      if (tid + NT4 * q < 32 * (kDLat / 8)) qv[q] = qg[tid + NT4 * q];
  }
  __builtin_amdgcn_sched_barrier(0);
  mla_body_w4(src, t_n, ps_n, qv, j0, j1, c2, cv, rm, r, hg, split, out, lse, part_o, part_ml, nsplit, smem);
}

bool select_mla_fused(const CacheView& cv, int R, int k) {
  if (cv.latent_fmt != DSA_LATENT_FP8 || R <= 0 || mla_group(R) != 16) return false;
  // one workgroup per CU (the select's LDS): the whole grid in one round
  return (int64_t)mla_plan(R, k, true).nsplit * R * (kHQ / 16) <= kSelMlaMaxGroups;
}

hipError_t launch_select_mla(const float* scores, int64_t ld, const int32_t* row_ctx, int R, int max_ctx, int k,
                             int umax, int32_t* idx, const TopkWs& tw, const CacheView& cv, const RowMap& rm,
                             const uint16_t* q_lat, float sm_scale, float* out, float* lse, void* ws,
                             hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const int nsplit = mla_plan(R, k, true).nsplit;  // up to 4 rows: the 16-head eight-wave kernel
  const int ts = mla_split_tokens(k, nsplit);
  const float c2 = (float)((double)sm_scale * 1.4426950408889634);
  _Float16* part_o = nullptr;
  float* part_ml = nullptr;
  if (nsplit > 1) {
    part_o = static_cast<_Float16*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_up((size_t)R * nsplit * kHQ * kDV * 2, 256));
  }
  const int load_b = cand_plan(max_ctx, umax).per == 16 ? 1 : 0;
  const dim3 grid(nsplit, R, kHQ / 16);
  if (max_ctx > kTopkFullRow)
    hipLaunchKernelGGL(select_mla_kernel<true>, grid, dim3(SEL_NT), 0, stream, tw.cand_hi, tw.cand_lo, tw.floors,
                       scores, ld, row_ctx, max_ctx, k, umax, load_b, idx, q_lat, ts, c2, cv, rm, out, lse, part_o,
                       part_ml, nsplit);
  else
    hipLaunchKernelGGL(select_mla_kernel<false>, grid, dim3(SEL_NT), 0, stream, tw.cand_hi, tw.cand_lo, tw.floors,
                       scores, ld, row_ctx, max_ctx, k, umax, 0, idx, q_lat, ts, c2, cv, rm, out, lse, part_o,
                       part_ml, nsplit);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const CacheView& cv, const RowMap& rm, const uint16_t* q_lat, const int32_t* idx,
                             const int32_t* phys, int R, int k, float sm_scale, float* out, float* lse, void* ws,
                             int parts, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const bool nvf = cv.latent_fmt == DSA_LATENT_NVFP4;
  const MlaPlan plan = mla_plan(R, k, !nvf);
  const int nsplit = plan.nsplit;
  const int ts = mla_split_tokens(k, nsplit);
  const float c2 = (float)((double)sm_scale * 1.4426950408889634);
  _Float16* part_o = nullptr;
  float* part_ml = nullptr;
  if (nsplit > 1) {
    part_o = static_cast<_Float16*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_up((size_t)R * nsplit * kHQ * kDV * 2, 256));
  }
  auto go = [&](auto nv, auto group) {
    constexpr bool N = decltype(nv)::value;
    constexpr int G = decltype(group)::value;
    hipLaunchKernelGGL((sparse_mla_kernel<N, G>), dim3(nsplit, R, kHQ / G), dim3(NTM), 0, stream, idx, phys, q_lat, k,
                       ts, c2, cv, rm, out, lse, part_o, part_ml, nsplit);
  };
  if (!(parts & 1)) {
  } else if (mla_group(R) == 16) {
    if (nvf)
      go(std::true_type{}, std::integral_constant<int, 16>{});
    else
      go(std::false_type{}, std::integral_constant<int, 16>{});
  } else if (nvf) {
    go(std::true_type{}, std::integral_constant<int, 32>{});
  } else if (plan.four_wave) {
    // more workgroups than CUs (e.g. a prefill-append's unsplit rows, or batches of 32
    // rows and up): the four-wave kernel, two workgroups per CU
    hipLaunchKernelGGL(sparse_mla32_kernel, dim3(nsplit, R, kHQ / 32), dim3(NT4), 0, stream, idx, phys, q_lat, k, ts,
                       c2, cv, rm, out, lse, part_o, part_ml, nsplit);
  } else {
    go(std::false_type{}, std::integral_constant<int, 32>{});
  }
  if (nsplit > 1 && (parts & 2)) {
    const dim3 mg(kHQ * kMergeParts, R);
    if (nsplit <= 4)
      hipLaunchKernelGGL(mla_merge_kernel<4>, mg, dim3(NT), 0, stream, part_o, part_ml, nsplit, out, lse);
    else if (nsplit <= 8)
      hipLaunchKernelGGL(mla_merge_kernel<8>, mg, dim3(NT), 0, stream, part_o, part_ml, nsplit, out, lse);
    else if (nsplit <= 16)
      hipLaunchKernelGGL(mla_merge_kernel<16>, mg, dim3(NT), 0, stream, part_o, part_ml, nsplit, out, lse);
    else
      hipLaunchKernelGGL(mla_merge_kernel<32>, mg, dim3(NT), 0, stream, part_o, part_ml, nsplit, out, lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
