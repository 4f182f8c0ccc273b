// Shared device-side definitions for the DSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kHIdx = 32;    // indexer heads
constexpr int kDIdx = 128;   // indexer head dim
constexpr int kHQ = 96;      // latent-query heads
constexpr int kDLat = 576;   // latent width
constexpr int kDV = 512;     // value width
constexpr int kMaxK = 2048;
constexpr int kNvRec = 352;  // NVFP4 latent record: 256 B e2m1 + 32 e4m3 block scales + 64 e4m3 tail
constexpr int kWave = 64;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// One layer's view of the packed cache, passed to kernels by value.
struct CacheView {
  const uint8_t* pool;
  int64_t row_bytes;
  int64_t num_blocks;
  int64_t lat_off;     // latent page offset inside a row
  int64_t idx_off;     // index page offset inside a row
  int32_t block_size;  // power of two
  int32_t log2_bs;
  int32_t latent_fmt;  // DSA_LATENT_FP8 / DSA_LATENT_NVFP4
  uint32_t* status;    // this device's status word (nullable)
};

// Query-row to cache mapping.
struct RowMap {
  const int32_t* block_table;
  const int32_t* row_seq;
  const int32_t* row_ctx;
  int32_t bt_stride;
  int32_t max_ctx;  // host bound, also <= bt_stride * block_size
};

// Bits of the device status word (the DSA_DEV_* values of the C header).
constexpr uint32_t kStCtxClamped = 1u;    // a row length above max_ctx was clamped
constexpr uint32_t kStBlockClamped = 2u;  // a block-table entry outside the pool was met
constexpr uint32_t kStIndexRange = 4u;    // sparse MLA skipped an index past the block table

// Sets `bit` in the status word (no-op without one). Called only on the branches that
// repair bad data, so good data never reaches the atomic.
__device__ __forceinline__ void raise_status(uint32_t* st, uint32_t bit) {
  if (st != nullptr) atomicOr(st, bit);
}

// Eligible length of row r, clamped to [0, max_ctx].
__device__ __forceinline__ int row_len(const RowMap& m, int r, uint32_t* st) {
  int c = m.row_ctx[r];
  c = c < 0 ? 0 : c;
  if (c > m.max_ctx) {
    raise_status(st, kStCtxClamped);
    c = m.max_ctx;
  }
  return c;
}

// Physical block of token t of the block-table row `seq`, clamped into the pool.
__device__ __forceinline__ int64_t token_block(const CacheView& cv, const RowMap& m, int seq, int t) {
  int64_t b = m.block_table[(int64_t)seq * m.bt_stride + (t >> cv.log2_bs)];
  if ((uint64_t)b >= (uint64_t)cv.num_blocks) {
    raise_status(cv.status, kStBlockClamped);
    b = b < 0 ? 0 : cv.num_blocks - 1;
  }
  return b;
}

// Byte address of a token's page inside its block row (page base of the given kind).
__device__ __forceinline__ const uint8_t* row_base(const CacheView& cv, int64_t blk) {
  return cv.pool + blk * cv.row_bytes;
}

// max(x, 0) as one integer max on the bit pattern: a float with the sign bit set is a
// negative int32 (-0 and negative values give +0), a positive float keeps its bits.
// (fmaxf would first canonicalise an MFMA result, a second instruction per value.)
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// fp32 -> order-preserving unsigned key (larger float -> larger key), -0.0 == +0.0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Selection order: larger score first, then smaller token index.
__device__ __forceinline__ uint64_t composite_key(float s, int t) {
  return ((uint64_t)float_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

// Four e4m3 codes (little-endian in a dword) -> four exact bf16 values.
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t x, v2bf& lo, v2bf& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
}

// Eight e4m3 codes -> v8bf (element j = byte j).
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t a, uint32_t b) {
  v2bf p0, p1, p2, p3;
  e4m3x4_to_bf16(a, p0, p1);
  e4m3x4_to_bf16(b, p2, p3);
  v8bf r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8hf __attribute__((ext_vector_type(8)));

// Eight e4m3 codes -> v8 fp16 (exact: every e4m3 value is an fp16 value).
__device__ __forceinline__ v8hf e4m3x8_to_f16(uint32_t a, uint32_t b) {
  v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false);
  v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true);
  v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
  v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true);
  v8hf r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// ---- cross-lane exchange without the LDS path --------------------------------------
// x ^ J partner within the 64-lane wave: DPP quad permutes / row mirrors for J < 16,
// permlane swaps for 16 and 32 (lane semantics checked on gfx950).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}
template <int J>
__device__ __forceinline__ uint32_t xshfl(uint32_t v) {
  if constexpr (J == 1) return dpp_mov<0xB1>(v);                   // quad_perm [1,0,3,2]
  else if constexpr (J == 2) return dpp_mov<0x4E>(v);              // quad_perm [2,3,0,1]
  else if constexpr (J == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(v));  // half mirror, then quad reverse
  else if constexpr (J == 8) return dpp_mov<0x141>(dpp_mov<0x140>(v)); // row mirror, then half mirror
  else if constexpr (J == 16) {
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((threadIdx.x >> 4) & 1) ? p[0] : p[1];
  } else {
    static_assert(J == 32, "xor distance");
    auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return ((threadIdx.x >> 5) & 1) ? p[0] : p[1];
  }
}
template <int J>
__device__ __forceinline__ float xshflf(float v) {
  return __uint_as_float(xshfl<J>(__float_as_uint(v)));
}

// One compare-exchange stage of a descending bitonic network across the wave.
template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_desc_step(uint32_t v, int lane) {
  const uint32_t o = xshfl<J>(v);
  const bool take_max = ((lane & K) == 0) == ((lane & J) == 0);
  return take_max ? (v > o ? v : o) : (v < o ? v : o);
}
// Sort 64 values (one per lane) in descending lane order.
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t v, int lane) {
  v = bitonic_desc_step<2, 1>(v, lane);
  v = bitonic_desc_step<4, 2>(v, lane);  v = bitonic_desc_step<4, 1>(v, lane);
  v = bitonic_desc_step<8, 4>(v, lane);  v = bitonic_desc_step<8, 2>(v, lane);  v = bitonic_desc_step<8, 1>(v, lane);
  v = bitonic_desc_step<16, 8>(v, lane); v = bitonic_desc_step<16, 4>(v, lane);
  v = bitonic_desc_step<16, 2>(v, lane); v = bitonic_desc_step<16, 1>(v, lane);
  v = bitonic_desc_step<32, 16>(v, lane); v = bitonic_desc_step<32, 8>(v, lane); v = bitonic_desc_step<32, 4>(v, lane);
  v = bitonic_desc_step<32, 2>(v, lane);  v = bitonic_desc_step<32, 1>(v, lane);
  v = bitonic_desc_step<64, 32>(v, lane); v = bitonic_desc_step<64, 16>(v, lane); v = bitonic_desc_step<64, 8>(v, lane);
  v = bitonic_desc_step<64, 4>(v, lane);  v = bitonic_desc_step<64, 2>(v, lane);  v = bitonic_desc_step<64, 1>(v, lane);
  return v;
}

// Largest of 64 values (one per lane), returned uniform: running maxima down each 16-lane
// row (shifts of 1, 2, 4, 8), then the row maxima carried by the row broadcasts; lane 63
// ends with the wave's maximum.
__device__ __forceinline__ uint32_t wave_max_u32_last(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));   // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));   // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));   // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));   // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum across a 64-lane wave: shifts of 1, 2, 4, 8 inside each
// 16-lane row (zero fill), then the row totals carried by the row broadcasts.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT multiple of 64, <= 1024).
// `tmp` must hold NT/64 + 1 words of LDS. Returns the exclusive prefix; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int i = 0; i < NW; ++i) { uint32_t x = tmp[i]; tmp[i] = run; run += x; }
    tmp[NW] = run;
  }
  __syncthreads();
  uint32_t res = tmp[wid] + inc - v;
  *total = tmp[NW];
  __syncthreads();
  return res;
}

}  // namespace dsa
