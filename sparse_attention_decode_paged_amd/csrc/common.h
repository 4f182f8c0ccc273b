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
constexpr int kWave = 64;

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
};

// Query-row to cache mapping.
struct RowMap {
  const int32_t* block_table;
  const int32_t* row_seq;
  const int32_t* row_ctx;
  int32_t bt_stride;
  int32_t max_ctx;  // host bound, also <= bt_stride * block_size
};

// Eligible length of row r, clamped to [0, max_ctx].
__device__ __forceinline__ int row_len(const RowMap& m, int r) {
  int c = m.row_ctx[r];
  c = c < 0 ? 0 : c;
  return c > m.max_ctx ? m.max_ctx : c;
}

// Physical block of token t of the block-table row `seq`, clamped into the pool.
__device__ __forceinline__ int64_t token_block(const CacheView& cv, const RowMap& m, int seq, int t) {
  int64_t b = m.block_table[(int64_t)seq * m.bt_stride + (t >> cv.log2_bs)];
  if ((uint64_t)b >= (uint64_t)cv.num_blocks) b = b < 0 ? 0 : cv.num_blocks - 1;
  return b;
}

// Byte address of a token's page inside its block row (page base of the given kind).
__device__ __forceinline__ const uint8_t* row_base(const CacheView& cv, int64_t blk) {
  return cv.pool + blk * cv.row_bytes;
}

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

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive prefix sum across a 64-lane wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
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
