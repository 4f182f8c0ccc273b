// New-token cache append: quantise each row's new index key and latent and write them
// into the token's slot of its packed block row (vLLM "Day-0 support for Kimi K3.1
// Pro", fused front-end: the new token's index key is quantised and written, and its
// latent is written into the cache, before the step scores; section on the KV cache
// serving three kinds of state: one contiguous row per block).
//
// Quantiser, per vector (the pages leave it open; this is the same reading the cache
// generator uses):
//   FP8   scale = amax / 448 in fp32 (1 when amax = 0); y = x / scale (IEEE division),
//         clamped to +-448, rounded to the nearest e4m3 value with ties to the even
//         code; the sign bit follows the sign of y.
//   MXFP4 per 32 elements E = floor(log2 amax) - 2, clamped to [-127, 127] (0 when
//         amax = 0), stored as E + 127; y = x * 2^-E rounded to the nearest e2m1
//         magnitude with ties to the even code, 6 at most; no negative zero.
//   NVFP4 latent (352 B record: page 1 quotes the width only): s and y as for FP8;
//         dims 512..575 as e4m3 codes of y; each 16-dim block of the first 512 gets
//         the e4m3 code nearest to max|y_block| / 6 as its scale, and e2m1 codes of
//         y / (that scale's value), all 0 when the value is 0.
// One wave per row: 9 latent and 2 key values per lane, coalesced, byte stores.
#include "dsa.h"
#include "common.h"
#include "internal.h"

namespace dsa {

namespace {
// e4m3 code of y, |y| <= 448, round to nearest even. Exact: the significand is
// scaled by powers of two and rounded once by rintf (ties to even).
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t sign = __float_as_uint(y) >> 31;
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9 (8 steps reach code 0x08 = 2^-6)
    code = (uint32_t)rintf(a * 512.f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 255u) - 127;  // floor(log2 a)
    uint32_t m = (uint32_t)rintf(ldexpf(a, -e) * 8.f);        // 8 .. 16
    if (m == 16u) {
      m = 8u;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | (m - 8u);
  }
  return code | (sign << 7);
}

// e2m1 nibble of y: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code
// (each midpoint compares with > or >= so that it falls to the even side).
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  const float a = fminf(fabsf(y), 6.f);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                     (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.f);
  return m | ((y < 0.f && m > 0u) ? 8u : 0u);
}

__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, xshflf<1>(v));
  v = fmaxf(v, xshflf<2>(v));
  v = fmaxf(v, xshflf<4>(v));
  v = fmaxf(v, xshflf<8>(v));
  v = fmaxf(v, xshflf<16>(v));
  v = fmaxf(v, xshflf<32>(v));
  return v;
}

// Writes the FP8 codes (element lane + 64 i of a D-vector, i < D/64) and the scale.
template <int D>
__device__ __forceinline__ void put_fp8(uint8_t* codes, uint8_t* scale_at, const float* x, int lane) {
  constexpr int N = D / 64;
  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = x[lane + 64 * i];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max_f(amax);
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float y = fminf(fmaxf(__fdiv_rn(v[i], scale), -448.f), 448.f);
    codes[lane + 64 * i] = (uint8_t)e4m3_rne(y);
  }
  if (lane == 0) *reinterpret_cast<float*>(scale_at) = scale;
}

// NVFP4 latent record (element lane + 64 i of the 576-vector on this lane) and its scale.
__device__ __forceinline__ void put_nvfp4_latent(uint8_t* rec, uint8_t* scale_at, const float* x, int lane) {
  float v[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) v[i] = x[lane + 64 * i];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 9; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max_f(amax);
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
#pragma unroll
  for (int i = 0; i < 9; ++i) v[i] = fminf(fmaxf(__fdiv_rn(v[i], scale), -448.f), 448.f);
  rec[kDV / 2 + kDV / 16 + lane] = (uint8_t)e4m3_rne(v[8]);  // tail dim 512 + lane
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // block 4 i + lane / 16 = lanes 16 (lane / 16) .. + 15 of element row i
    float bm = fabsf(v[i]);
    bm = fmaxf(bm, xshflf<1>(bm));
    bm = fmaxf(bm, xshflf<2>(bm));
    bm = fmaxf(bm, xshflf<4>(bm));
    bm = fmaxf(bm, xshflf<8>(bm));
    const uint32_t sc = e4m3_rne(__fdiv_rn(bm, 6.f));
    const float scv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc, 1.0f, false)[0];
    const uint32_t nib = scv > 0.f ? e2m1_rne(__fdiv_rn(v[i], scv)) : 0u;
    const uint32_t hi = (uint32_t)__shfl_xor((int)nib, 1, 64);
    if ((lane & 1) == 0) rec[32 * i + (lane >> 1)] = (uint8_t)(nib | (hi << 4));
    if ((lane & 15) == 0) rec[kDV / 2 + 4 * i + (lane >> 4)] = (uint8_t)sc;
  }
  if (lane == 0) *reinterpret_cast<float*>(scale_at) = scale;
}
}  // namespace

__global__ __launch_bounds__(256) void cache_append_kernel(CacheView cv, int32_t index_fmt,
                                                           const int32_t* __restrict__ block_table, int32_t bt_stride,
                                                           const int32_t* __restrict__ row_seq,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ idx_key,
                                                           const float* __restrict__ latent, int R) {
  const int r = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;  // whole wave
  const int p = pos[r];
  if (p < 0 || (int64_t)(p >> cv.log2_bs) >= (int64_t)bt_stride) return;
  const int64_t blk = block_table[(int64_t)row_seq[r] * bt_stride + (p >> cv.log2_bs)];
  if (blk < 0 || blk >= cv.num_blocks) {  // never write outside the pool
    if (lane == 0) raise_status(cv.status, kStBlockClamped);
    return;
  }
  const int slot = p & (cv.block_size - 1);
  uint8_t* row = const_cast<uint8_t*>(cv.pool) + blk * cv.row_bytes;

  if (latent != nullptr) {
    uint8_t* page = row + cv.lat_off;
    if (cv.latent_fmt == DSA_LATENT_NVFP4)
      put_nvfp4_latent(page + (int64_t)slot * kNvRec, page + (int64_t)cv.block_size * kNvRec + 4 * slot,
                       latent + (int64_t)r * kDLat, lane);
    else
      put_fp8<kDLat>(page + (int64_t)slot * kDLat, page + (int64_t)cv.block_size * kDLat + 4 * slot,
                     latent + (int64_t)r * kDLat, lane);
  }
  if (idx_key == nullptr) return;
  uint8_t* page = row + cv.idx_off;
  const float* x = idx_key + (int64_t)r * kDIdx;
  if (index_fmt == DSA_INDEX_FP8) {
    put_fp8<kDIdx>(page + (int64_t)slot * kDIdx, page + (int64_t)cv.block_size * kDIdx + 4 * slot, x, lane);
    return;
  }
  // MXFP4: lane l holds elements l (group l / 32) and l + 64 (group 2 + l / 32)
  constexpr int kHalf = kDIdx / 2;  // packed bytes per key
  uint8_t* codes = page + (int64_t)slot * kHalf;
  uint8_t* e8 = page + (int64_t)cv.block_size * kHalf + 4 * slot;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float v = x[lane + 64 * i];
    float amax = fabsf(v);
    amax = fmaxf(amax, xshflf<1>(amax));
    amax = fmaxf(amax, xshflf<2>(amax));
    amax = fmaxf(amax, xshflf<4>(amax));
    amax = fmaxf(amax, xshflf<8>(amax));
    amax = fmaxf(amax, xshflf<16>(amax));  // max over the 32-lane group
    int E = 0;
    if (amax > 0.f) {
      E = (int)((__float_as_uint(amax) >> 23) & 255u) - 127 - 2;  // floor(log2 amax) - 2 (subnormal amax clamps)
      E = E < -127 ? -127 : (E > 127 ? 127 : E);
    }
    const uint32_t nib = e2m1_rne(ldexpf(v, -E));
    const uint32_t hi = (uint32_t)__shfl_xor((int)nib, 1, 64);
    if ((lane & 1) == 0) codes[(lane + 64 * i) >> 1] = (uint8_t)(nib | (hi << 4));
    if ((lane & 31) == 0) e8[2 * i + (lane >> 5)] = (uint8_t)(E + 127);
  }
}

hipError_t launch_cache_append(const CacheView& cv, int32_t index_fmt, const int32_t* block_table, int32_t bt_stride,
                               const int32_t* row_seq, const int32_t* pos, const float* idx_key,
                               const float* latent, int R, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(cache_append_kernel, dim3((R + 3) / 4), dim3(256), 0, stream, cv, index_fmt, block_table,
                     bt_stride, row_seq, pos, idx_key, latent, R);
  return hipGetLastError();
}

}  // namespace dsa
