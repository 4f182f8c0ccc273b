// Sparse MLA: exact attention of 96 latent-query heads over the selected tokens,
// reading each selected token's FP8 latent straight from the packed paged cache.
//
// vLLM "Day-0 support for Kimi K3.1 Pro", section "Sparse attention in K3.1 Pro":
// MLA runs exactly, but only over the kept tokens; the AMD section's sparse MLA
// reads selected tokens directly from the FP8 KV cache and, for small batches,
// adds parallelism inside a query row. Absorbed queries live in the 576-wide
// latent space (keys = all 576 dims, values = first 512; page 3 model table: NoPE).
//
// Grid (split, row, head group of 32). A workgroup walks its split's slice of the
// row's index list 64 tokens at a time:
//   gather 64 latents (576 e4m3 bytes + fp32 scale) into LDS;
//   S = Q . C^T on 16x16x32 bf16 MFMAs (each wave: 16 tokens x 32 heads);
//   online softmax in the log2 domain (running max / sum per head);
//   P' = p * scale_t split into bf16 high and low parts in LDS;
//   O += P'_hi . codes + P'_lo . codes on 32x32x16 bf16 MFMAs (each wave: 128 of
//   the 512 value columns). The two-part P' keeps ~16 significant bits, so rows
//   dominated by a handful of tokens lose nothing visible to bf16 rounding.
// e4m3 codes convert to bf16 exactly; the per-token scale is applied to the
// logit and folded into P'. With one split the workgroup writes out / lse; with
// several it writes unnormalised partials (O, m, l) that the merge kernel
// combines by log-sum-exp.
#include "common.h"
#include "internal.h"

namespace dsa {

namespace {
constexpr int NT = 256;
constexpr int CH = kMlaChunk;           // 64 tokens per iteration
constexpr int PIECES = kDLat / 16;      // 36 16-byte pieces per latent
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
}  // namespace

__global__ __launch_bounds__(NT) void sparse_mla_kernel(CacheView cv, RowMap rm, const uint16_t* __restrict__ q_lat,
                                                        const int32_t* __restrict__ idx, int k, int ts, float c2,
                                                        float* __restrict__ out, float* __restrict__ lse,
                                                        float* __restrict__ part_o, float* __restrict__ part_ml,
                                                        int nsplit) {
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  __shared__ __attribute__((aligned(16))) uint16_t q_s[kMlaGroup * kDLat];
  __shared__ __attribute__((aligned(16))) uint8_t lat_s[CH * kDLat];
  __shared__ __attribute__((aligned(16))) uint16_t p_s[kMlaGroup * CH];
  __shared__ __attribute__((aligned(16))) uint16_t pl_s[kMlaGroup * CH];
  __shared__ float sc_s[CH];
  __shared__ float red_s[4][kMlaGroup];
  __shared__ float m_s[kMlaGroup], l_s[kMlaGroup], alpha_s[kMlaGroup];

  {
    const v4i* qg = reinterpret_cast<const v4i*>(q_lat + ((int64_t)r * kHQ + hg * kMlaGroup) * kDLat);
    v4i* qd = reinterpret_cast<v4i*>(q_s);
    for (int i = tid; i < kMlaGroup * kDLat / 8; i += NT) qd[i] = qg[i];
  }
  if (tid < kMlaGroup) {
    m_s[tid] = kNegInf;
    l_s[tid] = 0.f;
  }
  __syncthreads();

  v16f acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = v16f{};

  const int32_t* irow = idx + (int64_t)r * k;
  const int j0 = split * ts;
  const int j1 = (j0 + ts < k) ? j0 + ts : k;
  const int seq = rm.row_seq[r];
  const int bs_mask = cv.block_size - 1;

  for (int c0 = j0; c0 < j1; c0 += CH) {
    // ---- gather 64 latents ----
#pragma unroll
    for (int q = 0; q < (CH * PIECES) / NT; ++q) {
      int p = tid + NT * q;
      int tt = p / PIECES, pc = p - tt * PIECES;
      int j = c0 + tt;
      int t = j < j1 ? irow[j] : -1;
      t = t < rm.max_ctx ? t : -1;  // indices beyond the row bound are treated as empty
      v4i v = {0, 0, 0, 0};
      if (t >= 0) {
        int64_t blk = token_block(cv, rm, seq, t);
        const uint8_t* lp = row_base(cv, blk) + cv.lat_off + (int64_t)(t & bs_mask) * kDLat + pc * 16;
        v = *reinterpret_cast<const v4i*>(lp);
      }
      reinterpret_cast<v4i*>(lat_s)[p] = v;
    }
    if (tid < CH) {
      int j = c0 + tid;
      int t = j < j1 ? irow[j] : -1;
      t = t < rm.max_ctx ? t : -1;
      float s = 0.f;
      if (t >= 0) {
        int64_t blk = token_block(cv, rm, seq, t);
        s = *reinterpret_cast<const float*>(row_base(cv, blk) + cv.lat_off + (int64_t)cv.block_size * kDLat +
                                            (int64_t)(t & bs_mask) * 4);
      }
      sc_s[tid] = t >= 0 ? s : kNegInf;  // -inf marks an empty slot
    }
    __syncthreads();

    // ---- S = Q . C^T : wave w -> tokens [16w, 16w+16), heads 0..31 ----
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      const int hrow = lane & 15, kq = 8 * (lane >> 4);
      const uint8_t* lrow = lat_s + (16 * wid + hrow) * kDLat + kq;
      const uint16_t* qa0 = q_s + hrow * kDLat + kq;
      const uint16_t* qa1 = q_s + (16 + hrow) * kDLat + kq;
#pragma unroll 6
      for (int kk = 0; kk < kDLat / 32; ++kk) {
        v8bf a0 = *reinterpret_cast<const v8bf*>(qa0 + 32 * kk);
        v8bf a1 = *reinterpret_cast<const v8bf*>(qa1 + 32 * kk);
        uint2 raw = *reinterpret_cast<const uint2*>(lrow + 32 * kk);
        v8bf b = e4m3x8_to_bf16(raw.x, raw.y);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, s1, 0, 0, 0);
      }
    }
    // s0[i]: head 4*(lane>>4)+i, s1[i]: head 16+4*(lane>>4)+i, token tt
    const int tt = 16 * wid + (lane & 15);
    const float sct = sc_s[tt];
    const bool ok = sct != kNegInf;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = ok ? s0[i] * (sct * c2) : kNegInf;
      x[4 + i] = ok ? s1[i] * (sct * c2) : kNegInf;
    }
    float mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = x[i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
      mx[i] = v;
    }
    const int hb = 4 * (lane >> 4);
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red_s[wid][hb + i] = mx[i];
        red_s[wid][16 + hb + i] = mx[4 + i];
      }
    }
    __syncthreads();
    if (tid < kMlaGroup) {
      float cm = fmaxf(fmaxf(red_s[0][tid], red_s[1][tid]), fmaxf(red_s[2][tid], red_s[3][tid]));
      float mo = m_s[tid];
      float mn = fmaxf(mo, cm);
      alpha_s[tid] = (mn == kNegInf) ? 1.f : exp2f(mo - mn);
      m_s[tid] = mn;
    }
    __syncthreads();
    float ps[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int h = (i < 4) ? hb + i : 16 + hb + (i - 4);
      float mn = m_s[h];
      float p = (x[i] == kNegInf) ? 0.f : exp2f(x[i] - mn);
      ps[i] = p;
      const float pv = ok ? p * sct : 0.f;
      const __bf16 hi = (__bf16)pv;
      p_s[h * CH + tt] = __builtin_bit_cast(uint16_t, hi);
      pl_s[h * CH + tt] = bf16_bits(pv - (float)hi);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = ps[i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
      ps[i] = v;
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red_s[wid][hb + i] = ps[i];
        red_s[wid][16 + hb + i] = ps[4 + i];
      }
    }
    __syncthreads();
    if (tid < kMlaGroup) {
      l_s[tid] = l_s[tid] * alpha_s[tid] + (red_s[0][tid] + red_s[1][tid] + red_s[2][tid] + red_s[3][tid]);
    }

    // ---- O = alpha * O + P' . codes : wave w -> value columns [128w, 128w+128) ----
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float a = alpha_s[8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3)];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c][rr] *= a;
    }
#pragma unroll
    for (int ks = 0; ks < CH / 16; ++ks) {
      const int tk = 16 * ks + 8 * (lane >> 5);
      v8bf a = *reinterpret_cast<const v8bf*>(p_s + (lane & 31) * CH + tk);
      v8bf al = *reinterpret_cast<const v8bf*>(pl_s + (lane & 31) * CH + tk);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = 128 * wid + 32 * c + (lane & 31);
        const uint8_t* vp = lat_s + tk * kDLat + col;
        uint32_t w0 = (uint32_t)vp[0] | ((uint32_t)vp[kDLat] << 8) | ((uint32_t)vp[2 * kDLat] << 16) |
                      ((uint32_t)vp[3 * kDLat] << 24);
        uint32_t w1 = (uint32_t)vp[4 * kDLat] | ((uint32_t)vp[5 * kDLat] << 8) | ((uint32_t)vp[6 * kDLat] << 16) |
                      ((uint32_t)vp[7 * kDLat] << 24);
        v8bf b = e4m3x8_to_bf16(w0, w1);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc[c], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue ----
  if (nsplit == 1) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int h = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
      const float lv = l_s[h];
      const float inv = lv > 0.f ? 1.f / lv : 0.f;
      float* orow = out + ((int64_t)r * kHQ + hg * kMlaGroup + h) * kDV + 128 * wid + (lane & 31);
#pragma unroll
      for (int c = 0; c < 4; ++c) orow[32 * c] = acc[c][rr] * inv;
    }
    if (lse != nullptr && tid < kMlaGroup) {
      float lv = l_s[tid];
      lse[(int64_t)r * kHQ + hg * kMlaGroup + tid] = lv > 0.f ? (m_s[tid] + log2f(lv)) * 0.69314718055994531f : kNegInf;
    }
  } else {
    const int64_t pbase = ((int64_t)r * nsplit + split) * kHQ + hg * kMlaGroup;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int h = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
      float* orow = part_o + (pbase + h) * kDV + 128 * wid + (lane & 31);
#pragma unroll
      for (int c = 0; c < 4; ++c) orow[32 * c] = acc[c][rr];
    }
    if (tid < kMlaGroup) {
      part_ml[(pbase + tid) * 2 + 0] = m_s[tid];
      part_ml[(pbase + tid) * 2 + 1] = l_s[tid];
    }
  }
}

// out[r][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s ; empty splits (m = -inf) weigh 0.
__global__ __launch_bounds__(NT) void mla_merge_kernel(const float* __restrict__ part_o,
                                                       const float* __restrict__ part_ml, int nsplit,
                                                       float* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  float M = kNegInf;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(((int64_t)r * nsplit + s) * kHQ + h) * 2]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const int64_t base = ((int64_t)r * nsplit + s) * kHQ + h;
    float m = part_ml[base * 2];
    if (m == kNegInf) continue;
    float wgt = exp2f(m - M);
    L += wgt * part_ml[base * 2 + 1];
    o0 += wgt * part_o[base * kDV + tid];
    o1 += wgt * part_o[base * kDV + tid + NT];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* orow = out + ((int64_t)r * kHQ + h) * kDV;
  orow[tid] = o0 * inv;
  orow[tid + NT] = o1 * inv;
  if (lse != nullptr && tid == 0) lse[(int64_t)r * kHQ + h] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : kNegInf;
}

hipError_t launch_sparse_mla(const CacheView& cv, const RowMap& rm, const uint16_t* q_lat, const int32_t* idx,
                             int R, int k, float sm_scale, float* out, float* lse, void* ws, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const int nsplit = mla_splits(R, k);
  const int ts = mla_split_tokens(k, nsplit);
  const float c2 = (float)((double)sm_scale * 1.4426950408889634);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (nsplit > 1) {
    part_o = static_cast<float*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_up((size_t)R * nsplit * kHQ * kDV * 4, 256));
  }
  hipLaunchKernelGGL(sparse_mla_kernel, dim3(nsplit, R, kHQ / kMlaGroup), dim3(NT), 0, stream, cv, rm, q_lat, idx, k,
                     ts, c2, out, lse, part_o, part_ml, nsplit);
  if (nsplit > 1)
    hipLaunchKernelGGL(mla_merge_kernel, dim3(kHQ, R), dim3(NT), 0, stream, part_o, part_ml, nsplit, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
