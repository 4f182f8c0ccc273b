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
//   translate the 64 token ids to latent row offsets once (block table lookups),
//   then gather the 64 latents (576 e4m3 bytes each) into LDS;
//   S = Q . C^T on 16x16x32 bf16 MFMAs (each wave: 16 tokens x 32 heads);
//   online softmax in the log2 domain (running max / sum per head);
//   P'' = p * scale_t / (largest scale in the chunk), in [0, 1], as fp16 in LDS;
//   O += P'' . codes on 32x32x16 fp16 MFMAs (each wave: 128 of the 512 value
//   columns); e4m3 codes are exact in fp16, and fp16 P keeps 11 significant bits
//   (bf16's 8 were visibly too few on rows dominated by a handful of tokens).
//   The chunk's scale factor joins the per-head softmax rescale.
// e4m3 codes convert to bf16 exactly; the per-token scale is applied to the
// logit and folded into P'. With one split the workgroup writes out / lse; with
// several it writes unnormalised partials (O, m, l) that the merge kernel
// combines by log-sum-exp.
#include "common.h"
#include "internal.h"

namespace dsa {

namespace {
using v8h = v8hf;
constexpr int NT = 256;
constexpr int CH = kMlaChunk;           // 64 tokens per iteration
constexpr int PIECES = kDLat / 16;      // 36 16-byte pieces per latent
constexpr int QROW = kDLat + 8;         // LDS row strides padded by 16 bytes so that the
constexpr int LROW = kDLat + 16;        // 16 rows an MFMA fragment reads fall in distinct banks
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
}  // namespace

__global__ __launch_bounds__(NT) void sparse_mla_kernel(CacheView cv, RowMap rm, const uint16_t* __restrict__ q_lat,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ phys, int k, int ts, float c2,
                                                        float* __restrict__ out, float* __restrict__ lse,
                                                        float* __restrict__ part_o, float* __restrict__ part_ml,
                                                        int nsplit) {
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  __shared__ __attribute__((aligned(16))) uint16_t q_s[kMlaGroup * QROW];
  __shared__ __attribute__((aligned(16))) uint8_t lat_s[CH * LROW];
  __shared__ __attribute__((aligned(16))) _Float16 p_s[kMlaGroup * CH];
  __shared__ float sc_s[CH];
  __shared__ float red_s[4][kMlaGroup];
  __shared__ float m_s[kMlaGroup], l_s[kMlaGroup], alpha_s[kMlaGroup];

  const int32_t* irow = idx + (int64_t)r * k;
  const int j0 = split * ts;
  const int j1 = (j0 + ts < k) ? j0 + ts : k;
  const int seq = rm.row_seq[r];
  const int bs_mask = cv.block_size - 1;

  // Q fragment rows for this head group, straight to LDS (all loads issued first).
  {
    const v4i* qg = reinterpret_cast<const v4i*>(q_lat + ((int64_t)r * kHQ + hg * kMlaGroup) * kDLat);
    constexpr int QP = kDLat / 8;  // 72 16-byte pieces per head row
    constexpr int QN = kMlaGroup * QP / NT;
    static_assert(QN * NT == kMlaGroup * QP, "Q pieces per thread");
    v4i qv[QN];
#pragma unroll
    for (int q = 0; q < QN; ++q) qv[q] = qg[tid + NT * q];
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int i = tid + NT * q, h = i / QP, pc = i - h * QP;
      *reinterpret_cast<v4i*>(q_s + h * QROW + pc * 8) = qv[q];
    }
  }
  if (tid < kMlaGroup) {
    m_s[tid] = kNegInf;
    l_s[tid] = 0.f;
  }

  v16f acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = v16f{};
  float s_run = 1.f;  // acc holds O / s_run (token scales folded into P per chunk)

  for (int c0 = j0; c0 < j1; c0 += CH) {
    // ---- gather: 4 threads per token; each looks up its token's latent row and
    // issues its 9 of the 36 16-byte pieces (and the scale) right away ----
    {
      const int tt = tid >> 2, qtr = tid & 3;
      const int j = c0 + tt;
      int t = j < j1 ? irow[j] : -1;
      t = t < rm.max_ctx ? t : -1;
      const int tc = t >= 0 ? t : 0;  // every load below stays in the pool; empty slots are masked
      int64_t blk;
      int slot;
      if (phys != nullptr) {
        int ps = j < j1 ? phys[(int64_t)r * k + j] : 0;
        ps = ps >= 0 ? ps : 0;
        blk = (int64_t)ps >> cv.log2_bs;
        blk = blk < cv.num_blocks ? blk : cv.num_blocks - 1;
        slot = ps & bs_mask;
      } else {
        blk = token_block(cv, rm, seq, tc);
        slot = tc & bs_mask;
      }
      const uint8_t* page = cv.pool + blk * cv.row_bytes + cv.lat_off;
      const uint8_t* lrow = page + (int64_t)slot * kDLat;
      float sv = 0.f;
      if (qtr == 0) sv = *reinterpret_cast<const float*>(page + (int64_t)cv.block_size * kDLat + (int64_t)slot * 4);
      constexpr int PN = PIECES / 4;  // 9 pieces per thread
      v4i v[PN];
#pragma unroll
      for (int q = 0; q < PN; ++q) v[q] = *reinterpret_cast<const v4i*>(lrow + 16 * (qtr + 4 * q));
#pragma unroll
      for (int q = 0; q < PN; ++q)
        *reinterpret_cast<v4i*>(lat_s + tt * LROW + 16 * (qtr + 4 * q)) = t >= 0 ? v[q] : v4i{0, 0, 0, 0};
      if (qtr == 0) sc_s[tt] = t >= 0 ? sv : kNegInf;  // -inf marks an empty slot
    }
    __syncthreads();
    // largest token scale of the chunk, computed by every wave (no extra barrier)
    float smax;
    {
      float v = sc_s[lane];
      v = fmaxf(v, xshflf<1>(v));
      v = fmaxf(v, xshflf<2>(v));
      v = fmaxf(v, xshflf<4>(v));
      v = fmaxf(v, xshflf<8>(v));
      v = fmaxf(v, xshflf<16>(v));
      v = fmaxf(v, xshflf<32>(v));
      smax = v > 0.f ? v : 1.f;
    }

    // ---- S = Q . C^T : wave w -> tokens [16w, 16w+16), heads 0..31 ----
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      const int hrow = lane & 15, kq = 8 * (lane >> 4);
      const uint8_t* lrow = lat_s + (16 * wid + hrow) * LROW + kq;
      const uint16_t* qa0 = q_s + hrow * QROW + kq;
      const uint16_t* qa1 = q_s + (16 + hrow) * QROW + kq;
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
      v = fmaxf(v, xshflf<1>(v));
      v = fmaxf(v, xshflf<2>(v));
      v = fmaxf(v, xshflf<4>(v));
      v = fmaxf(v, xshflf<8>(v));
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
    // p = 2^(x - m); P'' = p * scale_t / smax in [0, 1] goes to the fp16 MFMA
    float ps[8];
    const float sfac = ok ? sct / smax : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int h = (i < 4) ? hb + i : 16 + hb + (i - 4);
      float p = (x[i] == kNegInf) ? 0.f : exp2f(x[i] - m_s[h]);
      ps[i] = p;
      p_s[h * CH + tt] = (_Float16)(p * sfac);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = ps[i];
      v += xshflf<1>(v);
      v += xshflf<2>(v);
      v += xshflf<4>(v);
      v += xshflf<8>(v);
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

    // ---- acc = acc * alpha * (s_run / smax) + P'' . codes : wave w -> columns [128w, 128w+128) ----
    const float rescale = s_run / smax;
    s_run = smax;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float a = alpha_s[8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3)] * rescale;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c][rr] *= a;
    }
#pragma unroll
    for (int ks = 0; ks < CH / 16; ++ks) {
      const int tk = 16 * ks + 8 * (lane >> 5);
      v8h a = *reinterpret_cast<const v8h*>(p_s + (lane & 31) * CH + tk);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = 128 * wid + 32 * c + (lane & 31);
        const uint8_t* vp = lat_s + tk * LROW + col;
        uint32_t w0 = (uint32_t)vp[0] | ((uint32_t)vp[LROW] << 8) | ((uint32_t)vp[2 * LROW] << 16) |
                      ((uint32_t)vp[3 * LROW] << 24);
        uint32_t w1 = (uint32_t)vp[4 * LROW] | ((uint32_t)vp[5 * LROW] << 8) | ((uint32_t)vp[6 * LROW] << 16) |
                      ((uint32_t)vp[7 * LROW] << 24);
        v8h b = e4m3x8_to_f16(w0, w1);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  __syncthreads();
  // ---- epilogue ----
  if (nsplit == 1) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int h = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
      const float lv = l_s[h];
      const float f = lv > 0.f ? s_run / lv : 0.f;
      float* orow = out + ((int64_t)r * kHQ + hg * kMlaGroup + h) * kDV + 128 * wid + (lane & 31);
#pragma unroll
      for (int c = 0; c < 4; ++c) orow[32 * c] = acc[c][rr] * f;
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
      for (int c = 0; c < 4; ++c) orow[32 * c] = acc[c][rr] * s_run;
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
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + (int64_t)r * nsplit * kHQ + h;
  float M = kNegInf;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[(int64_t)s * kHQ].x);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  const float* po = part_o + ((int64_t)r * nsplit * kHQ + h) * kDV + tid;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float2 e = ml[(int64_t)s * kHQ];
    const float x0 = po[(int64_t)s * kHQ * kDV], x1 = po[(int64_t)s * kHQ * kDV + NT];
    const float wgt = (e.x == kNegInf) ? 0.f : exp2f(e.x - M);
    L = fmaf(wgt, e.y, L);
    o0 = fmaf(wgt, x0, o0);
    o1 = fmaf(wgt, x1, o1);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* orow = out + ((int64_t)r * kHQ + h) * kDV;
  orow[tid] = o0 * inv;
  orow[tid + NT] = o1 * inv;
  if (lse != nullptr && tid == 0) lse[(int64_t)r * kHQ + h] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : kNegInf;
}

hipError_t launch_sparse_mla(const CacheView& cv, const RowMap& rm, const uint16_t* q_lat, const int32_t* idx,
                             const int32_t* phys, const float* pscale, int R, int k, float sm_scale, float* out,
                             float* lse, void* ws, hipStream_t stream) {
  (void)pscale;
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
  hipLaunchKernelGGL(sparse_mla_kernel, dim3(nsplit, R, kHQ / kMlaGroup), dim3(NT), 0, stream, cv, rm, q_lat, idx, phys,
                     k, ts, c2, out, lse, part_o, part_ml, nsplit);
  if (nsplit > 1)
    hipLaunchKernelGGL(mla_merge_kernel, dim3(kHQ, R), dim3(NT), 0, stream, part_o, part_ml, nsplit, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
