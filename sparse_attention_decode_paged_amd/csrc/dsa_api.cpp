// C ABI entry points: argument checks, workspace carving, kernel launches.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "dsa.h"
#include "internal.h"

using namespace dsa;

// The device status word: every GPU that runs this library holds its own copy. In host
// code the symbol's name is not a device address; status_word() looks the address up
// per device (hipGetSymbolAddress) and kernels receive that address.
__device__ uint32_t g_device_status;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<uint32_t*> g_status_addr[kMaxDevices];

// This device's status word, looked up on the first call on the device; NULL when the
// lookup fails (the kernels then report nothing).
uint32_t* status_word() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  uint32_t* p = g_status_addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* a = nullptr;
  if (hipGetSymbolAddress(&a, HIP_SYMBOL(g_device_status)) != hipSuccess || a == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_status_addr[dev].store(static_cast<uint32_t*>(a), std::memory_order_release);
  return static_cast<uint32_t*>(a);
}

// The decode step's workspace for callers that cannot allocate (dsa_decode_step_noalloc):
// one array per GPU. As with the status word, host code never passes the symbol's name;
// scratch_addr() looks up this device's address once and keeps it.
static __device__ __align__(256) uint8_t scratch[DSA_STATIC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_addr[kMaxDevices];

// This device's address of `scratch`, looked up (with the device current) on the first
// call on the device; NULL when the lookup fails.
void* scratch_addr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* a = nullptr;
  if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch_addr[dev].store(a, std::memory_order_release);
  return a;
}

thread_local std::string g_detail;

dsa_status fail(dsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return st;
}

dsa_status ok() {
  g_detail.clear();
  return DSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

dsa_status check_cache(const dsa_cache_desc* c, int32_t layer, CacheView* cv) {
  if (c == nullptr) return fail(DSA_ERR_NULL, "cache descriptor is NULL");
  if (c->pool == nullptr) return fail(DSA_ERR_NULL, "cache pool is NULL");
  if (c->block_size <= 0 || (c->block_size & (c->block_size - 1)) != 0 || c->block_size > 65536)
    return fail(DSA_ERR_LAYOUT, "block_size %d is not a power of two in [1, 65536]", c->block_size);
  if (c->num_layers < 1 || c->num_layers > DSA_MAX_LAYERS)
    return fail(DSA_ERR_LAYOUT, "num_layers %d out of [1, %d]", c->num_layers, DSA_MAX_LAYERS);
  if (layer < 0 || layer >= c->num_layers) return fail(DSA_ERR_ARG, "layer %d out of [0, %d)", layer, c->num_layers);
  if (c->num_blocks < 1) return fail(DSA_ERR_LAYOUT, "num_blocks %lld < 1", (long long)c->num_blocks);
  if (c->row_bytes <= 0 || (c->row_bytes & 15)) return fail(DSA_ERR_ALIGN, "row_bytes %lld is not a positive multiple of 16", (long long)c->row_bytes);
  if (!aligned16(c->pool)) return fail(DSA_ERR_ALIGN, "pool is not 16-byte aligned");
  if (c->index_fmt != DSA_INDEX_FP8 && c->index_fmt != DSA_INDEX_MXFP4)
    return fail(DSA_ERR_UNSUPPORTED, "index_fmt %d", c->index_fmt);
  if (c->latent_fmt != DSA_LATENT_FP8 && c->latent_fmt != DSA_LATENT_NVFP4)
    return fail(DSA_ERR_UNSUPPORTED, "latent_fmt %d", c->latent_fmt);
  const int64_t bs = c->block_size;
  const int64_t lat_page = bs * ((c->latent_fmt == DSA_LATENT_FP8 ? DSA_D_LAT : kNvRec) + 4);
  const int64_t idx_page = c->index_fmt == DSA_INDEX_FP8 ? bs * (DSA_D_IDX + 4) : bs * (DSA_D_IDX / 2 + 4);
  for (int l = 0; l < c->num_layers; ++l) {
    if (c->lat_off[l] < 0 || (c->lat_off[l] & 15) || c->lat_off[l] + lat_page > c->row_bytes)
      return fail(DSA_ERR_LAYOUT, "layer %d latent page [%lld, +%lld) does not fit a %lld-byte row or is misaligned", l,
                  (long long)c->lat_off[l], (long long)lat_page, (long long)c->row_bytes);
    if (c->idx_off[l] < 0 || (c->idx_off[l] & 15) || c->idx_off[l] + idx_page > c->row_bytes)
      return fail(DSA_ERR_LAYOUT, "layer %d index page [%lld, +%lld) does not fit a %lld-byte row or is misaligned", l,
                  (long long)c->idx_off[l], (long long)idx_page, (long long)c->row_bytes);
  }
  if (c->num_blocks * (int64_t)c->block_size > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "num_blocks * block_size exceeds 2^31 token slots");
  cv->pool = static_cast<const uint8_t*>(c->pool);
  cv->row_bytes = c->row_bytes;
  cv->num_blocks = c->num_blocks;
  cv->lat_off = c->lat_off[layer];
  cv->idx_off = c->idx_off[layer];
  cv->block_size = c->block_size;
  cv->log2_bs = ilog2(c->block_size);
  cv->latent_fmt = c->latent_fmt;
  cv->status = status_word();
  return DSA_OK;
}

dsa_status check_rows(const dsa_cache_desc* c, const int32_t* bt, int32_t bt_stride, const int32_t* row_seq,
                      const int32_t* row_ctx, int32_t R, int32_t max_ctx, bool need_ctx, RowMap* rm) {
  if (R < 0 || R > 65535) return fail(DSA_ERR_ARG, "R %d out of [0, 65535]", R);
  if (bt == nullptr || row_seq == nullptr) return fail(DSA_ERR_NULL, "block_table / row_seq is NULL");
  if (need_ctx && row_ctx == nullptr) return fail(DSA_ERR_NULL, "row_ctx is NULL");
  if (bt_stride < 1) return fail(DSA_ERR_ARG, "bt_stride %d < 1", bt_stride);
  if (max_ctx < 0 || max_ctx > kMaxCtx) return fail(DSA_ERR_ARG, "max_ctx %d out of [0, %d]", max_ctx, kMaxCtx);
  if ((int64_t)max_ctx > (int64_t)bt_stride * c->block_size)
    return fail(DSA_ERR_ARG, "max_ctx %d exceeds block-table capacity %lld", max_ctx,
                (long long)bt_stride * c->block_size);
  rm->block_table = bt;
  rm->row_seq = row_seq;
  rm->row_ctx = row_ctx;
  rm->bt_stride = bt_stride;
  rm->max_ctx = max_ctx;
  return DSA_OK;
}

int64_t scores_ld(int32_t max_ctx) {
  int64_t ld = ((int64_t)max_ctx + 63) / 64 * 64;
  return ld < 64 ? 64 : ld;
}

size_t decode_ws(int32_t R, int32_t max_ctx, int32_t k) {
  return align_up((size_t)R * scores_ld(max_ctx) * 4, 256) + topk_ws_bytes(R, max_ctx) +
         align_up((size_t)R * k * 4, 256) + mla_ws_bytes(R, k);
}

// The indexer for the cache's key format: FP8 (q_idx_scale = R x 32 fp32) or MXFP4
// (q_idx_scale = R x 32 x 4 E8M0 bytes).
// rows_per_seq > 1: runs of that many consecutive rows share a sequence, so the row-group
// kernel (FP8 or MXFP4) reads each key once per group of up to kRowsPerGroupMax rows.
hipError_t launch_indexer(int32_t index_fmt, const CacheView& cv, const RowMap& rm, const void* q_idx,
                          const void* q_idx_scale, const float* w, int R, int32_t rows_per_seq, float* scores,
                          int64_t ld, const TopkWs* ws, hipStream_t s) {
  if (index_fmt == DSA_INDEX_FP8 && rows_per_seq > 1) {
    const int G = rows_per_seq < kRowsPerGroupMax ? rows_per_seq : kRowsPerGroupMax;
    return launch_indexer_fp8_rows(cv, rm, static_cast<const uint8_t*>(q_idx), static_cast<const float*>(q_idx_scale),
                                   w, R, G, scores, ld, ws, s);
  }
  if (index_fmt == DSA_INDEX_MXFP4 && rows_per_seq > 1) {
    const int G = rows_per_seq < kRowsPerGroupMax ? rows_per_seq : kRowsPerGroupMax;
    return launch_indexer_mxfp4_rows(cv, rm, static_cast<const uint8_t*>(q_idx),
                                     static_cast<const uint8_t*>(q_idx_scale), w, R, G, scores, ld, ws, s);
  }
  if (index_fmt == DSA_INDEX_MXFP4)
    return launch_indexer_mxfp4(cv, rm, static_cast<const uint8_t*>(q_idx), static_cast<const uint8_t*>(q_idx_scale), w,
                                R, scores, ld, ws, s);
  return launch_indexer_fp8(cv, rm, static_cast<const uint8_t*>(q_idx), static_cast<const float*>(q_idx_scale), w, R,
                            scores, ld, ws, s);
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_ARG: return "argument out of range";
    case DSA_ERR_LAYOUT: return "inconsistent cache layout";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_ALIGN: return "misaligned pointer or offset";
    case DSA_ERR_HIP: return "HIP launch failed";
    case DSA_ERR_UNSUPPORTED: return "unsupported format or shape";
    default: return "unknown status";
  }
}

const char* dsa_last_error_detail(void) { return g_detail.c_str(); }

dsa_status dsa_device_status(void* stream, int32_t clear, uint32_t* status) {
  if (status == nullptr) return fail(DSA_ERR_NULL, "status is NULL");
  uint32_t* p = status_word();
  if (p == nullptr) return fail(DSA_ERR_HIP, "the device status word has no address on this device");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, p, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && clear) {
    static const uint32_t zero = 0u;
    e = hipMemcpyAsync(p, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  if (e != hipSuccess) return hip_status(e, "device_status");
  *status = v;
  return ok();
}

int64_t dsa_decode_scores_ld(int32_t max_ctx) { return scores_ld(max_ctx); }

size_t dsa_workspace_bytes(int32_t op, int32_t R, int32_t max_ctx, int32_t k) {
  if (R < 0 || max_ctx < 0 || k < 1 || k > DSA_MAX_K) return 0;
  switch (op) {
    case DSA_OP_TOPK: return topk_ws_bytes(R, max_ctx);
    case DSA_OP_SPARSE_MLA: return mla_ws_bytes(R, k);
    case DSA_OP_DECODE_STEP: return decode_ws(R, max_ctx, k);
    default: return 0;
  }
}

dsa_status dsa_indexer_score_multi(const dsa_cache_desc* cache, int32_t layer, const void* q_idx,
                                   const void* q_idx_scale, const float* w, const int32_t* block_table,
                                   int32_t bt_stride, const int32_t* row_seq, const int32_t* row_ctx, int32_t R,
                                   int32_t max_ctx, int32_t rows_per_seq, float* scores, int64_t ld_scores,
                                   void* stream) {
  CacheView cv;
  RowMap rm;
  dsa_status st = check_cache(cache, layer, &cv);
  if (st) return st;
  if ((st = check_rows(cache, block_table, bt_stride, row_seq, row_ctx, R, max_ctx, true, &rm))) return st;
  if (q_idx == nullptr || q_idx_scale == nullptr || w == nullptr || scores == nullptr)
    return fail(DSA_ERR_NULL, "q_idx / q_idx_scale / w / scores is NULL");
  if (ld_scores < max_ctx) return fail(DSA_ERR_ARG, "ld_scores %lld < max_ctx %d", (long long)ld_scores, max_ctx);
  if (rows_per_seq < 1) return fail(DSA_ERR_ARG, "rows_per_seq %d < 1", rows_per_seq);
  if (!aligned16(q_idx)) return fail(DSA_ERR_ALIGN, "q_idx is not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(q_idx_scale) & 3u) return fail(DSA_ERR_ALIGN, "q_idx_scale is not 4-byte aligned");
  if (R == 0) return ok();
  return hip_status(launch_indexer(cache->index_fmt, cv, rm, q_idx, q_idx_scale, w, R, rows_per_seq, scores, ld_scores,
                                   nullptr, static_cast<hipStream_t>(stream)),
                    "indexer");
}

dsa_status dsa_indexer_score(const dsa_cache_desc* cache, int32_t layer, const void* q_idx, const void* q_idx_scale,
                             const float* w, const int32_t* block_table, int32_t bt_stride, const int32_t* row_seq,
                             const int32_t* row_ctx, int32_t R, int32_t max_ctx, float* scores, int64_t ld_scores,
                             void* stream) {
  return dsa_indexer_score_multi(cache, layer, q_idx, q_idx_scale, w, block_table, bt_stride, row_seq, row_ctx, R,
                                 max_ctx, 1, scores, ld_scores, stream);
}

dsa_status dsa_topk(const float* scores, int64_t ld_scores, const int32_t* row_ctx, int32_t R, int32_t max_ctx,
                    int32_t k, int32_t* idx, void* workspace, size_t ws_bytes, void* stream) {
  if (scores == nullptr || row_ctx == nullptr || idx == nullptr) return fail(DSA_ERR_NULL, "scores / row_ctx / idx is NULL");
  if (R < 0 || R > 65535) return fail(DSA_ERR_ARG, "R %d out of [0, 65535]", R);
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_ARG, "k %d out of [1, %d]", k, DSA_MAX_K);
  if (max_ctx < 0 || max_ctx > kMaxCtx) return fail(DSA_ERR_ARG, "max_ctx %d out of [0, %d]", max_ctx, kMaxCtx);
  if (ld_scores < max_ctx) return fail(DSA_ERR_ARG, "ld_scores %lld < max_ctx %d", (long long)ld_scores, max_ctx);
  const size_t need = topk_ws_bytes(R, max_ctx);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(workspace)) return fail(DSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (R == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  TopkWs tw = topk_ws_carve(workspace, R, max_ctx);
  CacheView st{};  // no cache: carries only the status word
  st.status = status_word();
  hipError_t e = launch_topk_send(scores, ld_scores, row_ctx, R, max_ctx, tw, s);
  if (e == hipSuccess)
    e = launch_topk_select(scores, ld_scores, row_ctx, R, max_ctx, k, 512, idx, tw, nullptr, &st, nullptr, s);
  return hip_status(e, "topk");
}

dsa_status dsa_sparse_mla(const dsa_cache_desc* cache, int32_t layer, const uint16_t* q_lat, const int32_t* block_table,
                          int32_t bt_stride, const int32_t* row_seq, const int32_t* idx, int32_t R, int32_t k,
                          float sm_scale, float* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  CacheView cv;
  RowMap rm;
  dsa_status st = check_cache(cache, layer, &cv);
  if (st) return st;
  // idx entries must lie inside the block-table row: allow the full row capacity
  const int32_t cap = (int32_t)((int64_t)bt_stride * cache->block_size > kMaxCtx ? kMaxCtx : (int64_t)bt_stride * cache->block_size);
  if ((st = check_rows(cache, block_table, bt_stride, row_seq, nullptr, R, cap, false, &rm))) return st;
  if (q_lat == nullptr || idx == nullptr || out == nullptr) return fail(DSA_ERR_NULL, "q_lat / idx / out is NULL");
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_ARG, "k %d out of [1, %d]", k, DSA_MAX_K);
  if (!aligned16(q_lat)) return fail(DSA_ERR_ALIGN, "q_lat is not 16-byte aligned");
  const size_t need = mla_ws_bytes(R, k);
  if (mla_plan(R, k, cv.latent_fmt == DSA_LATENT_FP8).nsplit > 1 && (workspace == nullptr || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (R == 0) return ok();
  return hip_status(launch_sparse_mla(cv, rm, q_lat, idx, nullptr, R, k, sm_scale, out, lse, workspace, 3,
                                      static_cast<hipStream_t>(stream)),
                    "sparse_mla");
}

dsa_status dsa_cache_append(const dsa_cache_desc* cache, int32_t layer, const int32_t* block_table, int32_t bt_stride,
                            const int32_t* row_seq, const int32_t* pos, const float* idx_key, const float* latent,
                            int32_t R, void* stream) {
  CacheView cv;
  dsa_status st = check_cache(cache, layer, &cv);
  if (st) return st;
  if (R < 0 || R > 65535) return fail(DSA_ERR_ARG, "R %d out of [0, 65535]", R);
  if (R == 0) return ok();
  if (block_table == nullptr || row_seq == nullptr || pos == nullptr)
    return fail(DSA_ERR_NULL, "block_table / row_seq / pos is NULL");
  if (idx_key == nullptr && latent == nullptr) return fail(DSA_ERR_NULL, "both idx_key and latent are NULL");
  if (bt_stride < 1) return fail(DSA_ERR_ARG, "bt_stride %d < 1", bt_stride);
  if ((reinterpret_cast<uintptr_t>(idx_key) | reinterpret_cast<uintptr_t>(latent)) & 3u)
    return fail(DSA_ERR_ALIGN, "idx_key / latent is not 4-byte aligned");
  return hip_status(launch_cache_append(cv, cache->index_fmt, block_table, bt_stride, row_seq, pos, idx_key, latent, R,
                                        static_cast<hipStream_t>(stream)),
                    "cache_append");
}

dsa_status dsa_decode_step_stages(const dsa_cache_desc* cache, int32_t layer, const void* q_idx,
                                  const void* q_idx_scale, const float* w, const uint16_t* q_lat,
                                  const int32_t* block_table, int32_t bt_stride, const int32_t* row_seq,
                                  const int32_t* row_ctx, int32_t R, int32_t max_ctx, int32_t k, int32_t rows_per_seq,
                                  float sm_scale, int32_t* idx, float* out, float* lse, void* workspace,
                                  size_t ws_bytes, uint32_t stages, void* stream) {
  CacheView cv;
  RowMap rm;
  dsa_status st = check_cache(cache, layer, &cv);
  if (st) return st;
  if ((st = check_rows(cache, block_table, bt_stride, row_seq, row_ctx, R, max_ctx, true, &rm))) return st;
  if (q_idx == nullptr || q_idx_scale == nullptr || w == nullptr || q_lat == nullptr || idx == nullptr || out == nullptr)
    return fail(DSA_ERR_NULL, "q_idx / q_idx_scale / w / q_lat / idx / out is NULL");
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_ARG, "k %d out of [1, %d]", k, DSA_MAX_K);
  if (rows_per_seq < 1) return fail(DSA_ERR_ARG, "rows_per_seq %d < 1", rows_per_seq);
  if (stages == 0u || (stages & ~(uint32_t)DSA_STAGE_ALL) != 0u) return fail(DSA_ERR_ARG, "stages 0x%x", stages);
  if (!aligned16(q_idx) || !aligned16(q_lat)) return fail(DSA_ERR_ALIGN, "q_idx / q_lat is not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(q_idx_scale) & 3u) return fail(DSA_ERR_ALIGN, "q_idx_scale is not 4-byte aligned");
  const size_t need = decode_ws(R, max_ctx, k);
  if (workspace == nullptr || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(workspace)) return fail(DSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (R == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* p = static_cast<uint8_t*>(workspace);
  const int64_t ld = scores_ld(max_ctx);
  float* scores = reinterpret_cast<float*>(p);
  p += align_up((size_t)R * ld * 4, 256);
  TopkWs tw = topk_ws_carve(p, R, max_ctx);
  p += topk_ws_bytes(R, max_ctx);
  int32_t* phys = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)R * k * 4, 256);
  void* mla_ws = p;
  hipError_t e = hipSuccess;
  if (stages & DSA_STAGE_INDEXER)
    e = launch_indexer(cache->index_fmt, cv, rm, q_idx, q_idx_scale, w, R, rows_per_seq, scores, ld, &tw, s);
  const int umax = send_umax(rows_per_seq);
  // the selected tokens lie below max_ctx, so the row map's bound is unchanged
  int parts = ((stages & DSA_STAGE_ATTENTION) ? 1 : 0) | ((stages & DSA_STAGE_MERGE) ? 2 : 0);
  if (e == hipSuccess && (stages & DSA_STAGE_TOPK) && (parts & 1) && select_mla_fused(cv, R, k)) {
    // select and attention in one launch; the page slots stay on chip
    e = launch_select_mla(scores, ld, row_ctx, R, max_ctx, k, umax, idx, tw, cv, rm, q_lat, sm_scale, out, lse,
                          mla_ws, s);
    parts &= 2;
  } else if (e == hipSuccess && (stages & DSA_STAGE_TOPK)) {
    e = launch_topk_select(scores, ld, row_ctx, R, max_ctx, k, umax, idx, tw, phys, &cv, &rm, s);
  }
  if (e == hipSuccess && parts) e = launch_sparse_mla(cv, rm, q_lat, idx, phys, R, k, sm_scale, out, lse, mla_ws, parts, s);
  return hip_status(e, "decode_step");
}

dsa_status dsa_decode_step_multi(const dsa_cache_desc* cache, int32_t layer, const void* q_idx,
                                 const void* q_idx_scale, const float* w, const uint16_t* q_lat,
                                 const int32_t* block_table, int32_t bt_stride, const int32_t* row_seq,
                                 const int32_t* row_ctx, int32_t R, int32_t max_ctx, int32_t k, int32_t rows_per_seq,
                                 float sm_scale, int32_t* idx, float* out, float* lse, void* workspace,
                                 size_t ws_bytes, void* stream) {
  return dsa_decode_step_stages(cache, layer, q_idx, q_idx_scale, w, q_lat, block_table, bt_stride, row_seq, row_ctx, R,
                                max_ctx, k, rows_per_seq, sm_scale, idx, out, lse, workspace, ws_bytes, DSA_STAGE_ALL,
                                stream);
}

dsa_status dsa_decode_step(const dsa_cache_desc* cache, int32_t layer, const void* q_idx, const void* q_idx_scale,
                           const float* w, const uint16_t* q_lat, const int32_t* block_table, int32_t bt_stride,
                           const int32_t* row_seq, const int32_t* row_ctx, int32_t R, int32_t max_ctx, int32_t k,
                           float sm_scale, int32_t* idx, float* out, float* lse, void* workspace, size_t ws_bytes,
                           void* stream) {
  return dsa_decode_step_multi(cache, layer, q_idx, q_idx_scale, w, q_lat, block_table, bt_stride, row_seq, row_ctx, R,
                               max_ctx, k, 1, sm_scale, idx, out, lse, workspace, ws_bytes, stream);
}

dsa_status dsa_decode_step_noalloc(const dsa_cache_desc* cache, int32_t layer, const void* q_idx,
                                   const void* q_idx_scale, const float* w, const uint16_t* q_lat,
                                   const int32_t* block_table, int32_t bt_stride, const int32_t* row_seq,
                                   const int32_t* row_ctx, int32_t R, int32_t max_ctx, int32_t k,
                                   int32_t rows_per_seq, float sm_scale, int32_t* idx, float* out, float* lse,
                                   void* stream) {
  if (R < 0 || R > 65535) return fail(DSA_ERR_ARG, "R %d out of [0, 65535]", R);
  if (max_ctx < 0 || max_ctx > kMaxCtx) return fail(DSA_ERR_ARG, "max_ctx %d out of [0, %d]", max_ctx, kMaxCtx);
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_ARG, "k %d out of [1, %d]", k, DSA_MAX_K);
  const size_t need = decode_ws(R, max_ctx, k);
  if (need > (size_t)DSA_STATIC_SCRATCH_BYTES)
    return fail(DSA_ERR_WORKSPACE, "the step needs %zu bytes of workspace, more than the %u-byte static scratch",
                need, (unsigned)DSA_STATIC_SCRATCH_BYTES);
  void* ws = scratch_addr();
  if (ws == nullptr) return fail(DSA_ERR_HIP, "the static scratch has no address on this device");
  return dsa_decode_step_multi(cache, layer, q_idx, q_idx_scale, w, q_lat, block_table, bt_stride, row_seq, row_ctx, R,
                               max_ctx, k, rows_per_seq, sm_scale, idx, out, lse, ws, DSA_STATIC_SCRATCH_BYTES, stream);
}

size_t dsa_topk_dcp_workspace_bytes(int32_t R, int32_t max_ctx, int32_t k, int32_t W) {
  if (R < 0 || max_ctx < 0 || max_ctx > kMaxCtx || k < 1 || k > DSA_MAX_K || W < 2 || W > kDcpShardMax) return 0;
  return dcp_ws_bytes(R, max_ctx, k, W);
}

dsa_status dsa_topk_dcp(const float* scores, int64_t ld_scores, const int32_t* row_ctx, int32_t R, int32_t max_ctx,
                        int32_t k, int32_t W, int32_t* idx, uint32_t* resend_mask, uint32_t* words, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (scores == nullptr || row_ctx == nullptr || idx == nullptr) return fail(DSA_ERR_NULL, "scores / row_ctx / idx is NULL");
  if (W < 2 || W > kDcpShardMax) return fail(DSA_ERR_ARG, "W %d out of [2, %d]", W, kDcpShardMax);
  if (R < 0 || (int64_t)R * W > 65535) return fail(DSA_ERR_ARG, "R %d x W %d out of [0, 65535]", R, W);
  if (k < 1 || k > DSA_MAX_K) return fail(DSA_ERR_ARG, "k %d out of [1, %d]", k, DSA_MAX_K);
  if (max_ctx < 0 || max_ctx > kMaxCtx) return fail(DSA_ERR_ARG, "max_ctx %d out of [0, %d]", max_ctx, kMaxCtx);
  if (ld_scores < max_ctx) return fail(DSA_ERR_ARG, "ld_scores %lld < max_ctx %d", (long long)ld_scores, max_ctx);
  const size_t need = dcp_ws_bytes(R, max_ctx, k, W);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(workspace)) return fail(DSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (R == 0) return ok();
  return hip_status(launch_topk_dcp(scores, ld_scores, row_ctx, R, max_ctx, k, W, idx, resend_mask, words, workspace,
                                    static_cast<hipStream_t>(stream)),
                    "topk_dcp");
}

dsa_status dsa_hbm_read_probe(const void* p, size_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (p == nullptr || sink == nullptr) return fail(DSA_ERR_NULL, "buffer / sink is NULL");
  if (!aligned16(p) || (bytes & 15u)) return fail(DSA_ERR_ALIGN, "buffer is not 16-byte aligned or bytes %% 16 != 0");
  if (grid < 1 || grid > 65535) return fail(DSA_ERR_ARG, "grid %d out of [1, 65535]", grid);
  if (bytes == 0) return ok();
  return hip_status(launch_hbm_read(p, bytes, sink, grid, static_cast<hipStream_t>(stream)), "hbm_read_probe");
}

}  // extern "C"
