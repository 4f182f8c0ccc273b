/*
 * dsa.h - C ABI of a DeepSeek-style sparse attention (DSA) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (vLLM "Day-0 support for Kimi K3.1 Pro", section "Sparse attention
 * in K3.1 Pro"): a small indexer scores every earlier token of a query with 32
 * light heads, the 2,048 best tokens are kept, and MLA attention then runs
 * exactly, but over those tokens only. All cache reads go through a block table
 * into a packed per-block cache row (same page, section on the KV cache that
 * serves three kinds of state: one contiguous row per block holds every DSA
 * layer's latent page and index-key page; block and slot are turned into page
 * addresses before each step).
 *
 * Definitions used by every entry point (R query rows, layer l):
 *   score[r][t] = sum_{h<32} w[r][h] * ReLU(q_h . k_t),  t in [0, ctx[r])
 *   idx[r]      = the min(k, ctx[r]) tokens with the largest fp32 score, equal
 *                 scores ordered by lower token index; written in ascending token
 *                 order, the rest of the k slots set to -1
 *   out[r][h]   = sum_t softmax_t(sm_scale * q_lat[r][h] . c_t) * c_t[0:512]
 *                 over t in idx[r] (c_t = latent scale * e4m3 codes, 576 wide)
 *   lse[r][h]   = natural log of sum_t exp(sm_scale * q_lat[r][h] . c_t)
 *
 * Memory: every pointer argument except `cache` itself is a DEVICE pointer,
 * except where marked (host). The caller owns every buffer. The library never
 * allocates or frees, and only dsa_device_status synchronises; all work is enqueued
 * on `stream` (a hipStream_t; NULL = the default stream). Calls are stateless (apart
 * from the device status word at the end of this header) and may be made from
 * several host threads on different streams with different workspaces.
 *
 * Errors: a non-zero dsa_status is returned before anything is enqueued when an
 * argument is invalid; dsa_last_error_detail() then holds a message for the
 * calling thread. DSA_ERR_HIP is returned when a launch fails. Data-dependent
 * problems found on the device never fault: a row's ctx above the block-table
 * capacity or max_ctx is clamped, ctx <= 0 gives an empty row (idx all -1, out 0,
 * lse -inf), and a block id outside [0, num_blocks) is clamped into the pool
 * (that token's values are then unspecified). The kernels record each such repair
 * in a per-device status word (dsa_device_status, at the end of this header).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

#define DSA_H_IDX 32      /* indexer heads */
#define DSA_D_IDX 128     /* indexer head dim */
#define DSA_H_Q 96        /* latent-query heads */
#define DSA_D_LAT 576     /* latent width (attention keys) */
#define DSA_D_V 512       /* value width (first 512 latent dims) */
#define DSA_MAX_K 2048    /* largest supported top-k */
#define DSA_MAX_LAYERS 64

typedef int32_t dsa_status;
#define DSA_OK 0
#define DSA_ERR_NULL 1          /* a required pointer is NULL */
#define DSA_ERR_ARG 2           /* a size / count / index is out of range */
#define DSA_ERR_LAYOUT 3        /* cache descriptor is inconsistent */
#define DSA_ERR_WORKSPACE 4     /* workspace smaller than dsa_workspace_bytes() */
#define DSA_ERR_ALIGN 5         /* a pointer or offset is not 16-byte aligned */
#define DSA_ERR_HIP 6           /* a HIP launch failed */
#define DSA_ERR_UNSUPPORTED 7   /* format or shape not supported */

/* Index-key page formats (page 1, KV-cache section: FP8 keys are 132 B/token,
 * MXFP4 keys 68 B/token). */
#define DSA_INDEX_FP8 0    /* 128 e4m3 codes + fp32 scale per token */
#define DSA_INDEX_MXFP4 1  /* 64 B packed e2m1 (element 2i = low nibble) + 4 E8M0 per token */

/* Latent page formats (page 1, KV-cache section: a token's latent takes 576 B in
 * FP8 and 352 B in NVFP4). Each token record is followed, after the page's
 * block_size records, by one fp32 scale per token (the value scale s below). */
#define DSA_LATENT_FP8 0    /* 576 e4m3 codes: c[d] = s * e4m3[d] */
#define DSA_LATENT_NVFP4 1  /* 352 B: 256 B packed e2m1 for dims 0..511 (element 2i =
                             * low nibble), 32 e4m3 block scales (one per 16 dims),
                             * 64 e4m3 codes for dims 512..575:
                             * c[d] = s * e4m3(bsc[d/16]) * e2m1[d], d < 512;
                             * c[d] = s * e4m3(tail[d-512]), d >= 512 */

/*
 * Packed cache descriptor (host struct; `pool` is a device pointer).
 * Block row b starts at pool + b * row_bytes. Inside a row, layer l holds
 *   latent page at lat_off[l]: block_size records of W bytes (slot s at s*W;
 *                              W = 576 for DSA_LATENT_FP8, 352 for DSA_LATENT_NVFP4),
 *                              then block_size fp32 scales;
 *   index page  at idx_off[l]: FP8   block_size * 128 e4m3 codes, then block_size fp32 scales;
 *                              MXFP4 block_size * 64 packed bytes, then block_size * 4 E8M0.
 * Token t of a sequence lives in block block_table[seq][t / block_size], slot
 * t % block_size. block_size must be a power of two; pool, row_bytes and every
 * offset must be multiples of 16.
 */
typedef struct dsa_cache_desc {
  void* pool;
  int64_t row_bytes;
  int64_t num_blocks;
  int32_t block_size;
  int32_t num_layers;
  int32_t index_fmt;
  int32_t latent_fmt;  /* DSA_LATENT_FP8 (0) or DSA_LATENT_NVFP4 (1) */
  int64_t lat_off[DSA_MAX_LAYERS];
  int64_t idx_off[DSA_MAX_LAYERS];
} dsa_cache_desc;

/* Operation ids for dsa_workspace_bytes. */
#define DSA_OP_TOPK 1
#define DSA_OP_SPARSE_MLA 2
#define DSA_OP_DECODE_STEP 3

int32_t dsa_abi_version(void);
const char* dsa_status_string(dsa_status status);
/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* dsa_last_error_detail(void);

/* Bytes of device workspace an operation needs for R rows, max_ctx tokens and
 * top-k k. 0 for an unknown op. The workspace needs no initial contents. */
size_t dsa_workspace_bytes(int32_t op, int32_t R, int32_t max_ctx, int32_t k);
/* Row stride (floats) of the score array a decode step keeps at the start of
 * its workspace: scores of row r, token t are at ((float*)workspace)[r*ld + t]. */
int64_t dsa_decode_scores_ld(int32_t max_ctx);

/*
 * Indexer (page 1, "Sparse attention in K3.1 Pro": 32 light heads score every
 * earlier token; page 3, model table: 32 heads x 128 dims, FP8 keys; page 1,
 * AMD section: MXFP4 keys scored with native FP4 matrix instructions and fp32
 * accumulation, then a weighted reduction across heads).
 *   q_idx        FP8:   R x 32 x 128 e4m3 codes;   MXFP4: R x 32 x 64 packed e2m1
 *   q_idx_scale  FP8:   R x 32 fp32 (one positive scale per head);
 *                MXFP4: R x 32 x 4 E8M0 bytes (one per 32 elements)
 *   w            R x 32 fp32 head weights (any sign)
 *   block_table  int32 [num_seqs][bt_stride]; row_seq[r] selects the row of query r
 *   row_ctx      int32 [R]: query r scores tokens [0, row_ctx[r])
 *   max_ctx      host bound: row_ctx[r] <= max_ctx <= bt_stride * block_size
 *   scores       fp32 [R][ld_scores], ld_scores >= max_ctx; entries t >= ctx[r]
 *                are left untouched.
 * Key and query scales must be positive (the kernel factors them out of ReLU).
 * q_idx must be 16-byte and q_idx_scale 4-byte aligned (DSA_ERR_ALIGN otherwise).
 */
dsa_status dsa_indexer_score(const dsa_cache_desc* cache, int32_t layer,
                             const void* q_idx, const void* q_idx_scale, const float* w,
                             const int32_t* block_table, int32_t bt_stride,
                             const int32_t* row_seq, const int32_t* row_ctx,
                             int32_t R, int32_t max_ctx,
                             float* scores, int64_t ld_scores, void* stream);

/*
 * Exact top-k (page 1, fused decode path: an exact top-k selection emits the KV
 * rows attention reads; page 1, zero-mismatch RL: batch-invariant top-k).
 * Selection is per row, exact in fp32, ties -> lower token index, -0.0 == +0.0.
 *   scores  fp32 [R][ld_scores]; row_ctx as above; k in [1, 2048]
 *   idx     int32 [R][k] output, ascending tokens then -1 padding.
 *   workspace >= dsa_workspace_bytes(DSA_OP_TOPK, R, max_ctx, k)
 */
dsa_status dsa_topk(const float* scores, int64_t ld_scores, const int32_t* row_ctx,
                    int32_t R, int32_t max_ctx, int32_t k, int32_t* idx,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * Sparse MLA over the selected tokens (page 1, "Sparse attention in K3.1 Pro":
 * MLA runs exactly over the 2,048 kept tokens; page 1 AMD section: the selected
 * tokens are read directly from the FP8 cache; page 3 model table: NoPE).
 *   q_lat   bf16 bit patterns, R x 96 x 576 (absorbed query in latent space)
 *   idx     int32 [R][k]; entries < 0 are skipped, others must be < the row's
 *           block-table capacity
 *   out     fp32 [R][96][512]; lse fp32 [R][96] (may be NULL)
 *   workspace >= dsa_workspace_bytes(DSA_OP_SPARSE_MLA, R, 0, k)
 */
dsa_status dsa_sparse_mla(const dsa_cache_desc* cache, int32_t layer,
                          const uint16_t* q_lat, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* row_seq, const int32_t* idx, int32_t R, int32_t k,
                          float sm_scale, float* out, float* lse,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * The whole decode step for one layer: indexer -> exact top-k -> sparse MLA ->
 * split merge, enqueued back to back on one stream (page 1, fused DSA decode
 * path: a scorer and an exact top-k in two kernels, then sparse attention).
 * Arguments as in the three calls above. Scores stay in the workspace (see
 * dsa_decode_scores_ld); idx [R][k], out [R][96][512] and lse [R][96] (nullable)
 * are written. Rows may share a sequence (prefill-append: row r of an append of
 * T tokens on a P-token prefix uses row_ctx[r] = P + r + 1).
 *   workspace >= dsa_workspace_bytes(DSA_OP_DECODE_STEP, R, max_ctx, k)
 */
dsa_status dsa_decode_step(const dsa_cache_desc* cache, int32_t layer,
                           const void* q_idx, const void* q_idx_scale, const float* w,
                           const uint16_t* q_lat,
                           const int32_t* block_table, int32_t bt_stride,
                           const int32_t* row_seq, const int32_t* row_ctx,
                           int32_t R, int32_t max_ctx, int32_t k, float sm_scale,
                           int32_t* idx, float* out, float* lse,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * Several query rows per sequence (page 1: the 2K-token append on a 150K prefix,
 * every appended token a query row; the AMD section: several speculative-verify
 * tokens per sequence whose queries share one key scan, keys reused across query
 * rows). Same as dsa_indexer_score / dsa_decode_step, plus
 *   rows_per_seq  >= 1: rows come in runs of this many consecutive rows that share
 *                 a sequence (row_seq equal), e.g. T for a T-token append or the
 *                 draft length + 1 for speculative verification; 1 = no sharing.
 * With rows_per_seq > 1 the indexer reads each key once (FP8: and converts it once)
 * for up to 16 consecutive rows, for FP8 and MXFP4 keys alike. It is a performance
 * hint only: a row whose row_seq differs from the row before it reloads the keys, so
 * results never depend on it. DSA_ERR_ARG if rows_per_seq < 1.
 */
dsa_status dsa_indexer_score_multi(const dsa_cache_desc* cache, int32_t layer,
                                   const void* q_idx, const void* q_idx_scale, const float* w,
                                   const int32_t* block_table, int32_t bt_stride,
                                   const int32_t* row_seq, const int32_t* row_ctx,
                                   int32_t R, int32_t max_ctx, int32_t rows_per_seq,
                                   float* scores, int64_t ld_scores, void* stream);
dsa_status dsa_decode_step_multi(const dsa_cache_desc* cache, int32_t layer,
                                 const void* q_idx, const void* q_idx_scale, const float* w,
                                 const uint16_t* q_lat,
                                 const int32_t* block_table, int32_t bt_stride,
                                 const int32_t* row_seq, const int32_t* row_ctx,
                                 int32_t R, int32_t max_ctx, int32_t k, int32_t rows_per_seq,
                                 float sm_scale, int32_t* idx, float* out, float* lse,
                                 void* workspace, size_t ws_bytes, void* stream);

/*
 * New-token cache append, the step just before the hot path (page 1, fused
 * front-end: the new token's index key is quantised and written, and its latent is
 * written into the packed cache, before scoring). For each row r, token pos[r] of
 * block-table row row_seq[r] gets, for `layer`:
 *   idx_key  R x 128 fp32 (nullable): FP8 pool: e4m3 codes of x / s with one fp32
 *            scale s = amax / 448 (1 if amax = 0), values clamped to +-448, rounded to
 *            nearest, ties to the even code; MXFP4 pool: per 32 elements the E8M0
 *            exponent E + 127 with E = floor(log2 amax) - 2 (clamped to [-127, 127], 0
 *            if amax = 0) and e2m1 codes of x / 2^E, nearest, ties to even, at most 6.
 *   latent   R x 576 fp32 (nullable): e4m3 codes + fp32 scale as for an FP8 key.
 * (The quantiser is this library's reading; the pages do not spell one out.)
 * Rows whose pos is negative or past the table, or whose block id lies outside
 * [0, num_blocks), write nothing. Rows must target distinct slots (writes of two
 * rows to one slot race). DSA_ERR_NULL if both inputs are NULL.
 */
dsa_status dsa_cache_append(const dsa_cache_desc* cache, int32_t layer,
                            const int32_t* block_table, int32_t bt_stride,
                            const int32_t* row_seq, const int32_t* pos,
                            const float* idx_key, const float* latent,
                            int32_t R, void* stream);

/*
 * Exact top-k merge of decode context parallelism, emulated on one GPU (page 1,
 * long-context section on decode context parallelism with the sparse indexer: W
 * GPUs each hold every W-th token; sub-section on the exact top-k merge with ten
 * times less traffic: each sends its best ceil(1.5 k / W) candidates as 32-bit
 * words built from BF16 scores, all radix-select the same global top-k from the
 * gathered words, and a GPU holding more of the top-k than it sent resends its
 * full local top-k). Shard s of each row holds tokens t = s (mod W); each shard
 * ranks its own tokens, and the merge runs as the pages describe:
 *   word     (key << 16) | j for slot j of the shard's list (its tokens in
 *            ascending order), key = the score rounded to the nearest BF16 value
 *            (ties to even) as an order-preserving 16-bit key (b | 0x8000 for a
 *            non-negative bit pattern b, ~b & 0xFFFF for a negative one; -0 as +0)
 *   T        key of the k-th largest word (0 if fewer than k words were sent)
 *   resend   shard s resends iff it holds more tokens than it sent, sent at least
 *            one, and its smallest sent key is >= T
 *   result   exact fp32 top-k over the sent candidates with key >= T of the other
 *            shards and the full local top-k of the resending ones.
 * The result equals dsa_topk's on the same scores (the merge is exact).
 *   scores, ld_scores, row_ctx, R, max_ctx, k  as for dsa_topk; R * W <= 65535
 *   W            shards, 2 .. 32
 *   idx          int32 [R][k] output, as dsa_topk
 *   resend_mask  uint32 [R] output (nullable): bit s set when shard s resent
 *   words        uint32 [R][W * M] output (nullable), M = ceil(1.5 k / W): the word
 *                shard s sent at slot j at s * M + j, 0xFFFFFFFF where it sent none
 *   workspace >= dsa_topk_dcp_workspace_bytes(R, max_ctx, k, W), 16-byte aligned
 */
size_t dsa_topk_dcp_workspace_bytes(int32_t R, int32_t max_ctx, int32_t k, int32_t W);
dsa_status dsa_topk_dcp(const float* scores, int64_t ld_scores, const int32_t* row_ctx,
                        int32_t R, int32_t max_ctx, int32_t k, int32_t W, int32_t* idx,
                        uint32_t* resend_mask, uint32_t* words,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * Device status word. Data problems that the kernels repair instead of faulting
 * (see the top of this header) are also reported: each GPU holds one 32-bit word,
 * shared by every call on it, into which kernels OR
 *   DSA_DEV_CTX_CLAMPED    a row_ctx above max_ctx was used as max_ctx
 *                          (indexer, top-k, decode step);
 *   DSA_DEV_BLOCK_CLAMPED  a block-table entry outside [0, num_blocks) was met: reads
 *                          clamp it into the pool, cache appends skip the row;
 *   DSA_DEV_INDEX_RANGE    sparse MLA skipped an idx entry at or past the block-table
 *                          row's capacity.
 * The word keeps its bits until cleared. dsa_device_status waits for the work queued on
 * `stream` (it synchronises that stream, unlike every other call here), stores the word
 * of the current device in *status, and then clears it when `clear` is nonzero. Calls
 * that run concurrently on one device report into the same word. The word's device
 * address is looked up (hipGetSymbolAddress) on the library's first call on each
 * device; calls made while that lookup fails report nothing. dsa_topk_dcp does not
 * report. DSA_ERR_NULL for a NULL status, DSA_ERR_HIP if the word cannot be read.
 */
#define DSA_DEV_CTX_CLAMPED 1u
#define DSA_DEV_BLOCK_CLAMPED 2u
#define DSA_DEV_INDEX_RANGE 4u
dsa_status dsa_device_status(void* stream, int32_t clear, uint32_t* status);

/*
 * Measurement entry point, not a step of the method: dsa_decode_step_multi with the
 * same arguments and workspace, enqueuing only the kernels of the chosen stages, in
 * the step's order, so that each kernel of a decode step can be timed alone (the
 * benchmark's roofline times the step's own indexer launch this way). Running
 * DSA_STAGE_INDEXER, then DSA_STAGE_TOPK, then DSA_STAGE_ATTENTION | DSA_STAGE_MERGE on
 * one workspace equals one dsa_decode_step_multi call; a stage reads what the stages
 * before it left in the workspace (or in idx), so running a later stage alone repeats
 * its work on the previous call's intermediate results. A mask holding both
 * DSA_STAGE_TOPK and DSA_STAGE_ATTENTION may run them as one launch (the step does so
 * for one row with FP8 latents); that launch keeps the selected tokens' page slots on
 * chip, so a later DSA_STAGE_ATTENTION alone reads those of the last DSA_STAGE_TOPK run
 * without DSA_STAGE_ATTENTION. DSA_ERR_ARG for an empty mask or unknown bits.
 */
#define DSA_STAGE_INDEXER 1u    /* indexer scores and the top-k candidate stage */
#define DSA_STAGE_TOPK 2u       /* exact top-k selection (writes idx) */
#define DSA_STAGE_ATTENTION 4u  /* sparse MLA over idx */
#define DSA_STAGE_MERGE 8u      /* merge of the rows' split partials (when rows are split) */
#define DSA_STAGE_ALL 15u
dsa_status dsa_decode_step_stages(const dsa_cache_desc* cache, int32_t layer,
                                  const void* q_idx, const void* q_idx_scale, const float* w,
                                  const uint16_t* q_lat,
                                  const int32_t* block_table, int32_t bt_stride,
                                  const int32_t* row_seq, const int32_t* row_ctx,
                                  int32_t R, int32_t max_ctx, int32_t k, int32_t rows_per_seq,
                                  float sm_scale, int32_t* idx, float* out, float* lse,
                                  void* workspace, size_t ws_bytes, uint32_t stages, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): dsa_decode_step_multi without a
 * workspace argument. Its workspace is a static device array of DSA_STATIC_SCRATCH_BYTES
 * that every GPU running this library holds until the process ends; its address on a
 * device is looked up (hipGetSymbolAddress) on the call's first use there. The call
 * allocates and frees nothing. It returns DSA_ERR_WORKSPACE, before anything is enqueued,
 * when dsa_workspace_bytes(DSA_OP_DECODE_STEP, R, max_ctx, k) exceeds the array (32 MiB
 * covers e.g. one row of 1,048,576 tokens, or 16 rows of 65,536), and DSA_ERR_HIP when
 * the address lookup fails. Every call on one GPU uses the same array, which keeps the
 * last call's contents (the step needs no initial contents): calls that overlap in time
 * on one device (several streams or host threads) race, and the caller must serialise
 * them. Other arguments and errors as for dsa_decode_step_multi.
 */
#define DSA_STATIC_SCRATCH_BYTES (32u << 20)
dsa_status dsa_decode_step_noalloc(const dsa_cache_desc* cache, int32_t layer,
                                   const void* q_idx, const void* q_idx_scale, const float* w,
                                   const uint16_t* q_lat,
                                   const int32_t* block_table, int32_t bt_stride,
                                   const int32_t* row_seq, const int32_t* row_ctx,
                                   int32_t R, int32_t max_ctx, int32_t k, int32_t rows_per_seq,
                                   float sm_scale, int32_t* idx, float* out, float* lse,
                                   void* stream);

/*
 * Measurement reference, not a step of the method: reads every byte of
 * [p, p + bytes) once (16-byte nontemporal loads; `grid` workgroups of 256 threads
 * take 16-KB chunks in turn) and writes nothing, except *sink in the practically
 * impossible case that the XOR of the words one thread read equals 0x9E3779B9 (the
 * condition keeps the loads from being optimised away). Timed over a
 * buffer much larger than the last-level cache it gives the streaming-read rate the
 * indexer's HBM roofline can be compared with. p 16-byte aligned, bytes a multiple of
 * 16 (DSA_ERR_ALIGN), grid in [1, 65535] (DSA_ERR_ARG), sink a device uint32.
 */
dsa_status dsa_hbm_read_probe(const void* p, size_t bytes, uint32_t* sink, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
