/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) MLA decode library
 * (libmla_decode.so).
 *
 * Multi-head latent attention decode over a paged KV cache.  Every query
 * token has num_heads_q heads of width head_dim = 576: a 512-wide latent part
 * followed by a 64-wide rope part.  All heads of one KV group attend to one
 * shared cached row per key; V is the first head_dim_v = 512 columns of those
 * same rows.
 *
 * Sources (web pages; cited by title and section):
 *   - FlashMLA interface page (flash_mla_interface.py): docstrings of
 *     get_mla_metadata and flash_mla_with_kvcache -- argument shapes, the
 *     default scale 1/sqrt(head_dim), the causal flag, the outputs out and
 *     softmax_lse, and the metadata/attention call pair.
 *   - vLLM vllm.attention.ops.flashmla page: the same two calls; the
 *     platform gate is_flashmla_supported returning (supported, reason).
 *   - FlashInfer trtllm_batch_decode_with_kv_cache_mla page: query is
 *     q_nope ++ q_rope, the cache is ckv ++ kpe (512 + 64); caller-provided
 *     out; the note on fused fp8 scales bmm1/bmm2.
 *   - Ascend ATB MLA page (AtbMLAGetWorkspaceSize / AtbMLA): a status-code C
 *     API with a workspace-size query before the run.
 *
 * Conventions for every entry point:
 *   - Plain C types; device buffers are device pointers (hipMalloc'd or
 *     torch-owned); `stream` is a hipStream_t passed as void* (NULL = the
 *     default stream).
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; device calls only enqueue work on `stream`.
 *   - All arguments are validated on the host before any HIP call; on error
 *     nothing is enqueued and a non-zero mla_status is returned.  No entry
 *     point throws or aborts.
 *   - Layouts are dense row-major (C order) with the shapes given below.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Ints per row of the tile-scheduler table ("TileSchedulerMetaDataSize"). */
#define MLA_TILE_MD_INTS 8
/* Fixed shape of the absorbed-MLA problem (FlashInfer MLA page: kv_lora_rank
 * 512, qk_rope_head_dim 64). */
#define MLA_HEAD_DIM 576
#define MLA_HEAD_DIM_V 512
/* Tokens per scheduling page: the split-KV metadata counts sequence lengths
 * and split boundaries in pages of this many tokens, whatever the cache's
 * block size (FlashMLA interface page: the cache block of 64 tokens). */
#define MLA_PAGE_BLOCK_SIZE 64
/* The cache's page_block_size must be a multiple of this (the kernels copy a
 * block's rows in 16-token slices). */
#define MLA_PAGE_BLOCK_ALIGN 16
/* Largest batch the scheduler kernel accepts. */
#define MLA_MAX_BATCH 8192
/* Largest rows per KV head (s_q * num_heads_q / num_heads_k). */
#define MLA_MAX_ROWS 1024
/* Bytes of the library's static device scratch used by mla_decode_fwd_noalloc
 * (128 MiB per GPU, held until the process ends). */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,         /* null pointer, non-positive size, inconsistent sizes */
  MLA_ERR_UNSUPPORTED = 2,         /* valid request this build does not implement, or a non-gfx950 device */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < mla_workspace_bytes(...) */
  MLA_ERR_NO_DEVICE = 4,           /* no HIP device visible */
  MLA_ERR_HIP = 5                  /* a HIP runtime call or kernel launch failed */
};

enum mla_kv_dtype {
  MLA_KV_BF16 = 0,        /* cache rows are bf16 */
  MLA_KV_FP8_E4M3FN = 1   /* cache rows are OCP FP8 E4M3 codes (finite max 448) */
};

enum mla_q_dtype {
  MLA_Q_BF16 = 0,         /* q is bf16 */
  MLA_Q_FP8_E4M3FN = 1    /* q is OCP FP8 E4M3 codes (mla_decode_fwd_ext only) */
};

/* Human-readable text for a status code (static storage; never NULL).  The
 * UNSUPPORTED text of the last failing call on this thread names the reason,
 * as the vLLM platform gate returns (supported, reason). */
const char *mla_status_str(int status);

/* Host only.  Recommended balancing target (parts) for this head layout on
 * the current device: one persistent workgroup per compute unit, divided
 * among the row tiles and KV heads.  The tile table has num_parts rows.
 *   heads_per_head_k = s_q * num_heads_q / num_heads_k  (FlashMLA interface
 *   page, get_mla_metadata: num_heads_per_head_k).
 * Writes *num_parts; returns MLA_OK, INVALID_ARG, NO_DEVICE or UNSUPPORTED. */
int mla_num_parts(int batch, int heads_per_head_k, int num_heads_k, int *num_parts);

/* Device, asynchronous on `stream`.  The split-KV tile scheduler
 * (FlashMLA interface page, get_mla_metadata: returns
 * tile_scheduler_metadata (num_sm_parts, TileSchedulerMetaDataSize) int32 and
 * num_splits (batch + 1) int32).
 *   cache_seqlens : device int32[batch], keys per sequence (>= 0).
 *   num_parts     : balancing target P >= 1, the number of equal-cost parts
 *                   the work is cut into (mla_num_parts gives the recommended
 *                   one); mla_decode_fwd must get the same value.
 *   tile_md       : device int32[num_parts * MLA_TILE_MD_INTS], written; one
 *                   row per part.
 *   num_splits    : device int32[batch + 1], written: an exclusive prefix
 *                   sum, num_splits[0] = 0 and num_splits[b+1]-num_splits[b]
 *                   >= 1 is the number of splits of sequence b (at most
 *                   batch + num_parts - 1 splits in all).
 * Part p works on a run of consecutive sequences b0..b1; row p of tile_md is
 * [b0, first page of b0, b1, end page of b1 (exclusive), split index k of
 * b0's piece, payload W, fixed_cost, number of splits of the part]; the
 * sequences strictly between b0 and b1 are whole, and b1's piece (when
 * b1 > b0) starts at page 0 and is its split 0.  An idle part has
 * b0 = b1 = -1.  Split k of sequence b is partial slot num_splits[b] + k.
 * The table depends only on cache_seqlens, the head layout and num_parts, so
 * one call serves every layer of a decode step.  No device-to-host
 * synchronisation happens. */
int mla_get_metadata(const int32_t *cache_seqlens, int batch, int heads_per_head_k, int num_heads_k,
                     int32_t *tile_md, int num_parts, int32_t *num_splits, void *stream);

/* As mla_get_metadata with an explicit per-split overhead `fixed_cost`
 * (in page units, >= 1) of the balancing cost model.  Sequence b costs
 * fixed_cost + ceil(L_b / 64) units: ceil(fixed_cost / 2) overhead units,
 * one unit per 64-token page, then the other floor(fixed_cost / 2) overhead
 * units; units are laid end to end in batch order and cut into num_parts
 * equal ranges of at most W = ceil(total / num_parts) units. */
int mla_get_metadata_ex(const int32_t *cache_seqlens, int batch, int heads_per_head_k, int num_heads_k,
                        int num_parts, int fixed_cost, int32_t *tile_md, int32_t *num_splits, void *stream);

/* Host only.  Bytes of split workspace mla_decode_fwd needs (bf16 partial
 * outputs and fp32 log-sum-exps of up to batch + num_parts - 1 splits; the
 * partial outputs of each KV head are kept in whole blocks of 32 rows), written
 * to *bytes.  Returns MLA_OK or INVALID_ARG. */
int mla_workspace_bytes(int batch, int s_q, int num_heads_q, int num_heads_k, int head_dim_v, int num_parts,
                        size_t *bytes);

/* Device, asynchronous on `stream`.  MLA decode attention
 * (FlashMLA interface page, flash_mla_with_kvcache; the pages' native call
 * takes q, k_cache, head_dim_v, cache_seqlens, block_table, softmax_scale,
 * causal, tile_scheduler_metadata, num_splits).
 *   q            : device bf16 [batch][s_q][num_heads_q][head_dim].
 *   kv_cache     : device [num_blocks][page_block_size][num_heads_k][head_dim],
 *                  bf16 or e4m3fn codes per kv_dtype.  Token t of sequence b
 *                  is row t % page_block_size of block
 *                  block_table[b][t / page_block_size].
 *   block_table  : device int32 [batch][max_blocks_per_seq].  Entries past
 *                  ceil(cache_seqlens[b] / page_block_size) are never read;
 *                  the rest must lie in [0, num_blocks) (not checked: that
 *                  would need a device read).  Cache rows past
 *                  cache_seqlens[b] in a sequence's last block are never read.
 *   cache_seqlens: device int32 [batch],
 *                  0 <= L_b <= max_blocks_per_seq * page_block_size.
 *   softmax_scale: factor >= 0 on q.k before the softmax (bmm1_scale for an
 *                  fp8 cache; a negative value is UNSUPPORTED).  The Python
 *                  wrapper supplies 1/sqrt(head_dim) when the caller gives
 *                  none, as the pages' wrappers do.
 *   v_scale      : factor on the weighted sum of V (bmm2_scale; 1 for bf16).
 *   causal       : 0 or 1.  Query i of s_q sees keys t < L_b - s_q + 1 + i
 *                  (bottom-right alignment).  A row with no visible key gets
 *                  out = 0 and lse = -inf.
 *   tile_md, num_parts, num_splits: from mla_get_metadata for these
 *                  cache_seqlens and this head layout, in 64-token pages
 *                  for any page_block_size (tile_md has num_parts
 *                  rows; one persistent workgroup per part and 128-row tile
 *                  of each KV head walks its row's run of sequences).
 *   workspace    : device buffer of >= mla_workspace_bytes(...) bytes,
 *                  contents ignored on entry.
 *   out          : device bf16 [batch][s_q][num_heads_q][head_dim_v], written.
 *   lse          : device fp32 [batch][num_heads_q][s_q], written: natural
 *                  log of sum_t exp(softmax_scale * q.k_t).
 * q head h uses KV head h / (num_heads_q / num_heads_k).
 * Requires head_dim = 576, head_dim_v = 512, page_block_size a positive
 * multiple of MLA_PAGE_BLOCK_ALIGN (the pages' caches use 64; FlashInfer
 * MLA page and Ascend ATB MLA page: any page or block size), a gfx950
 * device, and s_q * num_heads_q / num_heads_k <= MLA_MAX_ROWS. */
int mla_decode_fwd(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                   const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                   const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                   int head_dim_v, float softmax_scale, float v_scale, int causal,
                   const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                   void *workspace, size_t workspace_bytes,
                   void *out, float *lse, void *stream);

/* The two stages of mla_decode_fwd, for callers that time or overlap them
 * (same arguments and validation as mla_decode_fwd).
 *   mla_decode_splits : attention over every split of the tile table; writes
 *                       out / lse of sequences with one split and the
 *                       partials (bf16 normalised output, fp32 log-sum-exp)
 *                       of the others into the workspace.
 *   mla_combine_splits: merges the partials of sequences with more than one
 *                       split by their log-sum-exps into out / lse.  Must run
 *                       after mla_decode_splits with the same arguments. */
int mla_decode_splits(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                      const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                      const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                      int head_dim_v, float softmax_scale, float v_scale, int causal,
                      const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                      void *workspace, size_t workspace_bytes,
                      void *out, float *lse, void *stream);
int mla_combine_splits(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                       const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                       const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                       int head_dim_v, float softmax_scale, float v_scale, int causal,
                       const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                       void *workspace, size_t workspace_bytes,
                       void *out, float *lse, void *stream);

/* Optional inputs of mla_decode_fwd_ext.  A zeroed struct (or a NULL ext)
 * is plain mla_decode_fwd.  Every pointer is a device pointer or NULL.
 *   sinks      : fp32 [num_heads_q], per-head sink logits (FlashInfer
 *                trtllm_batch_decode_with_kv_cache_mla page, sinks: a per-head
 *                extra term of the softmax denominator).  Read as a logit on
 *                the scale of softmax_scale * q.k: head h's denominator gains
 *                exp(sinks[h]), which carries no value, and lse includes it;
 *                -inf is no sink.  Values must be finite or -inf.
 *   bmm1_scale : fp32 [1]; when set, replaces softmax_scale (same page: the
 *                fused bmm1/bmm2 scales may be device tensors, which then
 *                take precedence).  Read on the device, so it cannot be
 *                validated on the host: a NaN, negative or infinite value
 *                makes every element of out and lse NaN.
 *   bmm2_scale : fp32 [1]; when set, replaces v_scale.
 *   kv_rope    : split cache (Ascend ATB MLA page, cacheMode KROPE_CTKV:
 *                ctKV [num_blocks, block_size, kv_heads, 512] and kRope
 *                [num_blocks, block_size, kv_heads, 64]).  When set,
 *                kv_cache holds the 512 latent columns
 *                [num_blocks][page_block_size][num_heads_k][512] and kv_rope the 64 rope
 *                columns [num_blocks][page_block_size][num_heads_k][64], both of kv_dtype;
 *                the block table indexes both.
 *   q_rope     : split query (same page: qNope and qRope).  When set, q holds
 *                [batch][s_q][num_heads_q][512] and q_rope the rope columns,
 *                bf16 [batch][s_q][num_heads_q][64].
 *   stages     : 0 or 3 = both stages; 1 = mla_decode_splits only; 2 =
 *                mla_combine_splits only (the combine applies the sinks of
 *                split sequences and the device bmm2_scale, so it must get the
 *                same ext).  Other values are INVALID_ARG.
 *   bmm1_scale_log2: fp32 [1]; when set, the factor on q.k in base 2, i.e.
 *                bmm1_scale * log2(e) (FlashInfer MLA page: the device-scale
 *                pair (bmm1_scale_log2_tensor, bmm2_scale_tensor)); it
 *                replaces softmax_scale and bmm1_scale.  Not validated on the
 *                host: a NaN, negative or infinite value makes out and lse NaN.
 *   qk_descale : fp32 [num_heads_q]; head h's scores are multiplied by
 *                qk_descale[h] on top of the scale (Ascend ATB MLA page,
 *                qkDescale [num_heads]).  Sink logits are not rescaled.  A
 *                NaN, negative or infinite entry makes head h's out and lse NaN.
 *   pv_descale : fp32 [num_heads_q]; head h's output is multiplied by
 *                pv_descale[h] on top of v_scale (Ascend ATB MLA page,
 *                pvDescale [num_heads]); lse does not depend on it.
 *   q_dtype    : MLA_Q_BF16 (0, default) or MLA_Q_FP8_E4M3FN (1): q holds
 *                e4m3fn codes [batch][s_q][num_heads_q][576], whose q_scale
 *                the caller folds into the scale (FlashInfer MLA page, note on
 *                fused scales: bmm1 = q_scale * k_scale * sm_scale /
 *                sqrt(576)).  An fp8 q must be joined (q_rope NULL) and
 *                needs an fp8 cache; other pairings are UNSUPPORTED.
 * head_dim stays 576 (the total width) in every layout. */
typedef struct mla_decode_ext {
  const float *sinks;
  const float *bmm1_scale;
  const float *bmm2_scale;
  const void *kv_rope;
  const void *q_rope;
  int stages;
  const float *bmm1_scale_log2;
  const float *qk_descale;
  const float *pv_descale;
  int q_dtype;
} mla_decode_ext;

/* mla_decode_fwd with the optional inputs above (NULL ext = mla_decode_fwd). */
int mla_decode_fwd_ext(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                       const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                       const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                       int head_dim_v, float softmax_scale, float v_scale, int causal,
                       const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                       void *workspace, size_t workspace_bytes,
                       void *out, float *lse, void *stream, const mla_decode_ext *ext);

/* mla_decode_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, validation and results as mla_decode_fwd, without the
 * workspace: the split partials live in a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on.
 * The caller still passes every input and output.  A problem whose
 * mla_workspace_bytes(...) exceeds MLA_NOALLOC_SCRATCH_BYTES is rejected with
 * MLA_ERR_WORKSPACE_TOO_SMALL before any device call.  No call allocates or
 * frees memory; the first call on a device looks up the array's address there
 * (hipGetSymbolAddress) and keeps it.  Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (concurrent streams or
 * threads) race and must be serialised by the caller. */
int mla_decode_fwd_noalloc(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                           const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                           const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                           int head_dim_v, float softmax_scale, float v_scale, int causal,
                           const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                           void *out, float *lse, void *stream);

/* Measurement aid, not part of the decode: reads `bytes` (a positive
 * multiple of 1024) of device memory at `src` into LDS with the same 16-byte
 * LDS-DMA instruction and cache hint as the decode's page copies, and writes
 * nothing.  Hardware counters of HBM traffic are calibrated against it: the
 * bytes such a read fetches are known exactly.  INVALID_ARG for a NULL src
 * or a bad size; the call is asynchronous on `stream`. */
int mla_lds_dma_read(const void *src, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
