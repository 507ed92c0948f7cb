// C-ABI layer of the MLA decode library: host-side validation, the device
// gate, scheduler policy and kernel launches.  Declarations and the contract
// of every entry point are in include/mla_decode.h.
#include "../../include/mla_decode.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "mla_kernels.h"

namespace {

thread_local char g_reason[256] = "";

int fail(int status, const char *reason) {
  std::strncpy(g_reason, reason, sizeof(g_reason) - 1);
  g_reason[sizeof(g_reason) - 1] = '\0';
  return status;
}

struct DeviceInfo {
  bool probed = false;
  bool gfx950 = false;
  int cus = 0;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Device gate (the vLLM platform check returns (supported, reason); here the
// reason is kept for mla_status_str).
int current_device(DeviceInfo *out) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(MLA_ERR_NO_DEVICE, "no HIP device is visible");
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo &d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDeviceProperties failed");
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.probed = true;
  }
  if (!d.gfx950) return fail(MLA_ERR_UNSUPPORTED, "the kernels are built for gfx950 (MI355X) only");
  *out = d;
  return MLA_OK;
}

int check_heads(int batch, int heads_per_head_k, int num_heads_k) {
  if (batch < 1 || heads_per_head_k < 1 || num_heads_k < 1)
    return fail(MLA_ERR_INVALID_ARG, "batch, heads_per_head_k and num_heads_k must be >= 1");
  if (batch > MLA_MAX_BATCH) return fail(MLA_ERR_UNSUPPORTED, "batch exceeds MLA_MAX_BATCH");
  if (heads_per_head_k > MLA_MAX_ROWS) return fail(MLA_ERR_UNSUPPORTED, "heads_per_head_k exceeds MLA_MAX_ROWS");
  return MLA_OK;
}

int row_tiles(int rows) { return (rows + mla::kRowsPerTile - 1) / mla::kRowsPerTile; }
// Partial outputs are stored in whole 32-row wave blocks.
size_t rows_pad(size_t rows) { return (rows + mla::kPartRows - 1) / mla::kPartRows * mla::kPartRows; }

// Per-split overhead in page units: a split loads its rows' q and writes its
// output rows (or a partial) on top of its pages, and waits for its first
// page.  On MI355X that measured about four bf16 pages for a 128-row tile;
// with fewer rows the q and output traffic shrinks but the first page's wait
// does not, and sweeps put the best value for a 16-row tile at 2-3 pages
// (1 page was 10% slower on the skewed 16-head decode).
int default_fixed_cost(int rows) { return std::max(2, std::min(rows, mla::kRowsPerTile) / 32); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char *mla_status_str(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return g_reason[0] ? g_reason : "invalid argument";
    case MLA_ERR_UNSUPPORTED: return g_reason[0] ? g_reason : "unsupported";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return g_reason[0] ? g_reason : "workspace smaller than mla_workspace_bytes()";
    case MLA_ERR_NO_DEVICE: return "no HIP device is visible";
    case MLA_ERR_HIP: return g_reason[0] ? g_reason : "HIP runtime error";
    default: return "unknown status";
  }
}

int mla_num_parts(int batch, int heads_per_head_k, int num_heads_k, int *num_parts) {
  if (!num_parts) return fail(MLA_ERR_INVALID_ARG, "num_parts is NULL");
  int rc = check_heads(batch, heads_per_head_k, num_heads_k);
  if (rc) return rc;
  DeviceInfo d;
  if ((rc = current_device(&d))) return rc;
  const int wgs_per_part = row_tiles(heads_per_head_k) * num_heads_k;
  *num_parts = std::max(1, d.cus / wgs_per_part);
  return MLA_OK;
}

int mla_get_metadata_ex(const int32_t *cache_seqlens, int batch, int heads_per_head_k, int num_heads_k,
                        int num_parts, int fixed_cost, int32_t *tile_md, int32_t *num_splits, void *stream) {
  int rc = check_heads(batch, heads_per_head_k, num_heads_k);
  if (rc) return rc;
  if (!cache_seqlens || !tile_md || !num_splits)
    return fail(MLA_ERR_INVALID_ARG, "cache_seqlens, tile_md and num_splits must be non-NULL");
  if (num_parts < 1 || num_parts > (1 << 20)) return fail(MLA_ERR_INVALID_ARG, "num_parts must be in [1, 2^20]");
  if (fixed_cost < 1 || fixed_cost > (1 << 20)) return fail(MLA_ERR_INVALID_ARG, "fixed_cost must be in [1, 2^20]");
  DeviceInfo d;
  if ((rc = current_device(&d))) return rc;
  hipError_t e = mla::launch_metadata(cache_seqlens, batch, num_parts, fixed_cost, tile_md, num_splits,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, hipGetErrorString(e));
  return MLA_OK;
}

int mla_get_metadata(const int32_t *cache_seqlens, int batch, int heads_per_head_k, int num_heads_k,
                     int32_t *tile_md, int num_parts, int32_t *num_splits, void *stream) {
  int rc = check_heads(batch, heads_per_head_k, num_heads_k);
  if (rc) return rc;
  return mla_get_metadata_ex(cache_seqlens, batch, heads_per_head_k, num_heads_k, num_parts,
                             default_fixed_cost(heads_per_head_k), tile_md, num_splits, stream);
}

int mla_workspace_bytes(int batch, int s_q, int num_heads_q, int num_heads_k, int head_dim_v, int num_parts,
                        size_t *bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || s_q < 1 || num_heads_q < 1 || num_heads_k < 1 || head_dim_v < 1 || num_parts < 1)
    return fail(MLA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (num_heads_q % num_heads_k) return fail(MLA_ERR_INVALID_ARG, "num_heads_q must be a multiple of num_heads_k");
  const size_t slots = (size_t)batch + (size_t)num_parts;
  const size_t rows = (size_t)s_q * (num_heads_q / num_heads_k);
  *bytes = align256(slots * num_heads_k * rows_pad(rows) * head_dim_v * sizeof(uint16_t)) +
           align256(slots * num_heads_k * rows * sizeof(float));
  return MLA_OK;
}

}  // extern "C"

namespace {

static int decode_call(int stage, const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                   const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                   const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                   int head_dim_v, float softmax_scale, float v_scale, int causal,
                   const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                   void *workspace, size_t workspace_bytes,
                   void *out, float *lse, void *stream, const mla_decode_ext *ext = nullptr) {
  if (!q || !kv_cache || !block_table || !cache_seqlens || !tile_md || !num_splits || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "q, kv_cache, block_table, cache_seqlens, tile_md, num_splits, out and lse must be non-NULL");
  if (batch < 1 || s_q < 1 || num_heads_q < 1 || num_heads_k < 1 || num_blocks < 1 || max_blocks_per_seq < 1 ||
      num_parts < 1 || head_dim < 1 || head_dim_v < 1 || page_block_size < 1)
    return fail(MLA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (num_heads_q % num_heads_k) return fail(MLA_ERR_INVALID_ARG, "num_heads_q must be a multiple of num_heads_k");
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(softmax_scale) || !std::isfinite(v_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale and v_scale must be finite");
  if (softmax_scale < 0.f) return fail(MLA_ERR_UNSUPPORTED, "softmax_scale must be >= 0");
  if (head_dim != MLA_HEAD_DIM) return fail(MLA_ERR_UNSUPPORTED, "head_dim must be 576 (512 latent + 64 rope)");
  if (head_dim_v != MLA_HEAD_DIM_V) return fail(MLA_ERR_UNSUPPORTED, "head_dim_v must be 512");
  if (page_block_size % MLA_PAGE_BLOCK_ALIGN)
    return fail(MLA_ERR_UNSUPPORTED, "page_block_size must be a multiple of 16");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3FN)
    return fail(MLA_ERR_UNSUPPORTED, "kv_dtype must be MLA_KV_BF16 or MLA_KV_FP8_E4M3FN");
  const int group = num_heads_q / num_heads_k;
  const long rows = (long)s_q * group;
  if (rows > MLA_MAX_ROWS) return fail(MLA_ERR_UNSUPPORTED, "s_q * num_heads_q / num_heads_k exceeds MLA_MAX_ROWS");
  if (batch > MLA_MAX_BATCH) return fail(MLA_ERR_UNSUPPORTED, "batch exceeds MLA_MAX_BATCH");
  // Row indices of out and of the partial slots are 32-bit in the kernels.
  if ((long long)batch * s_q * num_heads_q >= (1LL << 31) ||
      ((long long)batch + num_parts) * (long long)rows_pad(rows) * num_heads_k >= (1LL << 31))
    return fail(MLA_ERR_UNSUPPORTED, "batch * s_q * num_heads_q or the partial slots exceed 2^31 rows");
  size_t need = 0;
  int rc = mla_workspace_bytes(batch, s_q, num_heads_q, num_heads_k, head_dim_v, num_parts, &need);
  if (rc) return rc;
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than mla_workspace_bytes()");
  DeviceInfo d;
  if ((rc = current_device(&d))) return rc;

  mla::DecodeArgs a;
  a.q = (const uint16_t *)q;
  a.kv = (const uint8_t *)kv_cache;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.tile_md = tile_md;
  a.num_splits = num_splits;
  a.out = (uint16_t *)out;
  a.lse = lse;
  const size_t slots = (size_t)batch + (size_t)num_parts;
  a.part_o = (uint16_t *)workspace;
  a.part_lse = (float *)((char *)workspace +
                          align256(slots * rows_pad(rows) * num_heads_k * head_dim_v * sizeof(uint16_t)));
  a.batch = batch;
  a.s_q = s_q;
  a.hq = num_heads_q;
  a.hk = num_heads_k;
  a.group = group;
  a.rows = (int)rows;
  a.max_blocks = max_blocks_per_seq;
  a.row_tiles = row_tiles((int)rows);
  a.num_parts = num_parts;
  a.num_blocks = num_blocks;
  a.page_size = page_block_size;
  a.kv_fp8 = kv_dtype == MLA_KV_FP8_E4M3FN;
  a.causal = causal;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  a.q_stride = head_dim;
  a.q_rope = nullptr;
  a.kv_rope = nullptr;
  a.sinks = nullptr;
  a.bmm1_dev = nullptr;
  a.bmm2_dev = nullptr;
  a.bmm1_log2_dev = nullptr;
  a.qk_descale = nullptr;
  a.pv_descale = nullptr;
  a.q_fp8 = 0;
  if (ext) {
    a.q_rope = (const uint16_t *)ext->q_rope;
    a.q_stride = ext->q_rope ? MLA_HEAD_DIM_V : MLA_HEAD_DIM;
    a.kv_rope = (const uint8_t *)ext->kv_rope;
    a.sinks = ext->sinks;
    a.bmm1_dev = ext->bmm1_scale;
    a.bmm2_dev = ext->bmm2_scale;
    a.bmm1_log2_dev = ext->bmm1_scale_log2;
    a.qk_descale = ext->qk_descale;
    a.pv_descale = ext->pv_descale;
    a.q_fp8 = ext->q_dtype == MLA_Q_FP8_E4M3FN;
  }
  if (stage & 1) {
    hipError_t e = mla::launch_decode(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, hipGetErrorString(e));
  }
  if (stage & 2) {
    hipError_t e = mla::launch_combine(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, hipGetErrorString(e));
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_fwd(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                   const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                   const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                   int head_dim_v, float softmax_scale, float v_scale, int causal,
                   const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                   void *workspace, size_t workspace_bytes,
                   void *out, float *lse, void *stream) {
  return decode_call(3, q, batch, s_q, num_heads_q, head_dim, kv_cache, kv_dtype, num_blocks, page_block_size,
                     num_heads_k, block_table, max_blocks_per_seq, cache_seqlens, head_dim_v, softmax_scale, v_scale,
                     causal, tile_md, num_parts, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int mla_decode_splits(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                   const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                   const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                   int head_dim_v, float softmax_scale, float v_scale, int causal,
                   const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                   void *workspace, size_t workspace_bytes,
                   void *out, float *lse, void *stream) {
  return decode_call(1, q, batch, s_q, num_heads_q, head_dim, kv_cache, kv_dtype, num_blocks, page_block_size,
                     num_heads_k, block_table, max_blocks_per_seq, cache_seqlens, head_dim_v, softmax_scale, v_scale,
                     causal, tile_md, num_parts, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int mla_combine_splits(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                   const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                   const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                   int head_dim_v, float softmax_scale, float v_scale, int causal,
                   const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                   void *workspace, size_t workspace_bytes,
                   void *out, float *lse, void *stream) {
  return decode_call(2, q, batch, s_q, num_heads_q, head_dim, kv_cache, kv_dtype, num_blocks, page_block_size,
                     num_heads_k, block_table, max_blocks_per_seq, cache_seqlens, head_dim_v, softmax_scale, v_scale,
                     causal, tile_md, num_parts, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int mla_decode_fwd_ext(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                       const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                       const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                       int head_dim_v, float softmax_scale, float v_scale, int causal,
                       const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                       void *workspace, size_t workspace_bytes,
                       void *out, float *lse, void *stream, const mla_decode_ext *ext) {
  int stage = 3;
  if (ext) {
    if (ext->stages < 0 || ext->stages > 3) return fail(MLA_ERR_INVALID_ARG, "ext->stages must be 0, 1, 2 or 3");
    if (ext->stages) stage = ext->stages;
    if (ext->q_dtype != MLA_Q_BF16 && ext->q_dtype != MLA_Q_FP8_E4M3FN)
      return fail(MLA_ERR_UNSUPPORTED, "ext->q_dtype must be MLA_Q_BF16 or MLA_Q_FP8_E4M3FN");
    if (ext->q_dtype == MLA_Q_FP8_E4M3FN && ext->q_rope)
      return fail(MLA_ERR_UNSUPPORTED, "an fp8 q must be joined (q_rope NULL)");
    if (ext->q_dtype == MLA_Q_FP8_E4M3FN && kv_dtype != MLA_KV_FP8_E4M3FN)
      return fail(MLA_ERR_UNSUPPORTED, "an fp8 q needs an fp8 cache (kv_dtype MLA_KV_FP8_E4M3FN)");
  }
  return decode_call(stage, q, batch, s_q, num_heads_q, head_dim, kv_cache, kv_dtype, num_blocks, page_block_size,
                     num_heads_k, block_table, max_blocks_per_seq, cache_seqlens, head_dim_v, softmax_scale, v_scale,
                     causal, tile_md, num_parts, num_splits, workspace, workspace_bytes, out, lse, stream, ext);
}

int mla_decode_fwd_noalloc(const void *q, int batch, int s_q, int num_heads_q, int head_dim,
                           const void *kv_cache, int kv_dtype, int num_blocks, int page_block_size, int num_heads_k,
                           const int32_t *block_table, int max_blocks_per_seq, const int32_t *cache_seqlens,
                           int head_dim_v, float softmax_scale, float v_scale, int causal,
                           const int32_t *tile_md, int num_parts, const int32_t *num_splits,
                           void *out, float *lse, void *stream) {
  // The size check comes first, so an oversized request is refused before
  // any device call.
  size_t need = 0;
  int rc = mla_workspace_bytes(batch, s_q, num_heads_q, num_heads_k, head_dim_v, num_parts, &need);
  if (rc) return rc;
  if (need > MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "the problem's split workspace exceeds the static scratch (MLA_NOALLOC_SCRATCH_BYTES)");
  DeviceInfo d;
  if ((rc = current_device(&d))) return rc;
  void *ws = nullptr;
  hipError_t e = mla::noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, hipGetErrorString(e));
  return decode_call(3, q, batch, s_q, num_heads_q, head_dim, kv_cache, kv_dtype, num_blocks, page_block_size,
                     num_heads_k, block_table, max_blocks_per_seq, cache_seqlens, head_dim_v, softmax_scale, v_scale,
                     causal, tile_md, num_parts, num_splits, ws, MLA_NOALLOC_SCRATCH_BYTES, out, lse, stream);
}

int mla_lds_dma_read(const void *src, size_t bytes, void *stream) {
  if (!src || bytes == 0 || bytes % 1024) return fail(MLA_ERR_INVALID_ARG, "src must be non-NULL and bytes a positive multiple of 1024");
  DeviceInfo d;
  int rc = current_device(&d);
  if (rc) return rc;
  hipError_t e = mla::launch_lds_dma_read(src, bytes, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, hipGetErrorString(e));
  return MLA_OK;
}

}  // extern "C"
