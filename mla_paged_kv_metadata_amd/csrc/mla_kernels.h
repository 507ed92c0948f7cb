// Internal launch interface between the C-ABI layer (mla_api.cpp) and the
// gfx950 kernels.  Not installed; the public surface is include/mla_decode.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kHeadDim = 576;
constexpr int kHeadDimV = 512;
constexpr int kPage = 64;
constexpr int kRowsPerTile = 128;     // rows (query heads x s_q) per decode workgroup
constexpr int kPartRows = 32;         // rows per block of the partial outputs (one wave's rows)
constexpr int kMetaThreads = 256;

struct DecodeArgs {
  const uint16_t *q;          // bf16 bits [B][s_q][Hq][q_stride]
  const uint8_t *kv;          // [num_blocks][page_size][Hk][576 or 512] bf16 or e4m3fn
  const int32_t *block_table; // [B][max_blocks]
  const int32_t *seqlens;     // [B]
  const int32_t *tile_md;     // [num_parts][8], one row per part
  const int32_t *num_splits;  // [B+1]
  uint16_t *out;              // bf16 bits [B][s_q][Hq][512]
  float *lse;                 // [B][Hq][s_q]
  uint16_t *part_o;           // bf16 bits [slots][Hk][ceil(M/32)][32 x 512 in accumulator order],
                              // slots = batch + num_parts - 1
  float *part_lse;            // [slots][Hk][M]
  int batch, s_q, hq, hk, group, rows, max_blocks, row_tiles, num_parts, num_blocks;
  int page_size;              // tokens per cache block, a multiple of 16
  int kv_fp8, causal;
  float scale_log2;           // softmax_scale * log2(e)
  float v_scale;
  int q_stride;               // elements per q row: 576, or 512 with q_rope
  const uint16_t *q_rope;     // nullptr, or bf16 bits [B][s_q][Hq][64]: the rope columns of q
  const uint8_t *kv_rope;     // nullptr, or [num_blocks][page_size][Hk][64]: the rope columns of the
                              // cache (kv then holds [num_blocks][page_size][Hk][512])
  const float *sinks;         // nullptr, or fp32 [Hq] per-head sink logits
  const float *bmm1_dev;      // nullptr, or fp32 [1] replacing softmax_scale
  const float *bmm2_dev;      // nullptr, or fp32 [1] replacing v_scale
  const float *bmm1_log2_dev; // nullptr, or fp32 [1]: bmm1 * log2(e), replacing softmax_scale and bmm1_dev
  const float *qk_descale;    // nullptr, or fp32 [Hq]: per-head factor on the scores
  const float *pv_descale;    // nullptr, or fp32 [Hq]: per-head factor on the output
  int q_fp8;                  // q holds e4m3fn codes [B][s_q][Hq][576] (q_scale folded into bmm1)
};

hipError_t launch_metadata(const int32_t *seqlens, int batch, int num_parts, int fixed_cost,
                           int32_t *tile_md, int32_t *num_splits, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream);
// Device address of the static scratch array on the current device (looked
// up once per device).
hipError_t noalloc_scratch(void **ptr);
// Counter calibration: reads bytes (a multiple of 1 KiB) into LDS with the
// page copies' LDS-DMA instruction.
hipError_t launch_lds_dma_read(const void *src, size_t bytes, hipStream_t stream);

}  // namespace mla
