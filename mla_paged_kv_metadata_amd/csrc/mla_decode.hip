// MLA decode over a paged KV cache on gfx950 (MI355X): split-KV attention
// kernel and log-sum-exp combine.
//
// What is computed (FlashMLA interface page, docstring of
// flash_mla_with_kvcache): for every sequence b, query token i and head h,
//   out[b,i,h,:] = sum_t softmax_t(scale * q[b,i,h,:] . k_t) * v_t,
//   lse[b,h,i]   = ln sum_t exp(scale * q . k_t),
// where k_t is the 576-wide cached row of token t (fetched through
// block_table, 64 tokens per page) and v_t is its first 512 columns
// (FlashInfer MLA page: the cache is ckv ++ kpe and the wrappers pass no
// separate V cache).
//
// Design (per workgroup of 4 waves, 1 workgroup per CU):
//  * A workgroup owns one split of one sequence (a row of the scheduler
//    table: a contiguous page range) for a 128-row tile of one KV head; each
//    wave owns 32 rows (query heads, with s_q folded into rows).
//  * Pages are streamed HBM -> LDS with 16-byte LDS-DMA loads
//    (global_load_lds_dwordx4): bf16 pages double buffered (2 x 72 KiB), fp8
//    pages in three 36 KiB buffers.  Chunks are XOR-swizzled within each row
//    so that MFMA operand reads hit distinct banks.
//  * Scores are computed transposed, S^T[token][head] = K Q^T, on
//    v_mfma_f32_32x32x16_bf16 with K from LDS and Q^T resident in VGPRs.
//    In that layout each lane holds one head and 32 of the page's 64 tokens,
//    so the online-softmax row max/sum is a per-lane loop plus one exchange
//    with lane ^ 32.
//  * O^T[dim][head] = V^T P^T on the same MFMA, V^T read from the very same
//    LDS rows (columns 0..511) with ds_read_b64_tr_b16 transposing loads, P^T
//    straight from the score registers (the token order inside one k-step is
//    permuted identically on both operands).  Each lane's 256 accumulators
//    belong to one head, so the softmax rescale is a per-lane scalar.
//  * Softmax runs in base 2 with log2(e) folded into the scale.
//  * A sequence with one split writes bf16 out / fp32 lse directly; a split
//    sequence writes bf16 partials (O/l) and fp32 lse that the combine
//    kernel merges.
//  * fp8 (e4m3fn) caches stay as codes in LDS (half the bytes of a bf16
//    page) and feed the fp8 matrix core (v_mfma_scale_f32_32x32x64_f8f6f4)
//    as they are: q enters as two e4m3 terms (hi + lo / 16, one power-of-two
//    block scale per head) and P as one e4m3 term per 32-token tile with a
//    block exponent.  The fused bmm1/bmm2 scales of the FlashInfer MLA page
//    enter as softmax_scale and v_scale.
#include "mla_kernels.h"
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "../../include/mla_decode.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kRowChunks = kHeadDim * 2 / 16;        // 72 chunks of 16 B per bf16 row
constexpr int kPageBytes = kPage * kHeadDim * 2;     // 73728

// Race check build (-DMLA_SERIAL_COPIES=1): every page copy is issued only
// after a barrier that follows the whole workgroup's work on the previous
// page, so no copy overlaps any LDS read.  Its results must equal the
// default build's bit for bit (the arithmetic is the same); a difference
// would point at a copy racing with the reads of the page before it.
#ifndef MLA_SERIAL_COPIES
#define MLA_SERIAL_COPIES 0
#endif
constexpr bool kSerialCopies = MLA_SERIAL_COPIES != 0;
constexpr int kPageLoads = kPage * kRowChunks / kThreads;   // 18 DMA loads per thread per bf16 page
constexpr int kF8RowChunks = kHeadDim / 16;          // 36 chunks per fp8 row
constexpr int kF8PageBytes = kPage * kHeadDim;       // 36864
constexpr int kF8PageLoads = kPage * kF8RowChunks / kThreads;  // 9
constexpr int kKSteps = kHeadDim / 16;               // 36 k-steps of the QK^T MFMA
constexpr int kOTiles = kHeadDimV / 32;              // 16 output tiles of 32 dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

static_assert(kPage * kRowChunks % kThreads == 0, "page must split evenly over threads");
static_assert(kPage * kF8RowChunks % kThreads == 0, "fp8 page must split evenly over threads");

// LDS layout of a bf16 page: nine column groups of 8 chunks (16 B each);
// group j holds chunks 8j..8j+7 of all 64 tokens, 128 B per token, with the
// chunk index XOR-swizzled by h(t) = (t1, t2, t3) -> bits (2, 1, 0), t_k
// being bit k of the token.  On the 64-bank (256 B/clock) LDS this makes
// both operand reads conflict-free: 16 consecutive tokens reading one chunk
// (the K operand of S^T) hit 16 distinct 16-byte bank slots, and 4
// consecutive tokens x 4 aligned chunks (the V^T transposing reads of 32
// lanes) hit 16 distinct slots.  Returns the 16-byte chunk index of
// (token t, logical chunk c).  One wave-wide 1 KiB LDS-DMA store then covers
// 8 whole tokens of one group, so every lane's global source offset is a
// lane constant plus a wave-uniform term.
__device__ __forceinline__ int swz_h(int t) { return (((t >> 1) & 1) << 2) | (((t >> 2) & 1) << 1) | ((t >> 3) & 1); }
__device__ __forceinline__ int pos_bf16(int t, int c) { return (c >> 3) * 512 + t * 8 + ((c & 7) ^ swz_h(t)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane i's
// 16 bytes from src + kImm land at lds + 16 * i.  Written as inline assembly
// on purpose: the compiler cannot tell which LDS bytes a copy writes, so for
// its own copy intrinsic it waits for every copy in flight before any later
// transposing LDS read -- which would serialise the next page's copy with
// this page's PV product.  Completion is instead awaited explicitly
// (wait_vmcnt) before the barrier that publishes a page.  M0 holds the LDS
// base; an M0 write needs one wait state before an LDS-DMA instruction.  The
// instruction's immediate offset applies to the global and the LDS address
// alike, so M0 is lowered by it.  Cache pages are read exactly once, so the
// copy carries the non-temporal hint: the lines it brings into L2 go first,
// and q rows and partial outputs (which are reused) stay resident longer.
// M0 is listed as clobbered; the compiler warns that it may not preserve a
// reserved register across the asm, which is harmless here because nothing
// else in these kernels uses M0 (a CPU test compiles them and checks that
// every M0 write in the code is one of these).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int kImm, bool kNt = true>
__device__ __forceinline__ void lds_dma16(const uint8_t *src, LDS_AS void *lds) {
  static_assert(kImm >= 0 && kImm < 4096, "global offset field");
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds) - kImm;
  if constexpr (kNt)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2 nt" ::"v"(src),
                 "s"(base), "n"(kImm)
                 : "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(src), "s"(base),
                 "n"(kImm)
                 : "m0");
}
#pragma clang diagnostic pop

// q rows of a wave staged through LDS: the wave's 32 consecutive q rows
// (32 x 1152 B, contiguous in memory) are copied as 36 LDS-DMA instructions
// of 8 whole rows x 128 B each -- 8 cache lines per instruction, where the
// direct fragment loads touch 32 rows per instruction -- into a 36 KiB LDS
// region, then read back as the 36 MFMA B fragments.  Instruction i = 9R + c
// covers rows 8R .. 8R+7 and 16-byte chunks 8c .. 8c+7; lane 8r + j fetches
// chunk 8c + (j ^ qsw(r, R)) of row 8R + r, so that chunk C of row n sits at
// byte 1024 (9 (n / 8) + C / 8) + 16 (8 (n % 8) + ((C % 8) ^ qsw(n % 8, n / 8))).
// For one fragment (a fixed chunk) 16 consecutive rows then fall on 16
// distinct 16-byte bank slots: the slot is 8 (n % 2) + ((C % 8) ^ qsw), and
// qsw takes 8 distinct values over the rows of one parity.
__device__ __forceinline__ int qsw(int r, int R) { return (r >> 1) | ((R & 1) << 2); }
__device__ __forceinline__ void stage_q_rows(const uint8_t *qblock, LDS_AS uint8_t *region, int lane) {
  const int r = lane >> 3, j = lane & 7;
#pragma unroll
  for (int i = 0; i < 36; ++i) {
    const int R = i / 9, c = i % 9;
    lds_dma16<0, false>(qblock + (8 * R + r) * 1152 + 16 * (8 * c + (j ^ qsw(r, R))), region + 1024 * i);
  }
}
__device__ __forceinline__ const LDS_AS bf16x8 *q_row_chunk(const LDS_AS uint8_t *region, int n, int C) {
  return (const LDS_AS bf16x8 *)(region + 1024 * (9 * (n >> 3) + (C >> 3)) + 16 * (8 * (n & 7) + ((C & 7) ^ qsw(n & 7, n >> 3))));
}
__device__ __forceinline__ void read_q_rows(const LDS_AS uint8_t *region, int lane, bf16x8 (&qf)[36]) {
  const int n = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 36; ++ks) qf[ks] = *q_row_chunk(region, n, 2 * ks + hl);
}

// HBM -> LDS copy of one bf16 page (64 rows x 1152 B) into the layout above,
// as kPageLoads wave instructions per wave.  The LDS image is 72 slots of
// 1 KiB, slot I = 8 * group + token block (8 tokens); wave w copies token
// blocks 2w and 2w + 1 of every group, instruction k covering block
// 2w + (k & 1) of group k / 2.  Per lane the source is one of two lane
// addresses (k even / odd) plus the immediate 128 * (k / 2).  The whole page
// is copied; rows past the sequence end are zeroed in LDS afterwards
// (zero_tail_rows) before any wave reads them.
//
// Split cache (kSplit; Ascend ATB MLA page, cacheMode KROPE_CTKV: ctKV
// [num_blocks, block_size, kv_heads, 512] and kRope [.., 64] as two tensors):
// the eight latent groups come from the ctKV rows and group 8 (the 64 rope
// columns) from the kRope rows, into the same LDS image.
struct PageSrc {
  const uint8_t *even, *odd;             // this lane's source for token blocks 2w, 2w + 1 (group 0)
  const uint8_t *rope_even, *rope_odd;   // split cache: the same tokens' rope columns
};
// slice0 / rope0: the wave's first token (16 w) of the page in the cache
// (its 16 tokens are consecutive rows of one cache block).
template <bool kSplit>
__device__ __forceinline__ PageSrc page_src_bf16(const uint8_t *slice0, const uint8_t *rope0, int tok_stride,
                                                 int rope_stride, int lane) {
  const int lt = lane >> 3;
  // token t = 16w + 8*(k&1) + lt: h(t) = (lt1, lt2, k&1) -> chunk (lane & 7) ^ h(t)
  PageSrc p;
  p.even = slice0 + lt * tok_stride + ((lane & 7) ^ swz_h(lt)) * 16;
  p.odd = slice0 + (8 + lt) * tok_stride + ((lane & 7) ^ swz_h(lt + 8)) * 16;
  p.rope_even = p.rope_odd = nullptr;
  if (kSplit) {
    p.rope_even = rope0 + lt * rope_stride + ((lane & 7) ^ swz_h(lt)) * 16;
    p.rope_odd = rope0 + (8 + lt) * rope_stride + ((lane & 7) ^ swz_h(lt + 8)) * 16;
  }
  return p;
}
template <bool kSplit, int k>
__device__ __forceinline__ void dma_bf16_step(const PageSrc &p, LDS_AS uint8_t *dst, int wave) {
  const int I = 8 * (k >> 1) + 2 * wave + (k & 1);
  if constexpr (kSplit && (k >> 1) == 8) lds_dma16<0>((k & 1) ? p.rope_odd : p.rope_even, dst + I * 1024);
  else lds_dma16<128 * (k >> 1)>((k & 1) ? p.odd : p.even, dst + I * 1024);
}
template <bool kSplit, int k = 0>
__device__ __forceinline__ void dma_page_bf16(const PageSrc &p, LDS_AS uint8_t *dst, int wave) {
  if constexpr (k < kPageLoads) {
    dma_bf16_step<kSplit, k>(p, dst, wave);
    dma_page_bf16<kSplit, k + 1>(p, dst, wave);
  }
}

// Zero rows nvalid..63 of a bf16 page in LDS (the cache rows past a
// sequence's end may hold anything, and 0 * NaN would poison the PV product).
__device__ __forceinline__ void zero_tail_rows(LDS_AS uint8_t *page, int nvalid, int tid) {
  const int first = nvalid * kRowChunks;
  for (int i = first + tid; i < kPage * kRowChunks; i += kThreads) {
    const int t = i / kRowChunks, c = i - t * kRowChunks;
    *(LDS_AS u32x4 *)(page + pos_bf16(t, c) * 16) = u32x4{0u, 0u, 0u, 0u};
  }
}

// LDS layout of an fp8 page (64 tokens x 576 codes): nine column groups of
// 64 B, group g at 4096 g holding 64 B of every token at 64 t; within a
// token's 64 B, 16-byte chunk j sits at position j ^ ((t >> 2) & 3).  Both
// 8-byte operand reads are then conflict-free: 16 tokens reading one 8-byte
// half-chunk (K of S^T) cover (t % 4, position, half) without repeats, and so
// do the transposing reads of V^T (tokens base + {0..3, 8..11}, two halves).
// HBM -> LDS copy: slot I = 4 * group + token block (16 tokens), wave w
// copies token block w, instruction k covering group k (group 8, the rope
// columns, from the kRope rows of a split cache); lane l writes slot bytes
// 16 l, i.e. token 16 w + l / 4 at position l % 4, so it fetches chunk
// (l % 4) ^ ((l / 16) % 4) of the group.
template <bool kSplit>
__device__ __forceinline__ PageSrc page_src_fp8(const uint8_t *slice0, const uint8_t *rope0, int tok_stride,
                                                int rope_stride, int lane) {
  PageSrc p;
  const int chunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
  p.even = p.odd = slice0 + (lane >> 2) * tok_stride + chunk;
  p.rope_even = p.rope_odd = kSplit ? rope0 + (lane >> 2) * rope_stride + chunk : nullptr;
  return p;
}

// Zero tokens nvalid..63 of an fp8 page in LDS (cache rows past a sequence's
// end may hold NaN codes, and 0 * NaN would poison the PV product).
__device__ __forceinline__ void zero_tail_rows_fp8(LDS_AS uint8_t *page, int nvalid, int tid) {
  const int first = nvalid * kF8RowChunks;
  for (int i = first + tid; i < kPage * kF8RowChunks; i += kThreads) {
    const int t = i / kF8RowChunks, c = i - t * kF8RowChunks;
    *(LDS_AS u32x4 *)(page + 4096 * (c >> 2) + 64 * t + 16 * (c & 3)) = u32x4{0u, 0u, 0u, 0u};
  }
}

template <bool kSplit, int k>
__device__ __forceinline__ void dma_fp8_step(const PageSrc &p, LDS_AS uint8_t *dst, int wave) {
  if constexpr (kSplit && k == 8) lds_dma16<0>(p.rope_even, dst + (4 * k + wave) * 1024);
  else lds_dma16<64 * k>(p.even, dst + (4 * k + wave) * 1024);
}
template <bool kSplit, int k = 0>
__device__ __forceinline__ void dma_page_fp8(const PageSrc &p, LDS_AS uint8_t *dst, int wave) {
  if constexpr (k < kF8PageLoads) {
    dma_fp8_step<kSplit, k>(p, dst, wave);
    dma_page_fp8<kSplit, k + 1>(p, dst, wave);
  }
}

// Instruction k of a page copy for a k known only after loop unrolling (the
// switch folds away once k is a constant).
template <bool kSplit>
__device__ __forceinline__ void dma_bf16_dispatch(const PageSrc &p, LDS_AS uint8_t *dst, int wave, int k) {
  switch (k) {
#define MLA_DMA_CASE(n) \
  case n: dma_bf16_step<kSplit, n>(p, dst, wave); break;
    MLA_DMA_CASE(0) MLA_DMA_CASE(1) MLA_DMA_CASE(2) MLA_DMA_CASE(3) MLA_DMA_CASE(4) MLA_DMA_CASE(5)
    MLA_DMA_CASE(6) MLA_DMA_CASE(7) MLA_DMA_CASE(8) MLA_DMA_CASE(9) MLA_DMA_CASE(10) MLA_DMA_CASE(11)
    MLA_DMA_CASE(12) MLA_DMA_CASE(13) MLA_DMA_CASE(14) MLA_DMA_CASE(15) MLA_DMA_CASE(16) MLA_DMA_CASE(17)
#undef MLA_DMA_CASE
    default: break;
  }
}
template <bool kSplit>
__device__ __forceinline__ void dma_fp8_dispatch(const PageSrc &p, LDS_AS uint8_t *dst, int wave, int k) {
  switch (k) {
#define MLA_DMA_CASE(n) \
  case n: dma_fp8_step<kSplit, n>(p, dst, wave); break;
    MLA_DMA_CASE(0) MLA_DMA_CASE(1) MLA_DMA_CASE(2) MLA_DMA_CASE(3) MLA_DMA_CASE(4) MLA_DMA_CASE(5)
    MLA_DMA_CASE(6) MLA_DMA_CASE(7) MLA_DMA_CASE(8)
#undef MLA_DMA_CASE
    default: break;
  }
}

// One 64-token page for this wave's 32 rows, processed as two 32-token
// halves: scores, online softmax, PV.
//   key0 : sequence index of the page's first token; nvis: keys this lane's row may see.
// Reference max: a row's reference m is fixed by its first visible keys and
// probabilities are exp2(x - m).  They may exceed 1; that is exact (O and l
// share the reference) and safe while x - m <= kRefSlackLog2 (p <= 2^64, far
// from fp32/bf16 overflow).  A score beyond that slack does not rescale O in
// place (that would drag the 256 accumulators through the VGPR file); the row
// records the larger reference in m_restart and the caller re-runs the
// sequence segment from its first page.  Each re-run raises a reference by
// more than 64, so re-runs are finite, and they never happen unless a later
// score exceeds the first keys' maximum by 64/log2(e) ~ 44 natural-log units.
constexpr float kRefSlackLog2 = 64.0f;

// c + 0 * 0 on the matrix core: zeroes all O^T accumulators in the MFMA
// accumulation registers.  The zero operand comes from an opaque move at the
// point of use; a plain constant would be hoisted out of the sequence loop,
// where it would only occupy (or spill) four VGPRs between uses.
__device__ __forceinline__ void mfma_zero_all(f32x16 (&o)[kOTiles]) {
  unsigned z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  const bf16x8 zz = __builtin_bit_cast(bf16x8, u32x4{z, z, z, z});
#pragma unroll
  for (int t = 0; t < kOTiles; ++t) o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zz, zz, f32x16{}, 0, 0, 0);
}

// S^T accumulation steps on the matrix core with the accumulator pinned to
// ordinary VGPRs: the O^T accumulators fill all 256 AGPRs, and the compiler
// would otherwise place S^T there too and spill an O^T tile.  The first step
// takes an inline zero accumulator; the destination is early-clobber (a
// 32x32 MFMA destination may not overlap its A/B sources).  mfma_qk_drain
// supplies the wait states between the last matrix-core write of S^T and
// its first VALU read (19 > the 8-pass XDL requirement).  The A operands
// come straight from LDS reads, never from a VALU write just before.
__device__ __forceinline__ void mfma_qk_first(f32x16 &s, const bf16x8 &a, const bf16x8 &b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16 &s, const bf16x8 &a, const bf16x8 &b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk_drain(f32x16 &s) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(s));
}

// Exchange with lane ^ 32 through v_permlane32_swap (no LDS round trip):
// swapping a value with itself leaves the lower-half copy in r[0] and the
// upper-half copy in r[1] on every lane.
__device__ __forceinline__ float max_across_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Where the next page's HBM -> LDS copy goes; its wave instructions are
// spread over the first k-steps of this page's S^T product instead of being
// issued in one burst, so the wave keeps feeding the matrix core while the
// address unit drains them.
struct NextPage {
  PageSrc src;                // this lane's source addresses of the next page
  LDS_AS uint8_t *dst;        // its LDS page buffer
  int wave;
  bool valid;                 // workgroup-uniform
};

// A row's raw scores times its per-head qkDescale.
__device__ __forceinline__ void scale_scores(f32x16 &sc, float d) {
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[i] *= d;
}

// Returns true (wave-uniform) when some row of this wave needs a re-run.
//   scale_log2 > 0 (softmax_scale * log2 e, clamped away from 0 by the caller);
//   mask: some key of this page may be invisible to some row of the wave.
template <bool kSplit>
__device__ __forceinline__ bool attend_page(const LDS_AS uint8_t *pg, const bf16x8 (&qf)[kKSteps],
                                            f32x16 (&o)[kOTiles], float &m, float &l, float &m_restart,
                                            int lane, int key0, int nvis, float scale_log2, bool mask,
                                            const LDS_AS float *desc, bool descale, const NextPage &nx) {
  const int hl = lane >> 5;
  const int r = lane & 31;

  // K operand: logical chunk 2*ks + hl of token r (+32 for the second 32-token
  // tile) sits at byte 8192*(ks/4) + 128*r + 16*((2*(ks%4) + hl) ^ h(r)) (+4096):
  // four lane bases, the rest immediates.
  const LDS_AS uint8_t *kb[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) kb[v] = pg + r * 128 + ((2 * v + hl) ^ swz_h(r)) * 16;

  // V^T operand via transposing reads: in each 16-lane group, lane i gets
  // element i%4 of the 8-byte rows loaded by lanes 4r + i/4 (r = 0..3).
  // Lane (group g, slot 4*rr + qd) loads token ta = 16*ks + 4*xb + rr
  // (xb = g/2) for k-slots 0..3 and tb = ta + 8 for k-slots 4..7, at dims
  // 32*mt + 16*(g%2) + 4*qd, i.e. logical chunk 4*mt + y (y = 2*(g%2) + qd/2)
  // and byte 8*(qd%2) within it.  With h(ta) = 4*t1 + 2*xb (t1 = rr/2) and
  // h(tb) = h(ta) + 1 the byte offset is
  //   8192*(mt/2) + 2048*ks + 128*(4*xb + rr) + 64*((mt%2) ^ t1)
  //   + 16*(y ^ (2*xb [+1 for tb])) + 8*(qd%2) [+ 1024 for tb],
  // so four lane bases (ta/tb x even/odd mt) plus immediates address all reads.
  const int g = lane >> 4, s16 = lane & 15, rr = s16 >> 2, qd = s16 & 3;
  const int xb = g >> 1, t1 = rr >> 1, y = 2 * (g & 1) + (qd >> 1);
  const int la = (4 * xb + rr) * 128 + (y ^ (2 * xb)) * 16 + (qd & 1) * 8;
  const int lb = (4 * xb + rr) * 128 + 1024 + (y ^ (2 * xb + 1)) * 16 + (qd & 1) * 8;
  const LDS_AS uint8_t *va_even = pg + la + 64 * t1, *va_odd = pg + la + 64 * (1 - t1);
  const LDS_AS uint8_t *vb_even = pg + lb + 64 * t1, *vb_odd = pg + lb + 64 * (1 - t1);

  // LDS operand loads run ahead of their MFMAs (software pipeline); loads
  // complete in order, so each MFMA waits only for its own operand.
  auto kload = [&](int ks, int tile) {
    return *(const LDS_AS bf16x8 *)(kb[ks & 3] + 8192 * (ks >> 2) + tile * 4096);
  };
  auto vload = [&](int step) {
    const int ks = step >> 4, mt = step & 15;         // k-step of 16 tokens, 32-dim output tile
    const int ofs = 8192 * (mt >> 1) + 2048 * ks;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(((mt & 1) ? va_odd : va_even) + ofs));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(((mt & 1) ? vb_odd : vb_even) + ofs));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // Online softmax of one 32-token tile, in kSoftPieces pieces that are
  // placed between matrix-core instructions of the other tile, so the VALU
  // work runs while the matrix core computes.  In S^T a lane holds head r and
  // tokens (i/4)*8 + 4*hl + i%4 (s[i]) of the tile.  Tiles are independent:
  // O and l share the fixed reference m, so nothing is rescaled; the first
  // tile with a visible key fixes m.
  //   pieces 0-1: mask the scores of invisible keys (8 each); piece 0 first
  //               multiplies the row's scores by its qkDescale, if any
  //   pieces 2-5: running max over 4 scores each
  //   piece 6   : max across the lane halves, reference update, re-run flag
  //   pieces 7-14: probabilities exp2(s * scale_log2 - m), 2 each, and their sum
  //   piece 15  : P^T as bf16 (k-steps 2*tile and 2*tile + 1)
  //   piece 16  : row sum across the lane halves into l
  float mx = kNegInf, ps = 0.f, mu = 0.f;
  bool need = false;
  auto soft = [&](f32x16 &sc, bf16x8 &p_lo, bf16x8 &p_hi, int tok0, int piece) {
    if (piece < 2) {
      if (piece == 0 && descale) scale_scores(sc, desc[r]);
      if (mask) {
#pragma unroll
        for (int i = 8 * piece; i < 8 * piece + 8; ++i) {
          const int tok = tok0 + (i >> 2) * 8 + hl * 4 + (i & 3);
          if (tok >= nvis) sc[i] = kNegInf;
        }
      }
    } else if (piece < 6) {
      const int i0 = 4 * (piece - 2);
      const float t = fmaxf(fmaxf(sc[i0], sc[i0 + 1]), fmaxf(sc[i0 + 2], sc[i0 + 3]));
      mx = piece == 2 ? t : fmaxf(mx, t);
    } else if (piece == 6) {
      float t = max_across_halves(mx);
      t = (t == kNegInf) ? kNegInf : t * scale_log2;
      if (m == kNegInf) m = t;                          // first visible keys fix the reference
      const bool nd = t > m + kRefSlackLog2;
      if (nd) m_restart = fmaxf(m_restart, t);
      need |= nd;
      mu = (m == kNegInf) ? 0.f : m;
    } else if (piece < 15) {
      const int i0 = 2 * (piece - 7);
      sc[i0] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i0], scale_log2, -mu));
      sc[i0 + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i0 + 1], scale_log2, -mu));
      ps = (piece == 7 ? 0.f : ps) + (sc[i0] + sc[i0 + 1]);
    } else if (piece == 15) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p_lo[e] = (__bf16)sc[e];
        p_hi[e] = (__bf16)sc[8 + e];
      }
    } else {
      l += sum_across_halves(ps);
    }
  };
  constexpr int kSoftPieces = 17;

  // S^T = K Q^T, one 32-token tile after the other: step g runs k-step g % 36
  // of tile g / 36 (a single accumulation chain per tile; the matrix core
  // forwards an accumulator to the next MFMA of its chain).  K operands are
  // prefetched kPre steps ahead; the tile-0 softmax runs under the tile-1
  // chain.
  constexpr int kPre = 4;
  constexpr int kDmaEvery = 2 * kKSteps / kPageLoads;   // 4
  decltype(kload(0, 0)) kf[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) kf[i] = kload(i, 0);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s0, s1;
  bf16x8 pb[4];              // P^T operand for PV k-step ks: tile ks/2, scores 8*(ks%2) .. +7
  // One step of a tile's chain: MFMA, the operand kPre steps ahead (crossing
  // into tile 1 at the end of tile 0), and every kDmaEvery-th step one copy
  // instruction of the next page.
  auto qk_step = [&](f32x16 &sc, int tile, int ks) {
    const int g = tile * kKSteps + ks, sl = g % kPre;
    if (ks == 0) mfma_qk_first(sc, kf[sl], qf[0]);
    else mfma_qk(sc, kf[sl], qf[ks]);
    if (g + kPre < 2 * kKSteps) kf[sl] = kload((g + kPre) % kKSteps, (g + kPre) / kKSteps);
    if (nx.valid && g % kDmaEvery == 0) dma_bf16_dispatch<kSplit>(nx.src, nx.dst, nx.wave, g / kDmaEvery);
  };
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    qk_step(s0, 0, ks);
    __builtin_amdgcn_sched_barrier(0);                 // keep loads kPre steps ahead
  }
  // Tile 1, with tile 0's softmax pieces over its steps 1 .. kKSteps - 2.
  constexpr int kSoftBN = kKSteps - 2;
  static_assert(kSoftPieces <= kSoftBN && kSoftPieces <= 2 * kOTiles - 2, "one piece per step at most");
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    qk_step(s1, 1, ks);
    if (ks == 0) mfma_qk_drain(s0);                    // tile 0's last MFMA -> first VALU read
    const int j = ks - 1;
    if (j >= 0 && j < kSoftBN && (j + 1) * kSoftPieces / kSoftBN != j * kSoftPieces / kSoftBN)
      soft(s0, pb[0], pb[1], key0, j * kSoftPieces / kSoftBN);
    __builtin_amdgcn_sched_barrier(0);
  }
  // First V^T operands.
  // V^T operands run 3 MFMAs ahead: same-box A/B against 4 ahead, MTP causal
  // decode 341 -> 335 us, standard decode 62.9 -> 62.3 us; 6 ahead spills
  // registers and was slower.
  constexpr int kVPre = 3;
  decltype(vload(0)) vraw[kVPre];
#pragma unroll
  for (int i = 0; i < kVPre; ++i) vraw[i] = vload(i);

  // O^T += V^T P^T over 4 k-steps x 16 dim tiles; the tile-1 softmax runs
  // under the first two k-steps (tile 0's P), which do not need it.
  auto pv_step = [&](int step) {
    const int sl = step % kVPre;
    o[step & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vraw[sl], pb[step >> 4], o[step & 15], 0, 0, 0);
    if (step + kVPre < 4 * kOTiles) vraw[sl] = vload(step + kVPre);
  };
  constexpr int kSoftCN = 2 * kOTiles - 2;
#pragma unroll
  for (int step = 0; step < 2 * kOTiles; ++step) {
    pv_step(step);
    if (step == 0) mfma_qk_drain(s1);                  // tile 1's last MFMA -> first VALU read
    const int j = step - 1;
    if (j >= 0 && j < kSoftCN && (j + 1) * kSoftPieces / kSoftCN != j * kSoftPieces / kSoftCN)
      soft(s1, pb[2], pb[3], key0 + 32, j * kSoftPieces / kSoftCN);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int step = 2 * kOTiles; step < 4 * kOTiles; ++step) pv_step(step);
  return __ballot(need) != 0;
}

// One 32-token tile (tokens 32 tile .. +31 of a bf16 page, key0 = the
// tile's first token) for this wave's 32 rows: used when a workgroup has at
// most 32 rows, so that two waves share each page (wave w takes tile w) and
// each runs half the matrix-core work of attend_page.  The same scheme as
// attend_page (reference max, re-run flag, P^T straight from the scores),
// but the softmax cannot hide under another tile's products: scores (36
// MFMAs, copying this wave's quarter of the next page every 2nd step),
// softmax, then O^T += V^T P^T over the tile's two 16-token k-steps.  Tile 1
// accumulates output tiles 8..15 in o[0..7] and 0..7 in o[8..15] (o[mt]
// holds output tile mt ^ 8), so that both waves finish o[0..7] after the
// merge.
template <bool kSplit>
__device__ __forceinline__ bool attend_tile(const LDS_AS uint8_t *pg, const bf16x8 (&qf)[kKSteps],
                                            f32x16 (&o)[kOTiles], float &m, float &l, float &m_restart,
                                            int lane, int key0, int nvis, float scale_log2, bool mask,
                                            const LDS_AS float *desc, bool descale, const NextPage &nx, int tile) {
  const int hl = lane >> 5;
  const int r = lane & 31;
  // K of token r of the tile (see attend_page): four lane bases plus immediates.
  const LDS_AS uint8_t *kb[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) kb[v] = pg + tile * 4096 + r * 128 + ((2 * v + hl) ^ swz_h(r)) * 16;
  // V^T as in attend_page, restricted to the tile's k-steps 2 tile, 2 tile + 1.
  const int g = lane >> 4, s16 = lane & 15, rr = s16 >> 2, qd = s16 & 3;
  const int xb = g >> 1, t1 = rr >> 1, y = 2 * (g & 1) + (qd >> 1);
  const int la = (4 * xb + rr) * 128 + (y ^ (2 * xb)) * 16 + (qd & 1) * 8;
  const int lb = (4 * xb + rr) * 128 + 1024 + (y ^ (2 * xb + 1)) * 16 + (qd & 1) * 8;
  const LDS_AS uint8_t *pt = pg + 4096 * tile;
  const LDS_AS uint8_t *va_even = pt + la + 64 * t1, *va_odd = pt + la + 64 * (1 - t1);
  const LDS_AS uint8_t *vb_even = pt + lb + 64 * t1, *vb_odd = pt + lb + 64 * (1 - t1);
  auto kload = [&](int ks) { return *(const LDS_AS bf16x8 *)(kb[ks & 3] + 8192 * (ks >> 2)); };
  // Output tile mt ^ 8 tile for o[mt]: 32 KiB further on for mt < 8, back for mt >= 8.
  const int vswap = 32768 * tile;
  auto vload = [&](int step) {
    const int ks = step >> 4, mt = step & 15;         // k-step of the tile, accumulator mt
    const int ofs = 8192 * (mt >> 1) + 2048 * ks + (mt < 8 ? vswap : -vswap);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(((mt & 1) ? va_odd : va_even) + ofs));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(((mt & 1) ? vb_odd : vb_even) + ofs));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // Scores: one accumulation chain over the 36 k-steps, K operands 4 ahead.
  constexpr int kPre = 4;
  constexpr int kDmaEvery = kKSteps / kPageLoads;     // 2: this wave's 18 copy instructions
  bf16x8 kf[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) kf[i] = kload(i);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 sc;
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    const int sl = ks % kPre;
    if (ks == 0) mfma_qk_first(sc, kf[sl], qf[0]);
    else mfma_qk(sc, kf[sl], qf[ks]);
    if (ks + kPre < kKSteps) kf[sl] = kload(ks + kPre);
    if (nx.valid && ks % kDmaEvery == 0) dma_bf16_dispatch<kSplit>(nx.src, nx.dst, nx.wave, ks / kDmaEvery);
    __builtin_amdgcn_sched_barrier(0);
  }
  // V^T operands of the first PV steps load while the softmax runs.
  constexpr int kVPre = 3;
  bf16x8 vraw[kVPre];
#pragma unroll
  for (int i = 0; i < kVPre; ++i) vraw[i] = vload(i);
  mfma_qk_drain(sc);

  // Softmax of the tile (as attend_page's pieces, in one run).  In S^T a lane
  // holds head r and tokens (i/4)*8 + 4*hl + i%4 of the tile.
  if (descale) scale_scores(sc, desc[r]);
  if (mask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = key0 + (i >> 2) * 8 + hl * 4 + (i & 3);
      if (tok >= nvis) sc[i] = kNegInf;
    }
  }
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
  float t = max_across_halves(mx);
  t = (t == kNegInf) ? kNegInf : t * scale_log2;
  if (m == kNegInf) m = t;                            // first visible keys fix the reference
  const bool need = t > m + kRefSlackLog2;
  if (need) m_restart = fmaxf(m_restart, t);
  const float mu = (m == kNegInf) ? 0.f : m;
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sc[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], scale_log2, -mu));
    ps += sc[i];
  }
  bf16x8 pb[2];                                       // P^T for the tile's k-steps 0 and 1
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pb[0][e] = (__bf16)sc[e];
    pb[1][e] = (__bf16)sc[8 + e];
  }
  l += sum_across_halves(ps);

  // O^T += V^T P^T: 2 k-steps x 16 output tiles, V^T operands 3 ahead.
#pragma unroll
  for (int step = 0; step < 2 * kOTiles; ++step) {
    const int sl = step % kVPre;
    o[step & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vraw[sl], pb[step >> 4], o[step & 15], 0, 0, 0);
    if (step + kVPre < 2 * kOTiles) vraw[sl] = vload(step + kVPre);
  }
  return __ballot(need) != 0;
}

// ---------------------------------------------------------------------------
// fp8 (e4m3fn) cache on the fp8 matrix core: v_mfma_scale_f32_32x32x64_f8f6f4.
//
// A 32x32x64 8-bit operand holds 32 bytes per lane: lane (row c, half h),
// byte j is k = 16h + (j & 15) + 32 (j >> 4), and bytes 0..15 / 16..31 take
// the E8M0 block scale of lane c / lane c + 32 (two 32-k scale blocks per
// row; both checked on the device with integer test vectors).
//
//  * S^T = K Q^T per 64-dim k-block kb: k <-> dim 64 kb + k.  K (codes, scale
//    1) is the A operand, straight from the LDS page.  q (bf16) enters as two
//    e4m3 terms, q = 2^-e (hi + lo / 16), with one power-of-two e per head
//    that puts the head's largest |q| in [128, 256): hi = e4m3(2^e q),
//    lo = e4m3(16 (2^e q - hi)); the B scales 2^-e and 2^-(e+4) undo the
//    factors, so S^T accumulates sum_d code_d q_d with about 8 significant
//    bits of q (bf16 has 8).
//  * O^T += V^T P^T over all 64 tokens in one k-step: k <-> token tau(h, j) =
//    32 (j >> 4) + 8 ((j & 15) / 4) + 4h + (j & 3), which is where the S^T
//    accumulator of lane (c, h) already holds its 32 scores (tile j >> 4,
//    element j & 15), so P^T needs no lane exchange.  P enters as one e4m3
//    term per 32-token tile with a power-of-two block scale 2^E (E = the
//    tile's largest exponent), and the row sum l adds up the same rounded
//    values, so the normalised weights stay consistent.
// ---------------------------------------------------------------------------

// bf16 chunk (8 dims) of q that lane half h places in slot i (0..3) of
// k-block kb: slots 0-1 are bytes 0..15 (dims 64kb + 16h ..), slots 2-3
// bytes 16..31 (dims 64kb + 32 + 16h ..).
__device__ __forceinline__ int q_chunk_f8(int kb, int i, int h) { return 8 * kb + 2 * h + (i & 1) + 4 * (i >> 1); }

__device__ __forceinline__ float pow2f(int e) { return __int_as_float((e + 127) << 23); }   // e in [-126, 127]

// Packs four floats as e4m3 codes (round to nearest even; every input here
// is within the format's range) into one dword, byte i = x[i].
__device__ __forceinline__ unsigned pack_e4m3(float a, float b, float c, float d) {
  v2i16 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, 1.0f, true);
  return __builtin_bit_cast(unsigned, w);
}
// The four e4m3 codes of a dword as floats.
__device__ __forceinline__ f32x4 unpack_e4m3(unsigned v) {
  const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)v, 1.0f, false);
  const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)v, 1.0f, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// In place: q8[2kb] / q8[2kb+1] hold the bf16 q values of k-block kb's bytes
// 0..15 / 16..31 (16 bf16 each, loaded by q_chunk_f8); they become the hi and
// lo e4m3 terms (32 codes each).  s_hi / s_lo: the B-operand E8M0 scales.
// The lo conversion takes its factor 16 through the instruction's scale
// operand (a conversion to e4m3 divides by it): lo = e4m3((v - hv) / 2^-4).
__device__ __forceinline__ void quantize_q_f8(i32x8 (&q8)[18], int &s_hi, int &s_lo) {
  // Largest |q|: bf16 magnitudes (sign bits cleared) order as 16-bit integers.
  u16x2 mxv = {0, 0};
#pragma unroll
  for (int i = 0; i < 18; ++i)
#pragma unroll
    for (int w = 0; w < 8; ++w)
      mxv = __builtin_elementwise_max(mxv, __builtin_bit_cast(u16x2, (unsigned)q8[i][w] & 0x7fff7fffu));
  float mx = __uint_as_float((unsigned)max(mxv[0], mxv[1]) << 16);
  mx = max_across_halves(mx);                     // the head's largest |q| (both lane halves)
  // mx = f 2^x, f in [1, 2): e = 7 - x puts 2^e mx in [128, 256).
  const int x = ((__float_as_int(mx) >> 23) & 255) - 127;
  const int e = mx > 0.f ? max(-120, min(120, 7 - x)) : 0;
  const float up = pow2f(e);
  s_hi = 127 - e;
  s_lo = 127 - e - 4;
#pragma unroll
  for (int kb = 0; kb < 9; ++kb) {
    float v[32];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      v[2 * w] = bf16_lo((unsigned)q8[2 * kb][w]) * up;
      v[2 * w + 1] = bf16_hi((unsigned)q8[2 * kb][w]) * up;
      v[16 + 2 * w] = bf16_lo((unsigned)q8[2 * kb + 1][w]) * up;
      v[16 + 2 * w + 1] = bf16_hi((unsigned)q8[2 * kb + 1][w]) * up;
    }
    i32x8 hi, lo;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const unsigned h = pack_e4m3(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3]);
      const f32x4 hv = unpack_e4m3(h);
      hi[d] = (int)h;
      v2i16 r = {0, 0};
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v[4 * d] - hv[0], v[4 * d + 1] - hv[1], 0.0625f, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v[4 * d + 2] - hv[2], v[4 * d + 3] - hv[3], 0.0625f, true);
      lo[d] = (int)__builtin_bit_cast(unsigned, r);
    }
    q8[2 * kb] = hi;
    q8[2 * kb + 1] = lo;
  }
}

// Holds a value at this point of the instruction stream: an empty volatile
// asm that reads and rewrites it keeps its place among the matrix-core steps
// (inline asm), so the work producing the value cannot sink past them to
// where the value is used.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(int &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_elem(f32x16 &v, int i) {
  float x = v[i];
  pin(x);
  v[i] = x;
}

// Score steps on the fp8 matrix core with the accumulator in ordinary VGPRs
// (see mfma_qk_first); sa / sb: the E8M0 scales of the A and B operands.
__device__ __forceinline__ void mfma8_first(f32x16 &s, const i32x8 &a, const i32x8 &b, int sa, int sb) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
      : "=&v"(s) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void mfma8(f32x16 &s, const i32x8 &a, const i32x8 &b, int sa, int sb) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
      : "+v"(s) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// V^T of dim tile mt for one PV step over 64 tokens taken from two pages:
// tokens 32..63 of page `a` (k 0..31) and tokens 0..31 of page `b` (k
// 32..63), by four 8-bit transposing reads (R = 0..3: bytes 8R .. 8R+7 =
// tokens 16R + 8 (e / 4) + 4h + (e % 4) of the 64 k positions, e = 0..7).
// In each 16-lane group G output lane i gets byte i % 8 of the rows loaded
// by lanes 2e + i / 8, so source lane (G, s) loads token 16R + 8 (s / 8) +
// 4 (G / 2) + (s / 2) % 4, dims 32 mt + 16 (G % 2) + 8 (s % 2): chunk
// 2 (mt % 2) + G % 2 of group mt / 2, swizzled by ((t >> 2) & 3) =
// (2 (s / 8) + G / 2) & 3 (the same for t and t + 32).
struct VtPair {
  int off0, off1;                                  // lane offsets for even / odd dim tiles
  __device__ __forceinline__ explicit VtPair(int lane) {
    const int G = lane >> 4, sl16 = lane & 15;
    const int fv = (2 * (sl16 >> 3) + (G >> 1)) & 3;
    const int vlane = 64 * (8 * (sl16 >> 3) + 4 * (G >> 1) + ((sl16 >> 1) & 3)) + 8 * (sl16 & 1);
    off0 = vlane + 16 * ((G & 1) ^ fv);
    off1 = vlane + 16 * ((2 + (G & 1)) ^ fv);
  }
  __device__ __forceinline__ i32x8 load(const LDS_AS uint8_t *a, const LDS_AS uint8_t *b, int mt) const {
    const int o = ((mt & 1) ? off1 : off0) + 4096 * (mt >> 1);
    const v2i32 x0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i32 *)(a + o + 2048));
    const v2i32 x1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i32 *)(a + o + 3072));
    const v2i32 x2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i32 *)(b + o));
    const v2i32 x3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i32 *)(b + o + 1024));
    return i32x8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
  }
};

// One 64-token fp8 page for this wave's 32 rows on the fp8 matrix core (the
// fp8 counterpart of attend_page; same reference-max scheme and return).
// The PV step of a page pairs the previous page's tile 1 (k 0..31: its
// weights p1 with block exponent e1, carried in and out) with this page's
// tile 0 (k 32..63), so that this page's tile-1 softmax runs under the PV
// MFMAs instead of before them; at a split's first page (has_prev false) the
// first half has zero weights (over finite rows of this page), and
// attend_drain_f8 adds the last page's tile 1 after the split.  kVPre: V^T
// operands that many MFMAs ahead.
template <bool kSplit, int kVPre>
__device__ __forceinline__ bool attend_page_f8(const LDS_AS uint8_t *pg, const i32x8 (&q8)[18], int s_hi, int s_lo,
                                               f32x16 (&o)[kOTiles], float &m, float &l, float &lq, float &m_restart,
                                               int lane, int key0, int nvis, float scale_log2, bool mask,
                                               const LDS_AS float *desc, bool descale, bool q_lo,
                                               const NextPage &nx, const LDS_AS uint8_t *prev_pg,
                                               bool has_prev, u32x4 &p1, int &e1) {
  const int hl = lane >> 5;
  const int r = lane & 31;
  const int k127 = 127;                            // scale 1 for the cache codes

  // K of token r (+32 for tile 1), k-block kb: bytes 0..15 are chunk hl and
  // bytes 16..31 chunk 2 + hl of group kb, at 4096 kb + 64 t + 16 (chunk ^
  // ((t >> 2) & 3)) in the fp8 page layout: two lane bases plus immediates.
  const int f = (r >> 2) & 3;
  const LDS_AS uint8_t *ka = pg + 64 * r + 16 * (hl ^ f);
  const LDS_AS uint8_t *kc = pg + 64 * r + 16 * ((2 + hl) ^ f);
  auto kload = [&](int kb, int tile) -> i32x8 {
    const u32x4 x = *(const LDS_AS u32x4 *)(ka + 4096 * kb + 2048 * tile);
    const u32x4 y = *(const LDS_AS u32x4 *)(kc + 4096 * kb + 2048 * tile);
    return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  };
  const VtPair vt(lane);
  const LDS_AS uint8_t *va = has_prev ? prev_pg : pg;
  auto vload = [&](int mt) -> i32x8 { return vt.load(va, pg, mt); };

  // Online softmax of one 32-token tile in 17 pieces (as in attend_page): in
  // S^T a lane holds head r and tokens (i/4)*8 + 4*hl + i%4 of the tile.
  // Piece 6 also fixes the tile's block exponent E = floor(t - mu), t the
  // tile's largest scaled score, so that P' = 2^(s - mu - E) lies in (0, 2);
  // pieces 7-14 also sum P' exactly; piece 15 rounds P' to e4m3 (4 dwords)
  // and sums the rounded values; piece 16 adds 2^E times both sums (over
  // both lane halves) to l (exact, for lse) and lq (rounded, the normaliser
  // of the output, so that the weights it divides sum to one).
  float mx = kNegInf, ps = 0.f, psq = 0.f, mu = 0.f;
  int et[2] = {0, 0};
  bool need = false;
  u32x4 p8[2];
  auto soft = [&](f32x16 &sc, int tile, int tok0, int piece) {
    if (piece < 2) {
      if (piece == 0 && descale) scale_scores(sc, desc[r]);
      if (mask) {
#pragma unroll
        for (int i = 8 * piece; i < 8 * piece + 8; ++i) {
          const int tok = tok0 + (i >> 2) * 8 + hl * 4 + (i & 3);
          if (tok >= nvis) sc[i] = kNegInf;
        }
      }
#pragma unroll
      for (int i = 8 * piece; i < 8 * piece + 8; ++i) pin_elem(sc, i);
    } else if (piece < 6) {
      const int i0 = 4 * (piece - 2);
      const float t = fmaxf(fmaxf(sc[i0], sc[i0 + 1]), fmaxf(sc[i0 + 2], sc[i0 + 3]));
      mx = piece == 2 ? t : fmaxf(mx, t);
      pin(mx);
    } else if (piece == 6) {
      float t = max_across_halves(mx);
      t = (t == kNegInf) ? kNegInf : t * scale_log2;
      if (m == kNegInf) m = t;                          // first visible keys fix the reference
      const bool nd = t > m + kRefSlackLog2;
      if (nd) m_restart = fmaxf(m_restart, t);
      need |= nd;
      mu = (m == kNegInf) ? 0.f : m;
      const int e = t == kNegInf ? 0 : (int)floorf(t - mu);
      et[tile] = max(-100, min(100, e));
      mu += (float)et[tile];
      pin(mu);
      pin(et[tile]);
    } else if (piece < 15) {
      const int i0 = 2 * (piece - 7);
      sc[i0] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i0], scale_log2, -mu));
      sc[i0 + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i0 + 1], scale_log2, -mu));
      ps = (piece == 7 ? 0.f : ps) + (sc[i0] + sc[i0 + 1]);
      pin_elem(sc, i0);
      pin_elem(sc, i0 + 1);
      pin(ps);
    } else if (piece == 15) {
      psq = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned c = pack_e4m3(sc[4 * d], sc[4 * d + 1], sc[4 * d + 2], sc[4 * d + 3]);
        p8[tile][d] = c;
        const f32x4 back = unpack_e4m3(c);
        psq += (back[0] + back[1]) + (back[2] + back[3]);
        asm volatile("" : "+v"(p8[tile]));
      }
      pin(psq);
    } else {
      const float w = pow2f(et[tile]);
      l += sum_across_halves(ps) * w;
      lq += sum_across_halves(psq) * w;
      pin(l);
      pin(lq);
    }
  };
  constexpr int kSoftPieces = 17;

  // S^T = K Q^T: step g = 9 tile + kb runs the hi and lo MFMAs of k-block kb
  // (one accumulation chain per tile; q_lo false, for an e4m3 query whose lo
  // term is zero, skips the lo MFMAs); K fragments two steps ahead; one copy
  // instruction of the next page every second step (9 per fp8 page).
  constexpr int kPre = 2;
  i32x8 kf[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) kf[i] = kload(i, 0);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s0, s1;
  // A step's VALU work sits between its MFMAs: the two MFMAs of a step (and
  // the next step's) form one accumulation chain, so the wave cannot issue
  // past an MFMA until its predecessor is done, and only instructions placed
  // right after an MFMA run under it.  `mid` runs after the hi MFMA, `post`
  // (with the K reads and the copy) after the lo one.
  auto qk_step = [&](f32x16 &sc, int tile, int kb, auto &&mid, auto &&post) {
    const int g = tile * 9 + kb, sl = g % kPre;
    if (kb == 0) mfma8_first(sc, kf[sl], q8[0], k127, s_hi);
    else mfma8(sc, kf[sl], q8[2 * kb], k127, s_hi);
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
    if (q_lo) mfma8(sc, kf[sl], q8[2 * kb + 1], k127, s_lo);
    __builtin_amdgcn_sched_barrier(0);
    if (g + kPre < 18) kf[sl] = kload((g + kPre) % 9, (g + kPre) / 9);
    if (nx.valid && g < 9) dma_fp8_dispatch<kSplit>(nx.src, nx.dst, nx.wave, g);
    post();
  };
  auto nothing = [] {};
#pragma unroll
  for (int kb = 0; kb < 9; ++kb) {
    qk_step(s0, 0, kb, nothing, nothing);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Tile 1, with tile 0's softmax: one piece after each of its MFMAs.
#pragma unroll
  for (int kb = 0; kb < 9; ++kb) {
    qk_step(
        s1, 1, kb,
        [&] {
          if (kb == 0) mfma_qk_drain(s0);
          soft(s0, 0, key0, 2 * kb);
        },
        [&] {
          if (2 * kb + 1 < kSoftPieces) soft(s0, 0, key0, 2 * kb + 1);
        });
    __builtin_amdgcn_sched_barrier(0);
  }
  // PV: the previous page's tile 1 and this page's tile 0 (P^T bytes 0..15
  // and 16..31; lane half 0 supplies the first one's block scale, half 1 the
  // second's), with this page's tile-1 softmax one piece after each MFMA.
  i32x8 vf[kVPre];
#pragma unroll
  for (int i = 0; i < kVPre; ++i) vf[i] = vload(i);
  const i32x8 pt = {has_prev ? (int)p1[0] : 0, has_prev ? (int)p1[1] : 0, has_prev ? (int)p1[2] : 0,
                    has_prev ? (int)p1[3] : 0, (int)p8[0][0], (int)p8[0][1], (int)p8[0][2], (int)p8[0][3]};
  const int ps_scale = 127 + (hl ? et[0] : (has_prev ? e1 : 0));
  mfma_qk_drain(s1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mt = 0; mt < kOTiles; ++mt) {
    const int sl = mt % kVPre;
    o[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[sl], pt, o[mt], 0, 0, 0, k127, 0, ps_scale);
    if (mt + kVPre < kOTiles) vf[sl] = vload(mt + kVPre);
    __builtin_amdgcn_sched_barrier(0);               // keep the V^T loads kVPre steps ahead
    soft(s1, 1, key0 + 32, mt);
    __builtin_amdgcn_sched_barrier(0);
  }
  soft(s1, 1, key0 + 32, kSoftPieces - 1);
  p1 = p8[1];
  e1 = et[1];
  return __ballot(need) != 0;
}

// The PV step left over at the end of a split: the last page's tile 1 (p1,
// block exponent e1) as the first half, zero weights over that page's
// tokens 0..31 (finite rows) as the second.
__device__ __forceinline__ void attend_drain_f8(const LDS_AS uint8_t *pg, const u32x4 &p1, int e1,
                                                f32x16 (&o)[kOTiles], int lane) {
  const int hl = lane >> 5;
  const int k127 = 127;
  const VtPair vt(lane);
  const i32x8 pt = {(int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3], 0, 0, 0, 0};
  const int ps_scale = 127 + (hl ? 0 : e1);
  constexpr int kVPre = 2;
  i32x8 vf[kVPre];
#pragma unroll
  for (int i = 0; i < kVPre; ++i) vf[i] = vt.load(pg, pg, i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mt = 0; mt < kOTiles; ++mt) {
    const int sl = mt % kVPre;
    o[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[sl], pt, o[mt], 0, 0, 0, k127, 0, ps_scale);
    if (mt + kVPre < kOTiles) vf[sl] = vt.load(pg, pg, mt + kVPre);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Number of passes a segment may take when a score overshoots the reference
// max by more than kRefSlackLog2 (see attend_page).  Bounded so that a
// workgroup always terminates; a further overshoot in the last pass is
// accumulated as is (still finite up to 2^64 relative weights).
constexpr int kMaxPasses = 4;

// Rounds a pair of floats to a packed bf16 pair (round to nearest even).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  const bf16x2 v = bf16x2{(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

// The lane index is re-derived here through an opaque instruction: the
// lane-dependent addresses below are then computed where they are used
// instead of being hoisted out of the sequence loop, where they would only
// be spilled and reloaded (and a reload's wait would stall on the next
// page's copy and on the stores in flight).
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
// The same for a wave-uniform value: an opaque scalar copy, so that values
// derived from it are computed where used rather than kept live (in VGPRs)
// across the sequence loop.
__device__ __forceinline__ int uniform_here(int v) {
  int r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
  return r;
}
// Row coordinates of this lane (row = 32-row wave tile + lane % 32, clamped
// into range; query token qi and query head h of that row), re-derived from
// an opaque lane index where they are needed rather than kept live across
// the whole kernel.
struct RowCoord {
  int row, rowc, qi, h;
};
__device__ __forceinline__ RowCoord row_coord(int wrow0, int rows, int group, int hk) {
  const int lane = lane_id_here();
  RowCoord c;
  c.row = wrow0 + (lane & 31);
  c.rowc = min(c.row, rows - 1);
  c.qi = c.rowc / group;
  c.h = hk * group + (c.rowc - c.qi * group);
  return c;
}

// Writes this wave's 32 x 512 result rows (times f, rounded to bf16) to
// global memory straight from the accumulators: in O^T tile t a lane holds
// its row's dims in 4-dim pieces (8q + 4*(lane/32) .. +3); v_permlane32_swap
// with lane ^ 32 merges piece pairs into whole 16-byte chunks, so one store
// instruction writes 32 bytes (two adjacent chunks) of each of the 32 rows.
// (Staging the tile through LDS for longer contiguous runs measured no
// faster, and LDS is the page loop's busiest unit.)
//   row_idx : this lane's destination row index in units of 512 elements
//             (lanes l and l + 32 hold row l % 32 of the wave)
//   nrows   : number of valid rows of the wave (0..32)
// Output tiles of O^T as 8-value pieces (t, pp): o[t][8pp .. 8pp+7] times
// f, for all 16 tiles, or (kMerge) for o[0 .. 7], which hold output tiles
// 8 half .. 8 half + 7 (half wave-uniform, 0 or 1), plus f1 times the same
// elements of a second state that another wave left in LDS at xb (f32x4 h
// of piece i = 2t + pp of lane L at byte 16 ((2i + h) 64 + L)).  The second
// state's values are read one piece ahead, so that the LDS latency overlaps
// the previous piece's stores.  fn(output tile, pp, v) consumes each piece.
template <bool kMerge, typename Fn>
__device__ __forceinline__ void for_each_piece(const f32x16 (&o)[kOTiles], float f, const LDS_AS uint8_t *xb,
                                               float f1, int half, Fn &&fn) {
  constexpr int kNT = kMerge ? kOTiles / 2 : kOTiles;
  const int lane = lane_id_here();
  f32x4 xn[2] = {};
  auto xload = [&](int i) {
    xn[0] = *(const LDS_AS f32x4 *)(xb + ((2 * i) * 64 + lane) * 16);
    xn[1] = *(const LDS_AS f32x4 *)(xb + ((2 * i + 1) * 64 + lane) * 16);
  };
  if constexpr (kMerge) xload(0);
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int i = 2 * t + pp;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = o[t][8 * pp + e] * f;
      if constexpr (kMerge) {
        const f32x4 x0 = xn[0], x1 = xn[1];
        if (i + 1 < 2 * kNT) xload(i + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = __builtin_fmaf(x0[e], f1, v[e]);
          v[4 + e] = __builtin_fmaf(x1[e], f1, v[4 + e]);
        }
      }
      fn(kMerge ? t + kNT * half : t, pp, v);
    }
  }
}

template <bool kMerge = false>
__device__ __forceinline__ void store_rows(const f32x16 (&o)[kOTiles], float f, uint16_t *base, int row_idx,
                                           int nrows, const LDS_AS uint8_t *xb = nullptr, float f1 = 0.f,
                                           int half = 0) {
  const int lane = lane_id_here();
  const int r = lane & 31, hl = lane >> 5;
  uint16_t *row = base + (long)row_idx * kHeadDimV + 8 * (1 - hl);
  const bool full = nrows == 32;                      // wave-uniform
  for_each_piece<kMerge>(o, f, xb, f1, half, [&](int t, int pp, const float (&v)[8]) {
    // piece q holds dims 8q + 4*hl .. +3 of tile t
    const unsigned a0 = pack_bf16(v[0], v[1]);   // q = 2pp
    const unsigned a1 = pack_bf16(v[2], v[3]);
    const unsigned b0 = pack_bf16(v[4], v[5]);   // q = 2pp + 1
    const unsigned b1 = pack_bf16(v[6], v[7]);
    // After the swap lanes < 32 hold chunk 2pp + 1 (dims 32t + 16pp + 8 ..),
    // lanes >= 32 chunk 2pp (dims 32t + 16pp ..).
    const auto s0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
    if (full || r < nrows) *(u32x4 *)(row + 32 * t + 16 * pp) = u32x4{s0[0], s1[0], s0[1], s1[1]};
  });
}

// Writes this wave's 32 x 512 split partial (times f, rounded to bf16) in
// accumulator order: 16-byte chunk (2t + pp) * 64 + lane of the wave's 32 KiB
// block holds o[t][8pp .. 8pp + 7] of that lane, i.e. row lane % 32, dims
// 32t + 16pp + 4hl + {0..3} and 32t + 16pp + 8 + 4hl + {0..3} (hl = lane / 32).
// Each store instruction then writes 1 KiB contiguous; the row-major form
// above touches 32 rows per instruction, and on the standard B=64 decode the
// last split's epilogue took about 4.1 us that way against 2.0 us this way.
// Rows past the last real row of the block are written too (the workspace
// holds whole 32-row blocks) and never read.
template <bool kMerge = false>
__device__ __forceinline__ void store_acc_block(const f32x16 (&o)[kOTiles], float f, uint16_t *blk,
                                                const LDS_AS uint8_t *xb = nullptr, float f1 = 0.f, int half = 0) {
  uint16_t *p = blk + lane_id_here() * 8;
  for_each_piece<kMerge>(o, f, xb, f1, half, [&](int t, int pp, const float (&v)[8]) {
    const unsigned a0 = pack_bf16(v[0], v[1]);
    const unsigned a1 = pack_bf16(v[2], v[3]);
    const unsigned b0 = pack_bf16(v[4], v[5]);
    const unsigned b1 = pack_bf16(v[6], v[7]);
    *(u32x4 *)(p + (2 * t + pp) * 512) = u32x4{a0, a1, b0, b1};
  });
}

// Bijection of [0, n): workgroup w runs on XCD w % 8 (the dispatcher's
// round-robin); XCD x gets the x-th contiguous block of parts.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_part(int w, int n) {
  const int q = n / kXcds, r = n % kXcds, x = w % kXcds, i = w / kXcds;
  return x * q + min(x, r) + i;
}

// A device-held scale must be finite and >= 0 (the host rejects other
// values of the host-side scale).
__device__ __forceinline__ bool bad_value(float v) { return !(v >= 0.f && v < __builtin_inff()); }
// True when a device-held bmm1 scale (plain or log2 form) is NaN, negative or
// infinite (workgroup-uniform).
__device__ __forceinline__ bool bad_device_scale(const DecodeArgs &a) {
  return a.bmm1_log2_dev ? bad_value(*a.bmm1_log2_dev) : a.bmm1_dev && bad_value(*a.bmm1_dev);
}
// Factor on q.k in base 2: the device log2 form, else the device bmm1, else
// the host scale (workgroup-uniform).  A per-head qkDescale multiplies the
// scores themselves.  Clamped away from 0 (the reference-max logic
// multiplies -inf by it).
__device__ __forceinline__ float scores_scale_log2(const DecodeArgs &a) {
  const float s = a.bmm1_log2_dev ? *a.bmm1_log2_dev : a.bmm1_dev ? *a.bmm1_dev * kLog2e : a.scale_log2;
  return fmaxf(s, 1e-30f);
}
// Factor on head h's output: bmm2 (device or host) times its pvDescale.
__device__ __forceinline__ float row_v_scale(const DecodeArgs &a, int h) {
  const float v = a.bmm2_dev ? *a.bmm2_dev : a.v_scale;
  return a.pv_descale ? v * a.pv_descale[h] : v;
}

// kAnyBlock: the cache's block size is a.page_size (a multiple of 16) rather
// than the 64 tokens of a page, whose slice arithmetic is then shifts.
// kKeySplit (bf16 cache, at most 32 rows per workgroup): waves 0 and 1 hold
// the same 32 rows and take token tiles 0 and 1 of every page (attend_tile);
// their states merge at the end of each split.
template <bool kFp8, bool kSplit, bool kAnyBlock, bool kKeySplit = false>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(const DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  LDS_AS uint8_t *smem = (LDS_AS uint8_t *)smem_raw;
  // Two page buffers: 72 KiB each for bf16, 36 KiB each for fp8.
  // Page buffers: two for bf16 pages; three for fp8 pages, whose PV step
  // still reads the previous page while the next one is copied.
  constexpr int kBufs = kFp8 ? 3 : 2;
  LDS_AS uint8_t *const bufs[3] = {smem, smem + (kFp8 ? kF8PageBytes : kPageBytes), smem + 2 * kF8PageBytes};
  auto buf_next = [](int i) { return i + 1 == kBufs ? 0 : i + 1; };
  auto buf_prev = [](int i) { return i == 0 ? kBufs - 1 : i - 1; };
  volatile LDS_AS int *rerun_flag = (volatile LDS_AS int *)(smem + 2 * kPageBytes);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rt = blockIdx.y % a.row_tiles;
  const int hk = blockIdx.y / a.row_tiles;
  // Table row of this part: a run of sequences b0..b1, the first and last
  // possibly cut at a page boundary.  Workgroups are dealt to the 8 XCDs
  // round-robin; consecutive parts (which share sequences, hence q rows and
  // partial slots) are given to workgroups on the same XCD so that they meet
  // in its L2.
  const int part = xcd_part(blockIdx.x, a.num_parts);
  const int32_t *md = a.tile_md + (long)part * 8;
  const int b0 = md[0];
  if (b0 < 0 || b0 >= a.batch) return;                // idle part
  const int b1 = min(max(md[2], b0), a.batch - 1);
  const int nslots = a.batch + a.num_parts - 1;       // partial slots in the workspace

  const int wrow0 = rt * kRowsPerTile + (kKeySplit ? 0 : wave * 32);
  const bool active = kKeySplit ? wave < 2 : wrow0 < a.rows;   // wave-uniform
  const int qi_min = (rt * kRowsPerTile) / a.group;   // smallest query token of the tile
  // A device-held bmm1 scale replaces the host value (FlashInfer MLA page:
  // bmm1_scale / bmm2_scale may be device tensors).  It cannot be validated
  // on the host: a NaN, negative or infinite value makes every output NaN.
  const bool bad_scale = bad_device_scale(a);
  const float scale_log2 = scores_scale_log2(a);
  // Per-head qkDescale (Ascend ATB MLA page): each row's factor sits in LDS,
  // 32 per wave, and multiplies its raw scores in the softmax; rows keep their
  // head for the whole kernel.
  LDS_AS float *const desc_tab = (LDS_AS float *)(smem + 2 * kPageBytes + 16) + wave * 32;
  // The output factor of each row: bmm2 (device or host) times its head's
  // pvDescale, read once per split in the epilogue.
  LDS_AS float *const vfac_tab = desc_tab + kRowsPerTile;
  if (active && lane < 32) {
    const int h = row_coord(wrow0, a.rows, a.group, hk).h;
    if (a.qk_descale) desc_tab[lane] = a.qk_descale[h];
    vfac_tab[lane] = row_v_scale(a, h);
  }
  const bool descale = a.qk_descale != nullptr;

  const int elem = kFp8 ? 1 : 2;
  constexpr int kRowDim = kSplit ? kHeadDimV : kHeadDim;   // columns of a kv_cache row
  const int tok_stride = a.hk * kRowDim * elem;
  const uint8_t *kv_head = a.kv + (long)hk * kRowDim * elem;
  const int rope_stride = a.hk * (kHeadDim - kHeadDimV) * elem;
  const uint8_t *rope_head = kSplit ? a.kv_rope + (long)hk * (kHeadDim - kHeadDimV) * elem : nullptr;
  // Pages of the kernel are 64 tokens; cache blocks hold bs tokens (a
  // multiple of 16), so this wave's 16-token slice of page j, tokens
  // 64 j + 16 w .., is rows (64 j + 16 w) % bs .. of table entry
  // (64 j + 16 w) / bs.
  const int bs = kAnyBlock ? a.page_size : kPage;
  auto slice_tok = [&](int j) { return j * kPage + 16 * wave; };
  // This lane's copy sources for the slice starting at row `row` of cache
  // block blk (index clamped into the pool).
  auto src_of = [&](int blk, int row) -> PageSrc {
    const long pc = (long)max(0, min(blk, a.num_blocks - 1)) * bs + row;
    const uint8_t *t0 = kv_head + pc * tok_stride;
    const uint8_t *r0 = kSplit ? rope_head + pc * rope_stride : nullptr;
    return kFp8 ? page_src_fp8<kSplit>(t0, r0, tok_stride, rope_stride, lane)
                : page_src_bf16<kSplit>(t0, r0, tok_stride, rope_stride, lane);
  };
  // Lengths and page ranges are clamped so that every global address stays
  // inside its buffer whatever the table or cache_seqlens hold.
  auto seq_len = [&](int b) { return (int)max(0L, min((long)a.seqlens[b], (long)a.max_blocks * bs)); };
  auto seq_end = [&](int b, int nblk) { return b == b1 ? max(0, min(md[3], nblk)) : nblk; };

  // q of this lane's row for the bf16 matrix core (qf: dims 16 ks + 8 hl ..
  // +7) or, with an fp8 cache, for the fp8 matrix core (q8: bf16 chunks
  // q_chunk_f8 until quantize_q_f8 turns them into the hi / lo e4m3 terms at
  // the start of the split).
  bf16x8 qf[kFp8 ? 1 : kKSteps];
  i32x8 q8[kFp8 ? 18 : 1];
  int s_hi = 127, s_lo = 127;
  auto set_q8_chunk = [&](int kb, int i, const bf16x8 &v) {
    const u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
    for (int d = 0; d < 4; ++d) q8[2 * kb + (i >> 1)][4 * (i & 1) + d] = (int)w[d];
  };
  // Row (qi, h) of sequence b.  The rope columns (chunks 64..71) come from
  // q_rope when q is split (Ascend ATB MLA page: qNope [.., 512] and qRope
  // [.., 64]).
  auto load_q = [&](int b) {
    const RowCoord c = row_coord(wrow0, a.rows, a.group, hk);
    const long r = ((long)min(b, a.batch - 1) * a.s_q + c.qi) * a.hq + c.h;
    if constexpr (kFp8) {
      if (a.q_fp8) {
        // An e4m3 query (its q_scale folded into bmm1; the host admits it
        // with an fp8 cache only): the codes are the hi term as they are,
        // with a zero lo term and unit scales.
        const int hl = lane_id_here() >> 5;
        const uint8_t *qc = (const uint8_t *)a.q + r * kHeadDim;
#pragma unroll
        for (int kb = 0; kb < 9; ++kb) {
          const u32x4 x = *(const u32x4 *)(qc + 64 * kb + 16 * hl);
          const u32x4 y = *(const u32x4 *)(qc + 64 * kb + 32 + 16 * hl);
          q8[2 * kb] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
          q8[2 * kb + 1] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        return;
      }
      const int hl = lane_id_here() >> 5;
      const uint16_t *qn = a.q + r * a.q_stride;
      const uint16_t *qr = a.q_rope ? a.q_rope + r * (kHeadDim - kHeadDimV) : qn + kHeadDimV;
#pragma unroll
      for (int kb = 0; kb < 9; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int C = q_chunk_f8(kb, i, hl);        // 8 dims, C in 0..71
          set_q8_chunk(kb, i, *(const bf16x8 *)(C < kHeadDimV / 8 ? qn + 8 * C : qr + 8 * (C - kHeadDimV / 8)));
        }
    } else {
      // dims 16 ks + 8 hl .. +7
      const int hl8 = 8 * (lane_id_here() >> 5);
      const uint16_t *qn = a.q + r * a.q_stride + hl8;
      const uint16_t *qr = a.q_rope ? a.q_rope + r * (kHeadDim - kHeadDimV) + hl8 : qn + kHeadDimV;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        qf[ks] = *(const bf16x8 *)(ks < kHeadDimV / 16 ? qn + 16 * ks : qr + 16 * (ks - kHeadDimV / 16));
    }
  };

  int cur = 0;              // buffer that receives / holds the next page to process
  bool have_first = false;  // the first page of the current split is already in flight into it
  // Block-table entries of a split are fetched one split ahead: lane i holds
  // table entry base + i, base = the entry of the split's first token.
  int bt_pref = 0;
  {
    // The part's first block-table entries and length load together.  Then
    // either (a) its q rows are staged through LDS (stage_q_rows) and, once
    // every wave has read them back, its first page's copy goes out; or (b)
    // where the rows cannot be staged (split q, heads per KV head not a
    // multiple of 32, a partial 128-row tile, no first page) the page's copy
    // goes out first and then the direct q loads.  Every workgroup starts at
    // once and the start-up loads share HBM; the direct q loads touch 32 rows
    // per instruction and were the slower half of the start-up: on the
    // standard B=64 decode (a) took the decode from 62.8 to 61.5 us, and in
    // (b) requesting the page before q gained about 1 us over q first.
    // (Lanes past the split's blocks hold entries that are never used; the
    // index is clamped into the table row.)
    const int first0 = max(0, md[1]);
    const int base0 = first0 * kPage / bs;
    const int32_t *bt0 = a.block_table + (long)b0 * a.max_blocks;
    bt_pref = bt0[min(base0 + lane, a.max_blocks - 1)];
    // (a): the tile's 4 x 32 rows are whole 32-row runs of consecutive q rows
    // (no split q), and their 4 x 36 KiB fill both page buffers exactly.  The
    // copy depends on the table row alone, so it goes out before the length
    // of b0 has arrived.
    const bool staged = a.q_rope == nullptr && !a.q_fp8 && a.group % 32 == 0 &&
                        (rt + 1) * kRowsPerTile <= a.rows && a.q_stride == kHeadDim;   // workgroup-uniform
    LDS_AS uint8_t *region = smem + wave * 32 * kHeadDim * 2;
    if (staged) {
      const int qi = wrow0 / a.group, h0 = hk * a.group + wrow0 % a.group;
      const uint8_t *qblock = (const uint8_t *)(a.q + (((long)b0 * a.s_q + qi) * a.hq + h0) * kHeadDim);
      stage_q_rows(qblock, region, lane);
    }
    const int len0 = seq_len(b0);
    const int nblk0 = (len0 + kPage - 1) / kPage;
    const int hi0 = seq_end(b0, nblk0);
    if (staged) {
      wait_vmcnt<0>();
      if constexpr (kFp8) {
#pragma unroll
        for (int kb = 0; kb < 9; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x8 v = *q_row_chunk(region, lane & 31, q_chunk_f8(kb, i, lane >> 5));
            set_q8_chunk(kb, i, v);
          }
      } else {
        read_q_rows(region, lane, qf);
      }
      __syncthreads();                                // q read back before the page lands on it
    }
    if (hi0 > first0) {                               // then the split's first page is first0
      // (A slice past the sequence's end takes its last block: its rows are
      // masked, and table entries past the sequence are never used.)
      const int t = slice_tok(first0);
      const int k = min(t / bs, (len0 - 1) / bs);     // in [base0, base0 + 3]
      const PageSrc src = src_of(__builtin_amdgcn_readlane(bt_pref, k - base0), t % bs);
      if (kFp8) dma_page_fp8<kSplit>(src, bufs[0], wave);
      else dma_page_bf16<kSplit>(src, bufs[0], wave);
      have_first = true;
    }
    if (!staged && active) load_q(b0);              // waves without rows need no q
  }
  for (int b = b0; b <= b1; ++b) {
    const int L = seq_len(b);
    const int nblk = (L + kPage - 1) / kPage;
    const int hi = seq_end(b, nblk);
    const int lo = b == b0 ? max(0, min(md[1], hi)) : 0;
    const int first_slot = a.num_splits[b];
    const int nsplit = a.num_splits[b + 1] - first_slot;
    const int slot = max(0, min(first_slot + (b == b0 ? md[4] : 0), nslots - 1));
    const int nvis = a.causal ? max(0, min(L, L - a.s_q + 1 + row_coord(wrow0, a.rows, a.group, hk).qi)) : L;
    // Smallest visible-key count of the workgroup (its first query token sees
    // the fewest keys): pages at or past it need per-key masking.
    const int nvis_min = a.causal ? max(0, min(L, L - a.s_q + 1 + qi_min)) : L;
    const int32_t *bt = a.block_table + (long)b * a.max_blocks;
    // First page of the next split of this part (page 0 of b + 1), copied
    // while the last page of this split is processed.
    int next_blk = 0;                                     // block of this wave's slice of page 0 of b + 1
    bool next_has_pages = false;
    const int bt_this = bt_pref;                          // block-table lanes of this split (loaded earlier)
    if (b < b1) {
      const int Ln = seq_len(b + 1);
      const int nblk_n = (Ln + kPage - 1) / kPage;
      next_has_pages = seq_end(b + 1, nblk_n) > 0;
      if (next_has_pages) {
        const int32_t *bt_n = a.block_table + (long)(b + 1) * a.max_blocks;
        next_blk = bt_n[min(16 * wave / bs, max(0, (Ln + bs - 1) / bs - 1))];
        bt_pref = bt_n[min(lane, max(0, (Ln + bs - 1) / bs - 1))];   // next split starts at token 0
      }
    }
    if (tid == 0) *rerun_flag = 0;

    // l: the row sum of the probabilities; lq: with an fp8 cache, the sum of
    // the same probabilities as rounded for the matrix core (the output's
    // normaliser); equal to l otherwise.
    float m = kNegInf, l = 0.f, lq = 0.f, m_restart = kNegInf;
    // kKeySplit: wave 0's factors on its own O and on wave 1's (in LDS at merge_buf).
    float merge_a0 = 1.f, merge_a1 = 0.f;
    const LDS_AS uint8_t *merge_buf = smem;
    bool merged = false;                                  // workgroup-uniform
    // O^T accumulators start as the result of an all-zero MFMA so that they
    // live in accumulation registers from the first page on.
    f32x16 o[kOTiles];
    mfma_zero_all(o);

    if (hi > lo) {
      // Block-table entries of the split live in one VGPR, lane i holding
      // entry bt_base + i, so a lookup is a v_readlane instead of a global-
      // memory round trip per page; refilled when a slice leaves the window.
      const int nent = (L + bs - 1) / bs;                // table entries of the sequence
      int bt_base = lo * kPage / bs;
      int bt_vec = bt_this;
      auto block_of = [&](int k) -> int {                // table entry k (wave-uniform)
        if ((unsigned)(k - bt_base) >= 64u) {        // also on a re-run from lo
          bt_base = k;
          bt_vec = bt[min(k + lane, nent - 1)];
        }
        return __builtin_amdgcn_readlane(bt_vec, k - bt_base);
      };
      auto page_src = [&](int j) -> PageSrc {            // this wave's slice of page j
        if (!kAnyBlock) return src_of(block_of(j), 16 * wave);
        const int t = slice_tok(j);
        return src_of(block_of(min(t / bs, nent - 1)), t % bs);
      };
      if constexpr (kFp8) {
        if (a.q_fp8) {
          s_hi = s_lo = 127;                        // codes as loaded, lo term zero
        } else {
          quantize_q_f8(q8, s_hi, s_lo);
        }
      }
      for (int pass = 0;; ++pass) {
        bool need = false;
        // fp8: the previous page's tile-1 weights, not yet in O (see attend_page_f8).
        bool has_prev = false;
        u32x4 p1 = {0, 0, 0, 0};
        int e1 = 0;
        if (!have_first) {
          if (kFp8) dma_page_fp8<kSplit>(page_src(lo), bufs[cur], wave);
          else dma_page_bf16<kSplit>(page_src(lo), bufs[cur], wave);
        }
        have_first = false;
        for (int j = lo; j < hi; ++j) {
          // Page j has landed in every wave's share; every wave is done with
          // the buffer that the copy of the next page reuses (the previous
          // page's with two buffers; the one before it with three, where the
          // previous page is still read by this page's PV step).
          wait_vmcnt<0>();
          __syncthreads();
          const int nvalid = min(kPage, L - j * kPage);
          if (nvalid < kPage) {                     // the sequence's last, partial page
            if (kFp8) zero_tail_rows_fp8(bufs[cur], nvalid, tid);
            else zero_tail_rows(bufs[cur], nvalid, tid);
            __syncthreads();
          }
          NextPage nx;
          nx.valid = j + 1 < hi || next_has_pages;
          nx.src = j + 1 < hi ? page_src(j + 1) : src_of(next_blk, 16 * wave % bs);
          nx.dst = bufs[buf_next(cur)];
          nx.wave = wave;
          const bool copy_later = kSerialCopies && nx.valid;
          if constexpr (kSerialCopies) nx.valid = false;
          const LDS_AS uint8_t *pg = bufs[cur];
          if (active) {
            if constexpr (kFp8)
              // (V^T two ahead spills in the split-cache and any-block kernels)
              need |= attend_page_f8<kSplit, kSplit || kAnyBlock ? 1 : 2>(pg, q8, s_hi, s_lo, o, m, l, lq, m_restart, lane, j * kPage, nvis,
                                             scale_log2, (j + 1) * kPage > nvis_min, desc_tab, descale, !a.q_fp8,
                                             nx, bufs[buf_prev(cur)], has_prev, p1, e1);
            else if constexpr (kKeySplit)
              need |= attend_tile<kSplit>(pg, qf, o, m, l, m_restart, lane, j * kPage + 32 * wave, nvis, scale_log2,
                                  (j + 1) * kPage > nvis_min, desc_tab, descale, nx, wave);
            else
              need |= attend_page<kSplit>(pg, qf, o, m, l, m_restart, lane, j * kPage, nvis, scale_log2,
                                                 (j + 1) * kPage > nvis_min, desc_tab, descale, nx);
          } else if (nx.valid) {                    // a wave without rows still copies its share
            if (kFp8) dma_page_fp8<kSplit>(nx.src, nx.dst, wave);
            else dma_page_bf16<kSplit>(nx.src, nx.dst, wave);
          }
          if constexpr (kSerialCopies) {
            __syncthreads();                        // every wave is done with this page
            if (copy_later) {
              if (kFp8) dma_page_fp8<kSplit>(nx.src, nx.dst, wave);
              else dma_page_bf16<kSplit>(nx.src, nx.dst, wave);
            }
          }
          has_prev = true;
          cur = buf_next(cur);
        }
        // fp8: the last page's tile 1 (its buffer is intact: the next
        // split's first page went to the buffer after it).
        if (kFp8 && active && has_prev) attend_drain_f8(bufs[buf_prev(cur)], p1, e1, o, lane);
        if (need && lane == 0) *rerun_flag = 1;
        __syncthreads();
        const bool again = (*rerun_flag != 0) && (pass + 1 < kMaxPasses);   // workgroup-uniform
        __syncthreads();
        if (!again) {
          have_first = next_has_pages;              // page 0 of b + 1 is in flight into bufs[cur]
          if constexpr (kKeySplit) {
            // Waves 0 and 1 hold the states of tiles 0 and 1 of the same
            // rows; wave w finishes output tiles 8w .. 8w+7 of their merge.
            // Each sends the other half of its O^T, with its (m, l), through
            // the buffer of the split's last page (every wave is past it; the
            // next split's first page goes to the other buffer).  The common
            // reference is the larger m; each side is scaled by 2^(m - M).
            LDS_AS uint8_t *xb = bufs[buf_next(cur)];
            if (wave < 2) {
              // o[8..15] of either wave holds the output tiles its partner
              // finishes (wave 1 keeps output tiles 8..15 in o[0..7]; see
              // attend_tile): wave w sends them to region 1 - w.
              LDS_AS uint8_t *dst = xb + (1 - wave) * 32768;
#pragma unroll
              for (int t = 0; t < kOTiles / 2; ++t)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                  *(LDS_AS f32x4 *)(dst + ((t * 4 + q4) * 64 + lane) * 16) =
                      f32x4{o[t + 8][4 * q4], o[t + 8][4 * q4 + 1], o[t + 8][4 * q4 + 2], o[t + 8][4 * q4 + 3]};
              *(LDS_AS f32x2 *)(xb + 65536 + wave * 512 + lane * 8) = f32x2{m, l};
            }
            __syncthreads();
            if (wave < 2) {
              const f32x2 ml = *(const LDS_AS f32x2 *)(xb + 65536 + (1 - wave) * 512 + lane * 8);
              const float M = fmaxf(m, ml[0]);
              merge_a0 = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - M);
              merge_a1 = ml[0] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(ml[0] - M);
              // Both waves form the same merged l (the same two terms in
              // wave order), so their normalisers agree bit for bit.
              const float l0 = wave == 0 ? l : ml[1], l1 = wave == 0 ? ml[1] : l;
              const float a_0 = wave == 0 ? merge_a0 : merge_a1, a_1 = wave == 0 ? merge_a1 : merge_a0;
              l = l0 * a_0 + l1 * a_1;
              m = M;
              merge_buf = xb + wave * 32768;
            }
            merged = true;
          }
          break;
        }
        wait_vmcnt<0>();                            // drop the copy of the next split's first page
        if (tid == 0) *rerun_flag = 0;
        if (m_restart != kNegInf) m = m_restart;
        m_restart = kNegInf;
        l = 0.f;
        lq = 0.f;
        mfma_zero_all(o);
      }
    }
    // The next split's q is loaded first, so its latency hides behind the
    // epilogue (the next page's wait covers it).  With two waves per page the
    // merging epilogue needs the registers: q follows it.
    if (!kKeySplit && b < b1 && active) load_q(b + 1);

    // Epilogue.  A sequence with one split writes out / lse; otherwise the
    // split writes its normalised output (bf16) and lse to its partial slot,
    // which is its split number num_splits[b] + k.
    if (active) {
      const bool direct = nsplit <= 1;
      const RowCoord c = row_coord(wrow0, a.rows, a.group, hk);
      // Normaliser.  With a sink logit z (FlashInfer MLA page, sinks; a
      // sequence with one split takes it here, split sequences in the
      // combine) the denominator l 2^m gains e^z = 2^zs: with M = max(m, zs)
      // it is lt 2^M, lt = l 2^(m-M) + 2^(zs-M), and O (relative to 2^m) is
      // scaled by 2^(m-M) / lt.  Without a sink this is 1/l and m + log2 l.
      float zs = kNegInf;
      if (direct && a.sinks) zs = a.sinks[c.h] * kLog2e;
      const float mm = fmaxf(m, zs);
      float lt = 0.f, inv = 0.f;
      if (mm != kNegInf) {
        const float am = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mm);
        const float zt = __builtin_amdgcn_exp2f(zs - mm);
        lt = l * am + zt;
        // O holds sum_t p~_t v_t with the rounded weights p~ of an fp8 cache:
        // normalise by their sum (scaled to lt) so that they add up to one.
        inv = kFp8 ? (lq > 0.f ? l * am / (lt * lq) : 0.f) : am / lt;
      }
      const bool bad = bad_scale || (descale && bad_value(desc_tab[lane & 31]));
      if (bad) inv = __builtin_nanf("");
      const float lse_v = bad ? __builtin_nanf("") : lt > 0.f ? (mm + __log2f(lt)) * kLn2 : kNegInf;
      const int prow = (slot * a.hk + hk) * a.rows + c.rowc;
      const int orow = ((b * a.s_q + c.qi) * a.hq + c.h);
      const int rows_pad = (a.rows + kPartRows - 1) / kPartRows * kPartRows;
      const int nrows = max(0, min(32, uniform_here(a.rows) - wrow0));
      uint16_t *pblk = a.part_o + ((long)(slot * a.hk + hk) * rows_pad + wrow0) * kHeadDimV;
      if (kKeySplit && merged) {
        // Wave w stores output tiles 8w .. 8w+7 of the merged state (its o[0..7]).
        const float f = direct ? inv * vfac_tab[lane & 31] : inv;
        if (direct) store_rows<true>(o, f * merge_a0, a.out, orow, nrows, merge_buf, f * merge_a1, wave);
        else store_acc_block<true>(o, f * merge_a0, pblk, merge_buf, f * merge_a1, wave);
      } else if (kKeySplit && wave == 1) {
        // (no pages in this split: wave 0 alone writes the empty result)
      } else if (direct && (kKeySplit || a.pv_descale)) {
        store_rows(o, inv * vfac_tab[lane & 31], a.out, orow, nrows);
      } else if (direct) {
        store_rows(o, inv * (a.bmm2_dev ? *a.bmm2_dev : a.v_scale), a.out, orow, nrows);
      } else {
        store_acc_block(o, inv, pblk);
      }
      if (lane_id_here() < 32 && c.row < a.rows && (!kKeySplit || wave == 0)) {
        if (direct) a.lse[((long)b * a.hq + c.h) * a.s_q + c.qi] = lse_v;
        else a.part_lse[prow] = lse_v;
      }
    }
    if (kKeySplit && b < b1 && active) load_q(b + 1);
  }
}

// The combine works on units of one 32-row partial block and kSlots of its
// 32 chunk slots (slot = 2t + pp, see store_acc_block): 32 / kSlots units per
// block.  A lane owns one row (lane % 32) and, in each of its slots, 8 dims
// of it, so the per-row weights are per-lane scalars and every load is a
// contiguous 1 KiB per wave.
constexpr int kBlockSlots = 2 * kOTiles;                  // 32 chunk slots per 32-row block

// Running merge of splits 0..n-1 (kBatch per iteration, all their loads in
// flight together; the running max rescales the sums) of one unit into
// (mu, Z, acc): sum_k e^(lse_k - mu) = Z and sum_k e^(lse_k - mu) O_k = acc.
// Past the last split a batch either loads nothing (kGuard) or repeats the
// last split's loads, weighted 0 (cheaper when a wave merges many splits).
//   pl: this lane's row lse of split 0; po: this lane's first chunk of the
//   unit in split 0; lstride / ostride: elements between splits.
template <int kBatch, int kSlots, bool kGuard = false>
__device__ __forceinline__ void merge_splits(const float *pl, const uint16_t *po, long lstride, long ostride, int n,
                                             float &mu, float &Z, float (&acc)[kSlots][8]) {
  for (int k0 = 0; k0 < n; k0 += kBatch) {
    float lk[kBatch];
    bf16x8 vk[kBatch][kSlots];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int k = min(k0 + i, n - 1);               // past n: a repeat, weighted 0 below
      if (kGuard && k0 + i >= n) {                    // wave-uniform
        lk[i] = kNegInf;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) vk[i][j] = bf16x8{};
        continue;
      }
      lk[i] = pl[k * lstride];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) vk[i][j] = *(const bf16x8 *)(po + k * ostride + j * 512);
    }
    float mb = mu;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (k0 + i < n) mb = fmaxf(mb, lk[i]);
    if (mb == kNegInf) continue;                      // every split so far is empty
    const float sc = __builtin_amdgcn_exp2f((mu - mb) * kLog2e);   // 0 while mu = -inf
    Z *= sc;
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= sc;
    mu = mb;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float w = k0 + i < n ? __builtin_amdgcn_exp2f((lk[i] - mu) * kLog2e) : 0.f;
      Z += w;
#pragma unroll
      for (int j = 0; j < kSlots; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] += w * (float)vk[i][j][e];
    }
  }
}

// Folds the state (mu2, Z2, acc2) into (mu, Z, acc) (both relative to their
// own max; a state with mu = -inf is empty).
template <int kSlots>
__device__ __forceinline__ void fold_state(float &mu, float &Z, float (&acc)[kSlots][8], float mu2, float Z2,
                                           const float (&acc2)[kSlots][8]) {
  const float mm = fmaxf(mu, mu2);
  if (mm == kNegInf) return;
  const float s1 = mu == kNegInf ? 0.f : __builtin_amdgcn_exp2f((mu - mm) * kLog2e);
  const float s2 = mu2 == kNegInf ? 0.f : __builtin_amdgcn_exp2f((mu2 - mm) * kLog2e);
  Z = Z * s1 + Z2 * s2;
#pragma unroll
  for (int j = 0; j < kSlots; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] * s1 + acc2[j][e] * s2;
  mu = mm;
}

// Merge the split partials of every sequence with more than one split:
// out = v_scale * sum_k w_k O_k / sum_k w_k, w_k = exp(lse_k - max lse),
// lse = max + ln sum_k w_k.  Splits with lse = -inf weigh 0.  Workgroups of
// 4 waves and units of kCombineSlots slots; two launch shapes, chosen on the
// host:
//   - 4 units per workgroup, one wave per unit, 4 splits per round (batches
//     with a few splits per sequence);
//   - when there are more than 4 parts per sequence, so that some sequence
//     may be split many ways: one workgroup per unit.  A sequence with at
//     most kCombineWide splits is merged by the first wave alone (the others
//     exit at once); one with more spreads the splits over the 4 waves --
//     wave q merges splits q, q + 4, ... and the first wave folds the four
//     states from LDS in wave order -- so a sequence spread over hundreds of
//     parts gets four waves' worth of loads in flight.
// A sink logit z (FlashInfer MLA page, sinks) is folded last as a state
// (z, 1, 0): one more term of weight e^z and no value.
constexpr int kCombineWays = 4;
constexpr int kCombineWide = 8;
constexpr int kCombineSlots = 1;                      // chunk slots per unit (1 KiB per split and wave)
__host__ __device__ inline bool combine_per_unit(const DecodeArgs &a) { return a.num_parts > 4 * a.batch; }
__host__ __device__ inline int combine_units(const DecodeArgs &a, int slots) {
  return a.hk * ((a.rows + kPartRows - 1) / kPartRows) * (kBlockSlots / slots);
}
template <int kSlots, bool kWideShape>
__global__ __launch_bounds__(kCombineWays * 64) void mla_combine_kernel(const DecodeArgs a) {
  constexpr int kGroups = kBlockSlots / kSlots;       // units per 32-row block
  __shared__ float st_mu[kWideShape ? kCombineWays : 1][64], st_z[kWideShape ? kCombineWays : 1][64];
  __shared__ __attribute__((aligned(16))) float st_acc[kWideShape ? kCombineWays : 1][kSlots * 8][64];
  const int b = blockIdx.y;
  const int nrows = a.batch + a.num_parts - 1;        // partial slots written by the decode kernel
  const int slot0 = max(0, min(a.num_splits[b], nrows));
  const int n = min(a.num_splits[b + 1] - slot0, nrows - slot0);
  if (n <= 1) return;                                 // workgroup-uniform
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int unit;
  bool wide = false;                                  // workgroup-uniform
  if (kWideShape) {
    unit = blockIdx.x;
    wide = n > kCombineWide;
    if (!wide && wv != 0) return;
  } else {
    unit = blockIdx.x * kCombineWays + wv;
  }
  if (unit >= combine_units(a, kSlots)) return;               // wave-uniform (whole workgroups in the wide shape)
  const int blocks = (a.rows + kPartRows - 1) / kPartRows;
  const int g = unit % kGroups, blk = (unit / kGroups) % blocks, hk = unit / (kGroups * blocks);
  const int rows_pad = blocks * kPartRows;
  const int row = blk * kPartRows + (lane & 31);
  const int rowc = min(row, a.rows - 1);
  const int way = wide ? wv : 0, ways = wide ? kCombineWays : 1;
  float mu = kNegInf, Z = 0.f;
  float acc[kSlots][8] = {};
  if (way < n) {
    const long lstride = (long)a.hk * a.rows;
    const long ostride = (long)a.hk * rows_pad * kHeadDimV;
    const float *pl = a.part_lse + ((long)(slot0 + way) * a.hk + hk) * a.rows + rowc;
    const uint16_t *po = a.part_o + ((long)(slot0 + way) * a.hk + hk) * rows_pad * kHeadDimV +
                         (long)blk * kPartRows * kHeadDimV + (g * kSlots * 64 + lane) * 8;
    merge_splits<kWideShape ? 8 : 4, kSlots, !kWideShape>(pl, po, ways * lstride, ways * ostride, (n - way + ways - 1) / ways, mu, Z, acc);
  }
  if (kWideShape && wide) {
    st_mu[wv][lane] = mu;
    st_z[wv][lane] = Z;
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) st_acc[wv][j * 8 + e][lane] = acc[j][e];
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int q = 1; q < kCombineWays; ++q) {
      float accq[kSlots][8];
#pragma unroll
      for (int j = 0; j < kSlots; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) accq[j][e] = st_acc[q][j * 8 + e][lane];
      fold_state(mu, Z, acc, st_mu[q][lane], st_z[q][lane], accq);
    }
  }
  const int qi = rowc / a.group;
  const int h = hk * a.group + (rowc - qi * a.group);
  if (a.sinks) {
    const float zero[kSlots][8] = {};
    fold_state(mu, Z, acc, a.sinks[h], 1.f, zero);
  }
  const bool bad_scale = bad_device_scale(a) || (a.qk_descale && bad_value(a.qk_descale[h]));
  const float inv = bad_scale ? __builtin_nanf("") : Z > 0.f ? row_v_scale(a, h) / Z : 0.f;
  // Slot j of the unit is chunk slot 2t + pp = kSlots g + j: this lane
  // holds dims 32t + 16pp + 4hl + {0..3} (acc[j][0..3]) and + 8 (acc[j][4..7]).
  // v_permlane32_swap with lane ^ 32 forms whole 16-byte chunks: lanes < 32
  // then hold dims 32t + 16pp + 8 .. +15, lanes >= 32 dims 32t + 16pp .. +7.
  const int hl = lane >> 5;
  uint16_t *orow = a.out + (((long)b * a.s_q + qi) * a.hq + h) * kHeadDimV + 8 * (1 - hl);
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int tp = g * kSlots + j, t = tp >> 1, pp = tp & 1;
    const unsigned a0 = pack_bf16(acc[j][0] * inv, acc[j][1] * inv);
    const unsigned a1 = pack_bf16(acc[j][2] * inv, acc[j][3] * inv);
    const unsigned b0 = pack_bf16(acc[j][4] * inv, acc[j][5] * inv);
    const unsigned b1 = pack_bf16(acc[j][6] * inv, acc[j][7] * inv);
    const auto s0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
    if (row < a.rows) *(u32x4 *)(orow + 32 * t + 16 * pp) = u32x4{s0[0], s1[0], s0[1], s1[1]};
  }
  if (g == 0 && lane < 32 && row < a.rows)
    a.lse[((long)b * a.hq + h) * a.s_q + qi] = bad_scale ? __builtin_nanf("") : Z > 0.f ? mu + __logf(Z) : kNegInf;
}

// Counter calibration: streams `chunks` KiB from src into LDS with the page
// copies' instruction (global_load_lds_dwordx4 with the non-temporal hint),
// 1 KiB per wave instruction, up to 8 in flight per wave.  Nothing is
// written to global memory.
__global__ __launch_bounds__(256) void lds_dma_read_kernel(const uint8_t *src, long chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][8][1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const long stride = (long)gridDim.x * 4;
  int slot = 0;
  for (long c = (long)blockIdx.x * 4 + wave; c < chunks; c += stride) {
    lds_dma16<0>(src + c * 1024 + lane * 16, (LDS_AS void *)&ring[wave][slot][0]);
    if (++slot == 8) {
      wait_vmcnt<0>();
      slot = 0;
    }
  }
  wait_vmcnt<0>();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  // Two pages (bf16 size), the restart flag, per-row qkDescale and output factors.
  const size_t smem = 2 * (size_t)kPageBytes + 16 + 2 * kRowsPerTile * 4;
  const dim3 grid(a.num_parts, a.row_tiles * a.hk);   // one persistent workgroup per part
  auto launch = [&](auto kernel) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), smem, stream, a);
    return hipGetLastError();
  };
  // At most 32 rows per workgroup (bf16 cache): two waves split each page's tokens.
  const bool key_split = !a.kv_fp8 && a.rows <= 32;
  auto by_block = [&](auto fp8, auto split) -> hipError_t {
    constexpr bool f = decltype(fp8)::value, s = decltype(split)::value;
    if constexpr (!f) {
      if (key_split)
        return a.page_size == kPage ? launch(mla_decode_kernel<false, s, false, true>)
                                    : launch(mla_decode_kernel<false, s, true, true>);
    }
    return a.page_size == kPage ? launch(mla_decode_kernel<f, s, false>) : launch(mla_decode_kernel<f, s, true>);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (a.kv_fp8) return a.kv_rope ? by_block(T{}, T{}) : by_block(T{}, F{});
  return a.kv_rope ? by_block(F{}, T{}) : by_block(F{}, F{});
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream) {
  const int units = combine_units(a, kCombineSlots);
  if (combine_per_unit(a))
    hipLaunchKernelGGL((mla_combine_kernel<kCombineSlots, true>), dim3(units, a.batch), dim3(kCombineWays * 64), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((mla_combine_kernel<kCombineSlots, false>), dim3((units + kCombineWays - 1) / kCombineWays,
                       a.batch), dim3(kCombineWays * 64), 0, stream, a);
  return hipGetLastError();
}

// Device-resident scratch of the no-allocation entry point
// (mla_decode_fwd_noalloc): the partial outputs and log-sum-exps that
// mla_decode_fwd keeps in its caller's workspace.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code the array's
// name is only a stand-in for a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void *addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_lds_dma_read(const void *src, size_t bytes, hipStream_t stream) {
  const long chunks = (long)(bytes / 1024);
  const int grid = (int)std::min<long>(2048, std::max<long>(1, (chunks + 3) / 4));
  hipLaunchKernelGGL(lds_dma_read_kernel, dim3(grid), dim3(256), 0, stream, (const uint8_t *)src, chunks);
  return hipGetLastError();
}

}  // namespace mla
