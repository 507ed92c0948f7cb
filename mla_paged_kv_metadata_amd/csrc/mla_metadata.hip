// Split-KV tile scheduler for MLA decode (gfx950).
//
// The FlashMLA interface page (docstring of get_mla_metadata) fixes the
// outputs' shapes -- a (num_sm_parts, TileSchedulerMetaDataSize) int32 table
// and num_splits (batch + 1) int32, "splits per sample" -- but not their
// content.  The balancing rule is this library's own:
//   sequence b costs fixed_cost + nblk_b units (nblk_b = ceil(L_b / 64));
//   units of all sequences are laid end to end in batch order; part p owns
//   units [p*W, (p+1)*W) with W = ceil(total / num_parts).  Part p works on
//   sequence b if it owns one of b's page units (or, when b has no pages, b's
//   first unit); each such pair is one split of b.
// The table lists every split as its own row (batch + num_parts - 1 rows, the
// most splits possible): row num_splits[b] + k is split k of sequence b, so a
// decode workgroup handles exactly one (sequence, page range).  Every entry
// is a closed form of two prefix sums, so one workgroup computes the table in
// O(batch + rows) with no device-to-host traffic.
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kT = kMetaThreads;

__device__ __forceinline__ long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Exclusive scan over `n` int64 values held in smem[0..n), in place; smem[n] = total.
// Each thread scans a contiguous chunk; chunk sums are scanned in `tmp`.
__device__ void block_exclusive_scan(long long *smem, int n, long long *tmp) {
  const int tid = threadIdx.x;
  const int per = (n + kT - 1) / kT;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  long long s = 0;
  for (int i = lo; i < hi; ++i) s += smem[i];
  tmp[tid] = s;
  __syncthreads();
  for (int off = 1; off < kT; off <<= 1) {      // Hillis-Steele inclusive scan of chunk sums
    long long v = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += v;
    __syncthreads();
  }
  long long run = tid ? tmp[tid - 1] : 0;
  for (int i = lo; i < hi; ++i) {
    long long x = smem[i];
    smem[i] = run;
    run += x;
  }
  __syncthreads();
  if (tid == kT - 1) smem[n] = tmp[kT - 1];
  __syncthreads();
}

// largest b in [0, n] with pref[b] <= x  (pref strictly increasing because every cost >= 1)
__device__ __forceinline__ int upper_index(const long long *pref, int n, long long x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kT) void mla_metadata_kernel(const int32_t *__restrict__ seqlens, int B,
                                                           int num_parts, int fixed_cost,
                                                           int32_t *__restrict__ tile_md,
                                                           int32_t *__restrict__ num_splits) {
  extern __shared__ long long smem[];
  long long *pref = smem;                // B + 1 entries: cost prefix
  long long *cnt = smem + (B + 1);       // B + 1 entries: split-count prefix
  long long *tmp = smem + 2 * (B + 1);   // kT entries
  const int tid = threadIdx.x;
  const long long fc = fixed_cost;

  for (int b = tid; b < B; b += kT) pref[b] = fc + ceil_div(max(seqlens[b], 0), kPage);
  __syncthreads();
  block_exclusive_scan(pref, B, tmp);
  const long long total = pref[B];
  const long long W = max(1LL, ceil_div(total, num_parts));

  for (int b = tid; b < B; b += kT) {
    const long long nblk = pref[b + 1] - pref[b] - fc;
    const long long s = pref[b] + fc;                       // first page unit of b
    cnt[b] = nblk > 0 ? (s + nblk - 1) / W - s / W + 1 : 1;
  }
  __syncthreads();
  block_exclusive_scan(cnt, B, tmp);
  for (int b = tid; b <= B; b += kT) num_splits[b] = (int32_t)cnt[b];

  const long long splits = cnt[B];
  const int rows = B + num_parts - 1;
  for (int r = tid; r < rows; r += kT) {
    int32_t *row = tile_md + (size_t)r * 8;
    row[5] = (int32_t)W;
    row[6] = fixed_cost;
    if (r >= splits) {
      row[0] = -1; row[1] = 0; row[2] = 0; row[3] = 0; row[4] = 0; row[7] = -1;
      continue;
    }
    const int b = upper_index(cnt, B, r);                   // cnt strictly increasing
    const long long k = r - cnt[b];
    const long long n = cnt[b + 1] - cnt[b];
    const long long nblk = pref[b + 1] - pref[b] - fc;
    const long long s = pref[b] + fc;
    long long p, first = 0, end = 0;
    if (nblk > 0) {
      p = s / W + k;
      first = max(0LL, p * W - s);
      end = min(nblk, (p + 1) * W - s);
    } else {
      p = pref[b] / W;
    }
    row[0] = b; row[1] = (int32_t)first; row[2] = (int32_t)end; row[3] = (int32_t)k; row[4] = (int32_t)n;
    row[7] = (int32_t)p;
  }
}

}  // namespace

hipError_t launch_metadata(const int32_t *seqlens, int batch, int num_parts, int fixed_cost,
                           int32_t *tile_md, int32_t *num_splits, hipStream_t stream) {
  const size_t smem = (2 * (size_t)(batch + 1) + kT) * sizeof(long long);
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void *)mla_metadata_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mla_metadata_kernel, dim3(1), dim3(kT), smem, stream, seqlens, batch, num_parts,
                     fixed_cost, tile_md, num_splits);
  return hipGetLastError();
}

}  // namespace mla
