// Split-KV tile scheduler for MLA decode (gfx950).
//
// The FlashMLA interface page (docstring of get_mla_metadata) fixes the
// outputs' shapes -- a (num_sm_parts, TileSchedulerMetaDataSize) int32 table
// and num_splits (batch + 1) int32, "splits per sample" -- but not their
// content.  The balancing rule is this library's own:
//   sequence b costs fixed_cost + nblk_b units (nblk_b = ceil(L_b / 64)):
//   ceil(fixed_cost / 2) overhead units, its page units, then the other
//   floor(fixed_cost / 2) overhead units (a split's overhead is both its q
//   load at the start and its result stores at the end);
//   units of all sequences are laid end to end in batch order; part p owns
//   units [floor(p*total/P), floor((p+1)*total/P)) (P = num_parts), so parts
//   differ by at most one unit and none idles while total >= P.  Part p works on
//   sequence b if it owns one of b's page units (or, when b has no pages, b's
//   first unit); each such pair is one split of b, numbered k = 0, 1, ... in
//   part order.
// Row p of the table tells the persistent decode workgroup of part p what to
// do: [b0, first page of b0, b1, end page of b1, k of b0's split, W,
// fixed_cost, splits of the part] -- sequences strictly between b0 and b1 are
// whole.  Idle parts get b0 = b1 = -1.  Every entry is a closed form of the
// cost prefix sum (and num_splits of the split-count prefix sum), so one
// workgroup computes everything in O(batch + parts log batch) with no
// device-to-host traffic.
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kT = kMetaThreads;

__device__ __forceinline__ long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Exclusive scan over `n` int64 values held in smem[0..n), in place; smem[n] = total.
// Each thread scans a contiguous chunk; chunk sums are scanned within each
// wave by shuffles, then across the kT / 64 wave totals (held in `tmp`).
__device__ void block_exclusive_scan(long long *smem, int n, long long *tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + kT - 1) / kT;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  long long s = 0;
  for (int i = lo; i < hi; ++i) s += smem[i];
  long long incl = s;                              // inclusive scan of chunk sums within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    long long run = 0;
    for (int w = 0; w < kT / 64; ++w) {
      const long long t = tmp[w];
      tmp[w] = run;
      run += t;
    }
    tmp[kT / 64] = run;
  }
  __syncthreads();
  long long run = tmp[wave] + incl - s;
  for (int i = lo; i < hi; ++i) {
    const long long x = smem[i];
    smem[i] = run;
    run += x;
  }
  __syncthreads();
  if (tid == 0) smem[n] = tmp[kT / 64];
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

template <typename T>
__device__ __forceinline__ void fill_rows(int B, int num_parts, int fixed_cost,
                                          int32_t *__restrict__ tile_md, int32_t *__restrict__ num_splits,
                                          long long *pref, long long *cnt, long long *tmp) {
  const int tid = threadIdx.x;
  const T fc = fixed_cost;
  const T fs = (fc + 1) / 2;                                  // overhead units before a sequence's pages
  const T total = (T)pref[B];
  const T P = num_parts;
  const T W = max((T)1, (total + P - 1) / P);                 // most units of one part
  auto bound = [&](T p) -> T { return p * total / P; };
  auto part_of = [&](T u) -> T { return ((u + 1) * P - 1) / total; };   // u < total

  for (int b = tid; b < B; b += kT) {
    const T nblk = (T)(pref[b + 1] - pref[b]) - fc;
    const T s = (T)pref[b] + fs;                            // first page unit of b
    cnt[b] = nblk <= 0 ? 1 : (total >= P ? part_of(s + nblk - 1) - part_of(s) + 1 : nblk);
  }
  __syncthreads();
  block_exclusive_scan(cnt, B, tmp);
  for (int b = tid; b <= B; b += kT) num_splits[b] = (int32_t)cnt[b];

  for (int p = tid; p < num_parts; p += kT) {
    int32_t *row = tile_md + (size_t)p * 8;
    const T u0 = bound(p), u1 = bound(p + 1);
    auto works = [&](int b) -> bool {
      const T nblk = (T)(pref[b + 1] - pref[b]) - fc, s = (T)pref[b] + fs;
      if (nblk > 0) return s < u1 && s + nblk > u0;
      return u0 <= (T)pref[b] && (T)pref[b] < u1;
    };
    int b0 = -1, b1 = -1;
    if (u0 < u1) {
      const int b = upper_index(pref, B, u0);
      b0 = works(b) ? b : (b + 1 < B && works(b + 1) ? b + 1 : -1);
      if (b0 >= 0) {
        const int e = upper_index(pref, B, u1 - 1);
        b1 = works(e) ? e : e - 1;
      }
    }
    row[5] = (int32_t)W;
    row[6] = fixed_cost;
    if (b0 < 0) {
      row[0] = -1; row[1] = 0; row[2] = -1; row[3] = 0; row[4] = 0; row[7] = 0;
      continue;
    }
    const T n0 = (T)(pref[b0 + 1] - pref[b0]) - fc, s0 = (T)pref[b0] + fs;
    const T n1 = (T)(pref[b1 + 1] - pref[b1]) - fc, s1 = (T)pref[b1] + fs;
    T k0 = 0;
    if (n0 > 0) k0 = total >= P ? p - part_of(s0) : max(u0, s0) - s0;
    row[0] = b0;
    row[1] = n0 > 0 ? (int32_t)max((T)0, u0 - s0) : 0;
    row[2] = b1;
    row[3] = n1 > 0 ? (int32_t)min(n1, u1 - s1) : 0;
    row[4] = (int32_t)k0;
    row[7] = b1 - b0 + 1;
  }
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
  // The closed forms multiply a unit index by num_parts: 32-bit arithmetic
  // when that product stays below 2^31 (the common case), else 64-bit.
  if ((pref[B] + 1) * (long long)num_parts < (1LL << 31))
    fill_rows<int>(B, num_parts, fixed_cost, tile_md, num_splits, pref, cnt, tmp);
  else
    fill_rows<long long>(B, num_parts, fixed_cost, tile_md, num_splits, pref, cnt, tmp);
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
