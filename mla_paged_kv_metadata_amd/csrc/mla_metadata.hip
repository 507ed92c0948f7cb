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

// One step of a wave-wide inclusive scan of a 64-bit value held as two
// dwords: add the value that the DPP control `ctrl` moves in (lanes without
// a source, or in rows outside row_mask, add 0).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void scan_step(unsigned &lo, unsigned &hi) {
  const unsigned ylo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, kCtrl, kRowMask, 0xf, false);
  const unsigned yhi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)hi, kCtrl, kRowMask, 0xf, false);
  const unsigned nlo = lo + ylo;
  hi = hi + yhi + (nlo < lo ? 1u : 0u);
  lo = nlo;
}
// Inclusive scan over the 64 lanes of a wave: shifts by 1, 2, 4 and 8 lanes
// within each row of 16 (row_shr), then the last lane of row 0 / row 2 added
// to rows 1 / 3 (row_bcast:15) and lane 31 added to rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ long long wave_inclusive_scan(long long v) {
  unsigned lo = (unsigned)(unsigned long long)v, hi = (unsigned)((unsigned long long)v >> 32);
  scan_step<0x111, 0xf>(lo, hi);
  scan_step<0x112, 0xf>(lo, hi);
  scan_step<0x114, 0xf>(lo, hi);
  scan_step<0x118, 0xf>(lo, hi);
  scan_step<0x142, 0xa>(lo, hi);
  scan_step<0x143, 0xc>(lo, hi);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Exclusive scan over `n` int64 values held in smem[0..n), in place; smem[n] = total.
// Each thread scans a contiguous chunk; chunk sums are scanned within each
// wave (wave_inclusive_scan), and every thread adds the totals of the waves
// before its own (held in `tmp`).
__device__ void block_exclusive_scan(long long *smem, int n, long long *tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + kT - 1) / kT;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  long long s = 0;
  for (int i = lo; i < hi; ++i) s += smem[i];
  const long long incl = wave_inclusive_scan(s);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  long long before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kT / 64; ++w) {
    const long long t = tmp[w];
    before += w < wave ? t : 0;
    total += t;
  }
  long long run = before + incl - s;
  for (int i = lo; i < hi; ++i) {
    const long long x = smem[i];
    smem[i] = run;
    run += x;
  }
  if (tid == 0) smem[n] = total;
  __syncthreads();                                 // (also: tmp is free again)
}

// Largest b in [0, n] with pref[b] <= x, for two keys at once: binary
// lifting from b = 0 (pref[0] = 0 <= x) with steps 2^k .. 1, 2^(k+1) > n, the
// same number of steps in every lane and the two searches' LDS reads side by
// side.  pref is strictly increasing because every cost is >= 1.
__device__ __forceinline__ void upper_index2(const long long *pref, int n, long long x1, long long x2, int &r1,
                                             int &r2) {
  int p1 = 0, p2 = 0;
  for (int step = 1 << (31 - __builtin_clz((unsigned)n)); step > 0; step >>= 1) {
    const long long v1 = pref[min(p1 + step, n)], v2 = pref[min(p2 + step, n)];
    if (p1 + step <= n && v1 <= x1) p1 += step;
    if (p2 + step <= n && v2 <= x2) p2 += step;
  }
  r1 = p1;
  r2 = p2;
}

// Division of values in [0, 2^32) by a divisor d >= 1 that every lane shares:
// with m = floor((2^32 - 1) / d), mulhi(n, m) is floor(n / d) or at most 2
// below it, and two corrections finish it.
struct FastDiv {
  unsigned d, m;
  __device__ explicit FastDiv(unsigned dd) : d(dd), m(0xffffffffu / dd) {}
  __device__ __forceinline__ unsigned operator()(unsigned n) const {
    unsigned q = __umulhi(n, m);
    unsigned r = n - q * d;
    if (r >= d) {
      ++q;
      r -= d;
    }
    if (r >= d) ++q;
    return q;
  }
};

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
  // 32-bit instance: every product below stays under 2^31 (checked by the
  // caller), so the divisions by P and by total use FastDiv.
  [[maybe_unused]] const FastDiv div_p(sizeof(T) == 4 ? (unsigned)P : 1u), div_t(sizeof(T) == 4 ? (unsigned)total : 1u);
  auto bound = [&](T p) -> T {
    if constexpr (sizeof(T) == 4) return (T)div_p((unsigned)(p * total));
    else return p * total / P;
  };
  auto part_of = [&](T u) -> T {                             // u < total
    if constexpr (sizeof(T) == 4) return (T)div_t((unsigned)((u + 1) * P - 1));
    else return ((u + 1) * P - 1) / total;
  };

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
      int b, e;
      upper_index2(pref, B, u0, u1 - 1, b, e);
      b0 = works(b) ? b : (b + 1 < B && works(b + 1) ? b + 1 : -1);
      if (b0 >= 0) b1 = works(e) ? e : e - 1;
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
