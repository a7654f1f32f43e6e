// Cache compaction: the rows of K and V that the eviction list does not name,
// gathered per KV head into a compact cache in ascending token order.
//
// DropKV write-up, section 代码映射与边界 (code map and limits): the scorer's
// output is the per-head list of tokens to drop, to be applied to the cache by
// the caller; this is that application, for the layout the scorer reads
// (K, V [Hkv][n][d]). Kept token j of head g lands in row
// j - #{evicted indices < j} of the head's output.
//
// One workgroup per (block of kCT tokens, KV head), reading the list only
// where it needs it:
//   - two waves find the list range [lo, hi) of the block's tokens with
//     64-way searches (three or four rounds of 64 probes for 10^5 entries);
//   - the block's evicted tokens become a bitmap in LDS, the kept tokens are
//     ranked by a workgroup scan, and the block's rows land at output row
//     (block start - lo) + rank;
//   - the copy runs over (row, 16-byte unit) pairs, consecutive threads on
//     consecutive units, so reads of a row and writes of the output are
//     coalesced; K's rows first, then V's.
// Every workgroup also checks an equal share of the list (strictly increasing,
// inside [0, n)); a bad list sets the status bit, and no write can leave the
// output arrays whatever the list holds.
#include "dropkv_common.h"

namespace dropkv {

namespace {

constexpr int kT = 256;    // threads per workgroup
constexpr int kCT = 1024;  // tokens per workgroup
constexpr int kPerT = kCT / kT;
constexpr int kBatch = 16;  // copy units in flight per thread
static_assert(kCT % kT == 0 && kCT % 32 == 0 && kPerT <= 32, "token blocking");

struct CompactArgs {
  const char* k;
  const char* v;
  char* ok;
  char* ov;
  const int64_t* e;  // [Hkv][n_evict]
  int64_t n, n_evict, n_keep;
  int64_t row_bytes;
  int32_t upr;       // copy units per row
  int32_t nblk;      // token blocks per head
  int32_t* status;
};

// Lowest i in [0, len) with e[i] >= x (len if none) for a strictly increasing
// list: each round the 64 lanes of the calling wave probe 64 evenly spaced
// entries and keep the one gap where the comparison flips. For any list it
// returns some index in [0, len] after at most ~log_64(len) + 2 rounds.
__device__ int64_t lower_bound_wave(const int64_t* e, int64_t len, int64_t x) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, hi = len;  // the answer lies in [lo, hi]
  while (lo < hi) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t p = lo + (int64_t)lane * step;
    const bool less = p < hi && e[p] < x;
    const int c = __popcll(__builtin_amdgcn_ballot_w64(less));
    if (c == 0) {
      hi = lo;  // e[lo] >= x
    } else {
      const int64_t nhi = lo + (int64_t)c * step;
      lo = lo + (int64_t)(c - 1) * step + 1;
      hi = nhi < hi ? nhi : hi;
    }
  }
  return lo;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

template <typename U>
__global__ __launch_bounds__(kT) void k_compact(CompactArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)b * kCT;
  const int64_t t1 = (t0 + kCT < A.n) ? t0 + kCT : A.n;
  const int64_t* e = A.e + (size_t)g * A.n_evict;
  __shared__ uint32_t bits[kCT / 32];
  __shared__ uint16_t rows[kCT];
  __shared__ int64_t sh_lo, sh_hi;
  __shared__ uint32_t wsum[kT / 64];
  __shared__ int bad;
  if (threadIdx.x < kCT / 32) bits[threadIdx.x] = 0u;
  if (threadIdx.x == 0) bad = 0;
  // the two ends of the block's list range, searched by two waves at once
  if (wave == 0) {
    const int64_t lo = lower_bound_wave(e, A.n_evict, t0);
    if (lane == 0) sh_lo = lo;
  } else if (wave == 1) {
    const int64_t hi = lower_bound_wave(e, A.n_evict, t1);
    if (lane == 0) sh_hi = hi;
  }
  {
    // this workgroup's share of the list check (all shares cover every pair once)
    const int64_t per = (A.n_evict + A.nblk - 1) / A.nblk;
    const int64_t i0 = (int64_t)b * per;
    const int64_t i1 = (i0 + per < A.n_evict) ? i0 + per : A.n_evict;
    bool badl = false;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += kT) {
      const int64_t x = e[i];
      if (x < 0 || x >= A.n || (i > 0 && e[i - 1] >= x)) badl = true;
    }
    if (badl) bad = 1;
  }
  __syncthreads();
  const int64_t lo = sh_lo, hi = sh_hi > sh_lo ? sh_hi : sh_lo;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kT) {
    const int64_t x = e[i] - t0;
    if (x >= 0 && x < t1 - t0) atomicOr(&bits[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  // kept tokens of this block, ranked: thread t owns tokens kPerT*t .. +kPerT-1
  const int tok0 = kPerT * threadIdx.x;
  const uint32_t word = bits[tok0 >> 5] >> (tok0 & 31);
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < kPerT; ++j)
    if (t0 + tok0 + j < t1 && !((word >> j) & 1u)) keep |= 1u << j;
  const uint32_t cnt = __popc(keep);
  const uint32_t incl = wave_incl_scan(cnt);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < kT / 64; ++w) {
    const uint32_t s = wsum[w];
    before += w < wave ? s : 0u;
    total += s;
  }
#pragma unroll
  for (int j = 0; j < kPerT; ++j)
    if ((keep >> j) & 1u) rows[before++] = (uint16_t)(tok0 + j);
  __syncthreads();
  // kept tokens before this block: t0 - lo (exact for a valid list)
  const int64_t base = t0 - lo;
  // (row, unit) pairs of this block: at most kCT * 4096 * 4 / 2 < 2^31
  const uint32_t upr = (uint32_t)A.upr;
  const uint32_t units = total * upr;
  const char* ks = A.k + ((size_t)g * A.n + t0) * A.row_bytes;
  const char* vs = A.v + ((size_t)g * A.n + t0) * A.row_bytes;
  char* kd = A.ok + (size_t)g * A.n_keep * A.row_bytes;
  char* vd = A.ov + (size_t)g * A.n_keep * A.row_bytes;
  // unit i = r * upr + c; each thread walks i = threadIdx.x + m * kT, stepping
  // (r, c) by (kT / upr, kT % upr) with a carry instead of dividing. K first,
  // then V: two memory streams at a time instead of four.
  const uint32_t dr = (uint32_t)kT / upr, dc = (uint32_t)kT % upr;
  for (int tsr = 0; tsr < 2; ++tsr) {
    const char* src = tsr ? vs : ks;
    char* dstb = tsr ? vd : kd;
    uint32_t r = threadIdx.x / upr, c = threadIdx.x % upr;
    for (uint32_t i0 = threadIdx.x; i0 < units; i0 += (uint32_t)kT * kBatch) {
      U bk[kBatch];
      int64_t dst[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        dst[u] = -1;
        if (i0 + (uint32_t)u * kT < units) {
          const int64_t so = (int64_t)rows[r] * A.row_bytes + (int64_t)c * (int64_t)sizeof(U);
          bk[u] = *(const U*)(src + so);
          const int64_t orow = base + r;
          DKV_CHECK(rows[r] < (uint16_t)kCT && t0 + rows[r] < A.n, A.status);
          if (orow >= 0 && orow < A.n_keep) dst[u] = orow * A.row_bytes + (int64_t)c * (int64_t)sizeof(U);
        }
        r += dr;
        c += dc;
        if (c >= upr) {
          c -= upr;
          ++r;
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (dst[u] >= 0) *(U*)(dstb + dst[u]) = bk[u];
    }
  }
  if (threadIdx.x == 0 && bad) atomicOr(A.status, kStatusBadIndex);
}

}  // namespace

hipError_t launch_compact(int dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                          const int64_t* evict_idx, int64_t n_evict, void* out_k, void* out_v,
                          int32_t* status, hipStream_t st) {
  CompactArgs A{};
  A.k = (const char*)k;
  A.v = (const char*)v;
  A.ok = (char*)out_k;
  A.ov = (char*)out_v;
  A.e = evict_idx;
  A.n = n;
  A.n_evict = n_evict;
  A.n_keep = n - n_evict;
  A.row_bytes = (int64_t)d * (dtype == 0 ? 2 : 4);
  A.nblk = (int32_t)((n + kCT - 1) / kCT);
  A.status = status;
  auto aligned = [&](size_t a) {
    return A.row_bytes % (int64_t)a == 0 && (uintptr_t)k % a == 0 && (uintptr_t)v % a == 0 &&
           (uintptr_t)out_k % a == 0 && (uintptr_t)out_v % a == 0;
  };
  const dim3 grid(A.nblk, Hkv);
  if (aligned(16)) {
    A.upr = (int32_t)(A.row_bytes / 16);
    k_compact<uint4><<<grid, kT, 0, st>>>(A);
  } else if (aligned(4)) {
    A.upr = (int32_t)(A.row_bytes / 4);
    k_compact<uint32_t><<<grid, kT, 0, st>>>(A);
  } else {
    A.upr = (int32_t)(A.row_bytes / 2);
    k_compact<uint16_t><<<grid, kT, 0, st>>>(A);
  }
  return hipGetLastError();
}

}  // namespace dropkv
