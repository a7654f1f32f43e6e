// Cache compaction: the rows of K and V that the eviction list does not name,
// gathered per KV head into a compact cache in ascending token order.
//
// DropKV write-up, section 代码映射与边界 (code map and limits): the scorer's
// output is the per-head list of tokens to drop, to be applied to the cache by
// the caller; this is that application, for the layout the scorer reads
// (K, V [Hkv][n][d]). Kept token j of head g lands in row
// j - #{evicted indices < j} of the head's output.
//
// One workgroup per (block of kR output rows, KV head), so that every
// workgroup copies the same number of rows whatever the pattern of the list.
// With f(i) = e[i] - i (the number of kept tokens below the i-th evicted
// one, non-decreasing along a valid list), output row r holds token
// r + I(r), I(r) = #{i : f(i) <= r}. A workgroup finds I for its rows
// [r0, r1) in two dependent rounds of list reads:
//   - its threads read kS evenly spaced list entries (sample k at position
//     k * n_evict / kS); the samples with f <= r0 and f <= r1 - 1 bracket
//     I(r0) from below and I(r1 - 1) from above: I(r) = lo + #{i in [lo, hi):
//     f(i) <= r} for every row of the block;
//   - f over [lo, hi) goes to LDS (up to kCap entries), and each row's count
//     is a binary search there; a longer range (a long evicted run inside the
//     block's span) is searched in global memory instead.
// The copy then runs over (row, 16-byte unit) pairs, consecutive threads on
// consecutive units, K's and V's unit loaded together so that both streams
// are in flight, and stored with non-temporal stores. (A kept list, which
// the select stage can emit, makes the source rows plain list entries:
// k_compact_kept needs one round of list reads before the copy.) Every
// workgroup also checks an equal share of the list
// (strictly increasing, inside [0, n)); a bad list sets the status bit, and no
// read or write leaves the list or the output arrays whatever the list holds.
#include "dropkv_common.h"

namespace dropkv {

namespace {

constexpr int kT = 256;     // threads per workgroup
constexpr int kR = 128;     // output rows per workgroup
constexpr int kS = 512;     // list samples per workgroup
constexpr int kCap = 4096;  // list entries staged in LDS
constexpr int kBatch = 8;   // copy units in flight per thread and tensor
// 16-byte unit as a native vector (HIP's uint4 struct in the unit arrays went
// to scratch memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
static_assert(kS % kT == 0 && kCap % kT == 0 && kR <= kT, "blocking");

struct CompactArgs {
  const char* k;
  const char* v;
  char* ok;
  char* ov;
  const int64_t* e;  // [Hkv][n_evict]
  int64_t n, n_evict, n_keep;
  int64_t row_bytes;
  int32_t upr;       // copy units per row
  int32_t nblk;      // row blocks per head
  int32_t* status;
};

// list position of sample i (i <= kS; sample kS stands for the end of the list)
__device__ __forceinline__ int64_t sample_pos(int64_t ne, int i) { return (int64_t)i * ne / kS; }

// f(i) = e[i] - i, with the entry clamped to [0, n) so that a bad list still
// gives bounded values (the list check reports it)
__device__ __forceinline__ int64_t fval(const int64_t* e, int64_t i, int64_t n) {
  int64_t x = e[i];
  x = x < 0 ? 0 : (x >= n ? n - 1 : x);
  return x - i;
}

// Copies the block's output rows [r0, r1) of head g from the token rows
// src[0 .. r1 - r0) (in LDS) of K and V.
template <typename U>
__device__ __forceinline__ void copy_rows(const CompactArgs& A, const int32_t* src, int g, int64_t r0,
                                          int64_t r1) {
  // (row, unit) pairs of this block: at most kR * 4096 * 4 / 2 units
  const uint32_t upr = (uint32_t)A.upr;
  const uint32_t units = (uint32_t)(r1 > r0 ? r1 - r0 : 0) * upr;
  const char* ks = A.k + (size_t)g * A.n * A.row_bytes;
  const char* vs = A.v + (size_t)g * A.n * A.row_bytes;
  char* kd = A.ok + ((size_t)g * A.n_keep + r0) * A.row_bytes;
  char* vd = A.ov + ((size_t)g * A.n_keep + r0) * A.row_bytes;
  // unit i = r * upr + c; each thread walks i = threadIdx.x + m * kT, stepping
  // (r, c) by (kT / upr, kT % upr) with a carry instead of dividing
  const uint32_t dr = (uint32_t)kT / upr, dc = (uint32_t)kT % upr;
  uint32_t r = threadIdx.x / upr, c = threadIdx.x % upr;
  for (uint32_t i0 = threadIdx.x; i0 < units; i0 += (uint32_t)kT * kBatch) {
    U bk[kBatch], bv[kBatch];
    int64_t dst[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      dst[u] = -1;
      if (i0 + (uint32_t)u * kT < units) {
        const int64_t so = (int64_t)src[r] * A.row_bytes + (int64_t)c * (int64_t)sizeof(U);
        bk[u] = *(const U*)(ks + so);
        bv[u] = *(const U*)(vs + so);
        dst[u] = (int64_t)r * A.row_bytes + (int64_t)c * (int64_t)sizeof(U);
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
      if (dst[u] >= 0) {
        // written once, read by a later call: no need to keep them in the L2
        __builtin_nontemporal_store(bk[u], (U*)(kd + dst[u]));
        __builtin_nontemporal_store(bv[u], (U*)(vd + dst[u]));
      }
  }
}

template <typename U>
__global__ __launch_bounds__(kT) void k_compact(CompactArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t ne = A.n_evict;
  const int64_t* e = A.e + (size_t)g * ne;
  const int64_t r0 = (int64_t)b * kR;
  const int64_t r1 = (r0 + kR < A.n_keep) ? r0 + kR : A.n_keep;
  __shared__ int32_t fs[kCap];
  __shared__ int32_t src[kR];
  __shared__ uint32_t cnt[2];  // samples with f <= r0, with f <= r1 - 1
  __shared__ int bad;
  if (threadIdx.x < 2) cnt[threadIdx.x] = 0u;
  if (threadIdx.x == 0) bad = 0;
  // first load round: kS / kT samples per thread, and this workgroup's share
  // of the list check (all shares cover every adjacent pair once)
  int64_t sf[kS / kT];
#pragma unroll
  for (int u = 0; u < kS / kT; ++u) sf[u] = ne > 0 ? fval(e, sample_pos(ne, threadIdx.x + u * kT), A.n) : 0;
  {
    const int64_t per = (ne + A.nblk - 1) / A.nblk;
    const int64_t i0 = (int64_t)b * per;
    const int64_t i1 = (i0 + per < ne) ? i0 + per : ne;
    bool badl = false;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += kT) {
      const int64_t x = e[i];
      if (x < 0 || x >= A.n || (i > 0 && e[i - 1] >= x)) badl = true;
    }
    if (badl) bad = 1;
  }
  __syncthreads();
  if (ne > 0 && r1 > r0) {
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int u = 0; u < kS / kT; ++u) {
      c0 += __popcll(__builtin_amdgcn_ballot_w64(sf[u] <= r0));
      c1 += __popcll(__builtin_amdgcn_ballot_w64(sf[u] <= r1 - 1));
    }
    if (lane == 0) {
      if (c0) atomicAdd(&cnt[0], c0);
      if (c1) atomicAdd(&cnt[1], c1);
    }
  }
  __syncthreads();
  int64_t lo = 0, hi = 0;
  if (ne > 0 && r1 > r0) {
    const int c0 = (int)cnt[0], c1 = (int)cnt[1];
    lo = c0 > 0 ? sample_pos(ne, c0 - 1) + 1 : 0;
    hi = c1 < kS ? sample_pos(ne, c1) : ne;
    if (hi < lo) hi = lo;  // only for a bad list
  }
  const int64_t m = hi - lo;
  const bool staged = m <= kCap;  // same for every thread
  if (staged) {
    // second load round: f over [lo, hi) into LDS
    int32_t fv[kCap / kT];
#pragma unroll
    for (int u = 0; u < kCap / kT; ++u) {
      const int64_t j = threadIdx.x + u * kT;
      fv[u] = j < m ? (int32_t)fval(e, lo + j, A.n) : 0;
    }
#pragma unroll
    for (int u = 0; u < kCap / kT; ++u) fs[threadIdx.x + u * kT] = fv[u];
  }
  __syncthreads();
  if ((int64_t)threadIdx.x < r1 - r0) {
    const int64_t r = r0 + threadIdx.x;
    // #{j in [0, m): f(lo + j) <= r}: upper bound in a non-decreasing run
    int64_t a = 0, z = m;
    if (staged) {
      while (a < z) {
        const int64_t mid = (a + z) >> 1;
        if ((int64_t)fs[mid] <= r) a = mid + 1; else z = mid;
      }
    } else {
      while (a < z) {
        const int64_t mid = (a + z) >> 1;
        if (fval(e, lo + mid, A.n) <= r) a = mid + 1; else z = mid;
      }
    }
    int64_t t = r + lo + a;
    DKV_CHECK(t >= 0 && t < A.n, A.status);
    t = t < 0 ? 0 : (t >= A.n ? A.n - 1 : t);  // a bad list only
    src[threadIdx.x] = (int32_t)t;
  }
  __syncthreads();
  copy_rows<U>(A, src, g, r0, r1);
  if (threadIdx.x == 0 && bad) atomicOr(A.status, kStatusBadIndex);
}


// From a kept list: output row r0 + i of head g is token keep[g][r0 + i].
// Each thread checks its entry against the one before it (strictly
// increasing inside [0, n)); a bad entry sets the status bit and is clamped,
// so no read leaves the K/V arrays whatever the list holds.
template <typename U>
__global__ __launch_bounds__(kT) void k_compact_kept(CompactArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int64_t r0 = (int64_t)b * kR;
  const int64_t r1 = (r0 + kR < A.n_keep) ? r0 + kR : A.n_keep;
  const int64_t* kl = A.e + (size_t)g * A.n_keep;
  __shared__ int32_t src[kR];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  if ((int64_t)threadIdx.x < r1 - r0) {
    const int64_t r = r0 + threadIdx.x;
    int64_t t = kl[r];
    const int64_t prev = r > 0 ? kl[r - 1] : -1;
    if (t < 0 || t >= A.n || t <= prev) bad = 1;
    t = t < 0 ? 0 : (t >= A.n ? A.n - 1 : t);
    src[threadIdx.x] = (int32_t)t;
  }
  __syncthreads();
  copy_rows<U>(A, src, g, r0, r1);
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
  // at least one block per head: a head with nothing kept still checks its list
  const int64_t nb = (A.n_keep + kR - 1) / kR;
  A.nblk = (int32_t)(nb > 0 ? nb : 1);
  A.status = status;
  auto aligned = [&](size_t a) {
    return A.row_bytes % (int64_t)a == 0 && (uintptr_t)k % a == 0 && (uintptr_t)v % a == 0 &&
           (uintptr_t)out_k % a == 0 && (uintptr_t)out_v % a == 0;
  };
  const dim3 grid(A.nblk, Hkv);
  if (aligned(16)) {
    A.upr = (int32_t)(A.row_bytes / 16);
    k_compact<u32x4><<<grid, kT, 0, st>>>(A);
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

namespace dropkv {

hipError_t launch_compact_kept(int dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                               const int64_t* keep_idx, int64_t n_keep, void* out_k, void* out_v,
                               int32_t* status, hipStream_t st) {
  if (n_keep <= 0) return hipSuccess;
  CompactArgs A{};
  A.k = (const char*)k;
  A.v = (const char*)v;
  A.ok = (char*)out_k;
  A.ov = (char*)out_v;
  A.e = keep_idx;
  A.n = n;
  A.n_evict = n - n_keep;
  A.n_keep = n_keep;
  A.row_bytes = (int64_t)d * (dtype == 0 ? 2 : 4);
  A.nblk = (int32_t)((n_keep + kR - 1) / kR);
  A.status = status;
  auto aligned = [&](size_t a) {
    return A.row_bytes % (int64_t)a == 0 && (uintptr_t)k % a == 0 && (uintptr_t)v % a == 0 &&
           (uintptr_t)out_k % a == 0 && (uintptr_t)out_v % a == 0;
  };
  const dim3 grid(A.nblk, Hkv);
  if (aligned(16)) {
    A.upr = (int32_t)(A.row_bytes / 16);
    k_compact_kept<u32x4><<<grid, kT, 0, st>>>(A);
  } else if (aligned(4)) {
    A.upr = (int32_t)(A.row_bytes / 4);
    k_compact_kept<uint32_t><<<grid, kT, 0, st>>>(A);
  } else {
    A.upr = (int32_t)(A.row_bytes / 2);
    k_compact_kept<uint16_t><<<grid, kT, 0, st>>>(A);
  }
  return hipGetLastError();
}

}  // namespace dropkv
