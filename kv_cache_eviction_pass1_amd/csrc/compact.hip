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
// where it needs it, in two dependent rounds:
//   - its kT threads read kT evenly spaced list entries; counting those below
//     the block's first token t0 and below its end t1 brackets the two list
//     positions lo = #{e < t0} and hi = #{e < t1} within one sample spacing
//     each (sample i sits at position i * n_evict / kT);
//   - the threads read the bracketed list range [A, B) once: the entries below
//     t0 complete lo, those inside the block become a bitmap in LDS;
//   - the kept tokens are ranked by a workgroup scan and land at output row
//     (t0 - lo) + rank; the copy runs over (row, 16-byte unit) pairs,
//     consecutive threads on consecutive units, K's and V's unit loaded
//     together so that both streams are in flight.
// Every workgroup also checks an equal share of the list (strictly increasing,
// inside [0, n)); a bad list sets the status bit, and no read or write leaves
// the list or the output arrays whatever the list holds.
#include "dropkv_common.h"

namespace dropkv {

namespace {

constexpr int kT = 512;    // threads per workgroup
constexpr int kCT = 4096;  // tokens per workgroup
constexpr int kPerT = kCT / kT;
constexpr int kBatch = 8;  // copy units in flight per thread and tensor
static_assert(kCT % kT == 0 && kCT % 32 == 0 && kPerT <= 32 && 32 % kPerT == 0, "token blocking");

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

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// list position of sample i (i <= kT; sample kT stands for the end of the list)
__device__ __forceinline__ int64_t sample_pos(int64_t ne, int i) { return (int64_t)i * ne / kT; }

template <typename U>
__global__ __launch_bounds__(kT) void k_compact(CompactArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)b * kCT;
  const int64_t t1 = (t0 + kCT < A.n) ? t0 + kCT : A.n;
  const int64_t ne = A.n_evict;
  const int64_t* e = A.e + (size_t)g * ne;
  __shared__ uint32_t bits[kCT / 32];
  __shared__ uint16_t rows[kCT];
  __shared__ uint32_t wsum[kT / 64];
  __shared__ uint32_t cnt[3];  // samples below t0, samples below t1, bracketed entries below t0
  __shared__ int bad;
  if (threadIdx.x < kCT / 32) bits[threadIdx.x] = 0u;
  if (threadIdx.x < 3) cnt[threadIdx.x] = 0u;
  if (threadIdx.x == 0) bad = 0;
  // first load round: one list sample per thread, and this workgroup's share of the
  // list check (all shares cover every adjacent pair once)
  int64_t sv = INT64_MAX;
  if (ne > 0) sv = e[sample_pos(ne, threadIdx.x)];
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
  {
    const uint32_t c0 = __popcll(__builtin_amdgcn_ballot_w64(sv < t0));
    const uint32_t c1 = __popcll(__builtin_amdgcn_ballot_w64(sv < t1));
    if (lane == 0) {
      if (c0) atomicAdd(&cnt[0], c0);
      if (c1) atomicAdd(&cnt[1], c1);
    }
  }
  __syncthreads();
  // lo lies in [A0, pos(c0)], hi in [pos(c1 - 1) + 1, pos(c1)]: read [A0, B0)
  const int c0 = (int)cnt[0], c1 = (int)cnt[1];
  const int64_t A0 = c0 > 0 ? sample_pos(ne, c0 - 1) + 1 : 0;
  const int64_t B0 = sample_pos(ne, c1);
  uint32_t below = 0;
  for (int64_t i = A0 + threadIdx.x; i < B0; i += kT) {
    const int64_t x = e[i];
    if (x < t0) {
      ++below;
    } else if (x < t1) {
      const int64_t r = x - t0;
      atomicOr(&bits[r >> 5], 1u << (r & 31));
    }
  }
  {
    // wave sum of `below` (a few entries per thread at most)
    uint32_t wv = wave_incl_scan(below);
    wv = (uint32_t)__builtin_amdgcn_readlane((int)wv, 63);
    if (lane == 0 && wv) atomicAdd(&cnt[2], wv);
  }
  __syncthreads();
  // kept tokens of this block, ranked: thread t owns tokens kPerT*t .. +kPerT-1
  const int tok0 = kPerT * threadIdx.x;
  const uint32_t word = bits[tok0 >> 5] >> (tok0 & 31);
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < kPerT; ++j)
    if (t0 + tok0 + j < t1 && !((word >> j) & 1u)) keep |= 1u << j;
  const uint32_t nk = __popc(keep);
  const uint32_t incl = wave_incl_scan(nk);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = incl - nk, total = 0;
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
  // kept tokens before this block: t0 - lo, lo = A0 + bracketed entries below t0
  const int64_t lo = A0 + (int64_t)cnt[2];
  const int64_t base = t0 - lo;
  // (row, unit) pairs of this block: at most kCT * 4096 * 4 / 2 < 2^31
  const uint32_t upr = (uint32_t)A.upr;
  const uint32_t units = total * upr;
  const char* ks = A.k + ((size_t)g * A.n + t0) * A.row_bytes;
  const char* vs = A.v + ((size_t)g * A.n + t0) * A.row_bytes;
  char* kd = A.ok + (size_t)g * A.n_keep * A.row_bytes;
  char* vd = A.ov + (size_t)g * A.n_keep * A.row_bytes;
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
        const int64_t so = (int64_t)rows[r] * A.row_bytes + (int64_t)c * (int64_t)sizeof(U);
        bk[u] = *(const U*)(ks + so);
        bv[u] = *(const U*)(vs + so);
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
      if (dst[u] >= 0) {
        *(U*)(kd + dst[u]) = bk[u];
        *(U*)(vd + dst[u]) = bv[u];
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
