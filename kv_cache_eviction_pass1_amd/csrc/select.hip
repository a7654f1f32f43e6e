// Pooling, recent-window protection and bottom-k eviction per KV head.
//
// DropKV write-up, section 核心公式, prose after the equation ("Algorithm 1"):
// max-pool the scores, set the last observation window to +inf, evict the
// smallest. Readings: MaxPool1D with odd kernel, stride 1 and the window
// clipped to [0, n); the order among equal scores is the token index (lower
// evicted first); evicted indices are written in ascending order.
//
// Scores are non-negative, so the IEEE-754 bit pattern of a pooled score,
// read as uint32, orders exactly like its value (+inf = 0x7f800000 sorts
// last). The k-th smallest key is found by a 4-round radix select (8 bits per
// round, 256-bin histograms in LDS); then one ordered sweep writes every index
// whose key is below it plus the lowest-index ones equal to it.
#include "dropkv_common.h"

namespace dropkv {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? 0u : b;  // -0 (and any negative) sorts as +0
}

// Exclusive prefix sum over the block; returns this thread's prefix and the block total.
__device__ __forceinline__ int block_exclusive_scan(int x, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  if (wid == 0) {
    int s = lane < kWaves ? wsum[lane] : 0;
    int incl = s;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane < kWaves) wsum[kWaves + lane] = incl - s;  // exclusive wave offsets
    if (lane == kWaves - 1) wsum[2 * kWaves] = incl;
  }
  __syncthreads();
  const int res = wsum[kWaves + wid] + v - x;
  total = wsum[2 * kWaves];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kSelThreads) void k_select(
    const float* __restrict__ S, int64_t n, int w, int pool_kernel, int64_t n_evict,
    float* __restrict__ out_scores, int64_t* __restrict__ out_idx, int32_t* status) {
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const float* Sg = S + (size_t)g * n;
  float* Pg = out_scores + (size_t)g * n;
  const int half = pool_kernel / 2;
  const int64_t protect_from = n - w;

  __shared__ uint32_t hist[256];
  __shared__ int wsum[2 * kWaves + 1];
  __shared__ uint32_t sel_digit;
  __shared__ int64_t sel_rank;
  __shared__ int any_bad;

  if (tid == 0) any_bad = 0;
  __syncthreads();

  // 1. pool + protect
  bool bad = false;
  for (int64_t j = tid; j < n; j += kSelThreads) {
    const float sj = Sg[j];
    if (!finite_f(sj)) bad = true;
    const int64_t lo = j - half < 0 ? 0 : j - half;
    const int64_t hi = j + half >= n ? n - 1 : j + half;
    float mx = Sg[lo];
    for (int64_t t = lo + 1; t <= hi; ++t) mx = fmaxf(mx, Sg[t]);
    Pg[j] = (j >= protect_from) ? INFINITY : mx;
  }
  if (bad) any_bad = 1;
  __syncthreads();
  if (tid == 0 && any_bad) atomicOr(status, kStatusNonFinite);
  if (n_evict <= 0) return;
  __threadfence_block();
  __syncthreads();

  // 2. radix select of the n_evict-th smallest key (1-based rank)
  uint32_t prefix = 0, pmask = 0;
  int64_t rank = n_evict;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kSelThreads) hist[b] = 0;
    __syncthreads();
    for (int64_t j = tid; j < n; j += kSelThreads) {
      const uint32_t key = score_key(Pg[j]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4l..4l+3
      uint32_t c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2], c3 = hist[4 * tid + 3];
      int64_t loc = (int64_t)c0 + c1 + c2 + c3;
      int64_t incl = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int64_t y = __shfl_up(incl, o, 64);
        if (tid >= o) incl += y;
      }
      const int64_t excl = incl - loc;
      const unsigned long long hit = __ballot(incl >= rank);
      const int first = __ffsll((long long)hit) - 1;
      if (tid == first) {
        int64_t r = rank - excl;
        uint32_t dg = 4 * tid;
        const uint32_t cs[4] = {c0, c1, c2, c3};
        for (int b = 0; b < 4; ++b) {
          if (r <= (int64_t)cs[b]) { dg = 4 * tid + b; break; }
          r -= cs[b];
        }
        sel_digit = dg;
        sel_rank = r;
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    pmask |= 255u << shift;
    rank = sel_rank;
    __syncthreads();
  }
  const uint32_t tau = prefix;
  const int64_t need_eq = rank;  // how many keys equal to tau are evicted (lowest indices)

  // 3. ordered compaction
  int64_t out_pos = 0, eq_seen = 0;
  int64_t* og = out_idx + (size_t)g * n_evict;
  for (int64_t base = 0; base < n; base += kSelThreads) {
    const int64_t j = base + tid;
    uint32_t key = 0xffffffffu;
    if (j < n) key = score_key(Pg[j]);
    const int is_eq = (j < n && key == tau) ? 1 : 0;
    int eq_total;
    const int eq_before = block_exclusive_scan(is_eq, wsum, eq_total);
    const int take = (j < n) && (key < tau || (is_eq && eq_seen + eq_before < need_eq));
    int take_total;
    const int pos = block_exclusive_scan(take, wsum, take_total);
    if (take && out_pos + pos < n_evict) og[out_pos + pos] = j;
    out_pos += take_total;
    eq_seen += eq_total;
  }
}

__global__ void k_clear_status(int32_t* status) { *status = 0; }

}  // namespace

hipError_t launch_clear_status(int32_t* status, hipStream_t st) {
  k_clear_status<<<1, 1, 0, st>>>(status);
  return hipGetLastError();
}

hipError_t launch_select(const float* S, int64_t n, int32_t w, int32_t Hkv, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_idx, int32_t* status,
                         hipStream_t st) {
  k_select<<<Hkv, kSelThreads, 0, st>>>(S, n, w, pool_kernel, n_evict, out_scores, out_idx, status);
  return hipGetLastError();
}

}  // namespace dropkv
