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
// last). The n_evict-th smallest key tau is found by a radix select over
// many workgroups per head: digits of 12, 12 and 8 bits; each round builds
// LDS histograms, adds them into a global histogram, and the last workgroup
// to arrive picks the digit. Then every workgroup counts its keys below and
// equal to tau, the last one turns the counts into output offsets, and each
// workgroup writes its share of the indices in order.
#include "dropkv_common.h"

namespace dropkv {

namespace {

constexpr int kT = 256;           // threads per workgroup
constexpr int kPer = 16;          // consecutive elements per thread
constexpr int kChunk = kT * kPer; // elements per workgroup
constexpr int kMaxHalo = 512;     // pooling halo held in LDS (larger kernels read global memory)
constexpr int kBins1 = 4096, kBins2 = 4096, kBins3 = 256;

struct SelState {
  uint32_t prefix;
  uint32_t mask;
  int64_t rank;   // 1-based rank still to find among keys matching prefix/mask
  uint32_t tau;
  int64_t need;   // keys equal to tau that are evicted (lowest indices first)
  uint32_t arrive[4];
};

struct SelArgs {
  const float* S;
  float* P;        // out_scores
  int64_t* idx;    // out_evict_idx
  int64_t n, n_evict;
  int w, pool_half, nblk;
  uint32_t* hist;  // [Hkv][kBins1 + kBins2 + kBins3]
  SelState* st;    // [Hkv]
  int64_t* bc;     // [Hkv][nblk][4]: less, eq -> out offset, eq before
  int32_t* status;
};

__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? 0u : b;  // -0 (and any negative) sorts as +0
}

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int64_t ld_relaxed64(const int64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix sum over the workgroup (kT threads); also returns the total.
__device__ __forceinline__ int64_t wg_exclusive_scan(int64_t x, int64_t* wsum, int64_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int64_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  int64_t before = 0;
  for (int i = 0; i < wid; ++i) before += wsum[i];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + v - x;
}

// Returns true in every thread of the last workgroup of head g to finish `round`.
__device__ __forceinline__ bool last_to_arrive(SelState* st, int round, int nblk, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = atomicAdd(&st->arrive[round], 1u);
    *flag = (t == (uint32_t)nblk - 1) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

// Finds the bin holding rank `rank` (1-based) in a global histogram; updates st.
template <int PER>
__device__ void pick_digit(const uint32_t* h, int shift, uint32_t digit_mask, SelState* st,
                           int64_t rank, int64_t* wsum, uint32_t* sh_digit, int64_t* sh_rank) {
  uint32_t c[PER];
  int64_t loc = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = ld_relaxed(h + threadIdx.x * PER + i);
    loc += c[i];
  }
  int64_t total;
  const int64_t before = wg_exclusive_scan(loc, wsum, total);
  if (before < rank && rank <= before + loc) {
    int64_t r = rank - before;
    uint32_t dg = 0;
    int64_t rr = r;
    bool found = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!found && r <= (int64_t)c[i]) { dg = threadIdx.x * PER + i; rr = r; found = true; }
      if (!found) r -= c[i];
    }
    *sh_digit = dg;
    *sh_rank = rr;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    st->prefix |= (*sh_digit & digit_mask) << shift;
    st->mask |= digit_mask << shift;
    st->rank = *sh_rank;
  }
}

__device__ __forceinline__ void load_keys(const SelArgs& A, int g, int b, uint32_t (&key)[kPer]) {
  const int64_t j0 = (int64_t)b * kChunk + (int64_t)threadIdx.x * kPer;
  const float* Pg = A.P + (size_t)g * A.n;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int64_t j = j0 + e;
    key[e] = (j < A.n) ? score_key(Pg[j]) : 0xffffffffu;
  }
}

// Keys of a workgroup's range in strided order (element base + e*kT + tid):
// coalesced loads; histogram and counting rounds do not depend on the order.
__device__ __forceinline__ void load_keys_strided(const SelArgs& A, int g, int b, uint32_t (&key)[kPer]) {
  const int64_t base = (int64_t)b * kChunk + threadIdx.x;
  const float* Pg = A.P + (size_t)g * A.n;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int64_t j = base + (int64_t)e * kT;
    key[e] = (j < A.n) ? score_key(Pg[j]) : 0xffffffffu;
  }
}

// Round 1: pool + protect (writes out_scores) and the histogram of key bits 31..20.
__global__ __launch_bounds__(kT) void k_sel_pool(SelArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  __shared__ float sS[kChunk + 2 * kMaxHalo];
  __shared__ uint32_t hist[kBins1];
  __shared__ int64_t wsum[4];
  __shared__ int flag, bad;
  __shared__ uint32_t sh_digit;
  __shared__ int64_t sh_rank;
  const float* Sg = A.S + (size_t)g * A.n;
  float* Pg = A.P + (size_t)g * A.n;
  const int64_t base = (int64_t)b * kChunk;
  const int half = A.pool_half;
  const bool in_lds = half <= kMaxHalo;
  if (threadIdx.x == 0) bad = 0;
  for (int i = threadIdx.x; i < kBins1; i += kT) hist[i] = 0;
  if (in_lds) {
    for (int i = threadIdx.x; i < kChunk + 2 * half; i += kT) {
      const int64_t j = base - half + i;
      sS[i] = (j >= 0 && j < A.n) ? Sg[j] : 0.0f;  // S >= 0: zero padding = clipping
    }
  }
  __syncthreads();
  uint32_t key[kPer];
  bool nf = false;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int li = e * kT + threadIdx.x;  // consecutive threads, consecutive tokens
    const int64_t j = base + li;
    key[e] = 0xffffffffu;
    if (j < A.n) {
      float mx;
      if (in_lds) {
        const int c = li + half;
        mx = sS[c];
        if (!finite_f(mx)) nf = true;
        for (int t = c - half; t <= c + half; ++t) mx = fmaxf(mx, sS[t]);
      } else {
        mx = Sg[j];
        if (!finite_f(mx)) nf = true;
        const int64_t lo = j - half < 0 ? 0 : j - half;
        const int64_t hi = j + half >= A.n ? A.n - 1 : j + half;
        for (int64_t t = lo; t <= hi; ++t) mx = fmaxf(mx, Sg[t]);
      }
      const float p = (j >= A.n - A.w) ? INFINITY : mx;
      Pg[j] = p;
      key[e] = score_key(p);
    }
  }
  if (nf) bad = 1;
  if (A.n_evict > 0) {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (key[e] != 0xffffffffu) atomicAdd(&hist[key[e] >> 20], 1u);
  }
  __syncthreads();
  if (threadIdx.x == 0 && bad) atomicOr(A.status, kStatusNonFinite);
  if (A.n_evict <= 0) return;
  uint32_t* gh = A.hist + (size_t)g * (kBins1 + kBins2 + kBins3);
  for (int i = threadIdx.x; i < kBins1; i += kT)
    if (hist[i]) atomicAdd(gh + i, hist[i]);
  SelState* st = A.st + g;
  if (last_to_arrive(st, 0, A.nblk, &flag)) {
    if (threadIdx.x == 0) { st->prefix = 0; st->mask = 0; }
    pick_digit<kBins1 / kT>(gh, 20, 0xfffu, st, A.n_evict, wsum, &sh_digit, &sh_rank);
  }
}

// Rounds 2 and 3: histogram of the next digit among keys matching the prefix.
template <int ROUND>
__global__ __launch_bounds__(kT) void k_sel_refine(SelArgs A) {
  constexpr int BINS = ROUND == 1 ? kBins2 : kBins3;
  constexpr int SHIFT = ROUND == 1 ? 8 : 0;
  constexpr uint32_t DMASK = ROUND == 1 ? 0xfffu : 0xffu;
  const int b = blockIdx.x, g = blockIdx.y;
  __shared__ uint32_t hist[BINS];
  __shared__ int64_t wsum[4];
  __shared__ int flag;
  __shared__ uint32_t sh_digit;
  __shared__ int64_t sh_rank;
  SelState* st = A.st + g;
  const uint32_t prefix = ld_relaxed(&st->prefix), mask = ld_relaxed(&st->mask);
  const int64_t rank = ld_relaxed64(&st->rank);
  for (int i = threadIdx.x; i < BINS; i += kT) hist[i] = 0;
  __syncthreads();
  uint32_t key[kPer];
  load_keys_strided(A, g, b, key);
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (key[e] != 0xffffffffu && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> SHIFT) & DMASK], 1u);
  __syncthreads();
  uint32_t* gh = A.hist + (size_t)g * (kBins1 + kBins2 + kBins3) + (ROUND == 1 ? kBins1 : kBins1 + kBins2);
  for (int i = threadIdx.x; i < BINS; i += kT)
    if (hist[i]) atomicAdd(gh + i, hist[i]);
  if (last_to_arrive(st, ROUND, A.nblk, &flag)) {
    pick_digit<BINS / kT>(gh, SHIFT, DMASK, st, rank, wsum, &sh_digit, &sh_rank);
    if (ROUND == 2 && threadIdx.x == 0) {
      st->tau = st->prefix;
      st->need = st->rank;
    }
  }
}

// Counts keys below / equal to tau per workgroup; the last workgroup turns the
// counts into per-workgroup output offsets and "equal keys before" counts.
__global__ __launch_bounds__(kT) void k_sel_count(SelArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  __shared__ int64_t wsum[4];
  __shared__ int flag;
  SelState* st = A.st + g;
  const uint32_t tau = ld_relaxed(&st->tau);
  uint32_t key[kPer];
  load_keys_strided(A, g, b, key);
  int64_t less = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    less += (key[e] < tau) ? 1 : 0;
    eq += (key[e] == tau) ? 1 : 0;
  }
  int64_t tl, te;
  (void)wg_exclusive_scan(less, wsum, tl);
  (void)wg_exclusive_scan(eq, wsum, te);
  int64_t* bcg = A.bc + (size_t)g * A.nblk * 4;
  if (threadIdx.x == 0) { bcg[4 * b] = tl; bcg[4 * b + 1] = te; }
  if (last_to_arrive(st, 3, A.nblk, &flag)) {
    // per-workgroup output offsets: taken_i = less_i + clamp(need - eq_before_i, 0, eq_i)
    const int64_t need = ld_relaxed64(&st->need);
    int64_t out_carry = 0, eq_carry = 0;
    for (int i0 = 0; i0 < A.nblk; i0 += kT) {
      const int i = i0 + threadIdx.x;
      const int64_t l = i < A.nblk ? ld_relaxed64(bcg + 4 * i) : 0;
      const int64_t e = i < A.nblk ? ld_relaxed64(bcg + 4 * i + 1) : 0;
      int64_t etot;
      const int64_t eqb = eq_carry + wg_exclusive_scan(e, wsum, etot);
      int64_t take_eq = need - eqb;
      take_eq = take_eq < 0 ? 0 : (take_eq > e ? e : take_eq);
      int64_t ttot;
      const int64_t outb = out_carry + wg_exclusive_scan(l + take_eq, wsum, ttot);
      if (i < A.nblk) {
        bcg[4 * i + 2] = outb;
        bcg[4 * i + 3] = eqb;
      }
      out_carry += ttot;
      eq_carry += etot;
    }
  }
}

// Writes the evicted indices of each workgroup's range, in index order.
__global__ __launch_bounds__(kT) void k_sel_write(SelArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  __shared__ int64_t wsum[4];
  SelState* st = A.st + g;
  const uint32_t tau = ld_relaxed(&st->tau);
  const int64_t need = ld_relaxed64(&st->need);
  const int64_t* bcg = A.bc + (size_t)g * A.nblk * 4;
  const int64_t out0 = ld_relaxed64(bcg + 4 * b + 2), eq0 = ld_relaxed64(bcg + 4 * b + 3);
  uint32_t key[kPer];
  load_keys(A, g, b, key);
  int64_t eq = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) eq += (key[e] == tau) ? 1 : 0;
  int64_t tot;
  int64_t eq_before = eq0 + wg_exclusive_scan(eq, wsum, tot);
  bool take[kPer];
  int64_t nt = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    bool t = key[e] < tau;
    if (key[e] == tau) { t = eq_before < need; ++eq_before; }
    take[e] = t;
    nt += t ? 1 : 0;
  }
  int64_t pos = out0 + wg_exclusive_scan(nt, wsum, tot);
  int64_t* og = A.idx + (size_t)g * A.n_evict;
  const int64_t j0 = (int64_t)b * kChunk + (int64_t)threadIdx.x * kPer;
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (take[e]) {
      if (pos < A.n_evict) og[pos] = j0 + e;
      ++pos;
    }
}

// Zeroes the status word, the per-head flag counts and the select scratch
// (histograms and per-head selection state) in one launch.
__global__ void k_init(int32_t* status, int32_t* flagcount, uint32_t* hist, SelState* st, int Hkv) {
  const int g = blockIdx.x;
  uint32_t* h = hist + (size_t)g * (kBins1 + kBins2 + kBins3);
  for (int i = threadIdx.x; i < kBins1 + kBins2 + kBins3; i += blockDim.x) h[i] = 0;
  if (threadIdx.x == 0) {
    SelState z{};
    st[g] = z;
    if (flagcount) flagcount[g] = 0;
    if (g == 0) *status = 0;
  }
  (void)Hkv;
}

}  // namespace

size_t select_scratch_bytes(int64_t n, int32_t Hkv) {
  const int64_t nblk = (n + kChunk - 1) / kChunk;
  size_t b = sizeof(uint32_t) * (size_t)Hkv * (kBins1 + kBins2 + kBins3);
  b = (b + 255) / 256 * 256 + (sizeof(SelState) * (size_t)Hkv + 255) / 256 * 256;
  b += sizeof(int64_t) * 4 * (size_t)Hkv * nblk;
  return b + 256;
}

namespace {

struct SelPtrs {
  uint32_t* hist;
  SelState* st;
  int64_t* bc;
};

SelPtrs carve_sel(void* scratch, int32_t Hkv) {
  SelPtrs q;
  char* p = (char*)scratch;
  q.hist = (uint32_t*)p;
  p += (sizeof(uint32_t) * (size_t)Hkv * (kBins1 + kBins2 + kBins3) + 255) / 256 * 256;
  q.st = (SelState*)p;
  p += (sizeof(SelState) * (size_t)Hkv + 255) / 256 * 256;
  q.bc = (int64_t*)p;
  return q;
}

}  // namespace

hipError_t launch_init(int32_t* status, int32_t* flagcount, void* sel_scratch, int32_t Hkv,
                       hipStream_t st) {
  const SelPtrs q = carve_sel(sel_scratch, Hkv);
  k_init<<<Hkv, 256, 0, st>>>(status, flagcount, q.hist, q.st, Hkv);
  return hipGetLastError();
}

hipError_t launch_select(const float* S, int64_t n, int32_t w, int32_t Hkv, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_idx, int32_t* status,
                         void* scratch, hipStream_t st) {
  SelArgs A{};
  A.S = S;
  A.P = out_scores;
  A.idx = out_idx;
  A.n = n;
  A.n_evict = n_evict;
  A.w = w;
  A.pool_half = pool_kernel / 2;
  A.nblk = (int)((n + kChunk - 1) / kChunk);
  const SelPtrs q = carve_sel(scratch, Hkv);
  A.hist = q.hist;
  A.st = q.st;
  A.bc = q.bc;
  A.status = status;
  const dim3 grid(A.nblk, Hkv);
  k_sel_pool<<<grid, kT, 0, st>>>(A);
  if (n_evict > 0) {
    k_sel_refine<1><<<grid, kT, 0, st>>>(A);
    k_sel_refine<2><<<grid, kT, 0, st>>>(A);
    k_sel_count<<<grid, kT, 0, st>>>(A);
    k_sel_write<<<grid, kT, 0, st>>>(A);
  }
  return hipGetLastError();
}

}  // namespace dropkv
