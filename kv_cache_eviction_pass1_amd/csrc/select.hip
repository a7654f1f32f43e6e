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
// last). The n_evict-th smallest key tau is found by a radix select whose
// digits are key bits 31..20, 19..8 and 7..0. Three kernels, with no
// device-scope fence inside any of them (on this multi-XCD part a fence
// writes back the L2, which costs far more than a kernel boundary); the
// histograms and the candidate count start at zero (cleared by the first
// kernel of the scoring path, or by an init launch):
//   pool     many workgroups: pooled scores -> out_scores, histogram of digit 1;
//   cand     many workgroups: each derives digit 1 from the histogram, counts
//            per segment (8+ consecutive keys) the keys below digit 1's bin,
//            and compacts the keys inside that bin (the candidates) with
//            their indices, plus their digit-2 histogram;
//   write    many workgroups: each derives digits 2 and 3 from the candidates
//            (tau and `need`, how many keys equal to tau are evicted),
//            completes the per-segment counts with the candidates, turns the
//            counts of all earlier segments and its own into output offsets,
//            and writes its segments' evicted indices.
// Heads of up to 4096 tokens take one kernel instead (k_sel_small: one
// workgroup per head, everything in LDS), with the same results.
#include <type_traits>

#include "dropkv_common.h"

namespace dropkv {

namespace {

// 512 threads: two waves per SIMD hide part of the latency of these short,
// one-pass kernels (one workgroup per CU at the 128K shape)
constexpr int kT = 512;            // threads per workgroup (pool, cand, write)
constexpr int kChunk = 2048;       // pool: elements per workgroup (two workgroups per CU at the 128K layer: 1 us less than 4096)
constexpr int kPer = kChunk / kT;  // pool: elements per thread
constexpr int kKeys = 8;           // cand / write: keys per load group (segments are multiples of it)
constexpr int kMaxHalo = 512;      // pooling halo held in LDS (larger kernels read global memory)
constexpr int kBins1 = 4096;       // digit 1: key bits 31..20
constexpr int kBins2 = 4096;       // digit 2: key bits 19..8
constexpr int kBins3 = 256;        // digit 3: key bits 7..0
constexpr int kHistStride = kBins1 + kBins2 + 16;  // per head: hist1, hist2, candidate count
constexpr int kBinsPer = kBins1 / kT;  // digit-1 and digit-2 bins per thread
constexpr int kMaxWg = 32;         // cand / write workgroups per head
constexpr int kMaxSeg = kMaxWg * kT;  // segments per head
static_assert(kBins1 == kBins2 && kBinsPer % 4 == 0, "load_bins: whole 16-byte groups per thread");
static_assert(kChunk % kT == 0 && kKeys % 4 == 0, "pool and key groups");
static_assert(kMaxWg <= kT, "write: one earlier workgroup per thread");
static_assert(kBins3 <= kT, "digit-3 bins: at most one per thread of the write workgroup");

struct SelArgs {
  const float* S;
  float* P;        // out_scores
  int64_t* idx;    // out_evict_idx
  int64_t n, n_evict;
  int w, pool_half, nblk;
  int seg, nseg;   // keys per segment, segments per head
  bool vec4;       // P rows are 16-byte aligned (n % 4 == 0): vector loads
  uint32_t* hist;  // [Hkv][kHistStride]: hist1, hist2, candidate count (zeroed by init)
  uint2* cand;     // [Hkv][n]: (key, index) of the candidates
  uint32_t* seg_lt;   // [Hkv][nseg]: keys below digit 1's bin
  uint32_t* wg_lt;    // [Hkv][kMaxWg]: the same, summed over each cand workgroup's segments
  int32_t* status;
  FoldInfo fold;      // argmax terms of flagged rows to add to S (flagcount null: none)
  bool reject_negative;  // caller-given S: a negative entry raises kStatusNegative
  int64_t* keep;      // [Hkv][n - n_evict]: the kept token indices, ascending (null: not written)
};

__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? 0u : b;  // -0 (and any negative) sorts as +0
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (VALU only; lanes without a source read 0).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive prefix sums of two values over a workgroup of T threads (one
// barrier pair for both); totals returned in ta / tb. Sums must stay below 2^32.
template <int T>
__device__ __forceinline__ void wg_scan2(uint32_t xa, uint32_t xb, uint32_t (*wsum)[T / 64], uint32_t& ea,
                                         uint32_t& eb, uint32_t& ta, uint32_t& tb) {
  constexpr int NWV = T / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t va = wave_incl_scan(xa), vb = wave_incl_scan(xb);
  if (lane == 63) {
    wsum[0][wid] = va;
    wsum[1][wid] = vb;
  }
  __syncthreads();
  uint32_t ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    const uint32_t wa = wsum[0][i], wb = wsum[1][i];
    ba += (i < wid) ? wa : 0u;
    bb += (i < wid) ? wb : 0u;
    sa += wa;
    sb += wb;
  }
  ta = sa;
  tb = sb;
  ea = ba + va - xa;
  eb = bb + vb - xb;
  __syncthreads();
}

// Bin of a histogram holding the key of 1-based rank `rank`, and the rank
// inside that bin, from the counts c[] of bins threadIdx.x * PER + i (loaded
// by the caller); the result is in *bin / *rin for every thread on return.
template <int T, int PER>
__device__ __forceinline__ void find_bin_regs(const uint32_t (&c)[PER], int64_t rank, uint32_t (*wsum)[T / 64],
                                              int* bin, int64_t* rin) {
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) loc += c[i];
  uint32_t before, unused, total, unused2;
  wg_scan2<T>(loc, 0u, wsum, before, unused, total, unused2);
  if ((int64_t)before < rank && rank <= (int64_t)before + loc) {
    int64_t r = rank - before;
    int found = -1;
    int64_t rr = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (found < 0 && r <= (int64_t)c[i]) {
        found = threadIdx.x * PER + i;
        rr = r;
      }
      if (found < 0) r -= c[i];
    }
    *bin = found;
    *rin = rr;
  }
  __syncthreads();
}

// Counts of bins kBinsPer * threadIdx.x .. + kBinsPer - 1 of a 16-byte
// aligned histogram of kBins1 bins, in 16-byte loads.
__device__ __forceinline__ void load_bins(const uint32_t* h, uint32_t (&c)[kBinsPer]) {
  const uint4* p = reinterpret_cast<const uint4*>(h) + threadIdx.x * (kBinsPer / 4);
#pragma unroll
  for (int q = 0; q < kBinsPer / 4; ++q) {
    const uint4 v = p[q];
    c[4 * q] = v.x;
    c[4 * q + 1] = v.y;
    c[4 * q + 2] = v.z;
    c[4 * q + 3] = v.w;
  }
}

// Keys [j0, j0 + kKeys) of a head, 0xffffffff from `end` on.
__device__ __forceinline__ void load_keys(const float* Pg, int64_t j0, int64_t end, bool vec4,
                                          uint32_t (&key)[kKeys]) {
  if (vec4 && j0 + kKeys <= end) {
#pragma unroll
    for (int q = 0; q < kKeys / 4; ++q) {
      const float4 f = *(const float4*)(Pg + j0 + 4 * q);
      key[4 * q] = score_key(f.x);
      key[4 * q + 1] = score_key(f.y);
      key[4 * q + 2] = score_key(f.z);
      key[4 * q + 3] = score_key(f.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kKeys; ++e) key[e] = (j0 + e < end) ? score_key(Pg[j0 + e]) : 0xffffffffu;
  }
}

// Pool + protect (writes out_scores) and the histogram of digit 1.
__global__ __launch_bounds__(kT) void k_sel_pool(SelArgs A) {
  const int b = blockIdx.x, g = blockIdx.y;
  __shared__ float sS[kChunk + 2 * kMaxHalo];
  __shared__ uint32_t hist[kBins1];
  __shared__ float red[kT];
  __shared__ int bad;
  const float* Sg = A.S + (size_t)g * A.n;
  float* Pg = A.P + (size_t)g * A.n;
  const int64_t base = (int64_t)b * kChunk;
  const int half = A.pool_half;
  const bool in_lds = half <= kMaxHalo;
  // issued first: its latency overlaps the loads of the tile
  const int flagged = (in_lds && A.fold.flagcount) ? A.fold.flagcount[g] : 0;
  if (threadIdx.x == 0) bad = 0;
  for (int i = threadIdx.x; i < kBins1; i += kT) hist[i] = 0;
  if (in_lds) {
    // all loads in flight before the first LDS store (S >= 0: zero padding = clipping)
    float sv[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t j = base + e * kT + threadIdx.x;
      sv[e] = j < A.n ? Sg[j] : 0.0f;
    }
    const int ih = threadIdx.x < half ? threadIdx.x : (int)threadIdx.x - half + kChunk + half;
    float hv = 0.0f;
    const bool halo = threadIdx.x < 2 * half;
    if (halo) {
      const int64_t j = base - half + ih;
      hv = (j >= 0 && j < A.n) ? Sg[j] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) sS[half + e * kT + threadIdx.x] = sv[e];
    if (halo) sS[ih] = hv;
    for (int i = kT + threadIdx.x; i < 2 * half; i += kT) {  // halves above kT / 2 only
      const int ii = i < half ? i : i - half + kChunk + half;
      const int64_t j = base - half + ii;
      sS[ii] = (j >= 0 && j < A.n) ? Sg[j] : 0.0f;
    }
  }
  __syncthreads();
  if (flagged > 0) {
    // exact argmax terms of flagged rows, added in row order to this tile's
    // copy of S (workgroup 0 of the head records them in the row statistics)
    const FoldInfo& F = A.fold;
    for (int r = 0; r < F.Rg; ++r) {
      const int64_t row = (int64_t)g * F.Rg + r;
      if (!F.rs.flag[row]) continue;
      float R;
      int bits;
      const float val = fold_value<kT>(F, row, red, &R, &bits);
      const int js = F.rs.jstar[row];
      if (threadIdx.x == 0) {
        if (js < 0 || js >= A.n) {
          if (b == 0) atomicOr(A.status, kStatusNonFinite);
        } else {
          if (b == 0) {
            F.rs.rest[row] = R;
            F.rs.L[row] = 1.0f + R;
            F.rs.fixval[row] = val;
            if (bits) atomicOr(A.status, bits);
          }
          const int64_t li = js - (base - half);
          if (!bits && li >= 0 && li < kChunk + 2 * half) sS[li] += val * F.invG;
        }
      }
    }
    __syncthreads();
  }
  // token base + e * kT + threadIdx.x: consecutive threads, consecutive tokens
  float mx[kPer];
  bool nf = false, neg = false;
  if (in_lds) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      mx[e] = sS[half + e * kT + threadIdx.x];
      if (base + e * kT + threadIdx.x < A.n) {
        if (!finite_f(mx[e])) nf = true;  // max() would hide a NaN
        if (mx[e] < 0.0f) neg = true;     // -0.0 passes: it orders as +0
      }
    }
    // one window offset at a time: the kPer LDS reads of a step are independent
    for (int t = 0; t <= 2 * half; ++t) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) mx[e] = fmaxf(mx[e], sS[t + e * kT + threadIdx.x]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t j = base + e * kT + threadIdx.x;
      mx[e] = 0.0f;
      if (j < A.n) {
        mx[e] = Sg[j];
        if (!finite_f(mx[e])) nf = true;
        if (mx[e] < 0.0f) neg = true;
        const int64_t lo = j - half < 0 ? 0 : j - half;
        const int64_t hi = j + half >= A.n ? A.n - 1 : j + half;
        for (int64_t t = lo; t <= hi; ++t) mx[e] = fmaxf(mx[e], Sg[t]);
      }
    }
  }
  uint32_t key[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int64_t j = base + e * kT + threadIdx.x;
    key[e] = 0xffffffffu;
    if (j < A.n) {
      const float p = (j >= A.n - A.w) ? INFINITY : mx[e];
      Pg[j] = p;
      key[e] = score_key(p);
    }
  }
  if (nf) bad |= kStatusNonFinite;
  if (neg && A.reject_negative) bad |= kStatusNegative;
  if (A.n_evict > 0) {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (key[e] != 0xffffffffu) atomicAdd(&hist[key[e] >> 20], 1u);
  }
  __syncthreads();
  if (threadIdx.x == 0 && bad) atomicOr(A.status, bad);
  if (A.n_evict <= 0) return;
  uint32_t* gh = A.hist + (size_t)g * kHistStride;
  for (int i = threadIdx.x; i < kBins1; i += kT)
    if (hist[i]) atomicAdd(gh + i, hist[i]);
}

// Per segment: keys below digit 1's bin; the bin's keys become candidates.
__global__ __launch_bounds__(kT) void k_sel_cand(SelArgs A) {
  const int g = blockIdx.y;
  const int s = blockIdx.x * kT + threadIdx.x;
  __shared__ uint32_t hist2[kBins2];
  __shared__ uint32_t wsum[2][kT / 64];
  __shared__ int sh_bin;
  __shared__ int64_t sh_rin;
  __shared__ uint32_t sh_base;
  uint32_t* gh = A.hist + (size_t)g * kHistStride;
  const float* Pg = A.P + (size_t)g * A.n;
  const int64_t j0 = (int64_t)s * A.seg;
  const int64_t j1 = (s < A.nseg) ? ((j0 + A.seg < A.n) ? j0 + A.seg : A.n) : j0;
  // the segment's first keys and the digit-1 counts are loaded together
  uint32_t key0[kKeys];
  load_keys(Pg, j0, j1, A.vec4, key0);
  uint32_t c1[kBinsPer];
  load_bins(gh, c1);
  for (int i = threadIdx.x; i < kBins2; i += kT) hist2[i] = 0;
  find_bin_regs<kT, kBinsPer>(c1, A.n_evict, wsum, &sh_bin, &sh_rin);
  const uint32_t d1 = (uint32_t)sh_bin;
  uint32_t lt = 0, nc = 0;
  auto count_keys = [&](const uint32_t (&key)[kKeys]) {
#pragma unroll
    for (int e = 0; e < kKeys; ++e) {
      if (key[e] == 0xffffffffu) continue;
      const uint32_t top = key[e] >> 20;
      lt += top < d1 ? 1u : 0u;
      if (top == d1) {
        ++nc;
        atomicAdd(&hist2[(key[e] >> 8) & 0xfffu], 1u);
      }
    }
  };
  count_keys(key0);
  for (int64_t c0 = j0 + kKeys; c0 < j1; c0 += kKeys) {
    uint32_t key[kKeys];
    load_keys(Pg, c0, j1, A.vec4, key);
    count_keys(key);
  }
  if (s < A.nseg) A.seg_lt[(size_t)g * A.nseg + s] = lt;
  uint32_t before, unused, total, total_lt;
  wg_scan2<kT>(nc, lt, wsum, before, unused, total, total_lt);
  if (threadIdx.x == 0) {
    A.wg_lt[(size_t)g * kMaxWg + blockIdx.x] = total_lt;
    if (total > 0) sh_base = atomicAdd(gh + kBins1 + kBins2, total);
  }
  if (total > 0) {  // digit-2 counts (the barrier of the scan made hist2 complete)
    uint32_t* gh2 = gh + kBins1;
    for (int i = threadIdx.x; i < kBins2; i += kT)
      if (hist2[i]) atomicAdd(gh2 + i, hist2[i]);
  }
  __syncthreads();  // sh_base
  if (nc > 0) {
    uint2* cg = A.cand + (size_t)g * A.n;
    uint32_t pos = sh_base + before;
    auto emit_keys = [&](const uint32_t (&key)[kKeys], int64_t c0) {
#pragma unroll
      for (int e = 0; e < kKeys; ++e)
        if (key[e] != 0xffffffffu && (key[e] >> 20) == d1) {
          DKV_CHECK(pos < (uint32_t)A.n, A.status);
          cg[pos++] = make_uint2(key[e], (uint32_t)(c0 + e));
        }
    };
    emit_keys(key0, j0);
    for (int64_t c0 = j0 + kKeys; c0 < j1; c0 += kKeys) {
      uint32_t key[kKeys];
      load_keys(Pg, c0, j1, A.vec4, key);
      emit_keys(key, c0);
    }
  }
}

// tau, need, the output offsets of this workgroup's segments, and their
// evicted indices in index order. Every workgroup of a head derives the same
// tau from the same histograms and candidates. Everything that does not
// depend on tau is loaded in one round, the first kCandLds candidate slots
// included (read before their count is known; slots past it are ignored).
constexpr int kCandLds = 4096;        // candidates held in LDS (more are re-read from global memory)
constexpr int kTie = 1024;            // candidates sharing tau's digits 1 and 2, listed (more: a second pass)
constexpr int kStage = 2 * kCandLds;  // evicted indices staged per workgroup, as int32 over the candidate buffer

__global__ __launch_bounds__(kT) void k_sel_write(SelArgs A) {
  const int g = blockIdx.y;
  const int s0 = blockIdx.x * kT;  // first segment of this workgroup
  const int s = s0 + threadIdx.x;
  __shared__ uint2 cl[kCandLds + kT / 2];  // candidates; later kStage + kT staged uint32 slots
  __shared__ uint2 tie[kTie];
  __shared__ uint32_t hist3[kBins3];
  __shared__ uint32_t wlt[kT], weq[kT];
  __shared__ uint32_t wsum[2][kT / 64];
  __shared__ int sh_bin;
  __shared__ int64_t sh_rin;
  __shared__ uint32_t ntie;
  const uint32_t* gh = A.hist + (size_t)g * kHistStride;
  const uint32_t* sl = A.seg_lt + (size_t)g * A.nseg;
  const uint2* cg = A.cand + (size_t)g * A.n;
  const float* Pg = A.P + (size_t)g * A.n;
  // ---- the one round of loads
  uint32_t c1[kBinsPer], c2[kBinsPer];
  load_bins(gh, c1);
  load_bins(gh + kBins1, c2);
  const uint32_t nc = gh[kBins1 + kBins2];
  const uint32_t own_lt = s < A.nseg ? sl[s] : 0u;
  // keys below digit 1's bin in the workgroups of segments before this one's
  const uint32_t prev_lt = (int)threadIdx.x < (int)blockIdx.x ? A.wg_lt[(size_t)g * kMaxWg + threadIdx.x] : 0u;
  const int64_t j0 = (int64_t)s * A.seg;
  const int64_t j1 = (s < A.nseg) ? ((j0 + A.seg < A.n) ? j0 + A.seg : A.n) : j0;
  uint32_t key0[kKeys];
  load_keys(Pg, j0, j1, A.vec4, key0);
  const int64_t nspec = A.n < kCandLds ? A.n : kCandLds;
  {
    uint2 c16[kCandLds / kT];
#pragma unroll
    for (int k = 0; k < kCandLds / kT; ++k) {
      const int i = threadIdx.x + k * kT;
      c16[k] = i < nspec ? cg[i] : make_uint2(0xffffffffu, 0u);
    }
    if (threadIdx.x < kBins3) hist3[threadIdx.x] = 0;
    wlt[threadIdx.x] = 0;
    weq[threadIdx.x] = 0;
    if (threadIdx.x == 0) ntie = 0;
#pragma unroll
    for (int k = 0; k < kCandLds / kT; ++k) cl[threadIdx.x + k * kT] = c16[k];
  }
  find_bin_regs<kT, kBinsPer>(c1, A.n_evict, wsum, &sh_bin, &sh_rin);  // (its barriers also publish cl)
  const uint32_t d1 = (uint32_t)sh_bin;
  find_bin_regs<kT, kBinsPer>(c2, sh_rin, wsum, &sh_bin, &sh_rin);
  const uint32_t d2 = (uint32_t)sh_bin;
  const int64_t r2 = sh_rin;
  auto cand = [&](uint32_t i) { return i < (uint32_t)kCandLds ? cl[i] : cg[i]; };
  // counts of keys below tau (cb_lt) / equal to it (cb_eq) before this
  // workgroup's segments; wlt / weq: in each of its segments
  uint32_t cb_lt = 0, cb_eq = 0;
  auto count_lt = [&](uint32_t tok) {
    const int sg = (int)(tok / (uint32_t)A.seg);
    if (sg < s0) ++cb_lt;
    else if (sg < s0 + kT) atomicAdd(&wlt[sg - s0], 1u);
  };
  auto count_eq = [&](uint32_t tok) {
    const int sg = (int)(tok / (uint32_t)A.seg);
    if (sg < s0) ++cb_eq;
    else if (sg < s0 + kT) atomicAdd(&weq[sg - s0], 1u);
  };
  // one pass: digit 2 below d2 means below tau; equal goes to the digit-3
  // histogram and the tie list (every candidate has digit 1 == d1)
  auto sort_cand = [&](uint2 c) {
    const uint32_t dg = (c.x >> 8) & 0xfffu;
    if (dg < d2) {
      count_lt(c.y);
    } else if (dg == d2) {
      atomicAdd(&hist3[c.x & 0xffu], 1u);
      const uint32_t t = atomicAdd(&ntie, 1u);
      if (t < (uint32_t)kTie) tie[t] = c;
    }
  };
  const uint32_t ncl = nc < (uint32_t)kCandLds ? nc : (uint32_t)kCandLds;
  for (uint32_t i0 = 0; i0 < ncl; i0 += 4 * kT) {  // four LDS reads in flight
    uint2 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = i0 + k * kT + threadIdx.x;
      c[k] = i < ncl ? cl[i] : make_uint2(0xffffffffu, 0u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k * kT + threadIdx.x < ncl) sort_cand(c[k]);
  }
  for (uint32_t i = ncl + threadIdx.x; i < nc; i += kT) sort_cand(cg[i]);
  __syncthreads();
  uint32_t c3[1];
  c3[0] = threadIdx.x < kBins3 ? hist3[threadIdx.x] : 0u;
  find_bin_regs<kT, 1>(c3, r2, wsum, &sh_bin, &sh_rin);
  const uint32_t tau = (d1 << 20) | (d2 << 8) | (uint32_t)sh_bin;
  const int64_t need = sh_rin;
  const uint32_t nt = ntie;
  auto count_tie = [&](uint2 c) {
    if (c.x < tau) count_lt(c.y);
    else if (c.x == tau) count_eq(c.y);
  };
  if (nt <= (uint32_t)kTie) {
    for (uint32_t i = threadIdx.x; i < nt; i += kT) count_tie(tie[i]);
  } else {
    for (uint32_t i = threadIdx.x; i < nc; i += kT) {
      const uint2 c = cand(i);
      if (((c.x >> 8) & 0xfffu) == d2) count_tie(c);
    }
  }
  // counts below 2^31 (n fits in int32): 32-bit scans
  uint32_t x0, x1, tot_lt, tot_eq;
  wg_scan2<kT>(prev_lt + cb_lt, cb_eq, wsum, x0, x1, tot_lt, tot_eq);
  uint32_t lpre, epre, in_lt, in_eq;
  wg_scan2<kT>(own_lt + wlt[threadIdx.x], weq[threadIdx.x], wsum, lpre, epre, in_lt, in_eq);
  // this workgroup's evictions fill og[base, base + cnt)
  const int64_t taken0 = (int64_t)tot_eq < need ? (int64_t)tot_eq : need;
  const int64_t taken1 = (int64_t)tot_eq + in_eq < need ? (int64_t)tot_eq + in_eq : need;
  const int64_t base = (int64_t)tot_lt + taken0;
  const int64_t cnt = (int64_t)in_lt + (taken1 - taken0);
  const bool staged = cnt <= kStage;  // same for every thread
  uint32_t* stg = reinterpret_cast<uint32_t*>(cl);  // kStage slots, then one spare slot per thread
  int64_t* og = A.idx + (size_t)g * A.n_evict;
  // token indices, counts and positions fit in 32 bits (n < 2^31)
  const uint32_t need32 = (uint32_t)need;
  const uint32_t base32 = (uint32_t)base, cnt32 = (uint32_t)cnt;
  auto emit = [&](auto to_lds) {
    if (s >= A.nseg) return;
    uint32_t eqb = tot_eq + epre;
    uint32_t pos = tot_lt + lpre + (eqb < need32 ? eqb : need32);
    int64_t* kg = A.keep ? A.keep + (size_t)g * (size_t)(A.n - A.n_evict) : nullptr;
    const uint32_t n_keep32 = (uint32_t)(A.n - A.n_evict);
    auto emit_keys = [&](const uint32_t (&key)[kKeys], uint32_t q0) {
#pragma unroll
      for (int k = 0; k < kKeys; ++k) {
        const bool eq = key[k] == tau;
        const bool take = key[k] < tau || (eq && eqb < need32);
        eqb += eq ? 1u : 0u;
        if (kg && !take && key[k] != 0xffffffffu) {
          // a kept token j lands at j - #{evicted tokens below j} = j - pos
          const uint32_t kp = q0 + k - pos;
          DKV_CHECK(kp < n_keep32, A.status);
          if (kp < n_keep32) kg[kp] = (int64_t)(q0 + k);
        }
        if constexpr (decltype(to_lds)::value) {
          // no branch: a key not taken is written to this thread's spare slot
          const uint32_t r = pos - base32;  // wraps above cnt32 if ever below base
          stg[(take && r < cnt32) ? r : (uint32_t)(kStage + threadIdx.x)] = q0 + k;
        } else {
          DKV_CHECK(!take || pos < (uint32_t)A.n_evict, A.status);
          if (take && pos < (uint32_t)A.n_evict) og[pos] = (int64_t)(q0 + k);
        }
        pos += take ? 1u : 0u;
      }
    };
    emit_keys(key0, (uint32_t)j0);
    for (int64_t q0 = j0 + kKeys; q0 < j1; q0 += kKeys) {
      uint32_t key[kKeys];
      load_keys(Pg, q0, j1, A.vec4, key);
      emit_keys(key, (uint32_t)q0);
    }
  };
  if (!staged) {
    emit(std::false_type{});
    return;
  }
  emit(std::true_type{});
  __syncthreads();
  // consecutive threads, consecutive output slots; the LDS reads first (slot
  // i0 + k * kT + threadIdx.x < i0 + kOutPer * kT <= kStage while i0 < cnt32)
  constexpr int kOutPer = kStage / kT / 2;
  static_assert(kStage % (kOutPer * kT) == 0, "whole rounds of output slots");
  const int64_t lim = A.n_evict - base;  // >= cnt for consistent scores
  for (uint32_t i0 = 0; i0 < cnt32; i0 += kOutPer * kT) {
    uint32_t v[kOutPer];
#pragma unroll
    for (int k = 0; k < kOutPer; ++k) v[k] = stg[i0 + k * kT + threadIdx.x];
#pragma unroll
    for (int k = 0; k < kOutPer; ++k) {
      const uint32_t i = i0 + k * kT + threadIdx.x;
      DKV_CHECK(i >= cnt32 || (int64_t)i < lim, A.status);
      if (i < cnt32 && (int64_t)i < lim) og[base + i] = (int64_t)v[k];
    }
  }
}

// ---- short heads: the whole stage in one workgroup per KV head
//
// Up to kSmallT * PER tokens a head's scores fit in LDS, so one workgroup of
// kSmallT threads folds, pools and protects them, runs the three radix digits
// on the keys in LDS, and writes the evicted (and, on request, kept) indices
// in order through an LDS staging area: one launch instead of three, with no
// global histograms or candidate lists. Same results as the three-kernel
// path: the pooled values are the same maxima (zero padding, the same order
// of the folded terms) and the selection is unique under (value, index).
// Used for short heads only: one CU per head does all of the head's
// histogram atomics, which longer heads spread over many workgroups.
// 1024 threads x 4 tokens (4K heads): 17.0 -> 12.4 us against the three
// kernels; 512 x 8 took 14.1 us, and 1024 x 32 (32K heads) 61 us against 16.7.
constexpr int kSmallThreads = 1024;
constexpr int kSmallPer = 4;
constexpr int kSmallHalf = 32;  // widest pooling half-width on this path

// LDS index of token (or output slot) j: one word of padding per 32, so the
// threads' contiguous blocks of keys fall in distinct banks
__device__ __forceinline__ int spad(int j) { return j + (j >> 5); }

template <int kSmallT, int PER>
__global__ __launch_bounds__(kSmallT) void k_sel_small(SelArgs A) {
  static_assert(kBins1 % kSmallT == 0 && kBins3 <= kSmallT, "bins per thread");
  constexpr int kN = kSmallT * PER;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ uint32_t sk[kN + kN / 32];  // S, then keys, then the staged output slots
  __shared__ uint32_t hist[kBins1];
  __shared__ float red[kSmallT];
  __shared__ uint32_t wsum[2][kSmallT / 64];
  __shared__ int sh_bin;
  __shared__ int64_t sh_rin;
  __shared__ int bad;
  const int n = (int)A.n;
  const int ne = (int)A.n_evict;
  const float* Sg = A.S + (size_t)g * A.n;
  float* Pg = A.P + (size_t)g * A.n;
  const int flagged = A.fold.flagcount ? A.fold.flagcount[g] : 0;
  if (tid == 0) bad = 0;
  for (int j = tid; j < n; j += kSmallT) sk[spad(j)] = __float_as_uint(Sg[j]);
  __syncthreads();
  if (flagged > 0) {
    // exact argmax terms of flagged rows, added to S in row order (and
    // recorded in the row statistics)
    const FoldInfo& F = A.fold;
    for (int r = 0; r < F.Rg; ++r) {
      const int64_t row = (int64_t)g * F.Rg + r;
      if (!F.rs.flag[row]) continue;
      float R;
      int bits;
      const float val = fold_value<kSmallT>(F, row, red, &R, &bits);
      const int js = F.rs.jstar[row];
      if (tid == 0) {
        if (js < 0 || js >= n) {
          atomicOr(A.status, kStatusNonFinite);
        } else {
          F.rs.rest[row] = R;
          F.rs.L[row] = 1.0f + R;
          F.rs.fixval[row] = val;
          if (bits) atomicOr(A.status, bits);
          else sk[spad(js)] = __float_as_uint(__uint_as_float(sk[spad(js)]) + val * F.invG);
        }
      }
    }
    __syncthreads();
  }
  // pool (zero padding, as the LDS tile of the pool kernel), token i * kSmallT + tid
  const int half = A.pool_half;
  float pv[PER];
  bool nf = false, neg = false;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = i * kSmallT + tid;
    float m = 0.0f;
    if (j < n) {
      m = __uint_as_float(sk[spad(j)]);
      if (!finite_f(m)) nf = true;  // max() would hide a NaN
      if (m < 0.0f) neg = true;     // -0.0 passes: it orders as +0
    }
    pv[i] = m;
  }
  // one window offset at a time (a uniform loop): the PER reads of a step are independent
  for (int dt = -half; dt <= half; ++dt) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = i * kSmallT + tid + dt;
      pv[i] = fmaxf(pv[i], (t >= 0 && t < n) ? __uint_as_float(sk[spad(t)]) : 0.0f);
    }
  }
  if (nf) atomicOr(&bad, kStatusNonFinite);
  if (neg && A.reject_negative) atomicOr(&bad, kStatusNegative);
  __syncthreads();  // every read of S is done: the array takes the keys
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = i * kSmallT + tid;
    if (j < n) {
      const float p = (j >= n - A.w) ? INFINITY : pv[i];
      Pg[j] = p;
      sk[spad(j)] = score_key(p);
    }
  }
  if (tid == 0 && bad) atomicOr(A.status, bad);
  int64_t* kg = A.keep ? A.keep + (size_t)g * (size_t)(n - ne) : nullptr;
  if (ne <= 0) {
    if (kg)
      for (int j = tid; j < n; j += kSmallT) kg[j] = j;
    return;
  }
  int64_t* og = A.idx + (size_t)g * (size_t)ne;
  // radix digits 1 and 2 (12 bits each) and 3 (8 bits) of the n_evict-th key
  for (int b = tid; b < kBins1; b += kSmallT) hist[b] = 0;
  __syncthreads();  // keys complete, histogram cleared
  for (int j = tid; j < n; j += kSmallT) atomicAdd(&hist[sk[spad(j)] >> 20], 1u);
  __syncthreads();
  constexpr int kPerBin = kBins1 / kSmallT;
  uint32_t c[kPerBin];
#pragma unroll
  for (int i = 0; i < kPerBin; ++i) c[i] = hist[tid * kPerBin + i];
  find_bin_regs<kSmallT, kPerBin>(c, ne, wsum, &sh_bin, &sh_rin);
  const uint32_t d1 = (uint32_t)sh_bin;
  const int64_t r1 = sh_rin;
  for (int b = tid; b < kBins2; b += kSmallT) hist[b] = 0;
  __syncthreads();
  for (int j = tid; j < n; j += kSmallT) {
    const uint32_t key = sk[spad(j)];
    if ((key >> 20) == d1) atomicAdd(&hist[(key >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPerBin; ++i) c[i] = hist[tid * kPerBin + i];
  find_bin_regs<kSmallT, kPerBin>(c, r1, wsum, &sh_bin, &sh_rin);
  const uint32_t d2 = (uint32_t)sh_bin;
  const int64_t r2 = sh_rin;
  if (tid < kBins3) hist[tid] = 0;
  __syncthreads();
  const uint32_t top = (d1 << 12) | d2;
  for (int j = tid; j < n; j += kSmallT) {
    const uint32_t key = sk[spad(j)];
    if ((key >> 8) == top) atomicAdd(&hist[key & 0xffu], 1u);
  }
  __syncthreads();
  uint32_t c3[1];
  c3[0] = tid < kBins3 ? hist[tid] : 0u;
  find_bin_regs<kSmallT, 1>(c3, r2, wsum, &sh_bin, &sh_rin);
  const uint32_t tau = (top << 8) | (uint32_t)sh_bin;
  const uint32_t need = (uint32_t)sh_rin;  // keys equal to tau that are evicted (lowest indices)
  // each thread's contiguous block of tokens: counts, offsets, then the
  // evicted slots [0, ne) and the kept slots [ne, n) staged in the key array
  const int per = (n + kSmallT - 1) / kSmallT;
  const int j0 = tid * per;
  uint32_t kr[PER];
  uint32_t clt = 0, ceq = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = j0 + k;
    kr[k] = (k < per && j < n) ? sk[spad(j)] : 0xffffffffu;
    clt += kr[k] < tau ? 1u : 0u;
    ceq += kr[k] == tau ? 1u : 0u;
  }
  uint32_t blt, beq, tlt, teq;
  wg_scan2<kSmallT>(clt, ceq, wsum, blt, beq, tlt, teq);  // (its barriers: every key is read)
  uint32_t eqb = beq;
  uint32_t pos = blt + (beq < need ? beq : need);
  const uint32_t nkeep = (uint32_t)(n - ne);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = j0 + k;
    // no branch: an evicted token goes to slot pos, a kept one to ne + (j - pos)
    // (j - pos kept tokens below it); tokens past the block write nothing
    const bool valid = k < per && j < n;
    const bool eq = kr[k] == tau;
    const bool take = kr[k] < tau || (eq && eqb < need);
    eqb += (valid && eq) ? 1u : 0u;
    const uint32_t slot = take ? pos : (uint32_t)ne + ((uint32_t)j - pos);
    DKV_CHECK(!valid || slot < (uint32_t)n, A.status);
    if (valid && slot < (uint32_t)n) sk[spad((int)slot)] = (uint32_t)j;
    pos += (valid && take) ? 1u : 0u;
  }
  __syncthreads();
  for (int q = tid; q < ne; q += kSmallT) og[q] = (int64_t)sk[spad(q)];
  if (kg)
    for (int q = tid; q < (int)nkeep; q += kSmallT) kg[q] = (int64_t)sk[spad(ne + q)];
}

// Zeroes the status word, the per-head flag counts and the select histograms
// and candidate counts in one launch.
__global__ void k_init(int32_t* status, int32_t* flagcount, uint32_t* hist) {
  const int g = blockIdx.x;
  uint32_t* h = hist + (size_t)g * kHistStride;
  for (int i = threadIdx.x; i < kHistStride; i += blockDim.x) h[i] = 0;
  if (threadIdx.x == 0) {
    if (flagcount) flagcount[g] = 0;
    if (g == 0) *status = 0;
  }
}

// Every token kept (n_evict = 0): the kept list is 0 .. n - 1 for each head.
__global__ void k_keep_all(int64_t* keep, int64_t n, int32_t Hkv) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n * Hkv) keep[i] = i % n;
}

struct SelGeom {
  int seg, nseg;
};

SelGeom sel_geom(int64_t n) {
  int64_t seg = (n + kMaxSeg - 1) / kMaxSeg;
  seg = (seg + kKeys - 1) / kKeys * kKeys;
  if (seg < kKeys) seg = kKeys;
  SelGeom q;
  q.seg = (int)seg;
  q.nseg = (int)((n + seg - 1) / seg);
  return q;
}

struct SelPtrs {
  uint32_t* hist;
  uint2* cand;
  uint32_t* seg_lt;
  uint32_t* wg_lt;
  size_t bytes;
};

SelPtrs carve_sel(void* scratch, int64_t n, int32_t Hkv) {
  const SelGeom q = sel_geom(n);
  SelPtrs r{};
  char* base = (char*)scratch;
  size_t off = 0;
  auto take = [&](size_t b) {
    char* p = base ? base + off : nullptr;
    off += (b + 255) / 256 * 256;
    return p;
  };
  r.hist = (uint32_t*)take(sizeof(uint32_t) * (size_t)Hkv * kHistStride);
  r.cand = (uint2*)take(sizeof(uint2) * (size_t)Hkv * (size_t)n);
  r.seg_lt = (uint32_t*)take(sizeof(uint32_t) * (size_t)Hkv * q.nseg);
  r.wg_lt = (uint32_t*)take(sizeof(uint32_t) * (size_t)Hkv * kMaxWg);
  r.bytes = off;
  return r;
}

}  // namespace

size_t select_scratch_bytes(int64_t n, int32_t Hkv) { return carve_sel(nullptr, n, Hkv).bytes + 256; }

size_t select_zero_words(int32_t Hkv) { return (size_t)Hkv * kHistStride; }

// the 15 words after each head's candidate count (kHistStride = bins + 16)
static_assert(kHistStride - kBins1 - kBins2 - 1 >= kSelSpareWords, "spare words");
uint32_t* select_spare_words(void* sel_scratch, int32_t g) {
  return (uint32_t*)sel_scratch + (size_t)g * kHistStride + kBins1 + kBins2 + 1;
}

hipError_t launch_init(int32_t* status, int32_t* flagcount, void* sel_scratch, int32_t Hkv,
                       hipStream_t st) {
  // the histogram block sits first in the select scratch for every n
  k_init<<<Hkv, 256, 0, st>>>(status, flagcount, (uint32_t*)sel_scratch);
  return hipGetLastError();
}

hipError_t launch_select(const float* S, int64_t n, int32_t w, int32_t Hkv, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_idx, int32_t* status,
                         const FoldInfo* fold, void* scratch, hipStream_t st, bool reject_negative,
                         StageEvents* se, int64_t* keep_idx) {
  const SelGeom q = sel_geom(n);
  if (fold && fold->flagcount && pool_kernel / 2 > kMaxHalo) {
    // the pool kernel reads S from global memory for such wide kernels: fold first
    hipError_t e = launch_fold(*fold, n, Hkv, const_cast<float*>(S), status, st);
    if (e != hipSuccess) return e;
    fold = nullptr;
  }
  const SelPtrs p = carve_sel(scratch, n, Hkv);
  const bool small = pool_kernel / 2 <= kSmallHalf && n <= kSmallThreads * kSmallPer;
  SelArgs A{};
  A.S = S;
  A.P = out_scores;
  A.idx = out_idx;
  A.n = n;
  A.n_evict = n_evict;
  A.w = w;
  A.pool_half = pool_kernel / 2;
  A.nblk = (int)((n + kChunk - 1) / kChunk);
  A.seg = q.seg;
  A.nseg = q.nseg;
  A.vec4 = (n % 4 == 0) && ((uintptr_t)out_scores % 16 == 0);
  A.hist = p.hist;
  A.cand = p.cand;
  A.seg_lt = p.seg_lt;
  A.wg_lt = p.wg_lt;
  A.status = status;
  A.reject_negative = reject_negative;
  A.keep = keep_idx;
  if (fold) A.fold = *fold;
  if (small)
    return stage_launch(se, "select", kStageOnly, k_sel_small<kSmallThreads, kSmallPer>, dim3(Hkv),
                        dim3(kSmallThreads), st, A);
  hipError_t e = stage_launch(se, "select", n_evict > 0 ? kStageFirst : kStageOnly, k_sel_pool,
                              dim3(A.nblk, Hkv), dim3(kT), st, A);
  if (e == hipSuccess && n_evict <= 0 && keep_idx) {
    const int64_t total = n * Hkv;
    k_keep_all<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(keep_idx, n, Hkv);
    e = hipGetLastError();
  }
  if (e != hipSuccess || n_evict <= 0) return e;
  const dim3 gs((q.nseg + kT - 1) / kT, Hkv);
  e = stage_launch(se, "select", kStageMid, k_sel_cand, gs, dim3(kT), st, A);
  if (e != hipSuccess) return e;
  return stage_launch(se, "select", kStageLast, k_sel_write, gs, dim3(kT), st, A);
}

}  // namespace dropkv
