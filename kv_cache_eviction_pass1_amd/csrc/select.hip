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
// digits are key bits 31..20, 19..8 and 7..0. Four kernels, with no
// device-scope fence inside any of them (on this multi-XCD part a fence
// writes back the L2, which costs far more than a kernel boundary):
//   pool     many workgroups: pooled scores -> out_scores, histogram of digit 1;
//   cand     many workgroups: each derives digit 1 from the histogram, counts
//            per segment (16+ consecutive keys) the keys below digit 1's bin,
//            and compacts the keys inside that bin (the candidates) with
//            their indices, plus their digit-2 histogram;
//   write    many workgroups: each derives digits 2 and 3 from the candidates
//            (tau and `need`, how many keys equal to tau are evicted),
//            completes the per-segment counts with the candidates, turns the
//            counts of all earlier segments and its own into output offsets,
//            and writes its segments' evicted indices.
#include "dropkv_common.h"

namespace dropkv {

namespace {

constexpr int kT = 256;            // threads per workgroup (pool, cand, write)
constexpr int kPer = 16;           // pool: elements per thread
constexpr int kChunk = kT * kPer;  // pool: elements per workgroup
constexpr int kMaxHalo = 512;      // pooling halo held in LDS (larger kernels read global memory)
constexpr int kBins1 = 4096;       // digit 1: key bits 31..20
constexpr int kBins2 = 4096;       // digit 2: key bits 19..8
constexpr int kBins3 = 256;        // digit 3: key bits 7..0
constexpr int kHistStride = kBins1 + kBins2 + 16;  // per head: hist1, hist2, candidate count
constexpr int kMaxSeg = 8192;      // segments per head (bounds the prefix each write workgroup sums)
static_assert(kBins3 == kT, "digit-3 bins: one per thread of the write workgroup");

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
  int32_t* status;
  FoldInfo fold;      // argmax terms of flagged rows to add to S (flagcount null: none)
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

template <int T, int NB>
__device__ __forceinline__ void load_bins(const uint32_t* h, uint32_t (&c)[(NB + T - 1) / T]) {
  constexpr int PER = (NB + T - 1) / T;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = threadIdx.x * PER + i;
    c[i] = b < NB ? h[b] : 0u;
  }
}

// Keys [j0, j0 + 16) of a head, 0xffffffff from `end` on.
__device__ __forceinline__ void load16(const float* Pg, int64_t j0, int64_t end, bool vec4, uint32_t (&key)[16]) {
  if (vec4 && j0 + 16 <= end) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *(const float4*)(Pg + j0 + 4 * q);
      key[4 * q] = score_key(f.x);
      key[4 * q + 1] = score_key(f.y);
      key[4 * q + 2] = score_key(f.z);
      key[4 * q + 3] = score_key(f.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) key[e] = (j0 + e < end) ? score_key(Pg[j0 + e]) : 0xffffffffu;
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
  if (in_lds && A.fold.flagcount && A.fold.flagcount[g] > 0) {
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
  // the segment's first 16 keys and the digit-1 counts are loaded together
  uint32_t key0[16];
  load16(Pg, j0, j1, A.vec4, key0);
  uint32_t c1[kBins1 / kT];
  load_bins<kT, kBins1>(gh, c1);
  for (int i = threadIdx.x; i < kBins2; i += kT) hist2[i] = 0;
  find_bin_regs<kT, kBins1 / kT>(c1, A.n_evict, wsum, &sh_bin, &sh_rin);
  const uint32_t d1 = (uint32_t)sh_bin;
  uint32_t lt = 0, nc = 0;
  auto count16 = [&](const uint32_t (&key)[16]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (key[e] == 0xffffffffu) continue;
      const uint32_t top = key[e] >> 20;
      lt += top < d1 ? 1u : 0u;
      if (top == d1) {
        ++nc;
        atomicAdd(&hist2[(key[e] >> 8) & 0xfffu], 1u);
      }
    }
  };
  count16(key0);
  for (int64_t c0 = j0 + 16; c0 < j1; c0 += 16) {
    uint32_t key[16];
    load16(Pg, c0, j1, A.vec4, key);
    count16(key);
  }
  if (s < A.nseg) A.seg_lt[(size_t)g * A.nseg + s] = lt;
  uint32_t before, unused, total, unused2;
  wg_scan2<kT>(nc, 0u, wsum, before, unused, total, unused2);
  if (threadIdx.x == 0 && total > 0) sh_base = atomicAdd(gh + kBins1 + kBins2, total);
  __syncthreads();
  if (nc > 0) {
    uint2* cg = A.cand + (size_t)g * A.n;
    uint32_t pos = sh_base + before;
    auto emit16 = [&](const uint32_t (&key)[16], int64_t c0) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key[e] != 0xffffffffu && (key[e] >> 20) == d1) cg[pos++] = make_uint2(key[e], (uint32_t)(c0 + e));
    };
    emit16(key0, j0);
    for (int64_t c0 = j0 + 16; c0 < j1; c0 += 16) {
      uint32_t key[16];
      load16(Pg, c0, j1, A.vec4, key);
      emit16(key, c0);
    }
  }
  if (total > 0) {
    uint32_t* gh2 = gh + kBins1;
    for (int i = threadIdx.x; i < kBins2; i += kT)
      if (hist2[i]) atomicAdd(gh2 + i, hist2[i]);
  }
}

// tau, need, the output offsets of this workgroup's segments, and their
// evicted indices in index order. Every workgroup of a head derives the same
// tau from the same histograms and candidates. All loads that do not depend
// on tau are issued together first; the candidates are staged in LDS.
constexpr int kCandLds = 4096;  // candidates held in LDS (more are re-read from global memory)

__global__ __launch_bounds__(kT) void k_sel_write(SelArgs A) {
  const int g = blockIdx.y;
  const int s0 = blockIdx.x * kT;  // first segment of this workgroup
  const int s = s0 + threadIdx.x;
  __shared__ uint2 cl[kCandLds];
  __shared__ uint32_t hist3[kBins3];
  __shared__ uint32_t wlt[kT], weq[kT];
  __shared__ uint32_t wsum[2][kT / 64];
  __shared__ int sh_bin;
  __shared__ int64_t sh_rin;
  const uint32_t* gh = A.hist + (size_t)g * kHistStride;
  const uint32_t* sl = A.seg_lt + (size_t)g * A.nseg;
  const uint2* cg = A.cand + (size_t)g * A.n;
  const float* Pg = A.P + (size_t)g * A.n;
  // ---- round 1: histograms, candidate count, segment counts, this segment's first keys
  uint32_t c1[kBins1 / kT], c2[kBins2 / kT];
  load_bins<kT, kBins1>(gh, c1);
  load_bins<kT, kBins2>(gh + kBins1, c2);
  const uint32_t nc = gh[kBins1 + kBins2];
  const uint32_t own_lt = s < A.nseg ? sl[s] : 0u;
  uint32_t pre[kMaxSeg / kT];  // counts of the segments before this workgroup's
#pragma unroll
  for (int k = 0; k < kMaxSeg / kT; ++k) {
    const int t = threadIdx.x + k * kT;
    pre[k] = t < s0 ? sl[t] : 0u;
  }
  const int64_t j0 = (int64_t)s * A.seg;
  const int64_t j1 = (s < A.nseg) ? ((j0 + A.seg < A.n) ? j0 + A.seg : A.n) : j0;
  uint32_t key0[16];
  load16(Pg, j0, j1, A.vec4, key0);
  hist3[threadIdx.x] = 0;  // kT == kBins3
  wlt[threadIdx.x] = 0;
  weq[threadIdx.x] = 0;
  // ---- round 2: candidates into LDS
  const uint32_t ncl = nc < (uint32_t)kCandLds ? nc : (uint32_t)kCandLds;
  {
    uint2 c16[kCandLds / kT];
#pragma unroll
    for (int k = 0; k < kCandLds / kT; ++k) {
      const uint32_t i = threadIdx.x + k * kT;
      c16[k] = i < ncl ? cg[i] : make_uint2(0xffffffffu, 0u);
    }
#pragma unroll
    for (int k = 0; k < kCandLds / kT; ++k) cl[threadIdx.x + k * kT] = c16[k];
  }
  uint32_t before_lt = 0;
#pragma unroll
  for (int k = 0; k < kMaxSeg / kT; ++k) before_lt += pre[k];
  find_bin_regs<kT, kBins1 / kT>(c1, A.n_evict, wsum, &sh_bin, &sh_rin);  // (its barriers also publish cl)
  const uint32_t d1 = (uint32_t)sh_bin;
  find_bin_regs<kT, kBins2 / kT>(c2, sh_rin, wsum, &sh_bin, &sh_rin);
  const uint32_t d2 = (uint32_t)sh_bin;
  const int64_t r2 = sh_rin;
  auto cand = [&](uint32_t i) { return i < (uint32_t)kCandLds ? cl[i] : cg[i]; };
  for (uint32_t i = threadIdx.x; i < nc; i += kT) {
    const uint32_t key = cand(i).x;
    if (((key >> 8) & 0xfffu) == d2) atomicAdd(&hist3[key & 0xffu], 1u);
  }
  __syncthreads();
  uint32_t c3[1];
  c3[0] = hist3[threadIdx.x];
  find_bin_regs<kT, 1>(c3, r2, wsum, &sh_bin, &sh_rin);
  const uint32_t tau = (d1 << 20) | (d2 << 8) | (uint32_t)sh_bin;
  const int64_t need = sh_rin;
  // candidates below / equal to tau: before this workgroup's segments, or in one of them
  uint32_t cb_lt = 0, cb_eq = 0;
  for (uint32_t i = threadIdx.x; i < nc; i += kT) {
    const uint2 c = cand(i);
    if (c.x > tau) continue;
    const int sg = (int)(c.y / (uint32_t)A.seg);
    if (c.x < tau) {
      if (sg < s0) ++cb_lt;
      else if (sg < s0 + kT) atomicAdd(&wlt[sg - s0], 1u);
    } else {
      if (sg < s0) ++cb_eq;
      else if (sg < s0 + kT) atomicAdd(&weq[sg - s0], 1u);
    }
  }
  // counts below 2^31 (n fits in int32): 32-bit scans
  uint32_t x0, x1, tot_lt, tot_eq;
  wg_scan2<kT>((uint32_t)(before_lt + cb_lt), (uint32_t)cb_eq, wsum, x0, x1, tot_lt, tot_eq);
  uint32_t lpre, epre, t0, t1;
  wg_scan2<kT>(own_lt + wlt[threadIdx.x], weq[threadIdx.x], wsum, lpre, epre, t0, t1);
  const int64_t lb = (int64_t)tot_lt + lpre;
  int64_t eqb = (int64_t)tot_eq + epre;
  if (s >= A.nseg) return;
  int64_t pos = lb + (eqb < need ? eqb : need);
  int64_t* og = A.idx + (size_t)g * A.n_evict;
  auto emit16 = [&](const uint32_t (&key)[16], int64_t q0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      bool take = key[k] < tau;
      if (key[k] == tau) {
        take = eqb < need;
        ++eqb;
      }
      if (take) {
        if (pos < A.n_evict) og[pos] = q0 + k;
        ++pos;
      }
    }
  };
  emit16(key0, j0);
  for (int64_t q0 = j0 + 16; q0 < j1; q0 += 16) {
    uint32_t key[16];
    load16(Pg, q0, j1, A.vec4, key);
    emit16(key, q0);
  }
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

struct SelGeom {
  int seg, nseg;
};

SelGeom sel_geom(int64_t n) {
  int64_t seg = (n + kMaxSeg - 1) / kMaxSeg;
  seg = (seg + 15) / 16 * 16;
  if (seg < 16) seg = 16;
  SelGeom q;
  q.seg = (int)seg;
  q.nseg = (int)((n + seg - 1) / seg);
  return q;
}

struct SelPtrs {
  uint32_t* hist;
  uint2* cand;
  uint32_t* seg_lt;
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
  r.bytes = off;
  return r;
}

}  // namespace

size_t select_scratch_bytes(int64_t n, int32_t Hkv) { return carve_sel(nullptr, n, Hkv).bytes + 256; }

size_t select_zero_words(int32_t Hkv) { return (size_t)Hkv * kHistStride; }

hipError_t launch_init(int32_t* status, int32_t* flagcount, void* sel_scratch, int32_t Hkv,
                       hipStream_t st) {
  // the histogram block sits first in the select scratch for every n
  k_init<<<Hkv, 256, 0, st>>>(status, flagcount, (uint32_t*)sel_scratch);
  return hipGetLastError();
}

hipError_t launch_select(const float* S, int64_t n, int32_t w, int32_t Hkv, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_idx, int32_t* status,
                         const FoldInfo* fold, void* scratch, hipStream_t st) {
  const SelGeom q = sel_geom(n);
  if (fold && fold->flagcount && pool_kernel / 2 > kMaxHalo) {
    // the pool kernel reads S from global memory for such wide kernels: fold first
    hipError_t e = launch_fold(*fold, n, Hkv, const_cast<float*>(S), status, st);
    if (e != hipSuccess) return e;
    fold = nullptr;
  }
  const SelPtrs p = carve_sel(scratch, n, Hkv);
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
  A.status = status;
  if (fold) A.fold = *fold;
  k_sel_pool<<<dim3(A.nblk, Hkv), kT, 0, st>>>(A);
  if (n_evict > 0) {
    const dim3 gs((q.nseg + kT - 1) / kT, Hkv);
    k_sel_cand<<<gs, kT, 0, st>>>(A);
    k_sel_write<<<gs, kT, 0, st>>>(A);
  }
  return hipGetLastError();
}

}  // namespace dropkv
