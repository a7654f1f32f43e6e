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
//   tau      one workgroup per head: digits 2 and 3 from the candidates give
//            tau and `need` (how many keys equal to tau are evicted); the
//            candidates complete the per-segment counts, and a scan turns
//            them into per-segment output offsets;
//   write    many workgroups: every segment writes its evicted indices.
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
constexpr int kFT = 1024;          // threads of the tau workgroup
constexpr int kMaxSeg = 8192;      // segments per head (held in the tau workgroup's LDS)

struct SelState {
  uint32_t tau;
  uint32_t pad;
  int64_t need;  // keys equal to tau that are evicted (lowest indices first)
};

struct SelArgs {
  const float* S;
  float* P;        // out_scores
  int64_t* idx;    // out_evict_idx
  int64_t n, n_evict;
  int w, pool_half, nblk;
  int seg, nseg;   // keys per segment, segments per head
  bool vec4;       // P rows are 16-byte aligned (n % 4 == 0): vector loads
  uint32_t* hist;  // [Hkv][kHistStride]: hist1, hist2, candidate count (zeroed by init)
  SelState* st;    // [Hkv]
  uint2* cand;     // [Hkv][n]: (key, index) of the candidates
  uint32_t* seg_lt;   // [Hkv][nseg]: keys below digit 1's bin
  int64_t* seg_off;   // [Hkv][nseg][2]: output offset, tau-equal keys before the segment
  int32_t* status;
  FoldInfo fold;      // argmax terms of flagged rows to add to S (flagcount null: none)
};

__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? 0u : b;  // -0 (and any negative) sorts as +0
}

// Exclusive prefix sum over a workgroup of T threads; also returns the total.
template <int T>
__device__ __forceinline__ int64_t wg_exclusive_scan(int64_t x, int64_t* wsum, int64_t& total) {
  constexpr int NWV = T / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int64_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  int64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    const int64_t s = wsum[i];
    before += (i < wid) ? s : 0;
    tot += s;
  }
  total = tot;
  __syncthreads();
  return before + v - x;
}

// Bin of a histogram holding the key of 1-based rank `rank`, and the rank
// inside that bin, from the counts c[] of bins threadIdx.x * PER + i (loaded
// by the caller); the result is in *bin / *rin for every thread on return.
template <int T, int PER>
__device__ __forceinline__ void find_bin_regs(const uint32_t (&c)[PER], int64_t rank, int64_t* wsum, int* bin,
                                              int64_t* rin) {
  int64_t loc = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) loc += c[i];
  int64_t total;
  const int64_t before = wg_exclusive_scan<T>(loc, wsum, total);
  if (before < rank && rank <= before + loc) {
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
  __shared__ int64_t wsum[kT / 64];
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
  int64_t total;
  const int64_t before = wg_exclusive_scan<kT>(nc, wsum, total);
  if (threadIdx.x == 0 && total > 0) sh_base = atomicAdd(gh + kBins1 + kBins2, (uint32_t)total);
  __syncthreads();
  if (nc > 0) {
    uint2* cg = A.cand + (size_t)g * A.n;
    uint32_t pos = sh_base + (uint32_t)before;
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

// tau, need and the per-segment output offsets of one head.
constexpr int kCandRegs = 8;  // candidates per thread held in registers (else re-read)

__global__ __launch_bounds__(kFT) void k_sel_tau(SelArgs A) {
  const int g = blockIdx.x;
  __shared__ uint32_t slt[kMaxSeg];
  __shared__ uint32_t seq[kMaxSeg];
  __shared__ uint32_t hist3[kBins3];
  __shared__ int64_t wsum[kFT / 64];
  __shared__ int sh_bin;
  __shared__ int64_t sh_rin;
  const uint32_t* gh = A.hist + (size_t)g * kHistStride;
  const uint32_t* sl = A.seg_lt + (size_t)g * A.nseg;
  const uint2* cg = A.cand + (size_t)g * A.n;
  // every load that does not depend on tau, issued together
  uint32_t c1[kBins1 / kFT], c2[kBins2 / kFT];
  load_bins<kFT, kBins1>(gh, c1);
  load_bins<kFT, kBins2>(gh + kBins1, c2);
  const uint32_t nc = gh[kBins1 + kBins2];
  uint32_t lts[kMaxSeg / kFT];
#pragma unroll
  for (int i = 0; i < kMaxSeg / kFT; ++i) {
    const int sg = threadIdx.x + i * kFT;
    lts[i] = sg < A.nseg ? sl[sg] : 0u;
  }
  const bool in_regs = nc <= (uint32_t)(kCandRegs * kFT);
  uint2 cr[kCandRegs];
#pragma unroll
  for (int i = 0; i < kCandRegs; ++i) {
    const uint32_t ci = threadIdx.x + i * kFT;
    cr[i] = (in_regs && ci < nc) ? cg[ci] : make_uint2(0xffffffffu, 0u);
  }
  for (int i = threadIdx.x; i < kBins3; i += kFT) hist3[i] = 0;
#pragma unroll
  for (int i = 0; i < kMaxSeg / kFT; ++i) {
    const int sg = threadIdx.x + i * kFT;
    if (sg < A.nseg) {
      slt[sg] = lts[i];
      seq[sg] = 0;
    }
  }
  find_bin_regs<kFT, kBins1 / kFT>(c1, A.n_evict, wsum, &sh_bin, &sh_rin);
  const uint32_t d1 = (uint32_t)sh_bin;
  find_bin_regs<kFT, kBins2 / kFT>(c2, sh_rin, wsum, &sh_bin, &sh_rin);
  const uint32_t d2 = (uint32_t)sh_bin;
  const int64_t r2 = sh_rin;
  auto digit3 = [&](uint32_t key) {
    if (key != 0xffffffffu && ((key >> 8) & 0xfffu) == d2) atomicAdd(&hist3[key & 0xffu], 1u);
  };
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kCandRegs; ++i) digit3(cr[i].x);
  } else {
    for (uint32_t i = threadIdx.x; i < nc; i += kFT) digit3(cg[i].x);
  }
  __syncthreads();
  uint32_t c3[1];
  c3[0] = threadIdx.x < kBins3 ? hist3[threadIdx.x] : 0u;
  find_bin_regs<kFT, 1>(c3, r2, wsum, &sh_bin, &sh_rin);
  const uint32_t tau = (d1 << 20) | (d2 << 8) | (uint32_t)sh_bin;
  const int64_t need = sh_rin;
  if (threadIdx.x == 0) {
    A.st[g].tau = tau;
    A.st[g].need = need;
  }
  // per-segment counts: below tau = below digit 1's bin + candidates below tau
  auto fix = [&](uint2 c) {
    if (c.x == 0xffffffffu) return;
    const int sg = (int)(c.y / (uint32_t)A.seg);
    if (c.x < tau) atomicAdd(&slt[sg], 1u);
    else if (c.x == tau) atomicAdd(&seq[sg], 1u);
  };
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kCandRegs; ++i) fix(cr[i]);
  } else {
    for (uint32_t i = threadIdx.x; i < nc; i += kFT) fix(cg[i]);
  }
  __syncthreads();
  // thread t owns segments [t spt, (t+1) spt): offsets by one workgroup scan
  const int spt = (A.nseg + kFT - 1) / kFT;
  const int s0 = threadIdx.x * spt;
  int64_t l = 0, e = 0;
  for (int sg = s0; sg < s0 + spt && sg < A.nseg; ++sg) {
    l += slt[sg];
    e += seq[sg];
  }
  int64_t tot;
  // both counts are below 2^31: one scan of (eq << 32 | lt)
  const int64_t pk = wg_exclusive_scan<kFT>((e << 32) | l, wsum, tot);
  int64_t lb = pk & 0xffffffffLL, eb = pk >> 32;
  int64_t* so = A.seg_off + (size_t)g * A.nseg * 2;
  for (int sg = s0; sg < s0 + spt && sg < A.nseg; ++sg) {
    const int64_t taken_eq = eb < need ? eb : need;
    so[2 * sg] = lb + taken_eq;
    so[2 * sg + 1] = eb;
    lb += slt[sg];
    eb += seq[sg];
  }
}

// Writes the evicted indices of each segment, in index order.
__global__ __launch_bounds__(kT) void k_sel_write(SelArgs A) {
  const int g = blockIdx.y;
  const int s = blockIdx.x * kT + threadIdx.x;
  if (s >= A.nseg) return;
  const uint32_t tau = A.st[g].tau;
  const int64_t need = A.st[g].need;
  const int64_t* so = A.seg_off + ((size_t)g * A.nseg + s) * 2;
  int64_t pos = so[0], eqb = so[1];
  const float* Pg = A.P + (size_t)g * A.n;
  int64_t* og = A.idx + (size_t)g * A.n_evict;
  const int64_t j0 = (int64_t)s * A.seg;
  const int64_t j1 = (j0 + A.seg < A.n) ? j0 + A.seg : A.n;
  for (int64_t c0 = j0; c0 < j1; c0 += 16) {
    uint32_t key[16];
    load16(Pg, c0, j1, A.vec4, key);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      bool take = key[e] < tau;
      if (key[e] == tau) {
        take = eqb < need;
        ++eqb;
      }
      if (take) {
        if (pos < A.n_evict) og[pos] = c0 + e;
        ++pos;
      }
    }
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
  SelState* st;
  uint2* cand;
  uint32_t* seg_lt;
  int64_t* seg_off;
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
  r.st = (SelState*)take(sizeof(SelState) * (size_t)Hkv);
  r.cand = (uint2*)take(sizeof(uint2) * (size_t)Hkv * (size_t)n);
  r.seg_lt = (uint32_t*)take(sizeof(uint32_t) * (size_t)Hkv * q.nseg);
  r.seg_off = (int64_t*)take(sizeof(int64_t) * 2 * (size_t)Hkv * q.nseg);
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
  A.st = p.st;
  A.cand = p.cand;
  A.seg_lt = p.seg_lt;
  A.seg_off = p.seg_off;
  A.status = status;
  if (fold) A.fold = *fold;
  k_sel_pool<<<dim3(A.nblk, Hkv), kT, 0, st>>>(A);
  if (n_evict > 0) {
    const dim3 gs((q.nseg + kT - 1) / kT, Hkv);
    k_sel_cand<<<gs, kT, 0, st>>>(A);
    k_sel_tau<<<Hkv, kFT, 0, st>>>(A);
    k_sel_write<<<gs, kT, 0, st>>>(A);
  }
  return hipGetLastError();
}

}  // namespace dropkv
