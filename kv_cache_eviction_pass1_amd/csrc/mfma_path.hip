// MFMA DropKV path for bf16 inputs with head dim 128 on gfx950 (CDNA4).
//
// What is computed (DropKV write-up, section 核心公式: p = softmax(Kq/sqrt d),
// a = sum_j p_j v_j, Delta_j = p_j/(1-p_j)(a - v_j), s_j = sum over the
// window queries of ||Delta_j||^2; GQA mean per physical KV head):
//
//  pass 1  (k_pass1)  per (token chunk, KV head): flash-style streaming of
//          K/V tiles through LDS. X^T = K Q^T and O^T += V^T P^T run on
//          v_mfma_f32_32x32x16_bf16; the softmax is online (running max m,
//          sum l = sum 2^{(x-m) c}) in fp32, so the w x n attention matrix is
//          never stored. Writes per-chunk partials (m, l, A, tile of the max)
//          and ||v_j||^2.
//  merge   (k_merge)  combines the chunk partials per window row: m, l, a,
//          a in bf16, ||a_bf16||^2, the exponent bias m c + log2 l so that
//          p_j = 2^{x_j c - bias}, and flags rows with l < 2 (R < 1, i.e.
//          p_max > 1/2), locating their argmax.
//  fix-up  (k_fixup, k_fold) for flagged rows only: the argmax term from
//          D = sum_{i != j*} p_i (v_i - v_{j*}) summed directly, so that
//          neither 1 - p_{j*} nor a - v_{j*} cancels; rejects rows with
//          R <= 2^-24 (a probability that rounds to 1).
//  pass 2  (k_pass2)  per (token chunk, KV head): X = Q K^T and C = a V^T on
//          MFMA again; per element p = 2^{x c - bias}, r = p/(1-p), and
//          r^2 ||a - v_j||^2 with ||a - v_j||^2 = ||a||^2 - 2 a.v_j + ||v_j||^2
//          (the MFMA accumulator starts at -||a||^2/2). Each lane owns one
//          token and accumulates over its rows in registers.
//
// Layout conventions (32x32x16 bf16 MFMA): for both operands lane l holds
// row/column l%32 and the eight k-values 8*(l/32)..+7; the 32x32 fp32 result
// gives lane l column l%32 and rows 8*(v/4) + 4*(l/32) + v%4, v = 0..15.
// K/V tiles live in LDS as 64 rows of 256 bytes with the 16-byte chunks of
// row t XOR-permuted by swz(t) (bank-conflict free for both the 16-byte
// operand reads and the transposing 8-byte reads on gfx950's 64-bank LDS).
#include "dropkv_common.h"

namespace dropkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;                  // head dim of this path
constexpr int TT = 64;                   // tokens per LDS tile
constexpr int TILE_BYTES = TT * HD * 2;  // 16 KiB per tensor per tile
constexpr int MAXW = 8;                  // waves per workgroup (row blocks of 32)
constexpr int PSTRIDE = HD + 4;          // floats per pass-1 partial (A[128], m, l, best, pad)
constexpr int FXC = 8;                   // token chunks of the fix-up pass
constexpr int FXSTRIDE = HD + 2;         // floats per fix-up partial (sp, ps, D[128])

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_cvoid;

// Chunk permutation of token row t: a bijection on t mod 16 (16 consecutive
// rows read with ds_read_b128 hit 16 distinct 16-byte bank groups) whose top
// two bits differ within every aligned group of 4 rows (the 32 lanes of a
// ds_read_b64_tr_b16 read 4 rows x 64 bytes from 16 distinct bank groups).
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

// byte offset of element d of token row t inside a swizzled tile
__device__ __forceinline__ int toff(int t, int d) {
  return t * 256 + ((((d >> 3) ^ swz(t)) & 15) << 4) + ((d & 7) << 1);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// x[l] op x[l ^ 32] for a symmetric op, via v_permlane32_swap
__device__ __forceinline__ float pair_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ bf16x8 ld16(const char* p) { return *(const bf16x8*)p; }

// Wait until this wave's direct-to-LDS loads have landed, then barrier: after
// it every wave may read the tile. (s_waitcnt vmcnt(0); the compiler does not
// reliably order LDS-DMA completion before the workgroup barrier by itself.)
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
}

__device__ __forceinline__ bf16x8 tr_pair(const char* p0, const char* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
  union { s16x4 h[2]; bf16x8 v; } u;
  u.h[0] = lo;
  u.h[1] = hi;
  return u.v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Issue direct-to-LDS loads of one 64-token tile of one tensor: 16 wave
// instructions of 1 KiB (4 token rows each); instruction `inst` of `nw` waves.
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ head, int64_t tok0, int64_t n,
                                           char* lds, int wave, int nw, int lane) {
  for (int inst = wave; inst < 16; inst += nw) {
    const int row = inst * 4 + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    int64_t tok = tok0 + row;
    if (tok >= n) tok = n - 1;  // clamped rows are masked out by the consumers
    const uint16_t* gp = head + tok * HD + c * 8;
    __builtin_amdgcn_global_load_lds((gbl_cvoid*)gp, (lds_void*)(lds + inst * 1024), 16, 0, 0);
  }
}

// ---------------------------------------------------------------------------- pass 1

struct P1Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t n;
  int w, Rg, nw, tiles_per_chunk, Hkv;
  float c2;          // log2(e) / sqrt(d)
  float* part;       // [chunk][Hkv*Rg][PSTRIDE]
  float* nv;         // [Hkv][n]
};

// ||v_j||^2 of one LDS tile, 8 threads per token (row group 0 writes them)
__device__ __forceinline__ void p1_vnorms(const P1Args& A, const char* vb, int64_t tokbase_tile,
                                          int g, int64_t chunk_end) {
  const int nthr = A.nw * 64;
  for (int tt = threadIdx.x >> 3; tt < TT; tt += nthr >> 3) {
    const int sl = threadIdx.x & 7;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int d0 = sl * 16 + c * 8;
      const uint4 raw = *(const uint4*)(vb + toff(tt, d0));
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(wv[e] << 16), hi = __uint_as_float(wv[e] & 0xffff0000u);
        acc = fmaf(lo, lo, acc);
        acc = fmaf(hi, hi, acc);
      }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    const int64_t tok = tokbase_tile + tt;
    if (sl == 0 && tok < chunk_end) A.nv[(size_t)g * A.n + tok] = acc;
  }
}

// One 64-token tile of pass 1 for this wave's 32 rows (S^T layout: lane = row).
__device__ __forceinline__ void p1_tile(const P1Args& A, const char* kb, const char* vb,
                                        int64_t tokbase_tile, int lane, int64_t pos,
                                        const bf16x8 (&qb)[8], float& m_run, float& l_run, int& best,
                                        f32x16 (&O)[4]) {
  const int h = lane >> 5, l32 = lane & 31;
  const int gi = lane >> 4, srcl = lane & 15;
  const int dh = gi & 1;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const char* kt = kb + sub * 32 * 256;
    const char* vt = vb + sub * 32 * 256;
    bf16x8 ka[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[ks] = ld16(kt + toff(l32, ks * 16 + h * 8));
    f32x16 x = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) x = mfma(ka[ks], qb[ks], x);
    const int64_t tokbase = tokbase_tile + sub * 32;
    if (tokbase + 31 > A.n - A.w) {  // causal tail / ragged end: mask invisible keys
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int64_t tok = tokbase + (vv >> 2) * 8 + 4 * h + (vv & 3);
        if (tok > pos) x[vv] = -INFINITY;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int vv = 1; vv < 16; ++vv) mx = fmaxf(mx, x[vv]);
    mx = pair_max(mx);
    const bool up = mx > m_run;
    if (up) best = (int)(tokbase >> 5);
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float m_new = up ? mx : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * A.c2);
      if (up) {
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) O[db] *= alpha;
      }
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * A.c2;
    float e[16];
    float ls = 0.f;
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      e[vv] = __builtin_amdgcn_exp2f(fmaf(x[vv], A.c2, -mc));
      ls += e[vv];
    }
    l_run += ls;
    bf16x8 pb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[s][i] = (__bf16)e[8 * s + i];
    // O^T[d][row] += V^T[d][tok] P^T[tok][row]; k-slot 8h+i of step s is token
    // 16s + 8(i/4) + 4h + i%4 (the order in which X^T left the values in this lane)
    bf16x8 va[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int t0 = 16 * s + 4 * h + (srcl >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + 16 * dh + 4 * (srcl & 3);
        va[s][db] = tr_pair(vt + toff(t0, d), vt + toff(t0 + 8, d));
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db] = mfma(va[s][db], pb[s], O[db]);
  }
}

template <int N>
__device__ __forceinline__ void p1_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void p1_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_pass1(P1Args A) {
  __shared__ __attribute__((aligned(1024))) char kbuf[3][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf[3][TILE_BYTES];
  constexpr int kDmaPerTile = 32 / NW;  // direct-to-LDS instructions per wave per tile
  const int chunk = blockIdx.x, rg = blockIdx.y, g = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int rb = rg * NW + wave;
  const int row = rb * 32 + l32;
  const bool active = rb * 32 < A.Rg;
  const bool row_ok = row < A.Rg;
  const int64_t t0 = (int64_t)chunk * A.tiles_per_chunk * TT;
  int64_t t1 = t0 + (int64_t)A.tiles_per_chunk * TT;
  if (t1 > A.n) t1 = A.n;
  const int ntiles = (int)((t1 - t0 + TT - 1) / TT);
  const uint16_t* kh = A.k + (size_t)g * A.n * HD;
  const uint16_t* vh = A.v + (size_t)g * A.n * HD;
  const int64_t pos = A.n - A.w + ((row_ok ? row : 0) % A.w);

  bf16x8 qb[8];
  {
    const uint16_t* qr = A.q + ((size_t)g * A.Rg + (row_ok ? row : 0)) * HD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 t = *(const bf16x8*)(qr + ks * 16 + h * 8);
      if (!row_ok) t = bf16x8{};
      qb[ks] = t;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  int best = -1;
  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};

  if (ntiles > 0) {
    issue_tile(kh, t0, A.n, kbuf[0], wave, NW, lane);
    issue_tile(vh, t0, A.n, vbuf[0], wave, NW, lane);
  }
  if (ntiles > 1) {
    issue_tile(kh, t0 + TT, A.n, kbuf[1], wave, NW, lane);
    issue_tile(vh, t0 + TT, A.n, vbuf[1], wave, NW, lane);
  }
  // Per iteration the vector-memory ops are, in issue order: ||v||^2 stores of
  // tile t, then the loads of tile t+2; so `vmcnt <= one tile's loads` at the
  // top of iteration t+1 means tile t+1 has landed.
  for (int t = 0; t < ntiles; ++t) {
    const int64_t tb = t0 + (int64_t)t * TT;
    if (t + 1 < ntiles) p1_wait_vmcnt<kDmaPerTile>(); else p1_wait_vmcnt<0>();
    p1_lds_barrier();  // tile t in LDS for every wave; tile t-1's buffer is free
    const char* kc = kbuf[t % 3];
    const char* vc = vbuf[t % 3];
    if (rg == 0) p1_vnorms(A, vc, tb, g, t1);
    if (t + 2 < ntiles) {
      const int nb = (t + 2) % 3;
      issue_tile(kh, tb + 2 * TT, A.n, kbuf[nb], wave, NW, lane);
      issue_tile(vh, tb + 2 * TT, A.n, vbuf[nb], wave, NW, lane);
    }
    if (active) p1_tile(A, kc, vc, tb, lane, pos, qb, m_run, l_run, best, O);
  }
  if (!active) return;
  const float l_tot = pair_sum(l_run);
  if (!row_ok) return;
  float* pr = A.part + ((size_t)chunk * A.Hkv * A.Rg + (size_t)g * A.Rg + row) * PSTRIDE;
  // lane holds O^T rows d = 32db + 8i + 4h + (0..3) of this row's column
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 o = {O[db][4 * i], O[db][4 * i + 1], O[db][4 * i + 2], O[db][4 * i + 3]};
      *(float4*)(pr + 32 * db + 8 * i + 4 * h) = o;
    }
  if (h == 0) {
    pr[HD] = m_run;
    pr[HD + 1] = l_tot;
    pr[HD + 2] = __int_as_float(best);
  }
}

// ---------------------------------------------------------------------------- merge

struct MergeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* part;
  int64_t n;
  int w, Rg, Hkv, nchunks;
  float c2, inv_sqrt_d;
  RowStats rs;
  int32_t* flagcount;  // [Hkv]
  int32_t* status;
};

// One wave per window row; lane owns d = 2*lane, 2*lane+1.
__global__ __launch_bounds__(256) void k_merge(MergeArgs M) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)M.Hkv * M.Rg;
  if (row >= rows) return;
  const int g = (int)(row / M.Rg), r = (int)(row % M.Rg);
  const size_t cstride = (size_t)rows * PSTRIDE;
  const float* prow = M.part + (size_t)row * PSTRIDE;
  // lane c (< 64) holds chunk c's (m, l, best); more chunks fold in 64 at a time
  float mx = -INFINITY;
  int bt = -1;
  for (int c0 = 0; c0 < M.nchunks; c0 += 64) {
    const int c = c0 + lane;
    const float mc = c < M.nchunks ? prow[c * cstride + HD] : -INFINITY;
    float wm = mc;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
    if (wm > mx) {
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(mc == wm);
      const int first = __ffsll((long long)hit) - 1;  // lowest chunk attaining the max
      const float bf = c < M.nchunks ? prow[c * cstride + HD + 2] : 0.f;
      bt = __float_as_int(__shfl(bf, first, 64));
      mx = wm;
    }
  }
  float l = 0.f, a0 = 0.f, a1 = 0.f;
  for (int c0 = 0; c0 < M.nchunks; c0 += 64) {
    const int c = c0 + lane;
    const float mc = c < M.nchunks ? prow[c * cstride + HD] : -INFINITY;
    const float lc = c < M.nchunks ? prow[c * cstride + HD + 1] : 0.f;
    const float sc = (mc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mc - mx) * M.c2);
    float lw = lc * sc;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lw += __shfl_xor(lw, o, 64);
    l += lw;
    const int cn = (M.nchunks - c0) < 64 ? (M.nchunks - c0) : 64;
    int cc = 0;
    for (; cc + 8 <= cn; cc += 8) {
      float2 av[8];
      float sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        av[u] = *(const float2*)(prow + (size_t)(c0 + cc + u) * cstride + 2 * lane);
        sv[u] = __shfl(sc, cc + u, 64);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a0 = fmaf(av[u].x, sv[u], a0);
        a1 = fmaf(av[u].y, sv[u], a1);
      }
    }
    for (; cc < cn; ++cc) {
      const float2 av = *(const float2*)(prow + (size_t)(c0 + cc) * cstride + 2 * lane);
      const float sv = __shfl(sc, cc, 64);
      a0 = fmaf(av.x, sv, a0);
      a1 = fmaf(av.y, sv, a1);
    }
  }
  const float inv_l = 1.0f / l;
  const float x0 = a0 * inv_l, x1 = a1 * inv_l;
  const uint16_t b0 = f32_to_bf16_rne(x0), b1 = f32_to_bf16_rne(x1);
  const float f0 = bf16_to_f32(b0), f1 = bf16_to_f32(b1);
  float na = fmaf(f0, f0, f1 * f1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) na += __shfl_xor(na, o, 64);
  *(float2*)(M.rs.a + (size_t)row * HD + 2 * lane) = make_float2(x0, x1);
  *(uint32_t*)(M.rs.a_bf + (size_t)row * HD + 2 * lane) = (uint32_t)b0 | ((uint32_t)b1 << 16);
  bool bad = !finite_f(mx) || !finite_f(l) || !finite_f(x0) || !finite_f(x1);
  bad = __builtin_amdgcn_ballot_w64(bad) != 0;
  const bool flagged = (l < 2.0f) && !bad;
  int js = -1;
  if (flagged) {
    // lowest-index argmax inside the 32-token block where the running max was set
    const int64_t pos = M.n - M.w + (r % M.w);
    const int64_t tok = (int64_t)bt * 32 + (lane & 31);
    float x = -INFINITY;
    if (lane < 32 && tok <= pos && tok >= 0) {
      const uint16_t* qr = M.q + (size_t)row * HD;
      const uint16_t* kr = M.k + ((size_t)g * M.n + tok) * HD;
      float acc = 0.f;
      for (int c = 0; c < HD; ++c) acc = fmaf(bf16_to_f32(qr[c]), bf16_to_f32(kr[c]), acc);
      x = acc;
    }
    int jt = (x == -INFINITY) ? 0x7fffffff : (int)tok;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float xo = __shfl_xor(x, o, 64);
      const int jo = __shfl_xor(jt, o, 64);
      if (xo > x || (xo == x && jo < jt)) { x = xo; jt = jo; }
    }
    js = (jt == 0x7fffffff) ? -1 : jt;
  }
  if (lane == 0) {
    M.rs.m[row] = mx * M.inv_sqrt_d;
    M.rs.L[row] = l;
    M.rs.rest[row] = l - 1.0f;
    M.rs.na[row] = na;
    M.rs.bias[row] = mx * M.c2 + __log2f(l);
    M.rs.jstar[row] = js;
    M.rs.flag[row] = flagged ? 1 : 0;
    M.rs.fixval[row] = 0.f;
    if (bad) atomicOr(M.status, kStatusNonFinite);
    else if (flagged) atomicAdd(&M.flagcount[g], 1);
  }
}

// ---------------------------------------------------------------------------- fix-up

struct FixArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t n;
  int w, Rg, Hkv;
  float c2;
  RowStats rs;
  const int32_t* flagcount;
  float* fx;  // [FXC][Hkv*Rg][FXSTRIDE]
};

// Per flagged row and token chunk: sp = sum_{i != j*} p_i, ps = p_{j*} and
// D = sum_{i != j*} p_i (v_i - v_{j*}), with p_i = 2^{x_i c - bias}.
__global__ __launch_bounds__(256) void k_fixup(FixArgs F) {
  const int c = blockIdx.x, g = blockIdx.y;
  if (F.flagcount[g] == 0) return;
  const int tid = threadIdx.x;
  __shared__ float qs[HD], vstar[HD], ptile[256], red[256], redD[256];
  const int64_t cs = (F.n + FXC - 1) / FXC;
  const int64_t c0 = c * cs;
  const int64_t c1 = (c0 + cs < F.n) ? c0 + cs : F.n;
  for (int r = 0; r < F.Rg; ++r) {
    const int64_t row = (int64_t)g * F.Rg + r;
    if (!F.rs.flag[row]) continue;
    const int js = F.rs.jstar[row];
    if (js < 0 || js >= F.n) continue;
    const float bias = F.rs.bias[row];
    const int64_t pos = F.n - F.w + (r % F.w);
    const int64_t hi = (pos + 1 < c1) ? pos + 1 : c1;
    __syncthreads();
    if (tid < HD) {
      qs[tid] = bf16_to_f32(F.q[row * HD + tid]);
      vstar[tid] = bf16_to_f32(F.v[((size_t)g * F.n + js) * HD + tid]);
    }
    __syncthreads();
    float sp = 0.f, ps = 0.f, Dacc = 0.f;
    const int dim = tid & (HD - 1), sub = tid >> 7;
    for (int64_t b = c0; b < hi; b += 256) {
      const int64_t j = b + tid;
      float p = 0.f;
      if (j < hi) {
        const uint16_t* kr = F.k + ((size_t)g * F.n + j) * HD;
        float acc = 0.f;
        for (int cc = 0; cc < HD; ++cc) acc = fmaf(qs[cc], bf16_to_f32(kr[cc]), acc);
        p = __builtin_amdgcn_exp2f(fmaf(acc, F.c2, -bias));
        if (j == js) { ps = p; p = 0.f; }
        sp += p;
      }
      ptile[tid] = p;
      __syncthreads();
      const int cnt = (int)((hi - b) < 256 ? (hi - b) : 256);
      for (int t = sub; t < cnt; t += 2) {
        const float vv = bf16_to_f32(F.v[((size_t)g * F.n + b + t) * HD + dim]);
        Dacc = fmaf(ptile[t], vv - vstar[dim], Dacc);
      }
      __syncthreads();
    }
    redD[tid] = Dacc;
    const float spt = block_sum<256>(sp, red);
    const float pst = block_sum<256>(ps, red);
    float* o = F.fx + ((size_t)c * F.Hkv * F.Rg + row) * FXSTRIDE;
    if (tid < HD) o[2 + tid] = redD[tid] + redD[tid + HD];
    if (tid == 0) { o[0] = spt; o[1] = pst; }
  }
}

struct FoldArgs {
  int64_t n;
  int Rg, Hkv;
  float invG;
  RowStats rs;
  const int32_t* flagcount;
  const float* fx;
  float* S;
  int32_t* status;
};

// Adds the argmax terms of flagged rows into S, in row order (deterministic).
__global__ __launch_bounds__(HD) void k_fold(FoldArgs F) {
  const int g = blockIdx.x;
  if (F.flagcount[g] == 0) return;
  const int tid = threadIdx.x;
  __shared__ float red[HD];
  for (int r = 0; r < F.Rg; ++r) {
    const int64_t row = (int64_t)g * F.Rg + r;
    if (!F.rs.flag[row]) continue;
    float sp = 0.f, ps = 0.f, D = 0.f;
    for (int c = 0; c < FXC; ++c) {
      const float* o = F.fx + ((size_t)c * F.Hkv * F.Rg + row) * FXSTRIDE;
      sp += o[0];
      ps += o[1];
      D += o[2 + tid];
    }
    const float dn2 = block_sum<HD>(D * D, red);
    const int js = F.rs.jstar[row];
    if (tid == 0 && (js < 0 || js >= F.n)) atomicOr(F.status, kStatusNonFinite);
    if (tid == 0 && js >= 0 && js < F.n) {
      // R = sum_{i != j*} e_i / e_{j*}; ||a - v_{j*}|| = ||D|| / (ps + sp); p/(1-p) = 1/R
      const float R = sp / ps;
      const float tot = ps + sp;
      const float val = dn2 / (tot * tot) / (R * R);
      F.rs.rest[row] = R;
      F.rs.L[row] = 1.0f + R;
      F.rs.fixval[row] = val;
      if (!(ps > 0.f) || !finite_f(R)) atomicOr(F.status, kStatusNonFinite);
      else if (R <= kSingularRest) atomicOr(F.status, kStatusSingular);
      else F.S[(size_t)g * F.n + js] += val * F.invG;
    }
  }
}

// ---------------------------------------------------------------------------- pass 2

struct P2Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t n;
  int w, Rg, nw, tiles_per_chunk, Hkv;
  float c2, invG;
  RowStats rs;
  const float* nv;
  const int32_t* flagcount;
  float* S;  // [rg][Hkv][n]
};

__device__ __forceinline__ void p2_tile(const P2Args& P, const char* kb, const char* vb,
                                        int64_t tokbase_tile, int lane, bool active, int rb,
                                        const bf16x8 (&qa)[8], const bf16x8 (&aa)[8],
                                        const float (&bias)[16], const float (&cinit)[16],
                                        bool flagged, int g, float (*red)[TT][2], int wave) {
  const int h = lane >> 5, l32 = lane & 31;
  if (!active) return;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const char* kt = kb + sub * 32 * 256;
    const char* vt = vb + sub * 32 * 256;
    bf16x8 kbv[8], vbv[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kbv[ks] = ld16(kt + toff(l32, ks * 16 + h * 8));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) vbv[ks] = ld16(vt + toff(l32, ks * 16 + h * 8));
    f32x16 x = {};
    f32x16 cc;
#pragma unroll
    for (int i = 0; i < 16; ++i) cc[i] = cinit[i];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) x = mfma(qa[ks], kbv[ks], x);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) cc = mfma(aa[ks], vbv[ks], cc);
    const int64_t tok = tokbase_tile + sub * 32 + l32;
    if (tokbase_tile + sub * 32 + 31 > P.n - P.w) {
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int rr = rb * 32 + (vv >> 2) * 8 + 4 * h + (vv & 3);
        const int64_t pos = P.n - P.w + (rr % P.w);
        if (tok > pos) x[vv] = -INFINITY;
      }
    }
    float t1 = 0.f, t2 = 0.f;
    if (!flagged) {
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const float p = __builtin_amdgcn_exp2f(fmaf(x[vv], P.c2, -bias[vv]));
        const float r = p * __builtin_amdgcn_rcpf(1.0f - p);
        const float r2 = r * r;
        t2 += r2;
        t1 = fmaf(r2, cc[vv], t1);
      }
    } else {
      // some row of this KV head takes its argmax term from the fix-up
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int rr = rb * 32 + (vv >> 2) * 8 + 4 * h + (vv & 3);
        bool skip = false;
        if (rr < P.Rg) {
          const int64_t row = (int64_t)g * P.Rg + rr;
          skip = P.rs.flag[row] && (int64_t)P.rs.jstar[row] == tok;
        }
        const float p = skip ? 0.f : __builtin_amdgcn_exp2f(fmaf(x[vv], P.c2, -bias[vv]));
        const float r = p * __builtin_amdgcn_rcpf(1.0f - p);
        const float r2 = r * r;
        t2 += r2;
        t1 = fmaf(r2, cc[vv], t1);
      }
    }
    t1 = pair_sum(t1);
    t2 = pair_sum(t2);
    if (h == 0) {
      red[wave][sub * 32 + l32][0] = t1;
      red[wave][sub * 32 + l32][1] = t2;
    }
  }
}

__device__ __forceinline__ void p2_combine(const P2Args& P, float (*red)[TT][2], int nwa,
                                           int64_t tokbase_tile, int64_t chunk_end, int g) {
  if (threadIdx.x < TT) {
    const int64_t tok = tokbase_tile + threadIdx.x;
    if (tok < chunk_end) {
      float T1 = 0.f, T2 = 0.f;
      for (int wv = 0; wv < nwa; ++wv) {
        T1 += red[wv][threadIdx.x][0];
        T2 += red[wv][threadIdx.x][1];
      }
      // sum_rows r^2 (||a||^2 - 2 a.v + ||v||^2) = ||v||^2 T2 - 2 T1
      const float nvj = P.nv[(size_t)g * P.n + tok];
      const float s = fmaxf(fmaf(nvj, T2, -2.0f * T1), 0.0f) * P.invG;
      P.S[((size_t)blockIdx.y * P.Hkv + g) * P.n + tok] = s;
    }
  }
}

// ---- pass 2, fast path
//
// A workgroup has NW waves (2 per SIMD at NW = 8); each wave owns one 32-row
// block and walks its chunk in 32-token subtiles. K/V tiles of 64 tokens are
// triple-buffered in LDS (two tiles in flight). Per subtile the wave runs
// X = Q K^T and C = a V^T on MFMA (the accumulator of C starts at
// -||a||^2/2) and then the score VALU, in one of three forms chosen per
// subtile by a wave vote on the largest p = 2^{x c - bias}:
//   p < 2^-12 everywhere: r^2 = p^2 (1 + 2p + ...) is taken as 2^{2(x c - bias)}
//                          (relative error < 2p < 5e-4);
//   p < 2^-7  everywhere: r^2 = p^2 (1 + 2p + 3p^2) (error 4p^3 < 2e-6);
//   otherwise:            r^2 = (p / (1 - p))^2 with a reciprocal.

enum { kTierSquare = 0, kTierSeries = 1, kTierExact = 2 };

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS traffic only. __syncthreads() would also
// wait for every outstanding vector-memory operation (vmcnt(0)), including
// the direct-to-LDS loads of tiles still in flight; callers wait for the tile
// they need with wait_vmcnt<N>() first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ||v||^2 of the 64 tokens of a tile into LDS (one 4-byte direct-to-LDS load per lane)
__device__ __forceinline__ void issue_nv(const float* nvh, int64_t tok0, int64_t n, float* lds, int lane) {
  int64_t tok = tok0 + lane;
  if (tok >= n) tok = n - 1;
  __builtin_amdgcn_global_load_lds((gbl_cvoid*)(nvh + tok), (lds_void*)lds, 4, 0, 0);
}

template <int TIER>
__device__ __forceinline__ void p2_values(const f32x16& X, const f32x16& C, const float (&bias)[16],
                                          float c2, float& t1, float& t2) {
  float a1 = 0.f, a2 = 0.f;
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) {
    const float y = fmaf(X[vv], c2, -bias[vv]);
    float r2;
    if (TIER == kTierSquare) {
      r2 = __builtin_amdgcn_exp2f(y + y);
    } else {
      const float p = __builtin_amdgcn_exp2f(y);
      if (TIER == kTierSeries) {
        r2 = (p * p) * fmaf(p, fmaf(p, 3.0f, 2.0f), 1.0f);
      } else {
        const float r = p * __builtin_amdgcn_rcpf(1.0f - p);
        r2 = r * r;
      }
    }
    a2 += r2;
    a1 = fmaf(r2, C[vv], a1);
  }
  t1 = a1;
  t2 = a2;
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_pass2(P2Args P) {
  __shared__ __attribute__((aligned(1024))) char kbuf[3][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf[3][TILE_BYTES];
  __shared__ float red3[3][NW][TT];
  __shared__ float nvbuf[3][TT];
  constexpr int kDmaPerTile = 32 / NW + 1;  // direct-to-LDS instructions per wave per tile
  const int chunk = blockIdx.x, rg = blockIdx.y, g = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int rb = rg * NW + wave;
  const bool active = rb * 32 < P.Rg;
  int nwa = (P.Rg - rg * NW * 32 + 31) / 32;  // active waves
  if (nwa > NW) nwa = NW;
  const int64_t t0 = (int64_t)chunk * P.tiles_per_chunk * TT;
  int64_t t1 = t0 + (int64_t)P.tiles_per_chunk * TT;
  if (t1 > P.n) t1 = P.n;
  const int ntiles = (int)((t1 - t0 + TT - 1) / TT);
  const uint16_t* kh = P.k + (size_t)g * P.n * HD;
  const uint16_t* vh = P.v + (size_t)g * P.n * HD;
  const float* __restrict__ nvg = P.nv + (size_t)g * P.n;
  float* __restrict__ Sout = P.S + ((size_t)blockIdx.y * P.Hkv + g) * P.n;
  const bool flagged = P.flagcount[g] != 0;

  bf16x8 qa[8], aa[8];
  float bias[16], cinit[16];
  {
    const int row = rb * 32 + l32;
    const bool ok = row < P.Rg;
    const size_t grow = (size_t)g * P.Rg + (ok ? row : 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 tq = *(const bf16x8*)(P.q + grow * HD + ks * 16 + h * 8);
      bf16x8 ta = *(const bf16x8*)(P.rs.a_bf + grow * HD + ks * 16 + h * 8);
      if (!ok) { tq = bf16x8{}; ta = bf16x8{}; }
      qa[ks] = tq;
      aa[ks] = ta;
    }
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      const int rr = rb * 32 + (vv >> 2) * 8 + 4 * h + (vv & 3);
      const bool okr = rr < P.Rg;
      const size_t gr = (size_t)g * P.Rg + (okr ? rr : 0);
      bias[vv] = okr ? P.rs.bias[gr] : INFINITY;
      cinit[vv] = okr ? -0.5f * P.rs.na[gr] : 0.f;
    }
  }

  if (ntiles > 0) {
    issue_tile(kh, t0, P.n, kbuf[0], wave, NW, lane);
    issue_tile(vh, t0, P.n, vbuf[0], wave, NW, lane);
  }

  if (flagged) {
    // per-tile path with the argmax exclusion of flagged rows (double-buffered)
    float (*red)[TT][2] = (float (*)[TT][2])&red3[0][0][0];
    static_assert(3 * NW * TT >= NW * TT * 2, "reduction buffer");
    for (int it = 0; it < ntiles; ++it) {
      const int b = it & 1;
      tile_barrier();
      if (it + 1 < ntiles) {
        issue_tile(kh, t0 + (int64_t)(it + 1) * TT, P.n, kbuf[b ^ 1], wave, NW, lane);
        issue_tile(vh, t0 + (int64_t)(it + 1) * TT, P.n, vbuf[b ^ 1], wave, NW, lane);
      }
      p2_tile(P, kbuf[b], vbuf[b], t0 + (int64_t)it * TT, lane, active, rb, qa, aa, bias, cinit,
              true, g, red, wave);
      __syncthreads();
      p2_combine(P, red, nwa, t0 + (int64_t)it * TT, t1, g);
    }
    return;
  }

  // the fast path's only vector-memory loads are the direct-to-LDS tile loads
  // (K, V and ||v||^2), so `vmcnt <= one tile's loads` means the older tile landed
  if (ntiles > 0) issue_nv(nvg, t0, P.n, nvbuf[0], lane);
  if (ntiles > 1) {
    issue_tile(kh, t0 + TT, P.n, kbuf[1], wave, NW, lane);
    issue_tile(vh, t0 + TT, P.n, vbuf[1], wave, NW, lane);
    issue_nv(nvg, t0 + TT, P.n, nvbuf[1], lane);
  }
  const float c2 = P.c2;
  for (int t = 0; t < ntiles; ++t) {
    const int64_t tb = t0 + (int64_t)t * TT;
    if (t + 1 < ntiles) wait_vmcnt<kDmaPerTile>(); else wait_vmcnt<0>();
    lds_barrier();  // tile t in LDS for every wave; tile t-1's buffer is free
    if (t >= 1 && threadIdx.x < TT) {
      // scores of tile t-1 (all waves wrote their partials before this barrier)
      const int64_t tok = tb - TT + threadIdx.x;
      if (tok < t1) {
        float sacc = 0.f;
        for (int wv = 0; wv < nwa; ++wv) sacc += red3[(t - 1) % 3][wv][threadIdx.x];
        Sout[tok] = fmaxf(sacc, 0.0f) * P.invG;
      }
    }
    if (t + 2 < ntiles) {
      const int nb = (t + 2) % 3;
      issue_tile(kh, tb + 2 * TT, P.n, kbuf[nb], wave, NW, lane);
      issue_tile(vh, tb + 2 * TT, P.n, vbuf[nb], wave, NW, lane);
      issue_nv(nvg, tb + 2 * TT, P.n, nvbuf[nb], lane);
    }
    if (active) {
      const char* kc = kbuf[t % 3];
      const char* vc = vbuf[t % 3];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const char* kt = kc + sub * 32 * 256;
        const char* vt = vc + sub * 32 * 256;
        bf16x8 kb[8], vb[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kb[ks] = ld16(kt + toff(l32, ks * 16 + h * 8));
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) vb[ks] = ld16(vt + toff(l32, ks * 16 + h * 8));
        f32x16 X = {}, C;
#pragma unroll
        for (int i = 0; i < 16; ++i) C[i] = cinit[i];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) X = mfma(qa[ks], kb[ks], X);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) C = mfma(aa[ks], vb[ks], C);
        const int64_t tok = tb + sub * 32 + l32;
        float xm = -INFINITY;
        if (tb + sub * 32 + 31 > P.n - P.w) {
#pragma unroll
          for (int vv = 0; vv < 16; ++vv) {
            const int rr = rb * 32 + (vv >> 2) * 8 + 4 * h + (vv & 3);
            if (tok > P.n - P.w + (rr % P.w)) X[vv] = -INFINITY;
          }
        }
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) xm = fmaxf(xm, fmaf(X[vv], c2, -bias[vv]));
        float q1, q2;
        if (__builtin_amdgcn_ballot_w64(xm > -7.0f))
          p2_values<kTierExact>(X, C, bias, c2, q1, q2);
        else if (__builtin_amdgcn_ballot_w64(xm > -12.0f))
          p2_values<kTierSeries>(X, C, bias, c2, q1, q2);
        else
          p2_values<kTierSquare>(X, C, bias, c2, q1, q2);
        // this wave's rows: sum r^2 (||a||^2 - 2 a.v + ||v||^2) = ||v||^2 q2 - 2 q1
        const float sw = pair_sum(fmaf(nvbuf[t % 3][sub * 32 + l32], q2, -2.0f * q1));
        if (h == 0) red3[t % 3][wave][sub * 32 + l32] = sw;
      }
    }
  }
  __syncthreads();
  if (ntiles >= 1 && threadIdx.x < TT) {
    const int tl = ntiles - 1;
    const int64_t tok = t0 + (int64_t)tl * TT + threadIdx.x;
    if (tok < t1) {
      float sacc = 0.f;
      for (int wv = 0; wv < nwa; ++wv) sacc += red3[tl % 3][wv][threadIdx.x];
      Sout[tok] = fmaxf(sacc, 0.0f) * P.invG;
    }
  }
}

// Sum of the row-group partial scores (only when a KV head has > 8 row blocks).
__global__ void k_sum_rowgroups(const float* __restrict__ Sp, float* __restrict__ S, int64_t total, int nrg) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  float s = 0.f;
  for (int r = 0; r < nrg; ++r) s += Sp[(size_t)r * total + i];
  S[i] = s;
}


struct Plan {
  int Rg, RBt, nrg, nw, tiles, tpc1, nch1, tpc2, nch2;
  int nw2, nrg2;  // pass 2: waves per workgroup (1, 2 or 4; 64 rows each) and row groups
};

Plan make_plan(const Shape& s) {
  Plan p{};
  p.Rg = s.G() * s.w;
  p.RBt = (p.Rg + 31) / 32;
  p.nw = MAXW;  // pass 1: 32 rows per wave, power-of-two waves per workgroup
  while (p.nw > 1 && p.nw / 2 >= p.RBt) p.nw /= 2;
  p.nrg = (p.RBt + p.nw - 1) / p.nw;
  p.tiles = (int)((s.n + TT - 1) / TT);
  // pass 1: about one workgroup per CU (partials cost HBM traffic)
  const int target1 = 256, target2 = 512;
  int per = s.Hkv * p.nrg;
  p.nch1 = (target1 + per - 1) / per;
  if (p.nch1 > p.tiles) p.nch1 = p.tiles;
  if (p.nch1 < 1) p.nch1 = 1;
  p.tpc1 = (p.tiles + p.nch1 - 1) / p.nch1;
  p.nch1 = (p.tiles + p.tpc1 - 1) / p.tpc1;
  // pass 2: 32 rows per wave, 8 waves (256 rows) per workgroup, or fewer waves
  // (power of two) when the KV head has fewer row blocks
  p.nw2 = 8;
  while (p.nw2 > 1 && p.nw2 / 2 >= p.RBt) p.nw2 /= 2;
  p.nrg2 = (p.RBt + p.nw2 - 1) / p.nw2;
  const int per2 = s.Hkv * p.nrg2;
  (void)target2;
  p.nch2 = (256 + per2 - 1) / per2;
  if (p.nch2 > p.tiles) p.nch2 = p.tiles;
  if (p.nch2 < 1) p.nch2 = 1;
  p.tpc2 = (p.tiles + p.nch2 - 1) / p.nch2;
  p.nch2 = (p.tiles + p.tpc2 - 1) / p.tpc2;
  return p;
}

}  // namespace

bool mfma_supported(int dtype, int d) { return dtype == 0 && d == HD; }

int mfma_chunks(const Shape& s) { return make_plan(s).nch1; }

size_t mfma_extra_bytes(const Shape& s) {
  const Plan p = make_plan(s);
  size_t b = 0;
  b += sizeof(float) * (size_t)s.Hkv * s.n;                       // ||v||^2
  b += sizeof(float) * (size_t)FXC * s.Hkv * p.Rg * FXSTRIDE;     // fix-up partials
  if (p.nrg2 > 1) b += sizeof(float) * (size_t)p.nrg2 * s.Hkv * s.n;  // row-group partial S
  return b + 4 * 256;
}

hipError_t launch_mfma_path(const void* q, const void* k, const void* v, const Shape& s,
                            const Workspace& ws, hipStream_t st, StageEvents* se) {
  const Plan p = make_plan(s);
  // carve the path's extra buffers behind the common workspace
  char* extra = (char*)ws.extra;
  auto take = [&](size_t bytes) { char* r = extra; extra += (bytes + 255) / 256 * 256; return r; };
  float* nv = (float*)take(sizeof(float) * (size_t)s.Hkv * s.n);
  float* fx = (float*)take(sizeof(float) * (size_t)FXC * s.Hkv * p.Rg * FXSTRIDE);
  int32_t* flagcount = ws.flagcount;
  float* Spart = p.nrg2 > 1 ? (float*)take(sizeof(float) * (size_t)p.nrg2 * s.Hkv * s.n) : ws.S;
  const float c2 = kLog2e / sqrtf((float)HD);

  P1Args a1{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.w, p.Rg, p.nw,
            p.tpc1, s.Hkv, c2, ws.part, nv};
  record_stage(se, "start", st);
  {
    const dim3 grid1(p.nch1, p.nrg, s.Hkv);
    switch (p.nw) {
      case 8: k_pass1<8><<<grid1, 512, 0, st>>>(a1); break;
      case 4: k_pass1<4><<<grid1, 256, 0, st>>>(a1); break;
      case 2: k_pass1<2><<<grid1, 128, 0, st>>>(a1); break;
      default: k_pass1<1><<<grid1, 64, 0, st>>>(a1); break;
    }
  }
  record_stage(se, "pass1", st);
  MergeArgs am{(const uint16_t*)q, (const uint16_t*)k, ws.part, s.n, s.w, p.Rg, s.Hkv, p.nch1,
               c2, 1.0f / sqrtf((float)HD), ws.rs, flagcount, ws.status};
  const int64_t rows = (int64_t)s.Hkv * p.Rg;
  k_merge<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(am);
  record_stage(se, "merge", st);
  FixArgs af{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.w, p.Rg, s.Hkv, c2,
             ws.rs, flagcount, fx};
  k_fixup<<<dim3(FXC, s.Hkv), 256, 0, st>>>(af);
  record_stage(se, "fixup", st);
  P2Args a2{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.w, p.Rg, p.nw2,
            p.tpc2, s.Hkv, c2, 1.0f / (float)s.G(), ws.rs, nv, flagcount, Spart};
  const dim3 grid2(p.nch2, p.nrg2, s.Hkv);
  switch (p.nw2) {
    case 8: k_pass2<8><<<grid2, 512, 0, st>>>(a2); break;
    case 4: k_pass2<4><<<grid2, 256, 0, st>>>(a2); break;
    case 2: k_pass2<2><<<grid2, 128, 0, st>>>(a2); break;
    default: k_pass2<1><<<grid2, 64, 0, st>>>(a2); break;
  }
  record_stage(se, "pass2", st);
  if (p.nrg2 > 1) {
    const int64_t total = (int64_t)s.Hkv * s.n;
    k_sum_rowgroups<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(Spart, ws.S, total, p.nrg2);
    record_stage(se, "rowgroup_sum", st);
  }
  FoldArgs ao{s.n, p.Rg, s.Hkv, 1.0f / (float)s.G(), ws.rs, flagcount, fx, ws.S, ws.status};
  k_fold<<<s.Hkv, HD, 0, st>>>(ao);
  record_stage(se, "fold", st);
  return hipGetLastError();
}

}  // namespace dropkv
