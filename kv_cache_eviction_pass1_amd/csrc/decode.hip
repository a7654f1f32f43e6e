// Decode-time rescoring: the raw DropKV score of a growing cache, kept up to
// date as tokens are appended, with the observation window sliding over the
// last w query positions.
//
// Pages: the atlas summary (Limitations) leaves a decode-time kernel to future
// work and calls per-step decode bandwidth-bound; the write-up's core formula
// (核心公式) sums ||Delta_j||^2 over the window queries and averages over the
// query heads of a KV head. A window row's terms depend only on the keys it
// sees, which appending does not change, so one step is: add the terms of the
// G new rows of each KV head (position n - 1), subtract those of the G rows
// leaving the window (position n - 1 - w).
//
// Exactness of the subtraction. The raw score is kept in fp64, and a row's
// terms are always produced by the same kernel from the same stored row state
// (query, a, exponent bias, ...), so the terms subtracted when a row leaves are
// bit for bit the ones added when it entered; the fp64 sums then cancel them
// to rounding far below fp32, however much larger they were than what stays.
//
// Kernels (bf16, d = 128):
//   k_dec_stats / k_dec_merge  new rows' attention: max logit, exact rest mass
//       R = sum_{j != argmax} 2^{x_j - m}, argmax, a (VALU; 8 lanes per token);
//       the merge also stores the rows and moves the argmax terms (below)
//   k_dec_contrib  signed terms r^2 ||a - v_j||^2 of a list of rows for every
//       token (X = Q K^T and C = a V^T on 16x16x32 MFMA, 16-token subtiles per
//       wave, K and V read straight into the MFMA operands, 64 contiguous
//       bytes per token and load), added into the fp64 score
//   argmax terms of rows with p_max > 1/2 are scored apart and kept per row,
//       so the exact value added is the one later removed. The rows live in a
//       ring of w + 1 slots per KV head (position p in slot p mod (w + 1)), so
//       the appended position never shares a slot with the one leaving.
// The first window comes from the MFMA pass 1 + merge + argmax fix-up.
#include "dropkv_common.h"
#include "decode_state.h"

namespace dropkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int HD = 128;
constexpr int kRowBatch = 8;       // new rows per k_dec_stats launch
constexpr int kDecPart = HD + 4;   // floats per stats partial (A[128], m, R, j*, pad)
constexpr int kContribRows = 64;   // rows per k_dec_contrib launch in a step (operands and tables in LDS)
constexpr int kInitRows = 128;     // rows per launch when a whole window is scored (76 KB of LDS: two workgroups per CU)
constexpr int kOpStride = HD + 8;  // bf16 per staged operand row (272 bytes)
constexpr int kTokPerWg = 512;     // tokens per k_dec_contrib workgroup (4 waves x 8 subtiles of 16)
constexpr int kStatsTok = 2048;    // tokens per k_dec_stats workgroup

__device__ __forceinline__ uint16_t rne_bf16(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// sum over the 16 lanes of a DPP row, result in every lane of the row
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));  // row_mirror
  return x;
}

// ---------------------------------------------------------------------------- row table

// Row table index of query head h (of KV head g's G) at cache position pos.
__device__ __forceinline__ int64_t trow(int g, int64_t pos, int h, int w, int G) {
  return ((int64_t)g * (w + 1) + pos % (w + 1)) * G + h;
}

// State derived from (m, L, a) once, when a row is stored: a in bf16 for the
// MFMA, C's start value -||a_bf16||^2 / 2 and the exponent bias
// m log2(e) + log2(L), so that p_j = 2^{x_j log2(e)/sqrt(d) - bias}. One wave
// per row, lane = 2 dims.
__device__ __forceinline__ void derive_row(const DecRows& T, int64_t r, float m, float L, int lane) {
  const float2 av = *(const float2*)(T.a + r * HD + 2 * lane);
  const uint16_t b0 = rne_bf16(av.x), b1 = rne_bf16(av.y);
  const float f0 = bf16_to_f32(b0), f1 = bf16_to_f32(b1);
  float na = fmaf(f0, f0, f1 * f1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) na += __shfl_xor(na, o, 64);
  *(uint32_t*)(T.a_bf + r * HD + 2 * lane) = (uint32_t)b0 | ((uint32_t)b1 << 16);
  if (lane == 0) {
    T.cinit[r] = -0.5f * na;
    T.bias[r] = m * kLog2e + __log2f(L);
  }
}

struct LoadArgs {
  const uint16_t* q;  // [Hq][w][d] window queries
  RowStats rs;        // window rows r = h * w + i
  DecRows T;
  double* S64;
  int64_t n, n_max;
  int w, Hq, Hkv;
};

// Window rows of the first scoring into their slots (slot = position mod (w + 1)),
// and the fp64 score cleared. One wave per row; the score is cleared by a
// grid-stride loop.
__global__ __launch_bounds__(256) void k_dec_load(LoadArgs A) {
  const int lane = threadIdx.x & 63;
  const int G = A.Hq / A.Hkv;
  {
    const int64_t tot = (int64_t)A.Hkv * A.n_max;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x)
      A.S64[i] = 0.0;
  }
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)A.Hq * A.w) return;
  const int h = (int)(row / A.w), i = (int)(row % A.w);
  const int g = h / G, hl = h % G;
  const int64_t pos = A.n - A.w + i;
  const int64_t r = trow(g, pos, hl, A.w, G);
  *(uint32_t*)(A.T.q + r * HD + 2 * lane) = *(const uint32_t*)(A.q + row * HD + 2 * lane);
  *(float2*)(A.T.a + r * HD + 2 * lane) = *(const float2*)(A.rs.a + row * HD + 2 * lane);
  const float m = A.rs.m[row], L = A.rs.L[row];
  if (lane == 0) {
    A.T.m[r] = m;
    A.T.L[r] = L;
    A.T.R[r] = A.rs.rest[row];
    A.T.jstar[r] = A.rs.flag[row] ? A.rs.jstar[row] : -1;
    A.T.cstar[r] = 0.f;
  }
  derive_row(A.T, r, m, L, lane);
}

// ---------------------------------------------------------------------------- argmax terms

struct StarInitArgs {
  FoldInfo f;
  DecRows T;
  double* S64;
  int64_t n, n_max;
  int w;
  int32_t* status;
};

// First window: the argmax terms of flagged rows from the fix-up partials
// (exact rest mass and ||a - v_j*||^2 without cancellation), added to the
// score in row order and kept in the row slots. One block per KV head.
__global__ __launch_bounds__(HD) void k_dec_star_init(StarInitArgs A) {
  const int g = blockIdx.x;
  if (A.f.flagcount[g] == 0) return;
  const int G = A.f.Rg / A.w;
  __shared__ float red[HD];
  for (int rr = 0; rr < A.f.Rg; ++rr) {
    const int64_t row = (int64_t)g * A.f.Rg + rr;
    if (!A.f.rs.flag[row]) continue;
    float R;
    int bits;
    const float val = fold_value<HD>(A.f, row, red, &R, &bits);
    const int js = A.f.rs.jstar[row];
    if (threadIdx.x == 0) {
      const int hl = rr / A.w, i = rr % A.w;
      const int64_t r = trow(g, A.n - A.w + i, hl, A.w, G);
      if (js < 0 || js >= A.n) {
        atomicOr(A.status, kStatusNonFinite);
      } else if (bits) {
        atomicOr(A.status, bits);
      } else {
        A.T.R[r] = R;
        A.T.cstar[r] = val;
        A.S64[(size_t)g * A.n_max + js] += (double)val / (double)G;
      }
    }
  }
}

struct StarAllArgs {
  DecRows T;
  double* S64;
  int64_t n, n_max;
  int w, G;
};

// Rebuild: every window row's kept argmax term added, in row order. One thread per KV head.
__global__ void k_dec_star_all(StarAllArgs A) {
  const int g = blockIdx.x;
  if (threadIdx.x != 0) return;
  double* S = A.S64 + (size_t)g * A.n_max;
  for (int i = 0; i < A.w; ++i)
    for (int h = 0; h < A.G; ++h) {
      const int64_t r = trow(g, A.n - A.w + i, h, A.w, A.G);
      const int js = A.T.jstar[r];
      if (js >= 0 && js < A.n) S[js] += (double)A.T.cstar[r] / (double)A.G;
    }
}

// ---------------------------------------------------------------------------- new rows

struct StatsArgs {
  const uint16_t* qn;  // [Hq][d] query rows of the appended position
  const uint16_t* k;   // [Hkv][n_max][d]
  const uint16_t* v;
  float* part;         // [nch][Hkv][G][kDecPart]
  int64_t n, n_max;
  int G, Hkv, nch, r0, nr;  // rows r0 .. r0 + nr - 1 of each KV head's G (nr <= kRowBatch)
  float c2;                 // log2(e) / sqrt(d)
};

// Online state of one row over a set of tokens: largest logit m (log2 units),
// rest mass R = sum over the other tokens of 2^{x - m}, argmax j (lowest index
// among equal maxima) and A = sum 2^{x - m} v over all tokens.
struct OnState {
  float m, R;
  int j;
};

// (m1, R1, j1, A1) merged with (m2, R2, j2, A2); A holds the lane's D dims
template <int D>
__device__ __forceinline__ void on_merge(OnState& s1, float (&A1)[D], OnState s2, const float (&A2)[D]) {
  if (s2.m == -INFINITY) return;
  if (s1.m == -INFINITY) {
    s1 = s2;
#pragma unroll
    for (int i = 0; i < D; ++i) A1[i] = A2[i];
    return;
  }
  const bool win1 = s1.m > s2.m || (s1.m == s2.m && s1.j < s2.j);
  const float mx = fmaxf(s1.m, s2.m);
  const float f1 = __builtin_amdgcn_exp2f(s1.m - mx), f2 = __builtin_amdgcn_exp2f(s2.m - mx);
  s1.R = win1 ? s1.R + (s2.R + 1.0f) * f2 : s2.R + (s1.R + 1.0f) * f1;
  s1.j = win1 ? s1.j : s2.j;
  s1.m = mx;
#pragma unroll
  for (int i = 0; i < D; ++i) A1[i] = A1[i] * f1 + A2[i] * f2;
}

// sum over the 8 lanes of a DPP half-row, result in every lane of it
__device__ __forceinline__ float row8_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));  // row_half_mirror
  return x;
}

// Per (token chunk, KV head): 8 lanes per token (lane l%8 holds dims
// 8(l%8) .. +7 and 64 + 8(l%8) .. +7, so each load instruction reads 8 token
// rows x 128 contiguous bytes), rows held in registers. Each lane group keeps
// its rows' state against a lazy reference mref (log2 units): estar = 2^{m -
// mref} of the current maximum m, R' = sum over its other tokens of
// 2^{x - mref} (a new maximum moves the old one's weight into R', so nothing
// is ever subtracted) and acc = sum 2^{x - mref} v; the reference moves only
// when a logit exceeds it by more than 2^8. The eight lane groups and four
// waves are then merged into one partial per row, relative to m.
template <int NR>
__global__ __launch_bounds__(256) void k_dec_stats(StatsArgs A) {
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 7, grp = lane >> 3;
  constexpr int U = NR <= 2 ? 4 : (NR <= 4 ? 2 : 1);  // 32-token groups per round of loads (two rounds in flight)
  constexpr float kRef = 8.0f;
  const int64_t t0 = (int64_t)chunk * kStatsTok;
  int64_t t1 = t0 + kStatsTok;
  if (t1 > A.n) t1 = A.n;
  uint32_t q[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint16_t* qr = A.qn + ((size_t)(g * A.G + A.r0 + r)) * HD;
    const uint4 u0 = *(const uint4*)(qr + 8 * li), u1 = *(const uint4*)(qr + 64 + 8 * li);
    q[r][0] = u0.x; q[r][1] = u0.y; q[r][2] = u0.z; q[r][3] = u0.w;
    q[r][4] = u1.x; q[r][5] = u1.y; q[r][6] = u1.z; q[r][7] = u1.w;
  }
  float mref[NR], m[NR], estar[NR], Rp[NR], acc[NR][16];
  int jst[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    mref[r] = -INFINITY; m[r] = -INFINITY; estar[r] = 0.f; Rp[r] = 0.f; jst[r] = -1;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
  }
  const char* kc = (const char*)(A.k + ((size_t)g * A.n_max + t0) * HD);
  const char* vc = (const char*)(A.v + ((size_t)g * A.n_max + t0) * HD);
  const int nt = (int)(t1 - t0);
  const int lo = wave * 8 + grp;  // this lane group's token within each group of 32
  auto load = [&](int tb, uint4 (&k0)[U], uint4 (&k1)[U], uint4 (&v0)[U], uint4 (&v1)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int tr = tb + 32 * u + lo;
      tr = tr < nt ? tr : nt - 1;
      const uint32_t off = (uint32_t)tr * (HD * 2) + 16u * (uint32_t)li;
      k0[u] = *(const uint4*)(kc + off);
      k1[u] = *(const uint4*)(kc + off + 128);
      v0[u] = *(const uint4*)(vc + off);
      v1[u] = *(const uint4*)(vc + off + 128);
    }
  };
  auto process = [&](int tb, const uint4 (&k0)[U], const uint4 (&k1)[U], const uint4 (&v0)[U],
                     const uint4 (&v1)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tl = tb + 32 * u + lo;
      const bool ok = tl < nt;
      const uint32_t kw[8] = {k0[u].x, k0[u].y, k0[u].z, k0[u].w, k1[u].x, k1[u].y, k1[u].z, k1[u].w};
      const uint32_t vw[8] = {v0[u].x, v0[u].y, v0[u].z, v0[u].w, v1[u].x, v1[u].y, v1[u].z, v1[u].w};
      float vf[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vf[2 * i] = __uint_as_float(vw[i] << 16);
        vf[2 * i + 1] = __uint_as_float(vw[i] & 0xffff0000u);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[r][i]), __builtin_bit_cast(bf16x2, kw[i]),
                                              d, false);
        const float x = ok ? row8_sum(d) * A.c2 : -INFINITY;
        // move the reference when a logit passes it by more than 2^8 (rare; a wave decision)
        if (__builtin_amdgcn_ballot_w64(x > mref[r] + kRef)) {
          const bool mv = x > mref[r] + kRef;
          const float nref = mv ? x : mref[r];
          const float f = mv ? __builtin_amdgcn_exp2f(mref[r] - nref) : 1.0f;  // 0 from an empty state
          Rp[r] *= f;
          estar[r] *= f;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[r][i] *= f;
          mref[r] = nref;
        }
        const float e = ok ? __builtin_amdgcn_exp2f(x - mref[r]) : 0.f;
        const bool gt = x > m[r];
        Rp[r] += gt ? estar[r] : e;
        estar[r] = gt ? e : estar[r];
        jst[r] = gt ? (int)(t0 + tl) : jst[r];
        m[r] = gt ? x : m[r];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][i] = fmaf(e, vf[i], acc[r][i]);
      }
    }
  };
  constexpr int kRound = 32 * U;
  uint4 ka0[U], ka1[U], va0[U], va1[U], kb0[U], kb1[U], vb0[U], vb1[U];
  int tb = 0;
  if (tb < nt) load(tb, ka0, ka1, va0, va1);
  while (tb < nt) {
    if (tb + kRound < nt) load(tb + kRound, kb0, kb1, vb0, vb1);
    process(tb, ka0, ka1, va0, va1);
    tb += kRound;
    if (tb >= nt) break;
    if (tb + kRound < nt) load(tb + kRound, ka0, ka1, va0, va1);
    process(tb, kb0, kb1, vb0, vb1);
    tb += kRound;
  }
  // state relative to m: R = R' / estar, A = acc / estar (estar = 2^{m - mref} >= 2^-8... > 0)
  OnState st[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float inv = m[r] == -INFINITY ? 0.f : 1.0f / estar[r];
    st[r] = OnState{m[r], Rp[r] * inv, jst[r]};
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] *= inv;
  }
  // merge the eight lane groups of the wave (lanes li + 8 k), lower group first
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
      OnState s2{__shfl_xor(st[r].m, o, 64), __shfl_xor(st[r].R, o, 64), __shfl_xor(st[r].j, o, 64)};
      float a2[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) a2[i] = __shfl_xor(acc[r][i], o, 64);
      if (lane & o) {
        OnState s1 = s2;
        float a1[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) a1[i] = a2[i];
        on_merge<16>(s1, a1, st[r], acc[r]);
        st[r] = s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][i] = a1[i];
      } else {
        on_merge<16>(st[r], acc[r], s2, a2);
      }
    }
  }
  // then the four waves, in wave order; dims of lane li: 8 li + (0..7), 64 + 8 li + (0..7)
  __shared__ float ws[4][NR][kDecPart];
  if (grp == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ws[wave][r][8 * li + i] = acc[r][i];
        ws[wave][r][64 + 8 * li + i] = acc[r][8 + i];
      }
      if (li == 0) {
        ws[wave][r][HD] = st[r].m;
        ws[wave][r][HD + 1] = st[r].R;
        ws[wave][r][HD + 2] = __int_as_float(st[r].j);
      }
    }
  }
  __syncthreads();
  if (wave == 0 && grp == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      OnState s1{ws[0][r][HD], ws[0][r][HD + 1], __float_as_int(ws[0][r][HD + 2])};
      float a1[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a1[i] = ws[0][r][8 * li + i];
        a1[8 + i] = ws[0][r][64 + 8 * li + i];
      }
      for (int wv = 1; wv < 4; ++wv) {
        OnState s2{ws[wv][r][HD], ws[wv][r][HD + 1], __float_as_int(ws[wv][r][HD + 2])};
        float a2[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a2[i] = ws[wv][r][8 * li + i];
          a2[8 + i] = ws[wv][r][64 + 8 * li + i];
        }
        on_merge<16>(s1, a1, s2, a2);
      }
      float* o = A.part + (((size_t)chunk * A.Hkv + g) * A.G + A.r0 + r) * kDecPart;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[8 * li + i] = a1[i];
        o[64 + 8 * li + i] = a1[8 + i];
      }
      if (li == 0) {
        o[HD] = s1.m;
        o[HD + 1] = s1.R;
        o[HD + 2] = __int_as_float(s1.j);
      }
    }
  }
}

struct DMergeArgs {
  const float* part;
  const uint16_t* qn;
  const uint16_t* v;  // [Hkv][n_max][d]
  DecRows T;
  double* S64;
  int64_t n, n_max;
  int G, Hkv, w, nch;
  int32_t* status;
};

// One block per KV head, one wave per new row: the chunk partials merged
// (chunks across lanes; R = R_winner + sum over the other chunks of
// (R_c + 1) 2^{m_c - m}, so nothing is subtracted), the row stored in its
// slot (query, a, m, L = 1 + R, R, the argmax of rows with R < 1, derived
// state). Then, in row order, the argmax terms: added for the new rows with
// R < 1 (||a - v_j*||^2 / R^2, computed directly) and removed for the rows
// leaving the window (their kept value). Rejects R <= 2^-24 (singular) and
// non-finite rows.
__global__ __launch_bounds__(1024) void k_dec_merge(DMergeArgs A) {
  const int g = blockIdx.x, h = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ float s_val[64];
  __shared__ int s_js[64];
  if (h < A.G) {
    auto part = [&](int c) { return A.part + (((size_t)c * A.Hkv + g) * A.G + h) * kDecPart; };
    float m = -INFINITY, R = 0.f, a0 = 0.f, a1 = 0.f;
    int j = -1;
    for (int c0 = 0; c0 < A.nch; c0 += 32) {
      // this group of up to 32 chunks (lane = chunk): every load issued before any is used
      const int cn = A.nch - c0 < 32 ? A.nch - c0 : 32;
      const int c = c0 + (lane < cn ? lane : cn - 1);
      const float mc = lane < cn ? part(c)[HD] : -INFINITY;
      const float Rc = part(c)[HD + 1];
      const int jc = __float_as_int(part(c)[HD + 2]);
      float2 av[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) av[u] = *(const float2*)(part(c0 + (u < cn ? u : cn - 1)) + 2 * lane);
      float gm = mc;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o, 64));
      const int cw = __ffsll((long long)__builtin_amdgcn_ballot_w64(mc == gm)) - 1;  // lowest chunk at the max
      // this group's state relative to its own max gm
      float t = (lane == cw || mc == -INFINITY) ? (lane == cw ? Rc : 0.f)
                                                : (Rc + 1.0f) * __builtin_amdgcn_exp2f(mc - gm);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
      const int jg = __shfl(jc, cw, 64);
      float g0 = 0.f, g1 = 0.f;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const float mu = __shfl(mc, u, 64);
        const float su = (u < cn && mu != -INFINITY) ? __builtin_amdgcn_exp2f(mu - gm) : 0.f;
        g0 = fmaf(av[u].x, su, g0);
        g1 = fmaf(av[u].y, su, g1);
      }
      // fold the group into the running state (groups in chunk order)
      if (gm != -INFINITY) {
        if (m == -INFINITY) {
          m = gm; R = t; j = jg; a0 = g0; a1 = g1;
        } else {
          const bool win1 = m >= gm;  // earlier chunks hold lower indices
          const float mx = fmaxf(m, gm);
          const float f1 = __builtin_amdgcn_exp2f(m - mx), f2 = __builtin_amdgcn_exp2f(gm - mx);
          R = win1 ? R + (t + 1.0f) * f2 : t + (R + 1.0f) * f1;
          j = win1 ? j : jg;
          a0 = a0 * f1 + g0 * f2;
          a1 = a1 * f1 + g1 * f2;
          m = mx;
        }
      }
    }
    const float L = 1.0f + R;
    const float x0 = a0 / L, x1 = a1 / L;
    const int64_t r = trow(g, A.n - 1, h, A.w, A.G);
    *(float2*)(A.T.a + r * HD + 2 * lane) = make_float2(x0, x1);
    *(uint32_t*)(A.T.q + r * HD + 2 * lane) = *(const uint32_t*)(A.qn + ((size_t)g * A.G + h) * HD + 2 * lane);
    bool bad = !finite_f(m) || !finite_f(R) || !finite_f(x0) || !finite_f(x1);
    bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    const float m_nat = m / kLog2e;
    const int js = (!bad && R < 1.0f && j >= 0 && j < A.n) ? j : -1;
    float val = 0.f;
    if (js >= 0) {  // the argmax term, without cancellation
      const uint32_t vv = *(const uint32_t*)(A.v + ((size_t)g * A.n_max + js) * HD + 2 * lane);
      const float d0 = x0 - __uint_as_float(vv << 16), d1 = x1 - __uint_as_float(vv & 0xffff0000u);
      float dist = fmaf(d0, d0, d1 * d1);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) dist += __shfl_xor(dist, o, 64);
      val = dist / (R * R);
    }
    if (lane == 0) {
      A.T.m[r] = m_nat;
      A.T.L[r] = L;
      A.T.R[r] = R;
      A.T.jstar[r] = js;
      A.T.cstar[r] = val;
      s_val[h] = val;
      s_js[h] = js;
      if (bad) atomicOr(A.status, kStatusNonFinite);
      else if (R <= kSingularRest) atomicOr(A.status, kStatusSingular);
    }
    derive_row(A.T, r, m_nat, L, lane);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double* S = A.S64 + (size_t)g * A.n_max;
    const double invG = 1.0 / (double)A.G;
    for (int hh = 0; hh < A.G; ++hh) {
      if (s_js[hh] >= 0) S[s_js[hh]] += (double)s_val[hh] * invG;
      const int64_t ro = trow(g, A.n - 1 - A.w, hh, A.w, A.G);  // leaving row
      const int jo = A.T.jstar[ro];
      if (jo >= 0 && jo < A.n) S[jo] -= (double)A.T.cstar[ro] * invG;
    }
  }
}

// ---------------------------------------------------------------------------- signed terms

struct ContribArgs {
  const uint16_t* k;  // [Hkv][n_max][d]
  const uint16_t* v;
  DecRows T;
  double* S64;        // [Hkv][n_max]
  int64_t n, n_max;
  int w, G;
  int mode;           // 0: window entries e0 .. e1-1 (rows at n - w + e); 1: step (new rows +, leaving rows -)
  int e0, e1;
  float c2;           // log2(e) / sqrt(d)
};

// Row rr of this launch's list (per KV head): entry e = rr / G, query head rr % G.
__device__ __forceinline__ void entry_of(const ContribArgs& A, int e, int64_t& pos, float& sign) {
  if (A.mode == 0) {
    pos = A.n - A.w + e;
    sign = 1.0f;
  } else if (e == 0) {
    pos = A.n - 1;
    sign = 1.0f;
  } else {
    pos = A.n - 1 - A.w;
    sign = -1.0f;
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Operand layout (16x16x32 bf16 MFMA): lane l holds row / token l%16 and, at
// step ks, dims 32 ks + 8 (l/16) .. +7, so the four lanes of a token read 64
// adjacent bytes of its row and one load instruction covers 16 rows x 64 B.
// The result gives lane l token l%16 and rows 4 (l/16) + i, i = 0..3.
__device__ __forceinline__ int opoff(int lane, int ks) { return 64 * ks + 16 * (lane >> 4); }  // bytes

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// sum over the four 16-lane rows (lanes l, l^16, l^32, l^48), the same
// order in every lane: (row0 + row1) + (row2 + row3)
__device__ __forceinline__ float rows4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ double rows4_sum(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  const double y = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0])) +
                   __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
  const uint64_t w = (uint64_t)__double_as_longlong(y);
  auto lo2 = __builtin_amdgcn_permlane32_swap((uint32_t)w, (uint32_t)w, false, false);
  auto hi2 = __builtin_amdgcn_permlane32_swap((uint32_t)(w >> 32), (uint32_t)(w >> 32), false, false);
  return __longlong_as_double((long long)(((uint64_t)hi2[0] << 32) | lo2[0])) +
         __longlong_as_double((long long)(((uint64_t)hi2[1] << 32) | lo2[1]));
}

// Per (chunk of kTokPerWg tokens, KV head): each wave takes 16-token
// subtiles; per subtile and 16-row block X = Q K^T and C = a V^T - ||a||^2/2
// on MFMA, then per (row, token) the term r^2 ||a - v_j||^2 with
// r = p / (1 - p), for tokens the row sees other than its kept argmax,
// summed with the row's sign in fp64 and added to the score. Every element's
// value depends only on its row's stored state and its token, whatever else
// shares the block, so a row's terms are the same in every launch.
template <int ROWS>
__global__ __launch_bounds__(256) void k_dec_contrib(ContribArgs A) {
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = lane >> 4, l16 = lane & 15;
  const int nrows = (A.e1 - A.e0) * A.G;
  const int nb = (nrows + 15) / 16;
  __shared__ __attribute__((aligned(16))) float s_bias[ROWS];
  __shared__ __attribute__((aligned(16))) float s_cinit[ROWS];
  __shared__ __attribute__((aligned(16))) float s_sign[ROWS];
  __shared__ __attribute__((aligned(16))) int s_pos[ROWS];
  __shared__ __attribute__((aligned(16))) int s_js[ROWS];
  __shared__ int64_t s_row[ROWS];
  // per-token sums of this chunk, added to the score once every subtile is done
  // (a read-modify-write per subtile would wait for the prefetched loads too)
  __shared__ double s_tot[kTokPerWg];
  // the rows' query and a operands, staged in LDS (rows padded to 272 bytes,
  // so 16 rows read at one column hit distinct banks): reading them from
  // global memory here would wait for the loads of the next subtiles too
  // (vector loads complete in order)
  __shared__ __attribute__((aligned(16))) uint16_t s_op[2 * ROWS][kOpStride];
  for (int rr = threadIdx.x; rr < nb * 16; rr += blockDim.x) {
    if (rr < nrows) {
      int64_t pos;
      float sign;
      entry_of(A, A.e0 + rr / A.G, pos, sign);
      const int64_t r = trow(g, pos, rr % A.G, A.w, A.G);
      s_row[rr] = r;
      s_bias[rr] = A.T.bias[r];
      s_cinit[rr] = A.T.cinit[r];
      s_sign[rr] = sign;
      s_pos[rr] = (int)pos;
      s_js[rr] = A.T.jstar[r];
    } else {  // padding rows: p = 0
      s_row[rr] = -1;
      s_bias[rr] = INFINITY;
      s_cinit[rr] = 0.f;
      s_sign[rr] = 0.f;
      s_pos[rr] = -1;
      s_js[rr] = -1;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb * 16 * 32; i += blockDim.x) {
    const int rr = i >> 5, c = i & 31;  // 32 chunks of 16 bytes: q then a_bf
    const int64_t r = s_row[rr];
    uint4 u = make_uint4(0, 0, 0, 0);
    if (r >= 0) u = *(const uint4*)((const char*)((c < 16 ? A.T.q : A.T.a_bf) + r * HD) + 16 * (c & 15));
    *(uint4*)((char*)&s_op[(c < 16 ? 0 : ROWS) + rr][0] + 16 * (c & 15)) = u;
  }
  __syncthreads();
  const int64_t t0 = (int64_t)chunk * kTokPerWg;
  const double invG = 1.0 / (double)A.G;
  double* S = A.S64 + (size_t)g * A.n_max;
  // 32-bit byte offsets within the workgroup's chunk (at most kTokPerWg rows)
  const char* kc = (const char*)(A.k + ((size_t)g * A.n_max + t0) * HD);
  const char* vc = (const char*)(A.v + ((size_t)g * A.n_max + t0) * HD);
  const int nt = (int)((A.n - t0) < kTokPerWg ? (A.n - t0) : kTokPerWg);
  constexpr int NSUB = kTokPerWg / 16;

  auto valid = [&](int sub) { return sub < NSUB && sub * 16 < nt; };
  auto load_kv = [&](int sub, bf16x8 (&kb)[4], bf16x8 (&vb)[4]) {
    int tr = sub * 16 + l16;
    tr = tr < nt ? tr : nt - 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t off = (uint32_t)tr * (HD * 2) + (uint32_t)opoff(lane, ks);
      kb[ks] = *(const bf16x8*)(kc + off);
      vb[ks] = *(const bf16x8*)(vc + off);
    }
  };
  auto process = [&](int sub, const bf16x8 (&kb)[4], const bf16x8 (&vb)[4]) {
    const int tok = (int)t0 + sub * 16 + l16;
    // ||v_j||^2: exact bf16 squares, fp32 sums over this lane's 32 dims, then the token's four lanes
    float n0 = 0.f, n1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x2 p0 = {vb[ks][0], vb[ks][1]}, p1 = {vb[ks][2], vb[ks][3]};
      const bf16x2 p2 = {vb[ks][4], vb[ks][5]}, p3 = {vb[ks][6], vb[ks][7]};
      n0 = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, n0, false);
      n1 = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, n1, false);
      n0 = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, n0, false);
      n1 = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, n1, false);
    }
    const float nvj = rows4_sum(n0 + n1);
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) {
      // the block's query and a operands
      bf16x8 qa[4], aa[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qa[ks] = *(const bf16x8*)((const char*)&s_op[16 * b + l16][0] + opoff(lane, ks));
        aa[ks] = *(const bf16x8*)((const char*)&s_op[ROWS + 16 * b + l16][0] + opoff(lane, ks));
      }
      const int base = 16 * b + 4 * q4;  // this lane's four rows
      const float4 c4 = *(const float4*)(&s_cinit[base]);
      f32x4 X = {}, C = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) X = mfma16(qa[ks], kb[ks], X);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) C = mfma16(aa[ks], vb[ks], C);
      const float4 bi = *(const float4*)(&s_bias[base]);
      const float4 sg = *(const float4*)(&s_sign[base]);
      const int4 ps = *(const int4*)(&s_pos[base]);
      const int4 js = *(const int4*)(&s_js[base]);
      const float bv[4] = {bi.x, bi.y, bi.z, bi.w}, sv[4] = {sg.x, sg.y, sg.z, sg.w};
      const int pv[4] = {ps.x, ps.y, ps.z, ps.w}, jv[4] = {js.x, js.y, js.z, js.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // branch-free: tokens the row does not see, and its kept argmax, get 0
        const float p = __builtin_amdgcn_exp2f(fmaf(X[i], A.c2, -bv[i]));
        const float rr = p * __builtin_amdgcn_rcpf(1.0f - p);
        const float c = rr * rr * fmaxf(fmaf(-2.0f, C[i], nvj), 0.0f);
        acc += (double)((tok <= pv[i] && tok != jv[i]) ? sv[i] * c : 0.0f);
      }
    }
    const double total = rows4_sum(acc);
    if (q4 == 0) s_tot[sub * 16 + l16] = total;
  };
  // subtiles wave, wave + 4, ...: the next two subtiles' K and V are in
  // flight while one is processed (three register buffers in rotation)
  bf16x8 kb[3][4], vb[3][4];
  int sub = wave;
  if (valid(sub)) load_kv(sub, kb[0], vb[0]);
  if (valid(sub + 4)) load_kv(sub + 4, kb[1], vb[1]);
  while (true) {
    if (!valid(sub)) break;
    if (valid(sub + 8)) load_kv(sub + 8, kb[2], vb[2]);
    process(sub, kb[0], vb[0]);
    sub += 4;
    if (!valid(sub)) break;
    if (valid(sub + 8)) load_kv(sub + 8, kb[0], vb[0]);
    process(sub, kb[1], vb[1]);
    sub += 4;
    if (!valid(sub)) break;
    if (valid(sub + 8)) load_kv(sub + 8, kb[1], vb[1]);
    process(sub, kb[2], vb[2]);
    sub += 4;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt; i += blockDim.x) S[t0 + i] += s_tot[i] * invG;
}

__global__ void k_dec_zero(double* p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.0;
}

__global__ void k_dec_tof32(const double* S64, float* out, int64_t n, int64_t n_max, int Hkv) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)Hkv * n) return;
  const int64_t g = i / n, j = i % n;
  out[i] = (float)S64[g * n_max + j];
}

}  // namespace

// ---------------------------------------------------------------------------- launchers

DecState carve_decode_state(void* base, int64_t n_max, int32_t w, int32_t Hq, int32_t Hkv) {
  DecState S{};
  size_t off = 0;
  char* b = (char*)base;
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? (void*)(b + off) : nullptr;
    off = (off + bytes + 255) / 256 * 256;
    return p;
  };
  const int G = Hq / Hkv;
  const size_t rows = (size_t)Hkv * (w + 1) * G;
  S.S64 = (double*)take(sizeof(double) * (size_t)Hkv * n_max);
  S.T.q = (uint16_t*)take(2 * rows * HD);
  S.T.a = (float*)take(4 * rows * HD);
  S.T.a_bf = (uint16_t*)take(2 * rows * HD);
  S.T.m = (float*)take(4 * rows);
  S.T.L = (float*)take(4 * rows);
  S.T.R = (float*)take(4 * rows);
  S.T.cstar = (float*)take(4 * rows);
  S.T.bias = (float*)take(4 * rows);
  S.T.cinit = (float*)take(4 * rows);
  S.T.jstar = (int32_t*)take(4 * rows);
  S.nch = (int)((n_max + kStatsTok - 1) / kStatsTok);
  S.part = (float*)take(sizeof(float) * (size_t)S.nch * Hkv * G * kDecPart);
  // MFMA row statistics of the first window, sized for n_max (its buffers do
  // not grow with a shorter cache); its S and select scratch serve the select
  const Shape sh{n_max, w, Hq, Hkv, HD};
  S.ws_base = take(carve_workspace(nullptr, sh, true).bytes);
  S.bytes = off;
  return S;
}

hipError_t launch_decode_contrib(const void* k, const void* v, int64_t n, int64_t n_max, int32_t w, int G,
                                 int32_t Hkv, const DecState& S, int mode, hipStream_t st) {
  const float c2 = kLog2e / sqrtf((float)HD);
  const int nent = mode == 0 ? w : 2;
  // a step's 2G rows fit one small launch; a whole window takes launches of
  // up to kInitRows rows: fewer K/V reads than 64-row launches, while two
  // workgroups still fit a CU (256-row launches, one per CU, were slower)
  const int per = (mode == 0 ? kInitRows : kContribRows) / G;  // window entries per launch (G <= 16)
  const dim3 grid((unsigned)((n + kTokPerWg - 1) / kTokPerWg), Hkv);
  for (int e0 = 0; e0 < nent; e0 += per) {
    const int e1 = e0 + per < nent ? e0 + per : nent;
    ContribArgs a{(const uint16_t*)k, (const uint16_t*)v, S.T, S.S64, n, n_max, w, G, mode, e0, e1, c2};
    if (mode == 0)
      k_dec_contrib<kInitRows><<<grid, 256, 0, st>>>(a);
    else
      k_dec_contrib<kContribRows><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_init(const void* q, const void* k, const void* v, int64_t n, int64_t n_max, int32_t w,
                              int32_t Hq, int32_t Hkv, const DecState& S, int32_t* status, hipStream_t st) {
  const Shape sh{n, w, Hq, Hkv, HD};
  Workspace ws = carve_workspace(S.ws_base, sh, true);
  ws.status = status;
  FoldInfo fold{};
  hipError_t e = launch_mfma_rowstats(q, k, v, sh, n_max, ws, st, &fold);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)Hq * w;
  LoadArgs la{(const uint16_t*)q, ws.rs, S.T, S.S64, n, n_max, w, Hq, Hkv};
  k_dec_load<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(la);
  StarInitArgs sa{fold, S.T, S.S64, n, n_max, w, status};
  k_dec_star_init<<<Hkv, HD, 0, st>>>(sa);
  return launch_decode_contrib(k, v, n, n_max, w, Hq / Hkv, Hkv, S, 0, st);
}

hipError_t launch_decode_step(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                              int32_t w, int32_t Hq, int32_t Hkv, const DecState& S, int32_t* status,
                              hipStream_t st) {
  const int G = Hq / Hkv;
  const float c2 = kLog2e / sqrtf((float)HD);
  const int nch = (int)((n + kStatsTok - 1) / kStatsTok);
  for (int r0 = 0; r0 < G; r0 += kRowBatch) {
    const int nr = G - r0 < kRowBatch ? G - r0 : kRowBatch;
    StatsArgs a{(const uint16_t*)q_new, (const uint16_t*)k, (const uint16_t*)v, S.part, n, n_max, G, Hkv, nch,
                r0, nr, c2};
    const dim3 grid(nch, Hkv);
    switch (nr) {
      case 1: k_dec_stats<1><<<grid, 256, 0, st>>>(a); break;
      case 2: k_dec_stats<2><<<grid, 256, 0, st>>>(a); break;
      case 3: k_dec_stats<3><<<grid, 256, 0, st>>>(a); break;
      case 4: k_dec_stats<4><<<grid, 256, 0, st>>>(a); break;
      case 5: k_dec_stats<5><<<grid, 256, 0, st>>>(a); break;
      case 6: k_dec_stats<6><<<grid, 256, 0, st>>>(a); break;
      case 7: k_dec_stats<7><<<grid, 256, 0, st>>>(a); break;
      default: k_dec_stats<8><<<grid, 256, 0, st>>>(a); break;
    }
  }
  DMergeArgs ma{S.part, (const uint16_t*)q_new, (const uint16_t*)v, S.T, S.S64, n, n_max, G, Hkv, w, nch,
                status};
  k_dec_merge<<<Hkv, 64 * G, 0, st>>>(ma);
  return launch_decode_contrib(k, v, n, n_max, w, G, Hkv, S, 1, st);
}

hipError_t launch_decode_rebuild(const void* k, const void* v, int64_t n, int64_t n_max, int32_t w, int32_t Hq,
                                 int32_t Hkv, const DecState& S, int32_t* status, hipStream_t st) {
  const int G = Hq / Hkv;
  const int64_t cnt = (int64_t)Hkv * n_max;
  k_dec_zero<<<(unsigned)((cnt + 255) / 256), 256, 0, st>>>(S.S64, cnt);
  StarAllArgs sa{S.T, S.S64, n, n_max, w, G};
  k_dec_star_all<<<Hkv, 64, 0, st>>>(sa);
  (void)status;
  return launch_decode_contrib(k, v, n, n_max, w, G, Hkv, S, 0, st);
}

hipError_t launch_decode_scores(const DecState& S, int64_t n, int64_t n_max, int32_t Hkv, float* out,
                                hipStream_t st) {
  const int64_t tot = (int64_t)Hkv * n;
  k_dec_tof32<<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(S.S64, out, n, n_max, Hkv);
  return hipGetLastError();
}

hipError_t launch_decode_select(const DecState& S, int64_t n, int64_t n_max, int32_t w, int32_t Hq, int32_t Hkv,
                                int32_t pool_kernel, int64_t n_evict, float* out_scores, int64_t* out_idx,
                                int32_t* status, hipStream_t st) {
  const Shape sh{n_max, w, Hq, Hkv, HD};
  Workspace ws = carve_workspace(S.ws_base, sh, true);  // S [Hkv][n] and select scratch for n <= n_max
  hipError_t e = launch_decode_scores(S, n, n_max, Hkv, ws.S, st);
  if (e == hipSuccess) e = launch_init(ws.status, nullptr, ws.sel, Hkv, st);
  if (e == hipSuccess)
    e = launch_select(ws.S, n, w, Hkv, pool_kernel, n_evict, out_scores, out_idx, status, nullptr, ws.sel, st);
  return e;
}

}  // namespace dropkv
