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
//   k_dec_fused8 / k_dec_fused  the single-pass step: one read of K and V
//       through LDS tiles feeds both the new rows' statistics (as
//       k_dec_stats) and the terms of the leaving rows and of the rows the
//       previous single-pass step left pending (as k_dec_contrib); the new
//       rows' terms stay pending until the next step, a flush or a rebuild
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
constexpr int kInitRows = 128;     // rows per launch when a whole window is scored (two workgroups per CU: see below)
constexpr int kOpStride = HD + 8;  // bf16 per staged operand row (272 bytes)
// tokens per k_dec_contrib workgroup: 512 for a step's few rows (4 waves x 8
// subtiles of 16), 1024 for whole-window launches (their 128 rows keep each
// workgroup busy longer, and fewer workgroups stage the rows: 7% faster)
constexpr int tok_per_wg(int rows) { return rows > 64 ? 1024 : 512; }
constexpr int kStatsTok = 2048;    // tokens per k_dec_stats workgroup
// The single-pass step runs k_dec_fused8 (chunks of chunk_tok >= kStatsTok
// tokens) for groups of at most this many query heads per KV head, and
// k_dec_fused (chunks of exactly kStatsTok) above it.
constexpr int kFused8MaxG = 4;

// Compute units of the current device (read once per device; 256 on MI355X).
int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

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
  int64_t* pend;
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
  if (blockIdx.x == 0 && threadIdx.x == 0) A.pend[0] = -1;
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

// One lane's share of NR rows' online state (dims 8 li .. +7 and 64 + 8 li ..
// +7 of lane li of its 8-lane group, one token per group at a time), kept
// against a lazy reference mref (log2 units): estar = 2^{m - mref} of the
// current maximum m, R' = sum over its other tokens of 2^{x - mref} (a new
// maximum moves the old one's weight into R', so nothing is ever subtracted)
// and acc = sum 2^{x - mref} v; the reference moves only when a logit exceeds
// it by more than 2^8.
template <int NR>
struct StatsLane {
  uint32_t q[NR][8];
  float mref[NR], m[NR], estar[NR], Rp[NR], acc[NR][16];
  int jst[NR];
};

// query rows r0 .. r0 + NR - 1 of KV head g (qn: [Hq][d] bf16), empty state
template <int NR>
__device__ __forceinline__ void stats_begin(StatsLane<NR>& L, const uint16_t* qn, int g, int G, int r0, int li) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint16_t* qr = qn + ((size_t)(g * G + r0 + r)) * HD;
    const uint4 u0 = *(const uint4*)(qr + 8 * li), u1 = *(const uint4*)(qr + 64 + 8 * li);
    L.q[r][0] = u0.x; L.q[r][1] = u0.y; L.q[r][2] = u0.z; L.q[r][3] = u0.w;
    L.q[r][4] = u1.x; L.q[r][5] = u1.y; L.q[r][6] = u1.z; L.q[r][7] = u1.w;
    L.mref[r] = -INFINITY; L.m[r] = -INFINITY; L.estar[r] = 0.f; L.Rp[r] = 0.f; L.jst[r] = -1;
#pragma unroll
    for (int i = 0; i < 16; ++i) L.acc[r][i] = 0.f;
  }
}

// U tokens (global indices tok[u]; ok[u] = inside the cache) into every row's
// state, in token order. kw / vw: this lane's 16 dims of k and v of each token
// as bf16 pairs. All U x NR logits are formed first (independent dot-product
// chains), then the state updates run token by token, so the result is that
// of feeding the tokens one at a time. Wave-uniform control flow: every lane
// of the wave calls it together.
template <int NR, int U>
__device__ __forceinline__ void stats_tokens(StatsLane<NR>& L, const uint32_t (&kw)[U][8],
                                             const uint32_t (&vw)[U][8], const bool (&ok)[U], const int (&tok)[U],
                                             float c2) {
  constexpr float kRef = 8.0f;
  float x[U][NR];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, L.q[r][i]),
                                            __builtin_bit_cast(bf16x2, kw[u][i]), d, false);
      x[u][r] = ok[u] ? row8_sum(d) * c2 : -INFINITY;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float vf[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vf[2 * i] = __uint_as_float(vw[u][i] << 16);
      vf[2 * i + 1] = __uint_as_float(vw[u][i] & 0xffff0000u);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float xr = x[u][r];
      // move the reference when a logit passes it by more than 2^8 (rare; a wave decision)
      if (__builtin_amdgcn_ballot_w64(xr > L.mref[r] + kRef)) {
        const bool mv = xr > L.mref[r] + kRef;
        const float nref = mv ? xr : L.mref[r];
        const float f = mv ? __builtin_amdgcn_exp2f(L.mref[r] - nref) : 1.0f;  // 0 from an empty state
        L.Rp[r] *= f;
        L.estar[r] *= f;
#pragma unroll
        for (int i = 0; i < 16; ++i) L.acc[r][i] *= f;
        L.mref[r] = nref;
      }
      const float e = ok[u] ? __builtin_amdgcn_exp2f(xr - L.mref[r]) : 0.f;
      const bool gt = xr > L.m[r];
      L.Rp[r] += gt ? L.estar[r] : e;
      L.estar[r] = gt ? e : L.estar[r];
      L.jst[r] = gt ? tok[u] : L.jst[r];
      L.m[r] = gt ? xr : L.m[r];
#pragma unroll
      for (int i = 0; i < 16; ++i) L.acc[r][i] = fmaf(e, vf[i], L.acc[r][i]);
    }
  }
}

// The workgroup's partial per row (relative to its m) into out[r * kDecPart]:
// the eight lane groups of each of the four statistics waves (swave 0..3)
// merged (lower group first), then the four waves in order through ws. Every
// thread of the workgroup calls it (active: the lane belongs to a statistics
// wave); ends with the partials written (no trailing barrier).
template <int NR>
__device__ __forceinline__ void stats_finish(StatsLane<NR>& L, float (*ws)[NR][kDecPart], float* out, int lane,
                                             int swave, bool active) {
  const int li = lane & 7, grp = lane >> 3;
  const int wave = swave;
  if (active) {
    // state relative to m: R = R' / estar, A = acc / estar (estar = 2^{m - mref} >= 2^-8... > 0)
    OnState st[NR];
  #pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float inv = L.m[r] == -INFINITY ? 0.f : 1.0f / L.estar[r];
      st[r] = OnState{L.m[r], L.Rp[r] * inv, L.jst[r]};
  #pragma unroll
      for (int i = 0; i < 16; ++i) L.acc[r][i] *= inv;
    }
  #pragma unroll
    for (int r = 0; r < NR; ++r) {
  #pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        OnState s2{__shfl_xor(st[r].m, o, 64), __shfl_xor(st[r].R, o, 64), __shfl_xor(st[r].j, o, 64)};
        float a2[16];
  #pragma unroll
        for (int i = 0; i < 16; ++i) a2[i] = __shfl_xor(L.acc[r][i], o, 64);
        if (lane & o) {
          OnState s1 = s2;
          float a1[16];
  #pragma unroll
          for (int i = 0; i < 16; ++i) a1[i] = a2[i];
          on_merge<16>(s1, a1, st[r], L.acc[r]);
          st[r] = s1;
  #pragma unroll
          for (int i = 0; i < 16; ++i) L.acc[r][i] = a1[i];
        } else {
          on_merge<16>(st[r], L.acc[r], s2, a2);
        }
      }
    }
    // then the four waves, in wave order; dims of lane li: 8 li + (0..7), 64 + 8 li + (0..7)
    if (grp == 0) {
  #pragma unroll
      for (int r = 0; r < NR; ++r) {
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          ws[wave][r][8 * li + i] = L.acc[r][i];
          ws[wave][r][64 + 8 * li + i] = L.acc[r][8 + i];
        }
        if (li == 0) {
          ws[wave][r][HD] = st[r].m;
          ws[wave][r][HD + 1] = st[r].R;
          ws[wave][r][HD + 2] = __int_as_float(st[r].j);
        }
      }
    }
  }
  __syncthreads();
  if (active && wave == 0 && grp == 0) {
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
      float* o = out + (size_t)r * kDecPart;
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

// Per (token chunk, KV head): 8 lanes per token (lane l%8 holds dims
// 8(l%8) .. +7 and 64 + 8(l%8) .. +7, so each load instruction reads 8 token
// rows x 128 contiguous bytes), rows held in registers (StatsLane); the eight
// lane groups and four waves are then merged into one partial per row,
// relative to m.
template <int NR>
__global__ __launch_bounds__(256) void k_dec_stats(StatsArgs A) {
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 7, grp = lane >> 3;
  constexpr int U = NR <= 2 ? 4 : (NR <= 4 ? 2 : 1);  // 32-token groups per round of loads (two rounds in flight)
  const int64_t t0 = (int64_t)chunk * kStatsTok;
  int64_t t1 = t0 + kStatsTok;
  if (t1 > A.n) t1 = A.n;
  StatsLane<NR> L;
  stats_begin<NR>(L, A.qn, g, A.G, A.r0, li);
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
    uint32_t kw[U][8], vw[U][8];
    bool ok[U];
    int tok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tl = tb + 32 * u + lo;
      ok[u] = tl < nt;
      tok[u] = (int)(t0 + tl);
      const uint4 a0 = k0[u], a1 = k1[u], b0 = v0[u], b1 = v1[u];
      kw[u][0] = a0.x; kw[u][1] = a0.y; kw[u][2] = a0.z; kw[u][3] = a0.w;
      kw[u][4] = a1.x; kw[u][5] = a1.y; kw[u][6] = a1.z; kw[u][7] = a1.w;
      vw[u][0] = b0.x; vw[u][1] = b0.y; vw[u][2] = b0.z; vw[u][3] = b0.w;
      vw[u][4] = b1.x; vw[u][5] = b1.y; vw[u][6] = b1.z; vw[u][7] = b1.w;
    }
    stats_tokens<NR, U>(L, kw, vw, ok, tok, A.c2);
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
  __shared__ float ws[4][NR][kDecPart];
  stats_finish<NR>(L, ws, A.part + (((size_t)chunk * A.Hkv + g) * A.G + A.r0) * kDecPart, lane, wave, true);
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
  int64_t* pend;  // [2], see ContribArgs
  int deferred;   // 1: the new rows' terms are left pending (single-pass step)
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
  if (threadIdx.x == 0 && g == 0) {
    // pending rows: a single-pass step leaves the new position's terms
    // pending; a two-pass step adds them, and any left by an earlier step
    if (A.deferred) {
      A.pend[0] = A.n - 1;
    } else {
      A.pend[1] = A.pend[0];
      A.pend[0] = -1;
    }
  }
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
  int mode;           // which rows: see entry_of
  int e0, e1;         // mode 0: window entries e0 .. e1 - 1
  float c2;           // log2(e) / sqrt(d)
  const int64_t* pend;  // [2]: position whose terms are pending, position to add in this launch (-1: none)
};

// The launch's row list, per KV head: entry e holds the G query rows of one
// position. Mode 0 (a whole window): positions n - w + e for e in [e0, e1), +.
// Mode 1 (step): n - 1 (+), n - 1 - w (-), then pend[1] (+) if there is one.
// Mode 2 (flush): pend[1] (+) if there is one. Mode 3 (single-pass step):
// n - 1 - w (-), then pend[0] (+) if there is one. pp is the mode's pending
// position (read once per thread); one outside the rows the ring still holds
// (positions n - 1 - w .. n - 1) counts as none, so a state used before its
// init cannot send the row lookups out of the table.
__device__ __forceinline__ int64_t pending_of(const ContribArgs& A) {
  const int64_t pp = (A.mode == 1 || A.mode == 2) ? A.pend[1] : (A.mode == 3 ? A.pend[0] : -1);
  return (pp >= A.n - 1 - A.w && pp < A.n) ? pp : -1;
}
__device__ __forceinline__ int entry_count(const ContribArgs& A, int64_t pp) {
  const int has = pp >= 0 ? 1 : 0;
  return A.mode == 0 ? A.e1 - A.e0 : (A.mode == 1 ? 2 + has : (A.mode == 2 ? has : 1 + has));
}
__device__ __forceinline__ void entry_of(const ContribArgs& A, int64_t pp, int e, int64_t& pos, float& sign) {
  sign = 1.0f;
  if (A.mode == 0) {
    pos = A.n - A.w + A.e0 + e;
  } else if (A.mode == 1) {
    pos = e == 0 ? A.n - 1 : (e == 1 ? A.n - 1 - A.w : pp);
    sign = e == 1 ? -1.0f : 1.0f;
  } else if (A.mode == 2) {
    pos = pp;
  } else {
    pos = e == 0 ? A.n - 1 - A.w : pp;
    sign = e == 0 ? -1.0f : 1.0f;
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

// A launch's rows in LDS: exponent bias, C's start value, sign, position,
// kept argmax and slot per row, and the query and a operands (rows padded to
// 272 bytes, so 16 rows read at one column hit distinct banks). Reading the
// operands from global memory inside the token loop would wait for the loads
// of the next subtiles too (vector loads complete in order).
template <int ROWS>
struct ContribLds {
  float bias[ROWS], cinit[ROWS], sign[ROWS];
  int pos[ROWS], js[ROWS];
  int64_t row[ROWS];
  uint16_t op[2 * ROWS][kOpStride];
};

// k_dec_contrib<kInitRows> holds ContribLds<kInitRows> (71.5 KiB) and its
// per-token fp64 sums (8 KiB): two of them must fit in the CU's 160 KiB of LDS
// so that two workgroups share a CU.
static_assert(2 * (sizeof(ContribLds<kInitRows>) + sizeof(double) * tok_per_wg(kInitRows)) <= 160 * 1024,
              "whole-window contrib launches must keep two workgroups per CU");

// Fill L with the launch's rows of KV head g (padding rows up to a multiple of
// 16: p = 0); returns the number of 16-row blocks. Called by every thread;
// ends with a barrier.
template <int ROWS>
__device__ __forceinline__ int contrib_stage(const ContribArgs& A, ContribLds<ROWS>& L, int g) {
  const int64_t pp = pending_of(A);
  const int nrows = entry_count(A, pp) * A.G;
  const int nb = (nrows + 15) / 16;
  for (int rr = threadIdx.x; rr < nb * 16; rr += blockDim.x) {
    if (rr < nrows) {
      int64_t pos;
      float sign;
      entry_of(A, pp, rr / A.G, pos, sign);
      const int64_t r = trow(g, pos, rr % A.G, A.w, A.G);
      L.row[rr] = r;
      L.bias[rr] = A.T.bias[r];
      L.cinit[rr] = A.T.cinit[r];
      L.sign[rr] = sign;
      L.pos[rr] = (int)pos;
      L.js[rr] = A.T.jstar[r];
    } else {
      L.row[rr] = -1;
      L.bias[rr] = INFINITY;
      L.cinit[rr] = 0.f;
      L.sign[rr] = 0.f;
      L.pos[rr] = -1;
      L.js[rr] = -1;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb * 16 * 32; i += blockDim.x) {
    const int rr = i >> 5, c = i & 31;  // 32 chunks of 16 bytes: q then a_bf
    const int64_t r = L.row[rr];
    uint4 u = make_uint4(0, 0, 0, 0);
    if (r >= 0) u = *(const uint4*)((const char*)((c < 16 ? A.T.q : A.T.a_bf) + r * HD) + 16 * (c & 15));
    *(uint4*)((char*)&L.op[(c < 16 ? 0 : ROWS) + rr][0] + 16 * (c & 15)) = u;
  }
  __syncthreads();
  return nb;
}

// One 16-row block as a lane holds it: the query and a operands of row l%16
// and C's start value, exponent bias, sign, position and kept argmax of its
// four rows 4 (l/16) + i.
struct BlockRegs {
  bf16x8 qa[4], aa[4];
  float cinit[4], bias[4], sign[4];
  int pos[4], js[4];
};

// ||v_j||^2 of this lane's token: exact bf16 squares, fp32 sums over the
// lane's 32 dims, then over the token's four lanes (same order in each).
__device__ __forceinline__ float token_vnorm(const bf16x8 (&vb)[4]) {
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
  return rows4_sum(n0 + n1);
}

// The signed terms of one block for this lane's token tok (row l%16 of a
// 16-token subtile), added to acc in row order: X = Q K^T and
// C = a V^T - ||a||^2/2 on MFMA, then per (row, token) r^2 ||a - v_j||^2 with
// r = p / (1 - p), for tokens the row sees other than its kept argmax. Every
// element's value depends only on its row's stored state and its token,
// whatever else shares the block or the launch, so a row's terms are the same
// bit for bit in every kernel that uses this.
__device__ __forceinline__ void block_terms(const BlockRegs& B, const bf16x8 (&kb)[4], const bf16x8 (&vb)[4],
                                            float nvj, int tok, float c2, double& acc) {
  f32x4 X = {}, C = {B.cinit[0], B.cinit[1], B.cinit[2], B.cinit[3]};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) X = mfma16(B.qa[ks], kb[ks], X);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) C = mfma16(B.aa[ks], vb[ks], C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // branch-free: tokens the row does not see, and its kept argmax, get 0
    const float p = __builtin_amdgcn_exp2f(fmaf(X[i], c2, -B.bias[i]));
    const float rr = p * __builtin_amdgcn_rcpf(1.0f - p);
    const float c = rr * rr * fmaxf(fmaf(-2.0f, C[i], nvj), 0.0f);
    acc += (double)((tok <= B.pos[i] && tok != B.js[i]) ? B.sign[i] * c : 0.0f);
  }
}

// The signed terms of token tok over the staged rows, summed in fp64 in a
// fixed order (blocks, then rows); the sum is returned in all four lanes of
// the token.
template <int ROWS>
__device__ __forceinline__ double contrib_token(const ContribLds<ROWS>& L, int nb, const bf16x8 (&kb)[4],
                                                const bf16x8 (&vb)[4], int tok, int lane, float c2) {
  const int q4 = lane >> 4, l16 = lane & 15;
  const float nvj = token_vnorm(vb);
  double acc = 0.0;
  for (int b = 0; b < nb; ++b) {
    BlockRegs B;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      B.qa[ks] = *(const bf16x8*)((const char*)&L.op[16 * b + l16][0] + opoff(lane, ks));
      B.aa[ks] = *(const bf16x8*)((const char*)&L.op[ROWS + 16 * b + l16][0] + opoff(lane, ks));
    }
    const int base = 16 * b + 4 * q4;  // this lane's four rows
    const float4 c4 = *(const float4*)(&L.cinit[base]);
    const float4 bi = *(const float4*)(&L.bias[base]);
    const float4 sg = *(const float4*)(&L.sign[base]);
    const int4 ps = *(const int4*)(&L.pos[base]);
    const int4 js = *(const int4*)(&L.js[base]);
    B.cinit[0] = c4.x; B.cinit[1] = c4.y; B.cinit[2] = c4.z; B.cinit[3] = c4.w;
    B.bias[0] = bi.x; B.bias[1] = bi.y; B.bias[2] = bi.z; B.bias[3] = bi.w;
    B.sign[0] = sg.x; B.sign[1] = sg.y; B.sign[2] = sg.z; B.sign[3] = sg.w;
    B.pos[0] = ps.x; B.pos[1] = ps.y; B.pos[2] = ps.z; B.pos[3] = ps.w;
    B.js[0] = js.x; B.js[1] = js.y; B.js[2] = js.z; B.js[3] = js.w;
    block_terms(B, kb, vb, nvj, tok, c2, acc);
  }
  return rows4_sum(acc);
}

// The first 16 rows of a launch's list straight into registers (for a list
// of at most 16 rows; padding rows as contrib_stage makes them).
__device__ __forceinline__ void load_block_regs(const ContribArgs& A, int g, int lane, BlockRegs& B) {
  const int64_t pp = pending_of(A);
  const int nrows = entry_count(A, pp) * A.G;
  auto locate = [&](int rr, int64_t& r, int64_t& pos, float& sign) {
    if (rr >= nrows) return false;
    entry_of(A, pp, rr / A.G, pos, sign);
    r = trow(g, pos, rr % A.G, A.w, A.G);
    return true;
  };
  int64_t r, pos;
  float sign;
  const bool ok = locate(lane & 15, r, pos, sign);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    B.qa[ks] = ok ? *(const bf16x8*)((const char*)(A.T.q + r * HD) + opoff(lane, ks)) : bf16x8{};
    B.aa[ks] = ok ? *(const bf16x8*)((const char*)(A.T.a_bf + r * HD) + opoff(lane, ks)) : bf16x8{};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (locate(4 * (lane >> 4) + i, r, pos, sign)) {
      B.cinit[i] = A.T.cinit[r];
      B.bias[i] = A.T.bias[r];
      B.sign[i] = sign;
      B.pos[i] = (int)pos;
      B.js[i] = A.T.jstar[r];
    } else {
      B.cinit[i] = 0.f;
      B.bias[i] = INFINITY;
      B.sign[i] = 0.f;
      B.pos[i] = -1;
      B.js[i] = -1;
    }
  }
}

// Per (chunk of tok_per_wg(ROWS) tokens, KV head): each wave takes 16-token
// subtiles (wave, wave + 4, ...) with K and V read straight into the MFMA
// operands, the next two subtiles' loads in flight while one is processed.
template <int ROWS>
__global__ __launch_bounds__(256) void k_dec_contrib(ContribArgs A) {
  constexpr int kTokPerWg = tok_per_wg(ROWS);
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = lane >> 4, l16 = lane & 15;
  __shared__ __attribute__((aligned(16))) ContribLds<ROWS> cl;
  // per-token sums of this chunk, added to the score once every subtile is done
  // (a read-modify-write per subtile would wait for the prefetched loads too)
  __shared__ double s_tot[kTokPerWg];
  const int nb = contrib_stage<ROWS>(A, cl, g);
  if (nb == 0) return;
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
    const double total = contrib_token<ROWS>(cl, nb, kb, vb, (int)t0 + sub * 16 + l16, lane, A.c2);
    if (q4 == 0) s_tot[sub * 16 + l16] = total;
  };
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

// ---------------------------------------------------------------------------- single-pass step

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTileTok = 64;                    // tokens per LDS tile
constexpr int kTileBytes = kTileTok * HD * 2;   // 16 KiB per tensor
constexpr int kFusedRows = 16;                  // staged rows: leaving G + pending G (G <= 8)
constexpr int kTileBufs = 4;                    // LDS tile buffers: three tiles in flight

// Chunk permutation of token row t inside a tile: a bijection on t mod 16, so
// the 16 rows of a subtile read at one logical column hit 16 distinct 16-byte
// bank groups.
__device__ __forceinline__ int tswz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier ordering LDS traffic only (tile loads still in flight are
// waited for with wait_vmcnt first).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct-to-LDS loads of token rows [tok0, tok0 + 64) of one head (tok0 < n):
// wave instruction i = wave + 4 j fills tile bytes 1024 i .. +1023, lane l the
// 16-byte chunk (l % 16) of row 4 i + l / 16 with the row's logical chunk
// (l % 16) ^ tswz(row). The descriptor covers the rows before n only, so rows
// at or past n arrive as zeros (the consumers mask them; zero keeps 0 * V
// finite); base and range are scalar, a lane's address is its 32-bit offset
// inside the tile.
__device__ __forceinline__ void dec_issue_tile(const uint16_t* head, int64_t tok0, int64_t n, char* lds, int wave,
                                               int lane) {
  const int left = (int)(n - tok0);  // n < 2^31
  const __amdgpu_buffer_rsrc_t r = raw_rsrc(head + tok0 * HD, (left < kTileTok ? left : kTileTok) * (HD * 2));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int inst = wave + 4 * j;
    const int row = inst * 4 + (lane >> 4);
    const uint32_t off = (uint32_t)(row * (HD * 2) + (((lane & 15) ^ tswz(row)) << 4));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + inst * 1024), 16, off, 0, 0, 0);
  }
}

// The statistics share of one 64-token LDS tile for lane group (swave, grp):
// tokens 32 u + 8 swave + grp, u = 0, 1 (the token order of k_dec_stats).
template <int NR>
__device__ __forceinline__ void stats_tile(StatsLane<NR>& L, const char* kt, const char* vt, int swave, int grp,
                                           int li, int t, int64_t t0, int nt, float c2) {
  uint32_t kw[2][8], vw[2][8];
  bool ok[2];
  int tok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 32 * u + swave * 8 + grp;
    const int tl = t * kTileTok + row;
    ok[u] = tl < nt;
    tok[u] = (int)(t0 + tl);
    const int o0 = row * 256 + ((li ^ tswz(row)) << 4), o1 = row * 256 + (((8 + li) ^ tswz(row)) << 4);
    const uint4 k0 = *(const uint4*)(kt + o0), k1 = *(const uint4*)(kt + o1);
    const uint4 v0 = *(const uint4*)(vt + o0), v1 = *(const uint4*)(vt + o1);
    kw[u][0] = k0.x; kw[u][1] = k0.y; kw[u][2] = k0.z; kw[u][3] = k0.w;
    kw[u][4] = k1.x; kw[u][5] = k1.y; kw[u][6] = k1.z; kw[u][7] = k1.w;
    vw[u][0] = v0.x; vw[u][1] = v0.y; vw[u][2] = v0.z; vw[u][3] = v0.w;
    vw[u][4] = v1.x; vw[u][5] = v1.y; vw[u][6] = v1.z; vw[u][7] = v1.w;
  }
  stats_tokens<NR, 2>(L, kw, vw, ok, tok, c2);
}

struct FusedArgs {
  StatsArgs s;    // the new position's rows (r0 = 0, nr = G)
  ContribArgs c;  // mode 3: leaving rows and the pending rows
  int chunk_tok;  // tokens per workgroup (k_dec_fused8: a multiple of 64, >= kStatsTok)
};

// One step in one pass over K and V (per chunk of kStatsTok tokens, KV head):
// 64-token tiles of K and V land in LDS (four buffers, three tiles in flight);
// per tile every lane group takes two tokens of the new rows' statistics
// (StatsLane, as k_dec_stats) and every wave one 16-token subtile of terms of
// the leaving rows (-) and of the rows whose terms the previous step left
// pending (+) (contrib_token, as k_dec_contrib). The new rows' terms need
// their full statistics, so they stay pending until the next step or a flush.
template <int NR>
__global__ __launch_bounds__(256) void k_dec_fused(FusedArgs F) {
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 7, grp = lane >> 3, q4 = lane >> 4, l16 = lane & 15;
  __shared__ __attribute__((aligned(1024))) char kbuf[kTileBufs][kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vbuf[kTileBufs][kTileBytes];
  __shared__ __attribute__((aligned(16))) ContribLds<kFusedRows> cl;
  __shared__ double s_tot[kStatsTok];
  static_assert(4 * NR * kDecPart * sizeof(float) <= sizeof(kbuf), "stats merge space");
  const int nb = contrib_stage<kFusedRows>(F.c, cl, g);
  StatsLane<NR> L;
  stats_begin<NR>(L, F.s.qn, g, F.s.G, 0, li);
  const int64_t n = F.s.n;
  const int64_t t0 = (int64_t)chunk * kStatsTok;
  const int nt = (int)((n - t0) < kStatsTok ? (n - t0) : kStatsTok);
  const int ntiles = (nt + kTileTok - 1) / kTileTok;
  const uint16_t* kh = F.s.k + (size_t)g * F.s.n_max * HD;
  const uint16_t* vh = F.s.v + (size_t)g * F.s.n_max * HD;
  const float c2 = F.s.c2;
  for (int t = 0; t < kTileBufs - 1 && t < ntiles; ++t) {
    dec_issue_tile(kh, t0 + (int64_t)t * kTileTok, n, kbuf[t], wave, lane);
    dec_issue_tile(vh, t0 + (int64_t)t * kTileTok, n, vbuf[t], wave, lane);
  }
  for (int t = 0; t < ntiles; ++t) {
    // per wave 8 loads per tile, in issue order: the loads of the (at most
    // two) later tiles in flight may be outstanding once tile t has landed
    if (t + 2 < ntiles) wait_vmcnt<16>(); else if (t + 1 < ntiles) wait_vmcnt<8>(); else wait_vmcnt<0>();
    lds_barrier();  // tile t visible to every wave; tile t - 1's buffers are free
    if (t + 3 < ntiles) {
      const int b3 = (t + 3) % kTileBufs;
      dec_issue_tile(kh, t0 + (int64_t)(t + 3) * kTileTok, n, kbuf[b3], wave, lane);
      dec_issue_tile(vh, t0 + (int64_t)(t + 3) * kTileTok, n, vbuf[b3], wave, lane);
    }
    const char* kt = kbuf[t % kTileBufs];
    const char* vt = vbuf[t % kTileBufs];
    stats_tile<NR>(L, kt, vt, wave, grp, li, t, t0, nt, c2);
    {
      const int row = 16 * wave + l16;
      bf16x8 kb[4], vb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int o = row * 256 + (((4 * ks + q4) ^ tswz(row)) << 4);
        kb[ks] = *(const bf16x8*)(kt + o);
        vb[ks] = *(const bf16x8*)(vt + o);
      }
      const double total = contrib_token<kFusedRows>(cl, nb, kb, vb, (int)t0 + t * kTileTok + row, lane, c2);
      if (q4 == 0) s_tot[t * kTileTok + row] = total;
    }
  }
  lds_barrier();  // every wave is done with the tiles: their space takes the stats merge
  stats_finish<NR>(L, reinterpret_cast<float (*)[NR][kDecPart]>(&kbuf[0][0]),
                   F.s.part + (((size_t)chunk * F.s.Hkv + g) * F.s.G) * kDecPart, lane, wave, true);
  double* S = F.c.S64 + (size_t)g * F.c.n_max;
  const double invG = 1.0 / (double)F.c.G;
  for (int i = threadIdx.x; i < nt; i += blockDim.x) S[t0 + i] += s_tot[i] * invG;
}

// Rebuild: the score cleared; nothing stays pending (the rebuild scores every window row).
// The single-pass step with eight waves (two per SIMD), for at most four
// rows per position (the register budget of 512 threads; the leaving and
// pending rows then make one 16-row block, held in registers). Waves 4-7
// load the 64-token tiles into LDS (five buffers, all of LDS: four tiles in
// flight) and take the new rows' statistics (two tokens per lane group and
// tile, in the token order of k_dec_stats; with the same chunks the
// statistics are those of k_dec_stats bit for bit, with the longer chunks of
// long contexts they agree to fp32 rounding); waves 0-3 take the terms of one
// 16-token subtile each and add them to the score with fp64 atomic adds (one
// per token and launch, so the order does not matter), so they never wait
// for tile loads of their own and each SIMD interleaves an MFMA-heavy and a
// VALU-heavy wave.
template <int NR>
__global__ __launch_bounds__(512) void k_dec_fused8(FusedArgs F) {
  static_assert(NR <= 4, "register budget");
  constexpr int NB = 5;
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 7, grp = lane >> 3, l16 = lane & 15, q4 = lane >> 4;
  const bool stats_wave = wave >= 4;
  const int swave = wave & 3;
  __shared__ __attribute__((aligned(1024))) char kbuf[NB][kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vbuf[NB][kTileBytes];
  static_assert(4 * NR * kDecPart * sizeof(float) <= sizeof(kbuf), "stats merge space");
  BlockRegs B;
  load_block_regs(F.c, g, lane, B);
  StatsLane<NR> L;
  stats_begin<NR>(L, F.s.qn, g, F.s.G, 0, li);
  const int64_t n = F.s.n;
  const int64_t t0 = (int64_t)chunk * F.chunk_tok;
  const int nt = (int)((n - t0) < F.chunk_tok ? (n - t0) : F.chunk_tok);
  const int ntiles = (nt + kTileTok - 1) / kTileTok;
  const uint16_t* kh = F.s.k + (size_t)g * F.s.n_max * HD;
  const uint16_t* vh = F.s.v + (size_t)g * F.s.n_max * HD;
  const float c2 = F.s.c2;
  double* S = F.c.S64 + (size_t)g * F.c.n_max;
  const double invG = 1.0 / (double)F.c.G;
  // tile loads, statistics waves only: per tensor 16 wave loads of 1 KiB, wave 4 + s issues s, s + 4, s + 8, s + 12
  auto issue = [&](int64_t tok0, char* kd, char* vd) {
    dec_issue_tile(kh, tok0, n, kd, swave, lane);
    dec_issue_tile(vh, tok0, n, vd, swave, lane);
  };
  if (stats_wave)
    for (int t = 0; t < NB - 1 && t < ntiles; ++t) issue(t0 + (int64_t)t * kTileTok, kbuf[t], vbuf[t]);
  for (int t = 0; t < ntiles; ++t) {
    if (stats_wave) {
      // 8 loads per tile: the loads of the (at most three) later tiles in flight may be outstanding
      const int ahead = ntiles - 1 - t;
      if (ahead >= 3) wait_vmcnt<24>(); else if (ahead == 2) wait_vmcnt<16>(); else if (ahead == 1) wait_vmcnt<8>();
      else wait_vmcnt<0>();
    }
    lds_barrier();  // tile t visible to every wave; tile t - 1's buffers are free
    const char* kt = kbuf[t % NB];
    const char* vt = vbuf[t % NB];
    if (stats_wave) {
      if (t + NB - 1 < ntiles) {
        const int b = (t + NB - 1) % NB;
        issue(t0 + (int64_t)(t + NB - 1) * kTileTok, kbuf[b], vbuf[b]);
      }
      stats_tile<NR>(L, kt, vt, swave, grp, li, t, t0, nt, c2);
    } else {
      const int row = 16 * wave + l16;
      bf16x8 kb[4], vb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int o = row * 256 + (((4 * ks + q4) ^ tswz(row)) << 4);
        kb[ks] = *(const bf16x8*)(kt + o);
        vb[ks] = *(const bf16x8*)(vt + o);
      }
      const int tok = (int)t0 + t * kTileTok + row;
      double acc = 0.0;
      block_terms(B, kb, vb, token_vnorm(vb), tok, c2, acc);
      const double total = rows4_sum(acc);
      if (q4 == 0 && tok < n) atomicAdd(&S[tok], total * invG);
    }
  }
  lds_barrier();  // every wave is done with the tiles: their space takes the stats merge
  stats_finish<NR>(L, reinterpret_cast<float (*)[NR][kDecPart]>(&kbuf[0][0]),
                   F.s.part + (((size_t)chunk * F.s.Hkv + g) * F.s.G) * kDecPart, lane, swave, stats_wave);
}

__global__ void k_dec_zero(double* p, int64_t count, int64_t* pend) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.0;
  if (i == 0) pend[0] = -1;
}

// Flush: the pending position becomes the one this launch adds.
__global__ void k_dec_pend_take(int64_t* pend) {
  pend[1] = pend[0];
  pend[0] = -1;
}

// The kept score to fp32; reports (when status is given) terms still pending.
__global__ void k_dec_tof32(const double* S64, float* out, int64_t n, int64_t n_max, int Hkv, const int64_t* pend,
                            int32_t* status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0 && status != nullptr && pend[0] >= 0) atomicOr(status, kStatusPending);
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
  S.pend = (int64_t*)take(2 * sizeof(int64_t));
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
  if (mode != 0) {  // a step's (at most 3G <= 48) or a flush's rows: one launch
    const dim3 grid((unsigned)((n + tok_per_wg(kContribRows) - 1) / tok_per_wg(kContribRows)), Hkv);
    ContribArgs a{(const uint16_t*)k, (const uint16_t*)v, S.T, S.S64, n, n_max, w, G, mode, 0, 0, c2, S.pend};
    k_dec_contrib<kContribRows><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  // a whole window: launches of up to kInitRows rows, fewer K/V reads than
  // 64-row launches while two workgroups still fit a CU (256-row launches,
  // one per CU, were slower)
  const int per = kInitRows / G;  // window entries per launch (G <= 16)
  const dim3 grid((unsigned)((n + tok_per_wg(kInitRows) - 1) / tok_per_wg(kInitRows)), Hkv);
  for (int e0 = 0; e0 < w; e0 += per) {
    const int e1 = e0 + per < w ? e0 + per : w;
    ContribArgs a{(const uint16_t*)k, (const uint16_t*)v, S.T, S.S64, n, n_max, w, G, 0, e0, e1, c2, S.pend};
    k_dec_contrib<kInitRows><<<grid, 256, 0, st>>>(a);
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
  LoadArgs la{(const uint16_t*)q, ws.rs, S.T, S.S64, n, n_max, w, Hq, Hkv, S.pend};
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
                status, S.pend, 0};
  k_dec_merge<<<Hkv, 64 * G, 0, st>>>(ma);
  return launch_decode_contrib(k, v, n, n_max, w, G, Hkv, S, 1, st);
}

hipError_t launch_decode_step_deferred(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                                       int32_t w, int32_t Hq, int32_t Hkv, const DecState& S, int32_t* status,
                                       hipStream_t st) {
  const int G = Hq / Hkv;
  if (G > kRowBatch) return launch_decode_step(q_new, k, v, n, n_max, w, Hq, Hkv, S, status, st);
  const float c2 = kLog2e / sqrtf((float)HD);
  // k_dec_fused8 (one workgroup per CU by LDS): chunks sized so that the grid
  // is about one wave of workgroups (no second round with its pipeline refill
  // and tail), never below kStatsTok (the partials buffer holds n_max /
  // kStatsTok chunks); k_dec_fused keeps kStatsTok (its per-token sums sit in LDS)
  int64_t chunk_tok = kStatsTok;
  if (G <= kFused8MaxG) {
    const int64_t cus = device_cu_count();
    const int64_t per = ((n * Hkv + cus - 1) / cus + 63) / 64 * 64;
    if (per > chunk_tok) chunk_tok = per;
  }
  const int nch = (int)((n + chunk_tok - 1) / chunk_tok);
  FusedArgs f{StatsArgs{(const uint16_t*)q_new, (const uint16_t*)k, (const uint16_t*)v, S.part, n, n_max, G, Hkv,
                        nch, 0, G, c2},
              ContribArgs{(const uint16_t*)k, (const uint16_t*)v, S.T, S.S64, n, n_max, w, G, 3, 0, 0, c2,
                          S.pend},
              (int)chunk_tok};
  const dim3 grid(nch, Hkv);
  static_assert(kFused8MaxG == 4, "the switch below sends G = 1..4 to k_dec_fused8");
  if (G > kFused8MaxG && chunk_tok != kStatsTok) return hipErrorInvalidValue;  // k_dec_fused's chunks
  switch (G) {
    case 1: k_dec_fused8<1><<<grid, 512, 0, st>>>(f); break;
    case 2: k_dec_fused8<2><<<grid, 512, 0, st>>>(f); break;
    case 3: k_dec_fused8<3><<<grid, 512, 0, st>>>(f); break;
    case 4: k_dec_fused8<4><<<grid, 512, 0, st>>>(f); break;
    case 5: k_dec_fused<5><<<grid, 256, 0, st>>>(f); break;
    case 6: k_dec_fused<6><<<grid, 256, 0, st>>>(f); break;
    case 7: k_dec_fused<7><<<grid, 256, 0, st>>>(f); break;
    default: k_dec_fused<8><<<grid, 256, 0, st>>>(f); break;
  }
  DMergeArgs ma{S.part, (const uint16_t*)q_new, (const uint16_t*)v, S.T, S.S64, n, n_max, G, Hkv, w, nch,
                status, S.pend, 1};
  k_dec_merge<<<Hkv, 64 * G, 0, st>>>(ma);
  return hipGetLastError();
}

hipError_t launch_decode_flush(const void* k, const void* v, int64_t n, int64_t n_max, int32_t w, int32_t Hq,
                               int32_t Hkv, const DecState& S, hipStream_t st) {
  k_dec_pend_take<<<1, 1, 0, st>>>(S.pend);
  return launch_decode_contrib(k, v, n, n_max, w, Hq / Hkv, Hkv, S, 2, st);
}

hipError_t launch_decode_rebuild(const void* k, const void* v, int64_t n, int64_t n_max, int32_t w, int32_t Hq,
                                 int32_t Hkv, const DecState& S, int32_t* status, hipStream_t st) {
  const int G = Hq / Hkv;
  const int64_t cnt = (int64_t)Hkv * n_max;
  k_dec_zero<<<(unsigned)((cnt + 255) / 256), 256, 0, st>>>(S.S64, cnt, S.pend);
  StarAllArgs sa{S.T, S.S64, n, n_max, w, G};
  k_dec_star_all<<<Hkv, 64, 0, st>>>(sa);
  (void)status;
  return launch_decode_contrib(k, v, n, n_max, w, G, Hkv, S, 0, st);
}

hipError_t launch_decode_scores(const DecState& S, int64_t n, int64_t n_max, int32_t Hkv, float* out,
                                int32_t* status, hipStream_t st) {
  const int64_t tot = (int64_t)Hkv * n;
  k_dec_tof32<<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(S.S64, out, n, n_max, Hkv, S.pend, status);
  return hipGetLastError();
}

hipError_t launch_decode_select(const DecState& S, int64_t n, int64_t n_max, int32_t w, int32_t Hq, int32_t Hkv,
                                int32_t pool_kernel, int64_t n_evict, float* out_scores, int64_t* out_idx,
                                int32_t* status, hipStream_t st) {
  const Shape sh{n_max, w, Hq, Hkv, HD};
  Workspace ws = carve_workspace(S.ws_base, sh, true);  // S [Hkv][n] and select scratch for n <= n_max
  hipError_t e = launch_decode_scores(S, n, n_max, Hkv, ws.S, status, st);
  if (e == hipSuccess) e = launch_init(ws.status, nullptr, ws.sel, Hkv, st);
  if (e == hipSuccess)
    e = launch_select(ws.S, n, w, Hkv, pool_kernel, n_evict, out_scores, out_idx, status, nullptr, ws.sel, st);
  return e;
}

}  // namespace dropkv
