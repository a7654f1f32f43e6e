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
//          never stored. Writes per-chunk partials (m, l, A rounded to bf16,
//          tile of the max) and ||v_j||^2.
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

#include <climits>
#include <type_traits>

namespace dropkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;                  // head dim of this path
constexpr int TT = 64;                   // tokens per LDS tile
constexpr int TILE_BYTES = TT * HD * 2;  // 16 KiB per tensor per tile
constexpr int MAXW = 8;                  // waves per workgroup (row blocks of 32)
constexpr int PSTRIDE = HD / 2 + 4;      // 32-bit words per pass-1 partial (A[128] in bf16, m, l, best, mref)
constexpr int FXC = 8;                   // token chunks of the fix-up pass
constexpr int FXSTRIDE = HD + 2;         // floats per fix-up partial (sp, ps, D[128])

typedef __attribute__((address_space(3))) void lds_void;

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
__device__ __forceinline__ int pair_min(int x) {
  auto s = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return min((int)s[0], (int)s[1]);
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

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Lane byte offsets of the direct-to-LDS tile loads: load i of wave `wave`
// fetches token rows 4 (wave + i NW) .. +3 of the tile, lane l the 16-byte
// chunk (l%16) ^ swz(row) of row 4 (wave + i NW) + l/16. They do not depend
// on the tile. (Kept for NW >= 4 only: with fewer waves the offsets would
// occupy 8-16 registers, and those narrow workgroups recompute them per load.)
template <int NW>
struct DmaOff {
  static constexpr int kN = NW >= 4 ? 16 / NW : 1;
  uint32_t g[kN];
};

__device__ __forceinline__ uint32_t dma_offset(int inst, int lane) {
  const int row = inst * 4 + (lane >> 4);
  return (uint32_t)(row * 256 + (((lane & 15) ^ swz(row)) << 4));
}

template <int NW>
__device__ __forceinline__ DmaOff<NW> dma_offsets(int wave, int lane) {
  DmaOff<NW> o;
#pragma unroll
  for (int i = 0; i < DmaOff<NW>::kN; ++i) o.g[i] = dma_offset(wave + i * NW, lane);
  return o;
}

// Direct-to-LDS loads of the 64-token tile of one tensor that starts at
// token tok0: 16 wave instructions of 1 KiB (4 token rows each), instruction
// wave + i*NW of NW waves. The descriptor covers the tile's `rows` valid rows
// (64, or n - tok0 >= 1 on a ragged last tile), so the rows past n arrive as
// zeros (masked by every consumer, and zero keeps 0 * V finite) and nothing
// outside the tensor is read. Base, range and tile live in scalar registers:
// a lane's only address is its 32-bit offset inside the tile.
template <int NW>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ head, int64_t tok0, int rows, char* lds,
                                           int wave, int lane, const DmaOff<NW>& o) {
  const __amdgpu_buffer_rsrc_t r = raw_rsrc(head + tok0 * HD, rows * (HD * 2));
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i) {
    const int inst = wave + i * NW;
    const uint32_t off = NW >= 4 ? o.g[i < DmaOff<NW>::kN ? i : 0] : dma_offset(inst, lane);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + inst * 1024), 16, off, 0, 0, 0);
  }
}

// Valid rows of tile tl of a range [r0, r1) of tokens: 64 for the full tiles
// 0 .. nfull - 1 (nfull = (r1 - r0) / 64, a scalar 32-bit test), else the rest.
__device__ __forceinline__ int tile_rows(int tl, int nfull, int64_t r0, int64_t r1) {
  return tl < nfull ? TT : (int)(r1 - (r0 + (int64_t)tl * TT));
}

// As tile_rows, and 0 for a tile past the last one (ntiles): loads through a
// descriptor of zero range read nothing and write zeros. Loops that issue
// their loads unconditionally this way give the compiler the same sequence
// of memory operations on every path, so it can place its own waits for a
// register loaded one tile ahead without draining the tile loads behind it.
__device__ __forceinline__ int tile_rows_or0(int tl, int ntiles, int nfull, int64_t r0, int64_t r1) {
  return tl < ntiles ? tile_rows(tl, nfull, r0, r1) : 0;
}

// ---------------------------------------------------------------------------- pass 1

struct P1Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t n;
  int64_t ld;  // token rows per KV head in k and v (>= n)
  int w, Rg, nw, tiles_per_chunk, Hkv;
  float c2;          // log2(e) / sqrt(d)
  uint32_t* part;    // [chunk][Hkv*Rg][PSTRIDE]
  float* nv;         // [Hkv][n]
  int32_t* status;   // cleared here (read by later kernels only)
  int32_t* flagcount;  // [Hkv], cleared here
  uint32_t* zero;    // select state cleared here
  int64_t zero_words;
};

// Per-lane LDS byte offsets inside a tile, for the first 32-token subtile.
// The swizzle only looks at the token index mod 16, so the second subtile
// (+32 rows), the second 16-token MFMA step (+16 rows) and the buffer index
// are plain additive constants that fold into the instructions' offset field.
struct LdsOff {
  int k[8];  // 16-byte operand chunks: token l%32, dims 16ks + 8(l/32) .. +7
  int v[8];  // transposing reads: [2 db + second]
};

__device__ __forceinline__ LdsOff lds_offsets(int lane) {
  const int h = lane >> 5, l32 = lane & 31, srcl = lane & 15, dh = (lane >> 4) & 1;
  LdsOff o;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) o.k[ks] = toff(l32, ks * 16 + h * 8);
  const int t0 = 4 * h + (srcl >> 2);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = 32 * db + 16 * dh + 4 * (srcl & 3);
    o.v[2 * db] = toff(t0, d);
    o.v[2 * db + 1] = toff(t0 + 8, d);
  }
  return o;
}

// The same offsets with the transposing reads' LDS base folded in: v[i]
// becomes the LDS byte address of element v[i] of the first V buffer at
// vbase (p1_tile subtracts that base again in the pointer arithmetic, so the
// reads stay derived from the buffer and the compiler still knows which
// array they read: it does not wait for the tile loads in flight into the
// other buffers). The V buffers follow the three K buffers, so the later
// ones start beyond the 16-bit offset field of an LDS read; with their base
// held in these registers (which the compiler must not split up again) every
// buffer, subtile and step offset is an immediate of at most 44 KiB, and no
// per-read address arithmetic is left in the loop.
__device__ __forceinline__ LdsOff with_v_base(LdsOff o, const char* vbase) {
  const uint32_t b = lds_addr(vbase);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int x = o.v[i] + (int)b;
    asm volatile("" : "+v"(x));
    o.v[i] = x;
  }
  return o;
}

// ||v_j||^2 of the tiles, computed by pass 1 while V sits in LDS: NW lanes
// per token (wave w takes tokens (64/NW) w .. +64/NW-1), each squaring 128/NW
// dims with two-term dot products (bf16 squares are exact, sums fp32), then
// a swizzle reduction over the NW lanes. The LDS offsets are per-lane
// constants.
// (Narrow workgroups, NW < 4, recompute the offsets instead of keeping 8-16.)
template <int NW>
struct VnOff {
  static constexpr int kN = NW >= 4 ? 16 / NW : 1;
  int o[kN];
};

template <int NW>
__device__ __forceinline__ int vn_offset(int wave, int lane, int c) {
  return toff(wave * (TT / NW) + lane / NW, (lane % NW) * (HD / NW) + c * 8);
}

template <int NW>
__device__ __forceinline__ VnOff<NW> vn_offsets(int wave, int lane) {
  VnOff<NW> r;
#pragma unroll
  for (int c = 0; c < VnOff<NW>::kN; ++c) r.o[c] = vn_offset<NW>(wave, lane, c);
  return r;
}

template <int NW>
__device__ __forceinline__ void p1_vnorms(const char* vb, const VnOff<NW>& vo, float* nvtile, int64_t ntok,
                                          int wave, int lane, int32_t* status) {
  (void)status;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int c = 0; c < 16 / NW; ++c) {
    const int o = NW >= 4 ? vo.o[c < VnOff<NW>::kN ? c : 0] : vn_offset<NW>(wave, lane, c);
    const uint4 u = *(const uint4*)(vb + o);
    const bf16x2 p0 = __builtin_bit_cast(bf16x2, u.x), p1 = __builtin_bit_cast(bf16x2, u.y);
    const bf16x2 p2 = __builtin_bit_cast(bf16x2, u.z), p3 = __builtin_bit_cast(bf16x2, u.w);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, a1, false);
  }
  float acc = a0 + a1;
  // sum over the NW consecutive lanes of a token, in DPP lane moves (no LDS
  // round trip): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror
  if (NW >= 2) acc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0xB1, 0xf, 0xf, false));
  if (NW >= 4) acc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0x4E, 0xf, 0xf, false));
  if (NW >= 8) acc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0x141, 0xf, 0xf, false));
  const int tt = wave * (TT / NW) + lane / NW;
  if (lane % NW == 0 && tt < ntok) nvtile[tt] = acc;
  DKV_CHECK(tt < TT, status);
}

// Online-softmax state of one window row, held by the lane pair (l, l ^ 32)
// that shares the row's column of X^T; each lane sees half of every subtile's
// tokens.
//  m_true : largest logit among this lane's tokens so far (exact; the two
//           lanes are combined by p1_row_max at the end);
//  best   : 32-token block of the first occurrence of m_true;
//  mref   : reference exponent (log2 domain) of l and O, i.e. l = sum 2^{x c - mref},
//           always equal in both lanes of the pair (O sums over both);
//  nb     : -mref, or 0 while mref is -inf (no finite logit yet).
// The reference only moves when a logit exceeds it by more than kLazy (a
// factor 2^8 in p), so the O/l rescale runs a few times per chunk instead of
// at every new maximum; p stays below 2^8, well inside bf16 and fp32 range.
constexpr float kLazy = 8.0f;

struct P1State {
  float m_true, mref, l;
  int best;
  float nb;
};

// The row's largest logit and the first block holding it, from the two lanes
// of the pair (lowest block among the lanes that attain it). All 64 lanes of
// the wave must be active.
__device__ __forceinline__ void p1_row_max(P1State& st) {
  const float m = pair_max(st.m_true);
  st.best = pair_min(st.m_true == m ? st.best : INT_MAX);
  st.m_true = m;
}

// One 64-token tile of pass 1 for this wave's 32 rows (X^T layout: lane = row).
// kb: the tile's K buffer; vb0: the first V buffer, whose LDS address
// off.v already holds (with_v_base); vofs: byte offset of the tile's V buffer
// from it.
template <bool MASK>
__device__ __forceinline__ void p1_tile(float c2, const char* kb, const char* vb0, int vofs, int64_t tokbase_tile,
                                        const LdsOff& off, int lane, int64_t pos,
                                        const bf16x8 (&qb)[8], P1State& st, f32x16 (&O)[4]) {
  const int h = lane >> 5;
  const int vb0_addr = (int)lds_addr(vb0);
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const char* kt = kb + sub * 32 * 256;
    const char* vt = vb0 + (vofs + sub * 32 * 256 - vb0_addr);
    bf16x8 ka[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[ks] = ld16(kt + off.k[ks]);
    f32x16 x = {};
    // Raised issue priority over each MFMA group: the wave sharing this SIMD
    // then tends to be in its VALU phase meanwhile (measured ~3% faster).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) x = mfma(ka[ks], qb[ks], x);
    __builtin_amdgcn_s_setprio(0);
    // O^T[d][row] += V^T[d][tok] P^T[tok][row]; k-slot 8h+i of step s is token
    // 16s + 8(i/4) + 4h + i%4 (the order in which X^T left the values in this
    // lane). The transposing reads are issued here, so that their latency
    // passes under the softmax below.
    bf16x8 va[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        va[s][db] = tr_pair(vt + s * 16 * 256 + off.v[2 * db], vt + s * 16 * 256 + off.v[2 * db + 1]);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t tokbase = tokbase_tile + sub * 32;
    if (MASK) {  // causal tail / ragged end: hide keys after this row's position
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int64_t tok = tokbase + (vv >> 2) * 8 + 4 * h + (vv & 3);
        if (tok > pos) x[vv] = -INFINITY;
      }
    }
    // this lane's running maximum over its own tokens (the chain starts from
    // the running value, so no NaN quieting of the raw MFMA outputs is
    // needed); the pair is combined only when the reference moves
    float mx = fmaxf(fmaxf(st.m_true, x[0]), x[1]);
#pragma unroll
    for (int vv = 2; vv < 16; vv += 2) mx = fmaxf(fmaxf(mx, x[vv]), x[vv + 1]);
    if (mx > st.m_true) {
      st.m_true = mx;
      st.best = (int)(tokbase >> 5);
    }
    if (__builtin_amdgcn_ballot_w64(mx * c2 > st.mref + kLazy)) {
      const float nref = pair_max(st.m_true) * c2;  // the same in both lanes of the row
      if (nref > st.mref) {
        const float alpha = (st.mref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.mref - nref);
        st.l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) O[db] *= alpha;
        st.mref = nref;
        st.nb = -nref;
      }
    }
    float e[16];
    e[0] = __builtin_amdgcn_exp2f(fmaf(x[0], c2, st.nb));
    e[1] = __builtin_amdgcn_exp2f(fmaf(x[1], c2, st.nb));
    float ls0 = e[0], ls1 = e[1];
#pragma unroll
    for (int vv = 2; vv < 16; vv += 2) {
      e[vv] = __builtin_amdgcn_exp2f(fmaf(x[vv], c2, st.nb));
      e[vv + 1] = __builtin_amdgcn_exp2f(fmaf(x[vv + 1], c2, st.nb));
      ls0 += e[vv];
      ls1 += e[vv + 1];
    }
    st.l += ls0 + ls1;
    bf16x8 pb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[s][i] = (__bf16)e[8 * s + i];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db] = mfma(va[s][db], pb[s], O[db]);
    __builtin_amdgcn_s_setprio(0);
  }
}

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

template <int B>
using IntC = std::integral_constant<int, B>;

// Tiles [0, n_clean) of a chunk end at or before the first window position,
// so no row needs the causal mask there.
__device__ __forceinline__ int clean_tiles(int64_t n, int w, int64_t t0, int ntiles) {
  const int64_t lim = n - w + 1 - t0;  // tokens of this chunk visible to every row
  if (lim <= 0) return 0;
  const int64_t c = lim / TT;
  return c < ntiles ? (int)c : ntiles;
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_pass1(P1Args A) {
  __shared__ __attribute__((aligned(1024))) char kbuf[3][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf[3][TILE_BYTES];
  // Per tile and wave: 32/NW direct-to-LDS loads, then (row group 0) one
  // ||v||^2 store. vmcnt counts both, in issue order.
  constexpr int kDmaPerTile = 32 / NW;
  const int chunk = blockIdx.x, rg = blockIdx.y, g = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int rb = rg * NW + wave;
  const int row = rb * 32 + l32;
  const bool active = rb * 32 < A.Rg;
  const bool row_ok = row < A.Rg;
  const int64_t t0 = (int64_t)chunk * A.tiles_per_chunk * TT;
  int64_t t1 = t0 + (int64_t)A.tiles_per_chunk * TT;
  if (t1 > A.n) t1 = A.n;
  const int ntiles = (int)((t1 - t0 + TT - 1) / TT);
  const int nfull = (int)((t1 - t0) / TT);  // tiles 0 .. nfull - 1 end at or before t1 <= n
  const int nclean = clean_tiles(A.n, A.w, t0, ntiles);
  const uint16_t* kh = A.k + (size_t)g * A.ld * HD;
  const uint16_t* vh = A.v + (size_t)g * A.ld * HD;
  float* nvh = A.nv + (size_t)g * A.n;
  const int64_t pos = A.n - A.w + ((row_ok ? row : 0) % A.w);
  const float c2 = A.c2;
  const LdsOff off = with_v_base(lds_offsets(lane), vbuf[0]);
  const DmaOff<NW> doff = dma_offsets<NW>(wave, lane);
  const VnOff<NW> vno = vn_offsets<NW>(wave, lane);
  {
    // state of this call that later kernels accumulate into
    const int64_t wg = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
    for (int64_t i = wg * blockDim.x + threadIdx.x; i < A.zero_words; i += nthr) A.zero[i] = 0u;
    if (wg == 0)
      for (int i = threadIdx.x; i < A.Hkv; i += blockDim.x) A.flagcount[i] = 0;
    if (wg == 0 && threadIdx.x == 0) *A.status = 0;
  }

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
  P1State st{-INFINITY, -INFINITY, 0.f, -1, 0.f};
  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};

  if (ntiles > 0) {
    issue_tile<NW>(kh, t0, tile_rows(0, nfull, t0, t1), kbuf[0], wave, lane, doff);
    issue_tile<NW>(vh, t0, tile_rows(0, nfull, t0, t1), vbuf[0], wave, lane, doff);
  }
  if (ntiles > 1) {
    issue_tile<NW>(kh, t0 + TT, tile_rows(1, nfull, t0, t1), kbuf[1], wave, lane, doff);
    issue_tile<NW>(vh, t0 + TT, tile_rows(1, nfull, t0, t1), vbuf[1], wave, lane, doff);
  }
  // Per tile the vector-memory ops are, in issue order: the ||v||^2 store of
  // tile t, then the loads of tile t+2; so `vmcnt <= one tile's loads` at the
  // top of tile t+1 means tile t+1 has landed.
  auto head = [&](int t, const char* vc, char* kn, char* vn) {
    const int64_t tb = t0 + (int64_t)t * TT;
    if (t + 1 < ntiles) wait_vmcnt<kDmaPerTile>(); else wait_vmcnt<0>();
    lds_barrier();  // tile t in LDS for every wave; tile t-1's buffer is free
    if (rg == 0) p1_vnorms<NW>(vc, vno, nvh + tb, t1 - tb, wave, lane, A.status);
    if (t + 2 < ntiles) {
      issue_tile<NW>(kh, tb + 2 * TT, tile_rows(t + 2, nfull, t0, t1), kn, wave, lane, doff);
      issue_tile<NW>(vh, tb + 2 * TT, tile_rows(t + 2, nfull, t0, t1), vn, wave, lane, doff);
    }
  };
  auto clean = [&](auto bc, int t) {
    constexpr int B = decltype(bc)::value;
    constexpr int N2 = (B + 2) % 3;
    head(t, vbuf[B], kbuf[N2], vbuf[N2]);
    if (active) p1_tile<false>(c2, kbuf[B], vbuf[0], B * TILE_BYTES, t0 + (int64_t)t * TT, off, lane, pos, qb, st, O);
  };
  int t = 0;
  for (; t + 3 <= nclean; t += 3) {
    clean(IntC<0>{}, t);
    clean(IntC<1>{}, t + 1);
    clean(IntC<2>{}, t + 2);
  }
  for (; t < ntiles; ++t) {  // at most two clean tiles, then the masked tail
    const int b = t % 3, nb = (t + 2) % 3;
    head(t, vbuf[b], kbuf[nb], vbuf[nb]);
    if (active) p1_tile<true>(c2, kbuf[b], vbuf[0], b * TILE_BYTES, t0 + (int64_t)t * TT, off, lane, pos, qb, st, O);
  }
  if (!active) return;
  const float l_tot = pair_sum(st.l);
  p1_row_max(st);
  if (!row_ok) return;
  DKV_CHECK(chunk < (int)gridDim.x && g < A.Hkv && row < A.Rg && t1 <= A.n, A.status);
  uint32_t* pr = A.part + ((size_t)chunk * A.Hkv * A.Rg + (size_t)g * A.Rg + row) * PSTRIDE;
  // lane holds O^T rows d = 32db + 8i + 4h + (0..3) of this row's column; A
  // is stored rounded to bf16 (nearest even), two dims per word: the merge
  // rounds a to bf16 for pass 2 anyway, and the partials are read once
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 lo = {(__bf16)O[db][4 * i], (__bf16)O[db][4 * i + 1]};
      const bf16x2 hi = {(__bf16)O[db][4 * i + 2], (__bf16)O[db][4 * i + 3]};
      *(uint2*)(pr + 16 * db + 4 * i + 2 * h) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  if (h == 0) {
    pr[HD / 2] = __float_as_uint(st.m_true);
    pr[HD / 2 + 1] = __float_as_uint(l_tot);
    pr[HD / 2 + 2] = (uint32_t)st.best;
    pr[HD / 2 + 3] = __float_as_uint(st.mref);
  }
}

// ---------------------------------------------------------------------------- merge

struct MergeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint32_t* part;
  int64_t n;
  int64_t ld;  // token rows per KV head in k (>= n)
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
  const uint32_t* prow = M.part + (size_t)row * PSTRIDE;
  // lane c (< 64) holds chunk c's (m, l, best); more chunks fold in 64 at a time
  float mx = -INFINITY;
  int bt = -1;
  for (int c0 = 0; c0 < M.nchunks; c0 += 64) {
    const int c = c0 + lane;
    const float mc = c < M.nchunks ? __uint_as_float(prow[c * cstride + HD / 2]) : -INFINITY;
    float wm = mc;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
    if (wm > mx) {
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(mc == wm);
      const int first = __ffsll((long long)hit) - 1;  // lowest chunk attaining the max
      const int bf = c < M.nchunks ? (int)prow[c * cstride + HD / 2 + 2] : 0;
      bt = __shfl(bf, first, 64);
      mx = wm;
    }
  }
  float l = 0.f, a0 = 0.f, a1 = 0.f;
  for (int c0 = 0; c0 < M.nchunks; c0 += 64) {
    const int c = c0 + lane;
    // chunk c holds l and A relative to its own reference exponent mref
    const float rc = c < M.nchunks ? __uint_as_float(prow[c * cstride + HD / 2 + 3]) : -INFINITY;
    const float lc = c < M.nchunks ? __uint_as_float(prow[c * cstride + HD / 2 + 1]) : 0.f;
    const float sc = (rc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(rc - mx * M.c2);
    float lw = lc * sc;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lw += __shfl_xor(lw, o, 64);
    l += lw;
    const int cn = (M.nchunks - c0) < 64 ? (M.nchunks - c0) : 64;
    int cc = 0;
    for (; cc + 16 <= cn; cc += 16) {  // sixteen chunk rows in flight
      uint32_t av[16];
      float sv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        av[u] = prow[(size_t)(c0 + cc + u) * cstride + lane];
        sv[u] = __shfl(sc, cc + u, 64);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        a0 = fmaf(__uint_as_float(av[u] << 16), sv[u], a0);
        a1 = fmaf(__uint_as_float(av[u] & 0xffff0000u), sv[u], a1);
      }
    }
    for (; cc < cn; ++cc) {
      const uint32_t av = prow[(size_t)(c0 + cc) * cstride + lane];
      const float sv = __shfl(sc, cc, 64);
      a0 = fmaf(__uint_as_float(av << 16), sv, a0);
      a1 = fmaf(__uint_as_float(av & 0xffff0000u), sv, a1);
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
    DKV_CHECK(bt >= 0 && (int64_t)bt * 32 < M.n, M.status);
    float x = -INFINITY;
    if (lane < 32 && tok <= pos && tok >= 0) {
      const uint16_t* qr = M.q + (size_t)row * HD;
      const uint16_t* kr = M.k + ((size_t)g * M.ld + tok) * HD;
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
  int64_t ld;  // token rows per KV head in k and v (>= n)
  int w, Rg, Hkv;
  float c2;
  RowStats rs;
  const int32_t* flagcount;
  float* fx;  // [FXC][Hkv*Rg][FXSTRIDE]
};

// Per flagged row and token chunk: sp = sum_{i != j*} p_i, ps = p_{j*} and
// D = sum_{i != j*} p_i (v_i - v_{j*}), with p_i = 2^{x_i c - bias}; for a
// workgroup of T >= 128 threads (T/128 threads per dimension of D).
template <int T>
__device__ __forceinline__ void fixup_chunk(const FixArgs& F, int c, int g) {
  static_assert(T >= HD && T % HD == 0, "fix-up needs a multiple of 128 threads");
  if (F.flagcount[g] == 0) return;
  const int tid = threadIdx.x;
  __shared__ float qs[HD], vstar[HD], ptile[T], red[T], redD[T];
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
      vstar[tid] = bf16_to_f32(F.v[((size_t)g * F.ld + js) * HD + tid]);
    }
    __syncthreads();
    float sp = 0.f, ps = 0.f, Dacc = 0.f;
    const int dim = tid & (HD - 1), sub = tid / HD;
    for (int64_t b = c0; b < hi; b += T) {
      const int64_t j = b + tid;
      float p = 0.f;
      if (j < hi) {
        const uint16_t* kr = F.k + ((size_t)g * F.ld + j) * HD;
        float acc = 0.f;
        for (int cc = 0; cc < HD; ++cc) acc = fmaf(qs[cc], bf16_to_f32(kr[cc]), acc);
        p = __builtin_amdgcn_exp2f(fmaf(acc, F.c2, -bias));
        if (j == js) { ps = p; p = 0.f; }
        sp += p;
      }
      ptile[tid] = p;
      __syncthreads();
      const int cnt = (int)((hi - b) < T ? (hi - b) : T);
      for (int t = sub; t < cnt; t += T / HD) {
        const float vv = bf16_to_f32(F.v[((size_t)g * F.ld + b + t) * HD + dim]);
        Dacc = fmaf(ptile[t], vv - vstar[dim], Dacc);
      }
      __syncthreads();
    }
    redD[tid] = Dacc;
    const float spt = block_sum<T>(sp, red);
    const float pst = block_sum<T>(ps, red);
    float* o = F.fx + ((size_t)c * F.Hkv * F.Rg + row) * FXSTRIDE;
    if (tid < HD) {
      float d = 0.f;
      for (int q = 0; q < T / HD; ++q) d += redD[q * HD + tid];
      o[2 + tid] = d;
    }
    if (tid == 0) { o[0] = spt; o[1] = pst; }
  }
}

__global__ __launch_bounds__(256) void k_fixup(FixArgs F) { fixup_chunk<256>(F, blockIdx.x, blockIdx.y); }

struct FoldArgs {
  FoldInfo f;
  int64_t n;
  float* S;
  int32_t* status;
};

// Adds the argmax terms of flagged rows into S, in row order (deterministic),
// and records R, L and the term in the row statistics.
__global__ __launch_bounds__(HD) void k_fold(FoldArgs F) {
  const int g = blockIdx.x;
  if (F.f.flagcount[g] == 0) return;
  const int tid = threadIdx.x;
  __shared__ float red[HD];
  for (int r = 0; r < F.f.Rg; ++r) {
    const int64_t row = (int64_t)g * F.f.Rg + r;
    if (!F.f.rs.flag[row]) continue;
    float R;
    int bits;
    const float val = fold_value<HD>(F.f, row, red, &R, &bits);
    const int js = F.f.rs.jstar[row];
    if (tid == 0) {
      if (js < 0 || js >= F.n) {
        atomicOr(F.status, kStatusNonFinite);
        continue;
      }
      F.f.rs.rest[row] = R;
      F.f.rs.L[row] = 1.0f + R;
      F.f.rs.fixval[row] = val;
      if (bits) atomicOr(F.status, bits);
      else F.S[(size_t)g * F.n + js] += val * F.f.invG;
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
  int32_t* status;
  // Tile schedule of the fast path. ctr null: workgroup `chunk` takes tiles
  // [chunk * tiles_per_chunk, ...) of its head. Otherwise it takes its static
  // share [chunk * stat_tiles, (chunk + 1) * stat_tiles) and then claims
  // tiles of the pool [pool0, tiles) one at a time from the counter
  // ctr[g * ctr_stride + rg] (zero before the launch), so workgroups on
  // faster CUs take more of them. The flagged path always takes static chunks.
  uint32_t* ctr;
  int ctr_stride, stat_tiles, pool0, tiles;
};

__device__ __forceinline__ void p2_tile(const P2Args& P, const char* kb, const char* vb,
                                        int64_t tokbase_tile, int lane, bool active, int rb,
                                        const bf16x8 (&qa)[8], const bf16x8 (&aa)[8],
                                        const float (&bias)[16], const float (&cinit)[16],
                                        const int (&jst)[16], float (*red)[TT][2], int wave) {
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
    // some row of this KV head takes its argmax term from the fix-up: that
    // (row, token) pair is left out here (jst[vv], -1 for none; n < 2^31)
    float t1 = 0.f, t2 = 0.f;
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      const bool skip = jst[vv] == (int)tok;
      const float p = skip ? 0.f : __builtin_amdgcn_exp2f(fmaf(x[vv], P.c2, -bias[vv]));
      const float r = p * __builtin_amdgcn_rcpf(1.0f - p);
      const float r2 = r * r;
      t2 += r2;
      t1 = fmaf(r2, cc[vv], t1);
    }
    t1 = pair_sum(t1);
    t2 = pair_sum(t2);
    if (h == 0) {
      red[wave][sub * 32 + l32][0] = t1;
      red[wave][sub * 32 + l32][1] = t2;
    }
  }
}

template <bool NVC>
__device__ __forceinline__ void p2_combine(const P2Args& P, float (*red)[TT][2], int nwa,
                                           int64_t tokbase_tile, int64_t chunk_end, int g,
                                           const char* vtile) {
  if (threadIdx.x < TT) {
    const int64_t tok = tokbase_tile + threadIdx.x;
    if (tok < chunk_end) {
      float T1 = 0.f, T2 = 0.f;
      for (int wv = 0; wv < nwa; ++wv) {
        T1 += red[wv][threadIdx.x][0];
        T2 += red[wv][threadIdx.x][1];
      }
      // sum_rows r^2 (||a||^2 - 2 a.v + ||v||^2) = ||v||^2 T2 - 2 T1
      float nvj;
      if constexpr (NVC) {  // from the tile's V row (bf16 squares are exact, fp32 sums)
        float acc = 0.f;
        for (int c = 0; c < HD; c += 8) {
          const bf16x8 x = ld16(vtile + toff((int)threadIdx.x, c));
#pragma unroll
          for (int i = 0; i < 8; ++i) acc = fmaf((float)x[i], (float)x[i], acc);
        }
        nvj = acc;
      } else {
        nvj = P.nv[(size_t)g * P.n + tok];
      }
      const float s = fmaxf(fmaf(nvj, T2, -2.0f * T1), 0.0f) * P.invG;
      DKV_CHECK(tok < P.n, P.status);
      P.S[((size_t)blockIdx.y * P.Hkv + g) * P.n + tok] = s;
    }
  }
}

// ---- row state from given statistics (no pass 1)

struct ImportArgs {
  const float* m;         // [rows] largest logit, natural units (x = q.k / sqrt(d))
  const float* rest;      // [rows] R = sum_{j != argmax} exp(x_j - x_max)
  const int32_t* argmax;  // [rows] lowest index attaining x_max (read where R < 1)
  const float* a;         // [rows][HD] attention output
  int64_t n, rows;
  int Rg;
  RowStats rs;
  int32_t* flagcount;
  int32_t* status;
};

// One wave per window row: what the merge would leave for pass 2 (bias, a in
// bf16 and ||a_bf16||^2, the flag of rows with p_max > 1/2 and their argmax),
// computed from statistics supplied by the caller, e.g. by a prefill
// attention kernel that saw the same rows.
__global__ __launch_bounds__(256) void k_import(ImportArgs I) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= I.rows) return;
  const int g = (int)(row / I.Rg);
  const float2 av = *(const float2*)(I.a + (size_t)row * HD + 2 * lane);
  const uint16_t b0 = f32_to_bf16_rne(av.x), b1 = f32_to_bf16_rne(av.y);
  const float f0 = bf16_to_f32(b0), f1 = bf16_to_f32(b1);
  float na = fmaf(f0, f0, f1 * f1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) na += __shfl_xor(na, o, 64);
  *(float2*)(I.rs.a + (size_t)row * HD + 2 * lane) = av;
  *(uint32_t*)(I.rs.a_bf + (size_t)row * HD + 2 * lane) = (uint32_t)b0 | ((uint32_t)b1 << 16);
  const float m = I.m[row], R = I.rest[row];
  bool bad = !finite_f(av.x) || !finite_f(av.y);
  bad = __builtin_amdgcn_ballot_w64(bad) != 0 || !finite_f(m) || !finite_f(R) || !(R >= 0.f);
  const bool flagged = !bad && R < 1.0f;
  const int js = flagged ? I.argmax[row] : -1;
  if (lane == 0) {
    const float L = 1.0f + R;
    I.rs.m[row] = m;
    I.rs.L[row] = L;
    I.rs.rest[row] = R;
    I.rs.na[row] = na;
    I.rs.bias[row] = m * kLog2e + __log2f(L);
    I.rs.jstar[row] = js;
    I.rs.flag[row] = flagged ? 1 : 0;
    I.rs.fixval[row] = 0.f;
    if (bad || (flagged && (js < 0 || js >= I.n))) atomicOr(I.status, kStatusNonFinite);
    else if (flagged) atomicAdd(&I.flagcount[g], 1);
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

// ||v_j||^2 of this lane's two tokens (l32 and 32 + l32) of the tile at tok0,
// which holds `rows` valid tokens (the rest read as zero): two 4-byte buffer
// loads into registers. Pass 2 issues them one tile ahead, before the next
// tile's K/V loads, so the wait for a tile's K/V also covers them (vector
// memory operations complete in issue order).
__device__ __forceinline__ float2 load_nv_pair(const float* nvh, int64_t tok0, int rows, int l32) {
  const __amdgpu_buffer_rsrc_t r = raw_rsrc(nvh + tok0, rows * 4);
  float2 o;
  o.x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)l32 * 4u, 0, 0));
  o.y = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)l32 * 4u + 128u, 0, 0));
  return o;
}

// Score terms of one subtile from y2 = 2 (x c - bias) = log2 p^2:
// t1 = sum_rows r^2 C, t2 = sum_rows r^2 with r = p / (1 - p).
template <int TIER>
__device__ __forceinline__ void p2_values(const float (&y2)[16], const f32x16& C, float& t1, float& t2) {
  float a1 = 0.f, a2 = 0.f, b1 = 0.f, b2 = 0.f;
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) {
    float r2;
    if (TIER == kTierSquare) {
      r2 = __builtin_amdgcn_exp2f(y2[vv]);
    } else {
      const float p = __builtin_amdgcn_exp2f(0.5f * y2[vv]);
      if (TIER == kTierSeries) {
        r2 = (p * p) * fmaf(p, fmaf(p, 3.0f, 2.0f), 1.0f);
      } else {
        const float r = p * __builtin_amdgcn_rcpf(1.0f - p);
        r2 = r * r;
      }
    }
    if (vv & 1) {
      b2 += r2;
      b1 = fmaf(r2, C[vv], b1);
    } else {
      a2 += r2;
      a1 = fmaf(r2, C[vv], a1);
    }
  }
  t1 = a1 + b1;
  t2 = a2 + b2;
}

// One 32-token subtile of the pass-2 fast path for this wave's 32 rows:
// returns this wave's share of the score of token l%32 (valid in lanes < 32).
// NVC (||v_j||^2 not known yet): returns the share of sum r^2 C and leaves
// that of sum r^2 in *q2out; the workgroup folds ||v_j||^2 in later.
template <bool MASK, bool NVC>
__device__ __forceinline__ float p2_sub(const char* kt, const char* vt, float nvj, float* q2out, const LdsOff& off,
                                        const bf16x8 (&qa)[8], const bf16x8 (&aa)[8],
                                        const float (&nb2)[16], const float (&cinit)[16], float c2x2,
                                        int64_t tok, int rbase, int w) {
  bf16x8 kb[8], vb[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kb[ks] = ld16(kt + off.k[ks]);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) vb[ks] = ld16(vt + off.k[ks]);
  // all sixteen operand reads in flight before the first MFMA waits on one
  __builtin_amdgcn_sched_barrier(0);
  f32x16 X = {}, C;
#pragma unroll
  for (int i = 0; i < 16; ++i) C[i] = cinit[i];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) X = mfma(qa[ks], kb[ks], X);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) C = mfma(aa[ks], vb[ks], C);
  float y2[16];
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) {
    y2[vv] = fmaf(X[vv], c2x2, nb2[vv]);
    if (MASK) {  // row rbase + 8(vv/4) + vv%4 sits at window position row % w
      const int rpos = (rbase + (vv >> 2) * 8 + (vv & 3)) % w;
      if (tok > (int64_t)rpos) y2[vv] = -INFINITY;
    }
  }
  float ym = fmaxf(fmaxf(y2[0], y2[1]), y2[2]);
#pragma unroll
  for (int vv = 3; vv < 15; vv += 2) ym = fmaxf(fmaxf(ym, y2[vv]), y2[vv + 1]);
  ym = fmaxf(ym, y2[15]);
  float q1, q2;
  if (__builtin_amdgcn_ballot_w64(ym > -24.0f)) {
    if (__builtin_amdgcn_ballot_w64(ym > -14.0f))
      p2_values<kTierExact>(y2, C, q1, q2);
    else
      p2_values<kTierSeries>(y2, C, q1, q2);
  } else {
    p2_values<kTierSquare>(y2, C, q1, q2);
  }
  // this wave's rows: sum r^2 (||a||^2 - 2 a.v + ||v||^2) = ||v||^2 q2 - 2 q1
  if constexpr (NVC) {
    *q2out = pair_sum(q2);
    return pair_sum(q1);
  } else {
    return pair_sum(fmaf(nvj, q2, -2.0f * q1));
  }
}

// NVC: ||v_j||^2 is computed from the tile in LDS, once per workgroup and
// token (tile_vnorms), instead of read from the array pass 1 writes (the path
// that starts from given row statistics); the waves' shares of sum r^2 C and
// sum r^2 are reduced separately and ||v_j||^2 is folded in per token.
template <int NW, bool NVC>
__global__ __launch_bounds__(NW * 64) void k_pass2(P2Args P, FixArgs F) {
  // The three K and three V tile buffers are separate variables, not one
  // [3][TILE_BYTES] array each: with a compile-time buffer index (the clean
  // loop below is unrolled over the buffers) the compiler can then tell that
  // a read of the current tile and the direct-to-LDS loads in flight into a
  // later tile's buffer do not overlap, and places no wait for those loads
  // before the read.
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILE_BYTES], kbuf1[TILE_BYTES], kbuf2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILE_BYTES], vbuf1[TILE_BYTES], vbuf2[TILE_BYTES];
  auto kbuf = [&](int i) -> char* { return i == 0 ? kbuf0 : (i == 1 ? kbuf1 : kbuf2); };
  auto vbuf = [&](int i) -> char* { return i == 0 ? vbuf0 : (i == 1 ? vbuf1 : vbuf2); };
  __shared__ float red3[3][NW][TT];
  __shared__ float red3b[NVC ? 3 : 1][NW][TT];  // NVC: the waves' shares of sum r^2 per token
  __shared__ float nvbuf[NVC ? 3 : 1][TT];  // NVC: ||v_j||^2 of the tiles, formed in LDS
  constexpr int kDmaPerTile = 32 / NW;  // direct-to-LDS instructions per wave and tile (K and V)
  const int chunk = blockIdx.x, rg = blockIdx.y, g = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int rb = rg * NW + wave;
  const bool active = rb * 32 < P.Rg;
  int nwa = (P.Rg - rg * NW * 32 + 31) / 32;  // active waves
  if (nwa > NW) nwa = NW;
  const int64_t t0 = (int64_t)chunk * P.tiles_per_chunk * TT;
  int64_t t1 = t0 + (int64_t)P.tiles_per_chunk * TT;
  if (t1 > P.n) t1 = P.n;
  const int ntiles = (int)((t1 - t0 + TT - 1) / TT);
  const int nfull = (int)((t1 - t0) / TT);  // tiles 0 .. nfull - 1 end at or before t1 <= n
  const uint16_t* kh = P.k + (size_t)g * P.n * HD;
  const uint16_t* vh = P.v + (size_t)g * P.n * HD;
  const float* __restrict__ nvg = NVC ? nullptr : P.nv + (size_t)g * P.n;
  float* __restrict__ Sout = P.S + ((size_t)blockIdx.y * P.Hkv + g) * P.n;
  const bool flagged = P.flagcount[g] != 0;
  const DmaOff<NW> doff = dma_offsets<NW>(wave, lane);

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

  // the fast path's first tile: its static share starts at chunk * stat_tiles
  const bool dyn = P.ctr != nullptr && !flagged;
  const int gbase = dyn ? chunk * P.stat_tiles : chunk * P.tiles_per_chunk;
  if (ntiles > 0) {
    const int64_t f0 = (int64_t)gbase * TT;
    const int r0 = dyn ? (int)(P.n - f0 < TT ? P.n - f0 : TT) : tile_rows(0, nfull, t0, t1);
    issue_tile<NW>(kh, f0, r0, kbuf(0), wave, lane, doff);
    issue_tile<NW>(vh, f0, r0, vbuf(0), wave, lane, doff);
  }

  if (flagged) {
    // per-tile path with the argmax exclusion of flagged rows (double-buffered)
    float (*red)[TT][2] = (float (*)[TT][2])&red3[0][0][0];
    static_assert(3 * NW * TT >= NW * TT * 2, "reduction buffer");
    // per row of this lane: the token whose term the fix-up supplies (-1: none)
    int jst[16];
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      const int rr = rb * 32 + (vv >> 2) * 8 + 4 * h + (vv & 3);
      jst[vv] = -1;
      if (active && rr < P.Rg) {
        const size_t row = (size_t)g * P.Rg + rr;
        if (P.rs.flag[row]) jst[vv] = P.rs.jstar[row];
      }
    }
    for (int it = 0; it < ntiles; ++it) {
      const int b = it & 1;
      tile_barrier();
      if (it + 1 < ntiles) {
        issue_tile<NW>(kh, t0 + (int64_t)(it + 1) * TT, tile_rows(it + 1, nfull, t0, t1), kbuf(b ^ 1), wave, lane,
                       doff);
        issue_tile<NW>(vh, t0 + (int64_t)(it + 1) * TT, tile_rows(it + 1, nfull, t0, t1), vbuf(b ^ 1), wave, lane,
                       doff);
      }
      p2_tile(P, kbuf(b), vbuf(b), t0 + (int64_t)it * TT, lane, active, rb, qa, aa, bias, cinit, jst, red, wave);
      __syncthreads();
      p2_combine<NVC>(P, red, nwa, t0 + (int64_t)it * TT, t1, g, vbuf(b));
    }
    // the argmax fix-up of this head's flagged rows (independent of pass 2):
    // fix-up chunks chunk, chunk + gridDim.x, ... of row group 0's workgroups
    if constexpr (NW >= 2) {
      if (rg == 0) {
        __syncthreads();
        for (int c = chunk; c < FXC; c += gridDim.x) fixup_chunk<NW * 64>(F, c, g);
      }
    }
    return;
  }

  // The fast path's vector-memory operations per tile are, in issue order:
  // wave 0's score store, the next tile's ||v||^2 loads, (wave 0, pooled
  // tiles) the claim of a later tile and the K/V loads of the tile after
  // next, so `vmcnt <= one tile's K/V loads` at the top of tile t means tile
  // t's K/V and ||v||^2 and the claim issued one tile earlier have landed.
  //
  // The workgroup's tiles are its static share [gbase, static_end), then
  // tiles claimed from the head's pool. The claim for local tile u goes out
  // (wave 0, one lane) at the top of tile u - 3; its answer reaches every
  // wave through LDS at the top of tile u - 2, where tile u's loads are
  // issued. Claims only grow, so a workgroup's tiles ascend; once a claim
  // runs past the pool, its sequence ends. gp / g0 / g1: global tiles of
  // local tiles t - 1, t, t + 1 (-1: none) before the top of tile t.
  // claim_slot[t % 2] is written before barrier t and read after it; the
  // next write to that slot (top of t + 2) follows barrier t + 1, which every
  // reader has reached.
  __shared__ int claim_slot[2];
  const int static_end = gbase + (dyn ? P.stat_tiles : ntiles);
  uint32_t* const ctrp = dyn ? P.ctr + (size_t)g * P.ctr_stride + rg : nullptr;
  uint32_t pend = 0;  // wave 0, lane 0: the claim in flight
  int gp = -1, g0 = ntiles > 0 ? gbase : -1, g1 = (gbase + 1 < static_end) ? gbase + 1 : -1;
  // rows of global tile gt (0 for none: zero-range loads)
  const int last_tile = P.tiles - 1;
  const int last_rows = (int)(P.n - (int64_t)last_tile * TT);
  auto trows = [&](int gt) -> int { return gt < 0 ? 0 : (gt == last_tile ? last_rows : TT); };
  // local tile t + 3 is a pooled tile whose claim goes out at the top of t
  // (g2: the global tile of local t + 2)
  auto claims_next = [&](int g2) { return dyn && g2 >= 0 && g2 + 1 >= static_end; };
  // ||v_j||^2 of this lane's tokens of the current tile and of the next one
  // (the latter loaded one tile ahead; not in NVC mode)
  float2 nv_cur = make_float2(0.f, 0.f), nv_next = make_float2(0.f, 0.f);
  if (!NVC) nv_next = load_nv_pair(nvg, (int64_t)(g0 < 0 ? 0 : g0) * TT, trows(g0), l32);
  issue_tile<NW>(kh, (int64_t)(g1 < 0 ? 0 : g1) * TT, trows(g1), kbuf(1), wave, lane, doff);
  issue_tile<NW>(vh, (int64_t)(g1 < 0 ? 0 : g1) * TT, trows(g1), vbuf(1), wave, lane, doff);
  const float c2x2 = 2.0f * P.c2;
  const LdsOff off = lds_offsets(lane);
  float nb2[16];
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) nb2[vv] = -2.0f * bias[vv];
  const int rbase = rb * 32 + 4 * h;  // first row of this lane's 16 (masked tiles only)
  // global tiles [0, ncg) end at or before the first window position: no row needs the mask
  const int ncg = clean_tiles(P.n, P.w, 0, P.tiles);
  // scores of tile t-1 (every wave wrote its partial before the barrier at tile t)
  static_assert(TT == 64, "one wave combines a tile");
  auto combine = [&](int gt, const float (*red)[TT], int lt) {
    if (wave == 0) {  // wave-uniform: the other waves skip it with a scalar branch
      const int64_t tok = (int64_t)gt * TT + threadIdx.x;
      if (tok < P.n) {
        float sacc = 0.f;
        for (int wv = 0; wv < nwa; ++wv) sacc += red[wv][threadIdx.x];
        if constexpr (NVC) {  // sacc = sum r^2 C; ||v_j||^2 and sum r^2 from the tile's buffers
          const int b = lt % 3;
          float s2 = 0.f;
          for (int wv = 0; wv < nwa; ++wv) s2 += red3b[b][wv][threadIdx.x];
          sacc = fmaf(nvbuf[b][threadIdx.x], s2, -2.0f * sacc);
        }
        DKV_CHECK(tok < P.n && gt < P.tiles, P.status);
        Sout[tok] = fmaxf(sacc, 0.0f) * P.invG;
      }
    }
  };
  // NVC: ||v_j||^2 of tile t's 64 tokens into nvbuf[t % 3], shared by the
  // waves (8 lanes per token, 16 dims each); read by combine(t) after the
  // barrier at tile t + 1
  auto tile_vnorms = [&](int t) {
    const char* vt = vbuf(t % 3);
    const int li = lane & 7;
    for (int tk = wave * 8 + (lane >> 3); tk < TT; tk += NW * 8) {
      const bf16x8 x0 = ld16(vt + toff(tk, 8 * li)), x1 = ld16(vt + toff(tk, 64 + 8 * li));
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const bf16x2 p0 = {x0[i], x0[i + 1]}, p1 = {x1[i], x1[i + 1]};
        a0 = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, a1, false);
      }
      float a = a0 + a1;
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      a += __shfl_xor(a, 4, 64);
      if (li == 0) nvbuf[t % 3][tk] = a;
    }
  };
  // Top of local tile t: every head issues the same loads (past the last tile
  // with zero range, into a buffer nobody reads any more), so the wait at its
  // top is the same too. Returns the global tile of local t + 2.
  auto head = [&](int t, const float (*red_prev)[TT], char* kn, char* vn) -> int {
    wait_vmcnt<kDmaPerTile>();
    const bool pooled2 = claims_next(g1);  // local t + 2 was claimed at the top of t - 1
    if (pooled2 && wave == 0 && lane == 0) {
      const uint32_t gt = (uint32_t)P.pool0 + pend;
      claim_slot[t & 1] = gt < (uint32_t)P.tiles ? (int)gt : -1;
    }
    lds_barrier();  // tile t in LDS for every wave; tile t-1's buffer is free
    int g2 = -1;
    if (pooled2) g2 = __builtin_amdgcn_readfirstlane(claim_slot[t & 1]);
    else if (g1 >= 0 && g1 + 1 < static_end) g2 = g1 + 1;
    if (gp >= 0) combine(gp, red_prev, t - 1);
    if constexpr (!NVC) {
      nv_cur = nv_next;
      nv_next = load_nv_pair(nvg, (int64_t)(g1 < 0 ? 0 : g1) * TT, trows(g1), l32);
    }
    if (claims_next(g2) && wave == 0 && lane == 0) pend = atomicAdd(ctrp, 1u);
    issue_tile<NW>(kh, (int64_t)(g2 < 0 ? 0 : g2) * TT, trows(g2), kn, wave, lane, doff);
    issue_tile<NW>(vh, (int64_t)(g2 < 0 ? 0 : g2) * TT, trows(g2), vn, wave, lane, doff);
    return g2;
  };
  auto advance = [&](int g2) {
    gp = g0;
    g0 = g1;
    g1 = g2;
  };
  auto clean = [&](auto bc, int t) {
    constexpr int B = decltype(bc)::value;
    constexpr int N2 = (B + 2) % 3;
    const int g2 = head(t, red3[N2], kbuf(N2), vbuf(N2));
    if constexpr (NVC) tile_vnorms(t);
    if (active) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        float q2s = 0.f;
        const float sw = p2_sub<false, NVC>(kbuf(B) + sub * 32 * 256, vbuf(B) + sub * 32 * 256,
                                       NVC ? 0.f : (sub ? nv_cur.y : nv_cur.x), &q2s, off, qa, aa, nb2, cinit, c2x2,
                                       0, rbase, P.w);
        if (h == 0) {
          red3[B][wave][sub * 32 + l32] = sw;
          if constexpr (NVC) red3b[B][wave][sub * 32 + l32] = q2s;
        }
      }
    }
    advance(g2);
  };
  auto is_clean = [&]() { return g0 >= 0 && g0 < ncg; };
  int t = 0;
  for (;;) {
    if (!is_clean()) break;
    clean(IntC<0>{}, t++);
    if (!is_clean()) break;
    clean(IntC<1>{}, t++);
    if (!is_clean()) break;
    clean(IntC<2>{}, t++);
  }
  for (; g0 >= 0; ++t) {  // the masked tail: tiles that reach into the window
    const int b = t % 3, nb = (t + 2) % 3;
    const int g2 = head(t, red3[nb], kbuf(nb), vbuf(nb));
    if constexpr (NVC) tile_vnorms(t);
    if (active) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int64_t tok = (int64_t)g0 * TT + sub * 32 + l32 - (P.n - P.w);
        float q2s = 0.f;
        const float sw = p2_sub<true, NVC>(kbuf(b) + sub * 32 * 256, vbuf(b) + sub * 32 * 256,
                                      NVC ? 0.f : (sub ? nv_cur.y : nv_cur.x), &q2s, off, qa, aa, nb2, cinit, c2x2,
                                      tok, rbase, P.w);
        if (h == 0) {
          red3[b][wave][sub * 32 + l32] = sw;
          if constexpr (NVC) red3b[b][wave][sub * 32 + l32] = q2s;
        }
      }
    }
    advance(g2);
  }
  wait_vmcnt<0>();  // the zero-range loads of the last heads land before the LDS goes away
  __syncthreads();
  if (gp >= 0) combine(gp, red3[(t - 1) % 3], t - 1);
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
  int stat2;      // pass 2: static tiles per workgroup of the pooled schedule (0: static chunks)
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
  // at least four tiles per chunk: shorter chunks spend most of their time
  // filling the tile pipeline, and their partials cost the merge (4K Llama
  // layer: pass 1 + merge 17.8 -> 17.1 us)
  if (p.nch1 > p.tiles / 4) p.nch1 = p.tiles / 4;
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
  // Pass 2 gives each workgroup three quarters of its even share and pools
  // the rest: the clocks of the XCDs differ by several percent under this
  // load, and with fixed chunks the slowest XCD sets the pass time. The
  // pooled schedule needs >= 3 static tiles (its first claim goes out three
  // tiles ahead) and one counter word per row group.
  const int st = (p.tiles * 3 / 4) / p.nch2;
  p.stat2 = (st >= 3 && p.nrg2 <= kSelSpareWords) ? st : 0;
  return p;
}

// The pooled schedule's fields of P2Args (counters in the select scratch's
// spare words, zeroed before pass 2 by pass 1 or the init launch).
void set_schedule(P2Args& a, const Plan& p, void* sel) {
  a.tiles = p.tiles;
  a.ctr = nullptr;
  a.ctr_stride = 0;
  a.stat_tiles = 0;
  a.pool0 = 0;
  if (p.stat2 > 0) {
    a.ctr = select_spare_words(sel, 0);
    a.ctr_stride = (int)(select_spare_words(sel, 1) - a.ctr);
    a.stat_tiles = p.stat2;
    a.pool0 = p.nch2 * p.stat2;
  }
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

hipError_t launch_fold(const FoldInfo& fold, int64_t n, int32_t Hkv, float* S, int32_t* status,
                       hipStream_t st) {
  if (!fold.flagcount) return hipSuccess;
  FoldArgs ao{fold, n, S, status};
  k_fold<<<Hkv, HD, 0, st>>>(ao);
  return hipGetLastError();
}

hipError_t launch_mfma_path(const void* q, const void* k, const void* v, const Shape& s,
                            const Workspace& ws, hipStream_t st, StageEvents* se, bool fold_in_select,
                            FoldInfo* fold) {
  const Plan p = make_plan(s);
  // carve the path's extra buffers behind the common workspace
  char* extra = (char*)ws.extra;
  auto take = [&](size_t bytes) { char* r = extra; extra += (bytes + 255) / 256 * 256; return r; };
  float* nv = (float*)take(sizeof(float) * (size_t)s.Hkv * s.n);
  float* fx = (float*)take(sizeof(float) * (size_t)FXC * s.Hkv * p.Rg * FXSTRIDE);
  int32_t* flagcount = ws.flagcount;
  float* Spart = p.nrg2 > 1 ? (float*)take(sizeof(float) * (size_t)p.nrg2 * s.Hkv * s.n) : ws.S;
  const float c2 = kLog2e / sqrtf((float)HD);

  P1Args a1{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.n, s.w, p.Rg, p.nw,
            p.tpc1, s.Hkv, c2, ws.part, nv, ws.status, flagcount, (uint32_t*)ws.sel,
            (int64_t)select_zero_words(s.Hkv)};
  hipError_t e;
  {
    const dim3 grid1(p.nch1, p.nrg, s.Hkv);
    switch (p.nw) {
      case 8: e = stage_launch(se, "pass1", kStageOnly, k_pass1<8>, grid1, dim3(512), st, a1); break;
      case 4: e = stage_launch(se, "pass1", kStageOnly, k_pass1<4>, grid1, dim3(256), st, a1); break;
      case 2: e = stage_launch(se, "pass1", kStageOnly, k_pass1<2>, grid1, dim3(128), st, a1); break;
      default: e = stage_launch(se, "pass1", kStageOnly, k_pass1<1>, grid1, dim3(64), st, a1); break;
    }
    if (e != hipSuccess) return e;
  }
  MergeArgs am{(const uint16_t*)q, (const uint16_t*)k, ws.part, s.n, s.n, s.w, p.Rg, s.Hkv, p.nch1,
               c2, 1.0f / sqrtf((float)HD), ws.rs, flagcount, ws.status};
  const int64_t rows = (int64_t)s.Hkv * p.Rg;
  e = stage_launch(se, "merge", kStageOnly, k_merge, dim3((unsigned)((rows + 3) / 4)), dim3(256), st, am);
  if (e != hipSuccess) return e;
  FixArgs af{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.n, s.w, p.Rg, s.Hkv, c2,
             ws.rs, flagcount, fx};
  if (p.nw2 < 2) {  // wider workgroups run the fix-up inside pass 2
    e = stage_launch(se, "fixup", kStageOnly, k_fixup, dim3(FXC, s.Hkv), dim3(256), st, af);
    if (e != hipSuccess) return e;
  }
  P2Args a2{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.w, p.Rg, p.nw2,
            p.tpc2, s.Hkv, c2, 1.0f / (float)s.G(), ws.rs, nv, flagcount, Spart, ws.status};
  set_schedule(a2, p, ws.sel);
  const dim3 grid2(p.nch2, p.nrg2, s.Hkv);
  switch (p.nw2) {
    case 8: e = stage_launch(se, "pass2", kStageOnly, k_pass2<8, false>, grid2, dim3(512), st, a2, af); break;
    case 4: e = stage_launch(se, "pass2", kStageOnly, k_pass2<4, false>, grid2, dim3(256), st, a2, af); break;
    case 2: e = stage_launch(se, "pass2", kStageOnly, k_pass2<2, false>, grid2, dim3(128), st, a2, af); break;
    default: e = stage_launch(se, "pass2", kStageOnly, k_pass2<1, false>, grid2, dim3(64), st, a2, af); break;
  }
  if (e != hipSuccess) return e;
  if (p.nrg2 > 1) {
    const int64_t total = (int64_t)s.Hkv * s.n;
    e = stage_launch(se, "rowgroup_sum", kStageOnly, k_sum_rowgroups, dim3((unsigned)((total + 255) / 256)),
                     dim3(256), st, (const float*)Spart, ws.S, total, p.nrg2);
    if (e != hipSuccess) return e;
  }
  FoldInfo fi{flagcount, ws.rs, fx, s.Hkv, p.Rg, FXC, FXSTRIDE, HD, 1.0f / (float)s.G()};
  if (fold_in_select) {
    *fold = fi;
  } else if (fi.flagcount) {
    FoldArgs ao{fi, s.n, ws.S, ws.status};
    e = stage_launch(se, "fold", kStageOnly, k_fold, dim3(s.Hkv), dim3(HD), st, ao);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_mfma_rowstats(const void* q, const void* k, const void* v, const Shape& s, int64_t ld,
                                const Workspace& ws, hipStream_t st, FoldInfo* fold) {
  const Plan p = make_plan(s);
  char* extra = (char*)ws.extra;
  auto take = [&](size_t bytes) { char* r = extra; extra += (bytes + 255) / 256 * 256; return r; };
  float* nv = (float*)take(sizeof(float) * (size_t)s.Hkv * s.n);
  float* fx = (float*)take(sizeof(float) * (size_t)FXC * s.Hkv * p.Rg * FXSTRIDE);
  const float c2 = kLog2e / sqrtf((float)HD);
  P1Args a1{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, ld, s.w, p.Rg, p.nw,
            p.tpc1, s.Hkv, c2, ws.part, nv, ws.status, ws.flagcount, (uint32_t*)ws.sel,
            (int64_t)select_zero_words(s.Hkv)};
  const dim3 grid1(p.nch1, p.nrg, s.Hkv);
  switch (p.nw) {
    case 8: k_pass1<8><<<grid1, 512, 0, st>>>(a1); break;
    case 4: k_pass1<4><<<grid1, 256, 0, st>>>(a1); break;
    case 2: k_pass1<2><<<grid1, 128, 0, st>>>(a1); break;
    default: k_pass1<1><<<grid1, 64, 0, st>>>(a1); break;
  }
  MergeArgs am{(const uint16_t*)q, (const uint16_t*)k, ws.part, s.n, ld, s.w, p.Rg, s.Hkv, p.nch1,
               c2, 1.0f / sqrtf((float)HD), ws.rs, ws.flagcount, ws.status};
  const int64_t rows = (int64_t)s.Hkv * p.Rg;
  k_merge<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(am);
  FixArgs af{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, ld, s.w, p.Rg, s.Hkv, c2,
             ws.rs, ws.flagcount, fx};
  k_fixup<<<dim3(FXC, s.Hkv), 256, 0, st>>>(af);
  *fold = FoldInfo{ws.flagcount, ws.rs, fx, s.Hkv, p.Rg, FXC, FXSTRIDE, HD, 1.0f / (float)s.G()};
  return hipGetLastError();
}

hipError_t launch_mfma_from_stats(const void* q, const void* k, const void* v, const Shape& s,
                                  const Workspace& ws, hipStream_t st, const float* m,
                                  const float* rest, const int32_t* argmax, const float* a,
                                  FoldInfo* fold) {
  const Plan p = make_plan(s);
  char* extra = (char*)ws.extra;  // the same carve as launch_mfma_path (nv stays unused)
  auto take = [&](size_t bytes) { char* r = extra; extra += (bytes + 255) / 256 * 256; return r; };
  (void)take(sizeof(float) * (size_t)s.Hkv * s.n);
  float* fx = (float*)take(sizeof(float) * (size_t)FXC * s.Hkv * p.Rg * FXSTRIDE);
  int32_t* flagcount = ws.flagcount;
  float* Spart = p.nrg2 > 1 ? (float*)take(sizeof(float) * (size_t)p.nrg2 * s.Hkv * s.n) : ws.S;
  const float c2 = kLog2e / sqrtf((float)HD);
  hipError_t e = launch_init(ws.status, flagcount, ws.sel, s.Hkv, st);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)s.Hkv * p.Rg;
  ImportArgs ai{m, rest, argmax, a, s.n, rows, p.Rg, ws.rs, flagcount, ws.status};
  k_import<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(ai);
  FixArgs af{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.n, s.w, p.Rg, s.Hkv, c2,
             ws.rs, flagcount, fx};
  if (p.nw2 < 2) k_fixup<<<dim3(FXC, s.Hkv), 256, 0, st>>>(af);
  P2Args a2{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s.n, s.w, p.Rg, p.nw2,
            p.tpc2, s.Hkv, c2, 1.0f / (float)s.G(), ws.rs, nullptr, flagcount, Spart, ws.status};
  set_schedule(a2, p, ws.sel);
  const dim3 grid2(p.nch2, p.nrg2, s.Hkv);
  switch (p.nw2) {
    case 8: k_pass2<8, true><<<grid2, 512, 0, st>>>(a2, af); break;
    case 4: k_pass2<4, true><<<grid2, 256, 0, st>>>(a2, af); break;
    case 2: k_pass2<2, true><<<grid2, 128, 0, st>>>(a2, af); break;
    default: k_pass2<1, true><<<grid2, 64, 0, st>>>(a2, af); break;
  }
  if (p.nrg2 > 1) {
    const int64_t total = (int64_t)s.Hkv * s.n;
    k_sum_rowgroups<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(Spart, ws.S, total, p.nrg2);
  }
  *fold = FoldInfo{flagcount, ws.rs, fx, s.Hkv, p.Rg, FXC, FXSTRIDE, HD, 1.0f / (float)s.G()};
  return hipGetLastError();
}


// ---------------------------------------------------------------------------- prefill attention
//
// Causal prefill attention of every position (the pass a prefill runs
// anyway), which also hands over the window rows' statistics that scoring
// from given statistics consumes (largest logit, rest mass, argmax, output),
// so that scoring reads K and V once more instead of twice. DropKV write-up,
// section 核心公式: p = softmax(K q / sqrt d), a = sum_j p_j v_j, each row
// seeing keys 0..its position; the atlas summary (Experimental setup) names
// FlashAttention-2 as the basis of the paper's scorer.
//
// One workgroup per (block of PB consecutive positions, KV head): its rows
// are the G query heads of that KV head at those positions (row r: head
// g G + r / PB, position p0 + r % PB), so each K/V tile read serves all G
// heads. The workgroup streams K/V tiles 0 .. (p0 + PB - 1) / 64 through LDS
// exactly as pass 1 does (the same tile routine: QK^T and PV on MFMA, online
// softmax with a lazy reference), masks the diagonal tiles, and writes O in
// bf16. Blocks are taken heaviest (last) first.

namespace {

struct PrefillArgs {
  const uint16_t* q;  // [Hq][n][d]
  const uint16_t* k;  // [Hkv][n][d]
  const uint16_t* v;
  int64_t n;
  int w, G, PB, Rg, nblk, Hkv;
  float c2, inv_sqrt_d;
  uint16_t* o;         // [Hq][n][d] bf16
  float* m;            // window row r = h * w + i: largest logit (natural units)
  float* L;            // 1 + R relative to the largest logit
  int32_t* best;       // 32-token block where the largest logit first occurs
  float* a;            // [Hq * w][d] output in fp32
  int32_t* status;
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_prefill(PrefillArgs A) {
  __shared__ __attribute__((aligned(1024))) char kbuf[3][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf[3][TILE_BYTES];
  constexpr int kDmaPerTile = 32 / NW;
  const int blk = A.nblk - 1 - (int)blockIdx.x;  // heaviest first
  const int g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t p0 = (int64_t)blk * A.PB;
  const int row = wave * 32 + l32;
  const int t = row / A.PB;
  const int64_t pos = p0 + row % A.PB;
  const bool row_ok = row < A.Rg && pos < A.n;
  const bool active = wave * 32 < A.Rg;
  int64_t nkeys = p0 + A.PB;  // keys 0 .. nkeys - 1 are visible to some row
  if (nkeys > A.n) nkeys = A.n;
  const int ntiles = (int)((nkeys + TT - 1) / TT);
  const int nfull = (int)(nkeys / TT);  // tiles 0 .. nfull - 1 hold 64 keys each
  const int nclean = (int)((p0 + 1) / TT) < ntiles ? (int)((p0 + 1) / TT) : ntiles;  // tiles every row sees whole
  const uint16_t* kh = A.k + (size_t)g * A.n * HD;
  const uint16_t* vh = A.v + (size_t)g * A.n * HD;
  const int qh = g * A.G + (row_ok ? t : 0);
  const float c2 = A.c2;
  const LdsOff off = with_v_base(lds_offsets(lane), vbuf[0]);
  const DmaOff<NW> doff = dma_offsets<NW>(wave, lane);

  bf16x8 qb[8];
  {
    const uint16_t* qr = A.q + ((size_t)qh * A.n + (row_ok ? pos : 0)) * HD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 tq = *(const bf16x8*)(qr + ks * 16 + h * 8);
      if (!row_ok) tq = bf16x8{};
      qb[ks] = tq;
    }
  }
  P1State st{-INFINITY, -INFINITY, 0.f, -1, 0.f};
  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};

  if (ntiles > 0) {
    issue_tile<NW>(kh, 0, tile_rows(0, nfull, 0, nkeys), kbuf[0], wave, lane, doff);
    issue_tile<NW>(vh, 0, tile_rows(0, nfull, 0, nkeys), vbuf[0], wave, lane, doff);
  }
  if (ntiles > 1) {
    issue_tile<NW>(kh, TT, tile_rows(1, nfull, 0, nkeys), kbuf[1], wave, lane, doff);
    issue_tile<NW>(vh, TT, tile_rows(1, nfull, 0, nkeys), vbuf[1], wave, lane, doff);
  }
  // per tile and wave the only vector-memory ops are the tile loads, so
  // `vmcnt <= one tile's loads` at the top of tile t + 1 means it has landed
  auto head = [&](int tt, char* kn, char* vn) {
    const int64_t tb = (int64_t)tt * TT;
    if (tt + 1 < ntiles) wait_vmcnt<kDmaPerTile>(); else wait_vmcnt<0>();
    lds_barrier();
    if (tt + 2 < ntiles) {
      issue_tile<NW>(kh, tb + 2 * TT, tile_rows(tt + 2, nfull, 0, nkeys), kn, wave, lane, doff);
      issue_tile<NW>(vh, tb + 2 * TT, tile_rows(tt + 2, nfull, 0, nkeys), vn, wave, lane, doff);
    }
  };
  auto clean = [&](auto bc, int tt) {
    constexpr int B = decltype(bc)::value;
    constexpr int N2 = (B + 2) % 3;
    head(tt, kbuf[N2], vbuf[N2]);
    if (active) p1_tile<false>(c2, kbuf[B], vbuf[0], B * TILE_BYTES, (int64_t)tt * TT, off, lane, pos, qb, st, O);
  };
  int tt = 0;
  for (; tt + 3 <= nclean; tt += 3) {
    clean(IntC<0>{}, tt);
    clean(IntC<1>{}, tt + 1);
    clean(IntC<2>{}, tt + 2);
  }
  for (; tt < ntiles; ++tt) {  // at most two clean tiles, then the diagonal ones
    const int b = tt % 3, nb = (tt + 2) % 3;
    head(tt, kbuf[nb], vbuf[nb]);
    if (active) p1_tile<true>(c2, kbuf[b], vbuf[0], b * TILE_BYTES, (int64_t)tt * TT, off, lane, pos, qb, st, O);
  }
  if (!active) return;
  const float l_tot = pair_sum(st.l);
  p1_row_max(st);
  if (!row_ok) return;
  const float inv_l = 1.0f / l_tot;
  // lane holds O^T rows d = 32 db + 8 i + 4 h + (0..3) of its row's column
  DKV_CHECK(pos < A.n && qh < A.Hkv * A.G, A.status);
  uint16_t* orow = A.o + ((size_t)qh * A.n + pos) * HD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * h;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16_rne(O[db][4 * i] * inv_l) | ((uint32_t)f32_to_bf16_rne(O[db][4 * i + 1] * inv_l) << 16);
      pk.y = (uint32_t)f32_to_bf16_rne(O[db][4 * i + 2] * inv_l) |
             ((uint32_t)f32_to_bf16_rne(O[db][4 * i + 3] * inv_l) << 16);
      *(uint2*)(orow + d0) = pk;
    }
  if (pos >= A.n - A.w) {
    const int64_t wr = (int64_t)qh * A.w + (pos - (A.n - A.w));
    DKV_CHECK(wr >= 0 && wr < (int64_t)A.Hkv * A.G * A.w, A.status);
    float* ar = A.a + wr * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 ov = {O[db][4 * i] * inv_l, O[db][4 * i + 1] * inv_l, O[db][4 * i + 2] * inv_l,
                     O[db][4 * i + 3] * inv_l};
        *(float4*)(ar + 32 * db + 8 * i + 4 * h) = ov;
      }
    if (h == 0) {
      A.m[wr] = st.m_true * A.inv_sqrt_d;
      // l is relative to the reference exponent mref; L = l 2^(mref - x_max c)
      A.L[wr] = l_tot * __builtin_amdgcn_exp2f(st.mref - st.m_true * c2);
      A.best[wr] = st.best;
    }
  }
}

__global__ void k_zero_word(int32_t* p) {
  if (threadIdx.x == 0) *p = 0;
}

struct PrefillArgmaxArgs {
  const uint16_t* q;  // [Hq][n][d]
  const uint16_t* k;
  int64_t n;
  int w, G, Hq;
  const float* L;
  const int32_t* best;
  float* rest;        // out: R = L - 1
  int32_t* argmax;    // out: lowest index attaining the largest logit (search in its 32-token block)
  int32_t* status;
};

// One wave per window row: R from L, and the argmax inside the 32-token
// block where the running maximum was set (logits recomputed in fp32 from the
// bf16 inputs, lowest index on ties, as the merge of the scoring path does).
__global__ __launch_bounds__(256) void k_prefill_argmax(PrefillArgmaxArgs P) {
  const int lane = threadIdx.x & 63;
  const int64_t wr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wr >= (int64_t)P.Hq * P.w) return;
  const int qh = (int)(wr / P.w);
  const int64_t pos = P.n - P.w + wr % P.w;
  const int g = qh / P.G;
  const int bt = P.best[wr];
  const int64_t tok = (int64_t)bt * 32 + (lane & 31);
  float x = -INFINITY;
  if (lane < 32 && bt >= 0 && tok <= pos) {
    const uint16_t* qr = P.q + ((size_t)qh * P.n + pos) * HD;
    const uint16_t* kr = P.k + ((size_t)g * P.n + tok) * HD;
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
  if (lane == 0) {
    const float L = P.L[wr];
    P.rest[wr] = L - 1.0f;
    P.argmax[wr] = (jt == 0x7fffffff) ? -1 : jt;
    if (!finite_f(L) || jt == 0x7fffffff) atomicOr(P.status, kStatusNonFinite);
  }
}

}  // namespace

// Prefill attention (bf16, d = 128): O for every position, and the window
// rows' statistics m, R (rest), argmax and a. ws_L / ws_best (Hq * w each)
// hold 1 + R and the 32-token block of the maximum between the two kernels;
// they may be rest / argmax themselves (the second kernel converts each row
// in place).
hipError_t launch_prefill(const void* q_all, const void* k, const void* v, int64_t n, int32_t w, int32_t Hq,
                          int32_t Hkv, void* o, float* m, float* rest, int32_t* argmax, float* a, float* ws_L,
                          int32_t* ws_best, int32_t* status, hipStream_t st) {
  const int G = Hq / Hkv;
  int PB = (256 / G) / 32 * 32;  // positions per workgroup: G PB rows, at most 256
  if (PB < 8) PB = 256 / G;
  const int Rg = G * PB;
  const int nblk = (int)((n + PB - 1) / PB);
  int nw = MAXW;
  while (nw > 1 && (nw / 2) * 32 >= Rg) nw /= 2;
  PrefillArgs pa{(const uint16_t*)q_all, (const uint16_t*)k, (const uint16_t*)v, n, w, G, PB, Rg, nblk, Hkv,
                 kLog2e / sqrtf((float)HD), 1.0f / sqrtf((float)HD), (uint16_t*)o, m, ws_L, ws_best, a, status};
  k_zero_word<<<1, 64, 0, st>>>(status);  // the status word starts clear (a kernel, so the call can be captured)
  const dim3 grid(nblk, Hkv);
  switch (nw) {
    case 8: k_prefill<8><<<grid, 512, 0, st>>>(pa); break;
    case 4: k_prefill<4><<<grid, 256, 0, st>>>(pa); break;
    case 2: k_prefill<2><<<grid, 128, 0, st>>>(pa); break;
    default: k_prefill<1><<<grid, 64, 0, st>>>(pa); break;
  }
  PrefillArgmaxArgs pm{(const uint16_t*)q_all, (const uint16_t*)k, n, w, G, Hq, ws_L, ws_best, rest, argmax, status};
  const int64_t rows = (int64_t)Hq * w;
  k_prefill_argmax<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(pm);
  return hipGetLastError();
}

}  // namespace dropkv
