// Internal declarations shared by the HIP sources of libdropkv (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

namespace dropkv {

// Bits of the device status word (same values as DROPKV_STATUS_* in dropkv.h).
constexpr int kStatusSingular = 1;
constexpr int kStatusNonFinite = 2;
constexpr int kStatusBadIndex = 4;  // cache compaction: eviction list not increasing inside [0, n)
constexpr int kStatusNegative = 16;  // select on given scores: some S[g][j] < 0
constexpr int kStatusBounds = 32;    // checking build only: an index failed its bounds check

// Bounds checks of the checking build (-DDROPKV_DEBUG): a failed check ORs
// kStatusBounds into the call's status word (the access itself is left as it
// is; the release build compiles the checks away).
#ifdef DROPKV_DEBUG
#define DKV_CHECK(cond, status)                                 \
  do {                                                          \
    if (!(cond)) atomicOr((status), ::dropkv::kStatusBounds);   \
  } while (0)
#else
#define DKV_CHECK(cond, status) \
  do {                          \
  } while (0)
#endif

// A window row is rejected when its rest mass R = sum_{j != argmax} exp(x_j - x_max)
// is at most 2^-24: then 1/(1+R) rounds to 1 in binary32 (the singular-input rule).
constexpr float kSingularRest = 5.9604644775390625e-08f;  // 2^-24

constexpr float kLog2e = 1.4426950408889634f;

// Buffer descriptor of `bytes` bytes at p (a raw buffer: stride 0, 32-bit
// data format). Loads past `bytes` (the scalar offset included) return
// zeros, and a direct-to-LDS load writes those zeros: a tile read through a
// descriptor that covers only its valid rows needs no clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// Per-window-row statistics, row index r = h * window + i (query head h, window row i).
struct RowStats {
  float* m;         // largest logit x_max = max_j q.k_j / sqrt(d)  (natural units)
  float* rest;      // R = sum_{j != argmax} exp(x_j - x_max)
  float* L;         // 1 + R (softmax denominator relative to the max)
  int32_t* jstar;   // argmax (lowest index), or -1 if not tracked
  float* fixval;    // ||Delta_{argmax}||^2 computed without cancellation (valid where used)
  int32_t* flag;    // 1: the argmax term of this row comes from fixval, not the main pass
  float* a;         // [rows][d] attention output a = sum_j p_j v_j (fp32)
  uint16_t* a_bf;   // [rows][d] a rounded to bf16 (MFMA path)
  float* na;        // ||a||^2 from the bf16-rounded a (MFMA path)
  float* bias;      // per-row exponent offset for the score pass (MFMA path, log2 units)
};

// Device workspace, carved from one caller- or library-owned allocation.
struct Workspace {
  int32_t* status;  // OR of kStatus* bits
  float* S;         // [Hkv][n] GQA-mean raw scores
  RowStats rs;
  uint32_t* part;   // pass-1 partials (MFMA path): A in bf16, then m, l, best, mref
  void* extra;      // further MFMA-path buffers (see mfma_extra_bytes)
  void* sel;        // select-stage scratch (see select_scratch_bytes)
  int32_t* flagcount;  // [Hkv] rows per KV head whose argmax term comes from the fix-up
  int nchunks;      // pass-1 split count (MFMA path)
  size_t bytes;     // total bytes used
};

struct Shape {
  int64_t n;
  int32_t w, Hq, Hkv, d;
  int32_t G() const { return Hq / Hkv; }
  int64_t rows() const { return (int64_t)Hq * w; }
};

// Workspace layout for a shape (ws_base may be null to only size it).
Workspace carve_workspace(void* ws_base, const Shape& s, bool mfma);

// Launchers. Each returns hipSuccess or the launch error.
// Cache compaction (compact.hip): ORs kStatusBadIndex into *status for an
// invalid list, and copies the rows of k, v
// [Hkv][n][d] not listed in evict_idx [Hkv][n_evict] to out_k, out_v
// [Hkv][n - n_evict][d]; dtype 0 = bf16, 1 = fp32.
hipError_t launch_compact(int dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                          const int64_t* evict_idx, int64_t n_evict, void* out_k, void* out_v,
                          int32_t* status, hipStream_t st);
// The same from the kept list keep_idx [Hkv][n_keep] (ascending per head):
// output row r of head g is row keep_idx[g][r]; kStatusBadIndex for a list
// that is not strictly increasing inside [0, n).
hipError_t launch_compact_kept(int dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                               const int64_t* keep_idx, int64_t n_keep, void* out_k, void* out_v,
                               int32_t* status, hipStream_t st);
// Zeroes the status word, flagcount[Hkv] (may be null) and the select scratch.
hipError_t launch_init(int32_t* status, int32_t* flagcount, void* sel_scratch, int32_t Hkv,
                       hipStream_t st);
hipError_t launch_generic_rows(int dtype, const void* q, const void* k, const void* v,
                               const Shape& s, const Workspace& ws, hipStream_t st);
hipError_t launch_generic_scores(int dtype, const void* q, const void* k, const void* v,
                                 const Shape& s, const Workspace& ws, hipStream_t st);
// Exact argmax terms of the rows flagged by the MFMA path's merge (rows with
// p_max > 1/2): per-chunk fix-up partials (sp, ps, D[d]) that the select
// stage folds into S in row order. flagcount == nullptr: nothing to fold.
struct FoldInfo {
  const int32_t* flagcount;  // [Hkv]
  RowStats rs;
  const float* fx;           // [nchunk][Hkv * Rg][stride]
  int Hkv, Rg, nchunk, stride, d;
  float invG;
};

// reject_negative: S comes from the caller (dropkv_select), and any S < 0
// raises kStatusNegative; scores the library computed are >= 0 by
// construction, up to fp64 rounding residue in decode-time rescoring, which
// orders as +0.
struct StageEvents;
hipError_t launch_select(const float* S, int64_t n, int32_t w, int32_t Hkv, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_idx, int32_t* status,
                         const FoldInfo* fold, void* scratch, hipStream_t st, bool reject_negative = false,
                         StageEvents* se = nullptr, int64_t* keep_idx = nullptr);
size_t select_scratch_bytes(int64_t n, int32_t Hkv);
// 32-bit words at the start of the select scratch that must be zero before a call.
size_t select_zero_words(int32_t Hkv);
// Spare words of that zeroed block, free for other kernels of the call:
// select_spare_words(scratch, g)[i] for KV head g and i < kSelSpareWords.
constexpr int kSelSpareWords = 15;
uint32_t* select_spare_words(void* sel_scratch, int32_t g);
// Stage timing. Stage i runs from ev[i][0] to ev[i][1]. Kernels launched
// through stage_launch take these from their own dispatch (the begin time of
// a stage's first kernel, the end time of its last), so timing adds no packet
// between kernels; record_stage instead records marker events on the stream
// (a stage then runs from the previous marker to its own).
constexpr int kMaxStages = 12;
struct StageEvents {
  hipEvent_t ev[kMaxStages][2];
  const char* names[kMaxStages];
  int count;
};
hipError_t record_stage(StageEvents* se, const char* name, hipStream_t st);
// Roles of a kernel in its stage (bit 0: first kernel, bit 1: last kernel).
enum { kStageMid = 0, kStageFirst = 1, kStageLast = 2, kStageOnly = 3 };
// Launches `kern` on `st`; with se non-null the kernel's begin (kStageFirst) and
// end (kStageLast) times become stage `name`'s events.
template <typename F, typename... Args>
hipError_t stage_launch(StageEvents* se, const char* name, int role, F kern, dim3 grid, dim3 block,
                        hipStream_t st, Args... args) {
  if (!se || se->count >= kMaxStages) {
    hipLaunchKernelGGL(kern, grid, block, 0, st, args...);
    return hipGetLastError();
  }
  hipEvent_t e0 = (role & kStageFirst) ? se->ev[se->count][0] : nullptr;
  hipEvent_t e1 = (role & kStageLast) ? se->ev[se->count][1] : nullptr;
  hipExtLaunchKernelGGL(kern, grid, block, 0, st, e0, e1, 0u, args...);
  if (role & kStageLast) se->names[se->count++] = name;
  return hipGetLastError();
}
// MFMA path up to raw scores. Pass 1 also clears the status word, the flag
// counts and select_zero_words(Hkv) words of ws.sel (no separate init launch).
// fold_in_select: leave the flagged rows' argmax terms out of ws.S and return
// their description in *fold for launch_select to add (else *fold is unused
// and k_fold adds them to ws.S).
hipError_t launch_mfma_path(const void* q, const void* k, const void* v, const Shape& s,
                            const Workspace& ws, hipStream_t st, StageEvents* se, bool fold_in_select,
                            FoldInfo* fold);
// Adds the argmax terms described by `fold` into S [Hkv][n] (one block per head).
// MFMA path from caller-given row statistics (m, R, argmax, a per window row,
// row r = h * window + i): no pass 1; clears the status word, flag counts and
// select histograms itself; *fold as with fold_in_select.
hipError_t launch_mfma_from_stats(const void* q, const void* k, const void* v, const Shape& s,
                                  const Workspace& ws, hipStream_t st, const float* m,
                                  const float* rest, const int32_t* argmax, const float* a,
                                  FoldInfo* fold);
// MFMA pass 1, merge and the argmax fix-up partials only: the row statistics
// of the window rows in ws.rs (rest exact except for flagged rows, whose exact
// value and argmax term come from *fold). k and v hold ld >= n token rows per
// KV head. Clears the status word and flag counts like launch_mfma_path.
hipError_t launch_mfma_rowstats(const void* q, const void* k, const void* v, const Shape& s, int64_t ld,
                                const Workspace& ws, hipStream_t st, FoldInfo* fold);
hipError_t launch_fold(const FoldInfo& fold, int64_t n, int32_t Hkv, float* S, int32_t* status,
                       hipStream_t st);
// Prefill attention (bf16, d = 128; mfma_path.hip): O [Hq][n][d] for every
// position and, for the last w positions (row r = h * w + i), the largest
// logit m (natural units), the rest mass R, the argmax and the output a in
// fp32. ws_L, ws_best: scratch of Hq * w floats / ints. Clears *status first.
hipError_t launch_prefill(const void* q_all, const void* k, const void* v, int64_t n, int32_t w, int32_t Hq,
                          int32_t Hkv, void* o, float* m, float* rest, int32_t* argmax, float* a, float* ws_L,
                          int32_t* ws_best, int32_t* status, hipStream_t st);
bool mfma_supported(int dtype, int d);
int mfma_chunks(const Shape& s);
size_t mfma_extra_bytes(const Shape& s);

// ------------------------------------------------------------------ device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, size_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
};

__device__ __forceinline__ bool finite_f(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }

// Deterministic block reductions (fixed combination order). `red` must hold
// blockDim.x entries; every thread of the block must call them.
template <int NT>
__device__ __forceinline__ float block_sum(float x, float* red) {
  const int t = threadIdx.x;
  red[t] = x;
  __syncthreads();
#pragma unroll
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (t < o) red[t] = red[t] + red[t + o];
    __syncthreads();
  }
  float r = red[0];
  __syncthreads();
  return r;
}


// Argmax term ||Delta_{j*}||^2 of flagged row `row` from its fix-up partials
// (sp = sum_{i != j*} p_i, ps = p_{j*}, D = sum_{i != j*} p_i (v_i - v_{j*})),
// reduced over the NT threads of the calling block (threads t < F.d add D_t).
// Every thread returns the same value, R in *R_out and the status bits to
// raise in *bits (non-finite or singular row: the value must not be used).
template <int NT>
__device__ __forceinline__ float fold_value(const FoldInfo& F, int64_t row, float* red, float* R_out,
                                            int* bits) {
  const int tid = threadIdx.x;
  float sp = 0.f, ps = 0.f, D = 0.f;
  for (int c = 0; c < F.nchunk; ++c) {
    const float* o = F.fx + ((size_t)c * F.Hkv * F.Rg + row) * F.stride;
    sp += o[0];
    ps += o[1];
    if (tid < F.d) D += o[2 + tid];
  }
  const float dn2 = block_sum<NT>(D * D, red);
  // R = sum_{i != j*} e_i / e_{j*}; ||a - v_{j*}|| = ||D|| / (ps + sp); p/(1-p) = 1/R
  const float R = sp / ps;
  const float tot = ps + sp;
  *R_out = R;
  *bits = (!(ps > 0.f) || !finite_f(R)) ? kStatusNonFinite : (R <= kSingularRest ? kStatusSingular : 0);
  return dn2 / (tot * tot) / (R * R);
}

}  // namespace dropkv
