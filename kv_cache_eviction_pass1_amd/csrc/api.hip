// C-ABI entry points of libdropkv: validation, workspace, dispatch, status.
#include "../../include/dropkv.h"
#include "dropkv_common.h"
#include "decode_state.h"

#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

namespace dropkv {

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(DROPKV_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Library-owned grow-only workspace per device (plain entry points only).
struct DeviceWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::unordered_map<int, DeviceWs> g_ws;

// Scratch of dropkv_score_noalloc: one static device array, which every GPU
// the library runs on holds (at its own address) until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory: kernels
// and copies get the device address from hipGetSymbolAddress, looked up once
// per device (with that device current) and kept in g_scratch_dev.
constexpr size_t kNoAllocScratchBytes = (size_t)DROPKV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array (no allocation).
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DROPKV_ERR_DEVICE, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || ((uintptr_t)ptr & 255)) return fail(DROPKV_ERR_DEVICE, "scratch array address not 256-byte aligned");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return DROPKV_OK;
}

// Stage log: event sets of up to kLogCalls logged dropkv_score_ex calls per device.
constexpr int kLogCalls = 256;
struct StageLog {
  StageEvents slot[kLogCalls];
  bool created[kLogCalls] = {};
  int used = 0;
};
std::mutex g_log_mutex;
std::unordered_map<int, StageLog> g_log;

// Next free slot of the current device's log (events created on first use), or null.
StageEvents* log_slot() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_log_mutex);
  StageLog& L = g_log[dev];
  if (L.used >= kLogCalls) return nullptr;
  const int i = L.used;
  if (!L.created[i]) {
    // timing-only events: no system-scope fence (and its cache writeback) per record
    for (int e = 0; e < kMaxStages; ++e)
      for (int b = 0; b < 2; ++b)
        if (hipEventCreateWithFlags(&L.slot[i].ev[e][b], hipEventDisableSystemFence) != hipSuccess) return nullptr;
    L.created[i] = true;
  }
  L.slot[i].count = 0;
  L.used += 1;
  return &L.slot[i];
}

const char* validate(int dtype, int64_t n, int32_t w, int32_t Hq, int32_t Hkv, int32_t d) {
  if (dtype != DROPKV_BF16 && dtype != DROPKV_F32) return "dtype must be DROPKV_BF16 or DROPKV_F32";
  if (n < 2) return "n must be >= 2";
  if (w < 1 || (int64_t)w >= n) return "need 1 <= window < n";
  if (Hq < 1 || Hkv < 1) return "need Hq >= 1 and Hkv >= 1";
  if (Hq % Hkv != 0) return "Hq must be a multiple of Hkv";
  if (d < 1 || d > 256) return "need 1 <= d <= 256";
  if (n > ((int64_t)1 << 31) - 1) return "n must fit in int32 token indices";
  // element counts must fit comfortably in 64-bit byte offsets
  const double kv_elems = (double)Hkv * (double)n * (double)d;
  if (kv_elems > 1e15) return "K/V too large";
  if ((double)Hq * w > 1e8) return "too many window rows";
  return nullptr;
}

const char* validate_select(int64_t n, int32_t w, int32_t Hkv, int32_t pool_kernel, int64_t n_evict) {
  if (pool_kernel < 1 || pool_kernel % 2 == 0) return "pool_kernel must be odd and >= 1";
  if (n_evict < 0 || n_evict > n - w) return "need 0 <= n_evict <= n - window";
  (void)Hkv;
  return nullptr;
}

bool is_device_ptr(const void* p) {
  if (!p) return false;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

bool use_mfma(int dtype, int d, uint32_t flags) {
  return !(flags & DROPKV_FLAG_GENERIC) && mfma_supported(dtype, d);
}

// Run the scoring stages up to raw scores (ws.S) and row statistics.
// fold: when non-null (scoring calls), the MFMA path leaves the argmax terms
// of flagged rows for the select stage and describes them here; it stays
// zero-initialised (nothing to fold) on the generic path.
int run_scores(int dtype, const void* q, const void* k, const void* v, const Shape& s,
               const Workspace& ws, bool mfma, hipStream_t st, StageEvents* se = nullptr,
               FoldInfo* fold = nullptr) {
  hipError_t e;
  if (fold) *fold = FoldInfo{};
  if (mfma) {
    // pass 1 clears the status word, the flag counts and the select state
    e = launch_mfma_path(q, k, v, s, ws, st, se, fold != nullptr, fold);
    if (e != hipSuccess) return fail_hip(e, "mfma path");
  } else {
    e = launch_init(ws.status, ws.flagcount, ws.sel, s.Hkv, st);
    if (e != hipSuccess) return fail_hip(e, "init");
    (void)record_stage(se, "start", st);
    e = launch_generic_rows(dtype, q, k, v, s, ws, st);
    if (e != hipSuccess) return fail_hip(e, "generic row stats");
    (void)record_stage(se, "rows", st);
    e = launch_generic_scores(dtype, q, k, v, s, ws, st);
    if (e != hipSuccess) return fail_hip(e, "generic scores");
    (void)record_stage(se, "scores", st);
  }
  return DROPKV_OK;
}

// A singular row leaves its own scores undefined (often inf/NaN), which the
// select stage then also reports as non-finite: the singular bit wins.
int status_to_code(int32_t st_word) {
  if (st_word & kStatusSingular)
    return fail(DROPKV_ERR_SINGULAR, "a window row has a probability that rounds to 1 (singular)");
  if (st_word & kStatusNonFinite) return fail(DROPKV_ERR_NONFINITE, "non-finite inputs or scores");
  if (st_word & kStatusNegative) return fail(DROPKV_ERR_NEGATIVE, "negative raw score given to select");
  if (st_word & kStatusBounds) return fail(DROPKV_ERR_DEVICE, "a device-side bounds check failed (checking build)");
  return DROPKV_OK;
}

// Library-owned workspace for the current device; caller holds g_ws_mutex.
int get_workspace(size_t need, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  DeviceWs& w = g_ws[dev];
  if (w.bytes < need) {
    if (w.ptr) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    e = hipMalloc(&w.ptr, need);
    if (e != hipSuccess) return fail_hip(e, "hipMalloc workspace");
    w.bytes = need;
  }
  *out = w.ptr;
  return DROPKV_OK;
}

int sync_status(const Workspace& ws, hipStream_t st) {
  int32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, ws.status, sizeof(word), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return fail_hip(e, "status readback");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
  return status_to_code(word);
}

int check_inputs(const void* q, const void* k, const void* v) {
  if (!q || !k || !v) return fail(DROPKV_ERR_INVALID, "null input pointer");
  if (!is_device_ptr(q) || !is_device_ptr(k) || !is_device_ptr(v))
    return fail(DROPKV_ERR_INVALID, "q, k and v must be device pointers");
  return DROPKV_OK;
}

// Decode-time rescoring: shape checks shared by its entry points. `n` is the
// current token count; need_n is the smallest count the call accepts.
int check_decode(int64_t n, int64_t need_n, int64_t n_max, int32_t window, int32_t Hq, int32_t Hkv, int32_t d,
                 const void* state, size_t state_bytes) {
  if (d != 128) return fail(DROPKV_ERR_INVALID, "decode rescoring needs bf16 inputs with d = 128");
  if (window < 1) return fail(DROPKV_ERR_INVALID, "need window >= 1");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return fail(DROPKV_ERR_INVALID, "need Hq a positive multiple of Hkv >= 1");
  if (Hq / Hkv > 16) return fail(DROPKV_ERR_INVALID, "decode rescoring takes at most 16 query heads per KV head");
  if (n_max > ((int64_t)1 << 31) - 1) return fail(DROPKV_ERR_INVALID, "n_max must fit in int32 token indices");
  if (n < need_n || n > n_max) return fail(DROPKV_ERR_INVALID, "token count out of range for this call (see dropkv.h)");
  if ((double)Hkv * (double)n_max * 128.0 > 1e15 || (double)Hq * window > 1e8)
    return fail(DROPKV_ERR_INVALID, "shape too large");
  hipPointerAttribute_t attr;
  const bool plain_device = state && hipPointerGetAttributes(&attr, state) == hipSuccess &&
                            attr.type == hipMemoryTypeDevice;
  if (!plain_device) (void)hipGetLastError();
  // not managed memory: the single-pass step updates the score with fp64 atomic adds
  if (!state || ((uintptr_t)state & 255) || !plain_device)
    return fail(DROPKV_ERR_INVALID, "state must be a 256-byte aligned device pointer (device memory, not managed)");
  if (carve_decode_state(nullptr, n_max, window, Hq, Hkv).bytes > state_bytes)
    return fail(DROPKV_ERR_INVALID, "state too small (dropkv_decode_state_bytes)");
  return DROPKV_OK;
}

int check_from_stats(const void* q, const void* k, const void* v, int64_t n, int32_t window, int32_t Hq,
                     int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict, const float* m,
                     const float* rest, const int32_t* argmax, const float* a, float* out_scores,
                     int64_t* out_evict_idx) {
  if (const char* msg = validate(DROPKV_BF16, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, msg);
  if (!mfma_supported(DROPKV_BF16, d)) return fail(DROPKV_ERR_INVALID, "scoring from statistics needs bf16 inputs with d = 128");
  if (const char* msg = validate_select(n, window, Hkv, pool_kernel, n_evict)) return fail(DROPKV_ERR_INVALID, msg);
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!m || !rest || !argmax || !a || !is_device_ptr(m) || !is_device_ptr(rest) || !is_device_ptr(argmax) ||
      !is_device_ptr(a))
    return fail(DROPKV_ERR_INVALID, "m, rest, argmax and a must be device pointers");
  if (!out_scores || !is_device_ptr(out_scores)) return fail(DROPKV_ERR_INVALID, "out_scores must be a device pointer");
  if (n_evict > 0 && (!out_evict_idx || !is_device_ptr(out_evict_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  return DROPKV_OK;
}

int enqueue_from_stats(const void* q, const void* k, const void* v, const Shape& s, const Workspace& ws,
                       int32_t pool_kernel, int64_t n_evict, const float* m, const float* rest,
                       const int32_t* argmax, const float* a, float* out_scores, int64_t* out_evict_idx,
                       hipStream_t st) {
  FoldInfo fold{};
  hipError_t e = launch_mfma_from_stats(q, k, v, s, ws, st, m, rest, argmax, a, &fold);
  if (e != hipSuccess) return fail_hip(e, "score from statistics");
  e = launch_select(ws.S, s.n, s.w, s.Hkv, pool_kernel, n_evict, out_scores, out_evict_idx, ws.status, &fold,
                    ws.sel, st);
  if (e != hipSuccess) return fail_hip(e, "select");
  return DROPKV_OK;
}

int score_sync(int dtype, const void* q, const void* k, const void* v, int64_t n, int32_t w,
               int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
               float* out_scores, int64_t* out_idx, hipStream_t st) {
  g_last_error.clear();
  if (const char* m = validate(dtype, n, w, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (const char* m = validate_select(n, w, Hkv, pool_kernel, n_evict)) return fail(DROPKV_ERR_INVALID, m);
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!out_scores || !is_device_ptr(out_scores)) return fail(DROPKV_ERR_INVALID, "out_scores must be a device pointer");
  if (n_evict > 0 && (!out_idx || !is_device_ptr(out_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  const Shape s{n, w, Hq, Hkv, d};
  const bool mfma = use_mfma(dtype, d, 0);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  const size_t need = carve_workspace(nullptr, s, mfma).bytes;
  void* base = nullptr;
  if (int rc = get_workspace(need, &base)) return rc;
  Workspace ws = carve_workspace(base, s, mfma);
  FoldInfo fold{};
  if (int rc = run_scores(dtype, q, k, v, s, ws, mfma, st, nullptr, &fold)) return rc;
  hipError_t e = launch_select(ws.S, n, w, Hkv, pool_kernel, n_evict, out_scores, out_idx, ws.status, &fold, ws.sel, st);
  if (e != hipSuccess) return fail_hip(e, "select");
  return sync_status(ws, st);
}

}  // namespace

// ----------------------------------------------------------------- stage events

hipError_t record_stage(StageEvents* se, const char* name, hipStream_t st) {
  if (!se || se->count >= kMaxStages) return hipSuccess;
  if (name && std::strcmp(name, "start") == 0) return hipEventRecord(se->ev[se->count][0], st);
  // this marker closes the current stage and opens the next one
  se->names[se->count] = name;
  hipError_t e = hipEventRecord(se->ev[se->count][1], st);
  se->count += 1;
  if (e == hipSuccess && se->count < kMaxStages) e = hipEventRecord(se->ev[se->count][0], st);
  return e;
}

// ----------------------------------------------------------------- workspace layout

Workspace carve_workspace(void* base, const Shape& s, bool mfma) {
  Workspace ws{};
  size_t off = 0;
  char* b = (char*)base;
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? (void*)(b + off) : nullptr;
    off = align_up(off + bytes, 256);
    return p;
  };
  const size_t rows = (size_t)s.rows();
  ws.status = (int32_t*)take(sizeof(int32_t));
  ws.S = (float*)take(sizeof(float) * (size_t)s.Hkv * (size_t)s.n);
  ws.rs.m = (float*)take(sizeof(float) * rows);
  ws.rs.rest = (float*)take(sizeof(float) * rows);
  ws.rs.L = (float*)take(sizeof(float) * rows);
  ws.rs.jstar = (int32_t*)take(sizeof(int32_t) * rows);
  ws.rs.fixval = (float*)take(sizeof(float) * rows);
  ws.rs.flag = (int32_t*)take(sizeof(int32_t) * rows);
  ws.rs.a = (float*)take(sizeof(float) * rows * (size_t)s.d);
  ws.sel = take(select_scratch_bytes(s.n, s.Hkv));
  ws.flagcount = (int32_t*)take(sizeof(int32_t) * (size_t)s.Hkv);
  if (mfma) {
    ws.rs.a_bf = (uint16_t*)take(sizeof(uint16_t) * rows * (size_t)s.d);
    ws.rs.na = (float*)take(sizeof(float) * rows);
    ws.rs.bias = (float*)take(sizeof(float) * rows);
    ws.nchunks = mfma_chunks(s);
    ws.part = (uint32_t*)take(sizeof(uint32_t) * (size_t)ws.nchunks * rows * (size_t)(s.d / 2 + 4));
    ws.extra = take(mfma_extra_bytes(s));
  }
  ws.bytes = off;
  return ws;
}

}  // namespace dropkv

using namespace dropkv;

extern "C" {

int dropkv_score(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                 int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                 float* out_scores, int64_t* out_evict_idx, void* stream) {
  return score_sync(DROPKV_BF16, q, k, v, n, window, Hq, Hkv, d, pool_kernel, n_evict, out_scores,
                    out_evict_idx, (hipStream_t)stream);
}

int dropkv_score_f32(const float* q, const float* k, const float* v, int64_t n, int32_t window,
                     int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                     float* out_scores, int64_t* out_evict_idx, void* stream) {
  return score_sync(DROPKV_F32, q, k, v, n, window, Hq, Hkv, d, pool_kernel, n_evict, out_scores,
                    out_evict_idx, (hipStream_t)stream);
}

size_t dropkv_workspace_bytes(int32_t dtype, int64_t n, int32_t window, int32_t Hq, int32_t Hkv,
                              int32_t d) {
  if (validate(dtype, n, window, Hq, Hkv, d)) return 0;
  const Shape s{n, window, Hq, Hkv, d};
  // sized for the larger (MFMA) layout so any flag choice fits
  return carve_workspace(nullptr, s, mfma_supported(dtype, d)).bytes;
}

int dropkv_score_ex(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                    int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                    int64_t n_evict, float* out_scores, int64_t* out_evict_idx, void* workspace,
                    size_t workspace_bytes, int32_t* d_status, uint32_t flags, void* stream) {
  g_last_error.clear();
  if (const char* m = validate(dtype, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (const char* m = validate_select(n, window, Hkv, pool_kernel, n_evict))
    return fail(DROPKV_ERR_INVALID, m);
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!out_scores || !is_device_ptr(out_scores)) return fail(DROPKV_ERR_INVALID, "out_scores must be a device pointer");
  if (n_evict > 0 && (!out_evict_idx || !is_device_ptr(out_evict_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  if (!workspace || ((uintptr_t)workspace & 255) || !is_device_ptr(workspace))
    return fail(DROPKV_ERR_INVALID, "workspace must be a 256-byte aligned device pointer");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const Shape s{n, window, Hq, Hkv, d};
  const bool mfma = use_mfma(dtype, d, flags);
  Workspace ws = carve_workspace(workspace, s, mfma);
  if (ws.bytes > workspace_bytes) return fail(DROPKV_ERR_INVALID, "workspace too small");
  ws.status = d_status;
  hipStream_t st = (hipStream_t)stream;
  StageEvents* se = (flags & DROPKV_FLAG_STAGE_LOG) ? log_slot() : nullptr;
  FoldInfo fold{};
  if (int rc = run_scores(dtype, q, k, v, s, ws, mfma, st, se, &fold)) return rc;
  hipError_t e = launch_select(ws.S, n, window, Hkv, pool_kernel, n_evict, out_scores, out_evict_idx,
                               ws.status, &fold, ws.sel, st, false, se);
  if (e != hipSuccess) return fail_hip(e, "select");
  return DROPKV_OK;
}

int dropkv_score_keep_ex(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                         int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_evict_idx, int64_t* out_keep_idx,
                         void* workspace, size_t workspace_bytes, int32_t* d_status, uint32_t flags,
                         void* stream) {
  g_last_error.clear();
  if (n_evict < n && (!out_keep_idx || !is_device_ptr(out_keep_idx)))
    return fail(DROPKV_ERR_INVALID, "out_keep_idx must be a device pointer when tokens are kept");
  if (const char* m = validate(dtype, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (const char* m = validate_select(n, window, Hkv, pool_kernel, n_evict))
    return fail(DROPKV_ERR_INVALID, m);
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!out_scores || !is_device_ptr(out_scores)) return fail(DROPKV_ERR_INVALID, "out_scores must be a device pointer");
  if (n_evict > 0 && (!out_evict_idx || !is_device_ptr(out_evict_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  if (!workspace || ((uintptr_t)workspace & 255) || !is_device_ptr(workspace))
    return fail(DROPKV_ERR_INVALID, "workspace must be a 256-byte aligned device pointer");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const Shape s{n, window, Hq, Hkv, d};
  const bool mfma = use_mfma(dtype, d, flags);
  Workspace ws = carve_workspace(workspace, s, mfma);
  if (ws.bytes > workspace_bytes) return fail(DROPKV_ERR_INVALID, "workspace too small");
  ws.status = d_status;
  hipStream_t st = (hipStream_t)stream;
  StageEvents* se = (flags & DROPKV_FLAG_STAGE_LOG) ? log_slot() : nullptr;
  FoldInfo fold{};
  if (int rc = run_scores(dtype, q, k, v, s, ws, mfma, st, se, &fold)) return rc;
  hipError_t e = launch_select(ws.S, n, window, Hkv, pool_kernel, n_evict, out_scores, out_evict_idx,
                               ws.status, &fold, ws.sel, st, false, se, out_keep_idx);
  if (e != hipSuccess) return fail_hip(e, "select");
  return DROPKV_OK;
}

int dropkv_score_noalloc(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                         int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                         int64_t n_evict, float* out_scores, int64_t* out_evict_idx, int32_t* d_status,
                         uint32_t flags, void* stream) {
  g_last_error.clear();
  if (flags & DROPKV_FLAG_STAGE_LOG) return fail(DROPKV_ERR_INVALID, "the stage log is not available without allocation");
  if (const char* m = validate(dtype, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (const char* m = validate_select(n, window, Hkv, pool_kernel, n_evict))
    return fail(DROPKV_ERR_INVALID, m);
  const Shape s{n, window, Hq, Hkv, d};
  const bool mfma = use_mfma(dtype, d, flags);
  if (carve_workspace(nullptr, s, mfma).bytes > kNoAllocScratchBytes)
    return fail(DROPKV_ERR_INVALID, "shape needs more scratch than DROPKV_NOALLOC_SCRATCH_BYTES (use dropkv_score_ex)");
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!out_scores || !is_device_ptr(out_scores)) return fail(DROPKV_ERR_INVALID, "out_scores must be a device pointer");
  if (n_evict > 0 && (!out_evict_idx || !is_device_ptr(out_evict_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  void* base = nullptr;
  if (int rc = noalloc_scratch(&base)) return rc;
  Workspace ws = carve_workspace(base, s, mfma);
  ws.status = d_status;  // cleared by the path's first kernel, like every buffer that must start at zero
  hipStream_t st = (hipStream_t)stream;
  FoldInfo fold{};
  if (int rc = run_scores(dtype, q, k, v, s, ws, mfma, st, nullptr, &fold)) return rc;
  hipError_t e = launch_select(ws.S, n, window, Hkv, pool_kernel, n_evict, out_scores, out_evict_idx,
                               ws.status, &fold, ws.sel, st);
  if (e != hipSuccess) return fail_hip(e, "select");
  return DROPKV_OK;
}

int dropkv_prefill_attention(const void* q_all, const void* k, const void* v, int64_t n, int32_t window,
                             int32_t Hq, int32_t Hkv, int32_t d, void* out_o, float* out_m, float* out_rest,
                             int32_t* out_argmax, float* out_a, int32_t* d_status, void* stream) {
  g_last_error.clear();
  if (const char* m = validate(DROPKV_BF16, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (!mfma_supported(DROPKV_BF16, d)) return fail(DROPKV_ERR_INVALID, "prefill attention needs bf16 inputs with d = 128");
  if (Hq / Hkv > 32) return fail(DROPKV_ERR_INVALID, "prefill attention takes at most 32 query heads per KV head");
  if (int rc = check_inputs(q_all, k, v)) return rc;
  for (const void* p : {(const void*)out_o, (const void*)out_m, (const void*)out_rest, (const void*)out_argmax,
                        (const void*)out_a, (const void*)d_status})
    if (!p || !is_device_ptr(p)) return fail(DROPKV_ERR_INVALID, "outputs and d_status must be device pointers");
  hipError_t e = launch_prefill(q_all, k, v, n, window, Hq, Hkv, out_o, out_m, out_rest, out_argmax, out_a,
                                out_rest, out_argmax, d_status, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "prefill attention");
  return DROPKV_OK;
}

int dropkv_raw_scores(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                      int32_t window, int32_t Hq, int32_t Hkv, int32_t d, float* out_S,
                      uint32_t flags, void* stream) {
  g_last_error.clear();
  if (const char* m = validate(dtype, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!out_S || !is_device_ptr(out_S)) return fail(DROPKV_ERR_INVALID, "out_S must be a device pointer");
  const Shape s{n, window, Hq, Hkv, d};
  const bool mfma = use_mfma(dtype, d, flags);
  hipStream_t st = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  void* base = nullptr;
  if (int rc = get_workspace(carve_workspace(nullptr, s, mfma).bytes, &base)) return rc;
  Workspace ws = carve_workspace(base, s, mfma);
  if (int rc = run_scores(dtype, q, k, v, s, ws, mfma, st)) return rc;
  hipError_t e = hipMemcpyAsync(out_S, ws.S, sizeof(float) * (size_t)Hkv * n, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return fail_hip(e, "copy S");
  return sync_status(ws, st);
}

int dropkv_row_stats(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                     int32_t window, int32_t Hq, int32_t Hkv, int32_t d, float* out_m,
                     float* out_rest, int32_t* out_argmax, float* out_a, uint32_t flags,
                     void* stream) {
  g_last_error.clear();
  if (const char* m = validate(dtype, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (int rc = check_inputs(q, k, v)) return rc;
  for (const void* p : {(const void*)out_m, (const void*)out_rest, (const void*)out_argmax, (const void*)out_a})
    if (p && !is_device_ptr(p)) return fail(DROPKV_ERR_INVALID, "outputs must be device pointers");
  const Shape s{n, window, Hq, Hkv, d};
  const bool mfma = use_mfma(dtype, d, flags);
  hipStream_t st = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  void* base = nullptr;
  if (int rc = get_workspace(carve_workspace(nullptr, s, mfma).bytes, &base)) return rc;
  Workspace ws = carve_workspace(base, s, mfma);
  if (int rc = run_scores(dtype, q, k, v, s, ws, mfma, st)) return rc;
  const size_t rows = (size_t)s.rows();
  hipError_t e = hipSuccess;
  if (out_m && e == hipSuccess) e = hipMemcpyAsync(out_m, ws.rs.m, 4 * rows, hipMemcpyDeviceToDevice, st);
  if (out_rest && e == hipSuccess) e = hipMemcpyAsync(out_rest, ws.rs.rest, 4 * rows, hipMemcpyDeviceToDevice, st);
  if (out_argmax && e == hipSuccess) e = hipMemcpyAsync(out_argmax, ws.rs.jstar, 4 * rows, hipMemcpyDeviceToDevice, st);
  if (out_a && e == hipSuccess) e = hipMemcpyAsync(out_a, ws.rs.a, 4 * rows * d, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return fail_hip(e, "copy row stats");
  return sync_status(ws, st);
}

int dropkv_pass1_stats(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                       int32_t Hq, int32_t Hkv, int32_t d, float* out_m, float* out_rest,
                       int32_t* out_argmax, float* out_a, void* stream) {
  return dropkv_row_stats(DROPKV_BF16, q, k, v, n, window, Hq, Hkv, d, out_m, out_rest, out_argmax, out_a, 0u,
                          stream);
}

int dropkv_select(const float* S, int64_t n, int32_t window, int32_t Hkv, int32_t pool_kernel,
                  int64_t n_evict, float* out_scores, int64_t* out_evict_idx, void* stream) {
  g_last_error.clear();
  if (n < 2 || window < 1 || window >= n || Hkv < 1) return fail(DROPKV_ERR_INVALID, "need n >= 2, 1 <= window < n, Hkv >= 1");
  if (n > ((int64_t)1 << 31) - 1) return fail(DROPKV_ERR_INVALID, "n must fit in int32 token indices");
  if (const char* m = validate_select(n, window, Hkv, pool_kernel, n_evict)) return fail(DROPKV_ERR_INVALID, m);
  if (!S || !is_device_ptr(S) || !out_scores || !is_device_ptr(out_scores))
    return fail(DROPKV_ERR_INVALID, "S and out_scores must be device pointers");
  if (n_evict > 0 && (!out_evict_idx || !is_device_ptr(out_evict_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  hipStream_t st = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  void* base = nullptr;
  if (int rc = get_workspace(256 + select_scratch_bytes(n, Hkv), &base)) return rc;
  Workspace ws{};
  ws.status = (int32_t*)base;
  ws.sel = (char*)base + 256;
  hipError_t e = launch_init(ws.status, nullptr, ws.sel, Hkv, st);
  if (e == hipSuccess)
    e = launch_select(S, n, window, Hkv, pool_kernel, n_evict, out_scores, out_evict_idx, ws.status, nullptr,
                      ws.sel, st, /*reject_negative=*/true);
  if (e != hipSuccess) return fail_hip(e, "select");
  return sync_status(ws, st);
}

int dropkv_stage_times(int32_t dtype, const void* q, const void* k, const void* v, int64_t n,
                       int32_t window, int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel,
                       int64_t n_evict, float* out_scores, int64_t* out_evict_idx, uint32_t flags,
                       float* out_ms, char* out_names, int32_t names_bytes, int32_t* out_count,
                       void* stream) {
  g_last_error.clear();
  if (const char* m = validate(dtype, n, window, Hq, Hkv, d)) return fail(DROPKV_ERR_INVALID, m);
  if (const char* m = validate_select(n, window, Hkv, pool_kernel, n_evict)) return fail(DROPKV_ERR_INVALID, m);
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!out_scores || !is_device_ptr(out_scores)) return fail(DROPKV_ERR_INVALID, "out_scores must be a device pointer");
  if (n_evict > 0 && (!out_evict_idx || !is_device_ptr(out_evict_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  if (!out_ms || !out_count) return fail(DROPKV_ERR_INVALID, "out_ms and out_count are required");
  const Shape s{n, window, Hq, Hkv, d};
  const bool mfma = use_mfma(dtype, d, flags);
  hipStream_t st = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  void* base = nullptr;
  if (int rc = get_workspace(carve_workspace(nullptr, s, mfma).bytes, &base)) return rc;
  Workspace ws = carve_workspace(base, s, mfma);
  StageEvents se{};
  for (int i = 0; i < kMaxStages; ++i)
    for (int b = 0; b < 2; ++b) {
      hipError_t e = hipEventCreateWithFlags(&se.ev[i][b], hipEventDisableSystemFence);
      if (e != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags");
    }
  FoldInfo fold{};
  int rc = run_scores(dtype, q, k, v, s, ws, mfma, st, &se, &fold);
  if (rc == DROPKV_OK) {
    hipError_t e = launch_select(ws.S, n, window, Hkv, pool_kernel, n_evict, out_scores, out_evict_idx, ws.status,
                                 &fold, ws.sel, st, false, &se);
    if (e != hipSuccess) rc = fail_hip(e, "select");
  }
  if (rc == DROPKV_OK) rc = sync_status(ws, st);
  if (rc == DROPKV_OK || rc == DROPKV_ERR_SINGULAR || rc == DROPKV_ERR_NONFINITE) {
    std::string names;
    for (int i = 0; i < se.count; ++i) {
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, se.ev[i][0], se.ev[i][1]);
      out_ms[i] = ms;
      names += se.names[i];
      names += (i + 1 < se.count) ? "," : "";
    }
    *out_count = se.count;
    if (out_names && names_bytes > 0) {
      std::strncpy(out_names, names.c_str(), (size_t)names_bytes - 1);
      out_names[names_bytes - 1] = 0;
    }
  }
  for (int i = 0; i < kMaxStages; ++i)
    for (int b = 0; b < 2; ++b) (void)hipEventDestroy(se.ev[i][b]);
  return rc;
}

int dropkv_stage_log(float* out_ms, char* out_names, int32_t names_bytes, int32_t* out_count,
                     int32_t* out_calls) {
  g_last_error.clear();
  if (!out_ms || !out_count || !out_calls) return fail(DROPKV_ERR_INVALID, "out_ms, out_count and out_calls are required");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_log_mutex);
  StageLog& L = g_log[dev];
  const int calls = L.used;
  L.used = 0;
  *out_calls = calls;
  *out_count = 0;
  if (calls == 0) return DROPKV_OK;
  const StageEvents& s0 = L.slot[0];
  for (int c = 0; c < calls; ++c) {
    const StageEvents& sc = L.slot[c];
    if (sc.count != s0.count) return fail(DROPKV_ERR_INVALID, "logged calls ran different stages");
    for (int i = 0; i < sc.count; ++i)
      if (std::strcmp(sc.names[i], s0.names[i]) != 0)
        return fail(DROPKV_ERR_INVALID, "logged calls ran different stages");
    if (sc.count == 0) continue;
    e = hipEventSynchronize(sc.ev[sc.count - 1][1]);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
  }
  std::string names;
  for (int i = 0; i < s0.count; ++i) {
    double acc = 0.0;
    for (int c = 0; c < calls; ++c) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, L.slot[c].ev[i][0], L.slot[c].ev[i][1]);
      if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
      acc += ms;
    }
    out_ms[i] = (float)(acc / calls);
    names += s0.names[i];
    names += (i + 1 < s0.count) ? "," : "";
  }
  *out_count = s0.count;
  if (out_names && names_bytes > 0) {
    std::strncpy(out_names, names.c_str(), (size_t)names_bytes - 1);
    out_names[names_bytes - 1] = 0;
  }
  return DROPKV_OK;
}

int dropkv_score_from_stats(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                            int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                            const float* m, const float* rest, const int32_t* argmax, const float* a,
                            float* out_scores, int64_t* out_evict_idx, void* stream) {
  g_last_error.clear();
  if (int rc = check_from_stats(q, k, v, n, window, Hq, Hkv, d, pool_kernel, n_evict, m, rest, argmax, a,
                                out_scores, out_evict_idx))
    return rc;
  const Shape s{n, window, Hq, Hkv, d};
  hipStream_t st = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  void* base = nullptr;
  if (int rc = get_workspace(carve_workspace(nullptr, s, true).bytes, &base)) return rc;
  Workspace ws = carve_workspace(base, s, true);
  if (int rc = enqueue_from_stats(q, k, v, s, ws, pool_kernel, n_evict, m, rest, argmax, a, out_scores,
                                  out_evict_idx, st))
    return rc;
  return sync_status(ws, st);
}

int dropkv_score_from_stats_ex(const void* q, const void* k, const void* v, int64_t n, int32_t window,
                               int32_t Hq, int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict,
                               const float* m, const float* rest, const int32_t* argmax, const float* a,
                               float* out_scores, int64_t* out_evict_idx, void* workspace,
                               size_t workspace_bytes, int32_t* d_status, void* stream) {
  g_last_error.clear();
  if (int rc = check_from_stats(q, k, v, n, window, Hq, Hkv, d, pool_kernel, n_evict, m, rest, argmax, a,
                                out_scores, out_evict_idx))
    return rc;
  if (!workspace || ((uintptr_t)workspace & 255) || !is_device_ptr(workspace))
    return fail(DROPKV_ERR_INVALID, "workspace must be a 256-byte aligned device pointer");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const Shape s{n, window, Hq, Hkv, d};
  Workspace ws = carve_workspace(workspace, s, true);
  if (ws.bytes > workspace_bytes) return fail(DROPKV_ERR_INVALID, "workspace too small");
  ws.status = d_status;
  return enqueue_from_stats(q, k, v, s, ws, pool_kernel, n_evict, m, rest, argmax, a, out_scores,
                            out_evict_idx, (hipStream_t)stream);
}

int dropkv_compact(int32_t dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                   const int64_t* evict_idx, int64_t n_evict, void* out_k, void* out_v,
                   int32_t* d_status, void* stream) {
  g_last_error.clear();
  if (dtype != DROPKV_BF16 && dtype != DROPKV_F32) return fail(DROPKV_ERR_INVALID, "dtype must be DROPKV_BF16 or DROPKV_F32");
  if (n < 1 || n > ((int64_t)1 << 31) - 1) return fail(DROPKV_ERR_INVALID, "need 1 <= n < 2^31");
  if (Hkv < 1 || d < 1 || d > 4096) return fail(DROPKV_ERR_INVALID, "need Hkv >= 1 and 1 <= d <= 4096");
  if (n_evict < 0 || n_evict > n) return fail(DROPKV_ERR_INVALID, "need 0 <= n_evict <= n");
  if (!k || !v || !is_device_ptr(k) || !is_device_ptr(v)) return fail(DROPKV_ERR_INVALID, "k and v must be device pointers");
  if (n_evict > 0 && (!evict_idx || !is_device_ptr(evict_idx)))
    return fail(DROPKV_ERR_INVALID, "evict_idx must be a device pointer when n_evict > 0");
  if (n_evict < n && (!out_k || !out_v || !is_device_ptr(out_k) || !is_device_ptr(out_v)))
    return fail(DROPKV_ERR_INVALID, "out_k and out_v must be device pointers when tokens are kept");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  hipError_t e = launch_compact(dtype, k, v, n, Hkv, d, evict_idx, n_evict, out_k, out_v, d_status,
                                (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "compact");
  return DROPKV_OK;
}

int dropkv_compact_kept(int32_t dtype, const void* k, const void* v, int64_t n, int32_t Hkv, int32_t d,
                        const int64_t* keep_idx, int64_t n_keep, void* out_k, void* out_v,
                        int32_t* d_status, void* stream) {
  g_last_error.clear();
  if (dtype != DROPKV_BF16 && dtype != DROPKV_F32) return fail(DROPKV_ERR_INVALID, "dtype must be DROPKV_BF16 or DROPKV_F32");
  if (n < 1 || n > ((int64_t)1 << 31) - 1) return fail(DROPKV_ERR_INVALID, "need 1 <= n < 2^31");
  if (Hkv < 1 || d < 1 || d > 4096) return fail(DROPKV_ERR_INVALID, "need Hkv >= 1 and 1 <= d <= 4096");
  if (n_keep < 0 || n_keep > n) return fail(DROPKV_ERR_INVALID, "need 0 <= n_keep <= n");
  if (!k || !v || !is_device_ptr(k) || !is_device_ptr(v)) return fail(DROPKV_ERR_INVALID, "k and v must be device pointers");
  if (n_keep > 0 && (!keep_idx || !is_device_ptr(keep_idx)))
    return fail(DROPKV_ERR_INVALID, "keep_idx must be a device pointer when n_keep > 0");
  if (n_keep > 0 && (!out_k || !out_v || !is_device_ptr(out_k) || !is_device_ptr(out_v)))
    return fail(DROPKV_ERR_INVALID, "out_k and out_v must be device pointers when n_keep > 0");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  hipError_t e = launch_compact_kept(dtype, k, v, n, Hkv, d, keep_idx, n_keep, out_k, out_v, d_status,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "compact_kept");
  return DROPKV_OK;
}

size_t dropkv_decode_state_bytes(int64_t n_max, int32_t window, int32_t Hq, int32_t Hkv, int32_t d) {
  if (d != 128 || window < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq / Hkv > 16 || n_max < 2 ||
      n_max > ((int64_t)1 << 31) - 1)
    return 0;
  return carve_decode_state(nullptr, n_max, window, Hq, Hkv).bytes;
}

int dropkv_decode_init(const void* q, const void* k, const void* v, int64_t n, int64_t n_max, int32_t window,
                       int32_t Hq, int32_t Hkv, int32_t d, void* state, size_t state_bytes, int32_t* d_status,
                       void* stream) {
  g_last_error.clear();
  if (int rc = check_decode(n, (int64_t)window + 1, n_max, window, Hq, Hkv, d, state, state_bytes)) return rc;
  if (int rc = check_inputs(q, k, v)) return rc;
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const DecState S = carve_decode_state(state, n_max, window, Hq, Hkv);
  hipError_t e = launch_decode_init(q, k, v, n, n_max, window, Hq, Hkv, S, d_status, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "decode init");
  return DROPKV_OK;
}

int dropkv_decode_step(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                       int32_t window, int32_t Hq, int32_t Hkv, int32_t d, void* state, size_t state_bytes,
                       int32_t* d_status, void* stream) {
  g_last_error.clear();
  if (int rc = check_decode(n, (int64_t)window + 2, n_max, window, Hq, Hkv, d, state, state_bytes)) return rc;
  if (int rc = check_inputs(q_new, k, v)) return rc;
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const DecState S = carve_decode_state(state, n_max, window, Hq, Hkv);
  hipError_t e = launch_decode_step(q_new, k, v, n, n_max, window, Hq, Hkv, S, d_status, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "decode step");
  return DROPKV_OK;
}

int dropkv_decode_step_deferred(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                                int32_t window, int32_t Hq, int32_t Hkv, int32_t d, void* state, size_t state_bytes,
                                int32_t* d_status, void* stream) {
  g_last_error.clear();
  if (int rc = check_decode(n, (int64_t)window + 2, n_max, window, Hq, Hkv, d, state, state_bytes)) return rc;
  if (int rc = check_inputs(q_new, k, v)) return rc;
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const DecState S = carve_decode_state(state, n_max, window, Hq, Hkv);
  hipError_t e =
      launch_decode_step_deferred(q_new, k, v, n, n_max, window, Hq, Hkv, S, d_status, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "decode deferred step");
  return DROPKV_OK;
}

int dropkv_decode_flush(const void* k, const void* v, int64_t n, int64_t n_max, int32_t window, int32_t Hq,
                        int32_t Hkv, int32_t d, void* state, size_t state_bytes, void* stream) {
  g_last_error.clear();
  if (int rc = check_decode(n, (int64_t)window + 1, n_max, window, Hq, Hkv, d, state, state_bytes)) return rc;
  if (!k || !v || !is_device_ptr(k) || !is_device_ptr(v)) return fail(DROPKV_ERR_INVALID, "k and v must be device pointers");
  const DecState S = carve_decode_state(state, n_max, window, Hq, Hkv);
  hipError_t e = launch_decode_flush(k, v, n, n_max, window, Hq, Hkv, S, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "decode flush");
  return DROPKV_OK;
}

int dropkv_decode_rebuild(const void* k, const void* v, int64_t n, int64_t n_max, int32_t window, int32_t Hq,
                          int32_t Hkv, int32_t d, void* state, size_t state_bytes, int32_t* d_status,
                          void* stream) {
  g_last_error.clear();
  if (int rc = check_decode(n, (int64_t)window + 1, n_max, window, Hq, Hkv, d, state, state_bytes)) return rc;
  if (!k || !v || !is_device_ptr(k) || !is_device_ptr(v)) return fail(DROPKV_ERR_INVALID, "k and v must be device pointers");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const DecState S = carve_decode_state(state, n_max, window, Hq, Hkv);
  hipError_t e = launch_decode_rebuild(k, v, n, n_max, window, Hq, Hkv, S, d_status, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "decode rebuild");
  return DROPKV_OK;
}

int dropkv_decode_scores(const void* state, size_t state_bytes, int64_t n, int64_t n_max, int32_t window,
                         int32_t Hq, int32_t Hkv, int32_t d, float* out_S, void* stream) {
  g_last_error.clear();
  if (int rc = check_decode(n, (int64_t)window + 1, n_max, window, Hq, Hkv, d, state, state_bytes)) return rc;
  if (!out_S || !is_device_ptr(out_S)) return fail(DROPKV_ERR_INVALID, "out_S must be a device pointer");
  const DecState S = carve_decode_state(const_cast<void*>(state), n_max, window, Hq, Hkv);
  hipError_t e = launch_decode_scores(S, n, n_max, Hkv, out_S, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "decode scores");
  return DROPKV_OK;
}

int dropkv_decode_select(void* state, size_t state_bytes, int64_t n, int64_t n_max, int32_t window, int32_t Hq,
                         int32_t Hkv, int32_t d, int32_t pool_kernel, int64_t n_evict, float* out_scores,
                         int64_t* out_evict_idx, int32_t* d_status, void* stream) {
  g_last_error.clear();
  if (int rc = check_decode(n, (int64_t)window + 1, n_max, window, Hq, Hkv, d, state, state_bytes)) return rc;
  if (const char* m = validate_select(n, window, Hkv, pool_kernel, n_evict)) return fail(DROPKV_ERR_INVALID, m);
  if (!out_scores || !is_device_ptr(out_scores)) return fail(DROPKV_ERR_INVALID, "out_scores must be a device pointer");
  if (n_evict > 0 && (!out_evict_idx || !is_device_ptr(out_evict_idx)))
    return fail(DROPKV_ERR_INVALID, "out_evict_idx must be a device pointer when n_evict > 0");
  if (!d_status || !is_device_ptr(d_status)) return fail(DROPKV_ERR_INVALID, "d_status must be a device pointer");
  const DecState S = carve_decode_state(state, n_max, window, Hq, Hkv);
  hipError_t e = launch_decode_select(S, n, n_max, window, Hq, Hkv, pool_kernel, n_evict, out_scores, out_evict_idx,
                                      d_status, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "decode select");
  return DROPKV_OK;
}

int dropkv_uses_mfma(int32_t dtype, int32_t d) { return mfma_supported(dtype, d) ? 1 : 0; }

const char* dropkv_last_error(void) { return g_last_error.c_str(); }

const char* dropkv_last_error_string(void) { return g_last_error.c_str(); }

const char* dropkv_version(void) { return "dropkv-gfx950 0.1"; }

}  // extern "C"
