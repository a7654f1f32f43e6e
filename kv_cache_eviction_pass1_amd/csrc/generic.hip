// Plain-VALU DropKV path for any element type and head dim (d <= 256).
//
// Used for fp32 inputs and shapes the MFMA path does not cover. It favours
// accuracy over speed: logits and softmax in fp32 with expf, the output a and
// ||a - v_j||^2 as direct differences, and the argmax term of every row
// from D = sum_{i != j*} e_i (v_i - v_{j*}) so that 1 - p_{j*} never
// cancels (core formula of the DropKV write-up, section 核心公式:
// Delta_j = p_j/(1-p_j) (a - v_j); for j = j*, a - v_{j*} = D / L and
// p/(1-p) = 1/R, hence ||Delta_{j*}||^2 = ||D||^2 / (R L)^2).
#include "dropkv_common.h"

namespace dropkv {

namespace {

constexpr int kRowThreads = 256;

template <typename T>
__device__ __forceinline__ float dot_f_t(const float* __restrict__ qf, const T* __restrict__ kr, int d) {
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(qf[c], Elem<T>::get(kr, c), acc);
  return acc;
}

// One block per window row: max/argmax, rest mass R, a = sum p v, and the
// argmax term. Two sweeps over the visible keys; the second recomputes the
// logits with the same instruction sequence, so x_{j*} - m is exactly 0.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_generic_rows(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t n, int w,
    int Hq, int Hkv, int d, RowStats rs, int32_t* status) {
  const int row = blockIdx.x;
  const int h = row / w, i = row % w;
  const int G = Hq / Hkv, g = h / G;
  const int64_t last = n - w + i;  // keys 0..last are visible
  const T* kg = k + (size_t)g * n * d;
  const T* vg = v + (size_t)g * n * d;
  const int tid = threadIdx.x;

  __shared__ float qs[256];
  __shared__ float vstar[256];
  __shared__ float etile[kRowThreads];
  __shared__ float red[kRowThreads];
  __shared__ float redA[kRowThreads];
  __shared__ float redD[kRowThreads];
  __shared__ int64_t redj[kRowThreads];
  __shared__ int nan_seen;

  const float scale = 1.0f / sqrtf((float)d);
  if (tid == 0) nan_seen = 0;
  for (int c = tid; c < d; c += kRowThreads) qs[c] = Elem<T>::get(q, (size_t)row * d + c);
  __syncthreads();

  // sweep 1: max and lowest-index argmax
  float best = -INFINITY;
  int64_t bj = INT64_MAX;
  bool nan = false;
  for (int64_t j = tid; j <= last; j += kRowThreads) {
    float x = dot_f_t<T>(qs, kg + (size_t)j * d, d) * scale;
    if (x != x) nan = true;
    if (x > best) { best = x; bj = j; }
  }
  if (nan) nan_seen = 1;
  red[tid] = best;
  redj[tid] = bj;
  __syncthreads();
  for (int o = kRowThreads / 2; o > 0; o >>= 1) {
    if (tid < o) {
      float b = red[tid + o];
      int64_t jb = redj[tid + o];
      if (b > red[tid] || (b == red[tid] && jb < redj[tid])) { red[tid] = b; redj[tid] = jb; }
    }
    __syncthreads();
  }
  const float m = red[0];
  int64_t js = redj[0];
  const bool bad = nan_seen || !finite_f(m) || js == INT64_MAX;
  if (js == INT64_MAX) js = 0;
  __syncthreads();
  for (int c = tid; c < d; c += kRowThreads) vstar[c] = Elem<T>::get(vg, (size_t)js * d + c);

  // sweep 2: e_j = exp(x_j - m); R = sum_{j != j*} e_j; A = sum e_j v_j;
  // D = sum e_j (v_j - v_{j*}) (the j* term is exactly 0)
  const int nsub = kRowThreads / d;
  const int dim = tid % d, sub = tid / d;
  const bool active = sub < nsub;
  float A = 0.f, D = 0.f, Rp = 0.f;
  for (int64_t t0 = 0; t0 <= last; t0 += kRowThreads) {
    __syncthreads();
    const int64_t j = t0 + tid;
    float e = 0.f;
    if (j <= last) {
      float x = dot_f_t<T>(qs, kg + (size_t)j * d, d) * scale;
      e = expf(x - m);
      if (j != js) Rp += e;
    }
    etile[tid] = e;
    __syncthreads();
    if (active) {
      const int cnt = (int)((last + 1 - t0) < kRowThreads ? (last + 1 - t0) : kRowThreads);
      for (int t = sub; t < cnt; t += nsub) {
        const float ej = etile[t];
        const float vv = Elem<T>::get(vg, (size_t)(t0 + t) * d + dim);
        A = fmaf(ej, vv, A);
        D = fmaf(ej, vv - vstar[dim], D);
      }
    }
  }
  __syncthreads();
  redA[tid] = active ? A : 0.f;
  redD[tid] = active ? D : 0.f;
  const float R = block_sum<kRowThreads>(Rp, red);  // also syncs redA/redD
  const float L = 1.0f + R;
  float dsq = 0.f;
  if (tid < d) {
    float At = 0.f, Dt = 0.f;
    for (int s = 0; s < nsub; ++s) { At += redA[s * d + tid]; Dt += redD[s * d + tid]; }
    rs.a[(size_t)row * d + tid] = At / L;
    dsq = Dt * Dt;
  }
  __syncthreads();
  const float dnorm2 = block_sum<kRowThreads>(dsq, red);
  if (tid == 0) {
    rs.m[row] = m;
    rs.rest[row] = R;
    rs.L[row] = L;
    rs.jstar[row] = (int32_t)js;
    const float RL = R * L;
    rs.fixval[row] = dnorm2 / (RL * RL);
    rs.flag[row] = 1;
    if (bad || !finite_f(R)) atomicOr(status, kStatusNonFinite);
    else if (R <= kSingularRest) atomicOr(status, kStatusSingular);
  }
}

// One thread per (KV head, token): S_g(j) = (1/G) sum over the group's rows of
// ||Delta_j||^2, with ||a - v_j||^2 as a direct sum of squared differences.
template <typename T>
__global__ __launch_bounds__(256) void k_generic_scores(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t n, int w,
    int Hq, int Hkv, int d, RowStats rs, float* __restrict__ S) {
  const int g = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int G = Hq / Hkv;
  const T* kj = k + ((size_t)g * n + j) * d;
  const T* vj = v + ((size_t)g * n + j) * d;
  const float scale = 1.0f / sqrtf((float)d);
  float acc = 0.f;
  for (int t = 0; t < G; ++t) {
    for (int i = 0; i < w; ++i) {
      if (j > n - w + i) continue;  // not visible to this row: p_j = 0
      const int row = (g * G + t) * w + i;
      float c;
      if (j == rs.jstar[row]) {
        c = rs.fixval[row];
      } else {
        const T* qr = q + (size_t)row * d;
        float x = 0.f;
        for (int cc = 0; cc < d; ++cc) x = fmaf(Elem<T>::get(qr, cc), Elem<T>::get(kj, cc), x);
        x *= scale;
        const float e = expf(x - rs.m[row]);
        const float ratio = e / (rs.L[row] - e);  // p/(1-p) = e/(L-e)
        const float* ar = rs.a + (size_t)row * d;
        float dist = 0.f;
        for (int cc = 0; cc < d; ++cc) {
          const float df = ar[cc] - Elem<T>::get(vj, cc);
          dist = fmaf(df, df, dist);
        }
        c = ratio * ratio * dist;
      }
      acc += c;
    }
  }
  S[(size_t)g * n + j] = acc / (float)G;
}

}  // namespace

hipError_t launch_generic_rows(int dtype, const void* q, const void* k, const void* v,
                               const Shape& s, const Workspace& ws, hipStream_t st) {
  dim3 grid((unsigned)s.rows());
  if (dtype == 0)
    k_generic_rows<uint16_t><<<grid, kRowThreads, 0, st>>>((const uint16_t*)q, (const uint16_t*)k,
                                                           (const uint16_t*)v, s.n, s.w, s.Hq, s.Hkv,
                                                           s.d, ws.rs, ws.status);
  else
    k_generic_rows<float><<<grid, kRowThreads, 0, st>>>((const float*)q, (const float*)k,
                                                        (const float*)v, s.n, s.w, s.Hq, s.Hkv, s.d,
                                                        ws.rs, ws.status);
  return hipGetLastError();
}

hipError_t launch_generic_scores(int dtype, const void* q, const void* k, const void* v,
                                 const Shape& s, const Workspace& ws, hipStream_t st) {
  dim3 grid((unsigned)((s.n + 255) / 256), (unsigned)s.Hkv);
  if (dtype == 0)
    k_generic_scores<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)q, (const uint16_t*)k,
                                                     (const uint16_t*)v, s.n, s.w, s.Hq, s.Hkv, s.d,
                                                     ws.rs, ws.S);
  else
    k_generic_scores<float><<<grid, 256, 0, st>>>((const float*)q, (const float*)k, (const float*)v,
                                                  s.n, s.w, s.Hq, s.Hkv, s.d, ws.rs, ws.S);
  return hipGetLastError();
}

}  // namespace dropkv
