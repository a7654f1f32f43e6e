// Decode-time rescoring (decode.hip): state layout and launchers, for the
// C-ABI entry points in api.hip.
#pragma once

#include "dropkv_common.h"

namespace dropkv {

constexpr int kStatusPending = 8;  // the score was read while a single-pass step's terms were pending

// Decode-time rescoring state (decode.hip), carved from one caller-owned
// allocation. The window's rows live in a ring of w + 1 slots per KV head (the
// row at position p in slot p mod (w + 1), so the position being appended and
// the one leaving the window never share a slot); row index
// ((g * (w + 1) + slot) * G + h) for query head h of KV head g's G.
struct DecRows {
  uint16_t* q;      // [rows][128] query (bf16)
  float* a;         // [rows][128] attention output
  uint16_t* a_bf;   // [rows][128] a rounded to bf16 (MFMA operand)
  float* m;         // largest logit (natural units)
  float* L;         // 1 + R
  float* R;         // rest mass sum_{j != argmax} exp(x_j - m)
  float* cstar;     // argmax term added for this row (0 if none)
  float* bias;      // m log2(e) + log2(L)
  float* cinit;     // -||a_bf16||^2 / 2
  int32_t* jstar;   // argmax of rows with R < 1 (scored apart), else -1
};
// pend[0]: the position whose rows' terms a single-pass step left out of S
// (-1: none); pend[1]: the position a two-pass step or a flush adds (copied
// from pend[0] by the kernel before it).
struct DecState {
  double* S64;      // [Hkv][n_max] raw GQA-mean scores, fp64
  DecRows T;
  int64_t* pend;    // [2]
  float* part;      // new-row partials [nch][Hkv][G][132]
  int nch;
  void* ws_base;    // MFMA workspace for the first window's row statistics and for the select
  size_t bytes;
};
DecState carve_decode_state(void* base, int64_t n_max, int32_t w, int32_t Hq, int32_t Hkv);
// First window: row statistics (MFMA pass 1, merge, fix-up), slots, fp64 score.
// Clears *status first. k, v: [Hkv][n_max][128] bf16 holding n tokens.
hipError_t launch_decode_init(const void* q, const void* k, const void* v, int64_t n, int64_t n_max, int32_t w,
                              int32_t Hq, int32_t Hkv, const DecState& S, int32_t* status, hipStream_t st);
// One appended token (n counts it): new rows' statistics and argmax terms,
// signed terms of the new and the leaving rows. ORs status bits.
hipError_t launch_decode_step(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                              int32_t w, int32_t Hq, int32_t Hkv, const DecState& S, int32_t* status,
                              hipStream_t st);
// One appended token in one pass over K and V (G <= 8; larger groups take the
// two-pass step): the new rows' statistics, the leaving rows' terms
// subtracted and the terms an earlier single-pass step left pending added; the
// new rows' terms stay pending (pend[0] = n - 1).
hipError_t launch_decode_step_deferred(const void* q_new, const void* k, const void* v, int64_t n, int64_t n_max,
                                       int32_t w, int32_t Hq, int32_t Hkv, const DecState& S, int32_t* status,
                                       hipStream_t st);
// Adds the pending terms, if any.
hipError_t launch_decode_flush(const void* k, const void* v, int64_t n, int64_t n_max, int32_t w, int32_t Hq,
                               int32_t Hkv, const DecState& S, hipStream_t st);
// The fp64 score recomputed from the stored window rows (no new statistics).
hipError_t launch_decode_rebuild(const void* k, const void* v, int64_t n, int64_t n_max, int32_t w, int32_t Hq,
                                 int32_t Hkv, const DecState& S, int32_t* status, hipStream_t st);
// S in fp32; ORs kStatusPending into *status (if given) while terms are pending.
hipError_t launch_decode_scores(const DecState& S, int64_t n, int64_t n_max, int32_t Hkv, float* out,
                                int32_t* status, hipStream_t st);
hipError_t launch_decode_select(const DecState& S, int64_t n, int64_t n_max, int32_t w, int32_t Hq, int32_t Hkv,
                                int32_t pool_kernel, int64_t n_evict, float* out_scores, int64_t* out_idx,
                                int32_t* status, hipStream_t st);

}  // namespace dropkv
