// The q|k|v epilogue with the per-head QK RMSNorm (the Qwen3 attention of the base
// model that the Uno pages augment: ai-papers-daily summary, method key points).
#pragma once
#include "uno_internal.h"

// The projection was stored as float32 rows [M, ldi] (q heads, then K heads, then
// V heads; `perm` 1 when the columns of each head are in the pair-permuted order
// of the packed bf16 weights -- a 16-column tile holds dims 8j..8j+7 and
// hd/2+8j..+7 -- and 0 when natural).  Each q / k head is scaled by
// 1 / sqrt(mean(x^2) + eps) and its gain and then rotated pairwise (i, i + hd/2)
// at the row's position; v heads are copied.  q goes to qbuf [M, Hq * hd]; K / V
// go to slot row_slot[m] (row_pos[m] when null) of the row's sequence
// (seq_fixed - 1 when > 0, else call_seq[m / rows_per_seq]).  A position outside
// the RoPE table or a slot outside the sequence's pages sets the bounds flag in
// err and skips that head.
struct QkNormArgs {
  const float* in;
  int32_t ldi, M, n_q_heads, perm;
  const void* q_gain;   // [head_dim] of the storage type
  const void* k_gain;
  float eps;
  const int32_t* row_pos;
  const int32_t* row_slot;
  const int32_t* call_seq;
  int32_t seq_fixed, rows_per_seq;
  const float* rcos;    // [positions, hd/2]
  const float* rsin;
  void* qbuf;
  KvLayout kv;
  int32_t layer;
  int32_t* err;
};
template <typename T> hipError_t launch_qk_norm_rope(const QkNormArgs& a, hipStream_t s);
