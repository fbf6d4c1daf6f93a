// QK RMSNorm of the q|k|v projection, then RoPE and the q / paged K/V writes.
//
// The base model the pages augment is Qwen3-8B plus a LoRA (ai-papers-daily
// summary, method key points), whose attention RMS-normalises every query and key
// head over its head dimension, with a learned gain, before the rotary embedding.
// A head's 128 columns come from several workgroups of the projection, so the
// projection stores float32 and this row kernel finishes the epilogue.
#include "uno_qknorm.h"

namespace {

// (page, KV head) block holding a slot of a sequence, or null (bounds flag set)
template <typename T>
__device__ T* kv_block_of(const KvLayout& kv, int layer, int which, int seq, int slot, int h,
                          int32_t* err) {
  const int page = kv_page(kv, seq, slot);
  if (page < 0) {
    if (err) atomicOr(err, UNO_DEVERR_BOUNDS);
    return nullptr;
  }
  return kv_block<T>(kv, layer, which, page, h);
}

}  // namespace

// One wavefront per (row, head) of the float32 q|k|v projection: the sum of
// squares of a q / k head is reduced across the wave, the head is scaled by
// 1 / sqrt(mean(x^2) + eps) and its gain, then each rotary pair (i, i + hd/2) is
// rotated at the row's position; v heads pass through.  Every wave that starts
// also ends (no barriers), so the tail workgroup's spare waves simply return.
template <typename T>
__global__ void __launch_bounds__(256) k_qk_norm_rope(QkNormArgs a) {
  const int Hq = a.n_q_heads, Hkv = a.kv.n_kv_heads, H3 = Hq + 2 * Hkv;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long)a.M * H3) return;
  const int lane = threadIdx.x & 63;
  const int m = (int)(w / H3), head = (int)(w % H3);
  const int hd = a.kv.head_dim, half = hd / 2;
  const float* row = a.in + (size_t)m * a.ldi + (size_t)head * hd;
  // stored column of head dimension `dim`
  auto col = [&](int dim) {
    if (!a.perm) return dim;
    const int hi = dim >= half, i = hi ? dim - half : dim;
    return 16 * (i / 8) + 8 * hi + (i % 8);
  };
  const bool rot = head < Hq + Hkv;
  const int pos = a.row_pos[m];
  if (rot && (pos < 0 || pos >= a.kv.max_pages_per_seq * a.kv.page_size)) {
    if (lane == 0 && a.err) atomicOr(a.err, UNO_DEVERR_BOUNDS);
    return;
  }
  float rs = 1.0f;
  const T* g = nullptr;
  if (rot) {
    float ss = 0.0f;
    for (int dim = lane; dim < hd; dim += 64) {
      const float x = row[col(dim)];
      ss += x * x;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    rs = 1.0f / sqrtf(ss / (float)hd + a.eps);
    g = reinterpret_cast<const T*>(head < Hq ? a.q_gain : a.k_gain);
  }
  T* dst = nullptr;
  int which = 0, tok = 0;
  if (head >= Hq) {
    which = rot ? 0 : 1;
    const int h = head - Hq - which * Hkv;
    const int seq = a.seq_fixed > 0 ? a.seq_fixed - 1 : a.call_seq[m / a.rows_per_seq];
    const int slot = a.row_slot ? a.row_slot[m] : pos;
    dst = kv_block_of<T>(a.kv, a.layer, which, seq, slot, h, lane == 0 ? a.err : nullptr);
    if (!dst) return;
    tok = slot % a.kv.page_size;
  }
  T* q = reinterpret_cast<T*>(a.qbuf) + (size_t)m * Hq * hd + (size_t)head * hd;
  for (int i = lane; i < half; i += 64) {
    float x1 = row[col(i)], x2 = row[col(half + i)];
    if (rot) {
      x1 = x1 * rs * to_f(g[i]);
      x2 = x2 * rs * to_f(g[half + i]);
      const float cs = a.rcos[(size_t)pos * half + i], sn = a.rsin[(size_t)pos * half + i];
      const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
      x1 = y1;
      x2 = y2;
    }
    if (head < Hq) {
      q[i] = from_f<T>(x1);
      q[half + i] = from_f<T>(x2);
    } else {
      dst[kv_elem(a.kv, which, tok, i)] = from_f<T>(x1);
      dst[kv_elem(a.kv, which, tok, half + i)] = from_f<T>(x2);
    }
  }
}

template <typename T>
hipError_t launch_qk_norm_rope(const QkNormArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.kv.head_dim % 2 != 0 || a.ldi < (a.n_q_heads + 2 * a.kv.n_kv_heads) * a.kv.head_dim)
    return hipErrorInvalidValue;
  const long waves = (long)a.M * (a.n_q_heads + 2 * a.kv.n_kv_heads);
  uno_launch(k_qk_norm_rope<T>, dim3((unsigned)((waves + 3) / 4)), 256, 0, s, a);
  return hipGetLastError();
}
template hipError_t launch_qk_norm_rope<float>(const QkNormArgs&, hipStream_t);
template hipError_t launch_qk_norm_rope<bf16>(const QkNormArgs&, hipStream_t);
