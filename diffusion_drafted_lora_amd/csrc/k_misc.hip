// Row set-up, embedding gather, the softmax passes of the LM head, the total
// variation of the distillation forward, small device scatters and KV import /
// export.
//
// The decoder reading (pre-norm RMSNorm, rotate-half RoPE, grouped-query heads)
// is the plain Qwen3-8B-shaped one; the pages fix only that draft and verify
// share one KV cache (shibing624 reading notes of the Uno paper, method core).
#include "uno_internal.h"

namespace {

__device__ float block_sum_256(float v, float* sh) {
  // wave64 reduction, then the 4 wave totals in a fixed order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  __syncthreads();
  return t;
}

__global__ void k_rows_setup(RowsSetup a) {
  const int R = a.n * a.rows_per_seq;
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int i = r / a.rows_per_seq, j = r % a.rows_per_seq;
  const int sid = a.call_seq[i];
  const int n = a.len ? a.len[sid] : 0;
  int tok = 0, pos = 0;
  uint8_t g = 0;
  switch (a.mode) {
    case 0:  // draft: [t, MASK x (B-1)] at n..n+B-1, gate [0, 1, ..., 1]
      tok = (j == 0) ? a.pending[sid] : a.mask_id;
      pos = n + j;
      g = (j > 0) ? 1 : 0;
      break;
    case 1:  // verify: [y_1..y_B] at n+1..n+B, gate 0
      tok = a.draft_tok[(size_t)i * a.B + j];
      pos = n + 1 + j;
      g = 0;
      break;
    case 2:  // caller rows
      tok = a.in_tok ? a.in_tok[r] : 0;
      pos = a.in_pos[r];
      g = a.in_gate[r];
      break;
    case 4: {  // distillation: [x | MASK^L], both halves at RoPE positions 0..L-1
      // (Uno reading notes, "Diffusion Distillation": one forward over [x, z1]
      // with a block-causal mask; the gated LoRA is off on x and on on z1)
      const int Lx = a.rows_per_seq / 2;
      const bool noisy = j >= Lx;
      const int jj = noisy ? j - Lx : j;
      tok = noisy ? a.mask_id : a.in_tok[(size_t)i * Lx + jj];
      pos = jj;
      g = noisy ? 1 : 0;
      const int b0 = jj / a.B * a.B;
      a.row_slot[r] = j;
      // x row: slots [0, jj]; z1 row of block b: x slots [0, bB) and z1 slots bB..jj
      a.row_vis[3 * r] = noisy ? b0 : jj + 1;
      a.row_vis[3 * r + 1] = noisy ? Lx + b0 : INT_MAX;
      a.row_vis[3 * r + 2] = noisy ? Lx + jj : -1;
      break;
    }
    case 5: {  // tree verify: y_1 at n+1 (slot n+1), then chain k's depths 2..B
      // at positions n+2.. in slots base_k.. (base_k = n + 2 + k (B - 1), so chain
      // 0 sits at its own positions); every row sees the context through y_1 and
      // its own chain up to itself, gate 0
      const int Bm = a.B - 1;
      const int32_t* ch = a.draft_tok + (size_t)i * a.K * a.B;
      int slot, c0, d0;
      if (j == 0) {
        tok = ch[0];
        pos = n + 1;
        slot = n + 1;
        c0 = INT_MAX;
        d0 = -1;
      } else {
        const int k = (j - 1) / Bm, dd = (j - 1) % Bm + 2;
        tok = ch[k * a.B + dd - 1];
        pos = n + dd;
        c0 = n + 2 + k * Bm;
        slot = c0 + dd - 2;
        d0 = slot;
      }
      g = 0;
      a.row_slot[r] = slot;
      a.row_vis[3 * r] = n + 2;
      a.row_vis[3 * r + 1] = c0;
      a.row_vis[3 * r + 2] = d0;
      break;
    }
    default:  // prefill rows of one sequence
      tok = a.in_tok[r];
      pos = a.pos0 + r;
      g = 0;
      break;
  }
  a.row_tok[r] = tok;
  a.row_pos[r] = pos;
  a.row_gate[r] = g;
  if (j == 0 && a.call_n) {
    a.call_n[i] = n;
    a.call_it[i] = a.iter ? a.iter[sid] : 0;
  }
}

// x[r] = E[tok[r]] (or the given hidden row); also the first RMSNorm's input
// xg = T(x * g) and the fixed-point sum of x^2 (2^-32 units).  Each thread takes
// groups of eight consecutive columns (16-byte loads of the table row and the
// gains; eight consecutive columns are also eight consecutive elements of the
// fragment-tiled xg).
template <typename T>
__global__ void __launch_bounds__(256)
k_embed(const T* __restrict__ E, const int32_t* __restrict__ tok,
        const float* __restrict__ hidden_in, int d, int V, float* x, const T* g, T* xg,
        long long* ss, int32_t* err) {
  const int r = blockIdx.x;
  float* xr = x + (size_t)r * d;
  const T* er = nullptr;
  if (!hidden_in) {
    int t = tok[r];
    if (t < 0 || t >= V) {
      if (threadIdx.x == 0 && err) atomicOr(err, UNO_DEVERR_NUMERIC);
      t = 0;
    }
    er = E + (size_t)t * d;
  }
  float sq = 0.0f;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float v[8], gv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = hidden_in ? hidden_in[(size_t)r * d + c + e] : to_f(er[c + e]);
      gv[e] = xg ? to_f(g[c + e]) : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xr[c + e] = v[e];
      if (xg) xg[act_off<T>(r, c + e, d)] = from_f<T>(v[e] * gv[e]);
      sq += v[e] * v[e];
    }
  }
  if (ss) {
    // per-wave partials in fixed point, so the total does not depend on order
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if ((threadIdx.x & 63) == 0) ss_add(ss, r, threadIdx.x >> 6, sq, err);
  }
}


// Reduce the per-tile (max, sum exp) partials of one logits row (fixed order):
// each of the 1024 threads merges a strided subset with its loads issued first,
// then thread 0 merges the thread results in thread order.
__global__ void __launch_bounds__(1024)
k_row_stats(const float* __restrict__ tile_stats, int n_tiles, float* row_ml) {
  __shared__ float shm[1024], shs[1024];
  const int r = blockIdx.x;
  const float2* ts = reinterpret_cast<const float2*>(tile_stats + (size_t)r * n_tiles * 2);
  float m = -INFINITY, s = 0.0f;
  for (int t0 = threadIdx.x; t0 < n_tiles; t0 += 4 * blockDim.x) {
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * blockDim.x;
      v[u] = t < n_tiles ? ts[t] : make_float2(-INFINITY, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float mt = v[u].x, st = v[u].y;
      if (mt == -INFINITY) continue;
      if (mt > m) { s = s * expf(m - mt) + st; m = mt; }
      else s += st * expf(mt - m);
    }
  }
  shm[threadIdx.x] = m;
  shs[threadIdx.x] = s;
  __syncthreads();
  // tree merge in a fixed pairing (deterministic)
  for (int off = blockDim.x / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      const float m1 = shm[threadIdx.x], s1 = shs[threadIdx.x];
      const float m2 = shm[threadIdx.x + off], s2 = shs[threadIdx.x + off];
      const float M = fmaxf(m1, m2);
      float S = 0.0f;
      if (m1 != -INFINITY) S += s1 * expf(m1 - M);
      if (m2 != -INFINITY) S += s2 * expf(m2 - M);
      shm[threadIdx.x] = M;
      shs[threadIdx.x] = S;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    row_ml[2 * r] = shm[0];
    row_ml[2 * r + 1] = shs[0];
  }
}

__global__ void k_softmax(const float* __restrict__ logits, const float* __restrict__ row_ml,
                          int V, float* probs) {
  const int r = blockIdx.y;
  const float M = row_ml[2 * r], inv = 1.0f / row_ml[2 * r + 1];
  const size_t base = (size_t)r * V;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < V; j += gridDim.x * blockDim.x)
    probs[base + j] = expf(logits[base + j] - M) * inv;
}

// Total variation of one row pair: 0.5 * sum_v |p_T(v) - p_S(v)| with p = exp(l - max)
// / sum; strided per-thread sums, then a fixed-order block reduction.
__global__ void __launch_bounds__(256)
k_tv(const float* __restrict__ tl, const float* __restrict__ sl, const float* __restrict__ tml,
     const float* __restrict__ sml, int V, float* tv) {
  __shared__ float sh[4];
  const int r = blockIdx.x;
  const float mt = tml[2 * r], it = 1.0f / tml[2 * r + 1];
  const float ms = sml[2 * r], is = 1.0f / sml[2 * r + 1];
  const float* t = tl + (size_t)r * V;
  const float* s = sl + (size_t)r * V;
  float acc = 0.0f;
  for (int j = threadIdx.x; j < V; j += blockDim.x)
    acc += fabsf(expf(t[j] - mt) * it - expf(s[j] - ms) * is);
  acc = block_sum_256(acc, sh);
  if (threadIdx.x == 0) tv[r] = 0.5f * acc;
}

__global__ void k_tv_blocks(const float* __restrict__ tv_row, int nb, int B, float* tv_block) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  float acc = 0.0f;
  for (int i = 0; i < B; ++i) acc += tv_row[(size_t)b * B + i];
  tv_block[b] = acc / (float)B;
}

// One thread per 16-byte piece of the fragment-tiled output.
__global__ void k_pack(const bf16* __restrict__ src, bf16* __restrict__ dst, int rows, int cols,
                       int pair_hd) {
  const size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (q >= (size_t)rows * cols / 8) return;
  const int cb_n = cols / 32;
  const size_t block = q / 64;
  const int lane = (int)(q % 64);
  const int r = (int)(block / cb_n) * 16 + (lane & 15);
  const int c = (int)(block % cb_n) * 32 + (lane >> 4) * 8;
  int sr = r;
  if (pair_hd > 0) {
    const int i = r % pair_hd, j = i / 16, cc = i % 16;
    sr = r - i + (cc < 8 ? 8 * j + cc : pair_hd / 2 + 8 * j + (cc - 8));
  }
  *reinterpret_cast<uint4*>(dst + q * 8) =
      *reinterpret_cast<const uint4*>(src + (size_t)sr * cols + c);
}

// Row-major copy of a fragment-tiled bf16 activation, eight columns per thread
// (eight consecutive columns of a row are eight consecutive elements of a block).
__global__ void __launch_bounds__(256)
k_untile(const bf16* __restrict__ src, bf16* __restrict__ dst, int R, int C) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  const int per = C / 8;
  if (i >= (long)R * per) return;
  const int r = (int)(i / per), c = (int)(i % per) * 8;
  *reinterpret_cast<bf16x8*>(dst + (size_t)r * C + c) =
      *reinterpret_cast<const bf16x8*>(src + frag_off(r, c, C));
}

__global__ void k_set_list(SetList l) {
  for (int i = threadIdx.x; i < l.count; i += blockDim.x) l.dst[l.idx[i]] = l.val[i];
}

// Contiguous [layers][len][Hkv][hd] <-> pages of one sequence.
template <typename T>
__global__ void k_kv_copy(KvLayout kv, int seq, int len, T* k, T* v, int to_pages) {
  const int pos = blockIdx.x, layer = blockIdx.y;
  const int hd = kv.head_dim, Hkv = kv.n_kv_heads;
  const int page = kv_page(kv, seq, pos), tk = pos % kv.page_size;
  if (page < 0) return;
  for (int e = threadIdx.x; e < Hkv * hd; e += blockDim.x) {
    const int h = e / hd, i = e % hd;
    const size_t c = (((size_t)layer * len + pos) * Hkv + h) * hd + i;
    T* pk = kv_block<T>(kv, layer, 0, page, h) + kv_elem(kv, 0, tk, i);
    T* pv = kv_block<T>(kv, layer, 1, page, h) + kv_elem(kv, 1, tk, i);
    if (to_pages) { *pk = k[c]; *pv = v[c]; }
    else { k[c] = *pk; v[c] = *pv; }
  }
}


typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Read-only stream of n16 16-byte words: thread t reads words t, t + T, t + 2T, ...
// (T threads in the grid; each wave's loads are 1 KB contiguous), U loads in flight
// per thread, nontemporal like the linear kernels' weight stream; the xor of what a
// workgroup read goes to sink[workgroup], so the loads cannot be dropped.
template <int U>
__global__ void __launch_bounds__(1024)
k_stream_read(const i32x4_t* __restrict__ src, size_t n16, int32_t* sink) {
  __shared__ int red[16];
  const size_t T = (size_t)gridDim.x * blockDim.x;
  i32x4_t acc = {0, 0, 0, 0};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += U * T) {
    i32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * T;
      v[u] = j < n16 ? __builtin_nontemporal_load(src + j) : i32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  int x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = 0;
    for (int w = 0; w < (int)(blockDim.x + 63) / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_rows_setup(const RowsSetup& a, hipStream_t s) {
  const int R = a.n * a.rows_per_seq;
  if (R <= 0) return hipSuccess;
  uno_launch(k_rows_setup, (R + 255) / 256, 256, 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed(const T* E, const int32_t* tok, const float* hidden_in, int R, int d,
                        int V, float* x, const T* g, T* xg, long long* ss, int32_t* err,
                        hipStream_t s) {
  if (d % 8) return hipErrorInvalidValue;
  uno_launch(k_embed<T>, R, 256, 0, s, E, tok, hidden_in, d, V, x, g, xg, ss, err);
  return hipGetLastError();
}

hipError_t launch_row_stats(const float* tile_stats, int R, int n_tiles, float* row_ml,
                            hipStream_t s) {
  uno_launch(k_row_stats, R, 1024, 0, s, tile_stats, n_tiles, row_ml);
  return hipGetLastError();
}

hipError_t launch_softmax(const float* logits, const float* row_ml, int R, int V, float* probs,
                          hipStream_t s) {
  const int bx = (V + 1023) / 1024 < 64 ? (V + 1023) / 1024 : 64;
  uno_launch(k_softmax, dim3(bx, R), 256, 0, s, logits, row_ml, V, probs);
  return hipGetLastError();
}

hipError_t launch_tv(const float* t_logits, const float* s_logits, const float* t_ml,
                     const float* s_ml, int L, int V, float* tv_row, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  uno_launch(k_tv, L, 256, 0, s, t_logits, s_logits, t_ml, s_ml, V, tv_row);
  return hipGetLastError();
}

hipError_t launch_tv_blocks(const float* tv_row, int L, int B, float* tv_block, hipStream_t s) {
  if (L <= 0 || B <= 0 || L % B) return hipErrorInvalidValue;
  const int nb = L / B;
  uno_launch(k_tv_blocks, (nb + 255) / 256, 256, 0, s, tv_row, nb, B, tv_block);
  return hipGetLastError();
}

hipError_t launch_pack(const bf16* src, bf16* dst, int rows, int cols, int pair_hd, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return hipErrorInvalidValue;
  if (pair_hd > 0 && (pair_hd % 16 || rows % pair_hd)) return hipErrorInvalidValue;
  const size_t n = (size_t)rows * cols / 8;
  uno_launch(k_pack, (unsigned)((n + 255) / 256), 256, 0, s, src, dst, rows, cols, pair_hd);
  return hipGetLastError();
}

template <>
hipError_t launch_untile<bf16>(const bf16* src, bf16* dst, int R, int C, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (C % 32) return hipErrorInvalidValue;
  const long n = (long)R * (C / 8);
  uno_launch(k_untile, (unsigned)((n + 255) / 256), 256, 0, s, src, dst, R, C);
  return hipGetLastError();
}
template <>
hipError_t launch_untile<float>(const float* src, float* dst, int R, int C, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  return hipMemcpyAsync(dst, src, sizeof(float) * (size_t)R * C, hipMemcpyDeviceToDevice, s);
}

hipError_t launch_set_list(const SetList& l, hipStream_t s) {
  if (l.count <= 0) return hipSuccess;
  uno_launch(k_set_list, 1, 256, 0, s, l);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_kv_copy(const KvLayout& kv, int seq, int len, T* k, T* v, int to_pages,
                          hipStream_t s) {
  if (len <= 0) return hipSuccess;
  uno_launch(k_kv_copy<T>, dim3(len, kv.n_layers), 256, 0, s, kv, seq, len, k, v, to_pages);
  return hipGetLastError();
}

#define UNO_INST(T)                                                                         \
  template hipError_t launch_embed<T>(const T*, const int32_t*, const float*, int, int, int, \
                                      float*, const T*, T*, long long*, int32_t*,           \
                                      hipStream_t);                                         \
  template hipError_t launch_kv_copy<T>(const KvLayout&, int, int, T*, T*, int, hipStream_t);
UNO_INST(float)
UNO_INST(bf16)

hipError_t launch_stream_read(const void* src, size_t bytes, int workgroups, int threads, int loads,
                              int32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const i32x4_t* p = static_cast<const i32x4_t*>(src);
  switch (loads) {
    case 1: uno_launch(k_stream_read<1>, workgroups, threads, 0, s, p, n16, sink); break;
    case 2: uno_launch(k_stream_read<2>, workgroups, threads, 0, s, p, n16, sink); break;
    case 4: uno_launch(k_stream_read<4>, workgroups, threads, 0, s, p, n16, sink); break;
    case 8: uno_launch(k_stream_read<8>, workgroups, threads, 0, s, p, n16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
