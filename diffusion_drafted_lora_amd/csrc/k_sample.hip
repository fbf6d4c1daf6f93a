// Keyed sampling kernels of the Psi-Spec step: the integer inverse-CDF draw, the
// draft-slot draws, the accept/reject test and the commit.
//
// Method: the first drafted token is drawn from the AR row and always kept; the
// others come from the diffusion rows; verification keeps the longest accepted
// prefix and resamples the first rejected slot from max(0, p - q) renormalised
// (shibing624 reading notes of the Uno paper, section on the Psi-Spec sampler;
// the ai-papers-daily summary, method key points).  Keys and counters follow the
// Philox reading in uno.h.
//
// Determinism: a draw is an inverse CDF over integer weights trunc(w * 2^40).
// Integer sums are exact, so the chunked parallel scan below returns the same
// index as any sequential loop, whatever the reduction order.
#include "uno_internal.h"

namespace {

// Integer weight of entry j: modes 0 / 1 take trunc(w * 2^40) of the float row;
// mode 2 reads the integer masses of a uint64 row (the tree sampler's residual).
__device__ uint64_t row_iweight(const RowDesc& d, int mode, int j, int32_t* err) {
  if (mode == 2) return reinterpret_cast<const uint64_t*>(d.a)[j];
  return int_weight(row_weight(d, mode, j), err);
}

// Inclusive Hillis-Steele scan of one uint64 per thread in LDS; returns the
// exclusive prefix of this thread and writes the block total to *total.
__device__ uint64_t block_excl_scan(uint64_t v, uint64_t* sh, uint64_t* total) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < CDF_THREADS; off <<= 1) {
    const uint64_t add = (t >= off) ? sh[t - off] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  const uint64_t incl = sh[t];
  *total = sh[CDF_THREADS - 1];
  __syncthreads();
  return incl - v;
}

// Sum of the integer weights of one chunk, computed by the whole block.
__device__ uint64_t chunk_sum(const RowDesc& d, int mode, int c, int V, int32_t* err,
                              uint64_t* sh) {
  const int per = CDF_CHUNK / CDF_THREADS;
  const int j0 = c * CDF_CHUNK + threadIdx.x * per;
  uint64_t s = 0;
  for (int e = 0; e < per; ++e) {
    const int j = j0 + e;
    if (j < V) s += row_iweight(d, mode, j, err);
  }
  uint64_t tot;
  block_excl_scan(s, sh, &tot);
  return tot;
}

__global__ void __launch_bounds__(CDF_THREADS)
k_cdf_chunks(const RowDesc* __restrict__ desc, int V, int n_chunks, uint64_t* chunk_tot,
             int32_t* err) {
  __shared__ uint64_t sh[CDF_THREADS];
  const int c = blockIdx.x, r = blockIdx.y;
  const RowDesc d = desc[r];
  const uint64_t tot = chunk_sum(d, d.mode, c, V, err, sh);
  if (threadIdx.x == 0) chunk_tot[(size_t)r * n_chunks + c] = tot;
}

// One block per row: locate the chunk holding the threshold, then the index.
__global__ void __launch_bounds__(CDF_THREADS)
k_cdf_select(const RowDesc* __restrict__ desc, int V, int n_chunks,
             const uint64_t* __restrict__ chunk_tot, int32_t* err) {
  __shared__ uint64_t sh[CDF_THREADS];
  __shared__ uint64_t s_tot[1024];
  __shared__ uint64_t s_excl[1024];
  __shared__ int s_chunk;
  __shared__ int s_idx;
  const int r = blockIdx.x;
  const RowDesc d = desc[r];
  int mode = d.mode;

  // per-chunk totals and their exclusive prefix (n_chunks <= 1024)
  for (int c = threadIdx.x; c < n_chunks; c += CDF_THREADS)
    s_tot[c] = chunk_tot[(size_t)r * n_chunks + c];
  __syncthreads();
  uint64_t T = 0;
  for (int pass = 0; pass < 2; ++pass) {
    if (threadIdx.x == 0) {
      uint64_t run = 0;
      for (int c = 0; c < n_chunks; ++c) { s_excl[c] = run; run += s_tot[c]; }
      sh[0] = run;
    }
    __syncthreads();
    T = sh[0];
    __syncthreads();
    if (T != 0 || mode != 1) break;
    // residual without integer mass: fall back to the plain row a[]
    mode = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const uint64_t t = chunk_sum(d, 0, c, V, err, sh);
      if (threadIdx.x == 0) s_tot[c] = t;
    }
    __syncthreads();
  }
  if (T == 0) {
    if (threadIdx.x == 0) {
      if (err) atomicOr(err, UNO_DEVERR_NUMERIC);
      *d.out = -1;
    }
    return;
  }
  const uint64_t tau = __umul64hi(d.word, T);
  if (threadIdx.x == 0) s_chunk = -1;
  __syncthreads();
  for (int c = threadIdx.x; c < n_chunks; c += CDF_THREADS)
    if (s_tot[c] != 0 && s_excl[c] <= tau && tau - s_excl[c] < s_tot[c]) s_chunk = c;
  __syncthreads();
  const int c = s_chunk;
  const uint64_t tau_c = tau - s_excl[c];

  // within the chunk: per-thread sums, block scan, sequential search in one thread
  const int per = CDF_CHUNK / CDF_THREADS;
  const int j0 = c * CDF_CHUNK + threadIdx.x * per;
  uint64_t w[CDF_CHUNK / CDF_THREADS];
  uint64_t s = 0;
  for (int e = 0; e < per; ++e) {
    const int j = j0 + e;
    w[e] = (j < V) ? row_iweight(d, mode, j, nullptr) : 0;
    s += w[e];
  }
  uint64_t tot;
  const uint64_t base = block_excl_scan(s, sh, &tot);
  if (threadIdx.x == 0) s_idx = -1;
  __syncthreads();
  if (s != 0 && base <= tau_c && tau_c - base < s) {
    uint64_t run = base;
    for (int e = 0; e < per; ++e) {
      run += w[e];
      if (tau_c < run) { s_idx = j0 + e; break; }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) *d.out = s_idx;
}

__global__ void k_draft_desc(const float* probs, int n, int B, int V, uint64_t seed,
                             const int32_t* call_seq, const int32_t* call_n,
                             const int32_t* call_it, int32_t* out_tok, RowDesc* desc) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n * B) return;
  const int s = r / B, j = r % B;   // row j draws the token at position n + j + 1
  RowDesc d;
  d.a = probs + (size_t)r * V;
  d.b = nullptr;
  d.mode = 0;
  d.pad = 0;
  d.word = draw_word(seed, call_seq[s], call_n[s] + j + 1, STREAM_DRAFT, call_it[s]);
  d.out = out_tok + r;
  desc[r] = d;
}

__global__ void k_sample_desc(const float* w, int rows, int V, uint64_t seed,
                              const int32_t* seq_ids, const int32_t* pos, const int32_t* it,
                              int stream_id, int32_t* out, RowDesc* desc) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  RowDesc d;
  d.a = w + (size_t)r * V;
  d.b = nullptr;
  d.mode = 0;
  d.pad = 0;
  d.word = draw_word(seed, seq_ids[r], pos[r], stream_id, it[r]);
  d.out = out + r;
  desc[r] = d;
}

// One wavefront per sequence: lane i-2 tests slot i (i = 2..B); the first failing
// lane (ballot) is the first rejected slot k.  The test is one float32 multiply
// and a strict compare.  The correction row is the residual of slot k, or the
// bonus row p_{B+1} when every slot passes.
__global__ void __launch_bounds__(64)
k_accept_test(uint64_t seed, int B, int V, const float* __restrict__ p,
              const float* __restrict__ q, int q_stride, const int32_t* __restrict__ draft,
              const int32_t* call_seq, const int32_t* call_n, const int32_t* call_it,
              int32_t* k_out, int32_t* z_out, RowDesc* desc, int32_t* err) {
  const int s = blockIdx.x, lane = threadIdx.x;
  const int sid = call_seq[s], nn = call_n[s], it = call_it[s];
  const int i = lane + 2;
  bool fail = false;
  if (i <= B) {
    const int y = draft[(size_t)s * B + (i - 1)];
    if (y < 0 || y >= V) {
      if (err) atomicOr(err, UNO_DEVERR_NUMERIC);
      fail = true;
    } else {
      const float qy = q[((size_t)s * q_stride + (i - 2)) * V + y];
      const float py = p[((size_t)s * B + (i - 2)) * V + y];
      if (!(qy >= 0.0f && qy <= 1.0f) || !(py >= 0.0f && py <= 1.0f))
        if (err) atomicOr(err, UNO_DEVERR_NUMERIC);
      const float u = unif24(draw_word(seed, sid, nn + i, STREAM_ACCEPT, it));
      const float uq = __fmul_rn(u, qy);
      fail = !(uq < py);
    }
  }
  const uint64_t m = __ballot(fail);
  const int k = m ? (__ffsll((unsigned long long)m) - 1) + 2 : B + 1;
  if (lane == 0) {
    k_out[s] = k;
    RowDesc d;
    d.pad = 0;
    d.out = z_out + s;
    if (k <= B) {
      d.a = p + ((size_t)s * B + (k - 2)) * V;
      d.b = q + ((size_t)s * q_stride + (k - 2)) * V;
      d.mode = 1;
    } else {
      d.a = p + ((size_t)s * B + (B - 1)) * V;
      d.b = nullptr;
      d.mode = 0;
    }
    d.word = draw_word(seed, sid, nn + k, STREAM_RESAMPLE, it);
    desc[s] = d;
  }
}

// Emit y_1..y_{k-1}, z; advance the sequence state (when state pointers are given).
__global__ void k_accept_commit(int B, const int32_t* draft, const int32_t* k_in,
                                const int32_t* z, const int32_t* call_seq, int32_t* out,
                                int32_t* n_out, int32_t* len, int32_t* pending, int32_t* iter) {
  const int s = blockIdx.x, t = threadIdx.x;
  const int k = k_in[s];
  if (t <= B) {
    int v = -1;
    if (t < k - 1) v = draft[(size_t)s * B + t];
    else if (t == k - 1) v = z[s];
    if (out) out[(size_t)s * (B + 1) + t] = v;
  }
  if (t == 0) {
    if (n_out) n_out[s] = k;
    if (len) {
      const int sid = call_seq[s];
      len[sid] += k;
      pending[sid] = z[s];
      iter[sid] += 1;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-p (nucleus) truncation of probability rows, in place or out of place: one
// workgroup of 1024 threads per row.  The evaluations of the pages sample with
// top-p 0.95 and losslessness holds for that filtered law ([blog] "我的判断");
// the same truncation is applied to the AR and the draft laws.  Made exact so
// that it is reproducible bit for bit: masses are floor(p * 2^40) in int64 (exact
// and order-free sums), the target is max(1, ceil(top_p * W)) in double, the
// threshold is the largest value whose upper set {p >= tau} holds the target,
// and kept values are divided by float(W_kept * 2^-40).  top_p >= 1, or a row
// without fixed-point mass, is copied unchanged.
//
// The threshold comes from a radix descent over the bit pattern, which orders
// like the value for p > 0: three passes over bits 30..20, 19..9 and 8..0 (2048,
// 2048 and 512 bins of int64 mass in LDS, two copies split by wave parity).  The
// first histogram holds every positive entry, so its sum is W; the last pass
// yields the mass at or above tau, W_kept.  The row is read four times (three
// histograms and the output pass) and written once; fine bins keep the LDS
// atomics of neighbouring lanes on different addresses for most rows.
constexpr int TP_THREADS = 1024, TP_WAVES = TP_THREADS / 64;
constexpr int TP_BINS = 2048, TP_COPIES = 2;

UNO_DEV long long tp_mass(float p) {
  return p > 0.0f ? (long long)floor((double)p * 0x1p40) : 0;
}

// f(index, value) over the row, with 16-byte loads when the row allows them
template <class F>
UNO_DEV void tp_each(const float* p, int V, F&& f) {
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    const float4* p4 = reinterpret_cast<const float4*>(p);
    for (int i = threadIdx.x; i < (V >> 2); i += TP_THREADS) {
      const float4 v = p4[i];
      f(4 * i, v.x);
      f(4 * i + 1, v.y);
      f(4 * i + 2, v.z);
      f(4 * i + 3, v.w);
    }
  } else {
    for (int i = threadIdx.x; i < V; i += TP_THREADS) f(i, p[i]);
  }
}

// Sum of v over the threads >= threadIdx.x (a suffix over the workgroup);
// *total receives the sum over all threads.
UNO_DEV long long tp_block_suffix(long long v, long long* red, long long* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = __shfl_down(v, d);
    if (lane + d < 64) v += y;
  }
  __syncthreads();                        // the previous use of red[] is over
  if (lane == 0) red[w] = v;              // lane 0 holds the wave's total
  __syncthreads();
  long long hi = 0, all = 0;
#pragma unroll
  for (int i = 0; i < TP_WAVES; ++i) {
    const long long t = red[i];
    all += t;
    if (i > w) hi += t;
  }
  *total = all;
  return v + hi;
}

__global__ void __launch_bounds__(TP_THREADS)
k_top_p(const float* in, float* out, int V, float top_p) {
  __shared__ long long hist[TP_COPIES][TP_BINS];
  __shared__ long long red[TP_WAVES];
  __shared__ unsigned s_prefix;
  __shared__ long long s_above, s_kept;
  const float* p = in + (size_t)blockIdx.x * V;
  float* o = out + (size_t)blockIdx.x * V;
  const int tid = threadIdx.x;
  long long* h = hist[(tid >> 6) & (TP_COPIES - 1)];
  auto copy_row = [&] { tp_each(p, V, [&](int i, float v) { o[i] = v; }); };
  if (top_p >= 1.0f) {
    copy_row();
    return;
  }

  unsigned prefix = 0, mask = 0;
  long long above = 0, target = 0, kept = 0;   // above: mass strictly above the prefix group
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : pass == 1 ? 9 : 0;
    const unsigned nb = pass == 2 ? 512u : 2048u;
    for (int b = tid; b < TP_COPIES * TP_BINS; b += TP_THREADS) (&hist[0][0])[b] = 0;
    __syncthreads();
    tp_each(p, V, [&](int, float v) {
      const unsigned bits = __float_as_uint(v);
      if (v > 0.0f && (bits & mask) == prefix)
        atomicAdd(reinterpret_cast<unsigned long long*>(&h[(bits >> shift) & (nb - 1)]),
                  (unsigned long long)tp_mass(v));
    });
    __syncthreads();
    // this thread's bins 2t and 2t+1, summed over the copies (bins >= nb are empty)
    long long h0 = 0, h1 = 0;
#pragma unroll
    for (int c = 0; c < TP_COPIES; ++c) {
      h0 += hist[c][2 * tid];
      h1 += hist[c][2 * tid + 1];
    }
    long long total;
    const long long s0 = tp_block_suffix(h0 + h1, red, &total);   // mass of bins >= 2t
    if (pass == 0) {
      if (total == 0) {                    // W == 0: the same in every thread
        copy_row();
        return;
      }
      target = (long long)ceil((double)top_p * (double)total);
      if (target < 1) target = 1;
    }
    const long long s1 = s0 - h0;          // bins >= 2t+1
    const long long s2 = s1 - h1;          // bins >= 2t+2
    // the one bin where the running mass from the top first reaches the target
    if (above + s0 >= target && above + s1 < target) {
      s_prefix = prefix | ((2u * tid) << shift);
      s_above = above + s1;
      s_kept = above + s0;
    } else if (above + s1 >= target && above + s2 < target) {
      s_prefix = prefix | ((2u * tid + 1) << shift);
      s_above = above + s2;
      s_kept = above + s1;
    }
    __syncthreads();
    prefix = s_prefix;
    above = s_above;
    kept = s_kept;
    mask |= (nb - 1) << shift;
    __syncthreads();                       // s_* and hist are rewritten by the next pass
  }

  // prefix is now tau's bit pattern and kept the mass of {p >= tau}
  const float z = (float)((double)kept * 0x1p-40);
  tp_each(p, V, [&](int i, float v) {
    o[i] = (v > 0.0f && __float_as_uint(v) >= prefix) ? v / z : 0.0f;
  });
}

}  // namespace

hipError_t launch_top_p(const float* in, float* out, int rows, int V, float top_p, hipStream_t s) {
  if (rows <= 0 || V <= 0) return hipSuccess;
  uno_launch(k_top_p, rows, TP_THREADS, 0, s, in, out, V, top_p);
  return hipGetLastError();
}


hipError_t launch_cdf(const RowDesc* desc, int rows, int V, uint64_t* chunk_tot, int32_t* err,
                      hipStream_t s) {
  const int n_chunks = (V + CDF_CHUNK - 1) / CDF_CHUNK;
  if (rows <= 0) return hipSuccess;
  if (n_chunks > 1024) return hipErrorInvalidValue;
  uno_launch(k_cdf_chunks, dim3(n_chunks, rows), CDF_THREADS, 0, s, desc, V, n_chunks, chunk_tot, err);
  uno_launch(k_cdf_select, rows, CDF_THREADS, 0, s, desc, V, n_chunks, chunk_tot, err);
  return hipGetLastError();
}

hipError_t launch_draft_desc(const float* probs, int n, int B, int V, uint64_t seed,
                             const int32_t* call_seq, const int32_t* call_n,
                             const int32_t* call_it, int32_t* out_tok, RowDesc* desc,
                             hipStream_t s) {
  const int rows = n * B;
  uno_launch(k_draft_desc, (rows + 127) / 128, 128, 0, s, probs, n, B, V, seed, call_seq, call_n,
                                                  call_it, out_tok, desc);
  return hipGetLastError();
}

hipError_t launch_sample_desc(const float* w, int rows, int V, uint64_t seed,
                              const int32_t* seq_ids, const int32_t* pos, const int32_t* it,
                              int stream_id, int32_t* out, RowDesc* desc, hipStream_t s) {
  uno_launch(k_sample_desc, (rows + 127) / 128, 128, 0, s, w, rows, V, seed, seq_ids, pos, it,
                                                   stream_id, out, desc);
  return hipGetLastError();
}

hipError_t launch_accept_test(uint64_t seed, int n, int B, int V, const float* p,
                              const float* q, int q_stride, const int32_t* draft,
                              const int32_t* call_seq, const int32_t* call_n,
                              const int32_t* call_it, int32_t* k_out, int32_t* z_out,
                              RowDesc* desc, int32_t* err, hipStream_t s) {
  if (B > 65) return hipErrorInvalidValue;
  uno_launch(k_accept_test, n, 64, 0, s, seed, B, V, p, q, q_stride, draft, call_seq, call_n, call_it,
                                 k_out, z_out, desc, err);
  return hipGetLastError();
}

hipError_t launch_accept_commit(int n, int B, const int32_t* draft, const int32_t* k,
                                const int32_t* z, const int32_t* call_seq, int32_t* out,
                                int32_t* n_out, int32_t* len, int32_t* pending, int32_t* iter,
                                hipStream_t s) {
  const int threads = ((B + 1 + 63) / 64) * 64;
  uno_launch(k_accept_commit, n, threads, 0, s, B, draft, k, z, call_seq, out, n_out, len, pending,
                                        iter);
  return hipGetLastError();
}
