// Tree sampler kernels: the K-chain draft draws, the acceptance walk with
// recursive rejection sampling, and the K/V move of an accepted side chain.
//
// Method: the Psi-Spec sampler has a tree mode for single-request throughput
// (ai-papers-daily summary, method key points; shibing624 reading notes, section
// on the Psi-Spec sampler, which also fixes that rejection keeps the output law
// the AR model's).  The candidate-set construction did not survive on the pages;
// the reading used here: the chains share the first token and draw depths 2..B
// independently from the one draft forward's laws; the live chains at a depth
// (those matching the accepted path) are tried in chain order against a running
// residual, so the emitted token follows the AR law for any number of candidates.
//
// Exactness: trial 0 is the linear sampler's float32 test; later trials compare
// (u * q(c)) * T < R(c) in float64 (each product rounded once, no contraction)
// against integer residual masses R on the 2^-40 grid, whose sums are exact in any
// order, so every decision and draw is reproducible bit for bit.
#include "uno_tree.h"

namespace {

constexpr int TREE_THREADS = 1024;

__global__ void k_tree_draft_desc(const float* probs, int n, int K, int B, int V, uint64_t seed,
                                  const int32_t* call_seq, const int32_t* call_n,
                                  const int32_t* call_it, int32_t* chains, RowDesc* desc) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n * K * B) return;
  const int s = r / (K * B), k = (r / B) % K, d = r % B + 1;
  RowDesc x;
  x.a = probs + ((size_t)s * B + (d - 1)) * V;
  x.b = nullptr;
  x.mode = 0;
  x.pad = 0;
  x.word = draw_word(seed, call_seq[s], call_n[s] + d, STREAM_DRAFT, call_it[s], d == 1 ? 0 : k);
  x.out = chains + r;
  desc[r] = x;
}

// Sum over the workgroup; every thread receives the total.
__device__ uint64_t block_sum_u64(uint64_t v, uint64_t* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    v += (uint64_t)__shfl_xor((unsigned long long)v, off);
  __syncthreads();                       // the previous call's readers are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t t = 0;
  for (int i = 0; i < TREE_THREADS / 64; ++i) t += red[i];
  return t;
}

// The passes over the vocabulary take four entries per thread and step (16-byte
// loads of p and q, two 16-byte stores of R; the vocabulary is a multiple of 16)
// and keep several steps' loads in flight: one workgroup streams the rows.
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));

// R_1 = trunc(max(0, p - q) * 2^40), or trunc(p * 2^40) when that has no mass;
// returns its sum.
__device__ uint64_t resid_first(const float* p, const float* q, uint64_t* R, int V,
                                uint64_t* red, int32_t* err) {
  const f4_t* p4 = reinterpret_cast<const f4_t*>(p);
  const f4_t* q4 = reinterpret_cast<const f4_t*>(q);
  u64x2_t* R2 = reinterpret_cast<u64x2_t*>(R);
  uint64_t sum = 0;
#pragma unroll 4
  for (int x = threadIdx.x; x < V / 4; x += TREE_THREADS) {
    const f4_t pv = p4[x], qv = q4[x];
    uint64_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = int_weight(fmaxf(pv[e] - qv[e], 0.0f), err);
      sum += w[e];
    }
    R2[2 * x] = u64x2_t{w[0], w[1]};
    R2[2 * x + 1] = u64x2_t{w[2], w[3]};
  }
  uint64_t T = block_sum_u64(sum, red);
  if (T == 0) {
    sum = 0;
#pragma unroll 4
    for (int x = threadIdx.x; x < V / 4; x += TREE_THREADS) {
      const f4_t pv = p4[x];
      uint64_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = int_weight(pv[e], err);
        sum += w[e];
      }
      R2[2 * x] = u64x2_t{w[0], w[1]};
      R2[2 * x + 1] = u64x2_t{w[2], w[3]};
    }
    T = block_sum_u64(sum, red);
  }
  __syncthreads();                       // R visible to the deciding thread
  return T;
}

// One entry of R_{j+1} = R_j - min(R_j, floor(T_j * Q / 2^40)), Q = trunc(q * 2^40)
// (T_j < 2^58 and Q <= 2^40, so the 128-bit product shifted down fits 64 bits).
__device__ uint64_t resid_entry(uint64_t r, float qv, uint64_t T) {
  const uint64_t Qx = int_weight(qv, nullptr);
  const uint64_t sub = (__umul64hi(T, Qx) << 24) | ((T * Qx) >> 40);
  return r - (r < sub ? r : sub);
}

// R_{j+1} in place (R_j kept when the update leaves no mass); returns its sum.
__device__ uint64_t resid_next(const float* q, uint64_t* R, int V, uint64_t T, uint64_t* red) {
  const f4_t* q4 = reinterpret_cast<const f4_t*>(q);
  u64x2_t* R2 = reinterpret_cast<u64x2_t*>(R);
  uint64_t sum = 0;
#pragma unroll 4
  for (int x = threadIdx.x; x < V / 4; x += TREE_THREADS) {
    const f4_t qv = q4[x];
    const u64x2_t r0 = R2[2 * x], r1 = R2[2 * x + 1];
    sum += resid_entry(r0.x, qv[0], T) + resid_entry(r0.y, qv[1], T) +
           resid_entry(r1.x, qv[2], T) + resid_entry(r1.y, qv[3], T);
  }
  const uint64_t T2 = block_sum_u64(sum, red);
  if (T2 == 0) return T;
#pragma unroll 4
  for (int x = threadIdx.x; x < V / 4; x += TREE_THREADS) {
    const f4_t qv = q4[x];
    const u64x2_t r0 = R2[2 * x], r1 = R2[2 * x + 1];
    R2[2 * x] = u64x2_t{resid_entry(r0.x, qv[0], T), resid_entry(r0.y, qv[1], T)};
    R2[2 * x + 1] = u64x2_t{resid_entry(r1.x, qv[2], T), resid_entry(r1.y, qv[3], T)};
  }
  __syncthreads();
  return T2;
}

__global__ void __launch_bounds__(TREE_THREADS) k_tree_accept(TreeAcceptArgs a) {
  __shared__ int s_live[TREE_KMAX];
  __shared__ int s_nlive, s_ok, s_c;
  __shared__ uint64_t s_red[TREE_THREADS / 64];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int K = a.K, B = a.B, V = a.V;
  const int sid = a.seq_ids[s], nn = a.pos[s], it = a.iter[s];
  const float* P = a.p + (size_t)s * a.p_rows * V;
  const float* Q = a.q + (size_t)s * a.q_rows * V;
  const int32_t* ch = a.chains + (size_t)s * K * B;
  uint64_t* R = a.resid + (size_t)s * V;
  int32_t* path = a.path + (size_t)s * B;
  if (tid == 0) {
    for (int k = 0; k < K; ++k) s_live[k] = k;
    s_nlive = K;
    path[0] = ch[0];
  }
  __syncthreads();
  int stop = B + 1;
  int state = 0;                         // correction row: 1 linear residual, 2 R
  const float* prow = P;
  const float* qrow = Q;
  uint64_t T = 0;
  for (int d = 2; d <= B; ++d) {
    const int nl = s_nlive;
    prow = P + (size_t)tree_row(s_live[0], d - 1, B) * V;
    qrow = Q + (size_t)(d - 1) * V;
    int acc = -1;
    state = 0;
    for (int j = 0; j < nl; ++j) {
      if (tid == 0) {
        const int c = ch[s_live[j] * B + d - 1];
        bool ok = false;
        if (c < 0 || c >= V) {
          if (a.err) atomicOr(a.err, UNO_DEVERR_NUMERIC);
        } else {
          const float qy = qrow[c], py = prow[c];
          if (!(qy >= 0.0f && qy <= 1.0f) || !(py >= 0.0f && py <= 1.0f))
            if (a.err) atomicOr(a.err, UNO_DEVERR_NUMERIC);
          const float u = unif24(draw_word(a.seed, sid, nn + d, STREAM_ACCEPT, it, j));
          if (j == 0) ok = __fmul_rn(u, qy) < py;
          else ok = __dmul_rn(__dmul_rn((double)u, (double)qy), (double)T) < (double)R[c];
        }
        s_ok = ok ? 1 : 0;
        s_c = c;
      }
      __syncthreads();
      if (s_ok) {
        acc = s_c;
        break;
      }
      if (j == 0 && nl == 1) {             // the linear sampler's residual row
        state = 1;
        break;
      }
      T = j == 0 ? resid_first(prow, qrow, R, V, s_red, a.err) : resid_next(qrow, R, V, T, s_red);
      state = 2;
    }
    if (acc < 0) {
      stop = d;
      break;
    }
    __syncthreads();                       // every thread has read s_ok / s_c
    if (tid == 0) {
      path[d - 1] = acc;
      int m = 0;
      for (int i = 0; i < nl; ++i)
        if (ch[s_live[i] * B + d - 1] == acc) s_live[m++] = s_live[i];
      s_nlive = m;
    }
    __syncthreads();
  }
  if (tid == 0) {
    RowDesc x;
    x.pad = 0;
    x.out = a.z + s;
    if (stop == B + 1) {
      x.a = P + (size_t)tree_row(s_live[0], B, B) * V;
      x.b = nullptr;
      x.mode = 0;
    } else if (state == 1) {
      x.a = prow;
      x.b = qrow;
      x.mode = 1;
    } else {
      x.a = reinterpret_cast<const float*>(R);
      x.b = nullptr;
      x.mode = 2;
    }
    x.word = draw_word(a.seed, sid, nn + stop, STREAM_RESAMPLE, it);
    a.desc[s] = x;
    a.k_out[s] = stop;
    a.kstar[s] = s_live[0];
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
k_tree_kv_move(KvLayout kv, int B, const int32_t* call_seq, const int32_t* call_n,
               const int32_t* k_out, const int32_t* kstar, int32_t* err) {
  const int s = blockIdx.x;
  const int k = k_out[s], ks = kstar[s];
  if (ks <= 0 || k < 3) return;
  const int Hkv = kv.n_kv_heads, hd = kv.head_dim, ps = kv.page_size;
  const int l = blockIdx.y / (2 * Hkv), which = (blockIdx.y / Hkv) % 2, h = blockIdx.y % Hkv;
  const int nn = call_n[s], seq = call_seq[s];
  const int m = k - 2, base = nn + 2 + ks * (B - 1);
  for (int e = threadIdx.x; e < m * hd; e += 256) {
    const int t = e / hd, dim = e % hd;
    const int src = base + t, dst = nn + 2 + t;
    const int ps_src = kv_page(kv, seq, src), ps_dst = kv_page(kv, seq, dst);
    if (ps_src < 0 || ps_dst < 0) {
      if (err) atomicOr(err, UNO_DEVERR_BOUNDS);
      continue;
    }
    const T* sp = kv_block<const T>(kv, l, which, ps_src, h);
    T* dp = kv_block<T>(kv, l, which, ps_dst, h);
    dp[kv_elem(kv, which, dst % ps, dim)] = sp[kv_elem(kv, which, src % ps, dim)];
  }
}

}  // namespace

hipError_t launch_tree_draft_desc(const float* probs, int n, int K, int B, int V, uint64_t seed,
                                  const int32_t* call_seq, const int32_t* call_n,
                                  const int32_t* call_it, int32_t* chains, RowDesc* desc,
                                  hipStream_t s) {
  const int rows = n * K * B;
  if (rows <= 0) return hipSuccess;
  uno_launch(k_tree_draft_desc, (rows + 127) / 128, 128, 0, s, probs, n, K, B, V, seed, call_seq,
             call_n, call_it, chains, desc);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const TreeAcceptArgs& a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (a.K < 1 || a.K > TREE_KMAX || a.B < 1 || a.p_rows < 1 + a.K * (a.B - 1) || a.q_rows < a.B ||
      a.V % 4 != 0)
    return hipErrorInvalidValue;
  uno_launch(k_tree_accept, n, TREE_THREADS, 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_tree_kv_move(const KvLayout& kv, int n, int B, int n_layers,
                               const int32_t* call_seq, const int32_t* call_n,
                               const int32_t* k_out, const int32_t* kstar, int32_t* err,
                               hipStream_t s) {
  if (n <= 0 || B < 2) return hipSuccess;       // B = 1: no drafted depth to move
  uno_launch(k_tree_kv_move<T>, dim3(n, n_layers * 2 * kv.n_kv_heads), 256, 0, s, kv, B, call_seq,
             call_n, k_out, kstar, err);
  return hipGetLastError();
}
template hipError_t launch_tree_kv_move<float>(const KvLayout&, int, int, int, const int32_t*,
                                               const int32_t*, const int32_t*, const int32_t*,
                                               int32_t*, hipStream_t);
template hipError_t launch_tree_kv_move<bf16>(const KvLayout&, int, int, int, const int32_t*,
                                              const int32_t*, const int32_t*, const int32_t*,
                                              int32_t*, hipStream_t);
