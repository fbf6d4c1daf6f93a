// Block-causal attention over the paged KV cache shared by draft and verify.
//
// Method: draft and verify read one KV cache (shibing624 reading notes of the Uno
// paper, method core); a row at position m attends to its sequence's committed
// context plus the in-flight block up to itself, i.e. positions 0..m, because
// every block row's K/V is written at its position before attention runs.
//
// Split-context decomposition: a workgroup owns (sequence, KV head, 16-row tile,
// context chunk); the G = Hq / Hkv query heads of its KV head and the 16 rows
// share each K/V load.  The chunk is walked in 32-key sub-chunks with an online
// softmax; the partial (max, sum, unnormalised output) of every chunk is merged
// by a second kernel in chunk order (deterministic).
#include "uno_internal.h"

namespace {

constexpr int SUB = 32;   // keys per LDS sub-chunk

template <typename T, int MAXO>
__global__ void __launch_bounds__(256)
k_attn_partial(AttnArgs a, KvLayout kv) {
  extern __shared__ float smem[];
  const int c = blockIdx.x, kvh = blockIdx.y;
  const int row_tiles = (a.rows_per_seq + 15) / 16;
  const int si = blockIdx.z / row_tiles, rt = blockIdx.z % row_tiles;
  const int Hkv = kv.n_kv_heads, hd = kv.head_dim, G = a.n_q_heads / Hkv;
  const int seq = a.call_seq[si];
  const int r0 = si * a.rows_per_seq + rt * 16;
  const int nrows = min(16, a.rows_per_seq - rt * 16);
  const int NQ = 16 * G;               // query vectors of this block
  const int kstride = hd + 2;          // padded LDS row (in T elements)

  float* sQ = smem;                                  // [NQ][hd]
  float* sS = sQ + NQ * hd;                          // [NQ][SUB]
  float* sM = sS + NQ * SUB;                         // [NQ] running max
  float* sL = sM + NQ;                               // [NQ] running sum
  float* sF = sL + NQ;                               // [NQ] rescale factor
  int* sPos = reinterpret_cast<int*>(sF + NQ);       // [16]
  T* sK = reinterpret_cast<T*>(sPos + 16);           // [SUB][kstride]
  T* sV = sK + SUB * kstride;                        // [SUB][kstride]

  const int tid = threadIdx.x;
  if (tid < 16) sPos[tid] = (tid < nrows) ? a.row_pos[r0 + tid] : -1;
  __syncthreads();
  int maxpos = -1;
  for (int i = 0; i < nrows; ++i) maxpos = max(maxpos, sPos[i]);
  const int kbeg = c * a.chunk;
  if (kbeg > maxpos) return;           // no row sees this chunk (never combined)
  const int kend = min(kbeg + a.chunk, maxpos + 1);

  // queries: qi = g * 16 + row, head = kvh * G + g
  const T* Q = reinterpret_cast<const T*>(a.q);
  for (int e = tid; e < NQ * hd; e += 256) {
    const int qi = e / hd, d = e % hd, g = qi / 16, row = qi % 16;
    sQ[e] = (row < nrows) ? to_f(Q[(size_t)(r0 + row) * a.n_q_heads * hd + (kvh * G + g) * hd + d])
                          : 0.0f;
  }
  for (int qi = tid; qi < NQ; qi += 256) { sM[qi] = -INFINITY; sL[qi] = 0.0f; }

  // output accumulators: element e = tid + 256 * i of [NQ][hd]
  float o[MAXO];                       // NQ * hd <= 256 * MAXO
  const int nown = (NQ * hd + 255) / 256;
#pragma unroll
  for (int i = 0; i < MAXO; ++i) o[i] = 0.0f;

  const T* Kp = reinterpret_cast<const T*>(kv.pool);
  for (int k0 = kbeg; k0 < kend; k0 += SUB) {
    __syncthreads();
    // load K / V of positions k0 .. k0+SUB-1 (only positions < kend are read)
    for (int e = tid; e < SUB * hd; e += 256) {
      const int j = e / hd, d = e % hd, p = k0 + j;
      T kvk = from_f<T>(0.0f), kvv = from_f<T>(0.0f);
      const int page = (p < kend && p / kv.page_size < kv.max_pages_per_seq)
                           ? kv.block_table[(size_t)seq * kv.max_pages_per_seq + p / kv.page_size]
                           : -1;
      if (page >= 0 && page < kv.n_pages) {
        const size_t base =
            (((size_t)(a.layer * 2) * kv.n_pages + page) * Hkv + kvh) * kv.page_size +
            (p % kv.page_size);
        const size_t vbase =
            (((size_t)(a.layer * 2 + 1) * kv.n_pages + page) * Hkv + kvh) * kv.page_size +
            (p % kv.page_size);
        kvk = Kp[base * hd + d];
        kvv = Kp[vbase * hd + d];
      }
      sK[j * kstride + d] = kvk;
      sV[j * kstride + d] = kvv;
    }
    __syncthreads();
    // scores
    for (int e = tid; e < NQ * SUB; e += 256) {
      const int qi = e / SUB, j = e % SUB, p = k0 + j;
      const int rpos = sPos[qi % 16];
      float s = -INFINITY;
      if (p < kend && p <= rpos) {
        const float* q = sQ + qi * hd;
        const T* kr = sK + j * kstride;
        float acc = 0.0f;
        for (int d = 0; d < hd; ++d) acc += q[d] * to_f(kr[d]);
        s = acc * a.scale;
      }
      sS[e] = s;
    }
    __syncthreads();
    // online softmax update per query
    for (int qi = tid; qi < NQ; qi += 256) {
      float mx = sM[qi];
      for (int j = 0; j < SUB; ++j) mx = fmaxf(mx, sS[qi * SUB + j]);
      float f = 1.0f, l = sL[qi];
      if (mx == -INFINITY) {
        for (int j = 0; j < SUB; ++j) sS[qi * SUB + j] = 0.0f;
      } else {
        f = (sM[qi] == -INFINITY) ? 0.0f : expf(sM[qi] - mx);
        l *= f;
        for (int j = 0; j < SUB; ++j) {
          const float pj = expf(sS[qi * SUB + j] - mx);   // exp(-inf) = 0 for masked keys
          sS[qi * SUB + j] = pj;
          l += pj;
        }
        sM[qi] = mx;
      }
      sL[qi] = l;
      sF[qi] = f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXO; ++i) {
      const int e = tid + 256 * i;
      if (i < nown && e < NQ * hd) {
        const int qi = e / hd, d = e % hd;
        float acc = o[i] * sF[qi];
        const float* pr = sS + qi * SUB;
        for (int j = 0; j < SUB; ++j) acc += pr[j] * to_f(sV[j * kstride + d]);
        o[i] = acc;
      }
    }
  }
  // write partials of the valid rows
#pragma unroll
  for (int i = 0; i < MAXO; ++i) {
    const int e = tid + 256 * i;
    if (i < nown && e < NQ * hd) {
      const int qi = e / hd, d = e % hd, g = qi / 16, row = qi % 16;
      if (row < nrows) {
        const size_t ph = ((size_t)(r0 + row) * a.n_q_heads + kvh * G + g) * a.n_chunks + c;
        a.part_o[ph * hd + d] = o[i];
        if (d == 0) {
          a.part_ml[ph * 2] = sM[qi];
          a.part_ml[ph * 2 + 1] = sL[qi];
        }
      }
    }
  }
}

// Merge the chunk partials of one (row, head) in chunk order.
template <typename T>
__global__ void k_attn_combine(AttnArgs a, int hd) {
  const int r = blockIdx.x / a.n_q_heads, h = blockIdx.x % a.n_q_heads;
  const int nc = min(a.row_pos[r] / a.chunk + 1, a.n_chunks);
  const size_t ph0 = ((size_t)r * a.n_q_heads + h) * a.n_chunks;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, a.part_ml[(ph0 + c) * 2]);
  for (int d = threadIdx.x; d < hd; d += blockDim.x) {
    float L = 0.0f, acc = 0.0f;
    for (int c = 0; c < nc; ++c) {
      const float mc = a.part_ml[(ph0 + c) * 2];
      if (mc == -INFINITY) continue;
      const float f = expf(mc - M);
      L += a.part_ml[(ph0 + c) * 2 + 1] * f;
      acc += a.part_o[(ph0 + c) * hd + d] * f;
    }
    reinterpret_cast<T*>(a.out)[(size_t)r * a.n_q_heads * hd + h * hd + d] =
        from_f<T>(L > 0.0f ? acc / L : 0.0f);
  }
}

}  // namespace

template <typename T>
size_t attn_smem_bytes(int G, int hd) {
  const int NQ = 16 * G;
  return (size_t)(NQ * hd + NQ * SUB + 3 * NQ + 16) * 4 + (size_t)2 * SUB * (hd + 2) * sizeof(T);
}

template <typename T>
hipError_t launch_attention(const AttnArgs& a, const KvLayout& kv, hipStream_t s) {
  const int G = a.n_q_heads / kv.n_kv_heads;
  if (16 * G * kv.head_dim > 256 * 64 || a.chunk % SUB != 0) return hipErrorInvalidValue;
  const int R = a.n * a.rows_per_seq;
  if (R <= 0) return hipSuccess;
  const size_t smem = attn_smem_bytes<T>(G, kv.head_dim);
  const int nown = (16 * G * kv.head_dim + 255) / 256;
  const int row_tiles = (a.rows_per_seq + 15) / 16;
  dim3 grid(a.n_chunks, kv.n_kv_heads, a.n * row_tiles);
#define UNO_ATTN_CASE(MO)                                                                   \
  if (nown <= MO) {                                                                         \
    static bool set = false;                                                                \
    if (!set) {                                                                             \
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_partial<T, MO>),      \
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);          \
      set = true;                                                                           \
    }                                                                                       \
    k_attn_partial<T, MO><<<grid, 256, smem, s>>>(a, kv);                                   \
  } else
  UNO_ATTN_CASE(1) UNO_ATTN_CASE(4) UNO_ATTN_CASE(16) UNO_ATTN_CASE(32) UNO_ATTN_CASE(64)
  return hipErrorInvalidValue;
#undef UNO_ATTN_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_attn_combine<T><<<R * a.n_q_heads, kv.head_dim < 256 ? kv.head_dim : 256, 0, s>>>(
      a, kv.head_dim);
  return hipGetLastError();
}

template hipError_t launch_attention<float>(const AttnArgs&, const KvLayout&, hipStream_t);
template hipError_t launch_attention<bf16>(const AttnArgs&, const KvLayout&, hipStream_t);
template size_t attn_smem_bytes<float>(int, int);
template size_t attn_smem_bytes<bf16>(int, int);
