// Gated-LoRA linear: y = rs * (xg W^T) + (gate * bf16((alpha/r) t)) B^T with fused
// epilogues (q|k|v with RoPE and the paged K/V write, residual add that also
// produces the next RMSNorm input, SwiGLU, LM-head logits with per-tile softmax
// statistics, plain store, and the LoRA intermediate of the float32 path).
//
// Method: the diffusion weights are a LoRA on every projection, switched off on
// clean rows and on on noisy rows inside one forward (shibing624 reading notes of
// the Uno paper, "Diffusion Distillation" section; ai-papers-daily summary,
// method key points).  The gate multiplies the LoRA intermediate, so a gate-off
// row adds exact zeros, and a verify forward has no LoRA phase at all.
//
// RMSNorm is folded in: the producer of x (embedding or residual epilogue)
// stores xg = x * g of the next norm and adds x^2 to a fixed-point per-row sum;
// the consumer multiplies its base accumulator by rs = 1 / rms(x).
//
// bf16 kernel (gfx950): one workgroup owns a 16-row x (16*NT)-column output
// tile; its WAVES wavefronts split K and stream their slice of the weight rows
// straight from HBM into MFMA B-fragments (weights are [out, in], so a lane's 8
// consecutive k values are 16 contiguous bytes) against A-fragments of the
// activations (L2-resident), on v_mfma_f32_16x16x32_bf16.  Wave partials are
// summed in LDS in a fixed wave order (bit-reproducible).  The LoRA up-projection
// is a second K-phase over the rank with A = the gated intermediate.
#include "uno_internal.h"

#include <algorithm>

namespace {

UNO_DEV bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

UNO_DEV float rs_of(const GemmArgs& a, int m) {
  if (!a.ss_in || m >= a.M) return 1.0f;
  const float ms = (float)((double)a.ss_in[m] * LORA_FX_INV) * a.inv_d;
  return 1.0f / sqrtf(ms + a.eps);
}

// Column of output tile `tile` owned by lane column c.  The q|k|v projection uses
// a pair-permuted order: the 16 columns of a tile are 8 from the first half of a
// head and the 8 matching ones (+hd/2) from the second half, so each RoPE pair
// sits in one tile.
UNO_DEV int tile_col(const GemmArgs& a, int tile, int c) {
  if (a.epi != EPI_QKV) return tile * 16 + c;
  const int hd = a.kv.head_dim, tph = hd / 16;
  const int head = tile / tph, j = tile % tph;
  return head * hd + ((c < 8) ? 8 * j + c : hd / 2 + 8 * j + (c - 8));
}

UNO_DEV int find_seg(const GemmArgs& a, int col) {
  int s = 0;
  for (int i = 1; i < a.nseg; ++i)
    if (col >= a.seg[i].n0) s = i;
  return s;
}

template <typename T>
UNO_DEV T* kv_dst(const KvLayout& kv, int layer, int which, int seq, int pos, int h,
                  int32_t* err) {
  const int pi = pos / kv.page_size;
  const int page = (pos >= 0 && pi < kv.max_pages_per_seq)
                       ? kv.block_table[(size_t)seq * kv.max_pages_per_seq + pi] : -1;
  if (page < 0 || page >= kv.n_pages) {
    if (err) atomicOr(err, UNO_DEVERR_BOUNDS);
    return nullptr;
  }
  return reinterpret_cast<T*>(kv.pool) +
         ((((size_t)(layer * 2 + which) * kv.n_pages + page) * kv.n_kv_heads + h) *
              kv.page_size + (pos % kv.page_size)) * kv.head_dim;
}

// Epilogue of one element (row m, lane column c) of each of the NT tiles.  `finr`
// holds the 16 finished values of this row in tile 0 (the RoPE partner is
// finr[c ^ 8]).  Every thread of a 16-lane row group calls this (row sums use
// shuffles); `ok` says whether row m exists.
template <typename T, int NT>
UNO_DEV void epilogue(const GemmArgs& a, int m, int c, int tile0, int col_paired,
                      const float* v, const float* finr, bool ok) {
  switch (a.epi) {
    case EPI_STORE_F32:
      if (ok)
        for (int t = 0; t < NT; ++t)
          reinterpret_cast<float*>(a.out)[(size_t)m * a.ldo + (tile0 + t) * 16 + c] = v[t];
      break;
    case EPI_LORA_U: {
      if (!ok) break;
      const bool on = a.gate == nullptr || a.gate[m] != 0;
      for (int t = 0; t < NT; ++t)
        reinterpret_cast<T*>(a.out)[(size_t)m * a.ldo + (tile0 + t) * 16 + c] =
            from_f<T>(on ? a.scale * v[t] : 0.0f);
      break;
    }
    case EPI_RESID: {
      float sq = 0.0f;
      for (int t = 0; t < NT; ++t) {
        const int col = (tile0 + t) * 16 + c;
        if (ok) {
          const float xn = a.resid[(size_t)m * a.ldo + col] + v[t];
          a.resid[(size_t)m * a.ldo + col] = xn;
          if (a.xg_out)
            reinterpret_cast<T*>(a.xg_out)[(size_t)m * a.ldo + col] =
                from_f<T>(xn * to_f(reinterpret_cast<const T*>(a.g_next)[col]));
          sq += xn * xn;
        }
      }
      if (a.ss_out) {
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 16);
        if (ok && c == 0)
          atomicAdd(reinterpret_cast<unsigned long long*>(a.ss_out + m),
                    (unsigned long long)(long long)llrintf(sq * LORA_FX_SCALE));
      }
      break;
    }
    case EPI_SWIGLU: {
      if (!ok) break;
      const float g = v[0], u = v[1];
      reinterpret_cast<T*>(a.out)[(size_t)m * a.ldo + col_paired + c] =
          from_f<T>(g / (1.0f + expf(-g)) * u);
      break;
    }
    case EPI_QKV: {
      if (!ok) break;
      const int hd = a.kv.head_dim, half = hd / 2, tph = hd / 16;
      const int head = tile0 / tph, j = tile0 % tph;
      const int i = 8 * j + (c & 7);                 // pair index within the head
      const int dim = (c < 8) ? i : half + i;
      const int pos = a.row_pos[m];
      const int Hq = a.n_q_heads, Hkv = a.kv.n_kv_heads;
      float val = v[0];
      if (head < Hq + Hkv) {                         // q or k: rotate the pair
        if (pos < 0 || pos >= a.kv.max_pages_per_seq * a.kv.page_size) {
          if (a.err) atomicOr(a.err, UNO_DEVERR_BOUNDS);
          break;
        }
        const float x1 = finr[c & 7], x2 = finr[(c & 7) + 8];
        const float cs = a.rcos[(size_t)pos * half + i], sn = a.rsin[(size_t)pos * half + i];
        val = (c < 8) ? x1 * cs - x2 * sn : x2 * cs + x1 * sn;
      }
      if (head < Hq) {
        reinterpret_cast<T*>(a.qbuf)[(size_t)m * Hq * hd + head * hd + dim] = from_f<T>(val);
      } else {
        const int which = head < Hq + Hkv ? 0 : 1;
        const int h = head - Hq - which * Hkv;
        const int seq = a.call_seq[m / a.rows_per_seq];
        const int slot = a.row_slot ? a.row_slot[m] : pos;
        T* dst = kv_dst<T>(a.kv, a.layer, which, seq, slot, h, a.err);
        if (dst) dst[dim] = from_f<T>(val);
      }
      break;
    }
    default:
      break;
  }
}

// LM-head epilogue: logits with the MASK column at -inf and, per row and 16-column
// tile, (max, sum exp(l - max)).  The 16 lanes of a row are consecutive.
template <int NT>
UNO_DEV void logits_epilogue(const GemmArgs& a, int m, int c, int tile0, const float* v,
                             bool valid) {
  for (int t = 0; t < NT; ++t) {
    const int col = (tile0 + t) * 16 + c;
    const float l = (col == a.mask_col) ? -INFINITY : v[t];
    if (valid) reinterpret_cast<float*>(a.out)[(size_t)m * a.ldo + col] = l;
    float mx = l;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
    float e = (l == -INFINITY) ? 0.0f : expf(l - mx);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) e += __shfl_xor(e, off, 16);
    if (valid && c == 0) {
      a.tile_stats[((size_t)m * a.n_tiles + tile0 + t) * 2] = mx;
      a.tile_stats[((size_t)m * a.n_tiles + tile0 + t) * 2 + 1] = e;
    }
  }
}

template <int NT, int WAVES, int KU>
__global__ void __launch_bounds__(WAVES * 64)
k_gemm_bf16(GemmArgs a) {
  __shared__ float red[WAVES][NT][256];
  __shared__ float fin[256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int mt = blockIdx.y;
  const int grp = blockIdx.x;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;

  // weight-row pointers of this lane's column in each tile, and LoRA operands
  const bf16* Wp[NT];
  const bf16* Bp[NT];
  const long long* Up[NT];
  int ldu[NT];
  int tile0, col_paired = 0;
  if (a.paired) {
    const int c0 = grp * 16;
    col_paired = c0;
    tile0 = grp;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const GemmSeg& sg = a.seg[t];
      Wp[t] = reinterpret_cast<const bf16*>(sg.W) + (size_t)(c0 + r16) * a.K;
      Bp[t] = sg.Bl ? reinterpret_cast<const bf16*>(sg.Bl) + (size_t)(c0 + r16) * a.r : nullptr;
      Up[t] = sg.Ufx;
      ldu[t] = sg.ldu;
    }
  } else {
    tile0 = grp * NT;
    const GemmSeg& sg = a.seg[find_seg(a, tile_col(a, tile0, 0))];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int lc = tile_col(a, tile0 + t, r16) - sg.n0;
      Wp[t] = reinterpret_cast<const bf16*>(sg.W) + (size_t)lc * a.K;
      Bp[t] = sg.Bl ? reinterpret_cast<const bf16*>(sg.Bl) + (size_t)lc * a.r : nullptr;
      Up[t] = sg.Ufx;
      ldu[t] = sg.ldu;
    }
  }
  // workgroup 0 clears a fixed-point buffer that a later kernel accumulates into
  if (a.zero_ptr && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += WAVES * 64) a.zero_ptr[i] = 0;

  const int m_lane = mt * 16 + r16;
  const bool row_ok = m_lane < a.M;
  const bf16* Xp = reinterpret_cast<const bf16*>(a.X) + (size_t)(row_ok ? m_lane : 0) * a.ldx;

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- base phase: this wave's K slice
  const int kslice = a.K / WAVES;
  const int kb = w * kslice, ke = kb + kslice;
  int k = kb;
  const bf16x8 zero8 = {};
  for (; k + 32 * KU <= ke; k += 32 * KU) {
    bf16x8 af[KU], bfr[NT][KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) af[u] = row_ok ? load8(Xp + k + u * 32 + kq) : zero8;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < KU; ++u) bfr[t][u] = load8(Wp[t] + k + u * 32 + kq);
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u], bfr[t][u], acc[t], 0, 0, 0);
  }
  for (; k < ke; k += 32) {
    const bf16x8 af = row_ok ? load8(Xp + k + kq) : zero8;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, load8(Wp[t] + k + kq), acc[t], 0,
                                                       0, 0);
  }
  // ---- RMSNorm: scale rows of the base product by 1 / rms(x)
  if (a.ss_in) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float rs = rs_of(a, mt * 16 + (lane >> 4) * 4 + i);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][i] *= rs;
    }
  }

  // ---- LoRA phase: k over the rank, A = gate * bf16(scale * t), B = LoRA up
  if (a.r > 0) {
    const bool on = row_ok && (a.gate == nullptr || a.gate[m_lane] != 0);
    for (int kr = w * 32; kr < a.r; kr += 32 * WAVES) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (Up[t] == nullptr || Bp[t] == nullptr) continue;
        bf16x8 af = zero8;
        if (on) {
          const long long* tp = Up[t] + (size_t)m_lane * ldu[t] + kr + kq;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            af[e] = (bf16)(float)((double)a.scale * ((double)tp[e] * LORA_FX_INV));
        }
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, load8(Bp[t] + kr + kq), acc[t],
                                                         0, 0, 0);
      }
    }
  }

  // ---- fixed-order reduction of the wave partials
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][t][((lane >> 4) * 4 + i) * 16 + r16] = acc[t][i];
  __syncthreads();
  float v[NT];
  const int e = threadIdx.x & 255;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float sum = 0.0f;
    for (int ww = 0; ww < WAVES; ++ww) sum += red[ww][t][e];
    v[t] = sum;
  }
  if (threadIdx.x < 256) fin[e] = v[0];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int row = e >> 4, c = e & 15;
    const int m = mt * 16 + row;
    if (a.epi == EPI_LOGITS) logits_epilogue<NT>(a, m, c, tile0, v, m < a.M);
    else epilogue<bf16, NT>(a, m, c, tile0, col_paired, v, fin + row * 16, m < a.M);
  }
}


// ---------------------------------------------------------------------------
// Large-M variant (prefill, large batch, the distillation forward): a 128-row x
// 128-column tile per workgroup (2 x 2 waves of 64 x 64, i.e. 4 x 4 MFMA tiles
// each), K in steps of 64 through padded (bank-conflict-free) LDS tiles of X and
// W, the next K step prefetched into registers while the current one is
// multiplied.  The LoRA up-projection runs as extra K steps (A = the gated
// fixed-point intermediate, B = LoRA up rows).  In the paired (SwiGLU) case the W
// tile holds 64 gate rows and the matching 64 up rows, so the output is 128 x 64.
// When the N-tiles divide evenly over the 8 XCDs, all M-blocks of one N-tile run on
// one XCD and share its W tile in that XCD's L2.
constexpr int BM = 128, BN = 128, BK = 64, BKP = BK + 8;

__global__ void __launch_bounds__(256)
k_gemm_big(GemmArgs a, int mblocks) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  bf16* sA = reinterpret_cast<bf16*>(smem_raw);        // [BM][BKP]
  bf16* sB = sA + BM * BKP;                             // [BN][BKP]
  float* sC = reinterpret_cast<float*>(smem_raw);      // [BM][BN] after the K loop

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int lin = blockIdx.x, nb_n = gridDim.x / mblocks;
  int nb, mb;
  if (nb_n % 8 == 0) {                 // XCD-aware order (workgroups go round-robin to XCDs)
    const int xcd = lin % 8, slot = lin / 8;
    nb = xcd + 8 * (slot / mblocks);
    mb = slot % mblocks;
  } else {
    nb = lin / mblocks;
    mb = lin % mblocks;
  }
  const int m0 = mb * BM;
  const int outc = a.paired ? BN / 2 : BN;
  const int c0 = nb * outc;

  // segment and in-segment weight row of tile row j
  auto wrow = [&](int j, int* seg) -> int {
    if (a.paired) { *seg = j / 64; return c0 + (j % 64); }
    const int col = tile_col(a, (c0 + j) / 16, (c0 + j) % 16);
    const int sgi = find_seg(a, col);
    *seg = sgi;
    return col - a.seg[sgi].n0;
  };
  // each thread copies 4 16-byte pieces of A and 4 of B per K step:
  // piece p = tid + 256 * q -> tile row p / 8, k offset (p % 8) * 8
  const bf16* srcB[4];
  const bf16* srcBl[4];
  int rowA[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = tid + 256 * q, row = p / 8;
    int sg;
    const int wr = wrow(row, &sg);
    srcB[q] = reinterpret_cast<const bf16*>(a.seg[sg].W) + (size_t)wr * a.K;
    srcBl[q] = a.seg[sg].Bl ? reinterpret_cast<const bf16*>(a.seg[sg].Bl) + (size_t)wr * a.r
                            : nullptr;
    rowA[q] = m0 + row;
  }
  if (a.zero_ptr && blockIdx.x == 0)
    for (int i = tid; i < a.zero_n; i += 256) a.zero_ptr[i] = 0;

  const bf16* X = reinterpret_cast<const bf16*>(a.X);
  const bf16x8 zero8 = {};
  bf16x8 ra[4], rb[4];
  auto fetch = [&](int k) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = tid + 256 * q, kk = k + (p % 8) * 8;
      ra[q] = rowA[q] < a.M ? load8(X + (size_t)rowA[q] * a.ldx + kk) : zero8;
      rb[q] = load8(srcB[q] + kk);
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = a.K / BK;
  fetch(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = tid + 256 * q, row = p / 8, ko = (p % 8) * 8;
      *reinterpret_cast<bf16x8*>(sA + row * BKP + ko) = ra[q];
      *reinterpret_cast<bf16x8*>(sB + row * BKP + ko) = rb[q];
    }
    if (kt + 1 < nk) fetch((kt + 1) * BK);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * 64 + i * 16 + r16) * BKP + ks * 32 + kq);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sB + (wn * 64 + j * 16 + r16) * BKP + ks * 32 + kq);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // RMSNorm: scale rows of the base product by 1 / rms(x)
  if (a.ss_in) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rs = rs_of(a, m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j][e] *= rs;
      }
  }
  // LoRA phase: B = LoRA up rows via LDS; A = gate * bf16(scale * t) formed from
  // the fixed-point intermediate of the segment each 16-column tile belongs to
  if (a.r > 0) {
    for (int kr = 0; kr < a.r; kr += BK) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = tid + 256 * q, row = p / 8, ko = (p % 8) * 8;
        *reinterpret_cast<bf16x8*>(sB + row * BKP + ko) = srcBl[q] ? load8(srcBl[q] + kr + ko) : zero8;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int sg;
        (void)wrow(wn * 64 + j * 16, &sg);
        const GemmSeg& S = a.seg[sg];
        if (!S.Ufx || !S.Bl) continue;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
          const bf16x8 bfr =
              *reinterpret_cast<const bf16x8*>(sB + (wn * 64 + j * 16 + r16) * BKP + ks * 32 + kq);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 64 + i * 16 + r16;
            bf16x8 af = zero8;
            if (m < a.M && (a.gate == nullptr || a.gate[m] != 0)) {
              const long long* tp = S.Ufx + (size_t)m * S.ldu + kr + ks * 32 + kq;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                af[e] = (bf16)(float)((double)a.scale * ((double)tp[e] * LORA_FX_INV));
            }
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }
  // stage the finished tile in LDS and run the epilogue per 16 x 16 sub-tile:
  // 16 groups of 16 threads, group g takes sub-tiles g, g + 16, ...
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sC[(wm * 64 + i * 16 + (lane >> 4) * 4 + e) * BN + wn * 64 + j * 16 + r16] = acc[i][j][e];
  __syncthreads();
  const int g = tid >> 4, c = tid & 15;
  const int sub_n = outc / 16;
  for (int st = g; st < (BM / 16) * sub_n; st += 16) {
    const int sr = st / sub_n, sc = st % sub_n;
    const int tile0 = c0 / 16 + sc;
    for (int rr = 0; rr < 16; ++rr) {
      const int row = sr * 16 + rr, m = m0 + row;
      const float* finr = sC + row * BN + sc * 16;
      float v[2];
      v[0] = finr[c];
      v[1] = a.paired ? finr[64 + c] : 0.0f;
      if (a.epi == EPI_LOGITS) logits_epilogue<1>(a, m, c, tile0, v, m < a.M);
      else if (a.paired) epilogue<bf16, 2>(a, m, c, tile0, c0 + sc * 16, v, finr, m < a.M);
      else epilogue<bf16, 1>(a, m, c, tile0, 0, v, finr, m < a.M);
    }
  }
}

// float32 twin (small configurations): thread e of the 256 owns element
// (e / 16, e % 16) of each 16x16 tile and runs the K loop itself.  Segments may
// have any width (columns past the last segment are skipped).
template <int NT>
__global__ void __launch_bounds__(256)
k_gemm_f32(GemmArgs a) {
  __shared__ float fin[256];
  const int mt = blockIdx.y, grp = blockIdx.x;
  const int e = threadIdx.x, row = e >> 4, c = e & 15;
  const int m = mt * 16 + row;
  const int ntot = a.paired ? a.seg[0].N : a.seg[a.nseg - 1].n0 + a.seg[a.nseg - 1].N;
  int tile0, col_paired = 0;
  bool ok = m < a.M;
  const float* Wr[NT];
  const float* Br[NT];
  const float* Ur[NT];
  int ldu[NT];
  if (a.paired) {
    tile0 = grp;
    col_paired = grp * 16;
    ok = ok && col_paired + c < ntot;
    for (int t = 0; t < NT; ++t) {
      const GemmSeg& sg = a.seg[t];
      const int lc = ok ? col_paired + c : 0;
      Wr[t] = reinterpret_cast<const float*>(sg.W) + (size_t)lc * a.K;
      Br[t] = sg.Bl ? reinterpret_cast<const float*>(sg.Bl) + (size_t)lc * a.r : nullptr;
      Ur[t] = reinterpret_cast<const float*>(sg.U);
      ldu[t] = sg.ldu;
    }
  } else {
    tile0 = grp * NT;
    for (int t = 0; t < NT; ++t) {
      const int gcol = tile_col(a, tile0 + t, c);
      const bool cok = gcol < ntot;
      if (t == 0) ok = ok && cok;
      const GemmSeg& sg = a.seg[find_seg(a, cok ? gcol : 0)];
      const int lc = cok ? gcol - sg.n0 : 0;
      Wr[t] = reinterpret_cast<const float*>(sg.W) + (size_t)lc * a.K;
      Br[t] = sg.Bl ? reinterpret_cast<const float*>(sg.Bl) + (size_t)lc * a.r : nullptr;
      Ur[t] = reinterpret_cast<const float*>(sg.U);
      ldu[t] = sg.ldu;
    }
  }
  if (a.zero_ptr && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += 256) a.zero_ptr[i] = 0;
  const float* x = reinterpret_cast<const float*>(a.X) + (size_t)(m < a.M ? m : 0) * a.ldx;
  const float rs = rs_of(a, m);
  float v[NT];
  for (int t = 0; t < NT; ++t) {
    float s = 0.0f;
    if (ok) {
      for (int k = 0; k < a.K; ++k) s += x[k] * Wr[t][k];
      s *= rs;
      if (a.r > 0 && Ur[t] && Br[t]) {
        const float* u = Ur[t] + (size_t)m * ldu[t];
        for (int k = 0; k < a.r; ++k) s += u[k] * Br[t][k];
      }
    }
    v[t] = s;
  }
  fin[e] = v[0];
  __syncthreads();
  if (a.epi == EPI_LOGITS) logits_epilogue<NT>(a, m, c, tile0, v, ok);
  else epilogue<float, NT>(a, m, c, tile0, col_paired, v, fin + row * 16, ok);
}

// LoRA down-projection: one wave per (16 columns, K chunk, 16 rows); the fp32
// partial of its K chunk (times rs for a normalised input) is added in fixed point
// with 64-bit integer atomics, so the total is exact and independent of the order
// the chunks land in.
__global__ void __launch_bounds__(64)
k_lora_down(LoraDownArgs a) {
  const int lane = threadIdx.x, r16 = lane & 15, grp = lane >> 4, kq = grp * 8;
  const int col0 = blockIdx.x * 16, kc = blockIdx.y, mt = blockIdx.z;
  const int p = col0 / a.r, lc = col0 % a.r;
  const bf16* Ap = reinterpret_cast<const bf16*>(a.A[p]) + (size_t)(lc + r16) * a.K;
  const int m_lane = mt * 16 + r16;
  const bool row_ok = m_lane < a.M;
  const bf16* Xp = reinterpret_cast<const bf16*>(a.X) + (size_t)(row_ok ? m_lane : 0) * a.ldx;
  const int kb = kc * a.kchunk, ke = kb + a.kchunk;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero8 = {};
  for (int k = kb; k < ke; k += 64) {
    const bf16x8 x0 = row_ok ? load8(Xp + k + kq) : zero8;
    const bf16x8 x1 = row_ok ? load8(Xp + k + 32 + kq) : zero8;
    const bf16x8 w0 = load8(Ap + k + kq);
    const bf16x8 w1 = load8(Ap + k + 32 + kq);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, w0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, w1, acc, 0, 0, 0);
  }
  const int ncols = a.nproj * a.r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = mt * 16 + grp * 4 + i;
    if (m < a.M) {
      float v = acc[i];
      if (a.ss_in) {
        const float ms = (float)((double)a.ss_in[m] * LORA_FX_INV) * a.inv_d;
        v *= 1.0f / sqrtf(ms + a.eps);
      }
      const long long q = (long long)llrintf(v * LORA_FX_SCALE);
      atomicAdd(reinterpret_cast<unsigned long long*>(a.t + (size_t)m * ncols + col0 + r16),
                (unsigned long long)q);
    }
  }
}

__global__ void k_zero_i64(long long* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % a.kchunk || a.kchunk % 64 || a.r % 16) return hipErrorInvalidValue;
  dim3 grid(a.nproj * a.r / 16, a.K / a.kchunk, (a.M + 15) / 16);
  uno_launch(k_lora_down, grid, 64, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zero_i64(long long* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  uno_launch(k_zero_i64, blocks, 256, 0, s, p, n);
  return hipGetLastError();
}

template <>
hipError_t launch_gemm<bf16>(const GemmArgs& a, int n_cols_total, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % 32 != 0 || (a.r % 32) != 0 || n_cols_total % 16 != 0) return hipErrorInvalidValue;
  if (a.epi == EPI_QKV && (a.kv.head_dim % 16 != 0)) return hipErrorInvalidValue;
  const int outc = a.paired ? BN / 2 : BN;
  if (a.M >= 64 && a.K % BK == 0 && a.r % BK == 0 && n_cols_total % outc == 0 &&
      (a.epi != EPI_QKV || a.kv.head_dim % BN == 0 || BN % a.kv.head_dim == 0)) {
    const int mblocks = (a.M + BM - 1) / BM;
    const int nblocks = n_cols_total / outc;
    const size_t smem = (size_t)BM * BN * 4;
    uno_launch(k_gemm_big, nblocks * mblocks, 256, smem, s, a, mblocks);
    return hipGetLastError();
  }
  const int mtiles = (a.M + 15) / 16;
  dim3 grid(n_cols_total / 16, mtiles);
  if (a.paired) {
    if (a.K % 512 == 0) uno_launch(k_gemm_bf16<2, 16, 2>, grid, 1024, 0, s, a);
    else if (a.K % 128 == 0) uno_launch(k_gemm_bf16<2, 4, 1>, grid, 256, 0, s, a);
    else uno_launch(k_gemm_bf16<2, 1, 1>, grid, 64, 0, s, a);
  } else {
    if (a.epi == EPI_LOGITS && n_cols_total % 64 == 0 && a.K % 512 == 0) {
      // wide N: four column tiles per workgroup share each activation fragment
      dim3 g4(n_cols_total / 64, mtiles);
      uno_launch(k_gemm_bf16<4, 16, 2>, g4, 1024, 0, s, a);
    } else if (a.K % 1024 == 0) {
      uno_launch(k_gemm_bf16<1, 16, 4>, grid, 1024, 0, s, a);
    } else if (a.K % 128 == 0) {
      uno_launch(k_gemm_bf16<1, 4, 1>, grid, 256, 0, s, a);
    } else {
      uno_launch(k_gemm_bf16<1, 1, 1>, grid, 64, 0, s, a);
    }
  }
  return hipGetLastError();
}

template <>
hipError_t launch_gemm<float>(const GemmArgs& a, int n_cols_total, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.epi == EPI_LOGITS && n_cols_total % 16 != 0) return hipErrorInvalidValue;
  const int mtiles = (a.M + 15) / 16;
  dim3 grid((n_cols_total + 15) / 16, mtiles);
  if (a.paired) uno_launch(k_gemm_f32<2>, grid, 256, 0, s, a);
  else uno_launch(k_gemm_f32<1>, grid, 256, 0, s, a);
  return hipGetLastError();
}
