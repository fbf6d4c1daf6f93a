// Kernels of the distillation backward: the gradient of the block-wise TV loss
// with respect to the gated LoRA, base weights frozen (shibing624 reading notes,
// "Diffusion Distillation": the AR model is the frozen teacher and only the LoRA
// of the diffusion path is trained; the TV term compares the diffusion and AR
// distributions block by block).
//
// Every product of the backward runs through one MFMA GEMM (k_bw_gemm) with
// operand loaders for the layouts the backward meets: row-major activations and
// gradients (either axis contiguous), and the fragment-tiled weights read either
// way round.  A float32 operand (a gradient) enters as two bf16 terms,
// hi = bf16(v) and lo = bf16(v - hi), so that its 16 leading bits take part; the
// other operand is a stored bf16 value (weight, activation) and exact, and the
// products accumulate in float32.  Attention is formed explicitly per sequence
// and KV head: the scores against the x rows' keys, P V, dP and dq are GEMMs that
// skip the tiles and k steps past a tile's block-causal limit; each z1 block's own
// B keys (scores, P V, dP, and the dq, dk, dv of the block) run in small kernels;
// the softmax and its backward over both parts are row kernels.
#include "uno_internal.h"

namespace {

constexpr int BT = 128;           // output tile edge
constexpr int BK = 32;            // k per step (one 16x16x32 bf16 MFMA)
constexpr int LP = BK + 8;        // LDS row pitch in bf16 (80 B: spreads rows over banks)

UNO_DEV long off2(const Idx2& x, long i) {
  return (i >> x.sh) * x.hi + (i & ((1L << x.sh) - 1)) * x.lo;
}

UNO_DEV void split8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16 h = (bf16)v[j];
    hi[j] = h;
    lo[j] = (bf16)(v[j] - (float)h);    // v - h is exact in float32
  }
}

UNO_DEV bf16x8 ld_bf8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
UNO_DEV void ld_f8(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Output row of a q / k / v projection whose weight rows are stored in the RoPE
// pair order (each 16-row block of a head holds rows 8j..8j+7 and hd/2+8j..+7).
UNO_DEV long unpair_row(long p, int hd) {
  const long head = p / hd;
  const int w = (int)(p % hd), j = w >> 4, i = w & 15;
  return head * hd + (i < 8 ? 8 * j + i : hd / 2 + 8 * j + (i - 8));
}

UNO_DEV void store_out(const BwGemm& g, long row, long col, long cb, float v) {
  if (g.row_scale) v *= g.row_scale[row];
  v *= g.alpha;
  const long r = g.perm_hd ? unpair_row(row, g.perm_hd) : row;
  const long o = cb + off2(g.ci, r) + col;
  if (g.out_bf16) {
    bf16* C = reinterpret_cast<bf16*>(g.C);
    C[o] = (bf16)(g.accumulate ? (float)C[o] + v : v);
  } else {
    float* C = reinterpret_cast<float*>(g.C);
    C[o] = g.accumulate ? C[o] + v : v;
  }
}

// One 128 x 128 output tile per workgroup of 4 waves (2 x 2, 64 x 64 each);
// blockIdx.x = tile (+ split * tiles), blockIdx.z = batch.
template <int AM, int BMD>
__global__ void __launch_bounds__(256) k_bw_gemm(BwGemm g) {
  constexpr bool a_split = AM != BW_A_K16;
  constexpr bool b_split = BMD == BW_B_N32;
  __shared__ bf16 sAh[BT * LP];
  __shared__ bf16 sAl[a_split ? BT * LP : 8];
  __shared__ bf16 sBh[BT * LP];
  __shared__ bf16 sBl[b_split ? BT * LP : 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int tiles_n = (g.N + BT - 1) / BT, tiles = tiles_n * ((g.M + BT - 1) / BT);
  const int split = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int m0 = (tile / tiles_n) * BT, n0 = (tile % tiles_n) * BT;
  const long zo = blockIdx.z / g.bz, zi = blockIdx.z % g.bz;
  const char* Ab = reinterpret_cast<const char*>(g.A) +
                   (zo * g.a_bs + zi * g.a_bs2) * (AM == BW_A_K16 ? 2 : 4);
  const char* Bb = reinterpret_cast<const char*>(g.B) +
                   (zo * g.b_bs + zi * g.b_bs2) * (BMD == BW_B_N32 ? 4 : 2);
  const long cb = zo * g.c_bs + zi * g.c_bs2;
  // this split's k range, whole steps
  const int nsteps = (g.K + BK - 1) / BK;
  const int per = (nsteps + g.splits - 1) / g.splits;
  int s0 = split * per, s1 = min(nsteps, s0 + per);
  if (g.lim_mode) {   // block-causal key limit of this tile's rows
    const int lim = (((min(m0 + BT, g.M) - 1) / g.lim_G) / g.lim_B) * g.lim_B;
    if (g.lim_mode == 1 && n0 >= lim) return;
    if (g.lim_mode == 2) s1 = min(s1, (lim + BK - 1) / BK);
  }

  // staged operands of one step: two 8-element chunks of A and of B per thread
  float ra[2][8], rb[2][8];
  bf16x8 qa[2], qb[2];

  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * 256;
      // ---- A
      if (AM == BW_A_K16 || AM == BW_A_K32) {
        const int m = c >> 2, kq = (c & 3) * 8;
        const long gm = m0 + m, gk = k0 + kq;
        const bool ok = gm < g.M && gk < g.K;
        if (AM == BW_A_K16) {
          qa[h] = ok ? ld_bf8(reinterpret_cast<const bf16*>(Ab) + off2(g.ai, gm) + gk) : bf16x8{};
        } else {
          if (ok) ld_f8(reinterpret_cast<const float*>(Ab) + off2(g.ai, gm) + gk, ra[h]);
          else for (int j = 0; j < 8; ++j) ra[h][j] = 0.f;
        }
      } else {   // BW_A_M32: element (m, k) at A[off(k) + m]
        const int k = c >> 4, mq = (c & 15) * 8;
        const long gm = m0 + mq, gk = k0 + k;
        if (gm < g.M && gk < g.K) {
          ld_f8(reinterpret_cast<const float*>(Ab) + off2(g.ai, gk) + gm, ra[h]);
          if (g.kscale) {
            const float sc = g.kscale[gk];
            for (int j = 0; j < 8; ++j) ra[h][j] *= sc;
          }
        } else {
          for (int j = 0; j < 8; ++j) ra[h][j] = 0.f;
        }
      }
      // ---- B
      if (BMD == BW_B_K16) {
        const int n = c >> 2, kq = (c & 3) * 8;
        const long gn = n0 + n, gk = k0 + kq;
        qb[h] = (gn < g.N && gk < g.K)
                    ? ld_bf8(reinterpret_cast<const bf16*>(Bb) + off2(g.bi, gn) + gk) : bf16x8{};
      } else if (BMD == BW_B_TN) {   // stored [N][K] tiled; a chunk is one lane of a block
        const int blk = c >> 6, ln = c & 63;
        const long gn = n0 + blk * 16, gk = k0;
        qb[h] = (gn < g.N && gk < g.K)
                    ? ld_bf8(reinterpret_cast<const bf16*>(Bb) +
                             (((long)(n0 >> 4) + blk) * (g.b_cols >> 5) + (k0 >> 5)) * 512 + ln * 8)
                    : bf16x8{};
      } else if (BMD == BW_B_TT) {   // stored [K][N] tiled: element (n, k) = W[k][n]
        const int blk = c >> 6, ln = c & 63, rb = blk & 1, cbk = blk >> 1;
        const long gk = k0 + rb * 16, gn = n0 + cbk * 32;
        qb[h] = (gn < g.N && gk < g.K)
                    ? ld_bf8(reinterpret_cast<const bf16*>(Bb) +
                             (((long)(k0 >> 4) + rb) * (g.b_cols >> 5) + (n0 >> 5) + cbk) * 512 + ln * 8)
                    : bf16x8{};
      } else {   // BW_B_N16 / BW_B_N32: element (n, k) at B[off(k) + n]
        const int k = c >> 4, nq = (c & 15) * 8;
        const long gn = n0 + nq, gk = k0 + k;
        const bool ok = gn < g.N && gk < g.K;
        if (BMD == BW_B_N16) {
          qb[h] = ok ? ld_bf8(reinterpret_cast<const bf16*>(Bb) + off2(g.bi, gk) + gn) : bf16x8{};
        } else {
          if (ok) ld_f8(reinterpret_cast<const float*>(Bb) + off2(g.bi, gk) + gn, rb[h]);
          else for (int j = 0; j < 8; ++j) rb[h][j] = 0.f;
        }
      }
    }
  };

  auto stash = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + h * 256;
      if (AM == BW_A_K16) {
        *reinterpret_cast<bf16x8*>(&sAh[(c >> 2) * LP + (c & 3) * 8]) = qa[h];
      } else if (AM == BW_A_K32) {
        bf16x8 hi, lo;
        split8(ra[h], hi, lo);
        *reinterpret_cast<bf16x8*>(&sAh[(c >> 2) * LP + (c & 3) * 8]) = hi;
        *reinterpret_cast<bf16x8*>(&sAl[(c >> 2) * LP + (c & 3) * 8]) = lo;
      } else {
        bf16x8 hi, lo;
        split8(ra[h], hi, lo);
        const int k = c >> 4, mq = (c & 15) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sAh[(mq + j) * LP + k] = hi[j];
          sAl[(mq + j) * LP + k] = lo[j];
        }
      }
      if (BMD == BW_B_K16) {
        *reinterpret_cast<bf16x8*>(&sBh[(c >> 2) * LP + (c & 3) * 8]) = qb[h];
      } else if (BMD == BW_B_TN) {
        const int blk = c >> 6, ln = c & 63;
        *reinterpret_cast<bf16x8*>(&sBh[(blk * 16 + (ln & 15)) * LP + (ln >> 4) * 8]) = qb[h];
      } else if (BMD == BW_B_TT) {
        const int blk = c >> 6, ln = c & 63, rb = blk & 1, cbk = blk >> 1;
        const int k = rb * 16 + (ln & 15), nq = cbk * 32 + (ln >> 4) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) sBh[(nq + j) * LP + k] = qb[h][j];
      } else if (BMD == BW_B_N16) {
        const int k = c >> 4, nq = (c & 15) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) sBh[(nq + j) * LP + k] = qb[h][j];
      } else {
        bf16x8 hi, lo;
        split8(rb[h], hi, lo);
        const int k = c >> 4, nq = (c & 15) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sBh[(nq + j) * LP + k] = hi[j];
          sBl[(nq + j) * LP + k] = lo[j];
        }
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (s0 < s1) load(s0 * BK);
  for (int st = s0; st < s1; ++st) {
    stash();
    __syncthreads();
    if (st + 1 < s1) load((st + 1) * BK);   // in flight during the products
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    bf16x8 ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = *reinterpret_cast<const bf16x8*>(&sAh[(wm * 64 + i * 16 + fr) * LP + fk]);
      if (a_split) al[i] = *reinterpret_cast<const bf16x8*>(&sAl[(wm * 64 + i * 16 + fr) * LP + fk]);
      bh[i] = *reinterpret_cast<const bf16x8*>(&sBh[(wn * 64 + i * 16 + fr) * LP + fk]);
      if (b_split) bl[i] = *reinterpret_cast<const bf16x8*>(&sBl[(wn * 64 + i * 16 + fr) * LP + fk]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        if (a_split) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
        if (b_split) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
      }
    __syncthreads();
  }

  // epilogue: lane holds rows (lane / 16) * 4 + e, column lane % 16 of each block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        const long col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (row >= g.M || col >= g.N) continue;
        if (g.splits > 1) g.part[((long)split * g.M + row) * g.N + col] = acc[i][j][e];
        else store_out(g, row, col, cb, acc[i][j][e]);
      }
}

// Sum of the split partials in split order, then the GEMM's epilogue.
__global__ void k_bw_split_reduce(BwGemm g) {
  const long n = (long)g.M * g.N;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int p = 0; p < g.splits; ++p) s += g.part[(long)p * n + i];
    store_out(g, i / g.N, i % g.N, 0, s);
  }
}

// ---------------------------------------------------------------- row kernels

UNO_DEV float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

UNO_DEV float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
  for (int i = 0; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

// RMSNorm operands of a row: rs = 1 / sqrt(mean(x^2) + eps) and the stored
// gain-scaled input hg = bf16(x * g).
template <typename T>
__global__ void k_bw_rmsprep(const float* x, const T* gain, float eps, int d, bf16* hg, float* rs) {
  __shared__ float red[16];
  const long row = blockIdx.x;
  const float* xr = x + row * d;
  float ss = 0.f;
  for (int j = threadIdx.x; j < d; j += blockDim.x) ss += xr[j] * xr[j];
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) rs[row] = 1.0f / sqrtf(ss / d + eps);
  for (int j = threadIdx.x; j < d; j += blockDim.x) hg[row * d + j] = (bf16)(xr[j] * to_f(gain[j]));
}

// Gradient at x of h = hg * rs (hg = bf16(x * g), the rounding passed straight
// through): dx = dres + rs * g * dh - x * rs^3 * mean(hg * dh).
template <typename T>
__global__ void k_bw_rmsback(const float* x, const bf16* hg, const float* rs, const T* gain,
                             const float* dh, const float* dres, float* dx, int d) {
  __shared__ float red[16];
  const long row = blockIdx.x;
  float s = 0.f;
  for (int j = threadIdx.x; j < d; j += blockDim.x) s += (float)hg[row * d + j] * dh[row * d + j];
  s = block_sum(s, red) / d;
  const float r = rs[row], r3 = r * r * r;
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    const long o = row * d + j;
    dx[o] = (dres ? dres[o] : 0.f) + r * to_f(gain[j]) * dh[o] - x[o] * r3 * s;
  }
}

// Permuted position (RoPE pair order) of head-local column c.
UNO_DEV int pair_pos(int c, int hd) {
  const int half = hd / 2;
  return c < half ? 16 * (c >> 3) + (c & 7) : 16 * ((c - half) >> 3) + 8 + ((c - half) & 7);
}

// q / k after RoPE and v, stored bf16 in head order: Q [N][Hq*hd], Ks / Vs
// [N][Hkv*hd].  Y* are the projections in the stored pair order; row n = s * L + i
// sits at position i.
__global__ void k_bw_qkv_post(const float* Yq, const float* Yk, const float* Yv, const float* rcos,
                              const float* rsin, int L, int Hq, int Hkv, int hd, bf16* Q,
                              bf16* Ks, bf16* Vs) {
  const long n = blockIdx.x;
  const int i = (int)(n % L), half = hd / 2;
  const int qd = Hq * hd, kvd = Hkv * hd;
  for (int e = threadIdx.x; e < (Hq + Hkv) * half; e += blockDim.x) {
    const int h = e / half, c = e % half;
    const float cs = rcos[(size_t)i * half + c], sn = rsin[(size_t)i * half + c];
    if (h < Hq) {
      const float* y = Yq + n * qd + h * hd;
      const float y1 = y[pair_pos(c, hd)], y2 = y[pair_pos(c + half, hd)];
      Q[n * qd + h * hd + c] = (bf16)(y1 * cs - y2 * sn);
      Q[n * qd + h * hd + c + half] = (bf16)(y2 * cs + y1 * sn);
    } else {
      const int hk = h - Hq;
      const float* y = Yk + n * kvd + hk * hd;
      const float y1 = y[pair_pos(c, hd)], y2 = y[pair_pos(c + half, hd)];
      bf16* kr = Ks + n * kvd + hk * hd;
      kr[c] = (bf16)(y1 * cs - y2 * sn);
      kr[c + half] = (bf16)(y2 * cs + y1 * sn);
      const float* yv = Yv + n * kvd + hk * hd;
      bf16* vr = Vs + n * kvd + hk * hd;
      vr[c] = (bf16)yv[pair_pos(c, hd)];
      vr[c + half] = (bf16)yv[pair_pos(c + half, hd)];
    }
  }
}

// The transpose of k_bw_qkv_post: dq [N][Hq*hd] and the z1 keys' dk, dv [N][Hkv*hd]
// (head order) to the pair-ordered projection gradients; RoPE's transpose is the
// rotation by the opposite angle.
__global__ void k_bw_qkv_back(const float* dq, const float* dk, const float* dv, const float* rcos,
                              const float* rsin, int L, int Hq, int Hkv, int hd, float* dYq,
                              float* dYk, float* dYv) {
  const long n = blockIdx.x;
  const int i = (int)(n % L), half = hd / 2;
  const int qd = Hq * hd, kvd = Hkv * hd;
  for (int e = threadIdx.x; e < (Hq + Hkv) * half; e += blockDim.x) {
    const int h = e / half, c = e % half;
    const float cs = rcos[(size_t)i * half + c], sn = rsin[(size_t)i * half + c];
    if (h < Hq) {
      const float g1 = dq[n * qd + h * hd + c], g2 = dq[n * qd + h * hd + c + half];
      float* y = dYq + n * qd + h * hd;
      y[pair_pos(c, hd)] = g1 * cs + g2 * sn;
      y[pair_pos(c + half, hd)] = g2 * cs - g1 * sn;
    } else {
      const int hk = h - Hq;
      const float g1 = dk[n * kvd + hk * hd + c], g2 = dk[n * kvd + hk * hd + c + half];
      float* y = dYk + n * kvd + hk * hd;
      y[pair_pos(c, hd)] = g1 * cs + g2 * sn;
      y[pair_pos(c + half, hd)] = g2 * cs - g1 * sn;
      float* yv = dYv + n * kvd + hk * hd;
      yv[pair_pos(c, hd)] = dv[n * kvd + hk * hd + c];
      yv[pair_pos(c + half, hd)] = dv[n * kvd + hk * hd + c + half];
    }
  }
}

// Keys of the x rows that the GEMMs of one BT-row tile of rows m = i * G + g read
// (the tile's limit, rounded up to a k step): entries below it are written.
UNO_DEV int tile_keys(long m, int M, int G, int B, int L) {
  const long t0 = (m / BT) * BT;
  const int lim = (int)((((min(t0 + BT, (long)M) - 1) / G) / B) * B);
  return min(L, (lim + BK - 1) / BK * BK);
}

// Own-block scores of the z1 rows of block b (blockIdx.x) and KV head h
// (blockIdx.y): So[h][i * G + g][j] = q_(i, g) . k_(bB + j) for j <= i - bB.
__global__ void k_bw_own_scores(const bf16* Q, const bf16* Ks, int L, int Hq, int Hkv, int hd, int B,
                                float* So) {
  extern __shared__ float sk[];          // [B][hd] own keys
  const int b = blockIdx.x, h = blockIdx.y, G = Hq / Hkv, qd = Hq * hd, kvd = Hkv * hd;
  for (int e = threadIdx.x; e < B * hd; e += blockDim.x)
    sk[e] = (float)Ks[(size_t)(b * B + e / hd) * kvd + h * hd + e % hd];
  __syncthreads();
  for (int e = threadIdx.x; e < B * G * B; e += blockDim.x) {
    const int r = e / B, j = e % B, i = b * B + r / G, g = r % G;
    float acc = 0.f;
    if (j <= i - b * B) {
      const bf16* q = Q + (size_t)i * qd + (h * G + g) * hd;
      for (int d = 0; d < hd; ++d) acc += (float)q[d] * sk[j * hd + d];
    }
    So[((size_t)h * L * G + (size_t)i * G + g) * B + j] = acc;
  }
}

// Block-causal softmax of one sequence, in place: row m = i * G + g of KV head h
// (blockIdx.y) over the x keys < bB (St) and its own block's keys bB..i (So), with
// P = softmax(scale * S).  Invisible entries the GEMMs read become 0.
__global__ void k_bw_softmax(float* St, float* So, int L, int G, int B, float scale) {
  __shared__ float red[16];
  const long m = blockIdx.x, h = blockIdx.y;
  const int M = L * G, i = (int)(m / G), b0 = (i / B) * B, no = i - b0 + 1;
  const int lw = tile_keys(m, M, G, B, L);
  float* t = St + (h * (long)M + m) * L;
  float* o = So + (h * (long)M + m) * B;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < b0; j += blockDim.x) mx = fmaxf(mx, scale * t[j]);
  for (int j = threadIdx.x; j < no; j += blockDim.x) mx = fmaxf(mx, scale * o[j]);
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j < b0; j += blockDim.x) sum += expf(scale * t[j] - mx);
  for (int j = threadIdx.x; j < no; j += blockDim.x) sum += expf(scale * o[j] - mx);
  sum = block_sum(sum, red);
  const float inv = 1.0f / sum;
  for (int j = threadIdx.x; j < lw; j += blockDim.x) t[j] = j < b0 ? expf(scale * t[j] - mx) * inv : 0.f;
  for (int j = threadIdx.x; j < B; j += blockDim.x) o[j] = j < no ? expf(scale * o[j] - mx) * inv : 0.f;
}

// o = bf16(o32 + sum_j Po[., j] v_(bB + j)): the own block's share added to the x
// keys' share o32 [L][Hq*hd] of the z1 rows of block b (blockIdx.x), KV head h.
__global__ void k_bw_own_pv(const float* Po, const bf16* Vs, const float* o32, int L, int Hq, int Hkv,
                            int hd, int B, bf16* o) {
  extern __shared__ float sv[];          // [B][hd]
  const int b = blockIdx.x, h = blockIdx.y, G = Hq / Hkv, qd = Hq * hd, kvd = Hkv * hd;
  for (int e = threadIdx.x; e < B * hd; e += blockDim.x)
    sv[e] = (float)Vs[(size_t)(b * B + e / hd) * kvd + h * hd + e % hd];
  __syncthreads();
  for (int e = threadIdx.x; e < B * G * hd; e += blockDim.x) {
    const int r = e / hd, d = e % hd, i = b * B + r / G, g = r % G;
    const float* p = Po + ((size_t)h * L * G + (size_t)i * G + g) * B;
    const size_t oi = (size_t)i * qd + (h * G + g) * hd + d;
    float acc = o32[oi];
    for (int j = 0; j <= i - b * B; ++j) acc += p[j] * sv[j * hd + d];
    o[oi] = (bf16)acc;
  }
}

// dPo[., j] = dO . v_(bB + j) for the own block (j <= i - bB).
__global__ void k_bw_own_dp(const float* dO, const bf16* Vs, int L, int Hq, int Hkv, int hd, int B,
                            float* dPo) {
  extern __shared__ float sv[];
  const int b = blockIdx.x, h = blockIdx.y, G = Hq / Hkv, qd = Hq * hd, kvd = Hkv * hd;
  for (int e = threadIdx.x; e < B * hd; e += blockDim.x)
    sv[e] = (float)Vs[(size_t)(b * B + e / hd) * kvd + h * hd + e % hd];
  __syncthreads();
  for (int e = threadIdx.x; e < B * G * B; e += blockDim.x) {
    const int r = e / B, j = e % B, i = b * B + r / G, g = r % G;
    float acc = 0.f;
    if (j <= i - b * B) {
      const float* go = dO + (size_t)i * qd + (h * G + g) * hd;
      for (int d = 0; d < hd; ++d) acc += go[d] * sv[j * hd + d];
    }
    dPo[((size_t)h * L * G + (size_t)i * G + g) * B + j] = acc;
  }
}

// Softmax backward in place over the same entries: dS = scale * P * (dP - D),
// D = sum over the visible keys of P dP (the scale of the scores folded in).
__global__ void k_bw_softmax_back(const float* Pt, const float* Po, float* dPt, float* dPo, int L,
                                  int G, int B, float scale) {
  __shared__ float red[16];
  const long m = blockIdx.x, h = blockIdx.y;
  const int M = L * G, i = (int)(m / G), b0 = (i / B) * B, no = i - b0 + 1;
  const int lw = tile_keys(m, M, G, B, L);
  const long ot = (h * (long)M + m) * L, oo = (h * (long)M + m) * B;
  float s = 0.f;
  for (int j = threadIdx.x; j < b0; j += blockDim.x) s += Pt[ot + j] * dPt[ot + j];
  for (int j = threadIdx.x; j < no; j += blockDim.x) s += Po[oo + j] * dPo[oo + j];
  s = block_sum(s, red);
  for (int j = threadIdx.x; j < lw; j += blockDim.x)
    dPt[ot + j] = j < b0 ? scale * Pt[ot + j] * (dPt[ot + j] - s) : 0.f;
  for (int j = threadIdx.x; j < B; j += blockDim.x)
    dPo[oo + j] = j < no ? scale * Po[oo + j] * (dPo[oo + j] - s) : 0.f;
}

// Own-block backward of block b (blockIdx.x), KV head h: dq += dSo K_own, and the
// z1 keys' dk = dSo^T q, dv = Po^T dO (every (key, head) owned by one workgroup).
__global__ void k_bw_own_back(const float* dSo, const float* Po, const bf16* Q, const bf16* Ks,
                              const float* dO, int L, int Hq, int Hkv, int hd, int B, float* dq,
                              float* dk, float* dv) {
  extern __shared__ float sk[];
  const int b = blockIdx.x, h = blockIdx.y, G = Hq / Hkv, qd = Hq * hd, kvd = Hkv * hd;
  const size_t rb = (size_t)h * L * G + (size_t)b * B * G;     // first row of the block
  for (int e = threadIdx.x; e < B * hd; e += blockDim.x)
    sk[e] = (float)Ks[(size_t)(b * B + e / hd) * kvd + h * hd + e % hd];
  __syncthreads();
  for (int e = threadIdx.x; e < B * G * hd; e += blockDim.x) {
    const int r = e / hd, d = e % hd, i = b * B + r / G, g = r % G;
    const float* ds = dSo + (rb + r) * B;
    float acc = 0.f;
    for (int j = 0; j <= i - b * B; ++j) acc += ds[j] * sk[j * hd + d];
    dq[(size_t)i * qd + (h * G + g) * hd + d] += acc;
  }
  for (int e = threadIdx.x; e < B * hd; e += blockDim.x) {
    const int j = e / hd, d = e % hd;
    float ak = 0.f, av = 0.f;
    for (int r = j * G; r < B * G; ++r) {      // rows i >= bB + j see key bB + j
      const int i = b * B + r / G, g = r % G;
      const size_t qi = (size_t)i * qd + (h * G + g) * hd + d;
      ak += dSo[(rb + r) * B + j] * (float)Q[qi];
      av += Po[(rb + r) * B + j] * dO[qi];
    }
    dk[(size_t)(b * B + j) * kvd + h * hd + d] = ak;
    dv[(size_t)(b * B + j) * kvd + h * hd + d] = av;
  }
}

// SwiGLU product a = bf16(silu(g) * u).
__global__ void k_bw_swiglu(const float* Yg, const float* Yu, bf16* a, long n) {
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const float g = Yg[e];
    a[e] = (bf16)(g / (1.0f + expf(-g)) * Yu[e]);
  }
}

// Its backward, in place: Yg <- da * u * silu'(g), Yu <- da * silu(g).
__global__ void k_bw_swiglu_back(const float* da, float* Yg, float* Yu, long n) {
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const float g = Yg[e], u = Yu[e], sg = 1.0f / (1.0f + expf(-g));
    Yg[e] = da[e] * u * (sg + g * sg * (1.0f - sg));
    Yu[e] = da[e] * g * sg;
  }
}

// dL_TV / d(student logits) of one row and its TV: with N rows (inv2n = 1 / 2N)
// g(v) = sign(p_S(v) - p_T(v)) / 2N and dz(v) = p_S(v) (g(v) - sum_u p_S(u) g(u)).
__global__ void k_tv_grad(const float* T, const float* Sl, int V, float inv2n, float* dz,
                          float* tv_row) {
  __shared__ float red[16];
  const long row = blockIdx.x;
  const float* t = T + row * (long)V;
  const float* s = Sl + row * (long)V;
  float mt = -INFINITY, ms = -INFINITY;
  for (int j = threadIdx.x; j < V; j += blockDim.x) { mt = fmaxf(mt, t[j]); ms = fmaxf(ms, s[j]); }
  mt = block_max(mt, red);
  ms = block_max(ms, red);
  float st = 0.f, ss = 0.f;
  for (int j = threadIdx.x; j < V; j += blockDim.x) { st += expf(t[j] - mt); ss += expf(s[j] - ms); }
  st = block_sum(st, red);
  ss = block_sum(ss, red);
  const float it = 1.0f / st, is = 1.0f / ss;
  float c = 0.f, tv = 0.f;
  for (int j = threadIdx.x; j < V; j += blockDim.x) {
    const float pt = expf(t[j] - mt) * it, ps = expf(s[j] - ms) * is;
    const float sg = ps > pt ? 1.f : (ps < pt ? -1.f : 0.f);
    c += ps * sg;
    tv += fabsf(ps - pt);
  }
  c = block_sum(c, red);
  tv = block_sum(tv, red);
  if (threadIdx.x == 0 && tv_row) tv_row[row] = 0.5f * tv;
  float* d = dz + row * (long)V;
  for (int j = threadIdx.x; j < V; j += blockDim.x) {
    const float pt = expf(t[j] - mt) * it, ps = expf(s[j] - ms) * is;
    const float sg = ps > pt ? 1.f : (ps < pt ? -1.f : 0.f);
    d[j] = ps * (sg - c) * inv2n;
  }
}

// Mean of the rows' TV (double accumulation, one workgroup, fixed order).
__global__ void k_tv_mean(const float* tv_row, int rows, float* loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < rows; i += blockDim.x) s += tv_row[i];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < (int)blockDim.x; ++i) t += red[i];
    *loss = (float)(t / rows);
  }
}

template <int AM, int BMD>
hipError_t run_bw(const BwGemm& g, hipStream_t s) {
  const int tiles = ((g.M + BT - 1) / BT) * ((g.N + BT - 1) / BT);
  uno_launch(k_bw_gemm<AM, BMD>, dim3(tiles * g.splits, 1, g.batch), dim3(256), 0, s, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.splits == 1) return e;
  const long n = (long)g.M * g.N;
  uno_launch(k_bw_split_reduce, dim3((unsigned)std::min<long>((n + 255) / 256, 4096)), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bw_gemm(const BwGemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  if (g.splits < 1 || g.batch < 1 || g.bz < 1 || (g.splits > 1 && (g.batch != 1 || !g.part)))
    return hipErrorInvalidValue;
  if (g.lim_mode && (g.lim_G < 1 || g.lim_B < 1 || (g.lim_mode == 2 && g.splits != 1)))
    return hipErrorInvalidValue;
  // 16-byte operand chunks: the contiguous axis of every operand in whole 8s
  if (g.K % 8 || g.M % 8 || g.N % 8) return hipErrorInvalidValue;
  const bool tiled = g.bmode == BW_B_TN || g.bmode == BW_B_TT;
  if (tiled && (g.b_cols % 32 || (g.bmode == BW_B_TN ? g.K % 32 || g.N % 16 : g.K % 16 || g.N % 32)))
    return hipErrorInvalidValue;
#define BW_CASE(a, b) \
  if (g.amode == a && g.bmode == b) return run_bw<a, b>(g, s);
  BW_CASE(BW_A_K16, BW_B_TN)
  BW_CASE(BW_A_K16, BW_B_K16)
  BW_CASE(BW_A_K32, BW_B_N16)
  BW_CASE(BW_A_K32, BW_B_K16)
  BW_CASE(BW_A_K32, BW_B_TT)
  BW_CASE(BW_A_M32, BW_B_N16)
#undef BW_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_bw_rmsprep(const float* x, const T* gain, float eps, int rows, int d, bf16* hg,
                             float* rs, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  uno_launch(k_bw_rmsprep<T>, dim3(rows), dim3(256), 0, s, x, gain, eps, d, hg, rs);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bw_rmsback(const float* x, const bf16* hg, const float* rs, const T* gain,
                             const float* dh, const float* dres, float* dx, int rows, int d,
                             hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  uno_launch(k_bw_rmsback<T>, dim3(rows), dim3(256), 0, s, x, hg, rs, gain, dh, dres, dx, d);
  return hipGetLastError();
}

hipError_t launch_bw_qkv_post(const float* Yq, const float* Yk, const float* Yv, const float* rcos,
                              const float* rsin, int rows, int L, int Hq, int Hkv, int hd, bf16* Q,
                              bf16* Ks, bf16* Vs, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  uno_launch(k_bw_qkv_post, dim3(rows), dim3(256), 0, s, Yq, Yk, Yv, rcos, rsin, L, Hq, Hkv, hd, Q, Ks, Vs);
  return hipGetLastError();
}

hipError_t launch_bw_qkv_back(const float* dq, const float* dk, const float* dv, const float* rcos,
                              const float* rsin, int rows, int L, int Hq, int Hkv, int hd, float* dYq,
                              float* dYk, float* dYv, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  uno_launch(k_bw_qkv_back, dim3(rows), dim3(256), 0, s, dq, dk, dv, rcos, rsin, L, Hq, Hkv, hd, dYq, dYk, dYv);
  return hipGetLastError();
}

hipError_t launch_bw_own_scores(const bf16* Q, const bf16* Ks, int L, int Hq, int Hkv, int hd, int B,
                                float* So, hipStream_t s) {
  uno_launch(k_bw_own_scores, dim3(L / B, Hkv), dim3(256), (uint32_t)(B * hd * 4), s, Q, Ks, L, Hq, Hkv, hd, B, So);
  return hipGetLastError();
}

hipError_t launch_bw_softmax(float* St, float* So, int L, int G, int Hkv, int B, float scale,
                             hipStream_t s) {
  uno_launch(k_bw_softmax, dim3(L * G, Hkv), dim3(256), 0, s, St, So, L, G, B, scale);
  return hipGetLastError();
}

hipError_t launch_bw_own_pv(const float* Po, const bf16* Vs, const float* o32, int L, int Hq, int Hkv,
                            int hd, int B, bf16* o, hipStream_t s) {
  uno_launch(k_bw_own_pv, dim3(L / B, Hkv), dim3(256), (uint32_t)(B * hd * 4), s, Po, Vs, o32, L, Hq, Hkv, hd, B, o);
  return hipGetLastError();
}

hipError_t launch_bw_own_dp(const float* dO, const bf16* Vs, int L, int Hq, int Hkv, int hd, int B,
                            float* dPo, hipStream_t s) {
  uno_launch(k_bw_own_dp, dim3(L / B, Hkv), dim3(256), (uint32_t)(B * hd * 4), s, dO, Vs, L, Hq, Hkv, hd, B, dPo);
  return hipGetLastError();
}

hipError_t launch_bw_softmax_back(const float* Pt, const float* Po, float* dPt, float* dPo, int L,
                                  int G, int Hkv, int B, float scale, hipStream_t s) {
  uno_launch(k_bw_softmax_back, dim3(L * G, Hkv), dim3(256), 0, s, Pt, Po, dPt, dPo, L, G, B, scale);
  return hipGetLastError();
}

hipError_t launch_bw_own_back(const float* dSo, const float* Po, const bf16* Q, const bf16* Ks,
                              const float* dO, int L, int Hq, int Hkv, int hd, int B, float* dq,
                              float* dk, float* dv, hipStream_t s) {
  uno_launch(k_bw_own_back, dim3(L / B, Hkv), dim3(256), (uint32_t)(B * hd * 4), s, dSo, Po, Q, Ks, dO, L,
             Hq, Hkv, hd, B, dq, dk, dv);
  return hipGetLastError();
}

hipError_t launch_bw_swiglu(const float* Yg, const float* Yu, bf16* a, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  uno_launch(k_bw_swiglu, dim3((unsigned)std::min<long>((n + 255) / 256, 16384)), dim3(256), 0, s, Yg, Yu, a, n);
  return hipGetLastError();
}

hipError_t launch_bw_swiglu_back(const float* da, float* Yg, float* Yu, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  uno_launch(k_bw_swiglu_back, dim3((unsigned)std::min<long>((n + 255) / 256, 16384)), dim3(256), 0, s, da, Yg, Yu, n);
  return hipGetLastError();
}

hipError_t launch_tv_grad(const float* T, const float* S, int rows, int V, float inv2n, float* dz,
                          float* tv_row, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  uno_launch(k_tv_grad, dim3(rows), dim3(1024), 0, s, T, S, V, inv2n, dz, tv_row);
  return hipGetLastError();
}

hipError_t launch_tv_mean(const float* tv_row, int rows, float* loss, hipStream_t s) {
  uno_launch(k_tv_mean, dim3(1), dim3(256), 0, s, tv_row, rows, loss);
  return hipGetLastError();
}

#define UNO_BW_INST(T)                                                                       \
  template hipError_t launch_bw_rmsprep<T>(const float*, const T*, float, int, int, bf16*,  \
                                           float*, hipStream_t);                             \
  template hipError_t launch_bw_rmsback<T>(const float*, const bf16*, const float*, const T*, \
                                           const float*, const float*, float*, int, int,     \
                                           hipStream_t);
UNO_BW_INST(float)
UNO_BW_INST(bf16)
