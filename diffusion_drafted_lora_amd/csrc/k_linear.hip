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
// A weight fragment that is read exactly once per forward: a non-temporal load
// keeps the stream from evicting the activations and other reused lines from the
// caches (measured on this part: 12% faster at the gate/up shape).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
UNO_DEV bf16x8 load8_stream(const bf16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(p)));
}

UNO_DEV float rs_of(const GemmArgs& a, int m) {
  if (!a.ss_in || m >= a.M) return 1.0f;
  const float ms = fx_to_float(ss_row(a.ss_in, m, a.err)) * a.inv_d;
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

// (page, KV head) block holding a slot of a sequence, or null (bounds flag set)
template <typename T>
UNO_DEV T* kv_dst(const KvLayout& kv, int layer, int which, int seq, int slot, int h,
                  int32_t* err) {
  const int page = kv_page(kv, seq, slot);
  if (page < 0) {
    if (err) atomicOr(err, UNO_DEVERR_BOUNDS);
    return nullptr;
  }
  return kv_block<T>(kv, layer, which, page, h);
}

// Epilogue of one element (row m, lane column c) of each of the NT tiles.  `vp`
// is the finished tile-0 value of column c ^ 8 of the same row (the RoPE
// partner).  Every thread of a 16-lane row group calls this (row sums use
// shuffles); `ok` says whether row m exists.
// Epilogue operands that do not depend on the product, which the skinny kernel
// loads before or during its K loop: the residual values and next-norm gains of
// the thread's columns (EPI_RESID); the row's position and, once it has landed,
// the rotation of the thread's pair and the K/V page of the row's slot (EPI_QKV).
template <int NT> struct EpiPre {
  float res[NT];
  float g[NT];
  int pos;
  float cs, sn;   // EPI_QKV, q and k tiles: cos / sin of the thread's pair at pos
  int page;       // EPI_QKV, k and v tiles: page of the row's slot (-1: outside)
  int seq;        // EPI_QKV, k and v tiles: the row's sequence
  bool rot;       // cs, sn, page and seq are loaded
};

template <typename T, int NT, int EPI = -1>
UNO_DEV void epilogue(const GemmArgs& a, int m, int c, int tile0, int col_paired,
                      const float* v, float vp, bool ok, const EpiPre<NT>* pre = nullptr) {
  switch (EPI >= 0 ? EPI : a.epi) {
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
          const float xn = (pre ? pre->res[t] : a.resid[(size_t)m * a.ldo + col]) + v[t];
          a.resid[(size_t)m * a.ldo + col] = xn;
          if (a.xg_out) {
            const float gn = pre ? pre->g[t] : to_f(reinterpret_cast<const T*>(a.g_next)[col]);
            reinterpret_cast<T*>(a.xg_out)[act_off<T>(m, col, a.ldo)] = from_f<T>(xn * gn);
          }
          sq += xn * xn;
        }
      }
      if (a.ss_out) {
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 16);
        if (ok && c == 0) ss_add(a.ss_out, m, blockIdx.x, sq, a.err);
      }
      break;
    }
    case EPI_SWIGLU: {
      if (!ok) break;
      const float g = v[0], u = v[1];
      reinterpret_cast<T*>(a.out)[act_off<T>(m, col_paired + c, a.ldo)] =
          from_f<T>(g / (1.0f + expf(-g)) * u);
      break;
    }
    case EPI_QKV: {
      if (!ok) break;
      const int hd = a.kv.head_dim, half = hd / 2, tph = hd / 16;
      const int head = tile0 / tph, j = tile0 % tph;
      const int i = 8 * j + (c & 7);                 // pair index within the head
      const int dim = (c < 8) ? i : half + i;
      const int pos = pre ? pre->pos : a.row_pos[m];
      const bool rot = pre && pre->rot;
      const int Hq = a.n_q_heads, Hkv = a.kv.n_kv_heads;
      float val = v[0];
      if (head < Hq + Hkv) {                         // q or k: rotate the pair
        if (pos < 0 || pos >= a.kv.max_pages_per_seq * a.kv.page_size) {
          if (a.err) atomicOr(a.err, UNO_DEVERR_BOUNDS);
          break;
        }
        const float x1 = c < 8 ? v[0] : vp, x2 = c < 8 ? vp : v[0];
        const float cs = rot ? pre->cs : a.rcos[(size_t)pos * half + i];
        const float sn = rot ? pre->sn : a.rsin[(size_t)pos * half + i];
        val = (c < 8) ? x1 * cs - x2 * sn : x2 * cs + x1 * sn;
      }
      if (head < Hq) {
        reinterpret_cast<T*>(a.qbuf)[(size_t)m * Hq * hd + head * hd + dim] = from_f<T>(val);
      } else {
        const int which = head < Hq + Hkv ? 0 : 1;
        const int h = head - Hq - which * Hkv;
        const int seq = rot ? pre->seq : a.seq_fixed > 0 ? a.seq_fixed - 1 : a.call_seq[m / a.rows_per_seq];
        const int slot = a.row_slot ? a.row_slot[m] : pos;
        T* dst;
        if (rot) {
          if (pre->page < 0 && a.err) atomicOr(a.err, UNO_DEVERR_BOUNDS);
          dst = pre->page < 0 ? nullptr : kv_block<T>(a.kv, a.layer, which, pre->page, h);
        } else {
          dst = kv_dst<T>(a.kv, a.layer, which, seq, slot, h, a.err);
        }
        if (dst) dst[kv_elem(a.kv, which, slot % a.kv.page_size, dim)] = from_f<T>(val);
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

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
UNO_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One piece of a LoRA down-projection for a few rows: rank tile ct (16 columns of
// the nproj * r intermediate), K chunk kc, row tile mt.  The NW waves split the
// chunk's 32-wide K blocks; their partials are summed in LDS in wave order (red:
// NW rows of 256 floats, red_stride apart), scaled by the row's 1 / rms, and added
// to t in fixed point with one 64-bit integer atomic per element, so the total is
// exact and independent of the order the pieces land in.
template <int NW>
UNO_DEV void lora_down_piece(const LoraDownArgs& a, int ct, int kc, int mt, float* red,
                             int red_stride, float* s_rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r16 = lane & 15;
  const int col0 = ct * 16, p = col0 / a.r, lc = col0 % a.r, nkb = a.K / 32;
  // fragment-tiled operands: block (row block, k / 32), this lane's 16 bytes
  const bf16* Ap = reinterpret_cast<const bf16*>(a.A[p]) + (size_t)(lc / 16) * nkb * 512 + lane * 8;
  const int m_lane = mt * 16 + r16;
  const bool row_ok = m_lane < a.M;
  const bf16* Xp = reinterpret_cast<const bf16*>(a.X) + (size_t)mt * nkb * 512 + lane * 8;
  // row sums of x^2 (wave 0): lane l holds banks 4 (l % 4) .. +3 of row l / 4
  i64x2 ssq0 = {0, 0}, ssq1 = {0, 0};
  if (a.ss_in && w == 0 && mt * 16 + (lane >> 2) < a.M) {
    const i64x2* sp = reinterpret_cast<const i64x2*>(
        a.ss_in + (size_t)(mt * 16 + (lane >> 2)) * SS_BANKS + (lane & 3) * 4);
    ssq0 = sp[0];
    ssq1 = sp[1];
  }
  // this wave's share of the chunk's 32-wide K blocks, loaded four at a time
  const int cb = a.kchunk / 32, jb = kc * cb + w * cb / NW, je = kc * cb + (w + 1) * cb / NW;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero8 = {};
  for (int j = jb; j < je; j += 4) {
    bf16x8 x[4], wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = j + u < je;
      x[u] = (in && row_ok) ? load8(Xp + (size_t)(j + u) * 512) : zero8;
      wv[u] = in ? load8(Ap + (size_t)(j + u) * 512) : zero8;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[u], wv[u], acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[w * red_stride + ((lane >> 4) * 4 + i) * 16 + r16] = acc[i];
  if (w == 0) {
    long long sq = ssq0.x + ssq0.y + ssq1.x + ssq1.y;
    ss_check(ssq0.x | ssq0.y | ssq1.x | ssq1.y, a.err);
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    if ((lane & 3) == 0)
      s_rs[lane >> 2] = a.ss_in ? 1.0f / sqrtf(fx_to_float(sq) * a.inv_d + a.eps) : 1.0f;
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    const int e = threadIdx.x, row = e >> 4, m = mt * 16 + row;
    if (m < a.M) {
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) v += red[ww * red_stride + e];
      v *= s_rs[row];
      const long long q = (long long)llrintf(v * LORA_FX_SCALE);
      atomicAdd(reinterpret_cast<unsigned long long*>(a.t + (size_t)m * (a.nproj * a.r) + col0 + (e & 15)),
                (unsigned long long)q);
    }
  }
}

template <int NT, int WAVES, int KU>
__global__ void __launch_bounds__(WAVES * 64)
k_gemm_bf16(GemmArgs a) {
  static_assert(WAVES >= 4, "threads 0..255 own the 256 outputs of a tile");
  __shared__ float red[WAVES][NT][256];
  __shared__ float fin[256];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int mt = blockIdx.y;
  // fused LoRA down-projection: the first n_prod workgroups of the row tile produce
  // the intermediate, then publish it (release) by adding 1 to the launch counter
  // (The producers' only global writes are device-scope atomic adds, which the
  // device performs at its point of coherence across all XCDs -- the property every
  // multi-workgroup fixed-point sum of this library relies on.  Waiting for their
  // completion before the counter add orders them before it; no L2 write-back
  // fence is taken, which would stall the L2 the consumers are streaming through.)
  if ((int)blockIdx.x < a.n_prod) {
    const int nct = a.ld.nproj * a.ld.r / 16;
    lora_down_piece<WAVES>(a.ld, blockIdx.x % nct, blockIdx.x / nct, mt, &red[0][0][0], NT * 256, fin);
    wait_vmcnt<0>();                    // this thread's atomics are performed
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(a.sync + mt, 1u);
    return;
  }
  const int grp = blockIdx.x - a.n_prod;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int nkb = a.K / 32, nrb = a.r / 32;

  // this lane's fragment in block 0 of each tile's packed weight rows (and LoRA up)
  const bf16* Wp[NT];
  const bf16* Bp[NT];
  const long long* Up[NT];
  const bf16* Uu[NT];     // gated, scaled bf16 intermediate (large-M down-projection)
  int ldu[NT], ucol[NT];
  int tile0, col_paired = 0;
  if (a.paired) {
    col_paired = grp * 16;
    tile0 = grp;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const GemmSeg& sg = a.seg[t];
      Wp[t] = reinterpret_cast<const bf16*>(sg.W) + (size_t)grp * nkb * 512 + lane * 8;
      Bp[t] = sg.Bl ? reinterpret_cast<const bf16*>(sg.Bl) + (size_t)grp * nrb * 512 + lane * 8
                    : nullptr;
      Up[t] = sg.Ufx;
      Uu[t] = reinterpret_cast<const bf16*>(sg.U);
      ldu[t] = sg.ldu;
      ucol[t] = sg.ucol;
    }
  } else {
    tile0 = grp * NT;
    const GemmSeg& sg = a.seg[find_seg(a, tile0 * 16)];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int rb = tile0 + t - sg.n0 / 16;
      Wp[t] = reinterpret_cast<const bf16*>(sg.W) + (size_t)rb * nkb * 512 + lane * 8;
      Bp[t] = sg.Bl ? reinterpret_cast<const bf16*>(sg.Bl) + (size_t)rb * nrb * 512 + lane * 8
                    : nullptr;
      Up[t] = sg.Ufx;
      Uu[t] = reinterpret_cast<const bf16*>(sg.U);
      ldu[t] = sg.ldu;
      ucol[t] = sg.ucol;
    }
  }
  // every workgroup clears its share of a fixed-point buffer a later kernel fills
  if (a.zero_ptr) {
    const long ncons = (long)gridDim.x - a.n_prod;
    const long nwg = ncons * gridDim.y, wg = (long)blockIdx.y * ncons + grp;
    const long share = ((long)a.zero_n + nwg - 1) / nwg;
    const long z0 = wg * share, z1 = min((long)a.zero_n, z0 + share);
    for (long i = z0 + threadIdx.x; i < z1; i += WAVES * 64) a.zero_ptr[i] = 0;
  }

  const int m_lane = mt * 16 + r16;
  const bool row_ok = m_lane < a.M;
  const bf16* Xp = reinterpret_cast<const bf16*>(a.X) + (size_t)mt * nkb * 512 + lane * 8;

  // ---- operands that do not depend on the product, loaded before the K loop so
  // their latency hides behind the weight stream
  // (a) row sums of x^2: lane l holds banks 4 (l % 4) .. +3 of row l / 4 of the tile
  i64x2 ssq0 = {0, 0}, ssq1 = {0, 0};
  if (a.ss_in && mt * 16 + (lane >> 2) < a.M) {
    const i64x2* sp = reinterpret_cast<const i64x2*>(
        a.ss_in + (size_t)(mt * 16 + (lane >> 2)) * SS_BANKS + (lane & 3) * 4);
    ssq0 = sp[0];
    ssq1 = sp[1];
  }
  // (b) LoRA: wave w takes rank block w.  Its row's gate is read here; the raw
  // fixed-point t and the up-projection fragment are read after the weight stream
  // (a fused launch's intermediate is only ready then), which keeps their
  // registers free during the ring, so more workgroups fit a CU.
  // (four-tile LM-head instances have no adapter)
  constexpr bool kPreLora = NT <= 2;
  const bool fused = a.sync != nullptr;
  const bool lora_pre = kPreLora && a.r > 0 && w < nrb && Uu[0] == nullptr;
  bool gate_on = false;
  if (lora_pre) gate_on = row_ok && (a.gate == nullptr || a.gate[m_lane] != 0);
  // (c) epilogue operands of this thread's output element (threads 0..255)
  EpiPre<NT> pre{};
  {
    const int e = threadIdx.x & 255, m = mt * 16 + (e >> 4), c = e & 15;
    if (threadIdx.x < 256 && m < a.M) {
      if (a.epi == EPI_RESID) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int col = (tile0 + t) * 16 + c;
          pre.res[t] = a.resid[(size_t)m * a.ldo + col];
          pre.g[t] = a.xg_out ? to_f(reinterpret_cast<const bf16*>(a.g_next)[col]) : 0.0f;
        }
      } else if (a.epi == EPI_QKV) {
        pre.pos = a.row_pos[m];
      }
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- base phase: this wave's share of the 32-wide K blocks, streamed through
  // a ring of KU register slots.  Slot u is refilled with the block KU ahead as
  // soon as its MFMAs have issued, so KU blocks stay in flight up to the last
  // round, whose refills bring in the (je - jb) % KU trailing blocks.
  const int jb = w * nkb / WAVES, je = (w + 1) * nkb / WAVES;
  const int nfull = (je - jb) / KU, rem = (je - jb) % KU;
  const bf16x8 zero8 = {};
  bf16x8 ax[KU], bw[NT][KU];
  // Activation rows past M are the padding of a whole 16-row tile: an MFMA output
  // row depends on its own A row only, and those output rows are never stored.
  auto fill = [&](int u, int j) {
    ax[u] = load8(Xp + (size_t)j * 512);
#pragma unroll
    for (int t = 0; t < NT; ++t) bw[t][u] = load8_stream(Wp[t] + (size_t)j * 512);
  };
  auto consume = [&](int u) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[u], bw[t][u], acc[t], 0, 0, 0);
  };
  // q|k|v: the rotation and page loads depend on the row's position, so they go out
  // once the first ring round is in flight and land during the weight stream
  auto late_pre = [&]() {
    if (a.epi != EPI_QKV || threadIdx.x >= 256) return;
    const int e = threadIdx.x & 255, m = mt * 16 + (e >> 4), c = e & 15;
    if (m >= a.M) return;
    const int hd = a.kv.head_dim, half = hd / 2, tph = hd / 16;
    const int head = tile0 / tph, i = 8 * (tile0 % tph) + (c & 7);
    const int Hq = a.n_q_heads, Hkv = a.kv.n_kv_heads, pos = pre.pos;
    pre.cs = pre.sn = 0.0f;
    pre.page = -1;
    pre.seq = 0;
    if (head < Hq + Hkv && pos >= 0 && pos < a.kv.max_pages_per_seq * a.kv.page_size) {
      pre.cs = a.rcos[(size_t)pos * half + i];
      pre.sn = a.rsin[(size_t)pos * half + i];
    }
    if (head >= Hq) {
      pre.seq = a.seq_fixed > 0 ? a.seq_fixed - 1 : a.call_seq[m / a.rows_per_seq];
      pre.page = kv_page(a.kv, pre.seq, a.row_slot ? a.row_slot[m] : pos);
    }
    pre.rot = true;
  };
  int j = jb;
  if (nfull > 0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) fill(u, j + u);
    late_pre();
    for (int i = 1; i < nfull; ++i) {
      j += KU;
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        consume(u);
        fill(u, j + u);
      }
    }
    j += KU;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      consume(u);
      if (u < rem) fill(u, j + u);
    }
  } else {
#pragma unroll
    for (int u = 0; u < KU; ++u)
      if (u < rem) fill(u, j + u);
    late_pre();
  }
#pragma unroll
  for (int u = 0; u < KU; ++u)
    if (u < rem) consume(u);
  // ---- RMSNorm: scale rows of the base product by 1 / rms(x)
  if (a.ss_in) {
    long long sq = ssq0.x + ssq0.y + ssq1.x + ssq1.y;
    if (w == 0) ss_check(ssq0.x | ssq0.y | ssq1.x | ssq1.y, a.err);
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long long tot = __shfl(sq, ((lane >> 4) * 4 + i) * 4);
      const float rs = 1.0f / sqrtf(fx_to_float(tot) * a.inv_d + a.eps);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][i] *= rs;
    }
  }

  // ---- fused LoRA down-projection: wait until every producer of this row tile has
  // published its piece (bounded: a wait that runs out flags the context).  The
  // intermediate is then read with device-scope loads (below) rather than after an
  // acquire fence, which would invalidate the L2 lines other workgroups reuse.
  if (fused) {
    if (threadIdx.x == 0) {
      int spins = 0;
      while ((int)(__hip_atomic_load(a.sync + mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                   a.sync_target[mt]) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1 << 24)) {
          if (a.err) atomicOr(a.err, UNO_DEVERR_SYNC);
          break;
        }
      }
    }
    __syncthreads();
  }
  // the wave's first rank block: fixed-point t of its row and the LoRA-up fragment
  i64x2 tq[NT][4];
  bf16x8 bq[NT];
  if (lora_pre) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bq[t] = bf16x8{};
#pragma unroll
      for (int q = 0; q < 4; ++q) tq[t][q] = i64x2{0, 0};
      if (Up[t] == nullptr || Bp[t] == nullptr) continue;
      bq[t] = load8(Bp[t] + (size_t)w * 512);
      if (!gate_on) continue;
      const long long* tp = Up[t] + (size_t)m_lane * ldu[t] + w * 32 + kq;
      if (fused) {          // published by this launch's producers
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          tq[t][q].x = __hip_atomic_load(tp + 2 * q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          tq[t][q].y = __hip_atomic_load(tp + 2 * q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) tq[t][q] = reinterpret_cast<const i64x2*>(tp)[q];
      }
    }
  }
  // ---- LoRA phase: k over the rank, A = gate * bf16(scale * t), B = LoRA up
  if (a.r > 0 && !lora_pre) gate_on = row_ok && (a.gate == nullptr || a.gate[m_lane] != 0);
  if (lora_pre) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (Up[t] == nullptr || Bp[t] == nullptr) continue;
      bf16x8 af = zero8;
      if (gate_on) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          af[2 * q] = (bf16)(a.scale * fx_to_float(tq[t][q].x));
          af[2 * q + 1] = (bf16)(a.scale * fx_to_float(tq[t][q].y));
        }
      }
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq[t], acc[t], 0, 0, 0);
    }
  }
  if (a.r > 0) {
    for (int jr = lora_pre ? w + WAVES : w; jr < nrb; jr += WAVES) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if ((Up[t] == nullptr && Uu[t] == nullptr) || Bp[t] == nullptr) continue;
        bf16x8 af = zero8;
        if (Uu[t]) {
          if (row_ok) af = load8(Uu[t] + frag_off(m_lane, ucol[t] + jr * 32 + kq, ldu[t]));
        } else if (gate_on) {
          const long long* tp = Up[t] + (size_t)m_lane * ldu[t] + jr * 32 + kq;
          if (fused) {          // published by this launch's producers
#pragma unroll
            for (int e = 0; e < 8; ++e)
              af[e] = (bf16)(a.scale * fx_to_float(__hip_atomic_load(
                                  tp + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) af[e] = (bf16)(a.scale * fx_to_float(tp[e]));
          }
        }
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, load8(Bp[t] + (size_t)jr * 512),
                                                         acc[t], 0, 0, 0);
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
    else epilogue<bf16, NT>(a, m, c, tile0, col_paired, v, fin[row * 16 + (c ^ 8)], m < a.M, &pre);
  }
}


// Few-row product without a LoRA phase over 17..64 rows (the tree sampler's
// verify, verifies of two to four sequences): every weight block a wave streams
// is multiplied against the activations of all MT row tiles, so the weights are
// read from memory once per launch instead of once per 16-row tile.  Otherwise
// as k_gemm_bf16 (WAVES waves split K, KU blocks in flight per wave, fixed-order
// wave reduction in LDS, the same epilogues); row tiles past the rows are skipped.
template <int NT, int WAVES, int KU, int MT>
__global__ void __launch_bounds__(WAVES * 64)
k_gemm_bf16_rows(GemmArgs a) {
  static_assert(WAVES >= 4, "threads 0..255 own the 256 outputs of a tile");
  __shared__ float red[WAVES][MT][NT][256];
  __shared__ float fin[MT][256];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = blockIdx.x, mt0 = blockIdx.y * MT;
  const int mtiles = (a.M + 15) / 16;
  const int r16 = lane & 15;
  const int nkb = a.K / 32;
  const bf16* Wp[NT];
  int tile0, col_paired = 0;
  if (a.paired) {
    col_paired = grp * 16;
    tile0 = grp;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      Wp[t] = reinterpret_cast<const bf16*>(a.seg[t].W) + (size_t)grp * nkb * 512 + lane * 8;
  } else {
    tile0 = grp * NT;
    const GemmSeg& sg = a.seg[find_seg(a, tile0 * 16)];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      Wp[t] = reinterpret_cast<const bf16*>(sg.W) + (size_t)(tile0 + t - sg.n0 / 16) * nkb * 512 +
              lane * 8;
  }
  if (a.zero_ptr) {
    const long nwg = (long)gridDim.x * gridDim.y, wg = (long)blockIdx.y * gridDim.x + grp;
    const long share = ((long)a.zero_n + nwg - 1) / nwg;
    const long z0 = wg * share, z1 = min((long)a.zero_n, z0 + share);
    for (long i = z0 + threadIdx.x; i < z1; i += WAVES * 64) a.zero_ptr[i] = 0;
  }
  const bf16* Xp[MT];
  bool tile_ok[MT];
  i64x2 ssq0[MT], ssq1[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int mt = mt0 + mi;
    tile_ok[mi] = mt < mtiles;
    Xp[mi] = reinterpret_cast<const bf16*>(a.X) + (size_t)(tile_ok[mi] ? mt : 0) * nkb * 512 + lane * 8;
    ssq0[mi] = i64x2{0, 0};
    ssq1[mi] = i64x2{0, 0};
    if (a.ss_in && mt * 16 + (lane >> 2) < a.M) {
      const i64x2* sp = reinterpret_cast<const i64x2*>(
          a.ss_in + (size_t)(mt * 16 + (lane >> 2)) * SS_BANKS + (lane & 3) * 4);
      ssq0[mi] = sp[0];
      ssq1[mi] = sp[1];
    }
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mi][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int jb = w * nkb / WAVES, je = (w + 1) * nkb / WAVES;
  const int nfull = (je - jb) / KU, rem = (je - jb) % KU;
  const bf16x8 zero8 = {};
  bf16x8 ax[MT][KU], bw[NT][KU];
  auto fill = [&](int u, int j) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) ax[mi][u] = tile_ok[mi] ? load8(Xp[mi] + (size_t)j * 512) : zero8;
#pragma unroll
    for (int t = 0; t < NT; ++t) bw[t][u] = load8_stream(Wp[t] + (size_t)j * 512);
  };
  auto consume = [&](int u) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[mi][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[mi][u], bw[t][u], acc[mi][t], 0, 0, 0);
  };
  int j = jb;
  if (nfull > 0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) fill(u, j + u);
    for (int i = 1; i < nfull; ++i) {
      j += KU;
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        consume(u);
        fill(u, j + u);
      }
    }
    j += KU;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      consume(u);
      if (u < rem) fill(u, j + u);
    }
  } else {
#pragma unroll
    for (int u = 0; u < KU; ++u)
      if (u < rem) fill(u, j + u);
  }
#pragma unroll
  for (int u = 0; u < KU; ++u)
    if (u < rem) consume(u);
  if (a.ss_in) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      long long sq = ssq0[mi].x + ssq0[mi].y + ssq1[mi].x + ssq1[mi].y;
      if (w == 0) ss_check(ssq0[mi].x | ssq0[mi].y | ssq1[mi].x | ssq1[mi].y, a.err);
      sq += __shfl_xor(sq, 1);
      sq += __shfl_xor(sq, 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long tot = __shfl(sq, ((lane >> 4) * 4 + i) * 4);
        const float rs = 1.0f / sqrtf(fx_to_float(tot) * a.inv_d + a.eps);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mi][t][i] *= rs;
      }
    }
  }
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][mi][t][((lane >> 4) * 4 + i) * 16 + r16] = acc[mi][t][i];
  __syncthreads();
  const int e = threadIdx.x & 255;
  float v[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float sum = 0.0f;
      for (int ww = 0; ww < WAVES; ++ww) sum += red[ww][mi][t][e];
      v[mi][t] = sum;
    }
  if (threadIdx.x < 256)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) fin[mi][e] = v[mi][0];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int row = e >> 4, c = e & 15;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      if (!tile_ok[mi]) continue;
      const int m = (mt0 + mi) * 16 + row;
      if (a.epi == EPI_LOGITS) logits_epilogue<NT>(a, m, c, tile0, v[mi], m < a.M);
      else epilogue<bf16, NT>(a, m, c, tile0, col_paired, v[mi], fin[mi][row * 16 + (c ^ 8)], m < a.M);
    }
  }
}


// Eight consecutive finished columns col .. col+7 (col % 8 == 0) of row m of the
// large-M kernel: v holds them, vp the eight of columns col ^ 8 (the RoPE
// partners inside the 16-column tile).  Stores are 16 / 32 bytes wide.  EPI_RESID
// returns the eight x_new^2 summed (the caller reduces the row); LOGITS pairs with
// the neighbouring lane (lane ^ 1 holds the other half of the 16-column tile).
template <int EPI>
UNO_DEV float epilogue8(const GemmArgs& a, int m, int col, const float* v, const float* vp,
                        bool ok) {
  if (EPI == EPI_STORE_F32) {
    if (ok) {
      float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + (size_t)m * a.ldo + col);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    return 0.0f;
  }
  if (EPI == EPI_RESID) {
    if (!ok) return 0.0f;
    float4* r = reinterpret_cast<float4*>(a.resid + (size_t)m * a.ldo + col);
    const float4 r0 = r[0], r1 = r[1];
    float xn[8] = {r0.x + v[0], r0.y + v[1], r0.z + v[2], r0.w + v[3],
                   r1.x + v[4], r1.y + v[5], r1.z + v[6], r1.w + v[7]};
    r[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
    r[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
    float sq = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += xn[e] * xn[e];
    if (a.xg_out) {
      const bf16x8 gg = load8(reinterpret_cast<const bf16*>(a.g_next) + col);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)(xn[e] * (float)gg[e]);
      *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.xg_out) + frag_off(m, col, a.ldo)) = o;
    }
    return sq;
  }
  if (EPI == EPI_QKV) {
    if (!ok) return 0.0f;
    const int hd = a.kv.head_dim, half = hd / 2, tph = hd / 16;
    const int tile = col / 16, hi = (col / 8) & 1;
    const int head = tile / tph, j = tile % tph;
    const int dim0 = hi ? half + 8 * j : 8 * j;     // first of 8 consecutive dims
    const int pos = a.row_pos[m];
    const int Hq = a.n_q_heads, Hkv = a.kv.n_kv_heads;
    bf16x8 o;
    if (head < Hq + Hkv) {                          // q or k: rotate the pairs
      if (pos < 0 || pos >= a.kv.max_pages_per_seq * a.kv.page_size) {
        if (a.err) atomicOr(a.err, UNO_DEVERR_BOUNDS);
        return 0.0f;
      }
      const float* cr = a.rcos + (size_t)pos * half + 8 * j;
      const float* sr = a.rsin + (size_t)pos * half + 8 * j;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x1 = hi ? vp[e] : v[e], x2 = hi ? v[e] : vp[e];
        o[e] = (bf16)(hi ? x2 * cr[e] + x1 * sr[e] : x1 * cr[e] - x2 * sr[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    }
    if (head < Hq) {
      *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.qbuf) + (size_t)m * Hq * hd +
                                 head * hd + dim0) = o;
    } else {
      const int which = head < Hq + Hkv ? 0 : 1;
      const int h = head - Hq - which * Hkv;
      const int seq = a.seq_fixed > 0 ? a.seq_fixed - 1 : a.call_seq[m / a.rows_per_seq];
      const int slot = a.row_slot ? a.row_slot[m] : pos;
      bf16* blk = kv_dst<bf16>(a.kv, a.layer, which, seq, slot, h, a.err);
      if (!blk) return 0.0f;
      const int tk = slot % a.kv.page_size;
      if (which == 0) {
        *reinterpret_cast<bf16x8*>(blk + kv_elem(a.kv, 0, tk, dim0)) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) blk[kv_elem(a.kv, 1, tk, dim0 + e)] = o[e];
      }
    }
    return 0.0f;
  }
  if (EPI == EPI_LOGITS) {
    float l[8], mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      l[e] = (col + e == a.mask_col) ? -INFINITY : v[e];
      mx = fmaxf(mx, l[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    float se = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) se += (l[e] == -INFINITY) ? 0.0f : expf(l[e] - mx);
    se += __shfl_xor(se, 1);
    if (ok) {
      float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + (size_t)m * a.ldo + col);
      o[0] = make_float4(l[0], l[1], l[2], l[3]);
      o[1] = make_float4(l[4], l[5], l[6], l[7]);
      if (((col / 8) & 1) == 0) {
        a.tile_stats[((size_t)m * a.n_tiles + col / 16) * 2] = mx;
        a.tile_stats[((size_t)m * a.n_tiles + col / 16) * 2 + 1] = se;
      }
    }
    return 0.0f;
  }
  return 0.0f;
}

// ---------------------------------------------------------------------------
// Large-M variant (prefill, large batch, the distillation forward): a BM x BN
// output tile per workgroup of WM x WN wavefronts (each a (BM/WM) x (BN/WN) block
// of 16 x 16 MFMA tiles).  Operands move from HBM / L2 straight into LDS as whole
// 16 x 32 fragment blocks (global_load_lds_dwordx4: lane l's 16 bytes land at
// l * 16), so the LDS copy of a block is already in MFMA operand order and each
// lane reads its fragment back with one conflict-free 16-byte load.  A stage
// holds TKB consecutive 32-wide K blocks of the tile's BM / 16 activation blocks
// and BN / 16 weight blocks; TS stages form a ring, so TS - 1 stages are in flight
// while one is multiplied, with one barrier per stage.  The LoRA up-projection
// runs as further stages over the rank (A = the gated, scaled bf16 intermediate,
// fragment-tiled; B = the LoRA up rows).  Paired (SwiGLU) tiles interleave 16 gate
// rows and the matching 16 up rows, so a wavefront holds both halves of its
// outputs.  Workgroups of one column block are numbered onto one XCD (its L2 then
// serves that W tile to every row block).  The epilogue runs from the
// accumulators: in the MFMA layout the 16 lanes of a row group hold 16
// consecutive columns of one row, which is the epilogue's row group.
#ifndef UNO_TILE_TKB
#define UNO_TILE_TKB 2
#endif
constexpr int TKB = UNO_TILE_TKB;    // 32-wide K blocks per stage

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;


template <int BM, int BN, int WM, int WN, int TS>
constexpr size_t tile_smem_bytes() {
  const size_t ring = (size_t)TS * TKB * (BM + BN) / 16 * 1024;
  const size_t epi = (size_t)BM * (BN / WN + 4) * 4;
  return ring > epi ? ring : epi;
}

template <int BM, int BN, int WM, int WN, int TS, int EPI>
__global__ void __launch_bounds__(64 * WM * WN)
k_gemm_tile(GemmArgs a, int nbm, int nbn) {
  constexpr int NTH = 64 * WM * WN, TM = BM / WM, TN = BN / WN, NW = WM * WN;
  // gate/up pairs are interleaved in exactly the SwiGLU instantiations (the
  // launcher rejects any other combination)
  constexpr bool PAIRED = EPI == EPI_SWIGLU;
  constexpr int NBA = BM / 16, NBB = BN / 16, NBS = NBA + NBB;    // blocks per K block
  constexpr int NB = NBS * TKB;                                   // blocks per stage
  static_assert(NB % NW == 0, "every wave issues the same number of block loads");
  constexpr int P = NB / NW;                                      // block loads per wave and stage
  static_assert(TN % 32 == 0, "paired wave tiles hold whole gate/up pairs");
  static_assert(NTH >= BM, "one thread per tile row computes its norm");
  static_assert(TS >= 2 && TS <= 4, "ring depth");
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  __shared__ float s_rs[BM];

  const int nsl = ((EPI == EPI_TSLICE || EPI == EPI_STORE_F32) && a.k_slices > 1) ? a.k_slices : 1;
  const int total = nbm * nbn * nsl, per = (total + 7) / 8;
  const int t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= total) return;
  const int slice = t / (nbm * nbn), tt = t % (nbm * nbn);
  const int nb = tt / nbm, mb = tt % nbm;
  const int m0 = mb * BM;
  const int outc = PAIRED ? BN / 2 : BN;
  const int c0 = nb * outc;
  // the wave index is uniform: as a scalar it keeps the block addressing in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  const int r16 = lane & 15;
  const int nkb_all = a.K / 32, nkb = nkb_all / nsl, kb0 = slice * nkb, nrb = a.r / 32;
  const int mblocks = (a.M + 15) / 16;

  // every workgroup clears its share of a fixed-point buffer a later kernel fills
  if (a.zero_ptr) {
    const long share = ((long)a.zero_n + total - 1) / total;
    const long z0 = (long)t * share, z1 = min((long)a.zero_n, z0 + share);
    for (long i = z0 + tid; i < z1; i += NTH) a.zero_ptr[i] = 0;
  }
  // row norms of the tile (their loads complete before the block loads start, so
  // the ring's vmcnt accounting below only ever sees block loads)
  if (a.ss_in && tid < BM) s_rs[tid] = rs_of(a, m0 + tid);

  // weight row block of B block bi (16 rows) and its segment
  const int sg0 = PAIRED ? 0 : find_seg(a, c0);
  const int last_rb = (PAIRED ? a.seg[0].N : a.seg[sg0].N) / 16 - 1;
  auto brb = [&](int bi) {
    return min(PAIRED ? c0 / 16 + (bi >> 1) : (c0 - a.seg[sg0].n0) / 16 + bi, last_rb);
  };
  // Operand pointers as scalars (segments 0 and 1 when paired, the tile's segment
  // otherwise): nothing below indexes a.seg with a runtime value, which would make
  // the compiler copy the argument block into scratch.
  const bf16* const W0 = reinterpret_cast<const bf16*>(a.seg[sg0].W);
  const bf16* const W1 = PAIRED ? reinterpret_cast<const bf16*>(a.seg[1].W) : W0;
  const bf16* const B0 = reinterpret_cast<const bf16*>(a.seg[sg0].Bl);
  const bf16* const B1 = PAIRED ? reinterpret_cast<const bf16*>(a.seg[1].Bl) : B0;
  // LoRA passes: one per segment of the tile that has an adapter (pass p reads the
  // intermediate U_p at block column ucol_p of a row of ldu_p blocks)
  int lseg0 = 0, lseg1 = 0, nls = 0;
  const bf16 *U0 = nullptr, *U1 = nullptr;
  int ldu0 = 0, ldu1 = 0, uc0 = 0, uc1 = 0;
  if (a.r > 0 && slice == 0) {
#pragma unroll
    for (int k = 0; k < (PAIRED ? 2 : 1); ++k) {
      const GemmSeg& g = PAIRED ? a.seg[k] : a.seg[sg0];
      if (g.U && g.Bl) {
        if (nls == 0) { lseg0 = PAIRED ? k : sg0; U0 = reinterpret_cast<const bf16*>(g.U); ldu0 = g.ldu / 32; uc0 = g.ucol / 32; }
        else { lseg1 = k; U1 = reinterpret_cast<const bf16*>(g.U); ldu1 = g.ldu / 32; uc1 = g.ucol / 32; }
        ++nls;
      }
    }
  }
  const int n_base = nkb / TKB, spp = nrb / TKB;       // base stages, stages per LoRA pass
  const int nst = n_base + nls * spp;

  // block loads of stage st into ring slot `slot`: wave w loads blocks w * P .. + P - 1
  auto issue = [&](int st, int slot) {
    const int ls = st - n_base, pass = ls >= 0 ? ls / spp : 0;
    const bf16* const Up = pass == 0 ? U0 : U1;
    const int ldu = pass == 0 ? ldu0 : ldu1, uc = pass == 0 ? uc0 : uc1;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int bb = w * P + q, kk = bb / NBS, b = bb % NBS;
      const int mrow = min(m0 / 16 + b, mblocks - 1);
      const bool odd = PAIRED && ((b - NBA) & 1);      // the up half of a gate/up pair
      const bf16* src;
      if (ls < 0) {
        const int kb = kb0 + st * TKB + kk;
        if (b < NBA) src = reinterpret_cast<const bf16*>(a.X) + ((size_t)mrow * nkb_all + kb) * 512;
        else src = (odd ? W1 : W0) + ((size_t)brb(b - NBA) * nkb_all + kb) * 512;
      } else {
        const int jr = (ls % spp) * TKB + kk;
        if (b < NBA) src = Up + ((size_t)mrow * ldu + uc + jr) * 512;
        else src = (odd ? B1 : B0) + ((size_t)brb(b - NBA) * nrb + jr) * 512;
      }
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src + lane * 8),
                                       (lds_void_t*)(smem_raw + (slot * NB + bb) * 1024), 16, 0, 0);
    }
  };

  f32x4 acc[TM / 16][TN / 16];
#pragma unroll
  for (int i = 0; i < TM / 16; ++i)
#pragma unroll
    for (int j = 0; j < TN / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // RMSNorm: the base product's rows scale by 1 / rms(x) before the LoRA stages
  auto scale_rows = [&]() {
    if (!a.ss_in) return;
#pragma unroll
    for (int i = 0; i < TM / 16; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rs = s_rs[wm * TM + i * 16 + (lane >> 4) * 4 + e];
#pragma unroll
        for (int j = 0; j < TN / 16; ++j) acc[i][j][e] *= rs;
      }
  };

#pragma unroll
  for (int s = 0; s < TS - 1; ++s)
    if (s < nst) issue(s, s);
  for (int st = 0; st < nst; ++st) {
    // this wave's loads of stage st are done once at most the later stages' remain
    const int newer = min(TS - 2, nst - 1 - st);
    if (newer >= TS - 2) wait_vmcnt<(TS - 2) * P>();
    else if (newer == 2) wait_vmcnt<2 * P>();
    else if (newer == 1) wait_vmcnt<P>();
    else wait_vmcnt<0>();
    __syncthreads();          // every wave's loads of stage st landed; stage st - 1 consumed
    if (st + TS - 1 < nst) issue(st + TS - 1, (st + TS - 1) % TS);
    if (st == n_base) scale_rows();
    // in a paired LoRA pass only the wave's column blocks of that segment take part
    const int lsg = st < n_base ? -1 : (st - n_base) / spp == 0 ? lseg0 : lseg1;
#pragma unroll
    for (int kk = 0; kk < TKB; ++kk) {
      const char* base = smem_raw + ((st % TS) * NB + kk * NBS) * 1024 + lane * 16;
      bf16x8 af[TM / 16], bfr[TN / 16];
#pragma unroll
      for (int i = 0; i < TM / 16; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(base + (wm * (TM / 16) + i) * 1024);
#pragma unroll
      for (int j = 0; j < TN / 16; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(base + (NBA + wn * (TN / 16) + j) * 1024);
      // a paired LoRA pass adds its intermediate times the LoRA-up rows of its own
      // segment only: the other segment's column blocks (odd / even j, TN / 16 is
      // even) multiply a zero fragment, so the MFMA block stays branch-free
      if (PAIRED && lsg >= 0) {
#pragma unroll
        for (int j = 0; j < TN / 16; ++j)
          if ((j & 1) != lsg) bfr[j] = bf16x8{};
      }
#pragma unroll
      for (int i = 0; i < TM / 16; ++i)
#pragma unroll
        for (int j = 0; j < TN / 16; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  if (nst == n_base) scale_rows();
  __syncthreads();            // the ring is free for the epilogue

  // epilogue: one column slice of BN / WN at a time is staged in LDS (fp32) by the
  // wavefronts that own it; then each thread finishes items of 8 consecutive
  // columns of one row (16 / 32-byte stores).  A thread keeps the same rows in
  // every slice, so RESID sums each row's squares in registers and adds them once.
  constexpr int TNP = TN + 4;                          // padded row: rows 4 banks apart
  float* sC = reinterpret_cast<float*>(smem_raw);     // [BM][TNP]
  constexpr int IPR = (EPI == EPI_SWIGLU ? TN / 2 : TN) / 8;     // items per row
  constexpr int ITEMS = BM * IPR / NTH;
  static_assert(ITEMS * NTH == BM * IPR && NTH % IPR == 0, "epilogue items");
  float rsq[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) rsq[k] = 0.0f;
  for (int pass = 0; pass < WN; ++pass) {
    if (wn == pass) {
#pragma unroll
      for (int i = 0; i < TM / 16; ++i)
#pragma unroll
        for (int j = 0; j < TN / 16; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sC[(wm * TM + i * 16 + (lane >> 4) * 4 + e) * TNP + j * 16 + r16] = acc[i][j][e];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int it = tid + NTH * k, row = it / IPR, cl = (it % IPR) * 8, m = m0 + row;
      const float* fr = sC + row * TNP;
      float v[8], vp[8];
      if (EPI == EPI_TSLICE || EPI == EPI_STORE_F32) {
        if (m < a.M) {
          float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + (size_t)slice * a.slice_stride +
                                                (size_t)m * a.ldo + c0 + pass * TN + cl);
          o[0] = make_float4(fr[cl], fr[cl + 1], fr[cl + 2], fr[cl + 3]);
          o[1] = make_float4(fr[cl + 4], fr[cl + 5], fr[cl + 6], fr[cl + 7]);
        }
      } else if (EPI == EPI_SWIGLU) {
        // slice column pairs: 16 gate | 16 up per 16 outputs
        const int q = cl / 16, h8 = cl % 16;
        float g[8], u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { g[e] = fr[q * 32 + h8 + e]; u[e] = fr[q * 32 + 16 + h8 + e]; }
        if (m < a.M) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)(g[e] / (1.0f + expf(-g[e])) * u[e]);
          const int col = c0 + (pass * TN) / 2 + cl;
          *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.out) + frag_off(m, col, a.ldo)) = o;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { v[e] = fr[cl + e]; vp[e] = fr[(cl ^ 8) + e]; }
        const int col = c0 + pass * TN + cl;
        const bool in_cols = EPI != EPI_LOGITS || col < a.n_tiles * 16;
        rsq[k] += epilogue8<EPI>(a, m, col, v, vp, m < a.M && in_cols);
      }
    }
    __syncthreads();
  }
  if (EPI == EPI_RESID && a.ss_out) {
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      float sq = rsq[k];
#pragma unroll
      for (int off = IPR / 2; off > 0; off >>= 1) sq += __shfl_xor(sq, off, IPR);
      const int it = tid + NTH * k, m = m0 + it / IPR;
      if (it % IPR == 0 && m < a.M) ss_add(a.ss_out, m, blockIdx.x, sq, a.err);
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
  else epilogue<float, NT>(a, m, c, tile0, col_paired, v, fin[row * 16 + (c ^ 8)], ok);
}

// LoRA down-projection for a few rows: a workgroup of LD_WAVES wavefronts per
// (16 columns, K chunk, 16 rows).  The wavefronts split the chunk, their partials
// are summed in LDS in wave order, and the chunk's sum (times rs for a normalised
// input) is added to t in fixed point with one 64-bit integer atomic per element,
// so the total is exact and independent of the order the chunks land in.
constexpr int LD_WAVES = 8;

__global__ void __launch_bounds__(64 * LD_WAVES)
k_lora_down(LoraDownArgs a) {
  __shared__ float red[LD_WAVES][256];
  __shared__ float s_rs[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r16 = lane & 15;
  const int col0 = blockIdx.x * 16, kc = blockIdx.y, mt = blockIdx.z;
  const int p = col0 / a.r, lc = col0 % a.r, nkb = a.K / 32;
  // fragment-tiled operands: block (row block, k / 32), this lane's 16 bytes
  const bf16* Ap = reinterpret_cast<const bf16*>(a.A[p]) + (size_t)(lc / 16) * nkb * 512 + lane * 8;
  const int m_lane = mt * 16 + r16;
  const bool row_ok = m_lane < a.M;
  const bf16* Xp = reinterpret_cast<const bf16*>(a.X) + (size_t)mt * nkb * 512 + lane * 8;
  // row sums of x^2 (wave 0): lane l holds banks 4 (l % 4) .. +3 of row l / 4
  i64x2 ssq0 = {0, 0}, ssq1 = {0, 0};
  if (a.ss_in && w == 0 && mt * 16 + (lane >> 2) < a.M) {
    const i64x2* sp = reinterpret_cast<const i64x2*>(
        a.ss_in + (size_t)(mt * 16 + (lane >> 2)) * SS_BANKS + (lane & 3) * 4);
    ssq0 = sp[0];
    ssq1 = sp[1];
  }
  // this wave's share of the chunk's 32-wide K blocks, loaded four at a time
  const int cb = a.kchunk / 32, jb = kc * cb + w * cb / LD_WAVES, je = kc * cb + (w + 1) * cb / LD_WAVES;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero8 = {};
  for (int j = jb; j < je; j += 4) {
    bf16x8 x[4], wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = j + u < je;
      x[u] = (in && row_ok) ? load8(Xp + (size_t)(j + u) * 512) : zero8;
      wv[u] = in ? load8(Ap + (size_t)(j + u) * 512) : zero8;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[u], wv[u], acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[w][((lane >> 4) * 4 + i) * 16 + r16] = acc[i];
  if (w == 0) {
    long long sq = ssq0.x + ssq0.y + ssq1.x + ssq1.y;
    ss_check(ssq0.x | ssq0.y | ssq1.x | ssq1.y, a.err);
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    if ((lane & 3) == 0)
      s_rs[lane >> 2] = a.ss_in ? 1.0f / sqrtf(fx_to_float(sq) * a.inv_d + a.eps) : 1.0f;
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    const int e = threadIdx.x, row = e >> 4, m = mt * 16 + row;
    if (m < a.M) {
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < LD_WAVES; ++ww) v += red[ww][e];
      v *= s_rs[row];
      const long long q = (long long)llrintf(v * LORA_FX_SCALE);
      atomicAdd(reinterpret_cast<unsigned long long*>(a.t + (size_t)m * (a.nproj * a.r) + col0 + (e & 15)),
                (unsigned long long)q);
    }
  }
}

// Sum of the K-slice partials of the large-M down-projection, gated and scaled to
// the bf16 operand of the LoRA up-projection: eight columns per thread.
__global__ void __launch_bounds__(256)
k_lora_u(const float* __restrict__ t, int n_slices, long long stride, int M, int ncols,
         const uint8_t* __restrict__ gate, float scale, bf16* __restrict__ u) {
  const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
  const int per_row = ncols / 8;
  if (i >= (long)M * per_row) return;
  const int m = (int)(i / per_row), c = (int)(i % per_row) * 8;
  const size_t off = (size_t)m * ncols + c;
  bf16x8 o = {};
  if (gate == nullptr || gate[m] != 0) {
    float acc[8];
    const float4* p = reinterpret_cast<const float4*>(t + off);
    const float4 p0 = p[0], p1 = p[1];
    acc[0] = p0.x; acc[1] = p0.y; acc[2] = p0.z; acc[3] = p0.w;
    acc[4] = p1.x; acc[5] = p1.y; acc[6] = p1.z; acc[7] = p1.w;
    for (int sl = 1; sl < n_slices; ++sl) {
      const float4* q = reinterpret_cast<const float4*>(t + (size_t)sl * stride + off);
      const float4 q0 = q[0], q1 = q[1];
      acc[0] += q0.x; acc[1] += q0.y; acc[2] += q0.z; acc[3] += q0.w;
      acc[4] += q1.x; acc[5] += q1.y; acc[6] += q1.z; acc[7] += q1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)(scale * acc[e]);
  }
  *reinterpret_cast<bf16x8*>(u + frag_off(m, c, ncols)) = o;
}

__global__ void k_zero_i64(long long* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

// The residual epilogue of a K-split large-M product: row m, eight columns per
// thread, x_new = resid + the slices' partial sums added in slice order; stores
// x_new, the next norm's input bf16(x_new * g) (fragment-tiled) and adds the
// workgroup's share of the row's x_new^2 to one bank of its fixed-point sum.
__global__ void __launch_bounds__(256)
k_resid_slices(const float* __restrict__ part, int n_slices, long long stride, int N,
               float* __restrict__ resid, bf16* __restrict__ xg_out, const bf16* __restrict__ g_next,
               long long* __restrict__ ss_out, int32_t* err) {
  __shared__ float s_sq[4];
  const int m = blockIdx.y, col = (blockIdx.x * 256 + threadIdx.x) * 8;
  float sq = 0.0f;
  if (col < N) {
    const size_t off = (size_t)m * N + col;
    float4* r = reinterpret_cast<float4*>(resid + off);
    const float4 r0 = r[0], r1 = r[1];
    float xn[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float v[8];
    {
      const float4* p = reinterpret_cast<const float4*>(part + off);
      const float4 p0 = p[0], p1 = p[1];
      v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
      v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
    }
    for (int sl = 1; sl < n_slices; ++sl) {
      const float4* p = reinterpret_cast<const float4*>(part + (size_t)sl * stride + off);
      const float4 p0 = p[0], p1 = p[1];
      v[0] += p0.x; v[1] += p0.y; v[2] += p0.z; v[3] += p0.w;
      v[4] += p1.x; v[5] += p1.y; v[6] += p1.z; v[7] += p1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) xn[e] += v[e];
    r[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
    r[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += xn[e] * xn[e];
    if (xg_out) {
      const bf16x8 gg = load8(g_next + col);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)(xn[e] * (float)gg[e]);
      *reinterpret_cast<bf16x8*>(xg_out + frag_off(m, col, N)) = o;
    }
  }
  if (ss_out == nullptr) return;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
  if ((threadIdx.x & 63) == 0) s_sq[threadIdx.x >> 6] = sq;
  __syncthreads();
  if (threadIdx.x == 0) ss_add(ss_out, m, blockIdx.x, s_sq[0] + s_sq[1] + s_sq[2] + s_sq[3], err);
}

hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.kchunk <= 0 || a.K % a.kchunk || a.kchunk % 32 || a.r % 16) return hipErrorInvalidValue;
  dim3 grid(a.nproj * a.r / 16, a.K / a.kchunk, (a.M + 15) / 16);
  uno_launch(k_lora_down, grid, 64 * LD_WAVES, 0, s, a);
  return hipGetLastError();
}

bool launch_tile(const GemmArgs& a, int n_cols_total, hipStream_t s, hipError_t* err);

// Large-M LoRA down-projection: the tile kernel with K split into k_slices
// slices (a power of two up to 8, aiming at four workgroups per CU), each slice
// storing its float partial; k_lora_u adds them in slice order.
#ifndef UNO_LORA_TILE_TARGET
#define UNO_LORA_TILE_TARGET 1024
#endif
int lora_down_tile_slices(int M, int K, int ncols) {
  const long tiles = (long)((M + 127) / 128) * (ncols / 128);
  int S = 1;
  // at most 8 slices: at 2048 rows 16 slices of int64 partials cost more traffic
  // than their extra workgroups gain
  while (S < 8 && tiles * S < UNO_LORA_TILE_TARGET && (K / 32) % (2 * S) == 0 && K / 32 / (2 * S) >= 4)
    S *= 2;
  return S;
}

hipError_t launch_lora_u(const float* t, int n_slices, long long stride, int M, int ncols,
                         const uint8_t* gate, float scale, bf16* u, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (ncols % 8 || n_slices < 1) return hipErrorInvalidValue;
  const long n = (long)M * (ncols / 8);
  uno_launch(k_lora_u, (unsigned)((n + 255) / 256), 256, 0, s, t, n_slices, stride, M, ncols, gate,
             scale, u);
  return hipGetLastError();
}

bool lora_down_tile_fits(int M, int K, int ncols, int k_slices) {
  return M >= 64 && k_slices >= 1 && K % (32 * k_slices) == 0 && ncols % 128 == 0;
}

hipError_t launch_lora_down_tile(const GemmArgs& a, int ncols, hipStream_t s) {
  if (a.epi != EPI_TSLICE || a.r != 0 || !lora_down_tile_fits(a.M, a.K, ncols, a.k_slices))
    return hipErrorInvalidValue;
  hipError_t e;
  if (!launch_tile(a, ncols, s, &e)) return hipErrorInvalidValue;
  return e;
}

hipError_t launch_zero_i64(long long* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  uno_launch(k_zero_i64, blocks, 256, 0, s, p, n);
  return hipGetLastError();
}

// Large-M tile choice: the biggest tile that still gives every CU a workgroup and
// whose column blocks do not straddle a segment boundary.  Returns false when no
// tile fits (the skinny kernel then runs).
template <int BM, int BN, int WM, int WN, int TS, int EPI>
hipError_t run_tile(const GemmArgs& a, int n_cols_total, hipStream_t s) {
  const int outc = a.paired ? BN / 2 : BN;
  const int nbm = (a.M + BM - 1) / BM, nbn = (n_cols_total + outc - 1) / outc;
  const int nsl = ((EPI == EPI_TSLICE || EPI == EPI_STORE_F32) && a.k_slices > 1) ? a.k_slices : 1;
  const int grid = (nbm * nbn * nsl + 7) / 8 * 8;
  constexpr size_t smem = tile_smem_bytes<BM, BN, WM, WN, TS>();
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_tile<BM, BN, WM, WN, TS, EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  uno_launch(k_gemm_tile<BM, BN, WM, WN, TS, EPI>, grid, 64 * WM * WN, (uint32_t)smem, s, a, nbm, nbn);
  return hipGetLastError();
}

bool tile_fits(const GemmArgs& a, int n_cols_total, int BN) {
  const int outc = a.paired ? BN / 2 : BN;
  // logits of one segment may end in a ragged tile (its missing weight rows are
  // never stored: the kernel re-reads the last row block and drops the columns)
  if (a.epi == EPI_LOGITS && !a.paired && a.nseg == 1 && a.seg[0].n0 == 0 &&
      a.seg[0].N == n_cols_total && n_cols_total % 16 == 0)
    return true;
  if (n_cols_total % outc) return false;
  if (!a.paired)
    for (int i = 0; i < a.nseg; ++i)
      if (a.seg[i].n0 % BN || a.seg[i].N % BN) return false;
  return true;
}

#ifndef UNO_TILE_MIN_WG
#define UNO_TILE_MIN_WG 192
#endif
#ifndef UNO_TILE_TS1
#define UNO_TILE_TS1 3
#endif
#ifndef UNO_TILE_TS3
#define UNO_TILE_TS3 2
#endif
constexpr int kTileMinWG = UNO_TILE_MIN_WG;   // workgroups a larger tile must still give
constexpr int kTileTS1 = UNO_TILE_TS1;        // ring depth of the 256 x 128 tile
constexpr int kTileTS3 = UNO_TILE_TS3;        // ring depth of the 128 x 128 tile
// template arguments <BM, BN, WM, WN, TS> of the 256 x 256 and 256 x 128 tiles
#ifndef UNO_TILE_CFG0
#define UNO_TILE_CFG0 256, 256, 4, 4, 2
#endif
#ifndef UNO_TILE_CFG1
#define UNO_TILE_CFG1 256, 128, 4, 2, kTileTS1
#endif
#ifndef UNO_TILE_TALL_FIRST
#define UNO_TILE_TALL_FIRST 0
#endif
constexpr bool kTileTallFirst = UNO_TILE_TALL_FIRST;   // 128 x 256 before 256 x 128

// A residual product whose 256 x 256 tiles number at least 64 but fewer than
// kTileMinWG: S K slices of those tiles (S = 2 from 128 tiles, else 4) store float
// partials in the caller's workspace, then k_resid_slices adds them and runs the
// residual epilogue (measured on the o and down projections of the 8B shape at
// 2048 rows and in 1024-row prefill: faster than 256 x 128 tiles without a
// split).  False: not applicable.
bool launch_resid_split(const GemmArgs& a, int n_cols_total, hipStream_t s, hipError_t* err) {
  if (a.epi != EPI_RESID || !a.split_ws || a.paired || a.nseg != 1) return false;
  if (a.seg[0].Ufx && a.seg[0].Bl) return false;
  if (!tile_fits(a, n_cols_total, 256)) return false;
  const long tiles = (long)((a.M + 255) / 256) * (n_cols_total / 256);
  if (tiles < 64 || tiles >= kTileMinWG) return false;
  const int S = tiles >= 128 ? 2 : 4;
  if ((a.K / 32) % (S * TKB) || (a.r / 32) % TKB || a.ldo != n_cols_total || n_cols_total % 8) return false;
  const long long stride = (long long)a.M * n_cols_total;
  if (S * stride > a.split_cap) return false;
  GemmArgs b = a;
  b.epi = EPI_STORE_F32;
  b.out = a.split_ws;
  b.k_slices = S;
  b.slice_stride = stride;
  b.resid = nullptr;
  b.xg_out = nullptr;
  b.ss_out = nullptr;
  *err = run_tile<UNO_TILE_CFG0, EPI_STORE_F32>(b, n_cols_total, s);
  if (*err != hipSuccess) return true;
  uno_launch(k_resid_slices, dim3((n_cols_total / 8 + 255) / 256, a.M), 256, 0, s, a.split_ws, S, stride,
             n_cols_total, a.resid, reinterpret_cast<bf16*>(a.xg_out), reinterpret_cast<const bf16*>(a.g_next),
             a.ss_out, a.err);
  *err = hipGetLastError();
  return true;
}

bool launch_tile(const GemmArgs& a, int n_cols_total, hipStream_t s, hipError_t* err) {
  if (a.K % 32 || a.r % 32) return false;
  const int nsl = (a.epi == EPI_TSLICE && a.k_slices > 1) ? a.k_slices : 1;
  if (a.K % (32 * nsl) || (a.K / 32 / nsl) % TKB || (a.r / 32) % TKB) return false;
  // the tile kernel takes its LoRA intermediate as fragment-tiled bf16 only
  for (int i = 0; i < a.nseg; ++i)
    if (a.seg[i].Ufx && a.seg[i].Bl) return false;
  if (a.paired != (a.epi == EPI_SWIGLU)) return false;
  auto blocks = [&](int BM, int BN) {
    const int outc = a.paired ? BN / 2 : BN;
    return (long)((a.M + BM - 1) / BM) * ((n_cols_total + outc - 1) / outc) * nsl;
  };
  // the largest tile that still gives three quarters of the CUs a workgroup (the
  // 256-row tiles fill a CU's LDS alone), else the largest that gives half of
  // them one, else the 128 x 128 tile, whose two-stage ring lets two workgroups
  // share a CU (measured at batch 128, in 1024-row prefill and in the
  // distillation forward: at 2048 rows q|k|v keeps 256 x 256 on 192 workgroups,
  // o and down take 256 x 128 on 256 rather than 256 x 256 on 128)
  const bool f256 = tile_fits(a, n_cols_total, 256), f128 = tile_fits(a, n_cols_total, 128);
  int cfg = -1;
  for (const long want : {(long)kTileMinWG, 128L}) {
    if (f256 && blocks(256, 256) >= want) cfg = 0;
    else if (kTileTallFirst && f256 && blocks(128, 256) >= want) cfg = 2;
    else if (f128 && blocks(256, 128) >= want) cfg = 1;
    else if (f256 && blocks(128, 256) >= want) cfg = 2;
    if (cfg >= 0) break;
  }
  if (cfg < 0 && f128) cfg = 3;
  else if (cfg < 0 && f256) cfg = 2;
  if (cfg < 0) return false;
#define UNO_TILE_EPI(E)                                                          \
  case E:                                                                        \
    switch (cfg) {                                                               \
      case 0: *err = run_tile<UNO_TILE_CFG0, E>(a, n_cols_total, s); break;     \
      case 1: *err = run_tile<UNO_TILE_CFG1, E>(a, n_cols_total, s); break;     \
      case 2: *err = run_tile<128, 256, 2, 4, 3, E>(a, n_cols_total, s); break;  \
      default: *err = run_tile<128, 128, 2, 2, kTileTS3, E>(a, n_cols_total, s); break; \
    }                                                                            \
    return true;
  switch (a.epi) {
    UNO_TILE_EPI(EPI_STORE_F32)
    UNO_TILE_EPI(EPI_RESID)
    UNO_TILE_EPI(EPI_SWIGLU)
    UNO_TILE_EPI(EPI_LOGITS)
    UNO_TILE_EPI(EPI_QKV)
    UNO_TILE_EPI(EPI_TSLICE)
    default: return false;
  }
#undef UNO_TILE_EPI
}

#ifndef UNO_SK_GATEUP
#define UNO_SK_GATEUP 2, 4, 4
#endif
#ifndef UNO_SK_QKV
#define UNO_SK_QKV 1, 8, 2
#endif
#ifndef UNO_SK_O
#define UNO_SK_O 1, 12, 2
#endif
#ifndef UNO_SK_LMHEAD
#define UNO_SK_LMHEAD 2, 4, 8
#endif
#ifndef UNO_SK_DOWN
#define UNO_SK_DOWN 1, 12, 2
#endif

// One skinny launch: WAVES waves splitting K, KU blocks in flight per wave; a
// workgroup owns NT tiles of 16 columns (paired: the gate and up tiles of 16
// output columns).
template <int NT, int WAVES, int KU>
hipError_t launch_skinny(const GemmArgs& a, int n_cols_total, int mtiles, hipStream_t s) {
  const int per_wg = a.paired ? 16 : 16 * NT;
  if (n_cols_total % per_wg) return hipErrorInvalidValue;
  if (a.n_prod > 0) {
    // the producers' pieces must tile the intermediate and the chunks whole K blocks
    const LoraDownArgs& l = a.ld;
    if (!a.sync || l.r % 16 || l.kchunk <= 0 || l.kchunk % 32 || l.K % l.kchunk ||
        a.n_prod != l.nproj * l.r / 16 * (l.K / l.kchunk) || l.M != a.M || mtiles > 4)
      return hipErrorInvalidValue;
  }
  uno_launch(k_gemm_bf16<NT, WAVES, KU>, dim3(a.n_prod + n_cols_total / per_wg, mtiles),
             WAVES * 64, 0, s, a);
  return hipGetLastError();
}

// Few-row launch without a LoRA phase over MT = 4 row tiles per workgroup.
template <int NT, int WAVES, int KU>
hipError_t launch_skinny_rows(const GemmArgs& a, int n_cols_total, int mtiles, hipStream_t s) {
  const int per_wg = a.paired ? 16 : 16 * NT;
  if (n_cols_total % per_wg) return hipErrorInvalidValue;
  uno_launch(k_gemm_bf16_rows<NT, WAVES, KU, 4>, dim3(n_cols_total / per_wg, (mtiles + 3) / 4),
             WAVES * 64, 0, s, a);
  return hipGetLastError();
}

template <>
hipError_t launch_gemm<bf16>(const GemmArgs& a, int n_cols_total, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % 32 != 0 || (a.r % 32) != 0 || n_cols_total % 16 != 0) return hipErrorInvalidValue;
  if (a.epi == EPI_QKV && (a.kv.head_dim % 16 != 0)) return hipErrorInvalidValue;
  if (a.n_prod > 0 && a.M >= 64) return hipErrorInvalidValue;   // fused producers: skinny only
  if (a.M >= 64) {
    hipError_t e;
    if (launch_resid_split(a, n_cols_total, s, &e)) return e;
    if (launch_tile(a, n_cols_total, s, &e)) return e;
  }
  const int mtiles = (a.M + 15) / 16;
  const int nkb = a.K / 32;
  // 17..64 rows without a LoRA phase: the weights are streamed once for all row
  // tiles (shapes as the single-tile launches below, but two-tile workgroups keep
  // 2 blocks in flight per wave so that their registers allow every gate/up
  // workgroup to be resident at once)
  if (mtiles > 1 && a.r == 0 && a.n_prod == 0 && nkb >= 64) {
    if (a.paired) return launch_skinny_rows<2, 4, 2>(a, n_cols_total, mtiles, s);
    if (a.epi == EPI_LOGITS && n_cols_total % 32 == 0 && a.nseg == 1)
      return launch_skinny_rows<2, 4, 2>(a, n_cols_total, mtiles, s);
    if (a.epi == EPI_QKV) return launch_skinny_rows<UNO_SK_QKV>(a, n_cols_total, mtiles, s);
    return launch_skinny_rows<UNO_SK_O>(a, n_cols_total, mtiles, s);
  }
  // Launch shapes measured at the 8B decode shapes (one MI355X): many small
  // workgroups beat few large ones -- the paired gate/up tiles at 4 waves of 4
  // blocks in flight, q|k|v at 8 waves of 2, o at 12 of 2, down at 12 of 2, the LM
  // head at two 16-column tiles per workgroup of 4 waves of 8.
  if (a.paired) {
    if (nkb >= 64) return launch_skinny<UNO_SK_GATEUP>(a, n_cols_total, mtiles, s);
    return launch_skinny<2, 4, 1>(a, n_cols_total, mtiles, s);
  }
  if (a.epi == EPI_LOGITS && n_cols_total % 32 == 0 && a.nseg == 1 && nkb >= 32)
    return launch_skinny<UNO_SK_LMHEAD>(a, n_cols_total, mtiles, s);
  if (nkb >= 64) {
    if (a.epi == EPI_QKV) return launch_skinny<UNO_SK_QKV>(a, n_cols_total, mtiles, s);
    if (nkb >= 256) return launch_skinny<UNO_SK_DOWN>(a, n_cols_total, mtiles, s);
    return launch_skinny<UNO_SK_O>(a, n_cols_total, mtiles, s);
  }
  return launch_skinny<1, 4, 1>(a, n_cols_total, mtiles, s);
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
