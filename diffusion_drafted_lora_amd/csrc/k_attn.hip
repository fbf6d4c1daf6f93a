// Block-causal attention over the paged KV cache shared by draft and verify.
//
// Method: draft and verify read one KV cache (shibing624 reading notes of the Uno
// paper, method core); a row at position m attends to its sequence's committed
// context plus the in-flight block up to itself, i.e. positions 0..m, because
// every block row's K/V is written at its position before attention runs.  The
// distillation forward over [x, z1] (same notes, "Diffusion Distillation") uses
// per-row windows instead: an x row sees x up to itself, a z1 row of block b sees
// the clean blocks before b and z1 of block b up to itself.
//
// Split-context decomposition: a workgroup owns (sequence, KV head, 16-row tile,
// context chunk); the G = Hq / Hkv query heads of its KV head and the 16 rows
// share each K/V load.  The chunk is walked in 32-key sub-chunks with an online
// softmax; the partial (max, sum, unnormalised output) of every chunk is merged
// by a second kernel in chunk order (deterministic).
#include "uno_internal.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
UNO_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int SUB = 32;   // keys per LDS sub-chunk
constexpr int kMaxCombine = 64;   // chunk partials merged per (row, head)

// Visible-slot window (a, c, d) of row r: slots [0, a) and [c, d].
UNO_DEV void row_window(const AttnArgs& a, int r, bool ok, int* av, int* cv, int* dv) {
  *av = 0; *cv = INT_MAX; *dv = -1;
  if (!ok) return;
  if (a.row_vis) {
    *av = a.row_vis[3 * (size_t)r];
    *cv = a.row_vis[3 * (size_t)r + 1];
    *dv = a.row_vis[3 * (size_t)r + 2];
  } else {
    *av = a.row_pos[r] + 1;
  }
}

// Keys of a 16-row tile: virtual index p < A is slot p, p >= A is slot C + p - A.
// sw holds a[16], c[16], d[16].  The second range starts at or after A.
UNO_DEV void tile_window(const int* sw, int* A, int* C, int* nv) {
  int am = 0, cm = INT_MAX, dm = -1;
  for (int i = 0; i < 16; ++i) {
    am = max(am, sw[i]);
    if (sw[16 + i] <= sw[32 + i]) { cm = min(cm, sw[16 + i]); dm = max(dm, sw[32 + i]); }
  }
  cm = max(cm, am);
  *A = am;
  *C = cm;
  *nv = am + (dm >= cm ? dm - cm + 1 : 0);
}

UNO_DEV int vslot(int p, int A, int C) { return p < A ? p : C + (p - A); }
UNO_DEV bool seen(int sl, int av, int cv, int dv) { return sl < av || (sl >= cv && sl <= dv); }

// Every row's chunk count, written once per tile (chunk 0, KV head 0) for the
// combine; a window longer than n_chunks chunks trips the bounds flag.
UNO_DEV void publish_nc(const AttnArgs& a, int c, int kvh, int tid, int r0, int nrows, int nv) {
  if (c != 0 || kvh != 0 || tid >= nrows) return;
  const int nc = (nv + a.chunk - 1) / a.chunk;
  a.row_nc[r0 + tid] = min(nc, a.n_chunks);
  if (nc > a.n_chunks && a.err) atomicOr(a.err, UNO_DEVERR_BOUNDS);
}

template <typename T, int MAXO>
__global__ void __launch_bounds__(256)
k_attn_partial(AttnArgs a, KvLayout kv) {
  extern __shared__ float smem[];
  const int c = blockIdx.x, kvh = blockIdx.y;
  const int row_tiles = (a.rows_per_seq + 15) / 16;
  const int si = blockIdx.z / row_tiles, rt = blockIdx.z % row_tiles;
  const int Hkv = kv.n_kv_heads, hd = kv.head_dim, G = a.n_q_heads / Hkv;
  const int seq = a.seq_fixed > 0 ? a.seq_fixed - 1 : a.call_seq[si];
  const int r0 = si * a.rows_per_seq + rt * 16;
  const int nrows = min(16, a.rows_per_seq - rt * 16);
  const int NQ = 16 * G;               // query vectors of this block
  const int kstride = hd + 2;          // padded LDS row (in T elements)

  float* sQ = smem;                                  // [NQ][hd]
  float* sS = sQ + NQ * hd;                          // [NQ][SUB]
  float* sM = sS + NQ * SUB;                         // [NQ] running max
  float* sL = sM + NQ;                               // [NQ] running sum
  float* sF = sL + NQ;                               // [NQ] rescale factor
  int* sW = reinterpret_cast<int*>(sF + NQ);         // [3][16] row windows
  T* sK = reinterpret_cast<T*>(sW + 48);             // [SUB][kstride]
  T* sV = sK + SUB * kstride;                        // [SUB][kstride]

  const int tid = threadIdx.x;
  if (tid < 16) row_window(a, r0 + tid, tid < nrows, sW + tid, sW + 16 + tid, sW + 32 + tid);
  __syncthreads();
  int At, Ct, nv;
  tile_window(sW, &At, &Ct, &nv);
  publish_nc(a, c, kvh, tid, r0, nrows, nv);
  const int kbeg = c * a.chunk;
  if (kbeg >= nv) return;              // no row sees this chunk (never combined)
  const int kend = min(kbeg + a.chunk, nv);

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

  for (int k0 = kbeg; k0 < kend; k0 += SUB) {
    __syncthreads();
    // load K / V of virtual keys k0 .. k0+SUB-1 (only keys < kend are read)
    for (int e = tid; e < SUB * hd; e += 256) {
      const int j = e / hd, d = e % hd, p = k0 + j, sl = vslot(p, At, Ct);
      T kvk = from_f<T>(0.0f), kvv = from_f<T>(0.0f);
      const int page = p < kend ? kv_page(kv, seq, sl) : -1;
      if (page >= 0) {
        const int tk = sl % kv.page_size;
        kvk = kv_block<const T>(kv, a.layer, 0, page, kvh)[kv_elem(kv, 0, tk, d)];
        kvv = kv_block<const T>(kv, a.layer, 1, page, kvh)[kv_elem(kv, 1, tk, d)];
      }
      sK[j * kstride + d] = kvk;
      sV[j * kstride + d] = kvv;
    }
    __syncthreads();
    // scores
    for (int e = tid; e < NQ * SUB; e += 256) {
      const int qi = e / SUB, j = e % SUB, p = k0 + j, rw = qi % 16;
      float s = -INFINITY;
      if (p < kend && seen(vslot(p, At, Ct), sW[rw], sW[16 + rw], sW[32 + rw])) {
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

// Merge the chunk partials of one (row, head) in chunk order.  Every load goes
// out at once: wave 0 lane c takes chunk c's (max, sum), thread (half, d) takes
// dimension d of chunks 32 half .. 32 half + 31; wave 0 then forms the chunk
// weights (max and sum by a fixed shuffle tree), each thread sums its chunks in
// order and the two halves are added in LDS (half 0 + half 1).
template <typename T>
__global__ void __launch_bounds__(256)
k_attn_combine(AttnArgs a, int hd) {
  static_assert(kMaxCombine == 64, "one wave lane per chunk, two halves of 32");
  __shared__ float sf[kMaxCombine];
  __shared__ float sL;
  __shared__ float sh[128];
  const int r = blockIdx.x / a.n_q_heads, h = blockIdx.x % a.n_q_heads;
  const int nc = a.row_nc[r];
  const size_t ph0 = ((size_t)r * a.n_q_heads + h) * a.n_chunks;
  const int lane = threadIdx.x & 63, half = threadIdx.x >> 7, dl = threadIdx.x & 127;
  float mc = -INFINITY, sc = 0.0f;
  if (threadIdx.x < 64 && lane < nc) {
    mc = a.part_ml[(ph0 + lane) * 2];
    sc = a.part_ml[(ph0 + lane) * 2 + 1];
  }
  for (int d0 = 0; d0 < hd; d0 += 128) {
    const int d = d0 + dl, c0 = half * 32;
    const float* po = a.part_o + (ph0 + c0) * hd + d;
    float v[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) v[c] = (c0 + c < nc && d < hd) ? po[(size_t)c * hd] : 0.0f;
    if (d0 == 0) {
      if (threadIdx.x < 64) {
        float M = mc;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float f = (mc == -INFINITY) ? 0.0f : expf(mc - M);
        float L = sc * f;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
        sf[lane] = f;
        if (lane == 0) sL = L;
      }
      __syncthreads();
    }
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c)
      if (c0 + c < nc) acc += v[c] * sf[c0 + c];
    if (half == 1) sh[dl] = acc;
    __syncthreads();
    if (half == 0 && d < hd) {
      const float inv = sL > 0.0f ? 1.0f / sL : 0.0f;
      reinterpret_cast<T*>(a.out)[act_off<T>(r, h * hd + d, a.n_q_heads * hd)] =
          from_f<T>((acc + sh[dl]) * inv);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA variant (head_dim 128).  Wave g of the workgroup owns query head
// kvh * G + g for the tile's 16 rows.  Per 64-key sub-chunk: K (row-major) and
// V (transposed) are staged in LDS; S = Q K^T on v_mfma_f32_16x16x32_bf16 with Q
// held in registers; the online softmax runs in the accumulator layout (lane l
// holds rows 4*(l/16)+i of column l%16); P goes through LDS to become the A
// operand of P V.  Output accumulators share the row layout of S, so the
// rescale by exp(m_old - m_new) needs no data movement.
#ifndef UNO_ATTN_MK
#define UNO_ATTN_MK 64
#endif
constexpr int MK = UNO_ATTN_MK;   // keys per sub-chunk
static_assert(MK == 32 || MK == 64, "sub-chunks of 32 or 64 keys");
#ifndef UNO_ATTN_PF
#define UNO_ATTN_PF 2
#endif
constexpr int PFD = UNO_ATTN_PF;  // sub-chunks fetched ahead (register sets in turn)
static_assert(PFD == 1 || PFD == 2, "prefetch one or two sub-chunks ahead");
constexpr int HD = 128;           // head dim of the MFMA path
constexpr int KPAD = HD + 8;      // LDS row of K (bf16), 16-byte pad
constexpr int VPAD = MK + 8;      // LDS row of V^T (bf16)
constexpr int PPAD = MK + 8;      // LDS row of P (bf16)
constexpr int PGC = 1024;         // block-table entries cached per workgroup

// WIN: rows carry visibility windows (keys map to slots through two ranges);
// without, rows are plain causal and key p is slot p, so a V piece of eight
// aligned keys always lies in one page and needs no per-element path.
#ifndef UNO_ATTN_MIN_WAVES
#define UNO_ATTN_MIN_WAVES 2
#endif
template <bool WIN>
__global__ void __launch_bounds__(256, UNO_ATTN_MIN_WAVES)
k_attn_mfma(AttnArgs a, KvLayout kv) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  bf16* sK = reinterpret_cast<bf16*>(smem_raw);                 // [MK][KPAD]
  bf16* sVt = sK + MK * KPAD;                                   // [HD][VPAD]
  bf16* sP = sVt + HD * VPAD;                                   // [G][16][PPAD]
  __shared__ int sW[48];                                        // row windows a, c, d
  __shared__ int sPg[PGC];                                      // pages of the chunk's slots

  const int c = blockIdx.x, kvh = blockIdx.y;
  const int row_tiles = (a.rows_per_seq + 15) / 16;
  const int si = blockIdx.z / row_tiles, rt = blockIdx.z % row_tiles;
  const int Hkv = kv.n_kv_heads, G = a.n_q_heads / Hkv;
  const int seq = a.seq_fixed > 0 ? a.seq_fixed - 1 : a.call_seq[si];
  const int r0 = si * a.rows_per_seq + rt * 16;
  const int nrows = min(16, a.rows_per_seq - rt * 16);
  // one wave per query head of the KV head's group: G = 4 waves (checked at launch)
  constexpr int nthr = 256;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;

  // Loads that do not depend on each other go out together: row windows, the Q
  // fragments of this wave's head, and (below, for plain causal rows whose keys
  // are slots 0..pos) the first sub-chunk's K/V.
  if (tid < 16) row_window(a, r0 + tid, tid < nrows, sW + tid, sW + 16 + tid, sW + 32 + tid);
  const int kbeg = c * a.chunk;
  int kend = kbeg + MK;      // provisional bound of the first sub-chunk
  int At = INT_MAX, Ct = 0;  // identity key numbering until the windows are known
  const int head = kvh * G + w;
  const bf16* Q = reinterpret_cast<const bf16*>(a.q);
  bf16x8 qf[HD / 32];
  {
    const bool ok = r16 < nrows;
    const bf16* qr = Q + (size_t)(r0 + (ok ? r16 : 0)) * a.n_q_heads * HD + head * HD;
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + ks * 32 + grp * 8);
      qf[ks] = ok ? v : bf16x8{};
    }
  }
  // scores are scaled into the exp2 domain
  const float sc = a.scale * 1.4426950408889634f;

  float m[4], l[4];
  f32x4 o[HD / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.0f; }
#pragma unroll
  for (int d = 0; d < HD / 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16* myP = sP + w * 16 * PPAD;
  // K / V of a 64-key sub-chunk in 16-byte pieces, prefetched into registers two
  // sub-chunks ahead.  K piece e: key e / 16, dims (e % 16) * 8 .. +7 (a token row).
  // V piece e: dim (e % 256) / 2, keys ((e / 256) * 2 + e % 2) * 8 .. +7 (the V block
  // is dim-major, so eight consecutive tokens of one dim are 16 contiguous bytes;
  // pieces whose eight keys are not eight aligned slots of one page go by element).
  constexpr int PF_MAX = MK * (HD / 8) / 256;          // 4 for >= 256 threads
  const int npf = (MK * (HD / 8) + nthr - 1) / nthr;
  // pages are a power of two of slots (checked at launch): slot sl lies in page
  // entry sl >> psh at offset sl & pmask; a page's block of this layer and KV head
  // is pstride elements after the previous page's
  const int psh = kv.page_shift, pmask = kv.page_size - 1;
  const size_t pstride = (size_t)kv.n_kv_heads * kv.page_size * HD;
  const bf16* kb0 = kv_block<const bf16>(kv, a.layer, 0, 0, kvh);
  const bf16* vb0 = kv_block<const bf16>(kv, a.layer, 1, 0, kvh);
  const int32_t* bt = kv.block_table + (size_t)seq * kv.max_pages_per_seq;
  // block-table entry of slot sl, or -1 outside the sequence's reserved pages
  auto bt_page = [&](int sl) {
    const int pi = sl >> psh;
    if (sl < 0 || pi >= kv.max_pages_per_seq) return -1;
    const int page = bt[pi];
    return (page >= 0 && page < kv.n_pages) ? page : -1;
  };
  // two register sets in turn: sub-chunk i + 2 is fetched while i is multiplied
  bf16x8 pkA[PF_MAX], pvA[PF_MAX], pkB[PF_MAX], pvB[PF_MAX];
  // page of a slot: from the LDS copy of the chunk's block-table entries once it
  // is published (pages pl .. pl + npg - 1), else from the block table
  int pl = 0, npg = 0;
  auto page_of = [&](int sl) {
    const int pi = (sl >> psh) - pl;
    return (pi >= 0 && pi < npg) ? sPg[pi] : bt_page(sl);
  };
  auto fetch = [&](int k0, bf16x8 (&pk)[PF_MAX], bf16x8 (&pv)[PF_MAX]) {
#pragma unroll
    for (int q = 0; q < PF_MAX; ++q) {
      const int e = tid + q * nthr;
      bf16x8 kk = {}, vv = {};
      if (q < npf && e < MK * (HD / 8)) {
        const int key = e / (HD / 8), d8 = (e % (HD / 8)) * 8, p = k0 + key;
        const int sl = vslot(p, At, Ct);
        const int page = p < kend ? page_of(sl) : -1;
        if (page >= 0)
          kk = *reinterpret_cast<const bf16x8*>(kb0 + (size_t)page * pstride + (sl & pmask) * HD + d8);
        const int jj = (e >> 8) * 2 + (e & 1), d = (e & 255) >> 1, p0 = k0 + jj * 8;
        const int s0 = vslot(p0, At, Ct);
        if (!WIN || (p0 + 7 < kend && s0 % 8 == 0 && vslot(p0 + 7, At, Ct) == s0 + 7)) {
          const int pg = page_of(s0);
          if (pg >= 0)
            vv = *reinterpret_cast<const bf16x8*>(vb0 + (size_t)pg * pstride + (d << psh) + (s0 & pmask));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int pj = p0 + j, sj = vslot(pj, At, Ct);
            const int pg = pj < kend ? page_of(sj) : -1;
            if (pg >= 0) vv[j] = vb0[(size_t)pg * pstride + (d << psh) + (sj & pmask)];
          }
        }
      }
      pk[q] = kk;
      pv[q] = vv;
    }
  };
  // Keys at or beyond kend are staged as zeros: masked keys get probability 0, and
  // 0 * V must stay 0 (a slot that was never written may hold a NaN pattern).
  auto stage = [&](int k0, const bf16x8 (&pk)[PF_MAX], const bf16x8 (&pv)[PF_MAX]) {
#pragma unroll
    for (int q = 0; q < PF_MAX; ++q) {
      const int e = tid + q * nthr;
      if (q < npf && e < MK * (HD / 8)) {
        const int key = e / (HD / 8), d8 = (e % (HD / 8)) * 8;
        *reinterpret_cast<bf16x8*>(sK + key * KPAD + d8) = k0 + key < kend ? pk[q] : bf16x8{};
        const int jj = (e >> 8) * 2 + (e & 1), d = (e & 255) >> 1;
        bf16x8 vv = pv[q];
        if (k0 + MK > kend) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (k0 + jj * 8 + j >= kend) vv[j] = (bf16)0.0f;
        }
        *reinterpret_cast<bf16x8*>(sVt + d * VPAD + jj * 8) = vv;
      }
    }
  };
  // first sub-chunk of plain causal rows: slots beyond the rows are read (from
  // reserved pages only) and zeroed at staging; this keeps the window reads off
  // the critical path
  const bool causal = !WIN;
  if (causal) fetch(kbeg, pkA, pvA);
  __syncthreads();
  int nv;
  tile_window(sW, &At, &Ct, &nv);
  publish_nc(a, c, kvh, tid, r0, nrows, nv);
  if (kbeg >= nv) return;
  kend = min(kbeg + a.chunk, nv);
  // block-table entries of every slot the chunk reads (two slot ranges: keys
  // below At are slots themselves, the rest start at slot Ct); published by the
  // loop's first barrier
  int npg_all = 0;
  {
    int lo = INT_MAX, hi = -1;
    if (kbeg < At) { lo = kbeg; hi = min(kend, At) - 1; }
    if (kend > At) {
      const int b = max(kbeg, At);
      lo = min(lo, Ct + b - At);
      hi = max(hi, Ct + kend - 1 - At);
    }
    // (the first PFD sub-chunks are fetched below, before the copy is published,
    // so a chunk of at most PFD sub-chunks never reads it)
    if (hi >= lo && lo >= 0 && kend - kbeg > PFD * MK) {
      const int p0 = lo >> psh, p1 = hi >> psh;
      if (p1 - p0 + 1 <= PGC) { pl = p0; npg_all = p1 - p0 + 1; }
    }
    for (int i = tid; i < npg_all; i += nthr) sPg[i] = bt_page((pl + i) << psh);
  }
  if (!causal) fetch(kbeg, pkA, pvA);
  if (PFD == 2 && kbeg + MK < kend) fetch(kbeg + MK, pkB, pvB);
  npg = npg_all;
  int ra[4], rc[4], rd[4], lim[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = sW[grp * 4 + i];
    rc[i] = sW[16 + grp * 4 + i];
    rd[i] = sW[32 + grp * 4 + i];
    lim[i] = min(kend, ra[i]);
  }
  for (int k0 = kbeg, it = 0; k0 < kend; k0 += MK, ++it) {
    __syncthreads();               // previous sub-chunk fully consumed
    if (PFD == 1) {
      stage(k0, pkA, pvA);
      if (k0 + MK < kend) fetch(k0 + MK, pkA, pvA);
    } else if (it & 1) {
      stage(k0, pkB, pvB);
      if (k0 + 2 * MK < kend) fetch(k0 + 2 * MK, pkB, pvB);
    } else {
      stage(k0, pkA, pvA);
      if (k0 + 2 * MK < kend) fetch(k0 + 2 * MK, pkA, pvA);
    }
    __syncthreads();
    // S = Q K^T for 4 key tiles of 16
    f32x4 s[MK / 16];
#pragma unroll
    for (int j = 0; j < MK / 16; ++j) {
      s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(sK + (j * 16 + r16) * KPAD + ks * 32 + grp * 8);
        s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kb, s[j], 0, 0, 0);
      }
    }
    // mask, online softmax (rows 4*grp+i, column = key j*16 + r16)
    int ksl[MK / 16];
#pragma unroll
    for (int j = 0; j < MK / 16; ++j) {
      const int p = k0 + j * 16 + r16;
      ksl[j] = WIN ? (p < kend ? vslot(p, At, Ct) : INT_MAX) : p;
    }
    float mt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < MK / 16; ++j) {
        float v = s[j][i] * sc;
        // plain causal rows: keys are slots and row i sees slots below ra[i]
        const bool vis = WIN ? (ksl[j] != INT_MAX && seen(ksl[j], ra[i], rc[i], rd[i]))
                             : ksl[j] < lim[i];
        if (!vis) v = -INFINITY;
        s[j][i] = v;
        mx = fmaxf(mx, v);
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
      mt[i] = mx;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(m[i], mt[i]);
      const float f = (m[i] == -INFINITY) ? 0.0f : exp2f(m[i] - mn);
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < MK / 16; ++j) {
        const float pv = (s[j][i] == -INFINITY) ? 0.0f : exp2f(s[j][i] - mn);
        s[j][i] = pv;
        ps += pv;
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) ps += __shfl_xor(ps, off, 16);
      l[i] = l[i] * f + ps;
      m[i] = mn;
#pragma unroll
      for (int d = 0; d < HD / 16; ++d) o[d][i] *= f;
    }
    // P to LDS (bf16), row-major [16][MK]
#pragma unroll
    for (int j = 0; j < MK / 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) myP[(grp * 4 + i) * PPAD + j * 16 + r16] = (bf16)s[j][i];
    __syncthreads();
    // O += P V
#pragma unroll
    for (int ks = 0; ks < MK / 32; ++ks) {
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(myP + r16 * PPAD + ks * 32 + grp * 8);
#pragma unroll
      for (int d = 0; d < HD / 16; ++d) {
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(sVt + (d * 16 + r16) * VPAD + ks * 32 + grp * 8);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[d], 0, 0, 0);
      }
    }
  }
  // partials (or the final output when the context has one chunk)
  const bool single = a.n_chunks == 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = grp * 4 + i;
    if (row >= nrows) continue;
    const size_t rr = (size_t)(r0 + row);
    if (single) {
      const float inv = l[i] > 0.0f ? 1.0f / l[i] : 0.0f;
      bf16* out = reinterpret_cast<bf16*>(a.out);
#pragma unroll
      for (int d = 0; d < HD / 16; ++d)
        out[frag_off((int)rr, head * HD + d * 16 + r16, a.n_q_heads * HD)] = (bf16)(o[d][i] * inv);
    } else {
      const size_t ph = (rr * a.n_q_heads + head) * a.n_chunks + c;
#pragma unroll
      for (int d = 0; d < HD / 16; ++d) a.part_o[ph * HD + d * 16 + r16] = o[d][i];
      if (r16 == 0) {
        // stats in the natural-log domain, as the combine expects
        a.part_ml[ph * 2] = m[i] * 0.6931471805599453f;
        a.part_ml[ph * 2 + 1] = l[i];
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Plain-causal bf16 attention (head_dim 128, four query heads per KV head,
// 16-token pages) that streams K and V straight from the pages into a ring of
// RNS LDS stages with global_load_lds -- no register staging -- so RNS - 1
// sub-chunks of RMK keys are in flight while one is multiplied, with one barrier
// per sub-chunk.  Each 1 KB load instruction fills 64 16-byte LDS slots; the
// lanes pick their global chunks so that the stage is XOR-swizzled and every
// MFMA fragment read is free of bank conflicts:
//   K, key t of the sub-chunk, dims 8c..8c+7:  t * 256 + ((c ^ (t & 15)) * 16)
//   V, page p of the sub-chunk, dim d, tokens 8h..8h+7 of the page:
//                                              RMK * 256 + p * 4096 + d * 32 + ((h ^ ((d >> 3) & 1)) * 16)
// Keys at or past the chunk end are loaded from page 0 (in bounds, never seen):
// their scores are masked, and their V entries are zeroed in LDS before P.V (a
// slot that was never written may hold a NaN pattern, and 0 * NaN is NaN).
#ifndef UNO_ATTN_RING
#define UNO_ATTN_RING 2
#endif
#ifndef UNO_ATTN_RING_KEYS
#define UNO_ATTN_RING_KEYS 64
#endif
constexpr int RNS = UNO_ATTN_RING;              // ring stages
constexpr int RMK = UNO_ATTN_RING_KEYS;         // keys per stage
static_assert(RMK == 32 || RMK == 64, "stages of 32 or 64 keys");
constexpr int RPG = RMK / 16;                   // pages per stage
constexpr int RPPAD = RMK + 8;                  // LDS row of P (bf16)
#ifndef UNO_ATTN_RING_MIN_CHUNK
#define UNO_ATTN_RING_MIN_CHUNK 64
#endif
constexpr int kAttnRingMinChunk = UNO_ATTN_RING_MIN_CHUNK;   // shorter chunks: register staging
static_assert(RNS >= 2 && RNS <= 4, "ring depth");
constexpr int RSTAGE = RMK * HD * 2 * 2;        // one stage: K and V of RMK keys
constexpr int RVOFF = RMK * HD * 2;             // V part of a stage

// Windowed rows (WIN: the distillation forward's [x, z1] rows, the tree verify's
// chains) number their keys in whole pages: virtual pages below A16 = A rounded up
// to a page are the slots' own pages, the rest continue at the page of C rounded
// down (A = max a, C = min c, over the tile's rows).  The two ranges may share a
// page; each occurrence of a slot is masked by its own range -- slot < a in the
// first, c <= slot <= d in the second -- so no row sees a slot twice.
//
// RT row tiles per workgroup (RT x 4 waves; wave w takes query head w % 4 of its
// KV head and row tile w / 4 of the group): the tiles share every K/V stage, so
// long row sets (prefill, the distillation forward) stream their keys once per
// RT * 16 rows.  The keys walked are the union of the group's rows' windows.
template <bool WIN, int RT>
__global__ void __launch_bounds__(256 * RT, 1)
k_attn_ring(AttnArgs a, KvLayout kv) {
  constexpr int NWV = 4 * RT, NTH = 256 * RT, NR = 16 * RT;
  constexpr int RL = RSTAGE / 1024 / NWV;       // 1 KB load instructions per wave and stage
  static_assert(RL >= 1 && RL * NWV * 1024 == RSTAGE, "stage loads split evenly over the waves");
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  bf16* sP = reinterpret_cast<bf16*>(smem_raw + (size_t)RNS * RSTAGE);   // [NWV][16][RPPAD]
  __shared__ int sW[3 * NR];
  __shared__ int sPg[PGC];

  const int c = blockIdx.x, kvh = blockIdx.y;
  const int row_tiles = (a.rows_per_seq + 15) / 16, groups = (row_tiles + RT - 1) / RT;
  const int si = blockIdx.z / groups, tg = blockIdx.z % groups;
  const int G = 4;
  const int seq = a.seq_fixed > 0 ? a.seq_fixed - 1 : a.call_seq[si];
  const int rg0 = tg * NR;                                   // first row of the group
  const int r0g = si * a.rows_per_seq + rg0;
  const int nrows_g = min(NR, a.rows_per_seq - rg0);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, grp = lane >> 4;
  const int wt = w >> 2;                                     // this wave's row tile
  const int r0 = r0g + wt * 16;
  const int nrows = max(0, min(16, nrows_g - wt * 16));

  if (tid < NR) row_window(a, r0g + tid, tid < nrows_g, sW + tid, sW + NR + tid, sW + 2 * NR + tid);
  const int head = kvh * G + (w & 3);
  const bf16* Q = reinterpret_cast<const bf16*>(a.q);
  bf16x8 qf[HD / 32];
  {
    const bool ok = r16 < nrows;
    const bf16* qr = Q + (size_t)(r0 + (ok ? r16 : 0)) * a.n_q_heads * HD + head * HD;
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + ks * 32 + grp * 8);
      qf[ks] = ok ? v : bf16x8{};
    }
  }
  const float sc = a.scale * 1.4426950408889634f;    // scores in the exp2 domain
  // plain rows: the pages of the chunk's whole key range go out with the row and
  // query loads (virtual page p is the sequence's page p); which of them the rows
  // see is settled below.  Entries past the sequence's table read as -1.
  const int32_t* bt = kv.block_table + (size_t)seq * kv.max_pages_per_seq;
  const int p0 = (c * a.chunk) >> 4;
  constexpr int PPT = (PGC + NTH - 1) / NTH;
  int praw[PPT];
  if (!WIN) {
    const int npg_max = a.chunk >> 4;          // the launcher keeps a.chunk <= PGC * 16
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int i = tid + k * NTH;
      praw[k] = (i < npg_max && p0 + i < kv.max_pages_per_seq) ? bt[p0 + i] : -1;
    }
  }
  __syncthreads();
  int A16 = 0, C16 = 0, Am = 0, nv;
  if (WIN) {
    int am = 0, cm = INT_MAX, dm = -1;
    for (int i = 0; i < NR; ++i) {
      am = max(am, sW[i]);
      if (sW[NR + i] <= sW[2 * NR + i]) { cm = min(cm, sW[NR + i]); dm = max(dm, sW[2 * NR + i]); }
    }
    // tile-wide values: scalars (every lane computed the same)
    Am = __builtin_amdgcn_readfirstlane(am);
    A16 = (Am + 15) & ~15;
    C16 = __builtin_amdgcn_readfirstlane(dm >= cm ? (cm & ~15) : A16);
    nv = __builtin_amdgcn_readfirstlane(A16 + (dm >= cm ? dm - C16 + 1 : 0));
  } else {
    int am = 0;
    for (int i = 0; i < NR; ++i) am = max(am, sW[i]);
    nv = __builtin_amdgcn_readfirstlane(am);
  }
  publish_nc(a, c, kvh, tid, r0g, nrows_g, nv);
  const int kbeg = c * a.chunk;
  if (kbeg >= nv) return;
  const int kend = min(kbeg + a.chunk, nv);
  const int nsub = (kend - kbeg + RMK - 1) / RMK;

  // pages of the chunk's keys (kbeg is a multiple of 64, so of the page size);
  // entries outside the sequence's pages read page 0 (masked / zeroed below)
  const int npg = nsub * RPG;
  if (WIN) {
    for (int i = tid; i < npg; i += NTH) {
      const int vp = p0 + i;
      const int pi = vp >= (A16 >> 4) ? (C16 >> 4) + vp - (A16 >> 4) : vp;
      int page = (pi < kv.max_pages_per_seq && (vp << 4) < kend) ? bt[pi] : 0;
      sPg[i] = (page >= 0 && page < kv.n_pages) ? page : 0;
    }
  } else {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int i = tid + k * NTH;
      if (i < npg) {
        const int page = ((p0 + i) << 4) < kend ? praw[k] : 0;
        sPg[i] = (page >= 0 && page < kv.n_pages) ? page : 0;
      }
    }
  }
  const size_t pstride = (size_t)kv.n_kv_heads * 16 * HD;
  const bf16* kb0 = kv_block<const bf16>(kv, a.layer, 0, 0, kvh);
  const bf16* vb0 = kv_block<const bf16>(kv, a.layer, 1, 0, kvh);
  __syncthreads();

  // wave w issues the stage's load instructions w * RL .. + RL - 1: first the K
  // pages (four instructions of four tokens each), then the V pages (four
  // instructions of 32 dims each)
  auto issue = [&](int sub, int slot) {
#pragma unroll
    for (int q = 0; q < RL; ++q) {
      const int ins = w * RL + q, kind = ins / (4 * RPG), pg = (ins % (4 * RPG)) >> 2,
                part = ins & 3;
      const int page = sPg[sub * RPG + pg];
      const bf16* src;
      if (kind == 0) {
        const int tl = part * 4 + grp, cq = r16 ^ tl;      // token of the page, its data chunk
        src = kb0 + (size_t)page * pstride + tl * HD + cq * 8;
      } else {
        const int d = part * 32 + (lane >> 1), h = (lane & 1) ^ ((d >> 3) & 1);
        src = vb0 + (size_t)page * pstride + d * 16 + h * 8;
      }
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)src,
          (lds_void_t*)(smem_raw + (size_t)slot * RSTAGE + kind * RVOFF + pg * 4096 + part * 1024),
          16, 0, 0);
    }
  };

  float m[4], l[4];
  f32x4 o[HD / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.0f; }
#pragma unroll
  for (int d = 0; d < HD / 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  int lim[4], wc[4], wd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ri = wt * 16 + grp * 4 + i;                  // row of the group
    lim[i] = WIN ? sW[ri] : min(kend, sW[ri]);
    wc[i] = WIN ? sW[NR + ri] : 0;
    wd[i] = WIN ? sW[2 * NR + ri] : 0;
  }
  bf16* myP = sP + w * 16 * RPPAD;

#pragma unroll
  for (int st = 0; st < RNS - 1; ++st)
    if (st < nsub) issue(st, st);
  for (int it = 0; it < nsub; ++it) {
    // this wave's loads of sub-chunk it are done once at most the later ones remain
    const int newer = min(RNS - 2, nsub - 1 - it);
    if (newer >= 2) wait_vmcnt<2 * RL>();
    else if (newer == 1) wait_vmcnt<RL>();
    else wait_vmcnt<0>();
    __syncthreads();                 // every wave's loads landed; sub-chunk it - 1 consumed
    if (it + RNS - 1 < nsub) issue(it + RNS - 1, (it + RNS - 1) % RNS);
    const int k0 = kbeg + it * RMK;
    const char* stK = smem_raw + (size_t)(it % RNS) * RSTAGE;
    const char* stV = stK + RVOFF;
    // zero the V entries of keys no row may see whose slots need not hold data:
    // keys at or past the chunk end and, windowed, the first range's slots
    // [A, A16) up to its page end (tokens of this stage, relative indices)
    const int z0 = min(RMK, max(kend, k0) - k0);
    const int g0 = WIN ? max(Am, k0) - k0 : RMK, g1 = WIN ? min(A16, k0 + RMK) - k0 : 0;
    if (z0 < RMK || g0 < g1) {
      bf16* zV = reinterpret_cast<bf16*>(const_cast<char*>(stV));
      const int nz = RMK - z0, ng = g0 < g1 ? g1 - g0 : 0;
      for (int e = tid; e < (nz + ng) * HD; e += NTH) {
        const int t = e / HD, d = e % HD;
        const int kk = t < nz ? z0 + t : g0 + (t - nz);
        const int pg = kk >> 4, tk = kk & 15, h = (tk >> 3) ^ ((d >> 3) & 1);
        zV[(pg * 4096 + d * 32 + h * 16) / 2 + (tk & 7)] = (bf16)0.0f;
      }
      __syncthreads();
    }
    // S = Q K^T over RMK / 16 key tiles of 16
    constexpr int NJ = RMK / 16;
    f32x4 s[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = j * 16 + r16;
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        const int cq = (ks * 4 + grp) ^ r16;
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(stK + t * 256 + cq * 16);
        s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kb, s[j], 0, 0, 0);
      }
    }
    // mask (row grp*4+i sees keys below lim[i]; windowed rows: their slot ranges)
    // and the online softmax
    float mt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float v = s[j][i] * sc;
        const int kk = k0 + j * 16 + r16;
        bool hide;
        if (WIN) {
          const int sl = kk < A16 ? kk : C16 + (kk - A16);
          hide = kk >= kend || (kk < A16 ? sl >= lim[i] : (sl < wc[i] || sl > wd[i]));
        } else {
          hide = kk >= lim[i];
        }
        if (hide) v = -INFINITY;
        s[j][i] = v;
        mx = fmaxf(mx, v);
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
      mt[i] = mx;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(m[i], mt[i]);
      const float f = (m[i] == -INFINITY) ? 0.0f : exp2f(m[i] - mn);
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float pv = (s[j][i] == -INFINITY) ? 0.0f : exp2f(s[j][i] - mn);
        s[j][i] = pv;
        ps += pv;
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) ps += __shfl_xor(ps, off, 16);
      l[i] = l[i] * f + ps;
      m[i] = mn;
#pragma unroll
      for (int d = 0; d < HD / 16; ++d) o[d][i] *= f;
    }
    // P to this wave's LDS rows (bf16, row-major [16][RMK]), then O += P V
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) myP[(grp * 4 + i) * RPPAD + j * 16 + r16] = (bf16)s[j][i];
#pragma unroll
    for (int ks = 0; ks < RMK / 32; ++ks) {
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(myP + r16 * RPPAD + ks * 32 + grp * 8);
      const int pg = ks * 2 + (grp >> 1), h = grp & 1;
#pragma unroll
      for (int d = 0; d < HD / 16; ++d) {
        const int dim = d * 16 + r16;
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(
            stV + pg * 4096 + dim * 32 + ((h ^ ((dim >> 3) & 1)) * 16));
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[d], 0, 0, 0);
      }
    }
  }
  // partials (or the final output when the context has one chunk)
  const bool single = a.n_chunks == 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = grp * 4 + i;
    if (row >= nrows) continue;
    const size_t rr = (size_t)(r0 + row);
    if (single) {
      const float inv = l[i] > 0.0f ? 1.0f / l[i] : 0.0f;
      bf16* out = reinterpret_cast<bf16*>(a.out);
#pragma unroll
      for (int d = 0; d < HD / 16; ++d)
        out[frag_off((int)rr, head * HD + d * 16 + r16, a.n_q_heads * HD)] = (bf16)(o[d][i] * inv);
    } else {
      const size_t ph = (rr * a.n_q_heads + head) * a.n_chunks + c;
#pragma unroll
      for (int d = 0; d < HD / 16; ++d) a.part_o[ph * HD + d * 16 + r16] = o[d][i];
      if (r16 == 0) {
        a.part_ml[ph * 2] = m[i] * 0.6931471805599453f;
        a.part_ml[ph * 2 + 1] = l[i];
      }
    }
  }
}
}  // namespace

template <typename T>
size_t attn_smem_bytes(int G, int hd) {
  const int NQ = 16 * G;
  return (size_t)(NQ * hd + NQ * SUB + 3 * NQ + 48) * 4 + (size_t)2 * SUB * (hd + 2) * sizeof(T);
}

template <typename T>
hipError_t launch_attention(const AttnArgs& a, const KvLayout& kv, hipStream_t s) {
  const int G = a.n_q_heads / kv.n_kv_heads;
  if (16 * G * kv.head_dim > 256 * 64 || a.chunk % SUB != 0) return hipErrorInvalidValue;
  const int R = a.n * a.rows_per_seq;
  if (R <= 0) return hipSuccess;
  const int row_tiles = (a.rows_per_seq + 15) / 16;
  dim3 grid(a.n_chunks, kv.n_kv_heads, a.n * row_tiles);
  const bool mfma = sizeof(T) == 2 && kv.head_dim == HD && G == 4 && a.chunk % MK == 0 &&
                    kv.page_shift >= 3;
  if (mfma) {
    const size_t smem = (size_t)(MK * KPAD + HD * VPAD + G * 16 * PPAD) * 2;
    if (smem > 64 * 1024) {
      for (const void* f : {reinterpret_cast<const void*>(&k_attn_mfma<false>),
                            reinterpret_cast<const void*>(&k_attn_mfma<true>)}) {
        hipError_t ea = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (ea != hipSuccess) return ea;
      }
    }
    const bool ring = kv.page_size == 16 && a.chunk % 64 == 0 && a.chunk >= kAttnRingMinChunk &&
                      a.chunk <= PGC * 16;
    if (ring) {
      // 128 rows per sequence or more (prefill, the distillation forward): four row
      // tiles per workgroup share each K/V stage; decode blocks keep one
      const bool multi = a.rows_per_seq >= 128;
      const int RTn = multi ? 4 : 1;
      const size_t rsmem = (size_t)RNS * RSTAGE + (size_t)G * RTn * 16 * RPPAD * 2;
      const void* f = multi ? (a.row_vis ? reinterpret_cast<const void*>(&k_attn_ring<true, 4>)
                                         : reinterpret_cast<const void*>(&k_attn_ring<false, 4>))
                            : (a.row_vis ? reinterpret_cast<const void*>(&k_attn_ring<true, 1>)
                                         : reinterpret_cast<const void*>(&k_attn_ring<false, 1>));
      hipError_t ea = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)rsmem);
      if (ea != hipSuccess) return ea;
      if (multi) {
        dim3 g4(a.n_chunks, kv.n_kv_heads, a.n * ((row_tiles + 3) / 4));
        if (a.row_vis) uno_launch(k_attn_ring<true, 4>, g4, 1024, (uint32_t)rsmem, s, a, kv);
        else uno_launch(k_attn_ring<false, 4>, g4, 1024, (uint32_t)rsmem, s, a, kv);
      } else {
        if (a.row_vis) uno_launch(k_attn_ring<true, 1>, grid, 256, (uint32_t)rsmem, s, a, kv);
        else uno_launch(k_attn_ring<false, 1>, grid, 256, (uint32_t)rsmem, s, a, kv);
      }
    } else if (a.row_vis) {
      uno_launch(k_attn_mfma<true>, grid, 64 * G, smem, s, a, kv);
    } else {
      uno_launch(k_attn_mfma<false>, grid, 64 * G, smem, s, a, kv);
    }
  } else {
    const size_t smem = attn_smem_bytes<T>(G, kv.head_dim);
    const int nown = (16 * G * kv.head_dim + 255) / 256;
#define UNO_ATTN_CASE(MO)                                                                   \
  if (nown <= MO) {                                                                         \
    if (smem > 64 * 1024) {                                                                 \
      hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_partial<T, MO>), \
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); \
      if (ea != hipSuccess) return ea;                                                      \
    }                                                                                       \
    uno_launch(k_attn_partial<T, MO>, grid, 256, smem, s, a, kv);                                   \
  } else
    UNO_ATTN_CASE(1) UNO_ATTN_CASE(4) UNO_ATTN_CASE(16) UNO_ATTN_CASE(32) UNO_ATTN_CASE(64)
    return hipErrorInvalidValue;
#undef UNO_ATTN_CASE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_chunks == 1 && mfma) return hipSuccess;   // the MFMA kernel wrote the outputs directly
  uno_launch(k_attn_combine<T>, R * a.n_q_heads, 256, 0, s, a, kv.head_dim);
  return hipGetLastError();
}

template hipError_t launch_attention<float>(const AttnArgs&, const KvLayout&, hipStream_t);
template hipError_t launch_attention<bf16>(const AttnArgs&, const KvLayout&, hipStream_t);
template size_t attn_smem_bytes<float>(int, int);
template size_t attn_smem_bytes<bf16>(int, int);
