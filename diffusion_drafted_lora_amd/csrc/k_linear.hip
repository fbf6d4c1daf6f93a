// Gated-LoRA linear: y = x W^T + (gate * bf16((alpha/r) x A^T)) B^T with fused
// epilogues (store, LoRA intermediate, residual add, SwiGLU, LM-head logits with
// per-tile softmax statistics).
//
// Method: the diffusion weights are a LoRA on every projection, switched off on
// clean rows and on on noisy rows inside one forward (shibing624 reading notes of
// the Uno paper, "Diffusion Distillation" section; ai-papers-daily summary,
// method key points).  The gate multiplies the stored LoRA intermediate, so a
// gate-off row adds exact zeros and a verify forward skips the LoRA phase.
//
// bf16 kernel (gfx950): one workgroup owns a 16-row x (16*NT)-column output
// tile.  Its WAVES wavefronts split K; every wave streams its slice of the
// weight rows straight from HBM into MFMA B-fragments (weights are [out, in],
// so a lane's 8 consecutive k values are 16 contiguous bytes) and multiplies
// them with A-fragments of the activations (L2-resident) on
// v_mfma_f32_16x16x32_bf16.  The wave partials are summed in LDS in a fixed wave
// order, so results are bit-reproducible.  The LoRA up-projection is a second
// K-phase over the rank dimension with the intermediate as the A operand.
#include "uno_internal.h"

namespace {

template <typename T>
UNO_DEV void epilogue(const GemmArgs& a, int m, int c, int gcol0, int col_paired,
                      const float* v, int NT) {
  switch (a.epi) {
    case EPI_STORE_F32:
      for (int t = 0; t < NT; ++t)
        reinterpret_cast<float*>(a.out)[(size_t)m * a.ldo + gcol0 + t * 16 + c] = v[t];
      break;
    case EPI_LORA_U: {
      const bool on = a.gate == nullptr || a.gate[m] != 0;
      for (int t = 0; t < NT; ++t)
        reinterpret_cast<T*>(a.out)[(size_t)m * a.ldo + gcol0 + t * 16 + c] =
            from_f<T>(on ? a.scale * v[t] : 0.0f);
      break;
    }
    case EPI_RESID:
      for (int t = 0; t < NT; ++t) a.resid[(size_t)m * a.ldo + gcol0 + t * 16 + c] += v[t];
      break;
    case EPI_SWIGLU: {
      const float g = v[0], u = v[1];
      reinterpret_cast<T*>(a.out)[(size_t)m * a.ldo + col_paired + c] =
          from_f<T>(g / (1.0f + expf(-g)) * u);
      break;
    }
    default:
      break;
  }
}

// LM-head epilogue: logits with the MASK column at -inf and, per row and 16-column
// tile, (max, sum exp(l - max)).  The 16 lanes of a row are consecutive.
UNO_DEV void logits_epilogue(const GemmArgs& a, int m, int c, int gcol0, const float* v,
                             int NT, bool valid) {
  for (int t = 0; t < NT; ++t) {
    const int col = gcol0 + t * 16 + c;
    const float l = (col == a.mask_col) ? -INFINITY : v[t];
    if (valid) reinterpret_cast<float*>(a.out)[(size_t)m * a.ldo + col] = l;
    float mx = l;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
    float e = (l == -INFINITY) ? 0.0f : expf(l - mx);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) e += __shfl_xor(e, off, 16);
    if (valid && c == 0) {
      const int tile = (gcol0 + t * 16) / 16;
      a.tile_stats[((size_t)m * a.n_tiles + tile) * 2] = mx;
      a.tile_stats[((size_t)m * a.n_tiles + tile) * 2 + 1] = e;
    }
  }
}

// Locate the group's segment and columns.
UNO_DEV int find_seg(const GemmArgs& a, int gcol0) {
  int s = 0;
  for (int i = 1; i < a.nseg; ++i)
    if (gcol0 >= a.seg[i].n0) s = i;
  return s;
}

UNO_DEV bf16x8 load8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <int NT, int WAVES, int KU>
__global__ void __launch_bounds__(WAVES * 64)
k_gemm_bf16(GemmArgs a) {
  __shared__ float red[WAVES][NT][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int mt = blockIdx.y;
  const int grp = blockIdx.x;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;

  // tiles of this group: pointer to weight row (lane's column) and LoRA operands
  const bf16* Wp[NT];
  const bf16* Bp[NT];
  const bf16* Up[NT];
  int ldu[NT];
  int gcol0, col_paired = 0;
  if (a.paired) {
    const int c0 = grp * 16;
    col_paired = c0;
    gcol0 = c0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const GemmSeg& sg = a.seg[t];
      Wp[t] = reinterpret_cast<const bf16*>(sg.W) + (size_t)(c0 + r16) * a.K;
      Bp[t] = sg.Bl ? reinterpret_cast<const bf16*>(sg.Bl) + (size_t)(c0 + r16) * a.r : nullptr;
      Up[t] = reinterpret_cast<const bf16*>(sg.U);
      ldu[t] = sg.ldu;
    }
  } else {
    gcol0 = grp * 16 * NT;
    const GemmSeg& sg = a.seg[find_seg(a, gcol0)];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int lc = gcol0 - sg.n0 + t * 16 + r16;
      Wp[t] = reinterpret_cast<const bf16*>(sg.W) + (size_t)lc * a.K;
      Bp[t] = sg.Bl ? reinterpret_cast<const bf16*>(sg.Bl) + (size_t)lc * a.r : nullptr;
      Up[t] = reinterpret_cast<const bf16*>(sg.U);
      ldu[t] = sg.ldu;
    }
  }

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

  // ---- LoRA phase: k over the rank, A = gated intermediate U, B = LoRA up
  if (a.r > 0) {
    for (int kr = w * 32; kr < a.r; kr += 32 * WAVES) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (Up[t] == nullptr || Bp[t] == nullptr) continue;
        const bf16x8 af =
            row_ok ? load8(Up[t] + (size_t)m_lane * ldu[t] + kr + kq) : zero8;
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
  for (int e = threadIdx.x; e < 256; e += WAVES * 64) {
    float v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float s = 0.0f;
      for (int ww = 0; ww < WAVES; ++ww) s += red[ww][t][e];
      v[t] = s;
    }
    const int row = e >> 4, c = e & 15;
    const int m = mt * 16 + row;
    if (a.epi == EPI_LOGITS) logits_epilogue(a, m, c, gcol0, v, NT, m < a.M);
    else if (m < a.M) epilogue<bf16>(a, m, c, gcol0, col_paired, v, NT);
  }
}

// float32 twin (small configurations): thread e of the 256 owns element
// (e / 16, e % 16) of each 16x16 tile and runs the K loop itself.  Segments may
// have any width (columns past the last segment are skipped).
template <int NT>
__global__ void __launch_bounds__(256)
k_gemm_f32(GemmArgs a) {
  const int mt = blockIdx.y, grp = blockIdx.x;
  const int e = threadIdx.x, row = e >> 4, c = e & 15;
  const int m = mt * 16 + row;
  const int ntot = a.paired ? a.seg[0].N : a.seg[a.nseg - 1].n0 + a.seg[a.nseg - 1].N;
  int gcol0, col_paired = 0;
  bool ok = m < a.M;
  const float* Wr[NT];
  const float* Br[NT];
  const float* Ur[NT];
  int ldu[NT];
  if (a.paired) {
    gcol0 = grp * 16;
    col_paired = gcol0;
    ok = ok && gcol0 + c < ntot;
    for (int t = 0; t < NT; ++t) {
      const GemmSeg& sg = a.seg[t];
      const int lc = ok ? gcol0 + c : 0;
      Wr[t] = reinterpret_cast<const float*>(sg.W) + (size_t)lc * a.K;
      Br[t] = sg.Bl ? reinterpret_cast<const float*>(sg.Bl) + (size_t)lc * a.r : nullptr;
      Ur[t] = reinterpret_cast<const float*>(sg.U);
      ldu[t] = sg.ldu;
    }
  } else {
    gcol0 = grp * 16 * NT;
    for (int t = 0; t < NT; ++t) {
      const int gcol = gcol0 + t * 16 + c;
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
  const float* x = reinterpret_cast<const float*>(a.X) + (size_t)(m < a.M ? m : 0) * a.ldx;
  float v[NT];
  for (int t = 0; t < NT; ++t) {
    float s = 0.0f;
    if (ok) {
      for (int k = 0; k < a.K; ++k) s += x[k] * Wr[t][k];
      if (a.r > 0 && Ur[t] && Br[t]) {
        const float* u = Ur[t] + (size_t)m * ldu[t];
        for (int k = 0; k < a.r; ++k) s += u[k] * Br[t][k];
      }
    }
    v[t] = s;
  }
  if (a.epi == EPI_LOGITS) logits_epilogue(a, m, c, gcol0, v, NT, ok);
  else if (ok) epilogue<float>(a, m, c, gcol0, col_paired, v, NT);
}

}  // namespace

template <>
hipError_t launch_gemm<bf16>(const GemmArgs& a, int n_cols_total, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % 32 != 0 || (a.r % 32) != 0 || n_cols_total % 16 != 0) return hipErrorInvalidValue;
  const int mtiles = (a.M + 15) / 16;
  if (a.paired) {
    dim3 grid(n_cols_total / 16, mtiles);
    if (a.K % 256 == 0) k_gemm_bf16<2, 8, 2><<<grid, 512, 0, s>>>(a);
    else k_gemm_bf16<2, 1, 1><<<grid, 64, 0, s>>>(a);
  } else {
    dim3 grid(n_cols_total / 16, mtiles);
    if (a.K % 512 == 0) k_gemm_bf16<1, 8, 2><<<grid, 512, 0, s>>>(a);
    else if (a.K % 128 == 0) k_gemm_bf16<1, 4, 1><<<grid, 256, 0, s>>>(a);
    else k_gemm_bf16<1, 1, 1><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <>
hipError_t launch_gemm<float>(const GemmArgs& a, int n_cols_total, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.epi == EPI_LOGITS && n_cols_total % 16 != 0) return hipErrorInvalidValue;
  const int mtiles = (a.M + 15) / 16;
  dim3 grid((n_cols_total + 15) / 16, mtiles);
  if (a.paired) k_gemm_f32<2><<<grid, 256, 0, s>>>(a);
  else k_gemm_f32<1><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}
