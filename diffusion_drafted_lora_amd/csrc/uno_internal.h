// Internal declarations shared by the HIP sources of libuno (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <climits>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define UNO_DEV __device__ __forceinline__

// ---------------------------------------------------------------- storage types
template <typename T> UNO_DEV float to_f(T v);
template <> UNO_DEV float to_f<float>(float v) { return v; }
template <> UNO_DEV float to_f<bf16>(bf16 v) { return (float)v; }
template <typename T> UNO_DEV T from_f(float v);
template <> UNO_DEV float from_f<float>(float v) { return v; }
template <> UNO_DEV bf16 from_f<bf16>(float v) { return (bf16)v; }  // round to nearest even

// ------------------------------------------------------------- kernel launches
// Every launch goes through uno_launch.  When the runtime has armed a timer on
// the calling thread, the launch takes the timer's next event pair, which HIP
// stamps with that kernel's own start and end (hipExtLaunchKernel), so the time
// between kernels is not counted.
struct KernelTimer {
  virtual bool next(hipEvent_t* start, hipEvent_t* stop) = 0;
};
extern thread_local KernelTimer* g_kernel_timer;

template <typename... KArgs, typename... Args>
inline void uno_launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t smem,
                       hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (g_kernel_timer && !g_kernel_timer->next(&e0, &e1)) e0 = e1 = nullptr;
  hipExtLaunchKernelGGL(kernel, grid, block, smem, s, e0, e1, 0, static_cast<KArgs>(args)...);
}

// ------------------------------------------------------ fragment-tiled layout
// bf16 matrices that feed the MFMA kernels -- projection / LoRA / LM-head weights
// and the activations the linear kernels read -- are stored as 16 x 32 blocks of
// an [R, C] matrix (R a multiple of 16, C of 32), block (r / 16, c / 32) at
// ((r / 16) * (C / 32) + c / 32) * 512, and inside a block the element (r, c) at
// lane (c % 32) / 8 * 16 + r % 16, item c % 8: the operand order of
// v_mfma_f32_16x16x32_bf16 (lane l: row l % 16, k (l / 16) * 8 .. + 8), so a
// wavefront reads one block as one contiguous 1 KB access.
UNO_DEV size_t frag_off(int r, int c, int C) {
  return ((size_t)(r >> 4) * (size_t)(C >> 5) + (size_t)(c >> 5)) * 512 +
         (size_t)((((c & 31) >> 3) << 4) + (r & 15)) * 8 + (c & 7);
}
// Row-major for float32 contexts, fragment-tiled for bf16.
template <typename T> UNO_DEV size_t act_off(int r, int c, int C) {
  return sizeof(T) == 2 ? frag_off(r, c, C) : (size_t)r * C + c;
}
inline size_t round16(size_t r) { return (r + 15) / 16 * 16; }

// Row-major [rows, cols] bf16 -> fragment-tiled; pair_hd > 0 also reorders the
// rows of each pair_hd-row head so that every 16-row block holds rows
// 8j .. 8j+7 and pair_hd/2 + 8j .. +7 (the RoPE pairs of one tile).
hipError_t launch_pack(const bf16* src, bf16* dst, int rows, int cols, int pair_hd, hipStream_t s);

// Device error bits (sticky per context, OR-ed by kernels).
enum : int32_t {
  UNO_DEVERR_NUMERIC = 1,   // NaN / negative / >1 probability, or a row without mass
  UNO_DEVERR_BOUNDS = 2,    // a KV position outside the sequence's reserved pages
  UNO_DEVERR_SYNC = 4,      // a workgroup's bounded wait for another's result ran out
};

// ------------------------------------------------------------- Philox4x64-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11):
// round multipliers and the Weyl key increments of the 4x64 variant.
#define PHILOX_M0 0xD2E7470EE14C6C93ull
#define PHILOX_M1 0xCA5A826395121157ull
#define PHILOX_W0 0x9E3779B97F4A7C15ull
#define PHILOX_W1 0xBB67AE8584CAA73Bull

enum : int32_t { STREAM_DRAFT = 0, STREAM_ACCEPT = 1, STREAM_RESAMPLE = 2 };

// Word 0 of Philox4x64-10(key = (k0, k1), counter = (c0, c1, c2, c3)).
UNO_DEV uint64_t philox_word0(uint64_t k0, uint64_t k1, uint64_t c0, uint64_t c1,
                              uint64_t c2, uint64_t c3 = 0) {
  uint64_t x0 = c0, x1 = c1, x2 = c2, x3 = c3;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
    const uint64_t hi0 = __umul64hi(PHILOX_M0, x0), lo0 = PHILOX_M0 * x0;
    const uint64_t hi1 = __umul64hi(PHILOX_M1, x2), lo1 = PHILOX_M1 * x2;
    const uint64_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
    x0 = n0; x1 = lo1; x2 = n2; x3 = lo0;
  }
  return x0;
}

// The draw deciding absolute position `pos` in `stream` at iteration `it`; `c3`
// is 0 in the linear sampler and the chain / trial index in the tree sampler.
UNO_DEV uint64_t draw_word(uint64_t seed, int32_t seq_id, int32_t pos, int32_t stream,
                           int32_t it, int32_t c3 = 0) {
  return philox_word0(seed, (uint64_t)(uint32_t)seq_id, (uint64_t)(uint32_t)pos,
                      (uint64_t)(uint32_t)stream, (uint64_t)(uint32_t)it,
                      (uint64_t)(uint32_t)c3);
}

// Uniform in [0, 1 - 2^-24]: the top 24 bits of the word, exact in float32.
UNO_DEV float unif24(uint64_t w) { return (float)(uint32_t)(w >> 40) * 0x1p-24f; }

// Integer weight trunc(w * 2^40); flags NaN / negative / > 1 and treats them as 0.
UNO_DEV uint64_t int_weight(float w, int32_t* err) {
  if (!(w >= 0.0f && w <= 1.0f)) {   // catches NaN too
    if (err) atomicOr(err, UNO_DEVERR_NUMERIC);
    return 0;
  }
  return (uint64_t)(w * 0x1p40f);    // exact scaling; the cast truncates
}

// ------------------------------------------------------------------- sampling
// A categorical row to draw from: mode 0 -> weights a[j]; mode 1 -> the residual
// max(0, a[j] - b[j]) with a fallback to a[j] when the residual has no mass.
struct RowDesc {
  const float* a;
  const float* b;
  int32_t mode;
  int32_t pad;
  uint64_t word;
  int32_t* out;
};

UNO_DEV float row_weight(const RowDesc& d, int mode, int j) {
  float w = d.a[j];
  if (mode == 1) w = fmaxf(w - d.b[j], 0.0f);   // float32 subtraction
  return w;
}

constexpr int CDF_CHUNK = 2048;  // elements per chunk of the integer CDF
constexpr int CDF_THREADS = 256;

struct KvLayout {
  void* pool;
  int32_t n_pages, n_kv_heads, page_size, head_dim, n_layers;
  const int32_t* block_table;   // [max_seqs, max_pages_per_seq]
  int32_t max_pages_per_seq;
  int32_t page_shift;           // log2(page_size) for a power of two, else -1
};

// One (page, KV head) block of the pool holds page_size tokens x head_dim: K
// token-major ([token][dim], a token's K row contiguous) and V dim-major
// ([dim][token], eight consecutive tokens of one dim contiguous: the B-operand
// order of the P.V product).
template <typename T>
UNO_DEV T* kv_block(const KvLayout& kv, int layer, int which, int page, int h) {
  return reinterpret_cast<T*>(kv.pool) +
         (((size_t)(layer * 2 + which) * kv.n_pages + page) * kv.n_kv_heads + h) *
             (size_t)kv.page_size * kv.head_dim;
}
UNO_DEV size_t kv_elem(const KvLayout& kv, int which, int t, int d) {
  return which == 0 ? (size_t)t * kv.head_dim + d : (size_t)d * kv.page_size + t;
}
// page of a slot of a sequence, or -1 outside its reserved pages
UNO_DEV int kv_page(const KvLayout& kv, int seq, int slot) {
  const int pi = slot / kv.page_size;
  if (slot < 0 || pi >= kv.max_pages_per_seq) return -1;
  const int page = kv.block_table[(size_t)seq * kv.max_pages_per_seq + pi];
  return (page >= 0 && page < kv.n_pages) ? page : -1;
}

// ------------------------------------------------------------ GEMM interfaces
enum GemmEpi : int32_t {
  EPI_QKV = 5,         // pair-permuted q|k|v columns: RoPE, q -> qbuf, k / v -> KV pages
  EPI_STORE_F32 = 0,   // out_f32[m, n] = acc
  EPI_LORA_U = 1,      // out_t[m, n] = gate[m] ? T(scale * acc) : 0
  EPI_RESID = 2,       // resid[m, n] += acc
  EPI_SWIGLU = 3,      // out_t[m, n] = T(silu(acc_gate) * acc_up)    (paired segments)
  EPI_LOGITS = 4,      // out_f32[m, n] = acc (MASK column -inf) + per-tile max / sum-exp
  EPI_TSLICE = 6,      // out_f32[slice][m, n] = acc of K slice `slice` (LoRA down, large M)
};

// LoRA intermediates accumulated in fixed point: t = sum x*A in units of 2^-32
// (int64, order-independent integer sums).
constexpr float LORA_FX_SCALE = 4294967296.0f;     // 2^32
constexpr double LORA_FX_INV = 1.0 / 4294967296.0;
// t * 2^-32 in float from the two 32-bit halves (t = hi * 2^32 + lo, lo >= 0):
// two native conversions and one fma, within one float ulp of the exact value.
UNO_DEV float fx_to_float(long long t) {
  return fmaf((float)(unsigned)(t & 0xffffffffll), 0x1p-32f, (float)(int)(t >> 32));
}

// Fixed-point row sums of x^2 are spread over SS_BANKS int64 words per row
// ([row][bank]): a producer adds into the bank of its workgroup, so the hundreds
// of workgroups of a skinny residual epilogue do not queue on one address, and a
// consumer adds the banks (integer sums: exact in any order).
constexpr int SS_BANKS = 16;
typedef long long i64x2 __attribute__((ext_vector_type(2)));
// Range: a producer's partial must stay below 2^25 and a bank below 2^26 (2^58
// fixed-point units), so a row's sum of squares is exact below 2^30 (an rms of 512
// at d 4096).  At most 32 partials reach one bank, so clamping each partial to
// 2^25 keeps every bank below 2^62: nothing wraps silently -- a producer whose
// partial is out of range (or NaN) and a consumer that reads a bank of 2^58 or
// more set the numeric flag.
constexpr float SS_PART_MAX = 33554432.0f;          // 2^25
constexpr long long SS_BANK_MAX = 1LL << 58;
// A consumer's check of the banks it read (OR of the bank words).
UNO_DEV void ss_check(long long banks_or, int32_t* err) {
  if ((banks_or & ~(SS_BANK_MAX - 1)) != 0 && err) atomicOr(err, UNO_DEVERR_NUMERIC);
}
UNO_DEV long long ss_row(const long long* ss, int m, int32_t* err) {
  const i64x2* p = reinterpret_cast<const i64x2*>(ss + (size_t)m * SS_BANKS);
  long long t = 0, o = 0;
#pragma unroll
  for (int i = 0; i < SS_BANKS / 2; ++i) {
    const i64x2 v = p[i];
    t += v.x + v.y;
    o |= v.x | v.y;
  }
  ss_check(o, err);
  return t;
}
UNO_DEV void ss_add(long long* ss, int m, int bank, float sq, int32_t* err) {
  if (!(sq < SS_PART_MAX)) {                         // out of range, or NaN
    if (err) atomicOr(err, UNO_DEVERR_NUMERIC);
    sq = SS_PART_MAX;
  }
  atomicAdd(reinterpret_cast<unsigned long long*>(ss + (size_t)m * SS_BANKS + (bank & (SS_BANKS - 1))),
            (unsigned long long)(long long)llrintf(sq * LORA_FX_SCALE));
}

// LoRA down-projection of a group of projections sharing one input:
// t[m, p*r + j] += sum_k X[m, k] * A_p[j, k] (fixed point, int64 atomics).
struct LoraDownArgs {
  const void* X;
  int32_t ldx, M, K, r;
  const void* A[4];
  int32_t nproj;
  int32_t kchunk;
  long long* t;      // [M, nproj * r]
  const long long* ss_in;   // RMSNorm input (see GemmArgs), or null
  float inv_d, eps;
  int32_t* err;             // device error flags (sum-of-squares range)
};

struct GemmSeg {
  const void* W;     // [N, K] of the storage type
  const void* Bl;    // LoRA up [N, r] (or null)
  const void* U;     // gated, scaled LoRA intermediate of the storage type (or null):
                     // float32 row-major at column 0 of the segment; bf16 the whole
                     // fragment-tiled [M, ldu] buffer (segment at column ucol)
  const long long* Ufx;  // bf16 path: fixed-point t [M, ldu] (u = gate * bf16(scale * t))
  int32_t n0;        // first output column of this segment
  int32_t N;         // columns of this segment
  int32_t ldu;
  int32_t ucol;      // bf16 U: first column of this segment's intermediate in the
                     // fragment-tiled [M, ldu] buffer U points at
};

struct GemmArgs {
  const void* X;     // activations [M, ldx] of the storage type
  int32_t ldx, M, K, r;
  GemmSeg seg[4];
  int32_t nseg;
  int32_t paired;    // 1: segment 0 and 1 are computed at the same columns (SwiGLU)
  int32_t epi;
  int32_t ldo;
  void* out;
  float* resid;
  const uint8_t* gate;
  float scale;
  int32_t mask_col;  // EPI_LOGITS: column forced to -inf
  float* tile_stats; // EPI_LOGITS: [M, n_tiles, 2] (max, sum exp)
  int32_t n_tiles;   // EPI_LOGITS: total 16-column tiles
  int32_t zero_n;    // int64 words of zero_ptr cleared (spread over the workgroups)
  long long* zero_ptr;
  // RMSNorm input: X holds the stored x*g; the base accumulator of row m is
  // scaled by rs = 1 / sqrt(ss_in[m] * 2^-32 / d + eps) (ss_in: fixed-point sum x^2)
  const long long* ss_in;
  float inv_d, eps;
  // EPI_RESID producer: also store xg_out[m, n] = T(x_new * g_next[n]) and add the
  // row's x_new^2 (fixed point) to ss_out[m]
  void* xg_out;
  const void* g_next;
  long long* ss_out;
  // EPI_QKV: q/k rotated at row_pos[m]; K/V written at slot row_slot[m] of the
  // row's sequence (row_pos[m] when row_slot is null)
  const int32_t* row_pos;
  const int32_t* row_slot;
  const int32_t* call_seq;
  int32_t seq_fixed;   // > 0: every row belongs to sequence seq_fixed - 1 (saves a load)
  int32_t rows_per_seq, n_q_heads;
  const float* rcos;
  const float* rsin;
  void* qbuf;
  KvLayout kv;
  int32_t layer;
  int32_t* err;
  // EPI_TSLICE / EPI_STORE_F32 (large-M kernel): K is split into k_slices equal
  // slices, slice s storing its float partial sum at out + s * slice_stride
  // elements; only slice 0 adds the LoRA stages
  int32_t k_slices;
  long long slice_stride;
  // EPI_RESID at large M: float workspace of split_cap elements that a K-split
  // launch may use for its partial sums (null: never split)
  float* split_ws;
  long long split_cap;
  // Fused LoRA down-projection (few rows, skinny kernel): the first n_prod
  // workgroups of row tile mt compute pieces of the intermediate described by
  // `ld` (rank tile p % (ld.nproj * ld.r / 16), K chunk p / that) and then add 1 to
  // sync[mt]; the tile's other workgroups stream their base product meanwhile and
  // wait for sync[mt] to reach sync_target[mt] before the LoRA phase.  A tile's
  // producers are dispatched before its consumers (lower workgroup ids), so the
  // wait always ends; the counters only grow (each launch raises a tile's target
  // by n_prod).
  int32_t n_prod;
  uint32_t sync_target[4];
  uint32_t* sync;
  LoraDownArgs ld;
};

hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t s);
// Large-M LoRA down-projection on the tile kernel (EPI_TSLICE, no atomics): false
// when no tile shape fits the problem (the atomic kernel then serves it).
bool lora_down_tile_fits(int M, int K, int ncols, int k_slices);
int lora_down_tile_slices(int M, int K, int ncols);
hipError_t launch_lora_down_tile(const GemmArgs& a, int ncols, hipStream_t s);
// u[m, c] = gate[m] ? bf16(scale * sum_s t[s][m, c] * 2^-32) : 0 over the K-slice
// partials of the large-M down-projection ([M, ncols] each, `stride` apart); u is
// fragment-tiled [round16(M), ncols]
hipError_t launch_lora_u(const float* t, int n_slices, long long stride, int M, int ncols,
                         const uint8_t* gate, float scale, bf16* u, hipStream_t s);
hipError_t launch_zero_i64(long long* p, size_t n, hipStream_t s);

// ------------------------------------------------------------------ launchers
// Every launcher enqueues on `s` and returns the hipGetLastError of its launch.
template <typename T> hipError_t launch_gemm(const GemmArgs& a, int n_cols_total, hipStream_t s);

struct RowsSetup {
  int32_t mode;          // 0 draft, 1 verify, 2 forward (caller rows), 3 prefill,
                         // 4 distillation rows [x | MASK^L] (B = its block size),
                         // 5 tree verify (y_1, then K chains of depths 2..B)
  int32_t n, rows_per_seq, B, mask_id;
  int32_t K;                 // mode 5: chains per sequence (draft_tok is [n, K, B])
  const int32_t* call_seq;   // [n] sequence ids
  const int32_t* len;        // [max_seqs]
  const int32_t* pending;    // [max_seqs]
  const int32_t* iter;       // [max_seqs]
  const int32_t* draft_tok;  // [n, B] (verify)
  const int32_t* in_tok;     // forward / prefill: [n * rows]
  const int32_t* in_pos;     // forward: [n * rows]; prefill: first position (scalar in pos0)
  const uint8_t* in_gate;    // forward: [n * rows]
  int32_t pos0;              // prefill: position of the first row
  int32_t* row_tok;
  int32_t* row_pos;
  uint8_t* row_gate;
  int32_t* row_slot;         // modes 4, 5: KV slot of each row
  int32_t* row_vis;          // modes 4, 5: [R][3] visible slots [0, a) and [c, d]
  int32_t* call_n;           // [n] pending position n of each call sequence
  int32_t* call_it;          // [n] iteration
};
hipError_t launch_rows_setup(const RowsSetup& a, hipStream_t s);

// x[r] = E[tok[r]] (or hidden_in[r]); also xg[r] = T(x * g) and ss[r] += sum x^2.
template <typename T>
hipError_t launch_embed(const T* E, const int32_t* tok, const float* hidden_in, int R, int d,
                        int V, float* x, const T* g, T* xg, long long* ss, int32_t* err,
                        hipStream_t s);

// Attention rows see, in their sequence's KV slots, [0, row_pos] -- or, when
// row_vis is given, the slots [0, a) and [c, d] with (a, c, d) = row_vis[r]
// (the distillation forward's block-causal mask over [x, z1]).  The keys a
// 16-row tile walks are the union of its rows' windows, numbered virtually:
// [0, A) then [C, D] (A = max a, C = min c, D = max d).
struct AttnArgs {
  const void* q;             // [R, Hq * hd] of T
  void* out;                 // [R, Hq * hd] of T (activation layout: act_off)
  const int32_t* row_pos;    // [R]
  const int32_t* row_vis;    // [R][3] or null
  int32_t* row_nc;           // [R] context chunks that hold each row's partials
  const int32_t* call_seq;   // [n]
  int32_t seq_fixed;         // > 0: every row belongs to sequence seq_fixed - 1
  int32_t n, rows_per_seq, n_q_heads, n_chunks, chunk;
  float scale;
  float* part_o;             // [R * Hq, n_chunks, hd]
  float* part_ml;            // [R * Hq, n_chunks, 2]
  int32_t layer;
  int32_t pad;
  int32_t* err;              // device error flags
};
template <typename T> hipError_t launch_attention(const AttnArgs& a, const KvLayout& kv,
                                                  hipStream_t s);

hipError_t launch_row_stats(const float* tile_stats, int R, int n_tiles, float* row_ml,
                            hipStream_t s);
hipError_t launch_softmax(const float* logits, const float* row_ml, int R, int V, float* probs,
                          hipStream_t s);
// Per-row total variation 0.5 * sum_v |softmax(T_i) - softmax(S_i)| of L row pairs
// (logits with row stats (max, sum exp)), then the mean over each block of B rows.
hipError_t launch_tv(const float* t_logits, const float* s_logits, const float* t_ml,
                     const float* s_ml, int L, int V, float* tv_row, hipStream_t s);
hipError_t launch_tv_blocks(const float* tv_row, int L, int B, float* tv_block, hipStream_t s);

hipError_t launch_draft_desc(const float* probs, int n, int B, int V, uint64_t seed,
                             const int32_t* call_seq, const int32_t* call_n,
                             const int32_t* call_it, int32_t* out_tok, RowDesc* desc,
                             hipStream_t s);
hipError_t launch_sample_desc(const float* w, int rows, int V, uint64_t seed,
                              const int32_t* seq_ids, const int32_t* pos, const int32_t* it,
                              int stream_id, int32_t* out, RowDesc* desc, hipStream_t s);
hipError_t launch_cdf(const RowDesc* desc, int rows, int V, uint64_t* chunk_tot,
                      int32_t* err, hipStream_t s);
// q rows of sequence s start at q + s * q_stride * V (q_2 first).
hipError_t launch_accept_test(uint64_t seed, int n, int B, int V, const float* p,
                              const float* q, int q_stride, const int32_t* draft,
                              const int32_t* call_seq, const int32_t* call_n,
                              const int32_t* call_it, int32_t* k_out, int32_t* z_out,
                              RowDesc* desc, int32_t* err, hipStream_t s);
hipError_t launch_accept_commit(int n, int B, const int32_t* draft, const int32_t* k,
                                const int32_t* z, const int32_t* call_seq, int32_t* out,
                                int32_t* n_out, int32_t* len, int32_t* pending, int32_t* iter,
                                hipStream_t s);

struct SetList {            // small device scatter passed by value: dst[idx[i]] = val[i]
  int32_t* dst;
  int32_t count;
  int32_t idx[240];
  int32_t val[240];
};
hipError_t launch_set_list(const SetList& l, hipStream_t s);
// Read-only stream of `bytes` (a multiple of 16) by workgroups x threads threads,
// `loads` (1, 2, 4 or 8) 16-byte loads in flight per thread; sink: one int32 per
// workgroup.
hipError_t launch_stream_read(const void* src, size_t bytes, int workgroups, int threads, int loads,
                              int32_t* sink, hipStream_t s);

template <typename T>
hipError_t launch_kv_copy(const KvLayout& kv, int seq, int len, T* k, T* v, int to_pages,
                          hipStream_t s);

// Row-major copy [R, C] of an activation buffer of the linear kernels' layout
// (fragment-tiled bf16, row-major float32).
template <typename T>
hipError_t launch_untile(const T* src, T* dst, int R, int C, hipStream_t s);
template <> hipError_t launch_untile<bf16>(const bf16* src, bf16* dst, int R, int C, hipStream_t s);
template <> hipError_t launch_untile<float>(const float* src, float* dst, int R, int C, hipStream_t s);

// Records msg as the context-free last error (uno_last_error(NULL)); returns status.
int32_t uno_fail_global(int32_t status, const char* msg);
// Looks up the current device's address of the no-allocation scratch array.
hipError_t noalloc_prime();

// ------------------------------------------------------ distillation backward
// Index map of a strided axis: i -> (i >> sh) * hi + (i & (2^sh - 1)) * lo (a
// plain stride is {0, ld, 0}; sh > 0 walks rows i * G + g of G query heads).
struct Idx2 {
  int sh;
  long hi, lo;
};
inline Idx2 idx_ld(long ld) { return Idx2{0, ld, 0}; }

// Operand layouts of the backward GEMM C[m, n] = sum_k A(m, k) B(n, k).
enum : int {
  BW_A_K16 = 0,   // bf16, A(m, k) at A[ai(m) + k]
  BW_A_K32 = 1,   // float32 (two bf16 terms), A(m, k) at A[ai(m) + k]
  BW_A_M32 = 2,   // float32 (two bf16 terms), A(m, k) at A[ai(k) + m], times kscale[k]
};
enum : int {
  BW_B_TN = 0,    // fragment-tiled weight [N, K] (b_cols = K): B(n, k) = W[n][k]
  BW_B_TT = 1,    // fragment-tiled weight [K, N] (b_cols = N): B(n, k) = W[k][n]
  BW_B_K16 = 2,   // bf16, B(n, k) at B[bi(n) + k]
  BW_B_N16 = 3,   // bf16, B(n, k) at B[bi(k) + n]
  BW_B_N32 = 4,   // float32 (two bf16 terms), B(n, k) at B[bi(k) + n]
};
struct BwGemm {
  int amode, bmode;
  const void* A;
  Idx2 ai;
  long a_bs;                 // batch strides in elements (blockIdx.z)
  const void* B;
  Idx2 bi;
  long b_bs;
  int b_cols;                // columns of a tiled weight
  void* C;                   // C[ci(row) + col], float32 or bf16
  Idx2 ci;
  long c_bs;
  int M, N, K, batch, splits;
  float alpha;               // C = alpha * row_scale[m] * sum (+ C when accumulate)
  const float* row_scale;
  const float* kscale;
  int accumulate, out_bf16;
  int perm_hd;               // > 0: output rows are in the RoPE pair order of heads of
                             // perm_hd rows and are written to their head-order rows
  float* part;               // splits > 1: float32 [splits, M, N] partials
  // two-level batch: z -> (z / bz, z % bz) with strides (a_bs, a_bs2) etc.
  int bz;
  long a_bs2, b_bs2, c_bs2;
  // block-causal key limit over rows m = i * G + g: the rows of an output tile see
  // keys below lim = (i_last / lim_B) * lim_B, i_last the tile's last row position.
  // lim_mode 1: the N axis is keys, tiles at or past lim are skipped (not written);
  // lim_mode 2: the K axis is keys, the k loop stops at lim (rounded up to a step)
  int lim_mode, lim_G, lim_B;
};
hipError_t launch_bw_gemm(const BwGemm& g, hipStream_t s);
template <typename T>
hipError_t launch_bw_rmsprep(const float* x, const T* gain, float eps, int rows, int d, bf16* hg,
                             float* rs, hipStream_t s);
template <typename T>
hipError_t launch_bw_rmsback(const float* x, const bf16* hg, const float* rs, const T* gain,
                             const float* dh, const float* dres, float* dx, int rows, int d,
                             hipStream_t s);
hipError_t launch_bw_qkv_post(const float* Yq, const float* Yk, const float* Yv, const float* rcos,
                              const float* rsin, int rows, int L, int Hq, int Hkv, int hd, bf16* Q,
                              bf16* Ks, bf16* Vs, hipStream_t s);
hipError_t launch_bw_qkv_back(const float* dq, const float* dk, const float* dv, const float* rcos,
                              const float* rsin, int rows, int L, int Hq, int Hkv, int hd, float* dYq,
                              float* dYk, float* dYv, hipStream_t s);
// Attention of one sequence's z1 rows (rows m = i * G + g of each KV head h):
// St [Hkv][L*G][L] scores / probabilities over the x keys, So [Hkv][L*G][B] over
// the row's own block (key bB + j at column j); Q [L][Hq*hd] bf16, own K / V
// [L][Hkv*hd] bf16 (this sequence's rows).
hipError_t launch_bw_own_scores(const bf16* Q, const bf16* Ks, int L, int Hq, int Hkv, int hd, int B,
                                float* So, hipStream_t s);
hipError_t launch_bw_softmax(float* St, float* So, int L, int G, int Hkv, int B, float scale,
                             hipStream_t s);
hipError_t launch_bw_own_pv(const float* Po, const bf16* Vs, const float* o32, int L, int Hq, int Hkv,
                            int hd, int B, bf16* o, hipStream_t s);
hipError_t launch_bw_own_dp(const float* dO, const bf16* Vs, int L, int Hq, int Hkv, int hd, int B,
                            float* dPo, hipStream_t s);
hipError_t launch_bw_softmax_back(const float* Pt, const float* Po, float* dPt, float* dPo, int L,
                                  int G, int Hkv, int B, float scale, hipStream_t s);
hipError_t launch_bw_own_back(const float* dSo, const float* Po, const bf16* Q, const bf16* Ks,
                              const float* dO, int L, int Hq, int Hkv, int hd, int B, float* dq,
                              float* dk, float* dv, hipStream_t s);
hipError_t launch_bw_swiglu(const float* Yg, const float* Yu, bf16* a, long n, hipStream_t s);
hipError_t launch_bw_swiglu_back(const float* da, float* Yg, float* Yu, long n, hipStream_t s);
hipError_t launch_tv_grad(const float* T, const float* S, int rows, int V, float inv2n, float* dz,
                          float* tv_row, hipStream_t s);
hipError_t launch_tv_mean(const float* tv_row, int rows, float* loss, hipStream_t s);
