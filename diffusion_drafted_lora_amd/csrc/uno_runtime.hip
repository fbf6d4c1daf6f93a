// Host runtime of libuno: context, workspace layout, KV page allocator, argument
// validation, the forward plan and the C ABI of include/uno.h.
//
// The plan follows the method's two forwards per iteration (shibing624 reading
// notes of the Uno paper, section on the Psi-Spec sampler): a draft forward of
// [t, MASK x (B-1)] with the LoRA gated on for the mask rows, sampling of the
// drafted block, then an AR-only verify forward of the block, the accept/resample
// test and the commit.  No host synchronisation happens inside an iteration: the
// sequence state lives on the device, the host keeps only an upper bound of each
// sequence's length (refreshed from an asynchronous snapshot) to reserve pages.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/uno.h"
#include "uno_internal.h"
#include "uno_qknorm.h"
#include "uno_tree.h"

template <typename T> size_t attn_smem_bytes(int G, int hd);

namespace {

constexpr int kMaxChunks = 64;        // context chunks per (row, head) in attention
#ifndef UNO_ATTN_TARGET_WG
#define UNO_ATTN_TARGET_WG 1024
#endif
#ifndef UNO_ATTN_MIN_CHUNK
#define UNO_ATTN_MIN_CHUNK 64
#endif
constexpr int kAttnTargetWG = UNO_ATTN_TARGET_WG;   // workgroups the context split aims at
constexpr int kAttnMinChunk = UNO_ATTN_MIN_CHUNK;   // keys per chunk, at least (a multiple of 64)
constexpr size_t kAlign = 256;
constexpr int kSyncCounters = 16;     // per LoRA group (q|k|v, o, gate/up, down) and row tile

thread_local std::string g_last_error = "";

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t len, pending, iter, err, sync, block_table, rope_cos, rope_sin;
  size_t call_seq, call_n, call_it, row_tok, row_pos, row_gate, row_slot, row_vis, row_nc;
  size_t x, xn, qbuf, obuf, hbuf, ubuf, tfx, ss;
  size_t part_o, part_ml;
  size_t qkv32;                      // float32 q|k|v rows before the QK RMSNorm (qk_norm only)
  size_t part_o_floats, part_rows;   // capacities: float words, (row, head, chunk) triples / Hq
  size_t logits, tile_stats, row_ml, probs_d, probs_v;
  size_t desc, chunk_tot, draft_tok, acc_k, acc_z, aux_i32, tv;
  size_t tree_res, tree_path, tree_kstar;   // tree sampler (tree_chains > 0)
  size_t total;
};

// K-slice capacity of the fixed-point LoRA buffers (large-M down-projection)
size_t tfx_slices(size_t max_rows) { return max_rows <= 4096 ? 4 : 1; }

int pages_per_seq(const uno_config& c) { return (c.max_seq_len + c.page_size - 1) / c.page_size; }

Layout make_layout(const uno_config& c) {
  Layout L{};
  const size_t ts = c.dtype == UNO_BF16 ? 2 : 4;
  const size_t R = (size_t)c.max_rows;
  const size_t S = (size_t)c.max_seqs;
  const size_t d = c.d_model, q = (size_t)c.n_q_heads * c.head_dim,
               kv = (size_t)c.n_kv_heads * c.head_dim, F = c.ffn_dim, V = c.vocab,
               r = c.lora_rank > 0 ? c.lora_rank : 0, B = c.block_size;
  const size_t n_chunks_cdf = (V + CDF_CHUNK - 1) / CDF_CHUNK;
  const size_t Kt = c.tree_chains > 0 ? (size_t)c.tree_chains : 0;
  // draws of one draft (K chains of B), rows of one verify (1 + K (B - 1))
  const size_t rows_any = std::max(std::max(R, S * B), S * Kt * B);
  const size_t v_rows = std::max(B, 1 + Kt * (B - 1));
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  L.len = take(S * 4);
  L.pending = take(S * 4);
  L.iter = take(S * 4);
  L.err = take(4);
  L.sync = take(kSyncCounters * 4);      // hand-off counters of fused launches (zeroed at init)
  L.block_table = take(S * pages_per_seq(c) * 4);
  const size_t rope_rows = (size_t)pages_per_seq(c) * c.page_size;
  L.rope_cos = take(rope_rows * (c.head_dim / 2) * 4);
  L.rope_sin = take(rope_rows * (c.head_dim / 2) * 4);
  L.call_seq = take(S * 4);
  L.call_n = take(S * 4);
  L.call_it = take(S * 4);
  L.row_tok = take(R * 4);
  L.row_pos = take(R * 4);
  L.row_gate = take(R);
  L.row_slot = take(R * 4);
  L.row_vis = take(R * 3 * 4);
  L.row_nc = take(R * 4);
  L.x = take(R * d * 4);
  // activations read by the linear kernels: fragment-tiled in bf16, whole 16-row blocks
  L.xn = take(round16(R) * d * ts);
  L.qbuf = take(R * q * ts);
  L.obuf = take(round16(R) * q * ts);
  L.hbuf = take(round16(R) * F * ts);
  L.ubuf = take(round16(R) * 3 * r * ts + 16);
  // four LoRA intermediates: fixed-point words (few rows, atomics) or room for
  // up to tfx_slices float K-slice partials each (the large-M down-projection)
  L.tfx = take(4 * R * 3 * r * tfx_slices(R) * 8 + 16);
  static_assert(sizeof(long long) == 8, "fixed-point words");
  L.ss = take((size_t)(2 * c.n_layers + 1) * R * SS_BANKS * 8);   // fixed-point sums of x^2
  // Attention partials: a call splits the context into n_chunks <= target chunks,
  // target = ceil(kAttnTargetWG / groups) with groups = n * Hkv * ceil(rows / 16), so
  // rows * n_chunks <= 16 * kAttnTargetWG / Hkv + rows (and <= 64 * rows).  The
  // same buffer holds the K-split slices of the residual products (<= 4 * R * d
  // floats) between a layer's attention and the next.
  L.part_rows = std::min(R * kMaxChunks,
                         (size_t)16 * ((kAttnTargetWG + c.n_kv_heads - 1) / c.n_kv_heads) + 16 + R);
  L.part_o_floats = std::max(L.part_rows * c.n_q_heads * c.head_dim, (size_t)4 * R * d);
  L.part_o = take(L.part_o_floats * 4);
  L.part_ml = take(L.part_rows * c.n_q_heads * 2 * 4);
  L.qkv32 = take(c.qk_norm ? R * (q + 2 * kv) * 4 : 0);
  L.logits = take(R * V * 4);
  L.tile_stats = take(R * (V / 16) * 2 * 4);
  L.row_ml = take(R * 2 * 4);
  L.probs_d = take(S * B * V * 4);
  L.probs_v = take(S * v_rows * V * 4);
  L.desc = take(rows_any * sizeof(RowDesc));
  L.chunk_tot = take(rows_any * n_chunks_cdf * 8);
  L.draft_tok = take(S * B * std::max<size_t>(1, Kt) * 4);
  L.acc_k = take(S * 4);
  L.acc_z = take(S * 4);
  L.aux_i32 = take(rows_any * 4);
  L.tv = take(R * 4);
  L.tree_res = take(Kt ? S * V * 8 : 0);
  L.tree_path = take(S * B * 4);
  L.tree_kstar = take(S * 4);
  L.total = o;
  return L;
}

}  // namespace

struct uno_ctx {
  uno_config cfg{};
  bool bf16 = false;
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  void* kv = nullptr;
  Layout L{};
  int maxpp = 0;
  // weights
  const void* embed = nullptr;
  const void* lm_head = nullptr;
  const void* final_norm = nullptr;
  std::vector<const void*> attn_norm, mlp_norm, w[7], la[7], lb[7];
  std::vector<const void*> q_norm, k_norm;   // QK RMSNorm gains (qk_norm contexts)
  bool has_lora = false;
  // host page bookkeeping
  std::vector<int> free_pages;
  std::vector<std::vector<int>> seq_pages;
  std::vector<int> len_hi;          // upper bound of each committed length
  std::vector<char> live;           // sequence has been prefilled / imported
  std::vector<uint32_t> epoch;      // bumped when a slot's sequence is replaced
  std::vector<int> pt_idx, pt_val;  // pending block-table writes
  std::vector<int> uploaded_call;   // call_seq contents on the device
  // draft bookkeeping
  std::vector<int> drafted_ids;
  int drafted_tree = 0;             // chains of the pending draft (0: a linear draft)
  // asynchronous length snapshot
  int32_t* snap_host = nullptr;
  hipEvent_t snap_event = nullptr;
  bool snap_inflight = false;
  std::vector<int> snap_base;
  std::vector<uint32_t> snap_epoch;
  // producer counts issued so far on each hand-off counter (their targets)
  uint32_t sync_issued[kSyncCounters] = {};   // [group][row tile]
  // activation checkpoint of the distillation forward (uno_set_distill_checkpoint)
  float* ck_x = nullptr;
  void* ck_k = nullptr;
  void* ck_v = nullptr;
  int ck_batch = 0, ck_L = 0;
  // stage capture
  bool trace_on = false;
  uno_trace trace{};
  // kernel timing
  uint32_t tmask = 0;
  int32_t tperiod = 1;                  // record every tperiod-th call of a class
  uint64_t tcalls[UNO_KC_COUNT] = {};
  std::vector<hipEvent_t> tev;          // event pool, two per recorded launch
  struct TRec { int cls; int ev; double bytes, flops; bool call; };
  std::vector<TRec> trec;
  std::string err;

  template <typename P> P* at(size_t off) { return reinterpret_cast<P*>(ws + off); }
};

namespace {

uno_status fail(uno_ctx* c, uno_status s, const std::string& msg) {
  if (c) c->err = msg;
  g_last_error = msg;
  return s;
}

uno_status hip_fail(uno_ctx* c, hipError_t e, const char* where) {
  return fail(c, UNO_ERR_DEVICE, std::string(where) + ": " + hipGetErrorString(e));
}

#define UNO_HIP(ctx, call)                                   \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, #call);   \
  } while (0)

constexpr int kTimedLaunches = 32768;
}  // namespace

thread_local KernelTimer* g_kernel_timer = nullptr;

int32_t uno_fail_global(int32_t status, const char* msg) {
  g_last_error = msg;
  return status;
}

namespace {

// Arms the kernel timer for the launches of one call of a timed class: each of
// its kernels gets an event pair stamped with that kernel's start and end; the
// call's algorithmic bytes and flops go with its first kernel.
struct Timed : KernelTimer {
  uno_ctx* c;
  int cls;
  double bytes, flops;
  bool first = true;
  KernelTimer* saved;
  Timed(uno_ctx* c_, int cls_, double b, double f)
      : c(c_), cls(cls_), bytes(b), flops(f), saved(g_kernel_timer) {
    g_kernel_timer = ((c->tmask >> cls) & 1u) && c->tcalls[cls]++ % (uint64_t)c->tperiod == 0
                         ? this : nullptr;
  }
  ~Timed() { g_kernel_timer = saved; }
  bool next(hipEvent_t* e0, hipEvent_t* e1) override {
    const size_t i = c->trec.size() * 2;
    if (i + 2 > c->tev.size()) return false;
    *e0 = c->tev[i];
    *e1 = c->tev[i + 1];
    c->trec.push_back({cls, (int)i, first ? bytes : 0.0, first ? flops : 0.0, first});
    first = false;
    return true;
  }
};

// Algorithmic bytes and flops of one gated-LoRA linear launch: every weight,
// LoRA, activation and output element read or written once.
void gemm_cost(const GemmArgs& a, int ncols, size_t ts, double* bytes, double* flops) {
  const double M = a.M, K = a.K, r = a.r;
  const double wcols = a.paired ? 2.0 * ncols : (double)ncols;
  double b = wcols * K * ts + M * K * ts;
  double f = 2.0 * M * wcols * K;
  if (r > 0) {
    int nl = 0;
    for (int i = 0; i < a.nseg; ++i) if (a.seg[i].Bl) ++nl;
    const double lcols = a.paired ? 2.0 * ncols : (double)ncols;
    b += lcols * r * ts + M * r * nl * ts;
    f += 2.0 * M * lcols * r;
  }
  if (a.n_prod > 0) {   // fused LoRA down-projection: its A, the input and the atomics
    const double nc = (double)a.ld.nproj * a.ld.r;
    b += nc * a.ld.K * ts + M * nc * 8;
    f += 2.0 * M * nc * a.ld.K;
  }
  switch (a.epi) {
    case EPI_STORE_F32: b += M * ncols * 4; break;
    case EPI_LORA_U: b += M * ncols * ts; break;
    case EPI_RESID: b += M * ncols * 8; break;
    case EPI_SWIGLU: b += M * ncols * ts; break;
    case EPI_LOGITS: b += M * ncols * 4 + M * (ncols / 16) * 8; break;
    default: break;
  }
  *bytes = b;
  *flops = f;
}

uno_status check_config(const uno_config* c) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null config");
  if (c->n_layers < 1 || c->d_model < 16 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 2 || c->ffn_dim < 16 || c->vocab < 16 || c->max_seqs < 1 ||
      c->max_seq_len < 2 || c->page_size < 1 || c->n_pages < 1 || c->block_size < 1)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "config sizes out of range");
  if (c->mask_id != c->vocab - 1) return fail(nullptr, UNO_ERR_INVALID_ARG, "mask_id must be vocab-1");
  if (c->block_size > 64) return fail(nullptr, UNO_ERR_UNSUPPORTED, "block_size > 64");
  if (c->n_q_heads % c->n_kv_heads) return fail(nullptr, UNO_ERR_INVALID_ARG, "Hq % Hkv != 0");
  if (c->head_dim % 2 || c->head_dim > 256) return fail(nullptr, UNO_ERR_UNSUPPORTED, "head_dim");
  if (16 * (c->n_q_heads / c->n_kv_heads) * c->head_dim > 256 * 64)
    return fail(nullptr, UNO_ERR_UNSUPPORTED, "query group too large for the attention tile");
  if (c->vocab % 16 || c->d_model % 16 || c->ffn_dim % 16 ||
      (c->n_q_heads * c->head_dim) % 16 || (c->n_kv_heads * c->head_dim) % 16)
    return fail(nullptr, UNO_ERR_UNSUPPORTED, "dimensions must be multiples of 16");
  if (c->vocab > CDF_CHUNK * 1024) return fail(nullptr, UNO_ERR_UNSUPPORTED, "vocab too large");
  if (c->dtype != UNO_F32 && c->dtype != UNO_BF16) return fail(nullptr, UNO_ERR_INVALID_ARG, "dtype");
  if (c->dtype == UNO_BF16) {
    if (c->d_model % 32 || c->ffn_dim % 32 || (c->n_q_heads * c->head_dim) % 32)
      return fail(nullptr, UNO_ERR_UNSUPPORTED, "bf16 needs K dims multiple of 32");
    if (c->lora_rank % 32) return fail(nullptr, UNO_ERR_UNSUPPORTED, "bf16 LoRA rank % 32");
  }
  if (c->lora_rank < 0) return fail(nullptr, UNO_ERR_INVALID_ARG, "lora_rank < 0");
  if (c->lora_rank > 0 && c->lora_rank % 8 && c->dtype == UNO_F32)
    return fail(nullptr, UNO_ERR_UNSUPPORTED, "lora rank");
  if (c->max_rows < c->max_seqs * c->block_size)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "max_rows < max_seqs * block_size");
  if (!(c->top_p >= 0.0f)) return fail(nullptr, UNO_ERR_INVALID_ARG, "top_p < 0 or NaN");
  if (c->qk_norm != 0 && c->qk_norm != 1) return fail(nullptr, UNO_ERR_INVALID_ARG, "qk_norm must be 0 or 1");
  if (c->tree_chains < 0 || c->tree_chains > TREE_KMAX)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "tree_chains must be 0..16");
  return UNO_OK;
}

// Nucleus truncation of a block of probability rows in place, when the config asks.
bool top_p_on(const uno_config& c) { return c.top_p > 0.0f && c.top_p < 1.0f; }

size_t kv_bytes(const uno_config& c) {
  const size_t ts = c.dtype == UNO_BF16 ? 2 : 4;
  return (size_t)c.n_layers * 2 * c.n_pages * c.n_kv_heads * c.page_size * c.head_dim * ts;
}

KvLayout kv_layout(uno_ctx* c) {
  KvLayout k{};
  k.pool = c->kv;
  k.n_pages = c->cfg.n_pages;
  k.n_kv_heads = c->cfg.n_kv_heads;
  k.page_size = c->cfg.page_size;
  k.head_dim = c->cfg.head_dim;
  k.n_layers = c->cfg.n_layers;
  k.block_table = c->at<int32_t>(c->L.block_table);
  k.max_pages_per_seq = c->maxpp;
  k.page_shift = -1;
  for (int b = 0; b < 31; ++b)
    if (k.page_size == (1 << b)) k.page_shift = b;
  return k;
}

// Scatter a list of int32 values into device memory (kernel arguments carry the
// data, so nothing is staged in host memory).
uno_status scatter(uno_ctx* c, int32_t* dst, const std::vector<int>& idx,
                   const std::vector<int>& val) {
  for (size_t a = 0; a < idx.size(); a += 240) {
    SetList l{};
    l.dst = dst;
    l.count = (int)std::min<size_t>(240, idx.size() - a);
    for (int i = 0; i < l.count; ++i) { l.idx[i] = idx[a + i]; l.val[i] = val[a + i]; }
    UNO_HIP(c, launch_set_list(l, c->stream));
  }
  return UNO_OK;
}

uno_status flush_pages(uno_ctx* c) {
  if (c->pt_idx.empty()) return UNO_OK;
  uno_status s = scatter(c, c->at<int32_t>(c->L.block_table), c->pt_idx, c->pt_val);
  c->pt_idx.clear();
  c->pt_val.clear();
  return s;
}

// Reserve pages so that each sequence holds positions [0, upto[i]).  All or nothing.
uno_status reserve(uno_ctx* c, const std::vector<int>& seqs, const std::vector<int>& upto) {
  const int ps = c->cfg.page_size;
  size_t need = 0;
  for (size_t i = 0; i < seqs.size(); ++i) {
    const int want = (upto[i] + ps - 1) / ps;
    if (upto[i] > c->cfg.max_seq_len || want > c->maxpp)
      return fail(c, UNO_ERR_INVALID_ARG, "sequence would exceed max_seq_len");
    const int have = (int)c->seq_pages[seqs[i]].size();
    if (want > have) need += want - have;
  }
  if (need > c->free_pages.size()) return fail(c, UNO_ERR_OUT_OF_PAGES, "KV page pool exhausted");
  for (size_t i = 0; i < seqs.size(); ++i) {
    const int want = (upto[i] + ps - 1) / ps;
    auto& pg = c->seq_pages[seqs[i]];
    while ((int)pg.size() < want) {
      const int p = c->free_pages.back();
      c->free_pages.pop_back();
      c->pt_idx.push_back(seqs[i] * c->maxpp + (int)pg.size());
      c->pt_val.push_back(p);
      pg.push_back(p);
    }
  }
  return UNO_OK;
}

uno_status upload_call(uno_ctx* c, const std::vector<int>& seqs) {
  std::vector<int> idx, val;
  if (c->uploaded_call.size() < seqs.size()) c->uploaded_call.resize(seqs.size(), -1);
  for (size_t i = 0; i < seqs.size(); ++i)
    if (c->uploaded_call[i] != seqs[i]) {
      idx.push_back((int)i);
      val.push_back(seqs[i]);
      c->uploaded_call[i] = seqs[i];
    }
  return scatter(c, c->at<int32_t>(c->L.call_seq), idx, val);
}

// Fold a finished length snapshot into the host bounds.  A slot whose sequence
// was released, prefilled or imported after the snapshot was taken (its epoch
// moved on) keeps its bound: the snapshot describes the previous sequence.
void poll_snapshot(uno_ctx* c) {
  if (!c->snap_inflight) return;
  if (hipEventQuery(c->snap_event) != hipSuccess) return;
  for (int s = 0; s < c->cfg.max_seqs; ++s)
    if (c->live[s] && c->epoch[s] == c->snap_epoch[s])
      c->len_hi[s] = c->snap_host[s] + (c->len_hi[s] - c->snap_base[s]);
  c->snap_inflight = false;
}

// The slot's sequence is replaced (release, prefill, import).
void new_epoch(uno_ctx* c, int s) { ++c->epoch[s]; }

uno_status start_snapshot(uno_ctx* c) {
  if (c->snap_inflight) return UNO_OK;
  UNO_HIP(c, hipMemcpyAsync(c->snap_host, c->at<int32_t>(c->L.len),
                            sizeof(int32_t) * c->cfg.max_seqs, hipMemcpyDeviceToHost, c->stream));
  UNO_HIP(c, hipEventRecord(c->snap_event, c->stream));
  c->snap_base = c->len_hi;
  c->snap_epoch = c->epoch;
  c->snap_inflight = true;
  return UNO_OK;
}

uno_status exact_lengths(uno_ctx* c) {
  UNO_HIP(c, hipStreamSynchronize(c->stream));
  c->snap_inflight = false;
  std::vector<int32_t> lens(c->cfg.max_seqs);
  UNO_HIP(c, hipMemcpy(lens.data(), c->at<int32_t>(c->L.len), sizeof(int32_t) * lens.size(),
                       hipMemcpyDeviceToHost));
  for (int s = 0; s < c->cfg.max_seqs; ++s)
    if (c->live[s]) c->len_hi[s] = lens[s];
  return UNO_OK;
}

uno_status check_seqs(uno_ctx* c, int32_t n, const int32_t* ids, std::vector<int>& out,
                      bool need_live) {
  if (n < 1 || n > c->cfg.max_seqs || !ids) return fail(c, UNO_ERR_INVALID_ARG, "bad sequence count");
  out.assign(ids, ids + n);
  std::vector<char> seen(c->cfg.max_seqs, 0);
  for (int s : out) {
    if (s < 0 || s >= c->cfg.max_seqs) return fail(c, UNO_ERR_INVALID_ARG, "sequence id out of range");
    if (seen[s]) return fail(c, UNO_ERR_INVALID_ARG, "duplicate sequence id");
    seen[s] = 1;
    if (need_live && !c->live[s]) return fail(c, UNO_ERR_STATE, "sequence not prefilled");
  }
  return UNO_OK;
}

// ----------------------------------------------------------------- forward plan
struct FwdIn {
  int mode;                 // RowsSetup mode
  int n, rows_per_seq;
  const int32_t* in_tok;
  const float* in_hidden;
  const int32_t* in_pos;
  const uint8_t* in_gate;
  int pos0;
  int ctx_bound;            // every row position is < ctx_bound
  bool lora;                // run the LoRA phase (some gate may be on)
  float* hidden_out;
  float* probs_out;         // softmax of the logits (nullptr: no LM head)
  float* logits_out;        // copy of the logits (optional)
  // distillation forward (mode 4): rows [x | MASK^L] per sequence, block size dB;
  // teacher / student logits [n, L, V] (nullptr: workspace), per-row TV [n, L]
  // (nullptr: workspace) and per-block TV [n, L / dB] (nullptr: not formed)
  int dB;
  int tree_K;               // mode 5: chains per sequence
  float* teacher;
  float* student;
  float* tv_row;
  float* tv_block;
  // activation checkpoint of the distillation forward: the z1 rows' residual
  // stream entering layer l goes to ck_x + l * ck_stride (rows of the group's
  // sequences in order, [n * L, d]); slot n_layers takes the stream before the LM head
  float* ck_x;
  size_t ck_stride;
};

template <typename T>
uno_status forward_t(uno_ctx* c, const FwdIn& f) {
  const uno_config& g = c->cfg;
  hipStream_t s = c->stream;
  const int R = f.n * f.rows_per_seq;
  const int d = g.d_model, hd = g.head_dim, Hq = g.n_q_heads, Hkv = g.n_kv_heads;
  const int qd = Hq * hd, kvd = Hkv * hd, F = g.ffn_dim, V = g.vocab, r = g.lora_rank;
  const int L = g.n_layers;
  const bool lora = f.lora && c->has_lora && r > 0;
  const float sc = lora ? g.lora_alpha / (float)r : 0.0f;
  int32_t* err = c->at<int32_t>(c->L.err);

  RowsSetup rs{};
  rs.mode = f.mode;
  rs.n = f.n;
  rs.rows_per_seq = f.rows_per_seq;
  rs.B = g.block_size;
  rs.mask_id = g.mask_id;
  rs.call_seq = c->at<int32_t>(c->L.call_seq);
  rs.len = c->at<int32_t>(c->L.len);
  rs.pending = c->at<int32_t>(c->L.pending);
  rs.iter = c->at<int32_t>(c->L.iter);
  rs.draft_tok = c->at<int32_t>(c->L.draft_tok);
  rs.in_tok = f.in_tok;
  rs.in_pos = f.in_pos;
  rs.in_gate = f.in_gate;
  rs.pos0 = f.pos0;
  rs.row_tok = c->at<int32_t>(c->L.row_tok);
  rs.row_pos = c->at<int32_t>(c->L.row_pos);
  rs.row_gate = c->at<uint8_t>(c->L.row_gate);
  rs.row_slot = c->at<int32_t>(c->L.row_slot);
  rs.row_vis = c->at<int32_t>(c->L.row_vis);
  if (f.mode == 4) rs.B = f.dB;
  rs.K = f.tree_K;
  // rows whose K/V slot and visible window are given per row (not by position)
  const bool windowed = f.mode == 4 || f.mode == 5;
  rs.call_n = c->at<int32_t>(c->L.call_n);
  rs.call_it = c->at<int32_t>(c->L.call_it);
  {
    Timed t(c, UNO_KC_MISC, 0, 0);
    UNO_HIP(c, launch_rows_setup(rs, s));
  }

  float* x = c->at<float>(c->L.x);
  T* xg = c->at<T>(c->L.xn);      // gain-scaled RMSNorm input of the next consumer
  T* qbuf = c->at<T>(c->L.qbuf);
  T* obuf = c->at<T>(c->L.obuf);
  T* hbuf = c->at<T>(c->L.hbuf);
  T* ubuf = c->at<T>(c->L.ubuf);
  const uint8_t* gate = c->at<uint8_t>(c->L.row_gate);
  // fixed-point sums of x^2 per row: [2l] before attention of layer l, [2l+1]
  // before its MLP, [2L] before the LM head; SS_BANKS words per row
  long long* ssb = c->at<long long>(c->L.ss);
  auto SS = [&](int i) { return ssb + (size_t)i * R * SS_BANKS; };
  // stage capture of the armed trace (row-major copies into caller buffers)
  auto traced = [&](int l) -> const uno_trace_layer* {
    if (!c->trace_on) return nullptr;
    for (int i = 0; i < c->trace.n; ++i)
      if (c->trace.layer[i].layer == l) return &c->trace.layer[i];
    return nullptr;
  };
  auto cap_x = [&](float* dst) -> uno_status {
    if (dst) UNO_HIP(c, hipMemcpyAsync(dst, c->at<float>(c->L.x), sizeof(float) * R * d,
                                       hipMemcpyDeviceToDevice, s));
    return UNO_OK;
  };
  auto cap_act = [&](void* dst, const T* src, int cols) -> uno_status {
    if (dst) UNO_HIP(c, launch_untile<T>(src, reinterpret_cast<T*>(dst), R, cols, s));
    return UNO_OK;
  };
  // LoRA down-projection of each group (buffer b): qkv, o, gate/up, down.  Large M
  // (every group fits the tile kernel): tsl[b] K-slice float partials stored into
  // the tfx region, summed in slice order, gated and scaled into ubuf -- no
  // atomics, nothing to clear.  Few rows: integer atomics into buffer b, cleared by a later kernel.
  const int gK[4] = {d, qd, d, F}, gN[4] = {3 * r, r, 2 * r, r};
  long long* tfx = c->at<long long>(c->L.tfx);
  const size_t tcap = (size_t)c->cfg.max_rows * 3 * r * tfx_slices(c->cfg.max_rows) * 4;
  int tsl[4] = {0, 0, 0, 0};
  bool tile_lora = lora && c->bf16;
  for (int b = 0; b < 4 && tile_lora; ++b) {
    tsl[b] = lora_down_tile_slices(R, gK[b], gN[b]);
    while (tsl[b] > 1 && (size_t)tsl[b] * R * gN[b] > tcap) tsl[b] /= 2;
    tile_lora = lora_down_tile_fits(R, gK[b], gN[b], tsl[b]);
  }
  const size_t tstride = (size_t)R * 3 * r;
  long long* Bfx[4] = {tfx, tfx + tstride, tfx + 2 * tstride, tfx + 3 * tstride};
  {
    Timed t(c, UNO_KC_MISC, 0, 0);
    UNO_HIP(c, launch_zero_i64(ssb, (size_t)(2 * L + 1) * R * SS_BANKS, s));
    if (lora && c->bf16 && !tile_lora) UNO_HIP(c, launch_zero_i64(tfx, 4 * tstride, s));
  }
  if (!f.in_hidden && !c->embed) return fail(c, UNO_ERR_INVALID_ARG, "no embedding table");
  {
    Timed t(c, UNO_KC_MISC, 0, 0);
    UNO_HIP(c, launch_embed<T>(reinterpret_cast<const T*>(c->embed), rs.row_tok, f.in_hidden,
                               R, d, V, x, reinterpret_cast<const T*>(c->attn_norm[0]), xg,
                               SS(0), err, s));
  }

  KvLayout kv = kv_layout(c);
  // attention chunking: split the context until ~1024 workgroups exist (a large
  // batch provides them unsplit, which also saves the partial-merge pass), 64-key
  // multiples, at most kMaxChunks chunks
  // a single-sequence call names its sequence in the kernel arguments
  const int seq_fixed = (f.n == 1 && !c->uploaded_call.empty()) ? c->uploaded_call[0] + 1 : 0;
  const int row_tiles = (f.rows_per_seq + 15) / 16;
  const int groups = f.n * Hkv * row_tiles;
  int target = std::max(1, std::min(kMaxChunks, (kAttnTargetWG + groups - 1) / groups));
  // windowed rows number a tile's keys in whole pages of both ranges: up to 48
  // more than its rows' slots span
  const int ctxb = f.ctx_bound + (windowed ? 48 : 0);
  int chunk = (ctxb + target - 1) / target;
  chunk = std::max(kAttnMinChunk, (chunk + kAttnMinChunk - 1) / kAttnMinChunk * kAttnMinChunk);
  const int n_chunks = (ctxb + chunk - 1) / chunk;
  if (n_chunks > kMaxChunks || (size_t)R * n_chunks > c->L.part_rows)
    return fail(c, UNO_ERR_INVALID_ARG, "attention chunking exceeds the partial buffers");

  auto run_gemm = [&](const GemmArgs& a0, int ncols, int cls) -> uno_status {
    GemmArgs a = a0;
    a.err = err;
    double b, fl;
    gemm_cost(a, ncols, sizeof(T), &b, &fl);
    Timed t(c, cls, b, fl);
    UNO_HIP(c, launch_gemm<T>(a, ncols, s));
    return UNO_OK;
  };
  // the attention partials are free between a layer's combine and the next
  // layer's attention: the o and down products may split K into them
  auto split_ws = [&](GemmArgs& a) {
    a.split_ws = c->at<float>(c->L.part_o);
    a.split_cap = (long long)c->L.part_o_floats;
  };
  auto norm_in = [&](GemmArgs& a, int ss_idx) {
    a.ss_in = SS(ss_idx); a.inv_d = 1.0f / (float)d; a.eps = g.rms_eps;
  };
  // LoRA down-projections.  bf16: fixed-point buffers B0..B3 (qkv, o, gate/up,
  // down).  Large M: the tile kernel stores tsl[buf] K-slice partials.  Few rows:
  // split-K MFMA with integer atomics into a buffer that a later kernel of the
  // chain cleared (the zero_ptr of the consumer GEMMs; all cleared once per
  // forward above).  float32: a GEMM storing the gated, scaled intermediate.
  auto lora_down = [&](const T* X, int K, int nproj, const int* pidx, int l, int buf,
                       int ss_idx) -> uno_status {
    if (tile_lora) {
      GemmArgs a{};
      a.X = X; a.ldx = K; a.M = R; a.K = K; a.r = 0;
      a.nseg = nproj;
      a.err = err;
      for (int i = 0; i < nproj; ++i) {
        a.seg[i].W = c->la[pidx[i]][l];
        a.seg[i].n0 = i * r;
        a.seg[i].N = r;
      }
      if (ss_idx >= 0) norm_in(a, ss_idx);
      const int nc = nproj * r;
      a.epi = EPI_TSLICE; a.ldo = nc; a.out = tfx;
      a.k_slices = tsl[buf]; a.slice_stride = (long long)R * nc;
      double b, fl;
      gemm_cost(a, nc, sizeof(T), &b, &fl);
      // slices written, then read back with the gates; u written
      b += (double)R * nc * 4 * tsl[buf] * 2 + (double)R + (double)R * nc * sizeof(T);
      Timed t(c, UNO_KC_LORA_DOWN, b, fl);
      UNO_HIP(c, launch_lora_down_tile(a, nc, s));
      UNO_HIP(c, launch_lora_u(reinterpret_cast<const float*>(tfx), tsl[buf], a.slice_stride, R, nc, gate, sc,
                               reinterpret_cast<bf16*>(ubuf), s));
      return UNO_OK;
    }
    if (c->bf16) {
      LoraDownArgs a{};
      a.X = X; a.ldx = K; a.M = R; a.K = K; a.r = r; a.nproj = nproj; a.t = Bfx[buf];
      a.err = err;
      if (ss_idx >= 0) { a.ss_in = SS(ss_idx); a.inv_d = 1.0f / (float)d; a.eps = g.rms_eps; }
      for (int i = 0; i < nproj; ++i) a.A[i] = c->la[pidx[i]][l];
      // about 128 workgroups: K chunks of whole 32-wide blocks
      const int tiles = nproj * r / 16 * ((R + 15) / 16);
      const int tgt = std::max(1, (128 + tiles - 1) / tiles);
      int ks = 1;
      for (int cand = 1; cand <= K / 32; ++cand)
        if ((K / 32) % cand == 0 && cand <= tgt) ks = cand;
      a.kchunk = K / ks;
      const double b = (double)nproj * r * K * sizeof(T) + (double)R * K * sizeof(T) +
                       (double)R * nproj * r * 8 * 2;
      Timed t(c, UNO_KC_LORA_DOWN, b, 2.0 * R * nproj * r * K);
      UNO_HIP(c, launch_lora_down(a, s));
      return UNO_OK;
    }
    GemmArgs a{};
    a.X = X; a.ldx = K; a.M = R; a.K = K; a.r = 0;
    a.nseg = nproj;
    for (int i = 0; i < nproj; ++i) {
      a.seg[i].W = c->la[pidx[i]][l];
      a.seg[i].n0 = i * r;
      a.seg[i].N = r;
    }
    if (ss_idx >= 0) norm_in(a, ss_idx);
    a.epi = EPI_LORA_U; a.ldo = nproj * r; a.out = ubuf; a.gate = gate; a.scale = sc;
    return run_gemm(a, nproj * r, UNO_KC_LORA_DOWN);
  };
  // Few rows (the skinny kernel): the group's LoRA down-projection runs inside the
  // consumer launch as its first workgroups (GemmArgs::n_prod), which saves a
  // launch per group; the consumers wait for it only before their LoRA phase.
  const bool fuse_lora = lora && c->bf16 && !tile_lora && R < 64;
  auto fuse_down = [&](GemmArgs& a, const T* X, int K, int nproj, const int* pidx, int l, int buf,
                       int ss_idx) {
    LoraDownArgs& d2 = a.ld;
    d2.X = X; d2.ldx = K; d2.M = R; d2.K = K; d2.r = r; d2.nproj = nproj; d2.t = Bfx[buf];
    d2.err = err;
    if (ss_idx >= 0) { d2.ss_in = SS(ss_idx); d2.inv_d = 1.0f / (float)d; d2.eps = g.rms_eps; }
    for (int i = 0; i < nproj; ++i) d2.A[i] = c->la[pidx[i]][l];
    // about 128 producer workgroups per row tile: K chunks of whole 32-wide blocks
    const int tiles = nproj * r / 16;
    const int tgt = std::max(1, (128 + tiles - 1) / tiles);
    int ks = 1;
    for (int cand = 1; cand <= K / 32; ++cand)
      if ((K / 32) % cand == 0 && cand <= tgt) ks = cand;
    d2.kchunk = K / ks;
    a.n_prod = tiles * ks;
    a.sync = c->at<uint32_t>(c->L.sync) + 4 * buf;
    for (int mt = 0; mt < (R + 15) / 16; ++mt) {
      c->sync_issued[4 * buf + mt] += (uint32_t)a.n_prod;
      a.sync_target[mt] = c->sync_issued[4 * buf + mt];
    }
  };
  // attach the LoRA up-projection of segment `i` reading group buffer `buf`
  auto lora_up = [&](GemmArgs& a, int i, int proj, int l, int buf, int col, int ld) {
    a.seg[i].Bl = c->lb[proj][l];
    if (c->bf16 && !tile_lora) {
      a.seg[i].Ufx = Bfx[buf] + col;
    } else if (c->bf16) {
      a.seg[i].U = ubuf;          // fragment-tiled [R, ld], this segment at column col
      a.seg[i].ucol = col;
    } else {
      a.seg[i].U = ubuf + col;
    }
    a.seg[i].ldu = ld;
    a.gate = gate;
    a.scale = sc;
  };
  auto clear = [&](GemmArgs& a, int buf, int cols) {
    if (lora && c->bf16 && !tile_lora) { a.zero_ptr = Bfx[buf]; a.zero_n = R * cols; }
  };

  // z1 rows of every sequence of the group into checkpoint slot i
  auto cap_ck = [&](int i) -> uno_status {
    if (f.mode != 4 || !f.ck_x) return UNO_OK;
    const size_t Lx = f.rows_per_seq / 2;
    UNO_HIP(c, hipMemcpy2DAsync(f.ck_x + (size_t)i * f.ck_stride, Lx * d * sizeof(float),
                                x + Lx * d, (size_t)f.rows_per_seq * d * sizeof(float),
                                Lx * d * sizeof(float), f.n, hipMemcpyDeviceToDevice, s));
    return UNO_OK;
  };

  for (int l = 0; l < L; ++l) {
    const uno_trace_layer* tr = traced(l);
    if (tr) { if (uno_status st = cap_x(tr->x_in)) return st; }
    if (uno_status st = cap_ck(l)) return st;
    // --- attention block: q|k|v (+LoRA) with RoPE and the paged K/V write
    static const int pqkv[3] = {0, 1, 2};
    if (lora && !fuse_lora) { uno_status st = lora_down(xg, d, 3, pqkv, l, 0, 2 * l); if (st) return st; }
    {
      GemmArgs a{};
      if (fuse_lora) fuse_down(a, xg, d, 3, pqkv, l, 0, 2 * l);
      a.X = xg; a.ldx = d; a.M = R; a.K = d; a.r = lora ? r : 0;
      a.nseg = 3;
      const int n0s[3] = {0, qd, qd + kvd}, Ns[3] = {qd, kvd, kvd};
      for (int i = 0; i < 3; ++i) {
        a.seg[i].W = c->w[i][l];
        a.seg[i].n0 = n0s[i];
        a.seg[i].N = Ns[i];
        if (lora) lora_up(a, i, i, l, 0, i * r, 3 * r);
      }
      clear(a, 3, r);
      norm_in(a, 2 * l);
      const int32_t* slot = windowed ? rs.row_slot : nullptr;
      if (!c->cfg.qk_norm) {
        a.epi = EPI_QKV;
        a.row_pos = rs.row_pos; a.call_seq = rs.call_seq; a.rows_per_seq = f.rows_per_seq;
        a.seq_fixed = seq_fixed;
        a.row_slot = slot;
        a.n_q_heads = Hq; a.rcos = c->at<float>(c->L.rope_cos); a.rsin = c->at<float>(c->L.rope_sin);
        a.qbuf = qbuf; a.kv = kv; a.layer = l; a.err = err;
        if (uno_status st = run_gemm(a, qd + 2 * kvd, UNO_KC_LINEAR)) return st;
      } else {
        // QK RMSNorm: the head's norm spans tiles of several workgroups, so the
        // projection is stored as float32 and a row kernel normalises, rotates and
        // writes q and the pages
        float* y = c->at<float>(c->L.qkv32);
        a.epi = EPI_STORE_F32; a.ldo = qd + 2 * kvd; a.out = y;
        if (uno_status st = run_gemm(a, qd + 2 * kvd, UNO_KC_LINEAR)) return st;
        QkNormArgs qa{};
        qa.in = y; qa.ldi = qd + 2 * kvd; qa.M = R; qa.n_q_heads = Hq; qa.perm = c->bf16 ? 1 : 0;
        qa.q_gain = c->q_norm[l]; qa.k_gain = c->k_norm[l]; qa.eps = g.rms_eps;
        qa.row_pos = rs.row_pos; qa.row_slot = slot; qa.call_seq = rs.call_seq;
        qa.seq_fixed = seq_fixed; qa.rows_per_seq = f.rows_per_seq;
        qa.rcos = c->at<float>(c->L.rope_cos); qa.rsin = c->at<float>(c->L.rope_sin);
        qa.qbuf = qbuf; qa.kv = kv; qa.layer = l; qa.err = err;
        Timed t(c, UNO_KC_MISC, (double)R * (qd + 2 * kvd) * (4 + sizeof(T)), 0);
        UNO_HIP(c, launch_qk_norm_rope<T>(qa, s));
      }
    }
    if (tr && tr->q)
      UNO_HIP(c, hipMemcpyAsync(tr->q, qbuf, sizeof(T) * R * qd, hipMemcpyDeviceToDevice, s));
    {
      AttnArgs a{};
      a.q = qbuf; a.out = obuf; a.row_pos = rs.row_pos; a.call_seq = rs.call_seq;
      a.seq_fixed = seq_fixed;
      a.row_vis = windowed ? rs.row_vis : nullptr;
      a.row_nc = c->at<int32_t>(c->L.row_nc);
      a.err = err;
      a.n = f.n; a.rows_per_seq = f.rows_per_seq; a.n_q_heads = Hq;
      a.n_chunks = n_chunks; a.chunk = chunk; a.scale = 1.0f / sqrtf((float)hd);
      a.part_o = c->at<float>(c->L.part_o); a.part_ml = c->at<float>(c->L.part_ml);
      a.layer = l;
      // algorithmic bytes: queries, every visible K/V row of each sequence once
      // (bounded by ctx_bound; [x, z1]: 2L rows), partials written and read, outputs
      const double kv_rows = f.mode == 4 ? (double)f.rows_per_seq : (double)f.ctx_bound;
      const double kvb = (double)f.n * kv_rows * Hkv * hd * 2 * sizeof(T);
      const double pb = n_chunks > 1 ? (double)R * Hq * n_chunks * (hd + 2) * 4 * 2 : 0.0;
      const double io = (double)R * qd * sizeof(T) * 2;
      // flops: 4 * hd per (query head, visible key); [x, z1] row i sees i + 1 keys
      const double Lx = f.rows_per_seq / 2.0;
      const double fl = f.mode == 4 ? 4.0 * f.n * Hq * hd * Lx * (Lx + 1.0)
                                    : 4.0 * R * Hq * hd * (double)f.ctx_bound;
      Timed t(c, UNO_KC_ATTENTION, kvb + pb + io, fl);
      UNO_HIP(c, launch_attention<T>(a, kv, s));
    }
    if (tr) { if (uno_status st = cap_act(tr->attn, obuf, qd)) return st; }
    static const int po[1] = {3};
    if (lora && !fuse_lora) { uno_status st = lora_down(obuf, qd, 1, po, l, 1, -1); if (st) return st; }
    {
      GemmArgs a{};
      if (fuse_lora) fuse_down(a, obuf, qd, 1, po, l, 1, -1);
      a.X = obuf; a.ldx = qd; a.M = R; a.K = qd; a.r = lora ? r : 0;
      a.nseg = 1;
      a.seg[0].W = c->w[3][l]; a.seg[0].n0 = 0; a.seg[0].N = d;
      if (lora) lora_up(a, 0, 3, l, 1, 0, r);
      clear(a, 0, 3 * r);
      a.epi = EPI_RESID; a.ldo = d; a.resid = x;
      a.xg_out = xg; a.g_next = c->mlp_norm[l]; a.ss_out = SS(2 * l + 1);
      split_ws(a);
      if (uno_status st = run_gemm(a, d, UNO_KC_LINEAR)) return st;
    }
    if (tr) { if (uno_status st = cap_x(tr->x_mid)) return st; }
    // --- MLP block
    static const int pgu[2] = {4, 5};
    if (lora && !fuse_lora) { uno_status st = lora_down(xg, d, 2, pgu, l, 2, 2 * l + 1); if (st) return st; }
    {
      GemmArgs a{};
      if (fuse_lora) fuse_down(a, xg, d, 2, pgu, l, 2, 2 * l + 1);
      a.X = xg; a.ldx = d; a.M = R; a.K = d; a.r = lora ? r : 0;
      a.nseg = 2; a.paired = 1;
      for (int i = 0; i < 2; ++i) {
        a.seg[i].W = c->w[4 + i][l]; a.seg[i].n0 = 0; a.seg[i].N = F;
        if (lora) lora_up(a, i, 4 + i, l, 2, i * r, 2 * r);
      }
      clear(a, 1, r);
      norm_in(a, 2 * l + 1);
      a.epi = EPI_SWIGLU; a.ldo = F; a.out = hbuf;
      if (uno_status st = run_gemm(a, F, UNO_KC_LINEAR_SWIGLU)) return st;
    }
    if (tr) { if (uno_status st = cap_act(tr->act, hbuf, F)) return st; }
    static const int pd[1] = {6};
    if (lora && !fuse_lora) { uno_status st = lora_down(hbuf, F, 1, pd, l, 3, -1); if (st) return st; }
    {
      GemmArgs a{};
      if (fuse_lora) fuse_down(a, hbuf, F, 1, pd, l, 3, -1);
      a.X = hbuf; a.ldx = F; a.M = R; a.K = F; a.r = lora ? r : 0;
      a.nseg = 1;
      a.seg[0].W = c->w[6][l]; a.seg[0].n0 = 0; a.seg[0].N = d;
      if (lora) lora_up(a, 0, 6, l, 3, 0, r);
      clear(a, 2, 2 * r);
      a.epi = EPI_RESID; a.ldo = d; a.resid = x;
      a.xg_out = xg;
      a.g_next = (l + 1 < L) ? c->attn_norm[l + 1] : c->final_norm;
      a.ss_out = SS(2 * l + 2);
      split_ws(a);
      if (uno_status st = run_gemm(a, d, UNO_KC_LINEAR)) return st;
    }
    if (tr) { if (uno_status st = cap_x(tr->x_out)) return st; }
  }
  if (f.hidden_out)
    UNO_HIP(c, hipMemcpyAsync(f.hidden_out, x, sizeof(float) * R * d, hipMemcpyDeviceToDevice, s));
  if (f.mode == 4) {
    if (uno_status st = cap_ck(L)) return st;
    // teacher = x-row logits (AR weights), student = z1-row logits (AR + LoRA)
    if (!c->lm_head) return fail(c, UNO_ERR_INVALID_ARG, "no LM head");
    const int Lx = f.rows_per_seq / 2, nt = V / 16;
    float* lg = c->at<float>(c->L.logits);
    float* ts = c->at<float>(c->L.tile_stats);
    float* ml = c->at<float>(c->L.row_ml);
    std::vector<float*> dst(2 * f.n);
    for (int i = 0; i < f.n; ++i)
      for (int h = 0; h < 2; ++h) {
        const size_t r0 = (size_t)i * f.rows_per_seq + (size_t)h * Lx;
        float* user = h == 0 ? f.teacher : f.student;
        float* o = user ? user + (size_t)i * Lx * V : lg + r0 * V;
        dst[2 * i + h] = o;
        GemmArgs a{};
        a.X = xg + r0 * d;   // r0 is a multiple of 16 in bf16 (a whole fragment block)
        a.ldx = d; a.M = Lx; a.K = d; a.r = 0;
        a.nseg = 1;
        a.seg[0].W = c->lm_head; a.seg[0].n0 = 0; a.seg[0].N = V;
        a.ss_in = SS(2 * L) + r0 * SS_BANKS; a.inv_d = 1.0f / (float)d; a.eps = g.rms_eps;
        a.epi = EPI_LOGITS; a.ldo = V; a.out = o;
        a.mask_col = g.mask_id; a.tile_stats = ts + r0 * nt * 2; a.n_tiles = nt;
        if (uno_status st = run_gemm(a, V, UNO_KC_LM_HEAD)) return st;
      }
    Timed t(c, UNO_KC_SAMPLING, (double)R * V * 4 + (double)R * nt * 8, 0);
    UNO_HIP(c, launch_row_stats(ts, R, nt, ml, s));
    for (int i = 0; i < f.n; ++i) {
      const size_t r0 = (size_t)i * f.rows_per_seq;
      float* tvr = (f.tv_row ? f.tv_row : c->at<float>(c->L.tv)) + (size_t)i * Lx;
      UNO_HIP(c, launch_tv(dst[2 * i], dst[2 * i + 1], ml + r0 * 2, ml + (r0 + Lx) * 2, Lx, V,
                           tvr, s));
      if (f.tv_block)
        UNO_HIP(c, launch_tv_blocks(tvr, Lx, f.dB, f.tv_block + (size_t)i * (Lx / f.dB), s));
    }
    return UNO_OK;
  }
  if (f.probs_out || f.logits_out) {
    if (!c->lm_head) return fail(c, UNO_ERR_INVALID_ARG, "no LM head");
    GemmArgs a{};
    a.X = xg; a.ldx = d; a.M = R; a.K = d; a.r = 0;
    a.nseg = 1;
    a.seg[0].W = c->lm_head; a.seg[0].n0 = 0; a.seg[0].N = V;
    norm_in(a, 2 * L);
    a.epi = EPI_LOGITS; a.ldo = V; a.out = c->at<float>(c->L.logits);
    a.mask_col = g.mask_id; a.tile_stats = c->at<float>(c->L.tile_stats); a.n_tiles = V / 16;
    if (uno_status st = run_gemm(a, V, UNO_KC_LM_HEAD)) return st;
    if (c->trace_on && c->trace.logits)
      UNO_HIP(c, hipMemcpyAsync(c->trace.logits, c->at<float>(c->L.logits), sizeof(float) * R * V,
                                hipMemcpyDeviceToDevice, s));
    if (f.probs_out) {
      Timed t(c, UNO_KC_SAMPLING, (double)R * V * 8 + (double)R * (V / 16) * 8, 0);
      UNO_HIP(c, launch_row_stats(a.tile_stats, R, V / 16, c->at<float>(c->L.row_ml), s));
      UNO_HIP(c, launch_softmax(c->at<float>(c->L.logits), c->at<float>(c->L.row_ml), R, V,
                                f.probs_out, s));
    }
    if (f.logits_out)
      UNO_HIP(c, hipMemcpyAsync(f.logits_out, c->at<float>(c->L.logits), sizeof(float) * R * V,
                                hipMemcpyDeviceToDevice, s));
  }
  return UNO_OK;
}

uno_status forward(uno_ctx* c, const FwdIn& f) {
  return c->bf16 ? forward_t<bf16>(c, f) : forward_t<float>(c, f);
}

uno_status set_state(uno_ctx* c, int seq, int len, int pending, int iter) {
  uno_status st;
  if ((st = scatter(c, c->at<int32_t>(c->L.len), {seq}, {len}))) return st;
  if ((st = scatter(c, c->at<int32_t>(c->L.pending), {seq}, {pending}))) return st;
  return scatter(c, c->at<int32_t>(c->L.iter), {seq}, {iter});
}

}  // namespace

// ====================================================================== C ABI
// top-p truncation of `rows` probability rows of V (k_sample.hip; in place when in == out)
hipError_t launch_top_p(const float* in, float* out, int rows, int V, float top_p, hipStream_t s);

// ------------------------------------------------------ distillation backward
namespace {

// Projection shapes (out, in) in the order q, k, v, o, gate, up, down.
void proj_shape(const uno_config& g, int p, int* out, int* in) {
  const int d = g.d_model, qd = g.n_q_heads * g.head_dim, kvd = g.n_kv_heads * g.head_dim;
  const int F = g.ffn_dim;
  const int o[7] = {qd, kvd, kvd, d, F, F, d}, i[7] = {d, d, d, qd, d, d, F};
  *out = o[p];
  *in = i[p];
}

// Scratch of the backward over S sequences of L z1 rows (N = S * L), bytes from 0.
struct BwLayout {
  size_t hg1, rs1, hg2, rs2, x2, t[7], Yq, Yk, Yv, Q, Ks, Vs, Pt, Po, dPt, dPo, o32, o;
  size_t Yg, Yu, a, da, dt;
  size_t dx2, dh, dq, dk, dv, part, dy, tv, dz, lm_hg, lm_rs, lm_dh;
  size_t part_floats;
  int lm_rows;            // rows of one LM-head backward chunk
  size_t total;
};

constexpr int kBwMaxSplits = 16;
constexpr int kBwMaxB = 64;          // block sizes the own-block buffers hold

BwLayout bw_layout(const uno_config& g, size_t S, size_t L) {
  BwLayout W{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
  const size_t N = S * L, d = g.d_model, r = g.lora_rank, F = g.ffn_dim;
  const size_t qd = (size_t)g.n_q_heads * g.head_dim, kvd = (size_t)g.n_kv_heads * g.head_dim;
  const size_t wide = std::max({d, qd, F});
  W.hg1 = take(N * d * 2); W.rs1 = take(N * 4);
  W.hg2 = take(N * d * 2); W.rs2 = take(N * 4);
  W.x2 = take(N * d * 4);
  for (int p = 0; p < 7; ++p) W.t[p] = take(N * r * 2);
  W.Yq = take(N * qd * 4); W.Yk = take(N * kvd * 4); W.Yv = take(N * kvd * 4);
  W.Q = take(N * qd * 2);
  W.Ks = take(N * kvd * 2); W.Vs = take(N * kvd * 2);
  W.Pt = take(N * g.n_q_heads * L * 4);             // [S][Hkv][L * G][L]: x keys
  W.Po = take(N * g.n_q_heads * kBwMaxB * 4);       // [S][Hkv][L * G][B]: own block
  W.dPt = take(L * g.n_q_heads * L * 4);            // one sequence
  W.dPo = take(L * g.n_q_heads * kBwMaxB * 4);
  W.o32 = take(L * qd * 4);                         // one sequence
  W.o = take(N * qd * 2);
  W.Yg = take(N * F * 4); W.Yu = take(N * F * 4); W.a = take(N * F * 2);
  W.da = take(N * F * 4); W.dt = take(N * r * 4);
  W.dx2 = take(N * d * 4); W.dh = take(N * std::max(d, qd) * 4);
  W.dq = take(N * qd * 4); W.dk = take(N * kvd * 4); W.dv = take(N * kvd * 4);
  W.part_floats = std::max((size_t)kBwMaxSplits * r * wide, (size_t)4 * N * r);
  W.part = take(W.part_floats * 4);
  W.dy = take(N * d * 4);
  W.tv = take(N * 4);
  W.lm_rows = (int)std::min<size_t>(N, 2048);
  W.dz = take((size_t)W.lm_rows * g.vocab * 4);
  W.lm_hg = take((size_t)W.lm_rows * d * 2); W.lm_rs = take((size_t)W.lm_rows * 4);
  W.lm_dh = take((size_t)W.lm_rows * d * 4);
  W.total = o;
  return W;
}

int ilog2(int v) { int s = 0; while ((1 << s) < v) ++s; return s; }

// Splits of the k range for a GEMM with few output tiles and a long k: enough
// workgroups for the chip, at least four k steps each.
int bw_splits(int M, int N, int K, size_t part_floats) {
  const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int s = std::min(kBwMaxSplits, std::max(1, 512 / tiles));
  s = std::min(s, std::max(1, K / 128));
  while (s > 1 && (size_t)s * M * N > part_floats) --s;
  return s;
}

uno_status bw_check(uno_ctx* c, int S, int L, int B, void* scratch, size_t bytes, bool rope = true) {
  const uno_config& g = c->cfg;
  if (!c->bf16) return fail(c, UNO_ERR_UNSUPPORTED, "the backward runs in bf16 contexts");
  if (!c->has_lora) return fail(c, UNO_ERR_INVALID_ARG, "the context has no LoRA");
  const int G = g.n_q_heads / g.n_kv_heads;
  if (G & (G - 1)) return fail(c, UNO_ERR_UNSUPPORTED, "backward: query group must be a power of 2");
  if (S < 1 || L < 16 || L % 16 || B < 1 || B > kBwMaxB || L % B)
    return fail(c, UNO_ERR_INVALID_ARG, "backward: batch >= 1, L a multiple of 16 and of B");
  if (rope && g.qk_norm)
    return fail(c, UNO_ERR_UNSUPPORTED, "backward: the QK RMSNorm is not part of the layer backward");
  if (rope && L > c->maxpp * g.page_size)
    return fail(c, UNO_ERR_INVALID_ARG, "backward: L beyond the RoPE table");
  if (!scratch || bytes < bw_layout(g, S, L).total)
    return fail(c, UNO_ERR_INVALID_ARG, "backward: scratch smaller than uno_query_backward_bytes");
  return UNO_OK;
}

BwGemm bw_mk(int am, int bm, const void* A, Idx2 ai, const void* B, Idx2 bi, int b_cols, void* C,
             Idx2 ci, int M, int N, int K) {
  BwGemm x{};
  x.amode = am; x.bmode = bm;
  x.A = A; x.ai = ai; x.B = B; x.bi = bi; x.b_cols = b_cols; x.C = C; x.ci = ci;
  x.M = M; x.N = N; x.K = K; x.batch = 1; x.splits = 1; x.alpha = 1.0f; x.bz = 1;
  return x;
}

// One layer of the backward over the z1 rows of S sequences (N = S * L rows, row
// s * L + i at position i): recompute the gate-on forward from the layer input
// xin [N, d] and the x rows' K/V (kc / vc: sequence s at kc + s * kv_seq_stride,
// [L][Hkv][hd]), then propagate dy [N, d] to dx [N, d] and form the LoRA
// gradients ga[p] [r, in] and gb[p] [out, r] (overwritten).
uno_status layer_backward(uno_ctx* c, int l, int S, int L, int B, const float* xin, const bf16* kc,
                          const bf16* vc, long kv_seq_stride, const float* dy, float* dx,
                          float* const* ga, float* const* gb, char* ws, const BwLayout& W) {
  const uno_config& g = c->cfg;
  hipStream_t st = c->stream;
  const int N = S * L, d = g.d_model, r = g.lora_rank, F = g.ffn_dim, hd = g.head_dim;
  const int Hq = g.n_q_heads, Hkv = g.n_kv_heads, G = Hq / Hkv, LG = L * G;
  const int qd = Hq * hd, kvd = Hkv * hd, sh = ilog2(G);
  const float sc = g.lora_alpha / (float)r, ascale = 1.0f / std::sqrt((float)hd);
  auto F32 = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto BF = [&](size_t off) { return reinterpret_cast<bf16*>(ws + off); };
  auto Wt = [&](int p) { return c->w[p][l]; };
  auto At = [&](int p) { return c->la[p][l]; };
  auto Bt = [&](int p) { return c->lb[p][l]; };
  const bf16* g1 = static_cast<const bf16*>(c->attn_norm[l]);
  const bf16* g2 = static_cast<const bf16*>(c->mlp_norm[l]);
  const float* rcos = c->at<float>(c->L.rope_cos);
  const float* rsin = c->at<float>(c->L.rope_sin);
  auto gemm = [&](const BwGemm& x) -> uno_status {
    UNO_HIP(c, launch_bw_gemm(x, st));
    return UNO_OK;
  };
#define BW_DO(expr) do { if (uno_status s_ = (expr)) return s_; } while (0)
  // gated-LoRA projection recompute: t = bf16(s * rs * (h A^T)), y = rs * (h W^T) + t B^T
  auto proj_fwd = [&](int p, const bf16* h, const float* rs, void* y, bool y_acc) -> uno_status {
    int out, in;
    proj_shape(g, p, &out, &in);
    BwGemm a = bw_mk(BW_A_K16, BW_B_TN, h, idx_ld(in), At(p), {}, in, BF(W.t[p]), idx_ld(r), N, r, in);
    a.alpha = sc; a.row_scale = rs; a.out_bf16 = 1;
    BW_DO(gemm(a));
    BwGemm b = bw_mk(BW_A_K16, BW_B_TN, h, idx_ld(in), Wt(p), {}, in, y, idx_ld(out), N, out, in);
    b.row_scale = rs; b.accumulate = y_acc;
    BW_DO(gemm(b));
    BwGemm u = bw_mk(BW_A_K16, BW_B_TN, BF(W.t[p]), idx_ld(r), Bt(p), {}, r, y, idx_ld(out), N, out, r);
    u.accumulate = 1;
    return gemm(u);
  };
  // projection backward: dB = dY^T t, dt = dY B, dA = s (dt * ks)^T h, dh (+)= dY W + s dt A
  auto proj_back = [&](int p, const float* dY, const bf16* h, const float* ks, float* dh,
                       bool dh_acc, int perm) -> uno_status {
    int out, in;
    proj_shape(g, p, &out, &in);
    float* dt = F32(W.dt);
    BwGemm gB = bw_mk(BW_A_M32, BW_B_N16, dY, idx_ld(out), BF(W.t[p]), idx_ld(r), 0, gb[p], idx_ld(r), out, r, N);
    gB.perm_hd = perm;
    gB.splits = bw_splits(out, r, N, W.part_floats); gB.part = F32(W.part);
    BW_DO(gemm(gB));
    BwGemm gt = bw_mk(BW_A_K32, BW_B_TT, dY, idx_ld(out), Bt(p), {}, r, dt, idx_ld(r), N, r, out);
    BW_DO(gemm(gt));
    BwGemm gA = bw_mk(BW_A_M32, BW_B_N16, dt, idx_ld(r), h, idx_ld(in), 0, ga[p], idx_ld(in), r, in, N);
    gA.alpha = sc; gA.kscale = ks;
    gA.splits = bw_splits(r, in, N, W.part_floats); gA.part = F32(W.part);
    BW_DO(gemm(gA));
    BwGemm gh = bw_mk(BW_A_K32, BW_B_TT, dY, idx_ld(out), Wt(p), {}, in, dh, idx_ld(in), N, in, out);
    gh.accumulate = dh_acc;
    BW_DO(gemm(gh));
    BwGemm gl = bw_mk(BW_A_K32, BW_B_TT, dt, idx_ld(r), At(p), {}, in, dh, idx_ld(in), N, in, r);
    gl.alpha = sc; gl.accumulate = 1;
    return gemm(gl);
  };

  // ---------------- recompute of the gate-on forward
  UNO_HIP(c, launch_bw_rmsprep<bf16>(xin, g1, g.rms_eps, N, d, BF(W.hg1), F32(W.rs1), st));
  BW_DO(proj_fwd(0, BF(W.hg1), F32(W.rs1), F32(W.Yq), false));
  BW_DO(proj_fwd(1, BF(W.hg1), F32(W.rs1), F32(W.Yk), false));
  BW_DO(proj_fwd(2, BF(W.hg1), F32(W.rs1), F32(W.Yv), false));
  UNO_HIP(c, launch_bw_qkv_post(F32(W.Yq), F32(W.Yk), F32(W.Yv), rcos, rsin, N, L, Hq, Hkv, hd,
                                BF(W.Q), BF(W.Ks), BF(W.Vs), st));
  // attention per sequence and KV head: rows m = i * G + g against the x keys (GEMMs
  // that skip the keys no row of a tile sees) and the own block (small kernels)
  const Idx2 qrow{sh, (long)qd, (long)hd};
  const long pt_seq = (long)Hkv * LG * L, po_seq = (long)Hkv * LG * B;
  auto attn_gemm = [&](BwGemm x, int mode) {
    x.batch = Hkv; x.lim_mode = mode; x.lim_G = G; x.lim_B = B;
    return x;
  };
  for (int s = 0; s < S; ++s) {
    const bf16* Qs = BF(W.Q) + (size_t)s * L * qd;
    const bf16* Kt = kc + s * kv_seq_stride;
    const bf16* Vt = vc + s * kv_seq_stride;
    float* Pt = F32(W.Pt) + s * pt_seq;
    float* Po = F32(W.Po) + s * po_seq;
    BwGemm sg = attn_gemm(bw_mk(BW_A_K16, BW_B_K16, Qs, qrow, Kt, idx_ld(kvd), 0, Pt, idx_ld(L),
                                LG, L, hd), 1);
    sg.a_bs = (long)G * hd; sg.b_bs = hd; sg.c_bs = (long)LG * L;
    BW_DO(gemm(sg));
    UNO_HIP(c, launch_bw_own_scores(Qs, BF(W.Ks) + (size_t)s * L * kvd, L, Hq, Hkv, hd, B, Po, st));
    UNO_HIP(c, launch_bw_softmax(Pt, Po, L, G, Hkv, B, ascale, st));
    BwGemm og = attn_gemm(bw_mk(BW_A_K32, BW_B_N16, Pt, idx_ld(L), Vt, idx_ld(kvd), 0, F32(W.o32),
                                qrow, LG, hd, L), 2);
    og.a_bs = (long)LG * L; og.b_bs = hd; og.c_bs = (long)G * hd;
    BW_DO(gemm(og));
    UNO_HIP(c, launch_bw_own_pv(Po, BF(W.Vs) + (size_t)s * L * kvd, F32(W.o32), L, Hq, Hkv, hd, B,
                                BF(W.o) + (size_t)s * L * qd, st));
  }
  UNO_HIP(c, hipMemcpyAsync(F32(W.x2), xin, sizeof(float) * N * d, hipMemcpyDeviceToDevice, st));
  BW_DO(proj_fwd(3, BF(W.o), nullptr, F32(W.x2), true));
  UNO_HIP(c, launch_bw_rmsprep<bf16>(F32(W.x2), g2, g.rms_eps, N, d, BF(W.hg2), F32(W.rs2), st));
  BW_DO(proj_fwd(4, BF(W.hg2), F32(W.rs2), F32(W.Yg), false));
  BW_DO(proj_fwd(5, BF(W.hg2), F32(W.rs2), F32(W.Yu), false));
  UNO_HIP(c, launch_bw_swiglu(F32(W.Yg), F32(W.Yu), BF(W.a), (long)N * F, st));
  {   // the down projection's LoRA intermediate (its output is not needed)
    BwGemm a = bw_mk(BW_A_K16, BW_B_TN, BF(W.a), idx_ld(F), At(6), {}, F, BF(W.t[6]), idx_ld(r), N, r, F);
    a.alpha = sc; a.out_bf16 = 1;
    BW_DO(gemm(a));
  }

  // ---------------- backward
  BW_DO(proj_back(6, dy, BF(W.a), nullptr, F32(W.da), false, 0));
  UNO_HIP(c, launch_bw_swiglu_back(F32(W.da), F32(W.Yg), F32(W.Yu), (long)N * F, st));
  BW_DO(proj_back(4, F32(W.Yg), BF(W.hg2), F32(W.rs2), F32(W.dh), false, 0));
  BW_DO(proj_back(5, F32(W.Yu), BF(W.hg2), F32(W.rs2), F32(W.dh), true, 0));
  UNO_HIP(c, launch_bw_rmsback<bf16>(F32(W.x2), BF(W.hg2), F32(W.rs2), g2, F32(W.dh), dy,
                                     F32(W.dx2), N, d, st));
  BW_DO(proj_back(3, F32(W.dx2), BF(W.o), nullptr, F32(W.dh), false, 0));   // dh = dO
  for (int s = 0; s < S; ++s) {
    const bf16* Qs = BF(W.Q) + (size_t)s * L * qd;
    const bf16* Kt = kc + s * kv_seq_stride;
    const bf16* Vt = vc + s * kv_seq_stride;
    const float* Pt = F32(W.Pt) + s * pt_seq;
    const float* Po = F32(W.Po) + s * po_seq;
    float* dPt = F32(W.dPt);
    float* dPo = F32(W.dPo);
    const float* dO = F32(W.dh) + (size_t)s * L * qd;
    BwGemm pg = attn_gemm(bw_mk(BW_A_K32, BW_B_K16, dO, qrow, Vt, idx_ld(kvd), 0, dPt, idx_ld(L),
                                LG, L, hd), 1);
    pg.a_bs = (long)G * hd; pg.b_bs = hd; pg.c_bs = (long)LG * L;
    BW_DO(gemm(pg));
    UNO_HIP(c, launch_bw_own_dp(dO, BF(W.Vs) + (size_t)s * L * kvd, L, Hq, Hkv, hd, B, dPo, st));
    UNO_HIP(c, launch_bw_softmax_back(Pt, Po, dPt, dPo, L, G, Hkv, B, ascale, st));
    BwGemm qg = attn_gemm(bw_mk(BW_A_K32, BW_B_N16, dPt, idx_ld(L), Kt, idx_ld(kvd), 0,
                                F32(W.dq) + (size_t)s * L * qd, qrow, LG, hd, L), 2);
    qg.a_bs = (long)LG * L; qg.b_bs = hd; qg.c_bs = (long)G * hd;
    BW_DO(gemm(qg));
    UNO_HIP(c, launch_bw_own_back(dPo, Po, Qs, BF(W.Ks) + (size_t)s * L * kvd, dO, L, Hq, Hkv, hd, B,
                                  F32(W.dq) + (size_t)s * L * qd, F32(W.dk) + (size_t)s * L * kvd,
                                  F32(W.dv) + (size_t)s * L * kvd, st));
  }
  UNO_HIP(c, launch_bw_qkv_back(F32(W.dq), F32(W.dk), F32(W.dv), rcos, rsin, N, L, Hq, Hkv, hd,
                                F32(W.Yq), F32(W.Yk), F32(W.Yv), st));
  BW_DO(proj_back(0, F32(W.Yq), BF(W.hg1), F32(W.rs1), F32(W.dh), false, hd));
  BW_DO(proj_back(1, F32(W.Yk), BF(W.hg1), F32(W.rs1), F32(W.dh), true, hd));
  BW_DO(proj_back(2, F32(W.Yv), BF(W.hg1), F32(W.rs1), F32(W.dh), true, hd));
  UNO_HIP(c, launch_bw_rmsback<bf16>(xin, BF(W.hg1), F32(W.rs1), g1, F32(W.dh), F32(W.dx2), dx,
                                     N, d, st));
#undef BW_DO
  return UNO_OK;
}

// LM-head backward of rows [0, rows) (chunked): dx = d/dx of rms_norm(x) W_lm^T
// given dlogits; when teacher / student are given, dlogits are first formed from
// them (the TV gradient, 1 / (2 n_total) scale) with the rows' TV in tv_row.
uno_status lm_backward(uno_ctx* c, int rows, const float* xf, const float* dlogits,
                       const float* teacher, const float* student, int n_total, float* tv_row,
                       float* dx, char* ws, const BwLayout& W) {
  const uno_config& g = c->cfg;
  hipStream_t st = c->stream;
  const int d = g.d_model, V = g.vocab;
  const bf16* gf = static_cast<const bf16*>(c->final_norm);
  for (int r0 = 0; r0 < rows; r0 += W.lm_rows) {
    const int n = std::min(W.lm_rows, rows - r0);
    const float* dz = dlogits ? dlogits + (size_t)r0 * V : reinterpret_cast<float*>(ws + W.dz);
    if (!dlogits)
      UNO_HIP(c, launch_tv_grad(teacher + (size_t)r0 * V, student + (size_t)r0 * V, n, V,
                                0.5f / (float)n_total, reinterpret_cast<float*>(ws + W.dz),
                                tv_row ? tv_row + r0 : nullptr, st));
    bf16* hg = reinterpret_cast<bf16*>(ws + W.lm_hg);
    float* rs = reinterpret_cast<float*>(ws + W.lm_rs);
    float* dh = reinterpret_cast<float*>(ws + W.lm_dh);
    UNO_HIP(c, launch_bw_rmsprep<bf16>(xf + (size_t)r0 * d, gf, g.rms_eps, n, d, hg, rs, st));
    BwGemm h = bw_mk(BW_A_K32, BW_B_TT, dz, idx_ld(V), c->lm_head, {}, d, dh, idx_ld(d), n, d, V);
    UNO_HIP(c, launch_bw_gemm(h, st));
    UNO_HIP(c, launch_bw_rmsback<bf16>(xf + (size_t)r0 * d, hg, rs, gf, dh, nullptr,
                                       dx + (size_t)r0 * d, n, d, st));
  }
  return UNO_OK;
}

}  // namespace

extern "C" {

uno_status uno_pack_weight(const void* d_src, void* d_dst, int32_t rows, int32_t cols,
                           int32_t pair_hd, void* stream) {
  if (!d_src || !d_dst || d_src == d_dst)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "pack: null or aliased buffers");
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 32 ||
      (pair_hd && (pair_hd < 0 || pair_hd % 16 || rows % pair_hd)))
    return fail(nullptr, UNO_ERR_INVALID_ARG, "pack: rows % 16, cols % 32 and rows % pair_hd must be 0");
  hipError_t e = launch_pack(static_cast<const bf16*>(d_src), static_cast<bf16*>(d_dst), rows, cols,
                             pair_hd, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, UNO_ERR_DEVICE, std::string("pack: ") + hipGetErrorString(e));
  return UNO_OK;
}

uno_status uno_top_p(const float* d_in, float* d_out, int32_t rows, int32_t vocab, float top_p,
                     void* stream) {
  if (!d_in || !d_out) return fail(nullptr, UNO_ERR_INVALID_ARG, "top_p: null buffer");
  if (rows < 0 || vocab <= 0 || !(top_p > 0.0f))
    return fail(nullptr, UNO_ERR_INVALID_ARG, "top_p: rows >= 0, vocab > 0 and top_p > 0 required");
  hipError_t e = launch_top_p(d_in, d_out, rows, vocab, top_p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, UNO_ERR_DEVICE, std::string("top_p: ") + hipGetErrorString(e));
  return UNO_OK;
}

uno_status uno_stream_read(const void* d_src, size_t region_bytes, size_t bytes, int32_t reps,
                           int32_t workgroups, int32_t threads, int32_t loads, int32_t* d_sink,
                           void* stream) {
  if (!d_src || !d_sink || bytes == 0 || bytes % 16 || bytes > region_bytes || reps < 1 ||
      workgroups < 1 || threads < 64 || threads > 1024 || threads % 64 ||
      (loads != 1 && loads != 2 && loads != 4 && loads != 8))
    return fail(nullptr, UNO_ERR_INVALID_ARG,
                "stream_read: buffers, bytes a multiple of 16 within the region, reps >= 1, "
                "64..1024 threads (multiple of 64), loads 1, 2, 4 or 8 required");
  const size_t nwin = region_bytes / bytes;
  for (int32_t i = 0; i < reps; ++i) {
    const char* p = static_cast<const char*>(d_src) + (size_t)(i % nwin) * bytes;
    hipError_t e = launch_stream_read(p, bytes, workgroups, threads, loads, d_sink,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(nullptr, UNO_ERR_DEVICE, std::string("stream_read: ") + hipGetErrorString(e));
  }
  return UNO_OK;
}

uno_status uno_query_sizes(const uno_config* cfg, size_t* kv_pool_bytes, size_t* workspace_bytes) {
  uno_status s = check_config(cfg);
  if (s) return s;
  if (kv_pool_bytes) *kv_pool_bytes = kv_bytes(*cfg);
  if (workspace_bytes) *workspace_bytes = make_layout(*cfg).total;
  return UNO_OK;
}

uno_status uno_init(const uno_config* cfg, const uno_weights* wts, void* d_kv_pool,
                    size_t kv_pool_bytes, void* d_workspace, size_t workspace_bytes, void* stream,
                    uno_ctx** out) {
  if (!out) return fail(nullptr, UNO_ERR_INVALID_ARG, "null out");
  *out = nullptr;
  uno_status st = check_config(cfg);
  if (st) return st;
  if (!wts || !d_kv_pool || !d_workspace)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "null weights / kv pool / workspace");
  if (kv_pool_bytes < kv_bytes(*cfg)) return fail(nullptr, UNO_ERR_INVALID_ARG, "kv pool too small");
  const Layout L = make_layout(*cfg);
  if (workspace_bytes < L.total) return fail(nullptr, UNO_ERR_INVALID_ARG, "workspace too small");
  if (!wts->final_norm || !wts->attn_norm || !wts->mlp_norm)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "null norm weights");
  const int nl = cfg->n_layers;
  bool any_lora = false, all_lora = true;
  for (int p = 0; p < 7; ++p) {
    if (!wts->w[p]) return fail(nullptr, UNO_ERR_INVALID_ARG, "null projection array");
    for (int l = 0; l < nl; ++l)
      if (!wts->w[p][l]) return fail(nullptr, UNO_ERR_INVALID_ARG, "null projection weight");
    const bool has = wts->lora_a[p] && wts->lora_b[p];
    any_lora |= has;
    all_lora &= has;
    if (has)
      for (int l = 0; l < nl; ++l)
        if (!wts->lora_a[p][l] || !wts->lora_b[p][l])
          return fail(nullptr, UNO_ERR_INVALID_ARG, "null LoRA weight");
  }
  if (any_lora && !all_lora)
    return fail(nullptr, UNO_ERR_UNSUPPORTED, "LoRA must be on all seven projections or none");
  if (any_lora && cfg->lora_rank <= 0) return fail(nullptr, UNO_ERR_INVALID_ARG, "LoRA without rank");
  for (int l = 0; l < nl; ++l)
    if (!wts->attn_norm[l] || !wts->mlp_norm[l]) return fail(nullptr, UNO_ERR_INVALID_ARG, "null norm");
  if (cfg->qk_norm) {
    if (!wts->q_norm || !wts->k_norm) return fail(nullptr, UNO_ERR_INVALID_ARG, "qk_norm: null q_norm / k_norm array");
    for (int l = 0; l < nl; ++l)
      if (!wts->q_norm[l] || !wts->k_norm[l]) return fail(nullptr, UNO_ERR_INVALID_ARG, "qk_norm: null q / k norm");
  }

  uno_ctx* c = new (std::nothrow) uno_ctx();
  if (!c) return fail(nullptr, UNO_ERR_DEVICE, "host allocation failed");
  c->cfg = *cfg;
  c->bf16 = cfg->dtype == UNO_BF16;
  c->stream = reinterpret_cast<hipStream_t>(stream);
  c->ws = reinterpret_cast<char*>(d_workspace);
  c->kv = d_kv_pool;
  c->L = L;
  c->maxpp = pages_per_seq(*cfg);
  c->embed = wts->embed;
  c->lm_head = wts->lm_head;
  c->final_norm = wts->final_norm;
  c->attn_norm.assign(wts->attn_norm, wts->attn_norm + nl);
  c->mlp_norm.assign(wts->mlp_norm, wts->mlp_norm + nl);
  if (cfg->qk_norm) {
    c->q_norm.assign(wts->q_norm, wts->q_norm + nl);
    c->k_norm.assign(wts->k_norm, wts->k_norm + nl);
  }
  for (int p = 0; p < 7; ++p) {
    c->w[p].assign(wts->w[p], wts->w[p] + nl);
    if (any_lora) {
      c->la[p].assign(wts->lora_a[p], wts->lora_a[p] + nl);
      c->lb[p].assign(wts->lora_b[p], wts->lora_b[p] + nl);
    }
  }
  c->has_lora = any_lora;
  c->free_pages.resize(cfg->n_pages);
  for (int i = 0; i < cfg->n_pages; ++i) c->free_pages[i] = cfg->n_pages - 1 - i;
  c->seq_pages.assign(cfg->max_seqs, {});
  c->len_hi.assign(cfg->max_seqs, 0);
  c->live.assign(cfg->max_seqs, 0);
  c->epoch.assign(cfg->max_seqs, 0);
  c->snap_base.assign(cfg->max_seqs, 0);
  c->snap_epoch.assign(cfg->max_seqs, 0);

  auto bad = [&](hipError_t e, const char* w) {
    uno_status s2 = hip_fail(nullptr, e, w);
    if (c->snap_host) hipHostFree(c->snap_host);
    if (c->snap_event) hipEventDestroy(c->snap_event);
    delete c;
    return s2;
  };
  hipError_t e;
  // the current device's no-allocation scratch is looked up once, at set-up
  if ((e = noalloc_prime())) return bad(e, "no-allocation scratch lookup");
  if ((e = hipHostMalloc((void**)&c->snap_host, sizeof(int32_t) * cfg->max_seqs, hipHostMallocDefault)))
    return bad(e, "hipHostMalloc");
  if ((e = hipEventCreateWithFlags(&c->snap_event, hipEventDisableTiming))) return bad(e, "hipEventCreate");
  // state: lengths / pending / iterations zero, block table -1, error flag 0
  if ((e = hipMemsetAsync(c->ws + L.len, 0, L.block_table - L.len, c->stream))) return bad(e, "memset");
  if ((e = hipMemsetAsync(c->ws + L.block_table, 0xFF,
                          (size_t)cfg->max_seqs * c->maxpp * 4, c->stream))) return bad(e, "memset");
  // RoPE table in double on the host: angle = pos * theta^(-2i/hd)
  const int half = cfg->head_dim / 2;
  const int rope_rows = c->maxpp * cfg->page_size;
  std::vector<float> tc((size_t)rope_rows * half), tsn((size_t)rope_rows * half);
  for (int p = 0; p < rope_rows; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
      const double ang = (double)p * inv;
      tc[(size_t)p * half + i] = (float)std::cos(ang);
      tsn[(size_t)p * half + i] = (float)std::sin(ang);
    }
  if ((e = hipMemcpyAsync(c->ws + L.rope_cos, tc.data(), tc.size() * 4, hipMemcpyHostToDevice, c->stream)))
    return bad(e, "rope upload");
  if ((e = hipMemcpyAsync(c->ws + L.rope_sin, tsn.data(), tsn.size() * 4, hipMemcpyHostToDevice, c->stream)))
    return bad(e, "rope upload");
  if ((e = hipStreamSynchronize(c->stream))) return bad(e, "sync");
  *out = c;
  return UNO_OK;
}

uno_status uno_prefill(uno_ctx* c, int32_t n, const int32_t* seq_ids, const int32_t* d_prompts,
                       const int32_t* prompt_lens) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  std::vector<int> seqs;
  uno_status st = check_seqs(c, n, seq_ids, seqs, false);
  if (st) return st;
  if (!d_prompts || !prompt_lens) return fail(c, UNO_ERR_INVALID_ARG, "null prompts");
  for (int i = 0; i < n; ++i)
    if (prompt_lens[i] < 1 || prompt_lens[i] > c->cfg.max_seq_len)
      return fail(c, UNO_ERR_INVALID_ARG, "prompt length out of range");
  if (!c->embed) return fail(c, UNO_ERR_INVALID_ARG, "no embedding table");
  poll_snapshot(c);
  std::vector<int> upto(n);
  for (int i = 0; i < n; ++i) upto[i] = std::max(1, prompt_lens[i] - 1);
  if ((st = reserve(c, seqs, upto))) return st;
  if ((st = flush_pages(c))) return st;
  // the last prompt token (pending) is read on the device
  std::vector<int32_t> last(n);
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const int P = prompt_lens[i];
    if ((st = upload_call(c, {seqs[i]}))) return st;
    for (int a = 0; a < P - 1; a += c->cfg.max_rows) {
      const int rows = std::min(c->cfg.max_rows, P - 1 - a);
      FwdIn f{};
      f.mode = 3; f.n = 1; f.rows_per_seq = rows;
      f.in_tok = d_prompts + off + a;
      f.pos0 = a;
      f.ctx_bound = a + rows;
      f.lora = false;
      if ((st = forward(c, f))) return st;
    }
    // state: len = P-1, pending = prompt[P-1] (copied on the device), iter = 0
    if ((st = set_state(c, seqs[i], P - 1, 0, 0))) return st;
    UNO_HIP(c, hipMemcpyAsync(c->at<int32_t>(c->L.pending) + seqs[i], d_prompts + off + P - 1,
                              sizeof(int32_t), hipMemcpyDeviceToDevice, c->stream));
    c->len_hi[seqs[i]] = P - 1;
    c->live[seqs[i]] = 1;
    new_epoch(c, seqs[i]);
    off += P;
  }
  c->drafted_ids.clear();
  return UNO_OK;
}

namespace {

// The draft forward and its draws: K == 0 the linear block (B tokens), K >= 1 the
// tree's K chains of B tokens ([n, K, B], y_1 shared).
uno_status draft_impl(uno_ctx* c, int32_t n, const int32_t* seq_ids, int K, int32_t* d_tok,
                      float* d_probs) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  std::vector<int> seqs;
  uno_status st = check_seqs(c, n, seq_ids, seqs, true);
  if (st) return st;
  if (!c->embed || !c->lm_head) return fail(c, UNO_ERR_INVALID_ARG, "no embedding / LM head");
  const int B = c->cfg.block_size, V = c->cfg.vocab;
  // positions a step may write: the draft's n..n+B-1, the verify's n+1..n+B, and
  // for a tree the side chains' slots up to n + 1 + K (B - 1)
  const int span = std::max(B + 1, K > 0 ? 2 + K * (B - 1) : 0);
  if (K > 0 && n * (1 + K * (B - 1)) > c->cfg.max_rows)
    return fail(c, UNO_ERR_INVALID_ARG, "tree verify rows n * (1 + K (B - 1)) exceed max_rows");
  poll_snapshot(c);
  std::vector<int> upto(n);
  for (int i = 0; i < n; ++i) {
    upto[i] = c->len_hi[seqs[i]] + span;
    if (upto[i] > c->cfg.max_seq_len) {   // the bound may be loose: get exact lengths
      if ((st = exact_lengths(c))) return st;
      for (int j = 0; j < n; ++j) upto[j] = c->len_hi[seqs[j]] + span;
      break;
    }
  }
  int bound = 0;
  for (int i = 0; i < n; ++i) bound = std::max(bound, c->len_hi[seqs[i]] + B);
  if ((st = reserve(c, seqs, upto))) return st;
  if ((st = flush_pages(c))) return st;
  if ((st = upload_call(c, seqs))) return st;
  FwdIn f{};
  f.mode = 0; f.n = n; f.rows_per_seq = B;
  f.ctx_bound = bound;
  f.lora = true;
  f.probs_out = c->at<float>(c->L.probs_d);
  if ((st = forward(c, f))) return st;
  hipStream_t s = c->stream;
  RowDesc* desc = c->at<RowDesc>(c->L.desc);
  const int draws = n * B * std::max(1, K);
  Timed tsm(c, UNO_KC_SAMPLING, (double)draws * V * 8, 0);
  if (top_p_on(c->cfg))
    UNO_HIP(c, launch_top_p(f.probs_out, f.probs_out, n * B, V, c->cfg.top_p, s));
  if (K == 0)
    UNO_HIP(c, launch_draft_desc(f.probs_out, n, B, V, c->cfg.seed, c->at<int32_t>(c->L.call_seq),
                                 c->at<int32_t>(c->L.call_n), c->at<int32_t>(c->L.call_it),
                                 c->at<int32_t>(c->L.draft_tok), desc, s));
  else
    UNO_HIP(c, launch_tree_draft_desc(f.probs_out, n, K, B, V, c->cfg.seed,
                                      c->at<int32_t>(c->L.call_seq), c->at<int32_t>(c->L.call_n),
                                      c->at<int32_t>(c->L.call_it), c->at<int32_t>(c->L.draft_tok),
                                      desc, s));
  UNO_HIP(c, launch_cdf(desc, draws, V, c->at<uint64_t>(c->L.chunk_tot), c->at<int32_t>(c->L.err), s));
  if (d_tok)
    UNO_HIP(c, hipMemcpyAsync(d_tok, c->at<int32_t>(c->L.draft_tok), sizeof(int32_t) * draws,
                              hipMemcpyDeviceToDevice, s));
  if (d_probs)
    UNO_HIP(c, hipMemcpyAsync(d_probs, f.probs_out, sizeof(float) * (size_t)n * B * V,
                              hipMemcpyDeviceToDevice, s));
  c->drafted_ids = seqs;
  c->drafted_tree = K;
  return UNO_OK;
}

}  // namespace

uno_status uno_draft(uno_ctx* c, int32_t n, const int32_t* seq_ids, int32_t* d_draft, float* d_probs) {
  return draft_impl(c, n, seq_ids, 0, d_draft, d_probs);
}

uno_status uno_verify(uno_ctx* c, int32_t n, const int32_t* seq_ids, int32_t* d_out,
                      int32_t* d_n_out, float* d_probs) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  std::vector<int> seqs;
  uno_status st = check_seqs(c, n, seq_ids, seqs, true);
  if (st) return st;
  if (seqs != c->drafted_ids || c->drafted_tree != 0)
    return fail(c, UNO_ERR_STATE, "verify without a matching linear draft");
  if ((st = upload_call(c, seqs))) return st;     // another call may have changed the list
  const int B = c->cfg.block_size, V = c->cfg.vocab;
  int bound = 0;
  for (int sq : seqs) bound = std::max(bound, c->len_hi[sq] + B + 1);
  FwdIn f{};
  f.mode = 1; f.n = n; f.rows_per_seq = B;
  f.ctx_bound = bound;
  f.lora = false;
  f.probs_out = c->at<float>(c->L.probs_v);
  if ((st = forward(c, f))) return st;
  hipStream_t s = c->stream;
  RowDesc* desc = c->at<RowDesc>(c->L.desc);
  int32_t* err = c->at<int32_t>(c->L.err);
  const float* pd = c->at<float>(c->L.probs_d);
  Timed tsm(c, UNO_KC_SAMPLING, (double)n * V * 8 * 2, 0);
  if (top_p_on(c->cfg))
    UNO_HIP(c, launch_top_p(f.probs_out, f.probs_out, n * B, V, c->cfg.top_p, s));
  UNO_HIP(c, launch_accept_test(c->cfg.seed, n, B, V, f.probs_out, pd + V, B,
                                c->at<int32_t>(c->L.draft_tok), c->at<int32_t>(c->L.call_seq),
                                c->at<int32_t>(c->L.call_n), c->at<int32_t>(c->L.call_it),
                                c->at<int32_t>(c->L.acc_k), c->at<int32_t>(c->L.acc_z), desc, err, s));
  UNO_HIP(c, launch_cdf(desc, n, V, c->at<uint64_t>(c->L.chunk_tot), err, s));
  UNO_HIP(c, launch_accept_commit(n, B, c->at<int32_t>(c->L.draft_tok), c->at<int32_t>(c->L.acc_k),
                                  c->at<int32_t>(c->L.acc_z), c->at<int32_t>(c->L.call_seq), d_out,
                                  d_n_out, c->at<int32_t>(c->L.len), c->at<int32_t>(c->L.pending),
                                  c->at<int32_t>(c->L.iter), s));
  if (d_probs)
    UNO_HIP(c, hipMemcpyAsync(d_probs, f.probs_out, sizeof(float) * (size_t)n * B * V,
                              hipMemcpyDeviceToDevice, s));
  for (int sq : seqs) c->len_hi[sq] += B + 1;
  c->drafted_ids.clear();
  return start_snapshot(c);
}

uno_status uno_step(uno_ctx* c, int32_t n, const int32_t* seq_ids, int32_t* d_out, int32_t* d_n_out) {
  uno_status st = uno_draft(c, n, seq_ids, nullptr, nullptr);
  if (st) return st;
  return uno_verify(c, n, seq_ids, d_out, d_n_out, nullptr);
}

uno_status uno_tree_draft(uno_ctx* c, int32_t n, const int32_t* seq_ids, int32_t n_chains,
                          int32_t* d_chains, float* d_probs) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (n_chains < 1 || n_chains > c->cfg.tree_chains)
    return fail(c, UNO_ERR_INVALID_ARG, "n_chains must be 1..tree_chains");
  return draft_impl(c, n, seq_ids, n_chains, d_chains, d_probs);
}

uno_status uno_tree_verify(uno_ctx* c, int32_t n, const int32_t* seq_ids, int32_t* d_out,
                           int32_t* d_n_out, int32_t* d_kstar, float* d_probs) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  std::vector<int> seqs;
  uno_status st = check_seqs(c, n, seq_ids, seqs, true);
  if (st) return st;
  if (seqs != c->drafted_ids || c->drafted_tree < 1)
    return fail(c, UNO_ERR_STATE, "tree verify without a matching tree draft");
  if ((st = upload_call(c, seqs))) return st;
  const int B = c->cfg.block_size, V = c->cfg.vocab, K = c->drafted_tree;
  const int Rv = 1 + K * (B - 1);
  int bound = 0;
  for (int sq : seqs) bound = std::max(bound, c->len_hi[sq] + std::max(B + 1, 2 + K * (B - 1)));
  FwdIn f{};
  f.mode = 5; f.n = n; f.rows_per_seq = Rv; f.tree_K = K;
  f.ctx_bound = bound;
  f.lora = false;
  f.probs_out = c->at<float>(c->L.probs_v);
  if ((st = forward(c, f))) return st;
  hipStream_t s = c->stream;
  int32_t* err = c->at<int32_t>(c->L.err);
  Timed tsm(c, UNO_KC_SAMPLING, (double)n * V * 8 * 2, 0);
  if (top_p_on(c->cfg))
    UNO_HIP(c, launch_top_p(f.probs_out, f.probs_out, n * Rv, V, c->cfg.top_p, s));
  TreeAcceptArgs ta{};
  ta.p = f.probs_out; ta.p_rows = Rv;
  ta.q = c->at<float>(c->L.probs_d); ta.q_rows = B;
  ta.chains = c->at<int32_t>(c->L.draft_tok);
  ta.seq_ids = c->at<int32_t>(c->L.call_seq);
  ta.pos = c->at<int32_t>(c->L.call_n);
  ta.iter = c->at<int32_t>(c->L.call_it);
  ta.K = K; ta.B = B; ta.V = V; ta.seed = c->cfg.seed;
  ta.resid = c->at<uint64_t>(c->L.tree_res);
  ta.path = c->at<int32_t>(c->L.tree_path);
  ta.k_out = c->at<int32_t>(c->L.acc_k);
  ta.kstar = c->at<int32_t>(c->L.tree_kstar);
  ta.z = c->at<int32_t>(c->L.acc_z);
  ta.desc = c->at<RowDesc>(c->L.desc);
  ta.err = err;
  UNO_HIP(c, launch_tree_accept(ta, n, s));
  UNO_HIP(c, launch_cdf(ta.desc, n, V, c->at<uint64_t>(c->L.chunk_tot), err, s));
  const KvLayout kv = kv_layout(c);
  if (c->bf16)
    UNO_HIP(c, launch_tree_kv_move<bf16>(kv, n, B, c->cfg.n_layers, ta.seq_ids, ta.pos, ta.k_out,
                                         ta.kstar, err, s));
  else
    UNO_HIP(c, launch_tree_kv_move<float>(kv, n, B, c->cfg.n_layers, ta.seq_ids, ta.pos, ta.k_out,
                                          ta.kstar, err, s));
  UNO_HIP(c, launch_accept_commit(n, B, ta.path, ta.k_out, ta.z, ta.seq_ids, d_out, d_n_out,
                                  c->at<int32_t>(c->L.len), c->at<int32_t>(c->L.pending),
                                  c->at<int32_t>(c->L.iter), s));
  if (d_kstar)
    UNO_HIP(c, hipMemcpyAsync(d_kstar, ta.kstar, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, s));
  if (d_probs)
    UNO_HIP(c, hipMemcpyAsync(d_probs, f.probs_out, sizeof(float) * (size_t)n * Rv * V,
                              hipMemcpyDeviceToDevice, s));
  for (int sq : seqs) c->len_hi[sq] += B + 1;
  c->drafted_ids.clear();
  c->drafted_tree = 0;
  return start_snapshot(c);
}

uno_status uno_tree_step(uno_ctx* c, int32_t n, const int32_t* seq_ids, int32_t n_chains,
                         int32_t* d_out, int32_t* d_n_out) {
  uno_status st = uno_tree_draft(c, n, seq_ids, n_chains, nullptr, nullptr);
  if (st) return st;
  return uno_tree_verify(c, n, seq_ids, d_out, d_n_out, nullptr, nullptr);
}

uno_status uno_tree_accept(uno_ctx* c, int32_t n, int32_t n_chains, const float* d_p,
                           const float* d_q, const int32_t* d_chains, const int32_t* d_seq_ids,
                           const int32_t* d_pos, const int32_t* d_iter, int32_t* d_out,
                           int32_t* d_n_out, int32_t* d_kstar) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (c->cfg.tree_chains < 1) return fail(c, UNO_ERR_UNSUPPORTED, "context without tree_chains");
  if (n < 1 || n > c->cfg.max_seqs) return fail(c, UNO_ERR_INVALID_ARG, "bad count");
  if (n_chains < 1 || n_chains > TREE_KMAX) return fail(c, UNO_ERR_INVALID_ARG, "n_chains must be 1..16");
  if (!d_p || !d_q || !d_chains || !d_seq_ids || !d_pos || !d_iter)
    return fail(c, UNO_ERR_INVALID_ARG, "null input");
  const int B = c->cfg.block_size, V = c->cfg.vocab;
  hipStream_t s = c->stream;
  int32_t* err = c->at<int32_t>(c->L.err);
  TreeAcceptArgs ta{};
  ta.p = d_p; ta.p_rows = 1 + n_chains * (B - 1);
  ta.q = d_q; ta.q_rows = B;
  ta.chains = d_chains; ta.seq_ids = d_seq_ids; ta.pos = d_pos; ta.iter = d_iter;
  ta.K = n_chains; ta.B = B; ta.V = V; ta.seed = c->cfg.seed;
  ta.resid = c->at<uint64_t>(c->L.tree_res);
  ta.path = c->at<int32_t>(c->L.tree_path);
  ta.k_out = c->at<int32_t>(c->L.acc_k);
  ta.kstar = c->at<int32_t>(c->L.tree_kstar);
  ta.z = c->at<int32_t>(c->L.acc_z);
  ta.desc = c->at<RowDesc>(c->L.desc);
  ta.err = err;
  UNO_HIP(c, launch_tree_accept(ta, n, s));
  UNO_HIP(c, launch_cdf(ta.desc, n, V, c->at<uint64_t>(c->L.chunk_tot), err, s));
  UNO_HIP(c, launch_accept_commit(n, B, ta.path, ta.k_out, ta.z, d_seq_ids, d_out, d_n_out, nullptr,
                                  nullptr, nullptr, s));
  if (d_kstar)
    UNO_HIP(c, hipMemcpyAsync(d_kstar, ta.kstar, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, s));
  return UNO_OK;
}

uno_status uno_accept(uno_ctx* c, int32_t n, const float* d_p, const float* d_q, const int32_t* d_draft,
                      const int32_t* d_seq_ids, const int32_t* d_pos, const int32_t* d_iter,
                      int32_t* d_out, int32_t* d_n_out) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (n < 1 || n > c->cfg.max_seqs) return fail(c, UNO_ERR_INVALID_ARG, "bad count");
  if (!d_p || !d_draft || !d_seq_ids || !d_pos || !d_iter || (!d_q && c->cfg.block_size > 1))
    return fail(c, UNO_ERR_INVALID_ARG, "null input");
  const int B = c->cfg.block_size, V = c->cfg.vocab;
  hipStream_t s = c->stream;
  RowDesc* desc = c->at<RowDesc>(c->L.desc);
  int32_t* err = c->at<int32_t>(c->L.err);
  UNO_HIP(c, launch_accept_test(c->cfg.seed, n, B, V, d_p, d_q, B - 1, d_draft, d_seq_ids, d_pos,
                                d_iter, c->at<int32_t>(c->L.acc_k), c->at<int32_t>(c->L.acc_z), desc,
                                err, s));
  UNO_HIP(c, launch_cdf(desc, n, V, c->at<uint64_t>(c->L.chunk_tot), err, s));
  UNO_HIP(c, launch_accept_commit(n, B, d_draft, c->at<int32_t>(c->L.acc_k), c->at<int32_t>(c->L.acc_z),
                                  d_seq_ids, d_out, d_n_out, nullptr, nullptr, nullptr, s));
  return UNO_OK;
}

uno_status uno_sample(uno_ctx* c, int32_t rows, const float* d_w, const int32_t* d_seq_ids,
                      const int32_t* d_pos, const int32_t* d_iter, int32_t stream_id, int32_t* d_idx) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  const int cap = std::max(c->cfg.max_rows, c->cfg.max_seqs * c->cfg.block_size);
  if (rows < 1 || rows > cap) return fail(c, UNO_ERR_INVALID_ARG, "bad row count");
  if (!d_w || !d_seq_ids || !d_pos || !d_iter || !d_idx) return fail(c, UNO_ERR_INVALID_ARG, "null input");
  RowDesc* desc = c->at<RowDesc>(c->L.desc);
  UNO_HIP(c, launch_sample_desc(d_w, rows, c->cfg.vocab, c->cfg.seed, d_seq_ids, d_pos, d_iter,
                                stream_id, d_idx, desc, c->stream));
  UNO_HIP(c, launch_cdf(desc, rows, c->cfg.vocab, c->at<uint64_t>(c->L.chunk_tot),
                        c->at<int32_t>(c->L.err), c->stream));
  return UNO_OK;
}

uno_status uno_forward(uno_ctx* c, int32_t n, const int32_t* seq_ids, int32_t rows_per_seq,
                       const int32_t* d_tokens, const float* d_hidden_in, const int32_t* d_pos,
                       const uint8_t* d_gate, float* d_hidden_out, float* d_logits) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  std::vector<int> seqs;
  uno_status st = check_seqs(c, n, seq_ids, seqs, false);
  if (st) return st;
  if (rows_per_seq < 1 || n * rows_per_seq > c->cfg.max_rows)
    return fail(c, UNO_ERR_INVALID_ARG, "rows exceed max_rows");
  if ((!d_tokens && !d_hidden_in) || !d_pos || !d_gate)
    return fail(c, UNO_ERR_INVALID_ARG, "null row inputs");
  if (!d_hidden_in && !c->embed) return fail(c, UNO_ERR_INVALID_ARG, "no embedding table");
  if (d_logits && !c->lm_head) return fail(c, UNO_ERR_INVALID_ARG, "no LM head");
  const int R = n * rows_per_seq;
  std::vector<int32_t> pos(R);
  UNO_HIP(c, hipStreamSynchronize(c->stream));
  UNO_HIP(c, hipMemcpy(pos.data(), d_pos, sizeof(int32_t) * R, hipMemcpyDeviceToHost));
  std::vector<int> upto(n, 0);
  int bound = 0;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < rows_per_seq; ++j) {
      const int p = pos[(size_t)i * rows_per_seq + j];
      if (p < 0 || p >= c->cfg.max_seq_len) return fail(c, UNO_ERR_INVALID_ARG, "position out of range");
      upto[i] = std::max(upto[i], p + 1);
      bound = std::max(bound, p + 1);
    }
  poll_snapshot(c);
  if ((st = reserve(c, seqs, upto))) return st;
  if ((st = flush_pages(c))) return st;
  if ((st = upload_call(c, seqs))) return st;
  FwdIn f{};
  f.mode = 2; f.n = n; f.rows_per_seq = rows_per_seq;
  f.in_tok = d_tokens; f.in_hidden = d_hidden_in; f.in_pos = d_pos; f.in_gate = d_gate;
  f.ctx_bound = bound;
  f.lora = true;
  f.hidden_out = d_hidden_out;
  f.logits_out = d_logits;
  return forward(c, f);
}

uno_status uno_distill_forward(uno_ctx* c, int32_t batch, int32_t L, int32_t B, const int32_t* d_x,
                               float* d_teacher, float* d_student, float* d_tv_row,
                               float* d_tv_block) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (batch < 1 || L < 1 || B < 1 || L % B) return fail(c, UNO_ERR_INVALID_ARG, "bad batch / L / B");
  if (!d_x) return fail(c, UNO_ERR_INVALID_ARG, "null tokens");
  if (2 * L > c->cfg.max_rows || 2 * L > c->cfg.max_seq_len)
    return fail(c, UNO_ERR_INVALID_ARG, "2L exceeds max_rows or max_seq_len");
  if (c->bf16 && L % 16)
    return fail(c, UNO_ERR_INVALID_ARG, "bf16 contexts need L to be a multiple of 16");
  if (!c->embed || !c->lm_head) return fail(c, UNO_ERR_INVALID_ARG, "no embedding / LM head");
  if (!c->drafted_ids.empty()) return fail(c, UNO_ERR_STATE, "a drafted block awaits verification");
  // scratch sequences: slots holding no sequence and no pages
  std::vector<int> slots;
  for (int s = 0; s < c->cfg.max_seqs; ++s)
    if (!c->live[s] && c->seq_pages[s].empty()) slots.push_back(s);
  const int ps = c->cfg.page_size, pps = (2 * L + ps - 1) / ps;
  int nb = std::min<int>((int)slots.size(), c->cfg.max_rows / (2 * L));
  nb = std::min<int>(nb, (int)c->free_pages.size() / pps);
  nb = std::min(nb, batch);
  if (nb < 1) return fail(c, UNO_ERR_OUT_OF_PAGES, "no free sequence slot / pages for [x, z1]");
  const size_t V = c->cfg.vocab;
  const bool ck = c->ck_x != nullptr;
  if (ck && (c->ck_batch != batch || c->ck_L != L || !c->bf16))
    return fail(c, UNO_ERR_INVALID_ARG, "the armed checkpoint is for another batch / L (or not bf16)");
  poll_snapshot(c);
  for (int g0 = 0; g0 < batch; g0 += nb) {
    const int n = std::min(nb, batch - g0);
    std::vector<int> seqs(slots.begin(), slots.begin() + n);
    uno_status st;
    if ((st = reserve(c, seqs, std::vector<int>(n, 2 * L)))) return st;
    if ((st = flush_pages(c))) return st;
    if ((st = upload_call(c, seqs))) return st;
    FwdIn f{};
    f.mode = 4; f.n = n; f.rows_per_seq = 2 * L;
    f.in_tok = d_x + (size_t)g0 * L;
    f.ctx_bound = L + 32;     // the virtual key count of any 16-row tile is at most L + 16
    f.lora = true;
    f.dB = B;
    f.teacher = d_teacher ? d_teacher + (size_t)g0 * L * V : nullptr;
    f.student = d_student ? d_student + (size_t)g0 * L * V : nullptr;
    f.tv_row = d_tv_row ? d_tv_row + (size_t)g0 * L : nullptr;
    f.tv_block = d_tv_block ? d_tv_block + (size_t)g0 * (L / B) : nullptr;
    if (ck) {
      f.ck_x = c->ck_x + (size_t)g0 * L * c->cfg.d_model;
      f.ck_stride = (size_t)batch * L * c->cfg.d_model;
    }
    st = forward(c, f);
    // the x rows' K/V of every layer (positions 0..L-1 of each borrowed slot)
    for (int j = 0; ck && !st && j < n; ++j) {
      const size_t o = (size_t)(g0 + j) * c->cfg.n_layers * L * c->cfg.n_kv_heads * c->cfg.head_dim;
      hipError_t e = launch_kv_copy<bf16>(kv_layout(c), seqs[j], L, static_cast<bf16*>(c->ck_k) + o,
                                          static_cast<bf16*>(c->ck_v) + o, 0, c->stream);
      if (e != hipSuccess) st = hip_fail(c, e, "checkpoint K/V export");
    }
    // the pages go back to the pool (stream-ordered after the forward)
    for (int s : seqs) {
      auto& pg = c->seq_pages[s];
      for (size_t i = 0; i < pg.size(); ++i) {
        c->pt_idx.push_back(s * c->maxpp + (int)i);
        c->pt_val.push_back(-1);
        c->free_pages.push_back(pg[i]);
      }
      pg.clear();
    }
    uno_status st2 = flush_pages(c);
    if (st) return st;
    if (st2) return st2;
  }
  return UNO_OK;
}

uno_status uno_set_trace(uno_ctx* c, const uno_trace* t) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (!t) {
    c->trace_on = false;
    c->trace = uno_trace{};
    return UNO_OK;
  }
  if (t->n < 0 || t->n > 4) return fail(c, UNO_ERR_INVALID_ARG, "trace: n must be 0..4");
  for (int i = 0; i < t->n; ++i)
    if (t->layer[i].layer >= c->cfg.n_layers)
      return fail(c, UNO_ERR_INVALID_ARG, "trace: layer index >= n_layers");
  c->trace = *t;
  c->trace_on = true;
  return UNO_OK;
}

uno_status uno_kv_import(uno_ctx* c, int32_t seq_id, int32_t len, const void* d_k, const void* d_v,
                         int32_t pending, int32_t iter) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (seq_id < 0 || seq_id >= c->cfg.max_seqs) return fail(c, UNO_ERR_INVALID_ARG, "bad seq id");
  if (len < 0 || len >= c->cfg.max_seq_len || (len > 0 && (!d_k || !d_v)))
    return fail(c, UNO_ERR_INVALID_ARG, "bad length / buffers");
  if (pending < 0 || pending >= c->cfg.vocab || iter < 0) return fail(c, UNO_ERR_INVALID_ARG, "bad state");
  poll_snapshot(c);
  uno_status st;
  if ((st = reserve(c, {seq_id}, {std::max(len, 1)}))) return st;
  if ((st = flush_pages(c))) return st;
  const KvLayout kv = kv_layout(c);
  if (c->bf16)
    UNO_HIP(c, launch_kv_copy<bf16>(kv, seq_id, len, (bf16*)d_k, (bf16*)d_v, 1, c->stream));
  else
    UNO_HIP(c, launch_kv_copy<float>(kv, seq_id, len, (float*)d_k, (float*)d_v, 1, c->stream));
  if ((st = set_state(c, seq_id, len, pending, iter))) return st;
  c->len_hi[seq_id] = len;
  c->live[seq_id] = 1;
  new_epoch(c, seq_id);
  return UNO_OK;
}

uno_status uno_kv_export(uno_ctx* c, int32_t seq_id, int32_t len, void* d_k, void* d_v) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (seq_id < 0 || seq_id >= c->cfg.max_seqs) return fail(c, UNO_ERR_INVALID_ARG, "bad seq id");
  if (len < 1 || !d_k || !d_v) return fail(c, UNO_ERR_INVALID_ARG, "bad length / buffers");
  if ((int)c->seq_pages[seq_id].size() * c->cfg.page_size < len)
    return fail(c, UNO_ERR_INVALID_ARG, "positions not reserved");
  const KvLayout kv = kv_layout(c);
  if (c->bf16)
    UNO_HIP(c, launch_kv_copy<bf16>(kv, seq_id, len, (bf16*)d_k, (bf16*)d_v, 0, c->stream));
  else
    UNO_HIP(c, launch_kv_copy<float>(kv, seq_id, len, (float*)d_k, (float*)d_v, 0, c->stream));
  return UNO_OK;
}

uno_status uno_seq_state(uno_ctx* c, int32_t seq_id, int32_t* len, int32_t* pending, int32_t* iter) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (seq_id < 0 || seq_id >= c->cfg.max_seqs) return fail(c, UNO_ERR_INVALID_ARG, "bad seq id");
  UNO_HIP(c, hipStreamSynchronize(c->stream));
  int32_t v[3];
  UNO_HIP(c, hipMemcpy(&v[0], c->at<int32_t>(c->L.len) + seq_id, 4, hipMemcpyDeviceToHost));
  UNO_HIP(c, hipMemcpy(&v[1], c->at<int32_t>(c->L.pending) + seq_id, 4, hipMemcpyDeviceToHost));
  UNO_HIP(c, hipMemcpy(&v[2], c->at<int32_t>(c->L.iter) + seq_id, 4, hipMemcpyDeviceToHost));
  if (len) *len = v[0];
  if (pending) *pending = v[1];
  if (iter) *iter = v[2];
  return UNO_OK;
}

uno_status uno_release(uno_ctx* c, int32_t seq_id) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (seq_id < 0 || seq_id >= c->cfg.max_seqs) return fail(c, UNO_ERR_INVALID_ARG, "bad seq id");
  auto& pg = c->seq_pages[seq_id];
  for (size_t i = 0; i < pg.size(); ++i) {
    c->pt_idx.push_back(seq_id * c->maxpp + (int)i);
    c->pt_val.push_back(-1);
    c->free_pages.push_back(pg[i]);
  }
  pg.clear();
  c->live[seq_id] = 0;
  c->len_hi[seq_id] = 0;
  new_epoch(c, seq_id);
  if (std::find(c->drafted_ids.begin(), c->drafted_ids.end(), seq_id) != c->drafted_ids.end())
    c->drafted_ids.clear();
  uno_status st = flush_pages(c);
  if (st) return st;
  return set_state(c, seq_id, 0, 0, 0);
}

uno_status uno_sync(uno_ctx* c) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  UNO_HIP(c, hipStreamSynchronize(c->stream));
  int32_t e = 0;
  UNO_HIP(c, hipMemcpy(&e, c->at<int32_t>(c->L.err), 4, hipMemcpyDeviceToHost));
  poll_snapshot(c);
  if (e & UNO_DEVERR_BOUNDS) return fail(c, UNO_ERR_DEVICE, "device bounds check tripped");
  if (e & UNO_DEVERR_SYNC) return fail(c, UNO_ERR_DEVICE, "a workgroup's wait for another's result ran out");
  if (e & UNO_DEVERR_NUMERIC) return fail(c, UNO_ERR_NUMERIC, "NaN / negative probability or empty row");
  return UNO_OK;
}

uno_status uno_timing(uno_ctx* c, uint32_t class_mask) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (class_mask && c->tev.empty()) {
    c->tev.resize(2 * kTimedLaunches, nullptr);
    for (auto& e : c->tev) UNO_HIP(c, hipEventCreate(&e));
  }
  UNO_HIP(c, hipStreamSynchronize(c->stream));
  c->trec.clear();
  c->tmask = class_mask;
  for (auto& n : c->tcalls) n = 0;
  return UNO_OK;
}

uno_status uno_timing_every(uno_ctx* c, int32_t period) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (period < 1) return fail(c, UNO_ERR_INVALID_ARG, "timing period must be >= 1");
  c->tperiod = period;
  for (auto& n : c->tcalls) n = 0;
  return UNO_OK;
}

uno_status uno_timing_read(uno_ctx* c, int32_t cls, int64_t* launches, double* total_ms,
                           double* bytes, double* flops) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (cls < 0 || cls >= UNO_KC_COUNT) return fail(c, UNO_ERR_INVALID_ARG, "bad kernel class");
  UNO_HIP(c, hipStreamSynchronize(c->stream));
  int64_t n = 0;
  double ms = 0, b = 0, f = 0;
  for (const auto& r : c->trec) {
    if (r.cls != cls) continue;
    float e = 0;
    UNO_HIP(c, hipEventElapsedTime(&e, c->tev[r.ev], c->tev[r.ev + 1]));
    if (r.call) ++n;
    ms += e;
    b += r.bytes;
    f += r.flops;
  }
  if (launches) *launches = n;
  if (total_ms) *total_ms = ms;
  if (bytes) *bytes = b;
  if (flops) *flops = f;
  return UNO_OK;
}

uno_status uno_query_backward_bytes(const uno_config* cfg, int32_t batch, int32_t L, size_t* bytes) {
  uno_status s = check_config(cfg);
  if (s) return s;
  if (batch < 1 || L < 1 || !bytes) return fail(nullptr, UNO_ERR_INVALID_ARG, "backward bytes: batch, L >= 1");
  *bytes = bw_layout(*cfg, batch, L).total;
  return UNO_OK;
}

uno_status uno_set_distill_checkpoint(uno_ctx* c, float* d_x, void* d_k, void* d_v, int32_t batch,
                                      int32_t L) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (!d_x) {
    c->ck_x = nullptr; c->ck_k = c->ck_v = nullptr; c->ck_batch = c->ck_L = 0;
    return UNO_OK;
  }
  if (!d_k || !d_v || batch < 1 || L < 1)
    return fail(c, UNO_ERR_INVALID_ARG, "checkpoint: buffers and batch, L >= 1 required");
  c->ck_x = d_x; c->ck_k = d_k; c->ck_v = d_v; c->ck_batch = batch; c->ck_L = L;
  return UNO_OK;
}

uno_status uno_tv_backward(const float* d_teacher, const float* d_student, int32_t rows, int32_t vocab,
                           int32_t n_rows_total, float* d_dlogits, float* d_tv_row, void* stream) {
  if (!d_teacher || !d_student || !d_dlogits)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "tv_backward: null buffer");
  if (rows < 0 || vocab <= 0 || n_rows_total < 1)
    return fail(nullptr, UNO_ERR_INVALID_ARG, "tv_backward: rows >= 0, vocab > 0, n_rows_total >= 1");
  hipError_t e = launch_tv_grad(d_teacher, d_student, rows, vocab, 0.5f / (float)n_rows_total,
                                d_dlogits, d_tv_row, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, UNO_ERR_DEVICE, std::string("tv_backward: ") + hipGetErrorString(e));
  return UNO_OK;
}

uno_status uno_lm_head_backward(uno_ctx* c, int32_t rows, const float* d_x_final,
                                const float* d_dlogits, float* d_dx, void* d_scratch,
                                size_t scratch_bytes) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (!d_x_final || !d_dlogits || !d_dx) return fail(c, UNO_ERR_INVALID_ARG, "lm_head_backward: null buffer");
  if (!c->lm_head) return fail(c, UNO_ERR_INVALID_ARG, "no LM head");
  if (rows < 16 || rows % 16) return fail(c, UNO_ERR_INVALID_ARG, "lm_head_backward: rows a multiple of 16");
  if (uno_status s = bw_check(c, 1, rows, 1, d_scratch, scratch_bytes, false)) return s;
  return lm_backward(c, rows, d_x_final, d_dlogits, nullptr, nullptr, rows, nullptr, d_dx,
                     static_cast<char*>(d_scratch), bw_layout(c->cfg, 1, rows));
}

uno_status uno_lora_layer_backward(uno_ctx* c, int32_t layer, int32_t batch, int32_t L, int32_t B,
                                   const float* d_x_in, const void* d_k_ctx, const void* d_v_ctx,
                                   const float* d_dy, float* d_dx, float* const* d_grad_a,
                                   float* const* d_grad_b, void* d_scratch, size_t scratch_bytes) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, UNO_ERR_INVALID_ARG, "bad layer");
  if (!d_x_in || !d_k_ctx || !d_v_ctx || !d_dy || !d_dx || !d_grad_a || !d_grad_b)
    return fail(c, UNO_ERR_INVALID_ARG, "layer_backward: null buffer");
  for (int p = 0; p < 7; ++p)
    if (!d_grad_a[p] || !d_grad_b[p]) return fail(c, UNO_ERR_INVALID_ARG, "layer_backward: null gradient");
  if (uno_status s = bw_check(c, batch, L, B, d_scratch, scratch_bytes)) return s;
  const long kvd = (long)c->cfg.n_kv_heads * c->cfg.head_dim;
  return layer_backward(c, layer, batch, L, B, d_x_in, static_cast<const bf16*>(d_k_ctx),
                        static_cast<const bf16*>(d_v_ctx), (long)L * kvd, d_dy, d_dx, d_grad_a,
                        d_grad_b, static_cast<char*>(d_scratch), bw_layout(c->cfg, batch, L));
}

uno_status uno_distill_backward(uno_ctx* c, int32_t batch, int32_t L, int32_t B,
                                const float* d_teacher, const float* d_student,
                                const float* d_x_ckpt, const void* d_k_ckpt, const void* d_v_ckpt,
                                float* d_loss, float* d_tv_row, float* const* d_grad_a,
                                float* const* d_grad_b, void* d_scratch, size_t scratch_bytes) {
  if (!c) return fail(nullptr, UNO_ERR_INVALID_ARG, "null ctx");
  if (!d_teacher || !d_student || !d_x_ckpt || !d_k_ckpt || !d_v_ckpt || !d_grad_a || !d_grad_b)
    return fail(c, UNO_ERR_INVALID_ARG, "distill_backward: null buffer");
  for (int p = 0; p < 7; ++p)
    if (!d_grad_a[p] || !d_grad_b[p]) return fail(c, UNO_ERR_INVALID_ARG, "distill_backward: null gradient");
  if (!c->lm_head) return fail(c, UNO_ERR_INVALID_ARG, "no LM head");
  if (uno_status s = bw_check(c, batch, L, B, d_scratch, scratch_bytes)) return s;
  const uno_config& g = c->cfg;
  const BwLayout W = bw_layout(g, batch, L);
  char* ws = static_cast<char*>(d_scratch);
  const size_t N = (size_t)batch * L, d = g.d_model, r = g.lora_rank, nl = g.n_layers;
  const long kvd = (long)g.n_kv_heads * g.head_dim;
  float* dy = reinterpret_cast<float*>(ws + W.dy);
  float* tv = d_tv_row ? d_tv_row : reinterpret_cast<float*>(ws + W.tv);
  if (uno_status s = lm_backward(c, (int)N, d_x_ckpt + nl * N * d, nullptr, d_teacher, d_student,
                                 (int)N, tv, dy, ws, W))
    return s;
  if (d_loss) UNO_HIP(c, launch_tv_mean(tv, (int)N, d_loss, c->stream));
  for (int l = (int)nl - 1; l >= 0; --l) {
    float* ga[7];
    float* gb[7];
    for (int p = 0; p < 7; ++p) {
      int out, in;
      proj_shape(g, p, &out, &in);
      ga[p] = d_grad_a[p] + (size_t)l * r * in;
      gb[p] = d_grad_b[p] + (size_t)l * out * r;
    }
    // dx overwrites dy in place: a layer's last read of dy precedes its write of dx
    const bf16* kc = static_cast<const bf16*>(d_k_ckpt) + (size_t)l * L * kvd;
    const bf16* vc = static_cast<const bf16*>(d_v_ckpt) + (size_t)l * L * kvd;
    if (uno_status s = layer_backward(c, l, batch, L, B, d_x_ckpt + l * N * d, kc, vc,
                                      (long)nl * L * kvd, dy, dy, ga, gb, ws, W))
      return s;
  }
  return UNO_OK;
}

int32_t uno_free_pages(const uno_ctx* c) { return c ? (int32_t)c->free_pages.size() : 0; }

const char* uno_last_error(const uno_ctx* c) {
  return c ? c->err.c_str() : g_last_error.c_str();
}

void uno_destroy(uno_ctx* c) {
  if (!c) return;
  hipStreamSynchronize(c->stream);
  if (c->snap_host) hipHostFree(c->snap_host);
  if (c->snap_event) hipEventDestroy(c->snap_event);
  for (auto e : c->tev)
    if (e) hipEventDestroy(e);
  delete c;
}

}  // extern "C"
