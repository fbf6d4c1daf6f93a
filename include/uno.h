/*
 * uno.h -- C ABI of the MI355X (gfx950) Psi-Spec draft-and-verify decode step for
 * diffusion-augmented LLMs ("Uno").
 *
 * The method (pages cited by title and section):
 *   [summary]  ai-papers-daily summary of "Unlocking Lossless Speedups in LLMs via
 *              Discrete Diffusion", section "方法关键点" (method key points);
 *   [blog]     shibing624 reading notes "...Uno 的无损加速之路", sections
 *              "方法核心：一个模型，两套权重" (method core), "Diffusion Distillation：
 *              一步蒸馏 + 块级扩散" (distillation), "Ψ-Spec 采样器：起草、验证、两种模式"
 *              (the Psi-Spec sampler).
 *   One causal decoder holds the frozen AR weights plus a rank-r LoRA on every
 *   layer (r 128, alpha 256 for the 8B models) [summary; blog method core].  A draft
 *   forward (base + LoRA) proposes a block of B tokens in parallel; its first token
 *   uses the AR weights only and is always accepted.  A verify forward (base only)
 *   over the same KV cache scores the block, the longest accepted prefix is kept
 *   and the first rejected position is resampled from max(0, p - q) renormalised
 *   [blog Psi-Spec sampler].  Two forwards per iteration give 1 <= tokens per
 *   forward <= (B+1)/2.  One gated forward over [x, z1] with a block-causal mask
 *   yields teacher (AR) and student (AR+LoRA) logits [blog distillation].
 *
 * Readings the library fixes where the pages are silent:
 *   - decoder: pre-norm RMSNorm, rotate-half RoPE, grouped-query attention, SwiGLU,
 *     no biases, untied embedding and LM head; the MASK id's logit is -inf;
 *   - LoRA on all seven projections: y = h W^T + gate * bf16((alpha/r) h A^T) B^T;
 *   - draft rows [t, MASK x (B-1)] at positions n..n+B-1 with gate [0,1,..,1];
 *     verify rows [y_1..y_B] at n+1..n+B with gate 0; row r predicts position
 *     (its own position + 1);
 *   - accept y_i iff u_i * q_i(y_i) < p_i(y_i) in float32;
 *   - keyed randomness: Philox4x64-10, key (seed, seq_id), counter (position the
 *     draw decides, stream, iteration, 0), stream 0 draft / 1 accept / 2 resample;
 *     a categorical draw is an inverse CDF over trunc(w * 2^40) integers with
 *     threshold floor(word0 * T / 2^64); a uniform is (word0 >> 40) * 2^-24.
 *
 * Conventions for every call:
 *   - Device pointers are BORROWED: the caller owns weights, the KV pool, the
 *     workspace and every output buffer; the library frees none of them and calls
 *     no device allocator.  Pointers named d_* are device memory, others host.
 *   - Matrices are row-major.  Projection weights are [out, in] (K contiguous),
 *     LoRA down A is [r, in], LoRA up B is [out, r], embedding and LM head
 *     [vocab, d_model], norm gains [d_model].  Storage type is float32 or
 *     bfloat16 as uno_config.dtype says; logits and probabilities are float32.
 *   - Calls enqueue work on the context's stream and return without waiting,
 *     except the ones marked "syncs".
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns an error and changes no state.
 *   - Device-side faults of the method (NaN / negative probabilities, a row with
 *     no integer mass, a KV write outside a sequence's pages) set a sticky flag
 *     that uno_sync reports as UNO_ERR_NUMERIC / UNO_ERR_DEVICE.
 *   - A context belongs to one host thread; calls on one context are serialised
 *     on its stream.
 */
#ifndef UNO_H
#define UNO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct uno_ctx uno_ctx;

typedef enum {
  UNO_OK = 0,
  UNO_ERR_INVALID_ARG = 1,   /* bad shape, pointer, id or size; nothing enqueued      */
  UNO_ERR_OUT_OF_PAGES = 2,  /* the KV page pool cannot hold the requested positions  */
  UNO_ERR_STATE = 3,         /* call out of order (e.g. verify without a draft)       */
  UNO_ERR_NUMERIC = 4,       /* NaN / negative probability or a row with no mass      */
  UNO_ERR_DEVICE = 5,        /* a HIP call failed, or a device bounds check tripped   */
  UNO_ERR_UNSUPPORTED = 6    /* a shape the library does not implement                */
} uno_status;

typedef enum { UNO_F32 = 0, UNO_BF16 = 1 } uno_dtype;

/* Model shape and decoding limits.  mask_id must be vocab-1. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, mask_id;
  int32_t lora_rank;        /* 0: no LoRA (the draft then uses the base weights)    */
  float lora_alpha, rope_theta, rms_eps;
  int32_t block_size;       /* B, 1..64                                             */
  int32_t page_size;        /* tokens per KV page                                   */
  int32_t max_seqs;         /* sequence ids are 0..max_seqs-1                        */
  int32_t max_seq_len;      /* positions per sequence the KV cache must hold         */
  int32_t n_pages;          /* pages in the KV pool                                  */
  int32_t max_rows;         /* rows one forward may carry (>= max_seqs*block_size)   */
  int32_t dtype;            /* uno_dtype                                             */
  uint64_t seed;            /* Philox key word 0                                     */
  float top_p;              /* nucleus truncation of the draft and verify laws (the
                               uno_top_p rule, applied right after each softmax):
                               0 (the zero-initialised default) or >= 1 turns it off;
                               negative or NaN is UNO_ERR_INVALID_ARG              */
  int32_t qk_norm;          /* 1: RMS-normalise every query and key head over its
                               head_dim (gain uno_weights.q_norm / k_norm, eps
                               rms_eps) after the projection and before RoPE, as in
                               the Qwen3 attention of the base model the pages
                               augment (Qwen3-8B plus a LoRA [summary]); 0 (default):
                               off; other values are UNO_ERR_INVALID_ARG.  The
                               distillation backward calls return
                               UNO_ERR_UNSUPPORTED on such a context              */
  int32_t tree_chains;      /* most chains a tree call may use (0..16; 0, the
                               default: no tree calls).  The workspace grows by
                               max_seqs * (vocab * 8 + (1 + tree_chains (B - 1))
                               * vocab * 4) bytes or so; a tree call on n sequences
                               also needs max_rows >= n * (1 + K (B - 1))          */
} uno_config;

/* Weights: host arrays of device pointers, copied at uno_init (the device memory
 * they point to must outlive the context).  embed / lm_head may be NULL when only
 * hidden-state forwards (uno_forward with d_hidden_in / d_hidden_out) are used.
 * lora_a / lora_b may be NULL (no adapter on that projection).
 * Projection order: 0 q, 1 k, 2 v, 3 o, 4 gate, 5 up, 6 down.
 * float32 contexts take every matrix row-major.  bf16 contexts take lm_head, w,
 * lora_a and lora_b in the fragment-tiled layout that uno_pack_weight produces
 * from the row-major matrix (q, k, v and their lora_b packed with pair_hd =
 * head_dim, all others with pair_hd = 0); embed and the norm gains (final, attn,
 * mlp, q and k) stay row-major. */
typedef struct {
  const void* embed;                 /* [vocab, d]                 */
  const void* lm_head;               /* [vocab, d]                 */
  const void* final_norm;            /* [d]                        */
  const void* const* attn_norm;      /* [n_layers] -> [d]          */
  const void* const* mlp_norm;       /* [n_layers] -> [d]          */
  const void* const* w[7];           /* [n_layers] -> [out, in]    */
  const void* const* lora_a[7];      /* [n_layers] -> [r, in]      */
  const void* const* lora_b[7];      /* [n_layers] -> [out, r]     */
  const void* const* q_norm;         /* [n_layers] -> [head_dim]; read only when
                                        uno_config.qk_norm is 1 (then required) */
  const void* const* k_norm;         /* [n_layers] -> [head_dim]   */
} uno_weights;

/* Repack a row-major bf16 matrix [rows, cols] (device) into the fragment-tiled
 * layout the bf16 kernels stream (device, rows * cols elements, not aliasing
 * d_src): 16 x 32 blocks in row-block-major order, and inside a block element
 * (r, c) at position ((c % 32) / 8 * 16 + r % 16) * 8 + c % 8, which is the
 * operand order of the 16x16x32 bf16 matrix instruction, so one wavefront reads
 * a block as one contiguous 1 KB access.  pair_hd > 0 (q / k / v weights and
 * LoRA up-projections) also orders the rows of each head of pair_hd rows so
 * that each 16-row block holds rows 8j..8j+7 and pair_hd/2+8j..+7, the rotary
 * pairs of one output tile.  Requires rows % 16 == 0, cols % 32 == 0 and
 * rows % pair_hd == 0.  Enqueued on stream (a hipStream_t); no context needed. */
uno_status uno_pack_weight(const void* d_src, void* d_dst, int32_t rows, int32_t cols,
                           int32_t pair_hd, void* stream);

/* Top-p (nucleus) truncation of probability rows.  The pages' evaluations sample
 * at temperature 1 with top-p 0.95, and losslessness holds for that filtered law
 * (shibing624 reading notes, "我的判断"); applying the same truncation to the AR
 * law p and the draft law q keeps speculative rejection exact for it.  Row r of
 * d_in [rows, vocab] (float32 probabilities, >= 0) becomes row r of d_out: with
 * masses w_i = floor(p_i * 2^40) (int64), W = sum w_i and the target mass
 * T = max(1, ceil(top_p * W)) (double), tau is the largest value whose upper set
 * {p >= tau} holds at least T (ties kept); kept entries become p_i / Z with
 * Z = float(W_kept * 2^-40), the others 0.  top_p >= 1, or a row with W == 0, is
 * copied unchanged.  d_out may equal d_in (in place); device pointers; one
 * workgroup per row, enqueued on stream (a hipStream_t); no context needed.
 * UNO_ERR_INVALID_ARG for null buffers, rows < 0, vocab <= 0 or top_p <= 0. */
uno_status uno_top_p(const float* d_in, float* d_out, int32_t rows, int32_t vocab, float top_p,
                     void* stream);

/* Measurement helper, not a step of the method: `reps` back-to-back launches, launch
 * i reading `bytes` (a multiple of 16) of device memory at d_src + (i mod w) * bytes,
 * w = region_bytes / bytes, with `workgroups` workgroups of `threads` threads
 * (64..1024, a multiple of 64), each thread keeping `loads` (1, 2, 4 or 8)
 * nontemporal 16-byte loads in flight -- the weight stream of a linear launch
 * without its products, so the time per launch is the HBM floor of that launch
 * shape (a region well above the memory-side cache keeps every window in HBM).
 * d_sink: device int32 [workgroups], receives the xor of what each workgroup of the
 * last launch read.  Enqueued on `stream` (a hipStream_t; NULL: the null stream).
 * UNO_ERR_INVALID_ARG on a null buffer or a size outside these ranges. */
uno_status uno_stream_read(const void* d_src, size_t region_bytes, size_t bytes, int32_t reps,
                           int32_t workgroups, int32_t threads, int32_t loads, int32_t* d_sink,
                           void* stream);

/* Sizes of the caller-allocated KV pool and workspace for a config.
 * KV pool layout (exposed for inspection only; use uno_kv_import/export):
 * [layer][K|V][page][kv_head] blocks of page_size x head_dim of the storage type,
 * K token-major ([token][dim]) and V dim-major ([dim][token]). */
uno_status uno_query_sizes(const uno_config* cfg, size_t* kv_pool_bytes,
                           size_t* workspace_bytes);

/* Create a context on the current HIP device.  kv_pool / workspace are device
 * buffers of at least the queried sizes; stream is a hipStream_t (NULL = the
 * default stream).  Syncs (uploads the RoPE table). */
uno_status uno_init(const uno_config* cfg, const uno_weights* weights, void* d_kv_pool,
                    size_t kv_pool_bytes, void* d_workspace, size_t workspace_bytes,
                    void* stream, uno_ctx** out);

/* Prefill (the AR forward that fills the KV cache): for each listed sequence,
 * run gate-0 rows prompt[0..P-2] at positions 0..P-2 and leave prompt[P-1] as the
 * pending token; the sequence's iteration counter restarts at 0.
 * seq_ids, prompt_lens: host [n]; d_prompts: device int32, the prompts
 * concatenated in order.  Each prompt length is >= 1 and <= max_seq_len. */
uno_status uno_prefill(uno_ctx* ctx, int32_t n, const int32_t* seq_ids,
                       const int32_t* d_prompts, const int32_t* prompt_lens);

/* Draft forward [blog Psi-Spec sampler]: rows [t, MASK x (B-1)] at n..n+B-1 with
 * gate [0,1,...,1]; samples y_1 from row 0 (AR) and y_i from row i-1 (q_i).
 * d_draft: device int32 [n, B] (y_1..y_B), may be NULL.  d_probs: device float32
 * [n, B, vocab] (row 0 = p(y_1), rows 1.. = q_2..q_B), may be NULL.  With
 * config.top_p in (0, 1) every row is first truncated to its nucleus (the
 * uno_top_p rule): the draws and d_probs use the truncated laws. */
uno_status uno_draft(uno_ctx* ctx, int32_t n, const int32_t* seq_ids, int32_t* d_draft,
                     float* d_probs);

/* Verify forward + accept/resample + commit [blog Psi-Spec sampler]: rows
 * [y_1..y_B] at n+1..n+B with gate 0; accepts the longest prefix, resamples the
 * first rejected slot from max(0, p_k - q_k) (bonus row p_{B+1} if none fails),
 * commits positions n..n+k-1 and makes z pending.  d_out: device int32 [n, B+1]
 * (k tokens, then -1); d_n_out: device int32 [n] (k in [2, B+1]).  d_probs: device
 * float32 [n, B, vocab] (p_2..p_{B+1}), may be NULL.  With config.top_p in (0, 1)
 * the p rows are truncated to their nuclei before the accept test, like the draft
 * laws, so the emitted tokens follow the truncated AR law.  Needs a preceding
 * uno_draft of exactly these sequences. */
uno_status uno_verify(uno_ctx* ctx, int32_t n, const int32_t* seq_ids, int32_t* d_out,
                      int32_t* d_n_out, float* d_probs);

/* One Psi-Spec iteration [blog Psi-Spec sampler: a draft forward proposes the block,
 * one verify forward checks it, so every iteration costs two forwards and emits
 * between 2 and B+1 tokens]: uno_draft followed by uno_verify. */
uno_status uno_step(uno_ctx* ctx, int32_t n, const int32_t* seq_ids, int32_t* d_out,
                    int32_t* d_n_out);

/* Accept/resample on caller-given probabilities (the parity entry of the accept
 * kernel) [blog Psi-Spec sampler: keep the longest prefix the AR law accepts,
 * resample the first rejected slot from max(0, p - q) renormalised; blog
 * distillation section: the standard speculative rejection of Leviathan et al.,
 * Cor. 3.6], using the context's seed and workspace; the sequence state is not
 * touched.  d_p: [n, B, V] = p_2..p_{B+1}; d_q: [n, B-1, V] = q_2..q_B; d_draft:
 * [n, B] = y_1..y_B; d_seq_ids, d_pos, d_iter: device int32 [n] (Philox key word 1,
 * the pending position n, the iteration).  Outputs as uno_verify.  A NaN /
 * negative / unnormalisable row sets the sticky numeric flag (see uno_sync).
 * n <= max_seqs. */
uno_status uno_accept(uno_ctx* ctx, int32_t n, const float* d_p, const float* d_q,
                      const int32_t* d_draft, const int32_t* d_seq_ids, const int32_t* d_pos,
                      const int32_t* d_iter, int32_t* d_out, int32_t* d_n_out);

/* Tree sampler (the batch-1 mode of the Psi-Spec sampler) [summary: a linear
 * sampler for system throughput and a tree sampler for single-request throughput;
 * blog Psi-Spec sampler: one-step draft from the noise block, AR rejection keeps
 * the output law].  The pages lost how the tree's candidates are chosen; the
 * library reads it as follows.  The draft forward is uno_draft's; K chains share
 * y_1 and draw depths d = 2..B independently from the draft laws (chain k's draw
 * uses Philox counter (n + d, stream 0, iteration, k); chain 0 is uno_draft's
 * block).  The verify forward scores row y_1 at position n+1 and, for each chain,
 * its depths 2..B at positions n+2..n+B, every row seeing the context through y_1
 * and its own chain (the chains' K/V go to slots n + 2 + k (B - 1) + d - 2, so
 * chain 0 sits at its positions): 1 + K (B - 1) rows per sequence, gate 0.
 * Acceptance walks the depths: the live chains (those matching the accepted path)
 * are tried in chain order; trial j uses u_j = Philox counter (n + d, stream 1,
 * iteration, j); trial 0 is uno_verify's float32 test against p_d (the law of the
 * lowest live chain's previous row), a rejection replaces the target by the
 * integer residual R_1 = trunc(max(0, p_d - q_d) 2^40) (p_d when empty), later
 * ones by R_{j+1} = R_j - min(R_j, floor(T_j trunc(q_d 2^40) / 2^40)) (T_j = sum
 * R_j; kept when empty), and trial j >= 1 accepts c iff (u_j q_d(c)) T_j < R_j(c)
 * in float64.  When every live chain fails at depth d the step emits d tokens, the
 * last drawn from the last residual (counter (n + d, stream 2, iteration, 0));
 * when every depth passes it emits B + 1, the last from the lowest live chain's
 * bonus law.  The accepted path's K/V end at their positions.  With K = 1 this is
 * uno_draft + uno_verify draw for draw.  Requires uno_config.tree_chains >= K. */

/* Draft forward plus K chains: d_chains (device int32 [n, K, B], or NULL; entry 0
 * of every chain is y_1), d_probs as uno_draft.  UNO_ERR_INVALID_ARG for K outside
 * 1..tree_chains or n (1 + K (B - 1)) > max_rows. */
uno_status uno_tree_draft(uno_ctx* ctx, int32_t n, const int32_t* seq_ids, int32_t n_chains,
                          int32_t* d_chains, float* d_probs);

/* Verify forward of the pending tree draft, acceptance, K/V of the accepted path,
 * commit.  d_out [n, B+1], d_n_out [n] as uno_verify; d_kstar (device int32 [n],
 * or NULL): the lowest chain on the accepted path; d_probs (or NULL): the verify
 * laws [n, 1 + K (B - 1), V] in row order (y_1, then chain k's depths 2..B).
 * UNO_ERR_STATE without a matching uno_tree_draft. */
uno_status uno_tree_verify(uno_ctx* ctx, int32_t n, const int32_t* seq_ids, int32_t* d_out,
                           int32_t* d_n_out, int32_t* d_kstar, float* d_probs);

/* uno_tree_draft followed by uno_tree_verify. */
uno_status uno_tree_step(uno_ctx* ctx, int32_t n, const int32_t* seq_ids, int32_t n_chains,
                         int32_t* d_out, int32_t* d_n_out);

/* The tree acceptance on caller-given laws (its parity entry): d_p [n, 1 + K (B-1),
 * V] verify laws in uno_tree_verify's row order, d_q [n, B, V] the draft laws
 * (depth d uses row d - 1), d_chains [n, K, B]; d_seq_ids, d_pos, d_iter as
 * uno_accept.  Outputs d_out [n, B+1], d_n_out [n], d_kstar [n] (or NULL); the
 * sequence state is not touched.  Needs a context with tree_chains >= 1
 * (UNO_ERR_UNSUPPORTED otherwise); K <= 16, n <= max_seqs. */
uno_status uno_tree_accept(uno_ctx* ctx, int32_t n, int32_t n_chains, const float* d_p,
                           const float* d_q, const int32_t* d_chains, const int32_t* d_seq_ids,
                           const int32_t* d_pos, const int32_t* d_iter, int32_t* d_out,
                           int32_t* d_n_out, int32_t* d_kstar);

/* Accept/resample without a context and without allocating anything, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same kernels and the same results as
 * uno_accept on a context whose seed, block_size and vocab are these: d_p
 * [n, block_size, vocab] = p_2..p_{B+1}, d_q [n, block_size-1, vocab] = q_2..q_B
 * (may be NULL when block_size is 1), d_draft [n, block_size], d_seq_ids / d_pos /
 * d_iter [n] (device int32: Philox key word 1, the pending position, the
 * iteration); outputs d_out [n, block_size+1] and d_n_out [n] as uno_verify.
 * d_err (device int32, may be NULL): the call ORs its device error bits into it
 * (1: a NaN / negative / > 1 probability, a draft id outside the vocabulary, or a
 * row without integer mass), so the caller clears it beforehand.  Enqueued on
 * stream (a hipStream_t) on the current device; calls neither hipMalloc nor
 * hipFree.  Its working memory (row descriptors, CDF chunk sums, accept lengths,
 * drawn tokens) is one static device array of 1.05 MiB per GPU, kept until the
 * process ends and shared by every call on that GPU: calls that overlap on one
 * GPU race.  Limits: n <= 1024 and vocab <= 262144 (128 CDF chunks of 2048);
 * larger sizes, block_size outside 1..64 or a null required buffer give
 * UNO_ERR_INVALID_ARG before anything is enqueued (text in uno_last_error(NULL)). */
uno_status uno_accept_noalloc(uint64_t seed, int32_t n, int32_t block_size, int32_t vocab,
                              const float* d_p, const float* d_q, const int32_t* d_draft,
                              const int32_t* d_seq_ids, const int32_t* d_pos,
                              const int32_t* d_iter, int32_t* d_out, int32_t* d_n_out,
                              int32_t* d_err, void* stream);

/* Categorical draws on caller-given rows (the parity entry of the sampler):
 * row r of d_w [rows, V] (float32 weights in [0, 1]) is drawn with
 * Philox(key = (seed, d_seq_ids[r]), counter = (d_pos[r], stream_id, d_iter[r], 0)).
 * d_idx: device int32 [rows] (-1 when the row has no integer mass).
 * rows <= max_rows. */
uno_status uno_sample(uno_ctx* ctx, int32_t rows, const float* d_w, const int32_t* d_seq_ids,
                      const int32_t* d_pos, const int32_t* d_iter, int32_t stream_id,
                      int32_t* d_idx);

/* Raw forward (parity entry) of the one decoder with its gated LoRA [blog method
 * core: one model holds the AR weights and the LoRA; summary, method key points:
 * the gate switches the adapter per row]: rows_per_seq rows for each listed
 * sequence, row inputs either tokens (d_tokens [n*rows]) or hidden states
 * (d_hidden_in float32 [n*rows, d]); positions d_pos [n*rows] and gates d_gate
 * (uint8, 1 = LoRA on) [n*rows].  Each
 * row's K/V is written at its position (pages reserved as needed) and a row at
 * position m attends to its sequence's positions 0..m.  Committed lengths and
 * pending tokens are not changed.  Outputs (each may be NULL): the final residual
 * stream d_hidden_out float32 [n*rows, d] (before the final norm) and d_logits
 * float32 [n*rows, vocab]. */
uno_status uno_forward(uno_ctx* ctx, int32_t n, const int32_t* seq_ids, int32_t rows_per_seq,
                       const int32_t* d_tokens, const float* d_hidden_in, const int32_t* d_pos,
                       const uint8_t* d_gate, float* d_hidden_out, float* d_logits);

/* Distillation-style forward (Uno reading notes, "Diffusion Distillation": the
 * clean sequence x and the fully corrupted z1 = MASK^L run as [x, z1] in ONE
 * forward under a block-causal mask, the gated LoRA off on x rows and on on z1
 * rows, giving teacher (AR) and student (AR + LoRA) logits together, compared by
 * a block-wise total variation; ai-papers-daily summary, method key points).
 *   d_x        device int32 [batch, L] clean tokens in [0, vocab)
 *   d_teacher  device float32 [batch, L, vocab] x-row logits (MASK column -inf),
 *              or NULL
 *   d_student  device float32 [batch, L, vocab] z1-row logits, or NULL
 *   d_tv_row   device float32 [batch, L]: TV_i = 0.5 * sum_v |p_T,i - p_S,i|, or NULL
 *   d_tv_block device float32 [batch, L/B]: mean of TV_i over each block, or NULL
 * Row i of x and row i of z1 both sit at RoPE position i and both predict token
 * i+1.  Visibility: x row i sees x[0..i]; z1 row i of block b = i / B sees x[0, bB)
 * and z1[bB..i].  Requires L % B == 0, 2L <= max_rows and 2L <= max_seq_len (and
 * L % 16 == 0 in bf16 contexts: the halves start on whole 16-row blocks).
 * The [x, z1] K/V live in sequence slots that hold no sequence and no pages
 * (UNO_ERR_OUT_OF_PAGES when there is none, or too few free pages for 2L
 * positions); the call borrows them and returns them, so committed sequences are
 * untouched.  UNO_ERR_STATE between uno_draft and uno_verify.  Asynchronous. */
uno_status uno_distill_forward(uno_ctx* ctx, int32_t batch, int32_t L, int32_t B,
                               const int32_t* d_x, float* d_teacher, float* d_student,
                               float* d_tv_row, float* d_tv_block);

/* ---- Distillation backward (the training side of the [x, z1] forward).
 * The pages train only the LoRA of the diffusion path, with the AR weights frozen
 * as the teacher, and the block-wise total variation between the diffusion and
 * the AR distributions as the loss term that trained best (shibing624 reading
 * notes, "Diffusion Distillation"; ai-papers-daily summary, method key points).
 * The library reads the loss L_TV as the mean over sequences and blocks of the
 * block TV, a block's TV being the mean over its rows of
 * TV_i = 0.5 * sum_v |p_T,i(v) - p_S,i(v)| (so the mean of TV_i over all rows),
 * with the teacher law a constant, d|u|/du = 0 at u = 0 and every bf16 storage
 * rounding of the forward passed straight through.  Gradients are float32:
 * dL/dA_p [r, in] and dL/dB_p [out, r] row-major in the uno_weights row order
 * (q / k / v rows in head order, not the pair order of the packed weights).
 * The z1 rows' forward is recomputed layer by layer from a checkpoint; every
 * product runs on the bf16 matrix cores with float32 accumulation, a float32
 * gradient operand entering as two bf16 terms (hi = bf16(g), lo = bf16(g - hi)).
 * bf16 contexts with LoRA only (UNO_ERR_UNSUPPORTED otherwise); the query group
 * n_q_heads / n_kv_heads must be a power of two.  Scratch memory is the caller's
 * (uno_query_backward_bytes); all calls are asynchronous on the context's stream. */

/* Scratch bytes for a backward over `batch` sequences of L z1 rows (also the
 * bound of uno_lm_head_backward with batch 1 and L = rows). */
uno_status uno_query_backward_bytes(const uno_config* cfg, int32_t batch, int32_t L,
                                    size_t* bytes);

/* Arm (d_x != NULL) or disarm the activation checkpoint that the next
 * uno_distill_forward calls (of exactly this batch and L) fill:
 *   d_x  float32 [n_layers + 1][batch * L][d_model]: slot l holds the z1 rows'
 *        residual stream entering layer l, slot n_layers the stream entering the
 *        final norm (sequence b's rows at b * L);
 *   d_k, d_v  bf16 [batch][n_layers][L][n_kv_heads][head_dim]: the x rows' K
 *        (after RoPE) and V of every layer.
 * A distillation forward of another batch or L while armed is UNO_ERR_INVALID_ARG. */
uno_status uno_set_distill_checkpoint(uno_ctx* ctx, float* d_x, void* d_k, void* d_v,
                                      int32_t batch, int32_t L);

/* Gradient of L_TV at the student logits (parity entry; no context): for each of
 * `rows` rows of d_teacher / d_student [rows, vocab] (float32 logits, -inf
 * allowed), with N = n_rows_total rows in the whole loss,
 * g(v) = sign(p_S(v) - p_T(v)) / (2N) and d_dlogits(v) = p_S(v) (g(v) - sum_u p_S(u) g(u));
 * d_tv_row [rows] (may be NULL) receives TV_i.  Softmaxes in float32. */
uno_status uno_tv_backward(const float* d_teacher, const float* d_student, int32_t rows,
                           int32_t vocab, int32_t n_rows_total, float* d_dlogits, float* d_tv_row,
                           void* stream);

/* LM-head backward (parity entry): d_dx [rows, d] = the gradient at the final
 * residual stream d_x_final [rows, d] of logits = rms_norm(x) W_lm^T given
 * d_dlogits [rows, vocab].  rows a multiple of 16. */
uno_status uno_lm_head_backward(uno_ctx* ctx, int32_t rows, const float* d_x_final,
                                const float* d_dlogits, float* d_dx, void* d_scratch,
                                size_t scratch_bytes);

/* One layer of the backward (parity entry).  Rows: the z1 rows of `batch`
 * sequences of L rows (row b * L + i at position i, gate on), each block of B rows
 * attending to the x rows' keys before the block and causally to its own.
 *   d_x_in   float32 [batch * L, d]: the residual stream entering the layer;
 *   d_k_ctx, d_v_ctx  bf16 [batch][L][n_kv_heads][head_dim]: the x rows' K (after
 *            RoPE) and V of this layer;
 *   d_dy     float32 [batch * L, d]: dL / d(layer output);
 *   d_dx     float32 [batch * L, d]: dL / d(layer input) (may equal d_dy);
 *   d_grad_a[7], d_grad_b[7]: this layer's dL/dA_p [r, in], dL/dB_p [out, r]
 *            (overwritten). */
uno_status uno_lora_layer_backward(uno_ctx* ctx, int32_t layer, int32_t batch, int32_t L,
                                   int32_t B, const float* d_x_in, const void* d_k_ctx,
                                   const void* d_v_ctx, const float* d_dy, float* d_dx,
                                   float* const* d_grad_a, float* const* d_grad_b,
                                   void* d_scratch, size_t scratch_bytes);

/* The whole backward of one distillation forward: d_teacher / d_student [batch,
 * L, vocab] and the checkpoint buffers as that forward left them;
 * d_loss (float32 [1], may be NULL) = L_TV; d_tv_row [batch * L] (may be NULL);
 * d_grad_a[p] -> float32 [n_layers][r][in_p], d_grad_b[p] -> [n_layers][out_p][r]
 * (overwritten). */
uno_status uno_distill_backward(uno_ctx* ctx, int32_t batch, int32_t L, int32_t B,
                                const float* d_teacher, const float* d_student,
                                const float* d_x_ckpt, const void* d_k_ckpt,
                                const void* d_v_ckpt, float* d_loss, float* d_tv_row,
                                float* const* d_grad_a, float* const* d_grad_b, void* d_scratch,
                                size_t scratch_bytes);

/* Stage capture (parity instrumentation).  While a trace is armed, every forward
 * of the context (draft, verify, uno_forward, prefill chunks, the distillation
 * forward) copies, on its stream, the intermediates of up to four layers and its
 * logits into caller-owned device buffers, so each stage of the layer can be
 * checked on its own against a reference fed the same inputs.  R is the number
 * of rows of that forward, in call order (draft / verify: n * block_size; the
 * distillation forward: 2L per sequence; every prefill chunk overwrites the
 * previous one's).  Each pointer may be NULL (not captured).  Matrices are
 * row-major; "storage type" means bfloat16 or float32 as the config says.  The
 * KV cache itself is read with uno_kv_export.  Disarm before timing: the copies
 * are enqueued between the kernels. */
typedef struct {
  int32_t layer;     /* layer index; an entry with layer < 0 is ignored              */
  float* x_in;       /* [R, d_model] float32 residual stream entering the layer      */
  void* q;           /* [R, n_q_heads * head_dim] storage type: queries after RoPE    */
  void* attn;        /* [R, n_q_heads * head_dim] storage type: attention output      */
  float* x_mid;      /* [R, d_model] float32 residual after the o projection         */
  void* act;         /* [R, ffn_dim] storage type: SwiGLU product silu(g) * u         */
  float* x_out;      /* [R, d_model] float32 residual after the down projection      */
} uno_trace_layer;
typedef struct {
  int32_t n;                 /* entries of layer[] in use, 0..4                     */
  uno_trace_layer layer[4];
  float* logits;             /* [R, vocab] float32 logits (MASK column -inf) of the
                                forwards that run the LM head (draft, verify,
                                uno_forward with logits), or NULL                  */
} uno_trace;
/* Arm (trace != NULL; the struct is copied) or disarm (NULL) the capture.
 * UNO_ERR_INVALID_ARG when n is outside 0..4 or a layer index is >= n_layers. */
uno_status uno_set_trace(uno_ctx* ctx, const uno_trace* trace);

/* Copy a sequence's K/V for positions [0, len) in from / out to contiguous device
 * buffers [n_layers][len][n_kv_heads][head_dim] of the storage type.  Import
 * reserves pages, sets the committed length to len and the pending token and
 * iteration to the given values. */
uno_status uno_kv_import(uno_ctx* ctx, int32_t seq_id, int32_t len, const void* d_k,
                         const void* d_v, int32_t pending, int32_t iter);
uno_status uno_kv_export(uno_ctx* ctx, int32_t seq_id, int32_t len, void* d_k, void* d_v);

/* Committed length, pending token and iteration of a sequence.  Syncs. */
uno_status uno_seq_state(uno_ctx* ctx, int32_t seq_id, int32_t* len, int32_t* pending,
                         int32_t* iter);

/* Kernel timing (instrumentation).  While enabled, every kernel of the classes in
 * class_mask (bit i = class i) is launched with a pair of HIP events that the
 * runtime stamps with that kernel's own start and end on the context's stream
 * (gaps between kernels are not counted), and the algorithmic bytes and flops
 * each call must move / execute (weights, activations, LoRA, KV and outputs it
 * reads or writes once) are accumulated.  uno_timing clears the record;
 * uno_timing_read syncs and reports one class: calls (a call of a class may run
 * more than one kernel), summed kernel milliseconds, bytes and flops.  At most
 * 32768 kernels are recorded per enable. */
typedef enum {
  UNO_KC_LINEAR = 0,        /* gated-LoRA linear: q/k/v, o, down              */
  UNO_KC_LINEAR_SWIGLU = 1, /* gated-LoRA gate/up with the SwiGLU epilogue    */
  UNO_KC_LORA_DOWN = 2,     /* LoRA down-projection (the gated intermediate)  */
  UNO_KC_ATTENTION = 3,     /* paged block-causal attention (both kernels)    */
  UNO_KC_LM_HEAD = 4,       /* LM head with the softmax statistics            */
  UNO_KC_SAMPLING = 5,      /* softmax, TV, draws, accept / resample, commit  */
  UNO_KC_MISC = 6,          /* row set-up, embedding, buffer clears           */
  UNO_KC_COUNT = 7
} uno_kernel_class;
uno_status uno_timing(uno_ctx* ctx, uint32_t class_mask);
/* Record only the first of every `period` calls of each enabled class (period
 * >= 1; 1, the default, records every call).  The other calls launch without
 * events, so the events' own cost stays out of a timed stretch of work while
 * the recorded calls still sample it evenly.  Stays in force for the context;
 * uno_timing and this call restart the counting. */
uno_status uno_timing_every(uno_ctx* ctx, int32_t period);
uno_status uno_timing_read(uno_ctx* ctx, int32_t cls, int64_t* launches, double* total_ms,
                           double* bytes, double* flops);

/* Return a sequence's pages to the pool. */
uno_status uno_release(uno_ctx* ctx, int32_t seq_id);

/* Wait for the stream; report sticky device errors.  Syncs. */
uno_status uno_sync(uno_ctx* ctx);

/* Pages currently free in the pool (host bookkeeping, no sync). */
int32_t uno_free_pages(const uno_ctx* ctx);

/* Text of the last error on this context (never NULL). */
const char* uno_last_error(const uno_ctx* ctx);

void uno_destroy(uno_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* UNO_H */
