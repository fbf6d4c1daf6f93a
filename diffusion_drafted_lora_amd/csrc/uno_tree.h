// The tree sampler of the Psi-Spec step (the batch-1 mode): K drafted chains share
// one draft forward and one verify forward; acceptance walks the tree of their
// common prefixes with recursive rejection sampling (ai-papers-daily summary,
// method key points: a linear sampler for system throughput and a tree sampler for
// single-request throughput; the candidate-set construction is this library's
// reading, stated in uno.h).
#pragma once
#include "uno_internal.h"

constexpr int TREE_KMAX = 16;   // chains per sequence

// Verify row holding chain k's token at depth (1..B): row 0 is the shared y_1,
// then B - 1 rows per chain for depths 2..B.
UNO_DEV int tree_row(int k, int depth, int B) {
  return depth == 1 ? 0 : 1 + k * (B - 1) + (depth - 2);
}

// K chains per sequence: chain k's depth-d token is a draw from draft row d - 1
// with counter (n + d, draft stream, iteration, d == 1 ? 0 : k), written to
// chains[s][k][d - 1]; the descriptors feed launch_cdf (n * K * B rows).
hipError_t launch_tree_draft_desc(const float* probs, int n, int K, int B, int V, uint64_t seed,
                                  const int32_t* call_seq, const int32_t* call_n,
                                  const int32_t* call_it, int32_t* chains, RowDesc* desc,
                                  hipStream_t s);

struct TreeAcceptArgs {
  const float* p;            // [n, p_rows, V] verify laws (rows as tree_row)
  const float* q;            // [n, q_rows, V] draft laws; depth d uses row d - 1
  int32_t p_rows, q_rows;
  const int32_t* chains;     // [n, K, B]
  const int32_t* seq_ids;    // [n] (device)
  const int32_t* pos;        // [n] pending position of each sequence
  const int32_t* iter;       // [n]
  int32_t K, B, V;
  uint64_t seed;
  uint64_t* resid;           // [n, V] residual masses (scratch)
  int32_t* path;             // [n, B] accepted tokens y_1, ... (the emitted prefix)
  int32_t* k_out;            // [n] tokens emitted (the stop depth, B + 1 when all pass)
  int32_t* kstar;            // [n] lowest chain on the accepted path
  int32_t* z;                // [n] correction / bonus token (drawn by launch_cdf)
  RowDesc* desc;             // [n] the correction draw's row
  int32_t* err;
};
// One workgroup per sequence; the correction draws follow with launch_cdf(desc, n).
hipError_t launch_tree_accept(const TreeAcceptArgs& a, int n, hipStream_t s);

// After acceptance: when the accepted path follows chain kstar > 0, its K/V of
// depths 2..k_out-1 move from slots n + 2 + kstar (B - 1) + (d - 2) to their
// positions n + d (every layer, K and V).
template <typename T>
hipError_t launch_tree_kv_move(const KvLayout& kv, int n, int B, int n_layers,
                               const int32_t* call_seq, const int32_t* call_n,
                               const int32_t* k_out, const int32_t* kstar, int32_t* err,
                               hipStream_t s);
