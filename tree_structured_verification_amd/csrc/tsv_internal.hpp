// Host-side interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tsv.h"

namespace tsv {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Waves a streaming scan aims to keep in flight (about 16 per CU on a
// 256-CU part); fixed so that results never depend on the device.
constexpr int kScanWaves = 4096;

// ---- build_tree --------------------------------------------------------
struct TopkPlan {
  int rows, V, k, slots, nseg;
  bool vec;
};
TopkPlan topk_plan(int rows, int V, int k);
hipError_t launch_topk(const float* x, const TopkPlan& p, int* out_idx, float* out_p, hipStream_t s);

struct TreeArgs {
  const int* tk_idx;
  const float* tk_p;
  int B, gamma, k, N_max, cap, adaptive;
  // rows of top-k lists per request: gamma (one per position), or the
  // expanded nodes in level order when per_node is set
  int rows, per_node;
  // per-position lists: 0 = serial pops and level merge side by side,
  // 1 = serial pops only, 2 = level merge only
  int method;
  tsv_cost_fitted cost;
  const int* prefix_len;
  int* n_nodes;
  int* parent;
  int* token;
  int* depth;
  float* score;
  unsigned* anc_bits;
};
hipError_t launch_best_first(const TreeArgs& a, hipStream_t s);

// ---- select_global_budget ----------------------------------------------
constexpr int kMaxGlobalRequests = 4096;
constexpr int kMaxGlobalCandidates = 8192;   // B * N_max, sorted in LDS
struct GlobalBudgetArgs {
  int* n_nodes;
  int* parent;
  int* token;
  int* depth;
  float* score;
  unsigned* anc_bits;
  int B, N_max;
  const double* sps;
  long sps_len;
};
hipError_t launch_global_budget(const GlobalBudgetArgs& a, hipStream_t s);

// ---- unfold_chains -------------------------------------------------------
struct ChainArgs {
  const int* n_nodes;
  const int* parent;
  int B, N_max, gamma;
  int* n_chains;
  int* chain_len;
  int* chain_nodes;
};
hipError_t launch_unfold_chains(const ChainArgs& a, hipStream_t s);

// ---- compress_chains / refresh_compressed --------------------------------
struct CompressArgs {
  const void* rows;        // scratch rows [B][N_max], row_stride elements each
  long row_stride, E;
  int c;
  const float* tail;       // [B][E]
  const int* prefix_len;   // [B]
  const int* n_chains;     // [B]
  const int* chain_len;    // [B][N_max]
  const int* chain_nodes;  // [B][N_max][gamma]
  int B, N_max, gamma;
  float* entries;          // [B][N_max][(c - 1 + gamma) / c][E]
  int* n_entries;          // [B][N_max]
};
hipError_t launch_compress_chains(const CompressArgs& a, int dtype, bool vec, hipStream_t s);

struct RefreshArgs {
  const void* rows;
  long row_stride, E;
  int c;
  const int* prefix_len;
  const int* accept_len;   // [B]
  const int* accept_nodes; // [B][gamma]
  const int* n_chains;
  const int* chain_len;
  const int* chain_nodes;
  const float* entries;
  int B, N_max, gamma;
  float* comp;             // [B][Lc_cap][E]
  int Lc_cap;
  float* tail;             // [B][E]
  int* status;             // [B]
};
hipError_t launch_refresh_compressed(const RefreshArgs& a, int dtype, hipStream_t s);

// ---- accept_walk -------------------------------------------------------
struct ArgmaxPlan {
  int rows, V, nseg, seg_len;
  bool vec;
};
ArgmaxPlan argmax_plan(int rows, int V, int dtype);
hipError_t launch_accept_walk(const void* logits, int dtype, int B, int N_max,
                              int V, int gamma, const int* n_nodes,
                              const int* parent, const int* token,
                              int* accept_len, int* accept_nodes,
                              int* out_tokens, uint64_t* seg_best,
                              const ArgmaxPlan& p, hipStream_t s);

// ---- commit_path -------------------------------------------------------
hipError_t launch_commit(void* k_cache, void* v_cache, int* prefix_len,
                         const void* k_tree, const void* v_tree,
                         size_t row_bytes, const int* accept_len,
                         const int* accept_nodes, int B, int N_max, int L_cap,
                         size_t k_bytes, size_t v_bytes, int gamma,
                         int* status, hipStream_t s);

// ---- tree_verify_attn --------------------------------------------------
enum AttnPath { kPathValu = 0, kPathMfmaGqa = 1, kPathMfmaLatent = 2 };

struct AttnShape {
  int B, N_max, L_cap, Hq, Hkv, d_qk, d_v, dtype;
};
struct AttnPlan {
  AttnPath path;
  int RB;            // query rows (node x head) per work item
  int KT;            // keys per tile
  int min_chunk;     // smallest split of the key range
  int target_items;  // work items aimed for
  int items_max;     // bound on work items for any prefix lengths / node counts
  // grouped-query path (one kernel, split-K combined by the last split):
  int chunk;         // smallest split, in keys
  int S;             // splits per unit at most
  int units;         // request x KV head x row block
  int rbs;           // row blocks per (request, KV head)
  size_t off_cnt;    // arrival counters, one int per unit (zero between calls)
  size_t off_info, off_desc, off_ml, off_acc, bytes;
};
// `aligned` says whether pointers and strides allow 16-byte vector access;
// `shared_value` whether the value rows are the key rows (one latent head).
AttnPlan attn_plan(const AttnShape& sh, bool aligned, bool shared_value);

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kt;
  const void* vt;
  long stride;
  const int* prefix_len;
  const int* n_nodes;
  const unsigned* anc;
  int B, N_max, L_cap, Hq, Hkv, G, d_qk, d_v, W;
  float scale_log2;
  void* out;
  float* lse;
  int* info;        // [B][4] item_base, splits, rowblocks, prefix; then chunk, total
  int4* desc;       // [items_max] request, kv head, row block, split
  float* part_ml;   // [items_max][RB][2]
  float* part_acc;  // [items_max][RB][d_v]
  int RB, KT, items_max, target_items, min_chunk;
  int* counters;    // [units] arrival counters (grouped-query path)
  int chunk, S, units, rbs;
};
hipError_t launch_attention(const AttnArgs& a, AttnPath path, int dtype,
                            hipStream_t s);

}  // namespace tsv
