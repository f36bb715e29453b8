/*
 * tsv.h -- one round of tree-structured speculative verification on AMD
 * Instinct MI355X (gfx950), as a C ABI.
 *
 * Sources of the method (cited by page title and section):
 *   [review]   "Adapting Tree-Structured Speculative Decoding to DeepSeek-V4 for
 *              Efficient Inference" -- blog review of arXiv 2609.24698
 *   [dspark]   "DSpark: Speculative decoding ... LLM inference acceleration"
 *   [caddtree] "Cost-Aware Diffusion Draft Trees for Speculative Decoding"
 *              -- summary of arXiv 2606.01813
 *
 * A round is four calls, in this order:
 *   build_tree        drafter marginals -> best-first draft tree (+ budget)
 *                     (or build_tree_expand: per-node distributions -> tree;
 *                     select_global_budget: one budget across the batch)
 *   tree_verify_attn  branch-aware attention of every tree node
 *   accept_walk       target argmax -> longest accepted root-to-node path
 *   commit_path       accepted scratch KV -> persistent cache
 * (unfold_chains, compress_chains and refresh_compressed keep a per-chain
 * compressed state beside the KV and commit the accepted chain's part),
 * and, once per deployment, tsv_fit_cost: measured latencies -> the cost
 * model build_tree_fitted's adaptive budget uses.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer to a caller-owned, contiguous,
 *     row-major buffer, except `cost` (host).  The library never allocates,
 *     frees or synchronises, never reads device memory from the host and
 *     keeps no state between calls; calls are reentrant.
 *   - All work is enqueued on `s` (NULL = the default stream) and the call
 *     returns before it runs.
 *   - Host-side argument checks fail with a negative status before anything is
 *     launched.  A failed launch returns TSV_EHIP.  Conditions only the device
 *     can see are reported per request through output arrays (commit_path's
 *     `status`); no kernel traps.
 *   - Ragged per-request sizes (prefix lengths, node counts, accepted lengths)
 *     are read on the device only; out-of-range values are clamped, so a
 *     wrong size never leads to an access outside the documented shapes.
 *   - Floating-point inputs must be finite (marginals also non-negative);
 *     results for NaN inputs are unspecified but memory-safe.
 *   - `ws` is device scratch of at least tsv_workspace_size(...) bytes, owned
 *     by the caller, 256-byte aligned.  For the tree builders and
 *     accept_walk its contents on entry do not matter.  tree_verify_attn
 *     keeps arrival counters at the start of it (their number depends on B,
 *     N_max, Hq and Hkv only): that workspace must be all zero before its
 *     first call (e.g. one hipMemset at allocation) and again before the
 *     first call after a call with another B, N_max, Hq or Hkv; every call
 *     leaves the counters at zero, so calls at the same four sizes (any
 *     dtype, head widths or L_cap) reuse it without clearing.  It must not
 *     be shared with the other entry points.  Two calls that run
 *     concurrently need distinct workspaces.
 *
 * Notation: B requests; gamma drafter positions (= maximum tree depth);
 * V vocabulary; k top-k branches per position; N_max node capacity
 * (<= 128); n_b nodes of request b (the root excluded); l_b persistent
 * prefix length of request b (it includes the root, the last accepted
 * token); Hq / Hkv query / KV heads; d_qk / d_v key and value widths;
 * L_cap cache rows per request.
 */
#ifndef TSV_H
#define TSV_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { TSV_F32 = 0, TSV_BF16 = 1 };

enum {
  TSV_OK = 0,
  TSV_EINVAL = -1,       /* bad pointer, size or argument combination        */
  TSV_EUNSUPPORTED = -2, /* well-formed but outside what the kernels support */
  TSV_EWORKSPACE = -3,   /* workspace missing, misaligned or too small       */
  TSV_EHIP = -4          /* a kernel launch failed                           */
};

/* Round-cost coefficients ([caddtree] Methodology, item 1: the round cost is
 * the drafting cost plus a verification cost that grows with the tree size and
 * the context length):
 *   C(n; l) = c_d + C_v(n; l),  C_v(n; l) = a + b*n + c*n^2 + e*l*n.
 * Requirements: a + c_d > 0 and b, c, e >= 0 (so C > 0, convex and monotone
 * in n).  40 bytes, five doubles in this order. */
typedef struct {
  double a, b, c, e, c_d;
} tsv_cost;

/* The same family plus a term f*l that does not grow with the tree (reading
 * the prefix once), as tsv_fit_cost returns it from measured latencies
 * ([caddtree] Methodology, item 5: C_v is estimated once by convex regression
 * over node counts and context lengths):
 *   C_v(n; l) = a + b*n + c*n^2 + e*l*n + f*l,  f >= 0.
 * The first five fields are tsv_cost's; f = 0 gives exactly tsv_cost's
 * budgets. */
typedef struct {
  double a, b, c, e, c_d, f;
} tsv_cost_fitted;

/*
 * build_tree -- per-position top-k, then the greedy best-first tree.
 *
 * [caddtree] Methodology, items 2-4: the drafter's single-pass per-position
 * marginals give each candidate node a prefix probability (the product of the
 * marginals along its path); for a fixed node budget n the best tree holds
 * the n candidates of highest prefix probability, and the budget n* of a
 * round is found greedily by adding nodes best-first while the throughput
 * (1 + Phi_n) / C(n; l) still rises.  [review] "How it works", steps 1-2:
 * top-k branches per drafting step, pruned to the budget by score.
 *
 * Inputs
 *   marginals   fp32 [B][gamma][V]  drafter probabilities (finite, >= 0)
 *   top_k       1 <= top_k <= min(V, 128)
 *   n_budget    cost == NULL: the fixed budget D (n_b = min(D, #candidates));
 *               cost != NULL: the cap of the adaptive budget.  0 <= n_budget
 *               <= N_max.
 *   cost        HOST pointer or NULL (fixed budget)
 *   prefix_len  int32 [B], read only when cost != NULL (l in C_v)
 *   N_max       1 <= N_max <= 128; gamma <= 64; gamma * top_k <= 4096
 * Outputs (device, written for every b and every i < N_max)
 *   n_nodes     int32 [B]
 *   parent      int32 [B][N_max]  parent node index, -1 = child of the root
 *   token       int32 [B][N_max]  drafted token id
 *   depth       int32 [B][N_max]  1-based depth (= drafter position + 1)
 *   score       fp32  [B][N_max]  prefix probability
 *   anc_bits    uint32 [B][N_max][ceil(N_max/32)]  bit j of row i set iff node
 *               j is node i or one of its ancestors
 *   Entries i >= n_nodes[b] are -1 (ints), 0.0f (score) and 0 (anc_bits).
 * Workspace: tsv_workspace_size(0, B, gamma, V, top_k, N_max, ...) bytes,
 * any contents (it holds the per-position top-k table between the two
 * stages).
 * Order and ties
 *   top-k: probability descending, then token id ascending (-0 == +0).
 *   nodes: numbered in best-first order, i.e. ascending by the nested key
 *   (-score, depth, key(parent), rank), so parents precede children.
 *   Scores are fp32 products parent_score * q (root 1, round-to-nearest,
 *   never fused); Phi and C are fp64 in the order
 *   c_d + (((a + b*n) + c*(n*n)) + (e*l)*n); a node is added iff
 *   (1 + Phi_{n+1}) / C(n+1) > (1 + Phi_n) / C(n).
 */
int build_tree(const float* marginals, int B, int gamma, int V, int top_k,
               int n_budget, const tsv_cost* cost, const int* prefix_len,
               int N_max, int* n_nodes, int* parent, int* token, int* depth,
               float* score, unsigned* anc_bits, void* ws, size_t ws_bytes,
               hipStream_t s);

/*
 * build_tree_topk -- build_tree that also returns the per-position top-k
 * lists of its first stage, so that stage can be checked on its own.
 *
 * [caddtree] Methodology, item 2 and [review] "How it works", step 1: the
 * top-k tokens of every drafter position are the branches a node at that
 * depth may take.
 *
 * Arguments, results and errors are build_tree's, plus two outputs (device,
 * both required):
 *   topk_idx    int32 [B][gamma][top_k]  token ids, probability descending,
 *               then token id ascending
 *   topk_p      fp32  [B][gamma][top_k]  their probabilities (bit copies)
 * Same workspace as build_tree; the tree outputs are bit-identical to
 * build_tree's.
 */
int build_tree_topk(const float* marginals, int B, int gamma, int V, int top_k,
                    int n_budget, const tsv_cost* cost, const int* prefix_len,
                    int N_max, int* n_nodes, int* parent, int* token, int* depth,
                    float* score, unsigned* anc_bits, int* topk_idx, float* topk_p,
                    void* ws, size_t ws_bytes, hipStream_t s);

/*
 * build_tree_noalloc -- build_tree without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, results and errors are build_tree's without `ws` / `ws_bytes`:
 * the per-position top-k table between the two stages lives in a scratch
 * array of 4 MiB that the library holds on every GPU it runs on until the
 * process ends (its address is looked up once per device, on the first call
 * there).  Nothing is allocated or freed.  Limit: 8 * B * gamma * top_k <=
 * 4 MiB (e.g. 64 requests x 16 positions x top-128); larger calls return
 * TSV_EUNSUPPORTED before any launch.  The table's contents on entry do not
 * matter, so nothing is cleared.  Every call on one GPU uses the same array:
 * calls whose kernels may overlap on one GPU (different streams, or other
 * threads) race and must be serialised by the caller.
 */
int build_tree_noalloc(const float* marginals, int B, int gamma, int V, int top_k,
                       int n_budget, const tsv_cost* cost, const int* prefix_len,
                       int N_max, int* n_nodes, int* parent, int* token, int* depth,
                       float* score, unsigned* anc_bits, hipStream_t s);

/*
 * build_tree_fitted -- build_tree under a fitted cost model (the extra f*l
 * term, tsv_cost_fitted).
 *
 * [caddtree] Methodology, item 5: the verification cost measured on the
 * serving hardware and fitted by convex regression drives the same greedy
 * stop.  Arguments, results, workspace and errors are build_tree's; `cost`
 * (HOST, or NULL for the fixed budget) is a tsv_cost_fitted, and the stop
 * rule evaluates C in the order c_d + ((((a + b*n) + c*(n*n)) + (e*l)*n) +
 * f*l), so f = 0 reproduces build_tree bit for bit.
 */
int build_tree_fitted(const float* marginals, int B, int gamma, int V, int top_k,
                      int n_budget, const tsv_cost_fitted* cost, const int* prefix_len,
                      int N_max, int* n_nodes, int* parent, int* token, int* depth,
                      float* score, unsigned* anc_bits, void* ws, size_t ws_bytes,
                      hipStream_t s);

/*
 * build_tree_expand -- the same tree from per-node conditional expansion.
 *
 * [review] "How it works", steps 1-2, and its notation (s draft steps,
 * top-k, budget D): the drafter runs s steps; at each step every node of the
 * newest level branches into the top-k tokens of its OWN next-token
 * distribution (the toy: A -> {B, C}, then B -> {B, C} and C -> {A, B}), and
 * the candidates are pruned to the budget by cumulative score.  [review] "Our
 * perspective": pruning by cumulative score.  The budget rules are
 * build_tree's ([caddtree] Methodology, items 2-4).
 *
 * Inputs
 *   probs       fp32 [B][P][V]  the expanded nodes' next-token distributions
 *               (finite, >= 0), P = 1 + k + ... + k^(steps-1), in level order
 *               of the complete k-ary expansion: row 0 is the root's (the last
 *               accepted token), and the child of rank r (in the top-k order
 *               below) of the node with row i has row k*i + 1 + r.  Nodes of
 *               depth `steps` are leaves and have no row.
 *   steps       1 <= steps <= 64 (maximum depth)
 *   top_k       1 <= top_k <= min(V, 128); P * top_k <= 4096
 *   n_budget, cost, prefix_len, N_max   as for build_tree
 * Outputs       as for build_tree, with depth = draft step and
 *   topk_idx    int32 [B][P][top_k] or NULL   each row's top-k ids
 *   topk_p      fp32  [B][P][top_k] or NULL   and their probabilities
 * Order, ties and arithmetic are build_tree's: a candidate's score is the
 * fp32 product of the probabilities along its path, nodes are numbered by
 * the nested key (-score, depth, key(parent), rank), so the tree is
 * ancestor-closed and parents precede children.
 * Workspace: tsv_workspace_size(4, B, steps, V, top_k, N_max, ...).
 */
int build_tree_expand(const float* probs, int B, int steps, int V, int top_k,
                      int n_budget, const tsv_cost* cost, const int* prefix_len,
                      int N_max, int* n_nodes, int* parent, int* token, int* depth,
                      float* score, unsigned* anc_bits, int* topk_idx, float* topk_p,
                      void* ws, size_t ws_bytes, hipStream_t s);

/*
 * select_global_budget -- one verification budget for the whole batch.
 *
 * [dspark] Confidence-scheduled verification, hardware-aware prefix
 * scheduler: verification lengths are chosen by one global throughput
 * maximisation over the R active requests, Theta = tau * SPS(B), SPS a
 * table of engine steps per second at batch size B profiled once; a global
 * sort of the candidates and greedy admission respect each request's prefix
 * order (its survival probabilities do not increase along it), and admission
 * stops as soon as the throughput would fall.
 *
 * Applied to trees built by build_tree / build_tree_expand (typically with a
 * fixed budget as the per-request cap): request r's candidates are its first
 * n_nodes[r] nodes in best-first order with their scores a_{r,j};
 * tau = R + admitted scores, B = R + admitted nodes (every request verifies
 * its root plus its admitted nodes).  Candidates go in the order score
 * descending, request ascending, position ascending; the next one is
 * admitted iff (tau + a) * SPS(B + 1) > tau * SPS(B), in fp64 with tau summed
 * in admission order; the walk stops at the first refusal or when B + 1
 * reaches sps_len.  Every request keeps a prefix of its nodes, so its tree
 * stays ancestor-closed.
 *
 * In/out (device): n_nodes [B] (available -> admitted), and the tree arrays
 * of build_tree, whose entries at or past the admitted count are reset to
 * build_tree's padding (-1, 0.0f, 0).  sps: DEVICE double [sps_len],
 * finite and >= 0.  Scores must be finite and >= 0 (-0 == +0).
 * Limits: N_max <= 128, B <= 4096, B * N_max <= 8192.  One workgroup, no
 * workspace.
 */
int select_global_budget(int* n_nodes, int* parent, int* token, int* depth, float* score,
                         unsigned* anc_bits, int B, int N_max, const double* sps,
                         long sps_len, hipStream_t s);

/*
 * unfold_chains -- a draft tree as its root-to-leaf chains.
 *
 * [review] "How it works", step 4 (verify preprocess): the tree is unfolded
 * into chains -- the toy's A-B, A-C, A-B-B becomes Chain1 = A-B-B and
 * Chain2 = A-C -- so that the prefix's state is shared and everything after
 * the branch point is kept per chain; step 6 commits only the accepted
 * chain's state.
 *
 * A chain is the path from the root to one leaf (a node no node names as
 * parent), root side first; chains are numbered by their leaf's index; the
 * root (the last prefix token) is not part of a chain.
 * Inputs (device): n_nodes int32 [B], parent int32 [B][N_max] as written by
 * build_tree (parent values outside [-1, i) are read as -1, so a malformed
 * tree stays memory-safe); N_max <= 128; 1 <= gamma <= 64 (maximum depth).
 * Outputs (device): n_chains int32 [B]; chain_len int32 [B][N_max] (0 past
 * the last chain; a chain deeper than gamma keeps its first gamma nodes);
 * chain_nodes int32 [B][N_max][gamma], node indices, -1 past each chain.
 */
int unfold_chains(const int* n_nodes, const int* parent, int B, int N_max, int gamma,
                  int* n_chains, int* chain_len, int* chain_nodes, hipStream_t s);

/*
 * compress_chains -- every chain's compressed state (verify preprocess).
 *
 * [review] "How it works", steps 4 and 6, and "Secret weapon" (paper
 * sections 4.1-4.2 as summarised there): the prefix's compressed state is
 * reused, compression after the branch point is done per chain (one
 * compression over two chains would mix exclusive histories), and the
 * chains' temporary compressed tokens and intermediate buffers stay in a
 * scratch pad.  The pages give no formula for DeepSeek-V4's C4 / C128
 * compression; this library uses the block mean as a stand-in: entry j of a
 * token sequence is the mean of the rows of positions j*c .. j*c + c - 1,
 * and the intermediate buffer ("tail") is the fp32 sum of the rows of the
 * incomplete last block.
 *
 * For request b (prefix length l_b) and chain q < n_chains[b]: s = tail[b];
 * for t = 0 .. chain_len - 1, s += the scratch row of chain node t; when
 * l_b + t + 1 is a multiple of c, entry s / c is written and s restarts at
 * zero.  Each column is summed in that order in fp32.
 *   rows        dtype [B][N_max] rows of row_stride elements (the scratch
 *               keys or values, e.g. k_tree with E = Hkv*d_k); the first E
 *               columns are compressed
 *   tail        fp32 [B][E]; prefix_len int32 [B]
 *   n_chains, chain_len, chain_nodes  as written by unfold_chains (gamma)
 * Outputs (device): entries fp32 [B][N_max][M][E], M = (c - 1 + gamma) / c,
 * entries past each chain's count untouched; n_entries int32 [B][N_max]:
 * the count written, 0 past the last chain, -1 for a chain that cannot be
 * read (negative prefix length or a node index outside [0, N_max); nothing
 * written for it).
 * Requirements: 1 <= c <= 65536 (4 and 128 for C4 / C128); row_stride >= E >= 1,
 * E <= 2^24; N_max <= 128; 1 <= gamma <= 64.
 */
int compress_chains(const void* rows, int dtype, long row_stride, long E, int c,
                    const float* tail, const int* prefix_len, const int* n_chains,
                    const int* chain_len, const int* chain_nodes, int B, int N_max,
                    int gamma, float* entries, int* n_entries, hipStream_t s);

/*
 * refresh_compressed -- commit the accepted chain's compressed state.
 *
 * [review] "How it works", step 6: when a path is accepted only its chain's
 * KV and compressed state reach the persistent cache; the other chains'
 * temporary compressed tokens and buffers are dropped.  Call it after
 * accept_walk and before commit_path (prefix_len is the length before the
 * round's commit).
 *
 * For request b with m = accept_len[b]: q = the lowest-numbered chain whose
 * node m - 1 is accept_nodes[b][m-1] (any chain through it gives the same
 * result); the e = (l_b % c + m) / c blocks closed by the accepted tokens
 * are copied from entries[b][q] to comp[b][l_b / c ...]; tail[b] becomes
 * tail[b] plus the accepted rows when e == 0, else the sum of the accepted
 * rows after the last closed block (in sequence order, fp32).
 *   entries     as compress_chains wrote them for the same prefix lengths
 *   comp        fp32 [B][Lc_cap][E] persistent compressed entries (in/out)
 *   tail        fp32 [B][E] (in/out)
 * status int32 [B]: 0 done (m == 0 changes nothing); 1 l_b / c + e > Lc_cap
 * (nothing written); 2 m outside [0, gamma], l_b < 0, an accepted node
 * outside [0, N_max) or no chain holding the path (nothing written).
 * Requirements as for compress_chains; Lc_cap >= 0.
 */
int refresh_compressed(const void* rows, int dtype, long row_stride, long E, int c,
                       const int* prefix_len, const int* accept_len, const int* accept_nodes,
                       const int* n_chains, const int* chain_len, const int* chain_nodes,
                       const float* entries, int B, int N_max, int gamma, float* comp,
                       int Lc_cap, float* tail, int* status, hipStream_t s);

/*
 * tree_verify_attn -- branch-aware tree attention over a shared prefix.
 *
 * [review] Difficulty 1 (paper section 3.1) and "How it works", step 3: each
 * candidate attends only to its own ancestors, never to other branches;
 * section 6 as quoted: with dense attention the tree is a mask over the
 * shared KV.  For request b, node i < n_b and query head h the keys are the
 * prefix rows 0..l_b-1 plus the scratch rows j whose bit is set in
 * anc_bits[b][i]; out = softmax(sm_scale * q.K^T) V and
 * lse = log(sum(exp(sm_scale * q.K^T))) (natural log).  Query head h uses KV
 * head h / (Hq / Hkv).
 *
 * Layouts (dtype TSV_BF16 or TSV_F32 for q, caches, scratch and out)
 *   q         [B][N_max][Hq][d_qk]
 *   k_cache   [B][L_cap] rows of kv_row_stride elements; KV head g's key is
 *             at element offset g*d_qk of a row
 *   v_cache   same row layout; head g's value is at offset g*d_v.  A latent
 *             cache (one head whose value is the first d_v columns of the
 *             key) passes v_cache == k_cache.
 *   k_tree, v_tree  [B][N_max] rows of kv_row_stride elements (scratch pad)
 *   prefix_len int32 [B]  (clamped to [0, L_cap])
 *   n_nodes   int32 [B]   (clamped to [0, N_max])
 *   anc_bits  uint32 [B][N_max][ceil(N_max/32)]  as written by build_tree
 *   out       [B][N_max][Hq][d_v]  rows i >= n_b are left untouched
 *   lse       fp32 [B][N_max][Hq] or NULL
 * Requirements: Hq % Hkv == 0; kv_row_stride >= Hkv*max(d_qk, d_v);
 * 1 <= d_qk, d_v <= 576; B <= 4096.  Accumulation is fp32.
 * Workspace: tsv_workspace_size(1, ...) bytes (enough for every path at
 * these sizes), zero before the first call at these B, N_max, Hq, Hkv (see
 * the conventions above).  The key
 * range of a (request, KV head, row block) may be split over several
 * workgroups whose partial results are combined in fp32 (for bf16 heads of
 * width 128 the partial rows are exchanged normalised and rounded to bf16),
 * so the exact rounding of `out` depends on the split sizes (which depend on
 * B, N_max, L_cap and the head shape, never on the data or on timing).
 */
int tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const void* k_tree, const void* v_tree, long kv_row_stride,
                     const int* prefix_len, const int* n_nodes,
                     const unsigned* anc_bits, int B, int N_max, int L_cap,
                     int Hq, int Hkv, int d_qk, int d_v, int dtype,
                     float sm_scale, void* out, float* lse, void* ws,
                     size_t ws_bytes, hipStream_t s);

/*
 * accept_walk -- greedy acceptance of the longest matching path.
 *
 * [review] "How it works", steps 5-6 and [dspark] decoding cycle: the target
 * verifies all branches at once; the accepted tokens are the longest
 * root-to-node path whose every token equals the target's argmax at its
 * parent, followed by the target's own next token (the bonus).
 *
 *   target_logits  dtype [B][1 + N_max][V]; row 0 = the root's prediction,
 *                  row 1+i = node i's.  Only rows 0..n_b are read.
 *   n_nodes, parent, token  as written by build_tree
 * Outputs
 *   accept_len   int32 [B]          m_b, accepted tree nodes (bonus excluded)
 *   accept_nodes int32 [B][gamma]   accepted node indices, then -1
 *   out_tokens   int32 [B][gamma+1] accepted tokens, the bonus, then -1
 * argmax ties go to the lowest token id; the walk stops after gamma steps;
 * if several children of a node carry the argmax token (impossible for trees
 * from build_tree) the lowest node index is taken.
 */
int accept_walk(const void* target_logits, int dtype, int B, int N_max, int V,
                int gamma, const int* n_nodes, const int* parent,
                const int* token, int* accept_len, int* accept_nodes,
                int* out_tokens, void* ws, size_t ws_bytes, hipStream_t s);

/*
 * commit_path -- write the accepted chain into the persistent cache.
 *
 * [review] "Secret weapon" (paper section 4.2 as quoted) and "How it works",
 * step 6: tentative branch state stays in the scratch pad; after selection
 * only the accepted path's KV is written to the persistent cache and the
 * rest is discarded; the next round starts from the extended prefix.
 *
 * For j < m_b: cache row l_b + j <- scratch row accept_nodes[b][j] (the first
 * Hkv*d_k elements of a key row and Hkv*d_v of a value row); then
 * prefix_len[b] += m_b.  v_cache/v_tree may be NULL (latent cache).
 * status int32 [B]: 0 committed; 1 l_b + m_b > L_cap (nothing written);
 * 2 m_b outside [0, gamma], l_b < 0 or a node index outside [0, N_max)
 * (nothing written).  Rows of rejected nodes are never read.
 */
int commit_path(void* k_cache, void* v_cache, int* prefix_len,
                const void* k_tree, const void* v_tree, long kv_row_stride,
                const int* accept_len, const int* accept_nodes, int B,
                int N_max, int L_cap, int Hkv, int d_k, int d_v, int gamma,
                int dtype, int* status, hipStream_t s);

/*
 * tsv_fit_cost -- the convex, monotone verification cost from measured
 * latencies (host computation, run once, offline).
 *
 * [caddtree] Methodology, item 5: C_v(n; l) is estimated once by convex
 * regression on latencies measured over node counts and context lengths,
 * which keeps it convex and monotone so that the throughput objective of
 * item 3 stays unimodal (the greedy stop of build_tree is then exact).
 *
 * Fits C_v(n; l) = a + b*n + c*n^2 + e*l*n + f*l with a, b, c, e, f >= 0 by
 * non-negative least squares: the model is non-decreasing and convex in n
 * for every l, and non-decreasing in l.
 *
 * Inputs (HOST pointers): n, l, t double [m], the node count, context length
 * and measured verification latency of each point (finite, >= 0; t in any
 * time unit); 5 <= m <= 2^24; c_d the drafting cost in the same unit
 * (copied to out->c_d).
 * Output: *out (HOST) = {a, b, c, e, c_d, f}, ready for build_tree_fitted's
 * `cost`.
 * When every point has one context length, e and f are not separable from
 * b and a; the optimum's value is still unique and the first optimal
 * support in the order (a, b, c, e, f) is returned.
 * Returns TSV_OK, or TSV_EINVAL for null pointers, m out of range or
 * non-finite / negative inputs (out untouched).  Allocates nothing and
 * touches no device.
 */
int tsv_fit_cost(const double* n, const double* l, const double* t, int m,
                 double c_d, tsv_cost_fitted* out);

/* Workspace bytes needed by entry point `which` (0 build_tree,
 * 1 tree_verify_attn, 2 accept_walk, 3 commit_path, 4 build_tree_expand,
 * whose `gamma` argument is its number of steps) for these sizes.
 * Arguments an entry point does not use are ignored.  Returns 0 for
 * invalid sizes. */
size_t tsv_workspace_size(int which, int B, int gamma, int V, int top_k,
                          int N_max, int L_cap, int Hq, int Hkv, int d_qk,
                          int d_v, int dtype);

/* Static description of a status code. */
const char* tsv_status_string(int code);

/* Diagnostic switch for the tree selection of build_tree, build_tree_topk,
 * build_tree_fitted and build_tree_noalloc (per-position lists; the
 * cost-aware page, "Methodology", item 2).  Two exact methods compute the
 * same best-first tree: serial pops (one per node) and a level-by-level
 * merge; by default (method 0) both run side by side in each request's
 * workgroup and the first to finish writes the tree.  Method 1 runs the
 * serial pops only, method 2 the level merge only; every method returns
 * the same bits.  Process-wide (every device), read when a call is
 * launched; not synchronised with calls in flight on other host threads.
 * Returns the previous method, or TSV_EINVAL (setting unchanged) for a
 * method outside 0..2. */
int tsv_set_tree_method(int method);

#ifdef __cplusplus
}
#endif

#endif /* TSV_H */
