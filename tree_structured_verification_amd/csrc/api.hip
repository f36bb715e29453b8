// C ABI of the tree-structured verification library: argument checks,
// workspace layout and kernel launches.  Nothing here allocates, frees,
// synchronises or reads device memory.

#include <math.h>

#include <atomic>
#include <mutex>

#include "tsv_internal.hpp"

using namespace tsv;

// Scratch of build_tree_noalloc: the top-k table between its two kernels
// (8 bytes per list entry, B * gamma * top_k entries).  Every GPU the library
// runs on holds its own copy until the process ends; host code never uses
// this name as an address (it is a host-side stand-in), only the device
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t{4} << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxNodes = 128;
constexpr int kMaxGamma = 64;
// columns of a compressed row (grid y = columns / 1024 stays far below its limit)
constexpr long kMaxCompressCols = 1L << 24;
// tokens per compressed block
constexpr int kMaxBlock = 1 << 16;
constexpr int kMaxTopk = 128;
constexpr int kMaxTopkTable = 4096;  // gamma * top_k staged in LDS by the tree kernel
constexpr int kMaxHeadDim = 576;
constexpr int kMaxAttnBatch = 4096;   // request table of the attention planner lives in LDS

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int esize(int dtype) { return dtype == TSV_F32 ? 4 : 2; }
bool dtype_ok(int dtype) { return dtype == TSV_F32 || dtype == TSV_BF16; }

bool finite_nonneg(double x) { return isfinite(x) && x >= 0.0; }

int launch_status(hipError_t e) { return e == hipSuccess ? TSV_OK : TSV_EHIP; }

struct BuildLayout {
  TopkPlan plan;
  size_t off_idx, off_p, bytes;
};
// rows_per_b: top-k lists per request (gamma positions, or the expanded
// nodes of build_tree_expand)
BuildLayout build_layout(int B, int rows_per_b, int V, int top_k) {
  BuildLayout L;
  const int rows = B * rows_per_b;
  L.plan = topk_plan(rows, V, top_k);
  size_t off = 0;
  L.off_idx = off;
  off = align_up(off + static_cast<size_t>(rows) * top_k * sizeof(int));
  L.off_p = off;
  off = align_up(off + static_cast<size_t>(rows) * top_k * sizeof(float));
  L.bytes = off;
  return L;
}

bool build_sizes_ok(int B, int gamma, int V, int top_k, int N_max) {
  if (B < 1 || gamma < 1 || V < 1 || top_k < 1 || N_max < 1) return false;
  if (gamma > kMaxGamma || N_max > kMaxNodes || top_k > kMaxTopk || top_k > V) return false;
  if (gamma * top_k > kMaxTopkTable) return false;
  if (static_cast<long long>(B) * gamma > (1LL << 24)) return false;
  return true;
}

// Expanded nodes of an s-step, k-ary expansion: 1 + k + ... + k^(s-1), or
// -1 when that exceeds kMaxTopkTable (the tree kernel's list table).
int expanded_rows(int steps, int k) {
  long long rows = 0, level = 1;
  for (int d = 0; d < steps; ++d) {
    rows += level;
    if (rows > kMaxTopkTable) return -1;
    level *= k;
    if (level > kMaxTopkTable) level = kMaxTopkTable + 1;
  }
  return static_cast<int>(rows);
}

bool expand_sizes_ok(int B, int steps, int V, int top_k, int N_max) {
  if (B < 1 || steps < 1 || V < 1 || top_k < 1 || N_max < 1) return false;
  if (steps > kMaxGamma || N_max > kMaxNodes || top_k > kMaxTopk || top_k > V) return false;
  const int P = expanded_rows(steps, top_k);
  if (P < 0 || static_cast<long long>(P) * top_k > kMaxTopkTable) return false;
  if (static_cast<long long>(B) * P > (1LL << 24)) return false;
  return true;
}

bool cost_ok(const tsv_cost_fitted* cost) {
  return isfinite(cost->a) && isfinite(cost->c_d) && cost->a + cost->c_d > 0.0 &&
         finite_nonneg(cost->b) && finite_nonneg(cost->c) && finite_nonneg(cost->e) &&
         finite_nonneg(cost->f);
}

// The plain family as the fitted one with f = 0: the stop rule appends + f*l
// last, and v + 0.0 == v for the positive v it is added to, so the budgets
// are bit-identical.
tsv_cost_fitted widen(const tsv_cost& c) { return tsv_cost_fitted{c.a, c.b, c.c, c.e, c.c_d, 0.0}; }

// method of the per-position tree selection (tsv_set_tree_method)
std::atomic<int> g_tree_method{0};

// top-k of every list, then the best-first tree; shared by both builders
int launch_build(const float* probs, int B, int rows_per_b, int steps, int V, int top_k,
                 int n_budget, const tsv_cost_fitted* cost, const int* prefix_len, int N_max,
                 int* n_nodes, int* parent, int* token, int* depth, float* score,
                 unsigned* anc_bits, int* topk_idx, float* topk_p, void* ws,
                 size_t ws_bytes, hipStream_t s, bool per_node) {
  const BuildLayout L = build_layout(B, rows_per_b, V, top_k);
  if (!ws || ws_bytes < L.bytes || !aligned_to(ws, kAlign)) return TSV_EWORKSPACE;
  char* w = static_cast<char*>(ws);
  int* tk_idx = topk_idx ? topk_idx : reinterpret_cast<int*>(w + L.off_idx);
  float* tk_p = topk_p ? topk_p : reinterpret_cast<float*>(w + L.off_p);
  hipError_t e = launch_topk(probs, L.plan, tk_idx, tk_p, s);
  if (e != hipSuccess) return TSV_EHIP;
  TreeArgs a;
  a.tk_idx = tk_idx;
  a.tk_p = tk_p;
  a.B = B;
  a.gamma = steps;
  a.k = top_k;
  a.N_max = N_max;
  a.cap = n_budget;
  a.adaptive = cost ? 1 : 0;
  a.rows = rows_per_b;
  a.per_node = per_node ? 1 : 0;
  a.method = g_tree_method.load(std::memory_order_relaxed);
  a.cost = cost ? *cost : tsv_cost_fitted{0, 0, 0, 0, 0, 0};
  a.prefix_len = prefix_len;
  a.n_nodes = n_nodes;
  a.parent = parent;
  a.token = token;
  a.depth = depth;
  a.score = score;
  a.anc_bits = anc_bits;
  return launch_status(launch_best_first(a, s));
}

bool attn_sizes_ok(int B, int N_max, int L_cap, int Hq, int Hkv, int d_qk, int d_v) {
  if (B < 1 || N_max < 1 || N_max > kMaxNodes || L_cap < 0 || Hq < 1 || Hkv < 1) return false;
  if (B > kMaxAttnBatch) return false;
  if (Hq % Hkv != 0) return false;
  if (d_qk < 1 || d_v < 1 || d_qk > kMaxHeadDim || d_v > kMaxHeadDim) return false;
  if (static_cast<long long>(B) * N_max * Hq > (1LL << 30)) return false;
  return true;
}

size_t attn_bytes_any(const AttnShape& sh) {
  size_t m = 0;
  for (int mode = 0; mode < 4; ++mode) {
    const size_t x = attn_plan(sh, (mode & 1) != 0, (mode & 2) != 0).bytes;
    m = x > m ? x : m;
  }
  return m;
}

size_t walk_bytes(int B, int N_max, int V, int dtype) {
  const int rows = B * (N_max + 1);
  const ArgmaxPlan p = argmax_plan(rows, V, dtype);
  return align_up(static_cast<size_t>(rows) * p.nseg * sizeof(uint64_t));
}

// Argument checks shared by build_tree and its variants; TSV_OK when the
// call may go ahead.
int check_build(const float* marginals, int B, int gamma, int V, int top_k, int n_budget,
                const tsv_cost_fitted* cost, const int* prefix_len, int N_max,
                const int* n_nodes, const int* parent, const int* token, const int* depth,
                const float* score, const unsigned* anc_bits) {
  if (!marginals || !n_nodes || !parent || !token || !depth || !score || !anc_bits)
    return TSV_EINVAL;
  if (B < 1 || gamma < 1 || V < 1 || top_k < 1 || N_max < 1) return TSV_EINVAL;
  if (top_k > V || n_budget < 0 || n_budget > N_max) return TSV_EINVAL;
  if (!build_sizes_ok(B, gamma, V, top_k, N_max)) return TSV_EUNSUPPORTED;
  if (cost && (!prefix_len || !cost_ok(cost))) return TSV_EINVAL;
  return TSV_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the scratch array on the device of stream s (the current
// device for the null stream), looked up once per device with that device
// current.
int scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return TSV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TSV_EUNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return TSV_EHIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return TSV_EHIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return TSV_EHIP;
      if (e != hipSuccess || !p) return TSV_EHIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return TSV_OK;
}

}  // namespace

extern "C" {

int tsv_set_tree_method(int method) {
  if (method < 0 || method > 2) return TSV_EINVAL;
  return g_tree_method.exchange(method, std::memory_order_relaxed);
}

const char* tsv_status_string(int code) {
  switch (code) {
    case TSV_OK: return "ok";
    case TSV_EINVAL: return "invalid argument";
    case TSV_EUNSUPPORTED: return "unsupported shape or dtype";
    case TSV_EWORKSPACE: return "workspace missing, misaligned or too small";
    case TSV_EHIP: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t tsv_workspace_size(int which, int B, int gamma, int V, int top_k,
                          int N_max, int L_cap, int Hq, int Hkv, int d_qk,
                          int d_v, int dtype) {
  switch (which) {
    case 0:
      if (!build_sizes_ok(B, gamma, V, top_k, N_max)) return 0;
      return build_layout(B, gamma, V, top_k).bytes;
    case 1: {
      if (!attn_sizes_ok(B, N_max, L_cap, Hq, Hkv, d_qk, d_v) || !dtype_ok(dtype)) return 0;
      AttnShape sh{B, N_max, L_cap, Hq, Hkv, d_qk, d_v, dtype};
      return attn_bytes_any(sh);
    }
    case 2:
      if (B < 1 || N_max < 1 || N_max > kMaxNodes || V < 1 || !dtype_ok(dtype)) return 0;
      return walk_bytes(B, N_max, V, dtype);
    case 3:
      return 0;
    case 4:
      if (!expand_sizes_ok(B, gamma, V, top_k, N_max)) return 0;
      return build_layout(B, expanded_rows(gamma, top_k), V, top_k).bytes;
    default:
      return 0;
  }
}

int build_tree(const float* marginals, int B, int gamma, int V, int top_k,
               int n_budget, const tsv_cost* cost, const int* prefix_len,
               int N_max, int* n_nodes, int* parent, int* token, int* depth,
               float* score, unsigned* anc_bits, void* ws, size_t ws_bytes,
               hipStream_t s) {
  tsv_cost_fitted fc;
  if (cost) fc = widen(*cost);
  const tsv_cost_fitted* c = cost ? &fc : nullptr;
  const int st = check_build(marginals, B, gamma, V, top_k, n_budget, c, prefix_len, N_max,
                             n_nodes, parent, token, depth, score, anc_bits);
  if (st != TSV_OK) return st;
  return launch_build(marginals, B, gamma, gamma, V, top_k, n_budget, c, prefix_len, N_max,
                      n_nodes, parent, token, depth, score, anc_bits, nullptr, nullptr, ws,
                      ws_bytes, s, false);
}

int build_tree_topk(const float* marginals, int B, int gamma, int V, int top_k,
                    int n_budget, const tsv_cost* cost, const int* prefix_len,
                    int N_max, int* n_nodes, int* parent, int* token, int* depth,
                    float* score, unsigned* anc_bits, int* topk_idx, float* topk_p,
                    void* ws, size_t ws_bytes, hipStream_t s) {
  if (!topk_idx || !topk_p) return TSV_EINVAL;
  tsv_cost_fitted fc;
  if (cost) fc = widen(*cost);
  const tsv_cost_fitted* c = cost ? &fc : nullptr;
  const int st = check_build(marginals, B, gamma, V, top_k, n_budget, c, prefix_len, N_max,
                             n_nodes, parent, token, depth, score, anc_bits);
  if (st != TSV_OK) return st;
  return launch_build(marginals, B, gamma, gamma, V, top_k, n_budget, c, prefix_len, N_max,
                      n_nodes, parent, token, depth, score, anc_bits, topk_idx, topk_p, ws,
                      ws_bytes, s, false);
}

int build_tree_noalloc(const float* marginals, int B, int gamma, int V, int top_k,
                       int n_budget, const tsv_cost* cost, const int* prefix_len,
                       int N_max, int* n_nodes, int* parent, int* token, int* depth,
                       float* score, unsigned* anc_bits, hipStream_t s) {
  tsv_cost_fitted fc;
  if (cost) fc = widen(*cost);
  const tsv_cost_fitted* c = cost ? &fc : nullptr;
  const int st = check_build(marginals, B, gamma, V, top_k, n_budget, c, prefix_len, N_max,
                             n_nodes, parent, token, depth, score, anc_bits);
  if (st != TSV_OK) return st;
  if (build_layout(B, gamma, V, top_k).bytes > kNoAllocScratchBytes) return TSV_EUNSUPPORTED;
  void* ws = nullptr;
  const int sa = scratch_address(s, &ws);
  if (sa != TSV_OK) return sa;
  return launch_build(marginals, B, gamma, gamma, V, top_k, n_budget, c, prefix_len, N_max,
                      n_nodes, parent, token, depth, score, anc_bits, nullptr, nullptr, ws,
                      kNoAllocScratchBytes, s, false);
}

int build_tree_fitted(const float* marginals, int B, int gamma, int V, int top_k,
                      int n_budget, const tsv_cost_fitted* cost, const int* prefix_len,
                      int N_max, int* n_nodes, int* parent, int* token, int* depth,
                      float* score, unsigned* anc_bits, void* ws, size_t ws_bytes,
                      hipStream_t s) {
  const int st = check_build(marginals, B, gamma, V, top_k, n_budget, cost, prefix_len, N_max,
                             n_nodes, parent, token, depth, score, anc_bits);
  if (st != TSV_OK) return st;
  return launch_build(marginals, B, gamma, gamma, V, top_k, n_budget, cost, prefix_len, N_max,
                      n_nodes, parent, token, depth, score, anc_bits, nullptr, nullptr, ws,
                      ws_bytes, s, false);
}

int build_tree_expand(const float* probs, int B, int steps, int V, int top_k,
                      int n_budget, const tsv_cost* cost, const int* prefix_len,
                      int N_max, int* n_nodes, int* parent, int* token, int* depth,
                      float* score, unsigned* anc_bits, int* topk_idx, float* topk_p,
                      void* ws, size_t ws_bytes, hipStream_t s) {
  if (!probs || !n_nodes || !parent || !token || !depth || !score || !anc_bits)
    return TSV_EINVAL;
  if ((topk_idx == nullptr) != (topk_p == nullptr)) return TSV_EINVAL;
  if (B < 1 || steps < 1 || V < 1 || top_k < 1 || N_max < 1) return TSV_EINVAL;
  if (top_k > V || n_budget < 0 || n_budget > N_max) return TSV_EINVAL;
  if (!expand_sizes_ok(B, steps, V, top_k, N_max)) return TSV_EUNSUPPORTED;
  tsv_cost_fitted fc;
  if (cost) fc = widen(*cost);
  const tsv_cost_fitted* c = cost ? &fc : nullptr;
  if (c && (!prefix_len || !cost_ok(c))) return TSV_EINVAL;
  return launch_build(probs, B, expanded_rows(steps, top_k), steps, V, top_k, n_budget, c,
                      prefix_len, N_max, n_nodes, parent, token, depth, score, anc_bits,
                      topk_idx, topk_p, ws, ws_bytes, s, true);
}

int select_global_budget(int* n_nodes, int* parent, int* token, int* depth, float* score,
                         unsigned* anc_bits, int B, int N_max, const double* sps, long sps_len,
                         hipStream_t s) {
  if (!n_nodes || !parent || !token || !depth || !score || !anc_bits || !sps) return TSV_EINVAL;
  if (B < 1 || N_max < 1 || N_max > kMaxNodes || sps_len < 1) return TSV_EINVAL;
  if (B > kMaxGlobalRequests || static_cast<long long>(B) * N_max > kMaxGlobalCandidates)
    return TSV_EUNSUPPORTED;
  GlobalBudgetArgs a;
  a.n_nodes = n_nodes;
  a.parent = parent;
  a.token = token;
  a.depth = depth;
  a.score = score;
  a.anc_bits = anc_bits;
  a.B = B;
  a.N_max = N_max;
  a.sps = sps;
  a.sps_len = sps_len;
  return launch_status(launch_global_budget(a, s));
}

int unfold_chains(const int* n_nodes, const int* parent, int B, int N_max, int gamma,
                  int* n_chains, int* chain_len, int* chain_nodes, hipStream_t s) {
  if (!n_nodes || !parent || !n_chains || !chain_len || !chain_nodes) return TSV_EINVAL;
  if (B < 1 || N_max < 1 || N_max > kMaxNodes || gamma < 1 || gamma > kMaxGamma) return TSV_EINVAL;
  ChainArgs a;
  a.n_nodes = n_nodes;
  a.parent = parent;
  a.B = B;
  a.N_max = N_max;
  a.gamma = gamma;
  a.n_chains = n_chains;
  a.chain_len = chain_len;
  a.chain_nodes = chain_nodes;
  return launch_status(launch_unfold_chains(a, s));
}

int compress_chains(const void* rows, int dtype, long row_stride, long E, int c,
                    const float* tail, const int* prefix_len, const int* n_chains,
                    const int* chain_len, const int* chain_nodes, int B, int N_max,
                    int gamma, float* entries, int* n_entries, hipStream_t s) {
  if (!rows || !tail || !prefix_len || !n_chains || !chain_len || !chain_nodes || !entries ||
      !n_entries)
    return TSV_EINVAL;
  if (!dtype_ok(dtype) || E < 1 || row_stride < E || c < 1 || c > kMaxBlock) return TSV_EINVAL;
  if (B < 1 || N_max < 1 || N_max > kMaxNodes || gamma < 1 || gamma > kMaxGamma) return TSV_EINVAL;
  if (E > kMaxCompressCols || static_cast<long long>(B) * N_max > 0x7fffffffLL) return TSV_EUNSUPPORTED;
  CompressArgs a;
  a.rows = rows;
  a.row_stride = row_stride;
  a.E = E;
  a.c = c;
  a.tail = tail;
  a.prefix_len = prefix_len;
  a.n_chains = n_chains;
  a.chain_len = chain_len;
  a.chain_nodes = chain_nodes;
  a.B = B;
  a.N_max = N_max;
  a.gamma = gamma;
  a.entries = entries;
  a.n_entries = n_entries;
  // adjacent columns per thread: whole 4-column groups, rows and entries aligned
  const int es = esize(dtype);
  const bool vec = E % 4 == 0 && (row_stride * es) % (4 * es) == 0 && aligned_to(rows, 4 * es) &&
                   aligned_to(tail, 16) && aligned_to(entries, 16);
  return launch_status(launch_compress_chains(a, dtype, vec, s));
}

int refresh_compressed(const void* rows, int dtype, long row_stride, long E, int c,
                       const int* prefix_len, const int* accept_len, const int* accept_nodes,
                       const int* n_chains, const int* chain_len, const int* chain_nodes,
                       const float* entries, int B, int N_max, int gamma, float* comp,
                       int Lc_cap, float* tail, int* status, hipStream_t s) {
  if (!rows || !prefix_len || !accept_len || !accept_nodes || !n_chains || !chain_len ||
      !chain_nodes || !entries || !comp || !tail || !status)
    return TSV_EINVAL;
  if (!dtype_ok(dtype) || E < 1 || row_stride < E || c < 1 || c > kMaxBlock || Lc_cap < 0) return TSV_EINVAL;
  if (B < 1 || N_max < 1 || N_max > kMaxNodes || gamma < 1 || gamma > kMaxGamma) return TSV_EINVAL;
  if (E > kMaxCompressCols) return TSV_EUNSUPPORTED;
  RefreshArgs a;
  a.rows = rows;
  a.row_stride = row_stride;
  a.E = E;
  a.c = c;
  a.prefix_len = prefix_len;
  a.accept_len = accept_len;
  a.accept_nodes = accept_nodes;
  a.n_chains = n_chains;
  a.chain_len = chain_len;
  a.chain_nodes = chain_nodes;
  a.entries = entries;
  a.B = B;
  a.N_max = N_max;
  a.gamma = gamma;
  a.comp = comp;
  a.Lc_cap = Lc_cap;
  a.tail = tail;
  a.status = status;
  return launch_status(launch_refresh_compressed(a, dtype, s));
}

int tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const void* k_tree, const void* v_tree, long kv_row_stride,
                     const int* prefix_len, const int* n_nodes,
                     const unsigned* anc_bits, int B, int N_max, int L_cap,
                     int Hq, int Hkv, int d_qk, int d_v, int dtype,
                     float sm_scale, void* out, float* lse, void* ws,
                     size_t ws_bytes, hipStream_t s) {
  if (!q || !k_cache || !v_cache || !k_tree || !v_tree || !prefix_len || !n_nodes ||
      !anc_bits || !out)
    return TSV_EINVAL;
  if (!dtype_ok(dtype) || !isfinite(sm_scale)) return TSV_EINVAL;
  if (B < 1 || N_max < 1 || L_cap < 0 || Hq < 1 || Hkv < 1 || d_qk < 1 || d_v < 1)
    return TSV_EINVAL;
  if (Hq % Hkv != 0) return TSV_EINVAL;
  const long widest = static_cast<long>(Hkv) * (d_qk > d_v ? d_qk : d_v);
  if (kv_row_stride < widest) return TSV_EINVAL;
  if (!attn_sizes_ok(B, N_max, L_cap, Hq, Hkv, d_qk, d_v)) return TSV_EUNSUPPORTED;
  const int es = esize(dtype);
  const bool vec = aligned_to(q, 16) && aligned_to(k_cache, 16) && aligned_to(v_cache, 16) &&
                   aligned_to(k_tree, 16) && aligned_to(v_tree, 16) && aligned_to(out, 16) &&
                   (kv_row_stride * es) % 16 == 0;
  AttnShape sh{B, N_max, L_cap, Hq, Hkv, d_qk, d_v, dtype};
  // a latent cache: one KV head whose value is the start of the key row
  const bool shared = Hkv == 1 && v_cache == k_cache && v_tree == k_tree;
  const AttnPlan P = attn_plan(sh, vec, shared);
  if (!ws || ws_bytes < P.bytes || !aligned_to(ws, kAlign)) return TSV_EWORKSPACE;
  char* w = static_cast<char*>(ws);
  AttnArgs a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.kt = k_tree;
  a.vt = v_tree;
  a.stride = kv_row_stride;
  a.prefix_len = prefix_len;
  a.n_nodes = n_nodes;
  a.anc = anc_bits;
  a.B = B;
  a.N_max = N_max;
  a.L_cap = L_cap;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.d_qk = d_qk;
  a.d_v = d_v;
  a.W = (N_max + 31) / 32;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  a.info = reinterpret_cast<int*>(w + P.off_info);
  a.desc = reinterpret_cast<int4*>(w + P.off_desc);
  a.part_ml = reinterpret_cast<float*>(w + P.off_ml);
  a.part_acc = reinterpret_cast<float*>(w + P.off_acc);
  a.RB = P.RB;
  a.KT = P.KT;
  a.items_max = P.items_max;
  a.target_items = P.target_items;
  a.min_chunk = P.min_chunk;
  a.counters = reinterpret_cast<int*>(w + P.off_cnt);
  a.chunk = P.chunk;
  a.S = P.S;
  a.units = P.units;
  a.rbs = P.rbs;
  return launch_status(launch_attention(a, P.path, dtype, s));
}

int accept_walk(const void* target_logits, int dtype, int B, int N_max, int V,
                int gamma, const int* n_nodes, const int* parent,
                const int* token, int* accept_len, int* accept_nodes,
                int* out_tokens, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!target_logits || !n_nodes || !parent || !token || !accept_len || !accept_nodes ||
      !out_tokens)
    return TSV_EINVAL;
  if (!dtype_ok(dtype) || B < 1 || N_max < 1 || V < 1 || gamma < 1) return TSV_EINVAL;
  if (N_max > kMaxNodes || gamma > kMaxGamma) return TSV_EUNSUPPORTED;
  if (static_cast<long long>(B) * (N_max + 1) > (1LL << 26)) return TSV_EUNSUPPORTED;
  const int rows = B * (N_max + 1);
  ArgmaxPlan p = argmax_plan(rows, V, dtype);
  if (!aligned_to(target_logits, 16)) p.vec = false;
  if (!ws || ws_bytes < walk_bytes(B, N_max, V, dtype) || !aligned_to(ws, kAlign))
    return TSV_EWORKSPACE;
  return launch_status(launch_accept_walk(target_logits, dtype, B, N_max, V, gamma, n_nodes,
                                          parent, token, accept_len, accept_nodes, out_tokens,
                                          static_cast<uint64_t*>(ws), p,
                                          s));
}

int commit_path(void* k_cache, void* v_cache, int* prefix_len,
                const void* k_tree, const void* v_tree, long kv_row_stride,
                const int* accept_len, const int* accept_nodes, int B,
                int N_max, int L_cap, int Hkv, int d_k, int d_v, int gamma,
                int dtype, int* status, hipStream_t s) {
  if (!k_cache || !prefix_len || !k_tree || !accept_len || !accept_nodes || !status)
    return TSV_EINVAL;
  if ((v_cache == nullptr) != (v_tree == nullptr)) return TSV_EINVAL;
  if (!dtype_ok(dtype) || B < 1 || N_max < 1 || L_cap < 0 || Hkv < 1 || d_k < 1 || gamma < 1)
    return TSV_EINVAL;
  if (v_cache && d_v < 1) return TSV_EINVAL;
  if (gamma > kMaxGamma) return TSV_EUNSUPPORTED;
  const long vk = static_cast<long>(Hkv) * d_k;
  const long vv = v_cache ? static_cast<long>(Hkv) * d_v : 0;
  if (kv_row_stride < vk || kv_row_stride < vv) return TSV_EINVAL;
  const int es = esize(dtype);
  return launch_status(launch_commit(k_cache, v_cache, prefix_len, k_tree, v_tree,
                                     static_cast<size_t>(kv_row_stride) * es, accept_len,
                                     accept_nodes, B, N_max, L_cap, static_cast<size_t>(vk) * es,
                                     static_cast<size_t>(vv) * es, gamma, status,
                                     s));
}

}  // extern "C"
