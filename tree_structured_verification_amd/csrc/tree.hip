// build_tree, stage 2: greedy best-first tree with the throughput stop rule.
//
// [caddtree] Methodology, items 2-4: for a fixed node count the best tree is
// the greedy best-first one (highest prefix probability first); the round's
// budget is found by adding nodes in that order while the throughput
// (1 + Phi_n) / (C_d + C_v(n; l)) still rises.
//
// One wavefront per request.  The frontier holds, for every popped node, its
// best unpopped child and its next unpopped sibling -- enough because a
// node's children are ranked by probability, so a child never beats its
// better-ranked sibling or its parent.  Each frontier entry is one 64-bit key
// that orders exactly like the selection order
//   (score desc, depth asc, parent's position asc, rank asc),
// so a pop is a wave-wide max over at most 5 keys per lane.  Scores are fp32
// products (never fused); the stop rule is evaluated in fp64 with explicit
// round-to-nearest operations in a fixed order.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

constexpr int kFrontierSlots = 5;  // 64 * 5 >= 1 + 2 * 128 entries
constexpr int kMaxTopkTable = 4096;

__device__ __forceinline__ uint64_t frontier_key(float score, int depth, int parent, int rank) {
  return (static_cast<uint64_t>(ord_f32(score)) << 21) |
         (static_cast<uint64_t>(63 - (depth - 1)) << 15) |
         (static_cast<uint64_t>(255 - (parent + 1)) << 7) |
         static_cast<uint64_t>(127 - rank);
}

__device__ __forceinline__ double round_cost(const tsv_cost& c, int n, double l) {
  double m = static_cast<double>(n);
  double v = __dadd_rn(c.a, __dmul_rn(c.b, m));
  v = __dadd_rn(v, __dmul_rn(c.c, __dmul_rn(m, m)));
  v = __dadd_rn(v, __dmul_rn(__dmul_rn(c.e, l), m));
  return __dadd_rn(c.c_d, v);
}

__global__ __launch_bounds__(64) void best_first_kernel(TreeArgs a) {
  __shared__ float s_p[kMaxTopkTable];
  __shared__ int s_i[kMaxTopkTable];
  __shared__ int n_par[128], n_tok[128], n_dep[128];
  __shared__ float n_sc[128];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int gk = a.gamma * a.k;
  const size_t tbase = static_cast<size_t>(b) * gk;
  for (int e = lane; e < gk; e += 64) {
    s_p[e] = a.tk_p[tbase + e];
    s_i[e] = a.tk_idx[tbase + e];
  }
  __syncthreads();

  uint64_t fr[kFrontierSlots];
#pragma unroll
  for (int s = 0; s < kFrontierSlots; ++s) fr[s] = 0;
  int cnt = 0;
  auto push = [&](uint64_t key) {
    const int L = cnt & 63, S = cnt >> 6;
#pragma unroll
    for (int s = 0; s < kFrontierSlots; ++s)
      if (s == S && lane == L) fr[s] = key;
    ++cnt;
  };

  // the root's best child: score 1 * q, depth 1, rank 0
  push(frontier_key(__fmul_rn(1.0f, s_p[0]), 1, -1, 0));

  const double l = a.adaptive ? static_cast<double>(a.prefix_len[b]) : 0.0;
  double phi = 0.0;
  double theta = a.adaptive ? __ddiv_rn(1.0, round_cost(a.cost, 0, l)) : 0.0;

  int m = 0;
  while (m < a.cap) {
    uint64_t best = 0;
#pragma unroll
    for (int s = 0; s < kFrontierSlots; ++s) best = umax64(best, fr[s]);
    best = wave_max_u64(best);
    if (best == 0) break;  // every candidate taken
    const int rank = 127 - static_cast<int>(best & 127);
    const int par = 255 - static_cast<int>((best >> 7) & 255) - 1;
    const int dep = 63 - static_cast<int>((best >> 15) & 63) + 1;
    const float ps = par < 0 ? 1.0f : n_sc[par];
    const float sc = __fmul_rn(ps, s_p[(dep - 1) * a.k + rank]);
    if (a.adaptive) {
      const double phi2 = __dadd_rn(phi, static_cast<double>(sc));
      const double th2 = __ddiv_rn(__dadd_rn(1.0, phi2), round_cost(a.cost, m + 1, l));
      if (!(th2 > theta)) break;  // marginal gain not positive
      phi = phi2;
      theta = th2;
    }
    if (lane == 0) {
      n_par[m] = par;
      n_tok[m] = s_i[(dep - 1) * a.k + rank];
      n_dep[m] = dep;
      n_sc[m] = sc;
    }
#pragma unroll
    for (int s = 0; s < kFrontierSlots; ++s)
      if (fr[s] == best) fr[s] = 0;
    if (rank + 1 < a.k)
      push(frontier_key(__fmul_rn(ps, s_p[(dep - 1) * a.k + rank + 1]), dep, par, rank + 1));
    if (dep < a.gamma)
      push(frontier_key(__fmul_rn(sc, s_p[dep * a.k]), dep + 1, m, 0));
    ++m;
    wave_lds_sync();  // n_sc[m-1] is read by every lane in later pops
  }
  const int n = m;
  __syncthreads();

  const int W = (a.N_max + 31) >> 5;
  const size_t nb = static_cast<size_t>(b) * a.N_max;
  for (int i = lane; i < a.N_max; i += 64) {
    const bool v = i < n;
    a.parent[nb + i] = v ? n_par[i] : -1;
    a.token[nb + i] = v ? n_tok[i] : -1;
    a.depth[nb + i] = v ? n_dep[i] : -1;
    a.score[nb + i] = v ? n_sc[i] : 0.0f;
    uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
    if (v) {
      int j = i;
      while (j >= 0) {
        const uint32_t bit = 1u << (j & 31);
        const int wi = j >> 5;
        if (wi == 0) w0 |= bit;
        else if (wi == 1) w1 |= bit;
        else if (wi == 2) w2 |= bit;
        else w3 |= bit;
        j = n_par[j];
      }
    }
    unsigned* dst = a.anc_bits + (nb + i) * W;
    dst[0] = w0;
    if (W > 1) dst[1] = w1;
    if (W > 2) dst[2] = w2;
    if (W > 3) dst[3] = w3;
  }
  if (lane == 0) a.n_nodes[b] = n;
}

}  // namespace

hipError_t launch_best_first(const TreeArgs& a, hipStream_t s) {
  best_first_kernel<<<dim3(a.B), dim3(64), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tsv
