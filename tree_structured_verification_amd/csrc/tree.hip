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

// SLOTS frontier entries per lane; the frontier never holds more than
// 1 + 2 * cap entries, so 64 * SLOTS > 2 * cap suffices.
template <int SLOTS>
__global__ __launch_bounds__(64) void best_first_kernel(TreeArgs a) {
  __shared__ float s_p[kMaxTopkTable];
  __shared__ int s_i[kMaxTopkTable];
  __shared__ int n_par[128], n_dep[128], n_rank[128];
  __shared__ float n_sc[128];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int gk = a.gamma * a.k;
  const size_t tbase = static_cast<size_t>(b) * gk;
  // the table in batches of 8 loads per lane, all in flight together
  for (int e0 = 0; e0 < gk; e0 += 8 * 64) {
    float p[8];
    int ix[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * 64 + lane;
      p[u] = e < gk ? a.tk_p[tbase + e] : 0.f;
      ix[u] = e < gk ? a.tk_idx[tbase + e] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * 64 + lane;
      if (e < gk) {
        s_p[e] = p[u];
        s_i[e] = ix[u];
      }
    }
  }
  __syncthreads();

  // Frontier slot = 64-bit order key split in (hi = ordered score bits,
  // lo = depth/parent/rank fields, 0 = empty) plus the entry's exact score
  // and its parent's score, so a pop reads everything from the winner lane.
  // Updates are selects (no lane-dependent branches).
  uint32_t fhi[SLOTS], flo[SLOTS];
  float fsc[SLOTS], fps[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    fhi[s] = 0;
    flo[s] = 0;
    fsc[s] = 0.f;
    fps[s] = 0.f;
  }
  int cnt = 0;
  auto push = [&](float score, float parent_score, int depth, int parent, int rank) {
    const uint64_t key = frontier_key(score, depth, parent, rank);
    const uint32_t kh = static_cast<uint32_t>(key >> 32), kl = static_cast<uint32_t>(key);
    const bool mine = lane == (cnt & 63);
    const int S = cnt >> 6;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const bool w = mine && s == S;
      fhi[s] = w ? kh : fhi[s];
      flo[s] = w ? kl : flo[s];
      fsc[s] = w ? score : fsc[s];
      fps[s] = w ? parent_score : fps[s];
    }
    ++cnt;
  };

  // the root's best child: score 1 * q, depth 1, rank 0
  push(__fmul_rn(1.0f, s_p[0]), 1.0f, 1, -1, 0);

  const double l = a.adaptive ? static_cast<double>(a.prefix_len[b]) : 0.0;
  double phi = 0.0;
  double theta = a.adaptive ? __ddiv_rn(1.0, round_cost(a.cost, 0, l)) : 0.0;

  int m = 0;
  while (m < a.cap) {
    // best slot of this lane (hi, then lo)
    uint32_t bh = fhi[0], bl = flo[0];
    int bs = 0;
    float bsc = fsc[0], bps = fps[0];
#pragma unroll
    for (int s = 1; s < SLOTS; ++s) {
      const bool better = fhi[s] > bh || (fhi[s] == bh && flo[s] > bl);
      bh = better ? fhi[s] : bh;
      bl = better ? flo[s] : bl;
      bs = better ? s : bs;
      bsc = better ? fsc[s] : bsc;
      bps = better ? fps[s] : bps;
    }
    const uint32_t wh = wave_max_u32(bh);
    if (wh == 0) break;  // every candidate taken
    uint64_t cand = __ballot(bh == wh);
    uint32_t wl;
    if (__popcll(cand) == 1) {
      wl = __builtin_amdgcn_readlane(bl, __ffsll(static_cast<long long>(cand)) - 1);
    } else {  // equal scores: settle by depth, parent position, rank
      wl = wave_max_u32(bh == wh ? bl : 0u);
      cand = __ballot(bh == wh && bl == wl);
    }
    const int wlane = __ffsll(static_cast<long long>(cand)) - 1;
    const int wslot = __builtin_amdgcn_readlane(bs, wlane);
    const int rank = 127 - static_cast<int>(wl & 127);
    const int par = 255 - static_cast<int>((wl >> 7) & 255) - 1;
    const int dep = 63 - static_cast<int>((wl >> 15) & 63) + 1;
    const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bsc), wlane));
    const float ps = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bps), wlane));
    if (a.adaptive) {
      const double phi2 = __dadd_rn(phi, static_cast<double>(sc));
      const double th2 = __ddiv_rn(__dadd_rn(1.0, phi2), round_cost(a.cost, m + 1, l));
      if (!(th2 > theta)) break;  // marginal gain not positive
      phi = phi2;
      theta = th2;
    }
    if (lane == 0) {
      n_par[m] = par;
      n_dep[m] = dep;
      n_rank[m] = rank;
      n_sc[m] = sc;
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const bool w = lane == wlane && s == wslot;
      fhi[s] = w ? 0u : fhi[s];
      flo[s] = w ? 0u : flo[s];
    }
    const float q_sib = rank + 1 < a.k ? s_p[(dep - 1) * a.k + rank + 1] : 0.f;
    const float q_kid = dep < a.gamma ? s_p[dep * a.k] : 0.f;
    if (rank + 1 < a.k) push(__fmul_rn(ps, q_sib), ps, dep, par, rank + 1);
    if (dep < a.gamma) push(__fmul_rn(sc, q_kid), sc, dep + 1, m, 0);
    ++m;
  }
  const int n = m;
  __syncthreads();

  const int W = (a.N_max + 31) >> 5;
  const size_t nb = static_cast<size_t>(b) * a.N_max;
  for (int i = lane; i < a.N_max; i += 64) {
    const bool v = i < n;
    a.parent[nb + i] = v ? n_par[i] : -1;
    a.token[nb + i] = v ? s_i[(n_dep[i] - 1) * a.k + n_rank[i]] : -1;
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
  // frontier entries: at most 1 + 2 * cap (each pop adds two, removes one)
  const int need = 1 + 2 * a.cap;
  if (need <= 64)
    best_first_kernel<1><<<dim3(a.B), dim3(64), 0, s>>>(a);
  else if (need <= 128)
    best_first_kernel<2><<<dim3(a.B), dim3(64), 0, s>>>(a);
  else if (need <= 192)
    best_first_kernel<3><<<dim3(a.B), dim3(64), 0, s>>>(a);
  else
    best_first_kernel<5><<<dim3(a.B), dim3(64), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tsv
