// build_tree, stage 2: greedy best-first tree with the throughput stop rule.
//
// [caddtree] Methodology, items 2-4: for a fixed node count the best tree is
// the greedy best-first one (highest prefix probability first); the round's
// budget is found by adding nodes in that order while the throughput
// (1 + Phi_n) / (C_d + C_v(n; l)) still rises.
//
// Two sources of children.  Per position: a node at depth d branches on the
// top-k list of drafter position d (one list per position, shared by every
// node of that depth).  Per node ([review] "How it works", steps 1-2): every
// node of depth < s branches on the top-k of its own distribution; the lists
// are in level order of the complete k-ary expansion, so the child of rank r
// of the node whose token came from list i has list k*i + 1 + r (the root's
// list is 0).  Each frontier entry then carries the list its token came from.
//
// One wavefront per request.  The frontier holds, for every popped node, its
// best unpopped child and its next unpopped sibling -- enough because a
// node's children are ranked by probability, so a child never beats its
// better-ranked sibling or its parent.  Each frontier entry is one 64-bit key
// that orders exactly like the selection order
//   (score desc, depth asc, parent's position asc, rank asc),
// and the frontier is kept sorted by it across the lanes, so a pop reads
// lane 0.  Scores are fp32
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

// the exact score a frontier key was built from (inverse of ord_f32)
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 21);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ double round_cost(const tsv_cost_fitted& c, int n, double l) {
  double m = static_cast<double>(n);
  double v = __dadd_rn(c.a, __dmul_rn(c.b, m));
  v = __dadd_rn(v, __dmul_rn(c.c, __dmul_rn(m, m)));
  v = __dadd_rn(v, __dmul_rn(__dmul_rn(c.e, l), m));
  v = __dadd_rn(v, __dmul_rn(c.f, l));
  return __dadd_rn(c.c_d, v);
}

// The frontier is kept sorted (descending key) across the lanes: position
// P = 64 * s + lane of slot s.  A pop takes position 0 and shifts the rest
// down one place; an insert counts the keys above the new one (one ballot
// per slot) and shifts the positions from there up one place.  The shifts
// are whole-wavefront DPP moves (wave_shl / wave_shr), the boundary lane
// taking the neighbouring slot's value, so a round costs no wave-wide
// reduction.  Capacity 64 * SL >= cap: an entry pushed past it would need
// more pops than remain to reach the front, so dropping it changes nothing.
template <int CTRL>
__device__ __forceinline__ uint32_t wave_shift_u32(uint32_t v, uint32_t fill) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(fill), static_cast<int>(v),
                                                           CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t wave_shift_u64(uint64_t v, uint64_t fill) {
  const uint32_t lo = wave_shift_u32<CTRL>(static_cast<uint32_t>(v), static_cast<uint32_t>(fill));
  const uint32_t hi = wave_shift_u32<CTRL>(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(fill >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
constexpr int kShl1 = 0x130;  // lane l takes lane l + 1 (lane 63 takes the fill)
constexpr int kShr1 = 0x138;  // lane l takes lane l - 1 (lane 0 takes the fill)

template <int SL, bool PER_NODE, bool ADAPTIVE>
__global__ __launch_bounds__(64) void best_first_kernel(TreeArgs a) {
  __shared__ float s_p[kMaxTopkTable];
  __shared__ int s_i[kMaxTopkTable];
  __shared__ int n_par[128], n_dep[128], n_rank[128], n_row[128];
  __shared__ float n_sc[128];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int gk = a.rows * a.k;
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
  // the best child of a node at depth d has probability p[d][0]: lane d keeps it
  const float q_first = (!PER_NODE && lane < a.gamma) ? a.tk_p[tbase + static_cast<size_t>(lane) * a.k] : 0.f;
  __syncthreads();

  // entry = order key (0 = empty; it holds the node's exact score) and (per
  // node) the list its token comes from; the parent's score is read from
  // the popped nodes' record when the entry is popped
  uint64_t fk[SL];
  int frw[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    fk[s] = 0;
    frw[s] = 0;
  }
  auto insert = [&](uint64_t x, int xr) {
    int pos = 0;
#pragma unroll
    for (int s = 0; s < SL; ++s) pos += __popcll(__ballot(fk[s] > x));
    uint64_t ck = 0;
    int cr = 0;
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const uint64_t k63 = readlane_u64(fk[s], 63);
      const uint64_t shk = wave_shift_u64<kShr1>(fk[s], ck);
      const int P = s * 64 + lane;
      const bool keep = P < pos, here = P == pos;
      fk[s] = keep ? fk[s] : (here ? x : shk);
      ck = k63;
      if constexpr (PER_NODE) {
        const int r63 = __builtin_amdgcn_readlane(frw[s], 63);
        const int shr = static_cast<int>(wave_shift_u32<kShr1>(static_cast<uint32_t>(frw[s]), static_cast<uint32_t>(cr)));
        frw[s] = keep ? frw[s] : (here ? xr : shr);
        cr = r63;
      }
    }
  };
  auto drop_front = [&]() {
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const uint64_t nk = s + 1 < SL ? readlane_u64(fk[s + 1 < SL ? s + 1 : s], 0) : 0;
      fk[s] = wave_shift_u64<kShl1>(fk[s], nk);
      if constexpr (PER_NODE) {
        const int nr = s + 1 < SL ? __builtin_amdgcn_readlane(frw[s + 1 < SL ? s + 1 : s], 0) : 0;
        frw[s] = static_cast<int>(wave_shift_u32<kShl1>(static_cast<uint32_t>(frw[s]), static_cast<uint32_t>(nr)));
      }
    }
  };

  // the root's best child: score 1 * q, depth 1, rank 0
  {
    const float r0 = __fmul_rn(1.0f, s_p[0]);
    insert(frontier_key(r0, 1, -1, 0), 0);
  }

  const double l = ADAPTIVE ? static_cast<double>(a.prefix_len[b]) : 0.0;
  double phi = 0.0;
  double theta = ADAPTIVE ? __ddiv_rn(1.0, round_cost(a.cost, 0, l)) : 0.0;

  // Popped nodes' records stay in registers during the pops (node m at lane
  // m % 64 of slot m / 64; a parent's score is one readlane away) and go to
  // LDS once afterwards, so no pop waits on an LDS store or load of them.
  float r_sc[SL];
  int r_par[SL], r_dep[SL], r_rank[SL], r_row[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    r_sc[s] = 0.f;
    r_par[s] = r_dep[s] = r_rank[s] = r_row[s] = 0;
  }

  int m = 0;
  while (m < a.cap) {
    const uint64_t hk = readlane_u64(fk[0], 0);
    if (hk == 0) break;  // every candidate taken
    const uint32_t wl = static_cast<uint32_t>(hk);
    const int rank = 127 - static_cast<int>(wl & 127);
    const int par = 255 - static_cast<int>((wl >> 7) & 255) - 1;
    const int dep = 63 - static_cast<int>((wl >> 15) & 63) + 1;
    const float sc = key_score(hk);
    // list of the popped node's token (shared with its siblings) and the
    // list its children come from
    const int row = PER_NODE ? __builtin_amdgcn_readlane(frw[0], 0) : dep - 1;
    const int kid_row = PER_NODE ? a.k * row + 1 + rank : dep;
    // the sibling's table read is issued first and lands while the child
    // (built from registers alone, per position) is inserted
    const float q_sib = rank + 1 < a.k ? s_p[row * a.k + rank + 1] : 0.f;
    float q_kid = 0.f;
    if (dep < a.gamma) q_kid = PER_NODE ? s_p[kid_row * a.k] : readlane_f32(q_first, dep);
    // the parent was popped earlier: its score from the registers
    const float ps0 = readlane_f32(r_sc[0], par & 63);
    const float ps1 = readlane_f32(r_sc[SL - 1], par & 63);
    const float ps = par < 0 ? 1.0f : (par < 64 ? ps0 : ps1);
    // The stop rule is evaluated here but decided after this pop's inserts
    // (a stop discards them and the record below), so that its fp64
    // arithmetic overlaps the inserts instead of preceding them.
    double phi2 = 0.0, th2 = 0.0;
    if constexpr (ADAPTIVE) {
      phi2 = __dadd_rn(phi, static_cast<double>(sc));
      th2 = __ddiv_rn(__dadd_rn(1.0, phi2), round_cost(a.cost, m + 1, l));
    }
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      if (s == (m >> 6)) {
        const bool me = lane == (m & 63);
        r_sc[s] = me ? sc : r_sc[s];
        r_par[s] = me ? par : r_par[s];
        r_dep[s] = me ? dep : r_dep[s];
        r_rank[s] = me ? rank : r_rank[s];
        if constexpr (PER_NODE) r_row[s] = me ? row : r_row[s];
      }
    }
    drop_front();
    if (dep < a.gamma) {
      const float v = __fmul_rn(sc, q_kid);
      insert(frontier_key(v, dep + 1, m, 0), kid_row);
    }
    if (rank + 1 < a.k) {
      const float v = __fmul_rn(ps, q_sib);
      insert(frontier_key(v, dep, par, rank + 1), row);
    }
    if constexpr (ADAPTIVE) {
      if (!(th2 > theta)) break;  // marginal gain not positive
      phi = phi2;
      theta = th2;
    }
    ++m;
  }
  const int n = m;
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int i = s * 64 + lane;
    if (i < n) {
      n_par[i] = r_par[s];
      n_dep[i] = r_dep[s];
      n_rank[i] = r_rank[s];
      if constexpr (PER_NODE) n_row[i] = r_row[s];
      n_sc[i] = r_sc[s];
    }
  }
  __syncthreads();

  const int W = (a.N_max + 31) >> 5;
  const size_t nb = static_cast<size_t>(b) * a.N_max;
  for (int i = lane; i < a.N_max; i += 64) {
    const bool v = i < n;
    a.parent[nb + i] = v ? n_par[i] : -1;
    const int trow = v ? (PER_NODE ? n_row[i] : n_dep[i] - 1) : 0;
    a.token[nb + i] = v ? s_i[trow * a.k + n_rank[i]] : -1;
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
  // sorted frontier of 64 or 128 places (at least cap); the stop rule only
  // in the adaptive instances
  const dim3 g(a.B), blk(64);
#define TSV_BF(SL, PN)                                                   \
  if (a.adaptive) best_first_kernel<SL, PN, true><<<g, blk, 0, s>>>(a);  \
  else best_first_kernel<SL, PN, false><<<g, blk, 0, s>>>(a);
  if (a.per_node) {
    if (a.cap <= 64) {
      TSV_BF(1, true)
    } else {
      TSV_BF(2, true)
    }
  } else {
    if (a.cap <= 64) {
      TSV_BF(1, false)
    } else {
      TSV_BF(2, false)
    }
  }
#undef TSV_BF
  return hipGetLastError();
}

}  // namespace tsv
