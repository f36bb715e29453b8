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
// Serial pops (one wavefront): the frontier holds, for every popped node, its
// best unpopped child and its next unpopped sibling -- enough because a
// node's children are ranked by probability, so a child never beats its
// better-ranked sibling or its parent.  Each frontier entry is one 64-bit key
// that orders exactly like the selection order
//   (score desc, depth asc, parent's position asc, rank asc),
// and the frontier is kept sorted by it across the lanes, so a pop reads
// lane 0.  With per-position lists a second wavefront of the same workgroup
// builds the same tree level by level (far fewer dependent steps when few
// nodes below depth 1 are selected) and the first of the two to finish
// writes it.  Scores are fp32 products (never fused); the stop rule is
// evaluated in fp64 with explicit round-to-nearest operations in a fixed
// order.

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

// ---- the table of top-k lists, staged in LDS ------------------------------
// All loads of a batch are in flight together: U per thread (8 when that
// covers the table, else 16, fewer masked-off instructions for small tables).
template <int U>
__device__ __forceinline__ void load_table_batch(const TreeArgs& a, size_t tbase, int gk, int e0, int tid, int nth,
                                                 float* s_p, int* s_i) {
  float p[U];
  int ix[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = e0 + u * nth + tid;
    p[u] = e < gk ? a.tk_p[tbase + e] : 0.f;
    ix[u] = e < gk ? a.tk_idx[tbase + e] : 0;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = e0 + u * nth + tid;
    if (e < gk) {
      s_p[e] = p[u];
      s_i[e] = ix[u];
    }
  }
}
__device__ __forceinline__ void load_table(const TreeArgs& a, int b, int tid, int nth, float* s_p, int* s_i) {
  const int gk = a.rows * a.k;
  const size_t tbase = static_cast<size_t>(b) * gk;
  if (gk <= 8 * nth) {
    load_table_batch<8>(a, tbase, gk, 0, tid, nth, s_p, s_i);
  } else {
    for (int e0 = 0; e0 < gk; e0 += 16 * nth) load_table_batch<16>(a, tbase, gk, e0, tid, nth, s_p, s_i);
  }
}

// Two wavefronts of a workgroup may compute the same tree by different
// methods; the first to finish claims the result (an LDS word, 0 = open),
// the other sees the claim and stops.  A loop reads the word at the top of
// an iteration (claim_load) and tests it at the bottom (claim_seen), so the
// read's latency hides behind the iteration's work.
__device__ __forceinline__ int claim_load(int* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ bool claim_seen(int v) { return __builtin_amdgcn_readfirstlane(v) != 0; }
__device__ __forceinline__ bool claim(int* w, int id) {
  int won = 0;
  if (__lane_id() == 0) {
    int expected = 0;
    won = __hip_atomic_compare_exchange_strong(w, &expected, id, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP)
              ? 1
              : 0;
  }
  return __builtin_amdgcn_readfirstlane(won) != 0;
}

// Records of the selected nodes, in selection order (LDS).
struct NodeRecords {
  int* par;
  int* dep;
  int* rank;
  int* row;
  float* sc;
};

// ---- serial best-first pops ---------------------------------------------
// The frontier holds, for every popped node, its best unpopped child and its
// next unpopped sibling (children are ranked by probability, so a child
// never beats its better-ranked sibling or its parent), sorted across the
// lanes by a 64-bit key that orders exactly like the selection order.  One
// pop per node.  Returns the node count, or -1 when another wavefront has
// claimed the result first (RACE).
template <int SL, bool PER_NODE, bool ADAPTIVE, bool RACE>
__device__ __forceinline__ int serial_select(const TreeArgs& a, int b, int lane, const float* s_p, float q_first,
                                             int* winner, float (&r_sc)[SL], int (&r_par)[SL], int (&r_dep)[SL],
                                             int (&r_rank)[SL], int (&r_row)[SL]) {
  // entry = order key (0 = empty; it holds the node's exact score) and (per
  // node) the list its token comes from; the parent's score is read from
  // the popped nodes' records when the entry is popped
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
  // m % 64 of slot m / 64; a parent's score is one readlane away).
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    r_sc[s] = 0.f;
    r_par[s] = r_dep[s] = r_rank[s] = r_row[s] = 0;
  }

  int m = 0;
  while (m < a.cap) {
    // the other wavefront's claim, read now and tested after this pop
    const int other = RACE ? claim_load(winner) : 0;
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
    if (RACE && claim_seen(other)) return -1;
  }
  return m;
}

template <int SL, bool PER_NODE>
__device__ __forceinline__ void store_serial_records(int n, int lane, const float (&r_sc)[SL], const int (&r_par)[SL],
                                                     const int (&r_dep)[SL], const int (&r_rank)[SL],
                                                     const int (&r_row)[SL], const NodeRecords& o) {
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int i = s * 64 + lane;
    if (i < n) {
      o.par[i] = r_par[s];
      o.dep[i] = r_dep[s];
      o.rank[i] = r_rank[s];
      if constexpr (PER_NODE) o.row[i] = r_row[s];
      o.sc[i] = r_sc[s];
    }
  }
}

// ---- level-by-level selection (per-position lists) ------------------------
// The first c nodes of the selection order among depths <= d are contained in
// the first c among depths <= d-1 plus the children of its depth-(d-1)
// members (any prefix of the order is ancestor-closed), and depth 1 is the
// first list itself.  So the kept list K (at most cap nodes, in selection
// order) is built level by level: the members' children are merged in
// selection order (a sorted frontier of one entry per member: a member's
// children are ranked by probability) until the next child would fall at or
// beyond place cap; a child ranks after every kept node of equal or higher
// score, since it is deeper than all of them.  With short lists (k <= 8) a
// level's children are merged in batches of up to 64 instead of one at a
// time.  Cheap when few nodes below depth 1 make the cut (flat drafter
// distributions); a peaked distribution re-merges many nodes at every level,
// which is why the serial pops run beside it.
__device__ __forceinline__ int meta_pack(int par, int dep, int rank) { return (par + 1) | (dep << 8) | (rank << 16); }
__device__ __forceinline__ int meta_par(int v) { return (v & 255) - 1; }
__device__ __forceinline__ int meta_dep(int v) { return (v >> 8) & 127; }
__device__ __forceinline__ int meta_rank(int v) { return v >> 16; }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, ROW_MASK, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, ROW_MASK, 0xF, false));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
// Inclusive sum over the lanes (row shifts 1, 2, 4, 8, then the row totals
// broadcast into the following rows).  Used only where every partial sum is
// exact, so its association order does not matter.
__device__ __forceinline__ double wave_incl_sum_f64(double v) {
  v = __dadd_rn(v, dpp_f64<0x111, 0xF>(v));
  v = __dadd_rn(v, dpp_f64<0x112, 0xF>(v));
  v = __dadd_rn(v, dpp_f64<0x114, 0xF>(v));
  v = __dadd_rn(v, dpp_f64<0x118, 0xF>(v));
  v = __dadd_rn(v, dpp_f64<0x142, 0xA>(v));
  v = __dadd_rn(v, dpp_f64<0x143, 0xC>(v));
  return v;
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  return __longlong_as_double(static_cast<long long>(readlane_u64(static_cast<uint64_t>(__double_as_longlong(v)), l)));
}
__device__ __forceinline__ double wave_shr1_f64(double v, double fill) {
  return __longlong_as_double(static_cast<long long>(
      wave_shift_u64<kShr1>(static_cast<uint64_t>(__double_as_longlong(v)), static_cast<uint64_t>(__double_as_longlong(fill)))));
}

struct LevelScratch {
  float* sc;     // merged list, scores
  int* meta;     // merged list, packed parent / depth / rank
  float* bsc;    // next level's members: scores
  int* bmp;      //   ... places in the kept list; during a batch, old place -> new place
};

// Children per member below which a level is merged in batches (one lane per
// candidate child) rather than one child at a time.
constexpr int kBatchK = 8;

// Order of the batched merge (larger = earlier): score, then kept nodes ahead
// of children, then a smaller index (kept place or child index) first.
__device__ __forceinline__ uint64_t merge_key(float sc, bool kept, int idx) {
  return (static_cast<uint64_t>(ord_f32(sc)) << 32) | (kept ? 0x80000000u : 0u) |
         static_cast<uint32_t>(0xFFFF - idx);
}
// A bitonic sequence of 64 (key, origin) pairs across the lanes sorted
// descending: compare-exchanges at lane distances 32 .. 1.
template <int J>
__device__ __forceinline__ void kv_stage(uint64_t& k, int& o, int lane) {
  const uint64_t y = xor_lane_u64<J>(k);
  const int yo = static_cast<int>(xor_lane_u32<J>(static_cast<uint32_t>(o)));
  const bool lower = (lane & J) == 0;
  const bool take = lower ? y > k : y < k;
  k = take ? y : k;
  o = take ? yo : o;
}
__device__ __forceinline__ void kv_merge64(uint64_t& k, int& o, int lane) {
  kv_stage<32>(k, o, lane);
  kv_stage<16>(k, o, lane);
  kv_stage<8>(k, o, lane);
  kv_stage<4>(k, o, lane);
  kv_stage<2>(k, o, lane);
  kv_stage<1>(k, o, lane);
}
__device__ __forceinline__ int bperm_i(int src_lane, int v) {
  return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}
__device__ __forceinline__ float bperm_f(int src_lane, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

template <int SL, bool ADAPTIVE>
__device__ __forceinline__ int level_select(const TreeArgs& a, int b, int lane, const float* s_p, const LevelScratch& w,
                                            int* winner, float (&K_sc)[SL], int (&K_meta)[SL]) {
  const int k = a.k, cap = a.cap;
  const int kr = cap < k ? cap : k;
  int c = kr;
  // depth 1: the first list, in rank order (score 1 * q = q)
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int P = s * 64 + lane;
    K_sc[s] = P < c ? s_p[P] : 0.f;
    K_meta[s] = P < c ? meta_pack(-1, 1, P) : 0;
  }

  // members of the next level (lane t of slot s: member 64 s + t, in
  // selection order): at depth 1 the whole kept list; afterwards the children
  // merged at the level before, which all made the cut (the batched merge,
  // whose later batches can push out earlier ones' children, compacts the
  // kept nodes of the level's depth instead)
  int m = c;
  float M_sc[SL];
  int M_pos[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    M_sc[s] = K_sc[s];
    M_pos[s] = s * 64 + lane;
  }
  // list of position d: lane r of slot s holds q[d][64 s + r]; the next
  // level's list is read while this one merges
  auto load_row = [&](int d, float (&q)[SL]) {
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int P = s * 64 + lane;
      q[s] = (d <= a.gamma && P < k) ? s_p[(d - 1) * k + P] : 0.f;
    }
  };
  float qd[SL], qn[SL];
  load_row(2, qd);

  // Merge i children (in selection order: scores C_sc, parents' places C_mp,
  // ranks C_rank, kept nodes ahead C_pos) of depth d into the kept list.  A
  // kept node moves down by the children placed ahead of it (child j is
  // ahead of place P iff C_pos[j] <= P, counted in sh); parents follow
  // through the new places (npK, returned).
  auto apply_merge = [&](int i, int d, const float (&C_sc)[SL], const int (&C_mp)[SL], const int (&C_rank)[SL],
                         const int (&C_pos)[SL], const int (&sh)[SL], int (&npK)[SL]) {
#pragma unroll
    for (int s = 0; s < SL; ++s) npK[s] = s * 64 + lane + sh[s];
    auto newpos = [&](int old) {
      const int a0 = bperm_i(old & 63, npK[0]);
      const int a1 = SL > 1 ? bperm_i(old & 63, npK[SL - 1]) : a0;
      return old < 0 ? -1 : (old < 64 ? a0 : a1);
    };
    int kp[SL], cp[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      kp[s] = newpos(meta_par(K_meta[s]));
      cp[s] = newpos(C_mp[s]);
    }
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int P = s * 64 + lane;
      if (P < c && npK[s] < cap) {
        w.sc[npK[s]] = K_sc[s];
        w.meta[npK[s]] = meta_pack(kp[s], meta_dep(K_meta[s]), meta_rank(K_meta[s]));
      }
      if (P < i) {
        const int q = P + C_pos[s];
        w.sc[q] = C_sc[s];
        w.meta[q] = meta_pack(cp[s], d, C_rank[s]);
      }
    }
    c = cap < c + i ? cap : c + i;
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int P = s * 64 + lane;
      K_sc[s] = P < c ? w.sc[P] : 0.f;
      K_meta[s] = P < c ? w.meta[P] : 0;
    }
  };

  for (int d = 2; d <= a.gamma && m > 0; ++d) {
    load_row(d + 1, qn);
    if (kr <= kBatchK) {
      // Batches of the members' children, one candidate per lane (member
      // t0 + lane / kr, rank lane % kr), sorted across the lanes, merged in
      // member order: a child of a later batch ranks after an equal-score
      // child of an earlier one (its parent comes later), which the merged
      // list already holds, so the place rule stays "children of the batch
      // ahead + kept nodes of equal or higher score".
      const int per = 64 / kr;
      const int tl = lane / kr, rl = lane - tl * kr;
      bool stopped = false;
      const float q0 = readlane_f32(qd[0], 0);
      for (int t0 = 0; t0 < m; t0 += per) {
        // the batch's best possible child: the first child of its first
        // member (members pushed out, place -1, are a suffix); with the kept
        // list full it must beat the last kept node, else no later child can
        {
          const float ms0 = t0 < 64 ? readlane_f32(M_sc[0], t0 & 63) : readlane_f32(M_sc[SL - 1], t0 & 63);
          const int mp0 = t0 < 64 ? __builtin_amdgcn_readlane(M_pos[0], t0 & 63)
                                  : __builtin_amdgcn_readlane(M_pos[SL - 1], t0 & 63);
          const float last = (cap - 1) < 64 ? readlane_f32(K_sc[0], (cap - 1) & 63)
                                            : readlane_f32(K_sc[SL - 1], (cap - 1) & 63);
          if (mp0 < 0 || (c == cap && !(__fmul_rn(ms0, q0) > last))) break;
        }
        const int other = claim_load(winner);
        const int nb = (m - t0 < per ? m - t0 : per) * kr;
        const int t = t0 + tl;
        float msc = bperm_f(t & 63, M_sc[0]);
        int mpos = bperm_i(t & 63, M_pos[0]);
        if constexpr (SL > 1) {
          const float msc1 = bperm_f(t & 63, M_sc[SL - 1]);
          const int mpos1 = bperm_i(t & 63, M_pos[SL - 1]);
          msc = t < 64 ? msc : msc1;
          mpos = t < 64 ? mpos : mpos1;
        }
        const float qr = bperm_f(rl, qd[0]);
        // a member pushed out of the kept list by an earlier batch (place -1)
        // has at least cap kept nodes of higher or equal score ahead of it,
        // so none of its children can make the cut
        const bool valid = lane < nb && mpos >= 0;
        // the batch's children in selection order: lane i holds the i-th
        // (0 = none); the key carries score, parent place and rank
        const uint64_t key = sort64_desc(valid ? frontier_key(__fmul_rn(msc, qr), d, mpos, rl) : 0, lane);
        const uint32_t wl = static_cast<uint32_t>(key);
        const int crank = 127 - static_cast<int>(wl & 127);
        const int cpar = 255 - static_cast<int>((wl >> 7) & 255) - 1;
        const float cv = key_score(key);
        // Merge the batch into the kept list with one bitonic network: merge
        // keys order by score, kept nodes ahead of children on equal scores,
        // then by place / by child index; each entry carries its origin (kept
        // place P, or 128 + child index).  The kept list and the reversed
        // batch form a bitonic sequence whose larger half, taken place by
        // place, holds the first 64 * SL entries, still bitonic.
        uint64_t mk[SL];
        int org[SL];
#pragma unroll
        for (int s = 0; s < SL; ++s) {
          const int P = s * 64 + lane;
          mk[s] = P < c ? merge_key(K_sc[s], true, P) : 0;
          org[s] = P;
        }
        {
          const uint64_t ckr = reverse_lanes_u64(key != 0 ? merge_key(cv, false, lane) : 0);
          const bool t = ckr > mk[SL - 1];
          mk[SL - 1] = t ? ckr : mk[SL - 1];
          org[SL - 1] = t ? 128 + 63 - lane : org[SL - 1];
        }
        if constexpr (SL > 1) {
          const bool t = mk[1] > mk[0];
          const uint64_t k0 = mk[0];
          const int o0 = org[0];
          mk[0] = t ? mk[1] : mk[0];
          org[0] = t ? org[1] : org[0];
          mk[1] = t ? k0 : mk[1];
          org[1] = t ? o0 : org[1];
        }
#pragma unroll
        for (int s = 0; s < SL; ++s) kv_merge64(mk[s], org[s], lane);
        // the new kept list: its first cap entries
        int nk = 0, na = 0;
#pragma unroll
        for (int s = 0; s < SL; ++s) {
          const bool keep = mk[s] != 0 && s * 64 + lane < cap;
          nk += __popcll(__ballot(keep));
          na += __popcll(__ballot(keep && org[s] >= 128));
        }
        if (na == 0) {
          // no child of the batch made the cut (the kept list is unchanged):
          // the later batches' children score no higher
          if (claim_seen(other)) stopped = true;
          break;
        }
        // old place -> new place (-1: pushed past place cap)
#pragma unroll
        for (int s = 0; s < SL; ++s)
          if (s * 64 + lane < c) w.bmp[s * 64 + lane] = -1;
#pragma unroll
        for (int s = 0; s < SL; ++s)
          if (s * 64 + lane < nk && org[s] < 128) w.bmp[org[s]] = s * 64 + lane;
        // the origins' data: a kept node's score and packed record, a
        // child's parent place and rank (lane permutes of the old registers)
        float nsc[SL];
        int nmeta[SL];
#pragma unroll
        for (int s = 0; s < SL; ++s) {
          const int o = org[s];
          const int src = o & 63;
          float ks = bperm_f(src, K_sc[0]);
          int km = bperm_i(src, K_meta[0]);
          if constexpr (SL > 1) {
            const float ks1 = bperm_f(src, K_sc[SL - 1]);
            const int km1 = bperm_i(src, K_meta[SL - 1]);
            ks = (o & 64) ? ks1 : ks;
            km = (o & 64) ? km1 : km;
          }
          const int cp = bperm_i(src, cpar);
          const int crk = bperm_i(src, crank);
          const float cs = bperm_f(src, cv);
          const bool kept = o < 128;
          nsc[s] = kept ? ks : cs;
          nmeta[s] = kept ? km : meta_pack(cp, d, crk);   // parent: old place for now
        }
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < SL; ++s) {
          const int P = s * 64 + lane;
          const int po = meta_par(nmeta[s]);   // garbage past the new count: index kept in range
          const int pn = po < 0 ? -1 : w.bmp[po & 127];
          K_sc[s] = P < nk ? nsc[s] : 0.f;
          K_meta[s] = P < nk ? meta_pack(pn, meta_dep(nmeta[s]), meta_rank(nmeta[s])) : 0;
          // members' places after the merge (-1 once pushed past place cap)
          M_pos[s] = M_pos[s] >= 0 ? w.bmp[M_pos[s] & 127] : -1;
        }
        c = nk;
        if (claim_seen(other)) {
          stopped = true;
          break;
        }
      }
      if (stopped) return -1;
      // next members: the kept nodes of depth d, in order
      int nm = 0, tix[SL];
      bool mem[SL];
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        mem[s] = s * 64 + lane < c && meta_dep(K_meta[s]) == d;
        const uint64_t bm = __ballot(mem[s]);
        tix[s] = nm + static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0u)));
        nm += __popcll(bm);
      }
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        if (mem[s]) {
          w.bsc[tix[s]] = K_sc[s];
          w.bmp[tix[s]] = s * 64 + lane;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const int t2 = s * 64 + lane;
        M_sc[s] = t2 < nm ? w.bsc[t2] : 0.f;
        M_pos[s] = t2 < nm ? w.bmp[t2] : 0;
        qd[s] = qn[s];
      }
      m = nm;
      continue;
    }
    const float q0 = readlane_f32(qd[0], 0);
    // one frontier entry per member: its best unmerged child (the members'
    // first children are already in selection order)
    uint64_t H[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int t = s * 64 + lane;
      H[s] = t < m ? frontier_key(__fmul_rn(M_sc[s], q0), d, M_pos[s], 0) : 0;
    }
    auto insert = [&](uint64_t x) {
      int pos = 0;
#pragma unroll
      for (int s = 0; s < SL; ++s) pos += __popcll(__ballot(H[s] > x));
      uint64_t ck = 0;
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const uint64_t k63 = readlane_u64(H[s], 63);
        const uint64_t shk = wave_shift_u64<kShr1>(H[s], ck);
        const int P = s * 64 + lane;
        H[s] = P < pos ? H[s] : (P == pos ? x : shk);
        ck = k63;
      }
    };

    // merge: children in selection order, while they make the first cap
    int i = 0;
    float C_sc[SL];
    int C_mp[SL], C_rank[SL], C_pos[SL], sh[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      C_sc[s] = 0.f;
      C_mp[s] = C_rank[s] = C_pos[s] = sh[s] = 0;
    }
    // lanes holding kept nodes
    uint64_t kmask[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) kmask[s] = __ballot(s * 64 + lane < c);
    bool stopped = false;
    while (true) {
      // the serial wavefront's claim, read now and tested after this child
      const int other = claim_load(winner);
      const uint64_t hk = readlane_u64(H[0], 0);
      if (hk == 0) break;  // every member's children merged
      const uint32_t wl = static_cast<uint32_t>(hk);
      const int r = 127 - static_cast<int>(wl & 127);
      const int mp = 255 - static_cast<int>((wl >> 7) & 255) - 1;
      const float v = key_score(hk);
      // kept nodes ahead of the child: every one of equal or higher score
      int pos = 0;
#pragma unroll
      for (int s = 0; s < SL; ++s) pos += __popcll(__ballot(K_sc[s] >= v) & kmask[s]);
      if (i + pos >= cap) break;
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        if (s == (i >> 6)) {
          const bool me = lane == (i & 63);
          C_sc[s] = me ? v : C_sc[s];
          C_mp[s] = me ? mp : C_mp[s];
          C_rank[s] = me ? r : C_rank[s];
          C_pos[s] = me ? pos : C_pos[s];
        }
        sh[s] += pos <= s * 64 + lane ? 1 : 0;
      }
      ++i;
      // drop the merged child, enter its next sibling
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const uint64_t nk = s + 1 < SL ? readlane_u64(H[s + 1 < SL ? s + 1 : s], 0) : 0;
        H[s] = wave_shift_u64<kShl1>(H[s], nk);
      }
      // a child of rank >= cap trails its cap better-ranked siblings: never
      // kept (and the list row in registers covers ranks below 64 * SL)
      if (r + 1 < kr) {
        const int r1 = r + 1;
        float smp, qr;
        if constexpr (SL == 1) {
          smp = readlane_f32(K_sc[0], mp & 63);
          qr = readlane_f32(qd[0], r1 & 63);
        } else {
          smp = mp < 64 ? readlane_f32(K_sc[0], mp & 63) : readlane_f32(K_sc[SL - 1], mp & 63);
          qr = r1 < 64 ? readlane_f32(qd[0], r1 & 63) : readlane_f32(qd[SL - 1], r1 & 63);
        }
        insert(frontier_key(__fmul_rn(smp, qr), d, mp, r1));
      }
      if (claim_seen(other)) {
        stopped = true;
        break;
      }
    }
    if (stopped) return -1;
    if (i == 0) break;  // nothing of depth d kept: nothing deeper either

    int npK[SL];
    apply_merge(i, d, C_sc, C_mp, C_rank, C_pos, sh, npK);
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      // the merged children, in order, at their new places
      M_sc[s] = C_sc[s];
      M_pos[s] = s * 64 + lane + C_pos[s];
      qd[s] = qn[s];
    }
    m = i;
  }

  if constexpr (!ADAPTIVE) {
    return c;
  } else {
    // Stop rule over the kept list.  Phi at place P sums scores >= 2^-23 of
    // at most 128 nodes, so every partial sum is an exact multiple of
    // 2^(e-23), e >= -23, below 2^8: exact in fp64 in any order, equal to
    // the sequential sum.  From the first smaller score on, the sums are
    // taken one by one in order.
    const double l = static_cast<double>(a.prefix_len[b]);
    double inc[SL], ex[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int P = s * 64 + lane;
      inc[s] = wave_incl_sum_f64(P < c ? static_cast<double>(K_sc[s]) : 0.0);
    }
    double carry = 0.0;
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      inc[s] = __dadd_rn(inc[s], carry);
      ex[s] = wave_shr1_f64(inc[s], carry);
      carry = readlane_f64(inc[s], 63);
    }
    int t_ex = 0, stop = -1;
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int P = s * 64 + lane;
      const bool ok = P < c && K_sc[s] >= 0x1p-23f;
      t_ex += __popcll(__ballot(ok));
      const double th_in = __ddiv_rn(__dadd_rn(1.0, inc[s]), round_cost(a.cost, P + 1, l));
      const double th_ex = __ddiv_rn(__dadd_rn(1.0, ex[s]), round_cost(a.cost, P, l));
      const uint64_t sm = __ballot(ok && !(th_in > th_ex));
      if (sm != 0 && stop < 0) stop = s * 64 + static_cast<int>(__builtin_ctzll(sm));
    }
    if (stop >= 0) return stop;
    if (t_ex == c) return c;
    double phi = t_ex < 64 ? readlane_f64(ex[0], t_ex & 63) : readlane_f64(ex[SL - 1], t_ex & 63);
    double theta = __ddiv_rn(__dadd_rn(1.0, phi), round_cost(a.cost, t_ex, l));
    int n = t_ex;
    for (; n < c; ++n) {
      const float sn = n < 64 ? readlane_f32(K_sc[0], n & 63) : readlane_f32(K_sc[SL - 1], n & 63);
      const double phi2 = __dadd_rn(phi, static_cast<double>(sn));
      const double th2 = __ddiv_rn(__dadd_rn(1.0, phi2), round_cost(a.cost, n + 1, l));
      if (!(th2 > theta)) break;
      phi = phi2;
      theta = th2;
    }
    return n;
  }
}

// ---- outputs: parent, token, depth, score, ancestor bits ------------------
template <bool PER_NODE>
__device__ __forceinline__ void write_tree(const TreeArgs& a, int b, int tid, int nth, int n, const int* s_i,
                                           const NodeRecords& o) {
  const int W = (a.N_max + 31) >> 5;
  const size_t nb = static_cast<size_t>(b) * a.N_max;
  for (int i = tid; i < a.N_max; i += nth) {
    const bool v = i < n;
    a.parent[nb + i] = v ? o.par[i] : -1;
    const int trow = v ? (PER_NODE ? o.row[i] : o.dep[i] - 1) : 0;
    a.token[nb + i] = v ? s_i[trow * a.k + o.rank[i]] : -1;
    a.depth[nb + i] = v ? o.dep[i] : -1;
    a.score[nb + i] = v ? o.sc[i] : 0.0f;
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
        j = o.par[j];
      }
    }
    unsigned* dst = a.anc_bits + (nb + i) * W;
    dst[0] = w0;
    if (W > 1) dst[1] = w1;
    if (W > 2) dst[2] = w2;
    if (W > 3) dst[3] = w3;
  }
  if (tid == 0) a.n_nodes[b] = n;
}

// Per-node lists: serial pops, one wavefront per request.
template <int SL, bool ADAPTIVE>
__global__ __launch_bounds__(64) void best_first_node_kernel(TreeArgs a) {
  __shared__ float s_p[kMaxTopkTable];
  __shared__ int s_i[kMaxTopkTable];
  __shared__ int n_par[128], n_dep[128], n_rank[128], n_row[128];
  __shared__ float n_sc[128];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  load_table(a, b, lane, 64, s_p, s_i);
  __syncthreads();
  float r_sc[SL];
  int r_par[SL], r_dep[SL], r_rank[SL], r_row[SL];
  const int n = serial_select<SL, true, ADAPTIVE, false>(a, b, lane, s_p, 0.f, nullptr, r_sc, r_par, r_dep, r_rank,
                                                         r_row);
  const NodeRecords o{n_par, n_dep, n_rank, n_row, n_sc};
  store_serial_records<SL, true>(n, lane, r_sc, r_par, r_dep, r_rank, r_row, o);
  __syncthreads();
  write_tree<true>(a, b, lane, 64, n, s_i, o);
}

// Per-position lists: two wavefronts per request compute the same tree, the
// serial pops (wavefront 0) and the level-by-level merge (wavefront 1); the
// first to finish claims the result and writes the outputs, the other one
// sees the claim after at most one more pop or merged child and exits.
template <int SL, bool ADAPTIVE>
__global__ __launch_bounds__(128) void best_first_pos_kernel(TreeArgs a) {
  __shared__ float s_p[kMaxTopkTable];
  __shared__ int s_i[kMaxTopkTable];
  __shared__ int n_par[128], n_dep[128], n_rank[128];
  __shared__ float n_sc[128];
  __shared__ float l_sc[128], l_bsc[128];
  __shared__ int l_meta[128], l_bmp[128];
  __shared__ int s_winner;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // the best child of a node at depth d has probability p[d][0]: lane d keeps it
  const float q_first =
      (wave == 0 && lane < a.gamma) ? a.tk_p[static_cast<size_t>(b) * a.rows * a.k + static_cast<size_t>(lane) * a.k]
                                    : 0.f;
  load_table(a, b, tid, 128, s_p, s_i);
  if (tid == 0) s_winner = 0;
  __syncthreads();
  const NodeRecords o{n_par, n_dep, n_rank, nullptr, n_sc};
  if (wave == 0) {
    float r_sc[SL];
    int r_par[SL], r_dep[SL], r_rank[SL], r_row[SL];
    const int n = a.method == 2 ? -1
                                : serial_select<SL, false, ADAPTIVE, true>(a, b, lane, s_p, q_first, &s_winner, r_sc,
                                                                           r_par, r_dep, r_rank, r_row);
    if (n >= 0 && claim(&s_winner, 1)) {
      store_serial_records<SL, false>(n, lane, r_sc, r_par, r_dep, r_rank, r_row, o);
      wave_lds_sync();
      write_tree<false>(a, b, lane, 64, n, s_i, o);
    }
  } else {
    float K_sc[SL];
    int K_meta[SL];
    const LevelScratch w{l_sc, l_meta, l_bsc, l_bmp};
    const int n = a.method == 1 ? -1 : level_select<SL, ADAPTIVE>(a, b, lane, s_p, w, &s_winner, K_sc, K_meta);
    if (n >= 0 && claim(&s_winner, 2)) {
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const int i = s * 64 + lane;
        if (i < n) {
          n_par[i] = meta_par(K_meta[s]);
          n_dep[i] = meta_dep(K_meta[s]);
          n_rank[i] = meta_rank(K_meta[s]);
          n_sc[i] = K_sc[s];
        }
      }
      wave_lds_sync();
      write_tree<false>(a, b, lane, 64, n, s_i, o);
    }
  }
  // the other wavefront stops at its next pop after the claim and exits
}

}  // namespace

hipError_t launch_best_first(const TreeArgs& a, hipStream_t s) {
  // sorted frontiers of 64 or 128 places (at least cap); the stop rule only
  // in the adaptive instances
  const dim3 g(a.B);
#define TSV_BF(KERNEL, SL, THREADS)                                     \
  if (a.adaptive) KERNEL<SL, true><<<g, dim3(THREADS), 0, s>>>(a);      \
  else KERNEL<SL, false><<<g, dim3(THREADS), 0, s>>>(a);
  if (a.per_node) {
    if (a.cap <= 64) {
      TSV_BF(best_first_node_kernel, 1, 64)
    } else {
      TSV_BF(best_first_node_kernel, 2, 64)
    }
  } else {
    if (a.cap <= 64) {
      TSV_BF(best_first_pos_kernel, 1, 128)
    } else {
      TSV_BF(best_first_pos_kernel, 2, 128)
    }
  }
#undef TSV_BF
  return hipGetLastError();
}

}  // namespace tsv
