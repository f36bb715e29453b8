// build_tree, stage 1: per-position top-k over the drafter marginals.
//
// [caddtree] Methodology: the drafter's single forward pass yields one
// marginal distribution per block position; the tree branches on the most
// probable tokens of each position.  Order: probability descending, then
// token id ascending.
//
// Design (HBM-bound scan, rows of ~10^5 probabilities), one workgroup per
// row and one wavefront per contiguous segment of it:
//   * a wavefront keeps the best KS = 64 or 128 keys of its segment as a
//     sorted list spread over its 64 lanes (one or two slots per lane);
//   * it filters the stream with the larger of its own k-th best value and
//     the row's floor, the largest k-th best any wavefront of the row has
//     published (an LDS atomic max): k elements of the row are at least that
//     value, so nothing below it can reach the row's top k;
//   * survivors are appended to a per-wave 64-entry LDS queue; a full queue
//     is bitonic-sorted across lanes and merged into the list (elementwise
//     max against the reversed queue, then a bitonic merge), with lane
//     exchanges done by DPP and permlane swaps;
//   * the first k keys of every list are finally sorted together in LDS.
// Keys are unique (value, then lower index), so the result does not depend
// on the segmentation, on timing, or on the order elements are seen.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

// Inverse of ord_f32 for a non-zero ordered value.
__device__ __forceinline__ float ord_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Sorts one value per lane descending within each row of 16 lanes.
template <int K, int J>
__device__ __forceinline__ uint32_t bitonic16_pass(uint32_t x, int lane) {
  const uint32_t y = xor_lane_u32<J>(x);
  const bool lower = (lane & J) == 0;
  const bool desc = (lane & K) == 0 || K == 16;
  x = (lower == desc) ? umax32(x, y) : (x < y ? x : y);
  if constexpr (J > 1) x = bitonic16_pass<K, J / 2>(x, lane);
  return x;
}
__device__ __forceinline__ uint32_t sort16_desc_u32(uint32_t x, int lane) {
  x = bitonic16_pass<2, 1>(x, lane);
  x = bitonic16_pass<4, 2>(x, lane);
  x = bitonic16_pass<8, 4>(x, lane);
  return bitonic16_pass<16, 8>(x, lane);
}

template <int SLOTS>
struct WaveList {
  uint64_t v[SLOTS];
  int lane;

  __device__ void clear(int l) {
    lane = l;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) v[s] = 0;
  }

  // Merge 64 keys sorted descending across lanes (one per lane) into the
  // descending list, keeping the best 64*SLOTS.
  __device__ void merge(uint64_t q) {
    uint64_t qr = reverse_lanes_u64(q);  // ascending
    if (SLOTS == 1) {
      v[0] = umax64(v[0], qr);
    } else {
      v[SLOTS - 1] = umax64(v[SLOTS - 1], qr);
      uint64_t a = v[0], b = v[SLOTS - 1];
      v[0] = umax64(a, b);
      v[SLOTS - 1] = umin64(a, b);
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) v[s] = half_cleaner<32>(v[s]);
  }

  // Bitonic merge stages lane ^ J, ..., lane ^ 1 (descending result).
  template <int J>
  __device__ uint64_t half_cleaner(uint64_t x) const {
    const uint64_t o = xor_lane_u64<J>(x);
    x = (lane & J) == 0 ? umax64(x, o) : umin64(x, o);
    if constexpr (J > 1) x = half_cleaner<J / 2>(x);
    return x;
  }

  // Key at list position p (uniform p).
  __device__ uint64_t at(int p) const {
    uint64_t x = v[0];
    if (SLOTS > 1 && p >= 64) x = v[SLOTS - 1];
    return readlane_u64(x, p & 63);
  }
};

template <int SLOTS>
struct WaveSelect {
  WaveList<SLOTS> list;
  uint64_t tau;       // k-th best key so far (0 = fewer than k seen)
  float tau_v;        // its value, -inf while empty
  int qcount;         // wave-uniform
  int k;
  uint64_t* queue;    // this wave's 64 LDS slots
  uint32_t* pub;      // per segment: ordered bits of its m-th best value (LDS)
  int wave, nseg, m, r;

  __device__ void init(int kk, uint64_t* q, uint32_t* published, int w, int ns, int lane) {
    list.clear(lane);
    tau = 0;
    tau_v = -INFINITY;
    qcount = 0;
    k = kk;
    queue = q;
    pub = published;
    wave = w;
    nseg = ns;
    const int r0 = min(4, min(ns, kk));
    m = (kk + r0 - 1) / r0;
    r = (kk + m - 1) / m;  // <= r0 <= nseg
  }

  __device__ void flush() {
    wave_lds_sync();
    uint64_t x = list.lane < qcount ? queue[list.lane] : 0;
    wave_lds_sync();
    x = sort64_desc(x, list.lane);
    list.merge(x);
    qcount = 0;
    set_tau();
  }

  // tau = the list's k-th key; the value of its m-th key is published for
  // the row's floor (values only grow, so an old one stays a valid bound)
  __device__ void set_tau() {
    tau = list.at(k - 1);
    if (tau != 0) tau_v = ord_value(static_cast<uint32_t>(tau >> 32));
    const uint32_t om = static_cast<uint32_t>(list.at(m - 1) >> 32);
    if (list.lane == 0 && om != 0) pub[wave] = om;
  }

  // Filter value: the larger of the own k-th best and the row's floor, the
  // r-th largest published value: r segments each hold m >= k/r elements at
  // or above it, so k elements of the row are, and nothing below it can
  // reach the row's top k.  The published values are sorted across the
  // first 16 lanes (0 = not yet published, so too few gives no floor).
  __device__ float threshold() const {
    uint32_t o = list.lane < nseg ? __hip_atomic_load(pub + list.lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0u;
    o = sort16_desc_u32(o, list.lane);
    o = __builtin_amdgcn_readlane(o, r - 1);
    return o == 0 ? tau_v : fmaxf(tau_v, ord_value(o));
  }

  // Every lane offers one key (0 = nothing).
  __device__ void offer(uint64_t key) {
    bool pass = key > tau;
    uint64_t mask = __ballot(pass);
    if (mask == 0) return;
    int n = __popcll(mask);
    if (qcount + n > 64) {
      flush();
      pass = key > tau;
      mask = __ballot(pass);
      if (mask == 0) return;
      n = __popcll(mask);
    }
    if (pass) {
      int below = __builtin_amdgcn_mbcnt_hi(
          static_cast<uint32_t>(mask >> 32),
          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
      queue[qcount + below] = key;
    }
    qcount += n;
  }

  __device__ void finish() {
    if (qcount > 0) flush();
  }
};

constexpr int kMaxSegments = 16;
constexpr int kComputeUnits = 256;   // of the MI355X
constexpr int kBlock = 2048;   // elements a wavefront reads per block (32 per lane)
// the final merge holds every wave's list
constexpr int kMaxCand = kMaxSegments * 128;

// Element j (0..31) of this lane in a block starting at `base`: four
// adjacent elements per 16-byte load when the row allows vector access, one
// element per lane and load otherwise.
template <bool VEC>
__device__ __forceinline__ int blk_elem(int base, int j, int lane) {
  return VEC ? base + (j >> 2) * 256 + lane * 4 + (j & 3) : base + j * 64 + lane;
}

// A block is read through a buffer resource over [base, end) of the row
// (stride 0, dword 3 = 0x00020000, the raw 32-bit format of the CDNA buffer
// descriptor): loads past its end return zeros without touching memory and
// are never used, so no address is clamped and every load is issued without
// a condition (a block's wait then covers only its own loads).
template <bool VEC>
__device__ __forceinline__ void load_blk(float (&v)[32], const float* p, int base, int end, int lane) {
  const int avail = base < end ? end - base : 0;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p) + (base < end ? base : 0), 0, avail * 4, 0x00020000);
  if (VEC) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (u * 256 + lane * 4) * 4, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * u + c] = __uint_as_float(x[c]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (j * 64 + lane) * 4, 0, 0));
  }
}

// One workgroup per row.  The row is cut into blocks of kBlock elements;
// wave w of the W waves reads blocks w, w + W, w + 2W, ... (interleaved, so
// the waves of a row stream neighbouring blocks and finish together) and
// keeps its own list.
template <int SLOTS, bool VEC>
__global__ __launch_bounds__(64 * kMaxSegments) void topk_row_kernel(
    const float* __restrict__ x, int V, int k, int nseg,
    int* __restrict__ out_idx, float* __restrict__ out_p) {
  __shared__ uint64_t queue[kMaxSegments][64];
  __shared__ uint64_t cand[kMaxCand];
  __shared__ uint32_t published[kMaxSegments];
  __shared__ int cand_n;
  // wave-uniform values live in scalar registers (uniform branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = blockIdx.x;
  const int W = nseg;                         // waves of the workgroup
  const int nb = (V + kBlock - 1) / kBlock;   // blocks of the row, >= W
  const int end = V;
  const float* p = x + static_cast<size_t>(row) * V;

  // The first block is requested before anything else happens; the second
  // once the first has arrived, so that it is in flight while the first one
  // seeds the list (requested together, both land in one burst and nothing
  // is in flight during the seed).  A list of 128 takes two sorts and a
  // merge to seed: its second block is requested after them, still in time
  // for the first block's offers, leaving the memory path to the compute
  // unit's other workgroup meanwhile (4-5 us less on 1024 rows of top-128;
  // the same order costs 1 us with lists of 64).
  float b0[32], b1[32];
  int i0 = wave, i1 = wave + W;
  load_blk<VEC>(b0, p, i0 * kBlock, end, lane);
  if (threadIdx.x < kMaxSegments) published[threadIdx.x] = 0;
  if (threadIdx.x == 0) cand_n = 0;
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0) only: the first block is here
  asm volatile("" ::: "memory");
  if (SLOTS == 1) load_blk<VEC>(b1, p, i1 * kBlock, end, lane);

  WaveSelect<SLOTS> sel;
  sel.init(k, queue[wave], published, wave, W, lane);
  // Offers the elements of a block at or above thr, except element `skip1`
  // and `skip2` of this lane (the ones the first block seeded the list with).
  // A lane's passing elements of a 16-byte group become keys (0 for the
  // others), sorted descending by a five-step network, and are offered only
  // while some lane still has one, so a group usually costs one offer.  The
  // list's final contents do not depend on the order of the offers.
  auto offer_block = [&](const float (&v)[32], int base, float thr, int skip1, int skip2) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // the group's maximum decides first whether any key needs building
      const float gm = vmax3(vmax3(v[4 * u], v[4 * u + 1], v[4 * u + 2]), v[4 * u + 3], v[4 * u + 3]);
      if (__ballot(gm >= thr && blk_elem<VEC>(base, 4 * u, lane) < end) == 0) continue;
      uint64_t kk[4];
      bool any = false;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * u + c;
        const int e = blk_elem<VEC>(base, j, lane);
        const bool ok = e < end && v[j] >= thr && j != skip1 && j != skip2;
        kk[c] = ok ? sel_key(v[j], static_cast<uint32_t>(e)) : 0;
        any |= ok;
      }
      if (__ballot(any) == 0) continue;
      auto order = [](uint64_t& a, uint64_t& b) {
        const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
        a = hi;
        b = lo;
      };
      order(kk[0], kk[1]);
      order(kk[2], kk[3]);
      order(kk[0], kk[2]);
      order(kk[1], kk[3]);
      order(kk[1], kk[2]);
      sel.offer(kk[0]);
      if (__ballot(kk[1] != 0) != 0) {
        sel.offer(kk[1]);
        if (__ballot(kk[2] != 0) != 0) {
          sel.offer(kk[2]);
          if (__ballot(kk[3] != 0) != 0) sel.offer(kk[3]);
        }
      }
    }
  };
  auto process = [&](const float (&v)[32], int base) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      const int e = blk_elem<VEC>(base, j, lane);
      float g;
      if (VEC) {
        // a 16-byte group lies wholly inside or wholly outside the row
        g = vmax3(vmax3(v[j], v[j + 1], v[j + 2]), v[j + 3], v[j + 3]);
        g = e < end ? g : -INFINITY;
      } else {
        g = -INFINITY;
#pragma unroll
        for (int c = 0; c < 4; ++c) g = blk_elem<VEC>(base, j + c, lane) < end ? fmaxf(g, v[j + c]) : g;
      }
      m = fmaxf(m, g);
    }
    const float thr = sel.threshold();
    if (__ballot(m >= thr) == 0) return;
    offer_block(v, base, thr, -1, -1);
  };

  // A wave's first block seeds the list with every lane's best (and, for lists of 128,
  // second best) element in one sort; only the rest is offered.  Without the
  // seed the threshold admits everything until k keys are seen, and each 64
  // admissions cost a full sort and merge.
  {
    // a lane's best element is its largest value, the first one on ties
    // (element indices grow with j, and the lower index is the better key)
    float m1 = -INFINITY, m2 = -INFINITY;
    int j1 = -1, j2 = -1;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const bool ok = blk_elem<VEC>(i0 * kBlock, j, lane) < end && b0[j] > m1;
      m1 = ok ? b0[j] : m1;
      j1 = ok ? j : j1;
    }
    if (SLOTS > 1) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const bool ok = blk_elem<VEC>(i0 * kBlock, j, lane) < end && j != j1 && b0[j] > m2;
        m2 = ok ? b0[j] : m2;
        j2 = ok ? j : j2;
      }
    }
    const uint64_t k1 = j1 >= 0 ? sel_key(m1, static_cast<uint32_t>(blk_elem<VEC>(i0 * kBlock, j1, lane))) : 0;
    const uint64_t k2 = j2 >= 0 ? sel_key(m2, static_cast<uint32_t>(blk_elem<VEC>(i0 * kBlock, j2, lane))) : 0;
    sel.list.v[0] = sort64_desc(k1, lane);
    if (SLOTS > 1) sel.list.merge(sort64_desc(k2, lane));
    sel.set_tau();
    if (SLOTS > 1) {
      __builtin_amdgcn_sched_barrier(0);
      load_blk<VEC>(b1, p, i1 * kBlock, end, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    offer_block(b0, i0 * kBlock, sel.threshold(), j1, j2);
  }
  // two blocks in turn: one in flight while the other is scanned
  int inext = i1 + W;
  auto take = [&]() {
    const int i = inext;
    inext += W;
    return i;
  };
  while (i1 < nb) {
    const int i2 = take();
    load_blk<VEC>(b0, p, i2 * kBlock, end, lane);
    process(b1, i1 * kBlock);
    if (i2 >= nb) break;
    i1 = take();
    load_blk<VEC>(b1, p, i1 * kBlock, end, lane);
    process(b0, i2 * kBlock);
  }

  // Final merge.  A wave's own k best keys are the first k of its list once
  // its queue is merged in (an element passed the filter when it was seen,
  // the filter being a lower bound of the row's k-th value, and a list drops
  // a key only for 64 * SLOTS >= k better keys of the same wave), so the
  // row's top k is among the waves' first k keys.  Once every wave has
  // published its final value, the keys at or above the row floor (only
  // those can rank below k) are gathered in LDS; the rank of a key is the
  // number of gathered keys larger than it (keys are unique), and the key of
  // rank r < k is written to place r.
  sel.finish();
  __syncthreads();
  const int KL = 64 * SLOTS;
  const int kl = min(k, KL);
  {
    uint32_t o = lane < W ? published[lane] : 0u;
    o = sort16_desc_u32(o, lane);
    const uint32_t ofloor = __builtin_amdgcn_readlane(o, sel.r - 1);   // 0: no floor
    int n = 0;
    uint64_t mk[SLOTS];
#pragma unroll
    for (int s2 = 0; s2 < SLOTS; ++s2) {
      const uint64_t key = sel.list.v[s2];
      const bool keep = s2 * 64 + lane < kl && key != 0 && static_cast<uint32_t>(key >> 32) >= ofloor;
      mk[s2] = __ballot(keep);
      n += __popcll(mk[s2]);
    }
    int base = 0;
    if (lane == 0) base = __hip_atomic_fetch_add(&cand_n, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int s2 = 0; s2 < SLOTS; ++s2) {
      if ((mk[s2] >> lane) & 1) {
        const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mk[s2] >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mk[s2]), 0));
        cand[base + below] = sel.list.v[s2];
      }
      base += __popcll(mk[s2]);
    }
  }
  __syncthreads();
  const int C = cand_n;
  for (int i = threadIdx.x; i < C; i += blockDim.x) {
    const uint64_t key = cand[i];
    int rank = 0, j = 0;
    for (; j + 4 <= C; j += 4)
      rank += (cand[j] > key ? 1 : 0) + (cand[j + 1] > key ? 1 : 0) + (cand[j + 2] > key ? 1 : 0) +
              (cand[j + 3] > key ? 1 : 0);
    for (; j < C; ++j) rank += cand[j] > key ? 1 : 0;
    if (rank < k) {
      const uint32_t idx = sel_key_index(key);
      out_idx[static_cast<size_t>(row) * k + rank] = static_cast<int>(idx);
      // the key holds the value's exact bits except the sign of a zero,
      // so only a zero is read again
      float v = ord_value(static_cast<uint32_t>(key >> 32));
      if (v == 0.0f) v = p[idx];
      out_p[static_cast<size_t>(row) * k + rank] = v;
    }
  }
}

}  // namespace

TopkPlan topk_plan(int rows, int V, int k) {
  TopkPlan p;
  p.rows = rows;
  p.V = V;
  p.k = k;
  p.slots = k <= 64 ? 1 : 2;
  p.vec = (V % 4) == 0;
  // One wave per block of the row, at most kMaxSegments; with more rows than
  // compute units, half as many, so that two rows share a compute unit and
  // one streams while the other merges; with more than twice as many rows, a
  // quarter, so that four rows share one (1024 rows of 151936: all resident
  // at once, each wave seeding one list for 19 blocks; 136-138 against
  // 147-148 us with top-128 lists, 117-118 against 122-124 with top-32).
  const int nb = (V + kBlock - 1) / kBlock;
  const int most = rows > 2 * kComputeUnits ? kMaxSegments / 4
                   : rows > kComputeUnits   ? kMaxSegments / 2
                                            : kMaxSegments;
  p.nseg = nb < most ? nb : most;
  return p;
}

hipError_t launch_topk(const float* x, const TopkPlan& p, int* out_idx, float* out_p, hipStream_t s) {
  dim3 grid(p.rows), block(64 * p.nseg);
  if (p.slots == 1) {
    if (p.vec)
      topk_row_kernel<1, true><<<grid, block, 0, s>>>(x, p.V, p.k, p.nseg, out_idx, out_p);
    else
      topk_row_kernel<1, false><<<grid, block, 0, s>>>(x, p.V, p.k, p.nseg, out_idx, out_p);
  } else {
    if (p.vec)
      topk_row_kernel<2, true><<<grid, block, 0, s>>>(x, p.V, p.k, p.nseg, out_idx, out_p);
    else
      topk_row_kernel<2, false><<<grid, block, 0, s>>>(x, p.V, p.k, p.nseg, out_idx, out_p);
  }
  return hipGetLastError();
}

}  // namespace tsv
