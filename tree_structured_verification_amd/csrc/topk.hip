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

// One compare-exchange stage of a bitonic network over the 64 lanes: lanes
// l and l ^ J swap so that the block of K lanes holding l ends up descending
// (or ascending, for every other block when K < 64).
template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_stage(uint64_t x, int lane) {
  const uint64_t y = xor_lane_u64<J>(x);
  const bool lower = (lane & J) == 0;
  const bool desc = (lane & K) == 0;
  return (lower == desc) ? umax64(x, y) : umin64(x, y);
}
template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_pass(uint64_t x, int lane) {
  x = bitonic_stage<K, J>(x, lane);
  if constexpr (J > 1) x = bitonic_pass<K, J / 2>(x, lane);
  return x;
}
// Sorts one key per lane, descending over lanes 0..63.
__device__ __forceinline__ uint64_t sort64_desc(uint64_t x, int lane) {
  x = bitonic_pass<2, 1>(x, lane);
  x = bitonic_pass<4, 2>(x, lane);
  x = bitonic_pass<8, 4>(x, lane);
  x = bitonic_pass<16, 8>(x, lane);
  x = bitonic_pass<32, 16>(x, lane);
  return bitonic_pass<64, 32>(x, lane);
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

// One workgroup per row, wavefront w scanning segment w.
template <int SLOTS, bool VEC>
__global__ __launch_bounds__(64 * kMaxSegments) void topk_row_kernel(
    const float* __restrict__ x, int rows, int V, int k, int nseg, int seg_len,
    int* __restrict__ out_idx, float* __restrict__ out_p) {
  __shared__ uint64_t queue[kMaxSegments][64];
  __shared__ uint64_t keys[kMaxSegments * 128];   // list hand-over, up to 128 keys per wave
  __shared__ uint32_t published[kMaxSegments];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x;
  if (threadIdx.x < kMaxSegments) published[threadIdx.x] = 0;
  __syncthreads();
  // wave-uniform, so that a block's buffer resource lives in scalar registers
  const int beg = __builtin_amdgcn_readfirstlane(wave * seg_len);
  const int end = __builtin_amdgcn_readfirstlane(min(V, beg + seg_len));
  const float* p = x + static_cast<size_t>(row) * V;

  WaveSelect<SLOTS> sel;
  sel.init(k, queue[wave], published, wave, nseg, lane);

  // Warm-up on the first 1024 elements: seed the list with every lane's best
  // (and, for lists of 128, second best) element in one sort, then offer
  // only the rest.  Without the seed the threshold admits everything until k
  // keys are seen, and each 64 admissions cost a full sort and merge.
  {
    float v[16];
    int e0[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      // element order per lane is increasing in index, as in the main loop
      const int e = VEC ? beg + (u >> 2) * 256 + lane * 4 + (u & 3) : beg + u * 64 + lane;
      e0[u] = e;
      v[u] = e < end ? p[e] : -INFINITY;
    }
    uint64_t k1 = 0, k2 = 0;
    int u1 = -1, u2 = -1;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint64_t kk = e0[u] < end ? sel_key(v[u], e0[u]) : 0;
      if (kk > k1) { k2 = k1; u2 = u1; k1 = kk; u1 = u; }
      else if (kk > k2) { k2 = kk; u2 = u; }
    }
    sel.list.v[0] = sort64_desc(k1, lane);
    if (SLOTS > 1) sel.list.merge(sort64_desc(k2, lane));
    sel.set_tau();
    const float thr = sel.threshold();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool seeded = (u == u1) || (SLOTS > 1 && u == u2);
      const bool ok = e0[u] < end && !seeded && v[u] >= thr;
      if (__ballot(ok) == 0) continue;
      sel.offer(ok ? sel_key(v[u], e0[u]) : 0);
    }
  }

  if (VEC) {
    // blocks of 8 float4 per lane (2048 elements); a group past the end
    // re-reads the slice's last group and is ignored, so loads are
    // unconditional; two blocks alternate so that one is in flight while the
    // other is scanned
    // A block is read through a buffer resource over [base, end) of the row
    // (stride 0, dword 3 = 0x00020000, the raw 32-bit format of the CDNA
    // buffer descriptor): loads past its end return zeros without touching
    // memory and are never processed, so no address is clamped and the lane
    // offsets stay constant registers.
    auto load_block = [&](float4 (&raw)[8], int base) {
      const int avail = base < end ? end - base : 0;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(p) + (base < end ? base : 0), 0, avail * 4, 0x00020000);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (u * 256 + lane * 4) * 4, 0, 0);
        raw[u] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                             __uint_as_float(v[3]));
      }
    };
    auto process = [&](const float4 (&v)[8], int base) {
      float m4[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = base + u * 256 + lane * 4;
        const float m = vmax3(vmax3(v[u].x, v[u].y, v[u].z), v[u].w, v[u].w);
        m4[u] = e < end ? m : -INFINITY;
      }
      const float m = vmax3(vmax3(m4[0], m4[1], m4[2]), vmax3(m4[3], m4[4], m4[5]), vmax3(m4[6], m4[7], m4[7]));
      const float thr = sel.threshold();
      if (__ballot(m >= thr) == 0) return;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = base + u * 256 + lane * 4;
        const bool ok = e < end;
        if (__ballot(ok && m4[u] >= thr) == 0) continue;
        // The lane's elements at or above the filter become keys (0 for the
        // others), sorted descending by a five-step network; they are offered
        // only while some lane still has one, so a group usually costs one
        // or two offers instead of four.  The list's final contents do not
        // depend on the order of the offers.  (Indices stay static: a loop
        // over a lane's pending elements moved the block to scratch memory.)
        uint64_t k0 = ok && v[u].x >= thr ? sel_key(v[u].x, e) : 0;
        uint64_t k1 = ok && v[u].y >= thr ? sel_key(v[u].y, e + 1) : 0;
        uint64_t k2 = ok && v[u].z >= thr ? sel_key(v[u].z, e + 2) : 0;
        uint64_t k3 = ok && v[u].w >= thr ? sel_key(v[u].w, e + 3) : 0;
        auto order = [](uint64_t& a, uint64_t& b) {
          const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
          a = hi;
          b = lo;
        };
        order(k0, k1);
        order(k2, k3);
        order(k0, k2);
        order(k1, k3);
        order(k1, k2);
        sel.offer(k0);
        if (__ballot(k1 != 0) != 0) {
          sel.offer(k1);
          if (__ballot(k2 != 0) != 0) {
            sel.offer(k2);
            if (__ballot(k3 != 0) != 0) sel.offer(k3);
          }
        }
      }
    };
    // The next block's loads are issued without a condition (past the end
    // they return zeros, never processed): behind a branch, the wait
    // before the current block's last use would also cover them, and the
    // two blocks would no longer overlap.
    float4 b0[8], b1[8];
    const int first = beg + 1024;
    load_block(b0, first);
    for (int base = first; base < end; base += 4096) {
      load_block(b1, base + 2048);
      process(b0, base);
      if (base + 2048 >= end) break;
      load_block(b0, base + 4096);
      process(b1, base + 2048);
    }
  } else {
    for (int base = beg + 1024; base < end; base += 1024) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        int e = base + u * 64 + lane;
        v[u] = e < end ? p[e] : -INFINITY;
      }
      float m = -INFINITY;
#pragma unroll
      for (int u = 0; u < 16; ++u) m = fmaxf(m, v[u]);
      if (__ballot(m >= sel.threshold()) == 0) continue;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        int e = base + u * 64 + lane;
        sel.offer(e < end ? sel_key(v[u], e) : 0);
      }
    }
  }
  sel.finish();

  // Tree merge of the wave lists (each holds its segment's best keys, and
  // the row's top k is among them): in round r, wave w with w % 2r == r
  // hands its list through LDS to wave w - r, which merges it into its own.
  // A wave's LDS slot is read only in the round it sends, and it sends only
  // after its last merge, so one barrier per round orders everything.
  for (int r = 1; r < nseg; r <<= 1) {
    if ((wave & (2 * r - 1)) == r) {
#pragma unroll
      for (int s2 = 0; s2 < SLOTS; ++s2) keys[wave * 128 + s2 * 64 + lane] = sel.list.v[s2];
    }
    __syncthreads();
    if ((wave & (2 * r - 1)) == 0 && wave + r < nseg) {
#pragma unroll
      for (int s2 = 0; s2 < SLOTS; ++s2) sel.list.merge(keys[(wave + r) * 128 + s2 * 64 + lane]);
    }
  }
  if (wave != 0) return;
#pragma unroll
  for (int s2 = 0; s2 < SLOTS; ++s2) {
    const int pos = s2 * 64 + lane;
    if (pos >= k) continue;
    const uint64_t key = sel.list.v[s2];
    // every row holds V >= k elements, so the first k places are filled;
    // the guard keeps an impossible empty place inside the row
    const uint32_t idx = key ? sel_key_index(key) : 0u;
    out_idx[static_cast<size_t>(row) * k + pos] = static_cast<int>(idx);
    // re-read the element so the stored probability keeps its exact bits
    out_p[static_cast<size_t>(row) * k + pos] = p[idx];
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
  // segments of at least ~8k elements, at most kMaxSegments per row
  int nseg = (V + 8191) / 8192;
  if (nseg > kMaxSegments) nseg = kMaxSegments;
  if (nseg < 1) nseg = 1;
  int len = (V + nseg - 1) / nseg;
  len = (len + 1023) / 2048 * 2048 + 1024;  // one warm-up block of 1024, then steps of 2048
  p.seg_len = len;
  p.nseg = (V + len - 1) / len;
  return p;
}

size_t topk_ws_bytes(const TopkPlan&) { return 0; }

hipError_t launch_topk(const float* x, const TopkPlan& p, uint64_t*, int* out_idx, float* out_p,
                       hipStream_t s) {
  dim3 grid(p.rows), block(64 * p.nseg);
  if (p.slots == 1) {
    if (p.vec)
      topk_row_kernel<1, true><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, out_idx, out_p);
    else
      topk_row_kernel<1, false><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, out_idx, out_p);
  } else {
    if (p.vec)
      topk_row_kernel<2, true><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, out_idx, out_p);
    else
      topk_row_kernel<2, false><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, out_idx, out_p);
  }
  return hipGetLastError();
}

}  // namespace tsv
