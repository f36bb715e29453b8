// build_tree, stage 1: per-position top-k over the drafter marginals.
//
// [caddtree] Methodology: the drafter's single forward pass yields one
// marginal distribution per block position; the tree branches on the most
// probable tokens of each position.  Order: probability descending, then
// token id ascending.
//
// Design (HBM-bound scan, rows of ~10^5 probabilities):
//   * each wavefront owns one contiguous segment of one row and keeps the
//     best KS = 64 or 128 keys of that segment as a sorted list spread over
//     its 64 lanes (one or two slots per lane);
//   * a running threshold (the k-th best key so far) filters the stream: a
//     lane tests the max of 16 loaded values against it, so after a short
//     warm-up almost every 1 KiB load costs one compare and one ballot;
//   * survivors are appended to a per-wave 64-entry LDS queue; a full queue
//     is bitonic-sorted across lanes and merged into the list (elementwise
//     max against the reversed queue, then a bitonic merge);
//   * a second kernel merges the per-segment lists of a row the same way.
// Keys are unique (value, then lower index), so the result does not depend
// on the segmentation or on the order elements are seen.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

__device__ __forceinline__ uint64_t sort64_desc(uint64_t x, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t y = shfl_xor_u64(x, j);
      bool lower = (lane & j) == 0;
      bool desc = (lane & k) == 0;
      x = (lower == desc) ? umax64(x, y) : umin64(x, y);
    }
  }
  return x;
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
    uint64_t qr = shfl_u64(q, 63 - lane);  // ascending
    if (SLOTS == 1) {
      v[0] = umax64(v[0], qr);
    } else {
      v[SLOTS - 1] = umax64(v[SLOTS - 1], qr);
      uint64_t a = v[0], b = v[SLOTS - 1];
      v[0] = umax64(a, b);
      v[SLOTS - 1] = umin64(a, b);
    }
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) {
      bool lower = (lane & j) == 0;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        uint64_t o = shfl_xor_u64(v[s], j);
        v[s] = lower ? umax64(v[s], o) : umin64(v[s], o);
      }
    }
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

  __device__ void init(int kk, uint64_t* q, int lane) {
    list.clear(lane);
    tau = 0;
    tau_v = -INFINITY;
    qcount = 0;
    k = kk;
    queue = q;
  }

  __device__ void flush() {
    wave_lds_sync();
    uint64_t x = list.lane < qcount ? queue[list.lane] : 0;
    wave_lds_sync();
    x = sort64_desc(x, list.lane);
    list.merge(x);
    qcount = 0;
    tau = list.at(k - 1);
    if (tau != 0) {
      uint32_t o = static_cast<uint32_t>(tau >> 32);
      uint32_t bits = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
      tau_v = __uint_as_float(bits);
    }
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

template <int SLOTS, bool VEC>
__global__ __launch_bounds__(256) void topk_segment_kernel(
    const float* __restrict__ x, int rows, int V, int k, int nseg, int seg_len,
    uint64_t* __restrict__ seg_keys) {
  __shared__ uint64_t queue[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + wave;
  if (task >= rows * nseg) return;  // whole wave leaves; no block barriers below
  const int row = task / nseg, seg = task - row * nseg;
  const int beg = seg * seg_len;
  const int end = min(V, beg + seg_len);
  const float* p = x + static_cast<size_t>(row) * V;

  WaveSelect<SLOTS> sel;
  sel.init(k, queue[wave], lane);

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
    sel.tau = sel.list.at(k - 1);
    if (sel.tau != 0) {
      const uint32_t o = static_cast<uint32_t>(sel.tau >> 32);
      sel.tau_v = __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool seeded = (u == u1) || (SLOTS > 1 && u == u2);
      const bool ok = e0[u] < end && !seeded && v[u] >= sel.tau_v;
      if (__ballot(ok) == 0) continue;
      sel.offer(ok ? sel_key(v[u], e0[u]) : 0);
    }
  }

  if (VEC) {
    for (int base = beg + 1024; base < end; base += 2048) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int e = base + u * 256 + lane * 4;
        if (e < end) v[u] = *reinterpret_cast<const float4*>(p + e);
        else v[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
      float m = -INFINITY;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        m = fmaxf(m, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
      if (__ballot(m >= sel.tau_v) == 0) continue;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int e = base + u * 256 + lane * 4;
        bool ok = e < end;
        if (__ballot(ok && fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)) >= sel.tau_v) == 0)
          continue;
        sel.offer(ok ? sel_key(v[u].x, e) : 0);
        sel.offer(ok ? sel_key(v[u].y, e + 1) : 0);
        sel.offer(ok ? sel_key(v[u].z, e + 2) : 0);
        sel.offer(ok ? sel_key(v[u].w, e + 3) : 0);
      }
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
      if (__ballot(m >= sel.tau_v) == 0) continue;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        int e = base + u * 64 + lane;
        sel.offer(e < end ? sel_key(v[u], e) : 0);
      }
    }
  }
  sel.finish();
  uint64_t* out = seg_keys + static_cast<size_t>(task) * (64 * SLOTS);
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) out[s * 64 + lane] = sel.list.v[s];
}

// One workgroup per row: the first k keys of every segment list (only they
// can reach the row's top k) are sorted descending in LDS with a bitonic
// network; the first k are the row's top-k.
constexpr int kMergeCap = 4096;  // nseg * k, enforced by topk_plan

__global__ __launch_bounds__(256) void topk_merge_kernel(
    const float* __restrict__ x, int rows, int V, int k, int nseg, int ks,
    const uint64_t* __restrict__ seg_keys, int* __restrict__ out_idx,
    float* __restrict__ out_p) {
  __shared__ uint64_t keys[kMergeCap];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int n = nseg * k;
  int P = 1;
  while (P < n) P <<= 1;
  const uint64_t* src = seg_keys + static_cast<size_t>(row) * nseg * ks;
  for (int i = t; i < P; i += 256) {
    uint64_t v = 0;
    if (i < n) v = src[(i / k) * ks + (i % k)];
    keys[i] = v;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < P / 2; i += 256) {
        const int lo = 2 * i - (i & (stride - 1));   // lower index of the pair
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a < b) == desc) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int pos = t; pos < k; pos += 256) {
    const uint64_t key = keys[pos];
    // every row holds V >= k elements, so the first k slots are filled;
    // the guard keeps an impossible empty slot inside the row
    const uint32_t idx = key ? sel_key_index(key) : 0u;
    out_idx[static_cast<size_t>(row) * k + pos] = static_cast<int>(idx);
    // re-read the element so the stored probability keeps its exact bits
    out_p[static_cast<size_t>(row) * k + pos] = x[static_cast<size_t>(row) * V + idx];
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
  int want = (kScanWaves + rows - 1) / rows;
  int most = V / 4096 > 1 ? V / 4096 : 1;  // segments of at least ~4k elements
  if (most > kMergeCap / k) most = kMergeCap / k;
  int nseg = want < most ? want : most;
  if (nseg < 1) nseg = 1;
  int len = (V + nseg - 1) / nseg;
  len = (len + 1023) / 2048 * 2048 + 1024;  // one warm-up block of 1024, then steps of 2048
  p.seg_len = len;
  p.nseg = (V + len - 1) / len;
  return p;
}

size_t topk_ws_bytes(const TopkPlan& p) {
  return static_cast<size_t>(p.rows) * p.nseg * 64 * p.slots * sizeof(uint64_t);
}

hipError_t launch_topk(const float* x, const TopkPlan& p, uint64_t* seg_keys,
                       int* out_idx, float* out_p, hipStream_t s) {
  int tasks = p.rows * p.nseg;
  dim3 grid((tasks + 3) / 4), block(256);
  if (p.slots == 1) {
    if (p.vec)
      topk_segment_kernel<1, true><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, seg_keys);
    else
      topk_segment_kernel<1, false><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, seg_keys);
  } else {
    if (p.vec)
      topk_segment_kernel<2, true><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, seg_keys);
    else
      topk_segment_kernel<2, false><<<grid, block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, p.seg_len, seg_keys);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_merge_kernel<<<dim3(p.rows), block, 0, s>>>(x, p.rows, p.V, p.k, p.nseg, 64 * p.slots,
                                                   seg_keys, out_idx, out_p);
  return hipGetLastError();
}

}  // namespace tsv
