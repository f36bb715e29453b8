// select_global_budget: batch-global admission of draft-tree nodes.
//
// [dspark] Confidence-scheduled verification, hardware-aware prefix
// scheduler: verification lengths are chosen by one global throughput
// maximisation over the active requests, Theta = tau * SPS(B), with SPS a
// steps-per-second table profiled once; since each request's survival
// probabilities do not increase along its order, a global sort and greedy
// admission respects every request's prefix order, and admission stops as
// soon as the throughput would fall (early stopping).
//
// Applied to trees: a request's candidates are its build_tree nodes in
// best-first order, a_{r,j} their prefix probabilities; tau = R + admitted
// scores, B = R + admitted nodes; the global order is score descending, then
// request, then position ascending.
//
// One workgroup.  Every (request, position) is one 64-bit key
//   score bits << 32 | (65535 - request) << 16 | (65535 - position)
// (scores are non-negative, so their bits order like the values; -0 is
// folded to +0; 0 = nothing left), so the admission order is descending key
// order.  Each request's candidates are already in that order, so the walk
// is a k-way merge: wavefront lane l holds the best remaining key of the
// requests l, l + 64, ...; the wave maximum (VALU lane exchanges) is the
// next candidate; after an admission the owning lane moves that request's
// head one place and refreshes its maximum (from registers, with the next
// score read ahead, when there is one request per lane).  The cost is proportional to the admitted count,
// not to the number of candidates.  Scores and the reachable part of the
// table sit in LDS; the admission test is
// (tau + a) * SPS(B + 1) > tau * SPS(B) in fp64, tau summed in admission order.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

constexpr int kWave = 64;
constexpr int kBatch = 8;

__device__ __forceinline__ uint64_t cand_key(float s, int r, int j) {
  const uint32_t bits = s == 0.0f ? 0u : __float_as_uint(s);
  return (static_cast<uint64_t>(bits) << 32) | (static_cast<uint64_t>(65535 - r) << 16) |
         static_cast<uint64_t>(65535 - j);
}

__device__ __forceinline__ uint64_t max_u64(uint32_t lo, uint32_t hi, uint32_t lo2, uint32_t hi2) {
  const uint64_t a = (static_cast<uint64_t>(hi) << 32) | lo;
  const uint64_t b = (static_cast<uint64_t>(hi2) << 32) | lo2;
  return a > b ? a : b;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  const uint32_t lo2 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(lo), static_cast<int>(lo), CTRL, 0xF, 0xF, false));
  const uint32_t hi2 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(hi), static_cast<int>(hi), CTRL, 0xF, 0xF, false));
  return max_u64(lo, hi, lo2, hi2);
}

// Maximum over the 64 lanes, in every lane, with VALU lane exchanges only:
// lanes l and l ^ 32 (permlane32 swap), l and l ^ 16 (permlane16 swap), then
// within each row of 16: quad exchanges (xor 1, xor 2), half-row mirror and
// row mirror.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  {
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    v = max_u64(pl[0], ph[0], pl[1], ph[1]);
  }
  {
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    v = max_u64(pl[0], ph[0], pl[1], ph[1]);
  }
  v = dpp_max_u64<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_max_u64<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_max_u64<0x141>(v);   // row_half_mirror
  v = dpp_max_u64<0x140>(v);   // row_mirror
  return v;
}

__global__ __launch_bounds__(1024) void global_budget_kernel(GlobalBudgetArgs a) {
  __shared__ float sc[kMaxGlobalCandidates];
  __shared__ double sps_s[kMaxGlobalCandidates + 1];
  __shared__ int avail_s[kMaxGlobalRequests];
  __shared__ int counts[kMaxGlobalRequests];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int R = a.B, N = a.N_max;
  const int total = R * N;
  // staged in batches of kBatch independent loads per thread, so that a
  // batch costs one memory round trip
  for (int base = 0; base < total; base += nt * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * nt + tid;
      v[u] = i < total ? a.score[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * nt + tid;
      if (i < total) sc[i] = v[u];
    }
  }
  // the reachable table: B = R + m for m = 0 .. total
  for (int base = 0; base <= total; base += nt * kBatch) {
    double v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int m = base + u * nt + tid;
      const long idx = static_cast<long>(R) + m;
      v[u] = (m <= total && idx < a.sps_len) ? a.sps[idx] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int m = base + u * nt + tid;
      if (m <= total) sps_s[m] = v[u];
    }
  }
  for (int base = 0; base < R; base += nt * kBatch) {
    int v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int r = base + u * nt + tid;
      v[u] = r < R ? a.n_nodes[r] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int r = base + u * nt + tid;
      if (r < R) {
        avail_s[r] = clampi(v[u], 0, N);
        counts[r] = 0;
      }
    }
  }
  __syncthreads();

  if (tid < kWave && R <= kWave) {
    // one request per lane: its head position and the score after the head
    // stay in registers, the next score is read ahead
    const int lane = tid;
    const int r = lane;
    const int av = r < R ? avail_s[r] : 0;
    int j = 0;
    uint64_t mine = av > 0 ? cand_key(sc[r * N], r, 0) : 0;
    float nxt = av > 1 ? sc[r * N + 1] : 0.0f;
    double tau = static_cast<double>(R);
    for (int m = 0; m < total; ++m) {
      const uint64_t k = wave_max_u64(mine);
      if (k == 0 || static_cast<long>(R) + m + 1 >= a.sps_len) break;
      const double s = static_cast<double>(__uint_as_float(static_cast<uint32_t>(k >> 32)));
      const double tn = __dadd_rn(tau, s);
      if (!(__dmul_rn(tn, sps_s[m + 1]) > __dmul_rn(tau, sps_s[m]))) break;
      tau = tn;
      if (65535 - static_cast<int>((k >> 16) & 0xFFFF) == r) {
        ++j;
        mine = j < av ? cand_key(nxt, r, j) : 0;
        nxt = j + 1 < av ? sc[r * N + j + 1] : 0.0f;
      }
    }
    if (r < R) counts[r] = j;
  } else if (tid < kWave) {
    const int lane = tid;
    // best remaining key over this lane's requests
    auto lane_best = [&]() {
      uint64_t best = 0;
      for (int r = lane; r < R; r += kWave) {
        const int j = counts[r];
        if (j < avail_s[r]) {
          const uint64_t k = cand_key(sc[r * N + j], r, j);
          best = k > best ? k : best;
        }
      }
      return best;
    };
    uint64_t mine = lane_best();
    double tau = static_cast<double>(R);
    for (int m = 0; m < total; ++m) {
      const uint64_t k = wave_max_u64(mine);
      if (k == 0 || static_cast<long>(R) + m + 1 >= a.sps_len) break;
      const double s = static_cast<double>(__uint_as_float(static_cast<uint32_t>(k >> 32)));
      const double tn = __dadd_rn(tau, s);
      if (!(__dmul_rn(tn, sps_s[m + 1]) > __dmul_rn(tau, sps_s[m]))) break;
      tau = tn;
      const int r = 65535 - static_cast<int>((k >> 16) & 0xFFFF);
      if ((r & (kWave - 1)) == lane) {
        counts[r] += 1;
        mine = lane_best();
      }
    }
  }
  __syncthreads();
  // admitted counts, and build_tree's padding past them
  const int W = (N + 31) >> 5;
  for (int r = tid; r < R; r += nt) a.n_nodes[r] = counts[r];
  for (int i = tid; i < total; i += nt) {
    const int r = i / N, j = i - r * N;
    if (j >= counts[r]) {
      a.parent[i] = -1;
      a.token[i] = -1;
      a.depth[i] = -1;
      a.score[i] = 0.0f;
      for (int w = 0; w < W; ++w) a.anc_bits[static_cast<size_t>(i) * W + w] = 0u;
    }
  }
}

}  // namespace

hipError_t launch_global_budget(const GlobalBudgetArgs& a, hipStream_t s) {
  global_budget_kernel<<<dim3(1), dim3(1024), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tsv
