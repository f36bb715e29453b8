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
// folded to +0; an empty slot is key 0, below every valid key), sorted
// descending by a bitonic network in LDS.  The table entries the walk can
// reach are staged in LDS, and one wavefront walks the sorted keys 64 at a
// time: the lanes fetch the next 64 scores and table entries in parallel, and
// the admission test runs in order in fp64, exactly as
// (tau + a) * SPS(B + 1) > tau * SPS(B), tau accumulated in admission order.
// Admitted keys are then counted per request with LDS atomics.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

constexpr int kSortMax = kMaxGlobalCandidates;

__global__ __launch_bounds__(1024) void global_budget_kernel(GlobalBudgetArgs a) {
  __shared__ uint64_t keys[kSortMax];
  __shared__ double sps_s[kSortMax + 1];
  __shared__ int counts[kMaxGlobalRequests];
  __shared__ int s_admit;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int R = a.B, N = a.N_max;
  const int total = R * N;
  int P2 = 1;
  while (P2 < total) P2 <<= 1;

  for (int i = tid; i < P2; i += nt) {
    uint64_t k = 0;
    if (i < total) {
      const int r = i / N, j = i - r * N;
      const int avail = clampi(a.n_nodes[r], 0, N);
      if (j < avail) {
        const float s = a.score[i];
        const uint32_t bits = s == 0.0f ? 0u : __float_as_uint(s);
        k = (static_cast<uint64_t>(bits) << 32) | (static_cast<uint64_t>(65535 - r) << 16) |
            static_cast<uint64_t>(65535 - j);
      }
    }
    keys[i] = k;
  }
  // the reachable table: B = R + m for m = 0 .. total (entries past the table
  // are never read: the walk stops before them)
  for (int m = tid; m <= total; m += nt) {
    const long idx = static_cast<long>(R) + m;
    sps_s[m] = idx < a.sps_len ? a.sps[idx] : 0.0;
  }
  for (int r = tid; r < R; r += nt) counts[r] = 0;
  __syncthreads();

  // bitonic sort, descending
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P2 / 2; i += nt) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = keys[lo], y = keys[hi];
        if ((x < y) == desc) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  if (tid < 64) {
    const int lane = tid;
    double tau = static_cast<double>(R);
    int m = 0;
    bool go = true;
    for (int i0 = 0; go && i0 < total; i0 += 64) {
      const int i = i0 + lane;
      const uint64_t k = i < total ? keys[i] : 0;
      // before admitting entry i, B = R + i (every earlier entry admitted)
      const double t0 = i < total ? sps_s[i] : 0.0;
      const double t1 = i < total ? sps_s[i + 1] : 0.0;
      const int n_here = min(64, total - i0);
      for (int l = 0; l < n_here; ++l) {
        const uint64_t kl = readlane_u64(k, l);
        if (kl == 0 || static_cast<long>(R) + i0 + l + 1 >= a.sps_len) {
          go = false;
          break;
        }
        const double s = static_cast<double>(__uint_as_float(static_cast<uint32_t>(kl >> 32)));
        const double sp0 = __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, t0), l));
        const double sp1 = __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, t1), l));
        const double tn = __dadd_rn(tau, s);
        if (!(__dmul_rn(tn, sp1) > __dmul_rn(tau, sp0))) {
          go = false;
          break;
        }
        tau = tn;
        ++m;
      }
    }
    if (lane == 0) s_admit = m;
  }
  __syncthreads();
  const int admitted = s_admit;
  for (int i = tid; i < admitted; i += nt) {
    const int r = 65535 - static_cast<int>((keys[i] >> 16) & 0xFFFF);
    atomicAdd(&counts[r], 1);
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
