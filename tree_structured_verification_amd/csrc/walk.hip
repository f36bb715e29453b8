// accept_walk: greedy acceptance of the longest matching root-to-node path.
//
// [review] "How it works", steps 5-6, and [dspark] decoding cycle: the target
// scores every branch in one pass; the accepted tokens are the longest path
// from the root whose every token equals the target's argmax at its parent,
// then the target's own next token.
//
// Kernel 1 (HBM-bound scan): one wavefront per (verified row, segment) keeps
// the first maximum of its slice; rows beyond 1 + n_b are skipped.
// Kernel 2: one wavefront per request reduces the segments of its rows and
// walks at most gamma steps down the tree.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* out) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  __device__ static float one(const float* p) { return *p; }
};
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* out) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static float one(const uint16_t* p) { return bf16_to_f32(*p); }
};

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void argmax_segment_kernel(
    const T* __restrict__ logits, int B, int N_max, int V, int nseg, int seg_len,
    const int* __restrict__ n_nodes, uint64_t* __restrict__ seg_best) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows_per_b = N_max + 1;
  const int task = blockIdx.x * 4 + wave;
  if (task >= B * rows_per_b * nseg) return;
  const int row = task / nseg, seg = task - row * nseg;
  const int b = row / rows_per_b, r = row - b * rows_per_b;
  const int n = clampi(n_nodes[b], 0, N_max);
  if (r > n) return;  // row never read by the walk
  const int beg = seg * seg_len;
  const int end = min(V, beg + seg_len);
  const T* p = logits + static_cast<size_t>(row) * V;

  // each lane visits its elements in increasing index order and keeps the
  // first maximum; ties across lanes are settled by the key (lower index)
  float bv = -INFINITY;
  int bi = -1;
  if (VEC) {
    constexpr int N = Vec16<T>::N;
    constexpr int STEP = 64 * N;
    for (int base = beg; base < end; base += 8 * STEP) {
      float v[8][N];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int e = base + u * STEP + lane * N;
        if (e < end) Vec16<T>::load(p + e, v[u]);
        else {
#pragma unroll
          for (int c = 0; c < N; ++c) v[u][c] = -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int e = base + u * STEP + lane * N;
#pragma unroll
        for (int c = 0; c < N; ++c) {
          bool better = (e + c < end) && (v[u][c] > bv || bi < 0);
          bv = better ? v[u][c] : bv;
          bi = better ? e + c : bi;
        }
      }
    }
  } else {
    for (int e = beg + lane; e < end; e += 64) {
      float v = Vec16<T>::one(p + e);
      bool better = v > bv || bi < 0;
      bv = better ? v : bv;
      bi = better ? e : bi;
    }
  }
  uint64_t key = bi < 0 ? 0 : sel_key(bv, static_cast<uint32_t>(bi));
  key = wave_max_u64(key);
  if (lane == 0) seg_best[task] = key;
}

__global__ __launch_bounds__(64) void walk_kernel(
    const uint64_t* __restrict__ seg_best, int nseg, int N_max, int gamma,
    const int* __restrict__ n_nodes, const int* __restrict__ parent,
    const int* __restrict__ token, int* __restrict__ accept_len,
    int* __restrict__ accept_nodes, int* __restrict__ out_tokens) {
  __shared__ int s_arg[129];
  __shared__ int s_par[128], s_tok[128];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = clampi(n_nodes[b], 0, N_max);
  const int rows_per_b = N_max + 1;
  for (int r = lane; r <= n; r += 64) {
    const uint64_t* src = seg_best + (static_cast<size_t>(b) * rows_per_b + r) * nseg;
    uint64_t best = 0;
    for (int s = 0; s < nseg; ++s) best = umax64(best, src[s]);
    s_arg[r] = best ? static_cast<int>(sel_key_index(best)) : -1;
  }
  for (int i = lane; i < n; i += 64) {
    s_par[i] = parent[static_cast<size_t>(b) * N_max + i];
    s_tok[i] = token[static_cast<size_t>(b) * N_max + i];
  }
  __syncthreads();

  int cur = -1, m = 0, mine = -1;
  while (m < gamma) {
    const int want = s_arg[cur + 1];
    const bool h0 = lane < n && s_par[lane] == cur && s_tok[lane] == want;
    const bool h1 = lane + 64 < n && s_par[lane + 64] == cur && s_tok[lane + 64] == want;
    const uint64_t m0 = __ballot(h0), m1 = __ballot(h1);
    int j = -1;
    if (m0) j = __ffsll(static_cast<long long>(m0)) - 1;
    else if (m1) j = 64 + __ffsll(static_cast<long long>(m1)) - 1;
    if (j < 0) break;
    if (lane == m) mine = j;
    cur = j;
    ++m;
  }
  const int bonus = s_arg[cur + 1];
  if (lane == 0) accept_len[b] = m;
  const size_t an = static_cast<size_t>(b) * gamma;
  const size_t ot = static_cast<size_t>(b) * (gamma + 1);
  if (lane < gamma) {
    accept_nodes[an + lane] = lane < m ? mine : -1;
    out_tokens[ot + lane] = lane < m ? s_tok[mine] : (lane == m ? bonus : -1);
  }
  if (lane == 0) out_tokens[ot + gamma] = (m == gamma) ? bonus : -1;
}

}  // namespace

ArgmaxPlan argmax_plan(int rows, int V, int dtype) {
  ArgmaxPlan p;
  p.rows = rows;
  p.V = V;
  const int per16 = dtype == TSV_F32 ? 4 : 8;
  p.vec = (V % per16) == 0;
  int want = (kScanWaves + rows - 1) / rows;
  int most = V / 4096 > 1 ? V / 4096 : 1;
  int nseg = want < most ? want : most;
  if (nseg < 1) nseg = 1;
  int len = (V + nseg - 1) / nseg;
  len = (len + 2047) / 2048 * 2048;
  p.seg_len = len;
  p.nseg = (V + len - 1) / len;
  return p;
}

hipError_t launch_accept_walk(const void* logits, int dtype, int B, int N_max,
                              int V, int gamma, const int* n_nodes,
                              const int* parent, const int* token,
                              int* accept_len, int* accept_nodes,
                              int* out_tokens, uint64_t* seg_best,
                              const ArgmaxPlan& p, hipStream_t s) {
  const int tasks = B * (N_max + 1) * p.nseg;
  dim3 grid((tasks + 3) / 4), block(256);
  if (dtype == TSV_F32) {
    if (p.vec)
      argmax_segment_kernel<float, true><<<grid, block, 0, s>>>(
          static_cast<const float*>(logits), B, N_max, V, p.nseg, p.seg_len, n_nodes, seg_best);
    else
      argmax_segment_kernel<float, false><<<grid, block, 0, s>>>(
          static_cast<const float*>(logits), B, N_max, V, p.nseg, p.seg_len, n_nodes, seg_best);
  } else {
    if (p.vec)
      argmax_segment_kernel<uint16_t, true><<<grid, block, 0, s>>>(
          static_cast<const uint16_t*>(logits), B, N_max, V, p.nseg, p.seg_len, n_nodes, seg_best);
    else
      argmax_segment_kernel<uint16_t, false><<<grid, block, 0, s>>>(
          static_cast<const uint16_t*>(logits), B, N_max, V, p.nseg, p.seg_len, n_nodes, seg_best);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  walk_kernel<<<dim3(B), dim3(64), 0, s>>>(seg_best, p.nseg, N_max, gamma, n_nodes,
                                            parent, token, accept_len, accept_nodes,
                                            out_tokens);
  return hipGetLastError();
}

}  // namespace tsv
