// compress_chains / refresh_compressed: per-chain compressed state of the
// verify preprocess and its refresh along the accepted path.
//
// [review] "How it works", steps 4 and 6, and "Secret weapon": after the
// branch point every chain is compressed on its own (one compression over
// two chains would mix histories that exclude each other), the chains'
// temporary compressed tokens and intermediate buffers stay in a scratch
// pad, and after acceptance only the accepted chain's state reaches the
// persistent cache.  The compression itself is a stand-in (the pages give no
// formula for DeepSeek-V4's C4 / C128): entry j of a sequence is the mean of
// the rows of positions j*c .. j*c + c - 1; the intermediate buffer is the
// fp32 sum of the rows of the incomplete last block.
//
// Both kernels give every thread four columns of the rows and walk the
// tokens in sequence order, so each column is accumulated in exactly the
// order of the definition; a chain's rows are loaded eight tokens ahead of
// their additions.  When columns, row stride and buffers allow it, a
// thread's four columns are adjacent and move as one 8-byte (bf16) or
// 16-byte (fp32) load and one 16-byte store; otherwise they are strided by
// the workgroup size.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

constexpr int kCmpThreads = 256;
constexpr int kCmpCols = 4;                           // columns per thread
constexpr int kCmpSlice = kCmpThreads * kCmpCols;     // columns per workgroup
constexpr int kCmpAhead = 8;                          // tokens loaded ahead

template <typename T>
__device__ __forceinline__ float load_col(const T* p);
template <>
__device__ __forceinline__ float load_col<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_col<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// four adjacent columns starting at p (vector path)
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
  const uint2 x = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(x.x << 16);
  v[1] = __uint_as_float(x.x & 0xffff0000u);
  v[2] = __uint_as_float(x.y << 16);
  v[3] = __uint_as_float(x.y & 0xffff0000u);
}

// column k of this thread: adjacent (VEC) or strided by the workgroup size
template <bool VEC>
__device__ __forceinline__ long col_of(int k) {
  return VEC ? static_cast<long>(blockIdx.y) * kCmpSlice + threadIdx.x * kCmpCols + k
             : static_cast<long>(blockIdx.y) * kCmpSlice + threadIdx.x + k * kCmpThreads;
}

// Grid (B * N_max chain slots, column slices).
template <typename T, bool VEC>
__global__ __launch_bounds__(kCmpThreads) void compress_chains_kernel(CompressArgs a) {
  const int N = a.N_max, G = a.gamma;
  const int b = blockIdx.x / N, q = blockIdx.x % N;
  const bool writer = blockIdx.y == 0 && threadIdx.x == 0;
  const size_t slot = static_cast<size_t>(b) * N + q;
  const int nc = clampi(a.n_chains[b], 0, N);
  if (q >= nc) {
    if (writer) a.n_entries[slot] = 0;
    return;
  }
  const int len = clampi(a.chain_len[slot], 0, G);
  const int* nodes = a.chain_nodes + slot * G;
  const long long l = a.prefix_len[b];
  bool bad = l < 0;
  for (int t = 0; t < len; ++t) {
    const int nd = nodes[t];
    bad |= nd < 0 || nd >= N;
  }
  if (bad) {
    if (writer) a.n_entries[slot] = -1;
    return;
  }
  const T* rows = static_cast<const T*>(a.rows);
  const long E = a.E;
  long col[kCmpCols];
  float s[kCmpCols];
#pragma unroll
  for (int k = 0; k < kCmpCols; ++k) {
    col[k] = col_of<VEC>(k);
    s[k] = col[k] < E ? a.tail[static_cast<size_t>(b) * E + col[k]] : 0.f;
  }
  // vector path: E is a multiple of 4, so a thread's columns are all in or all out
  const bool live = col[0] < E;
  const int M = (a.c - 1 + G) / a.c;
  float* out = a.entries + slot * M * E;
  const long long phase = l % a.c;   // tokens already in the prefix's open block
  int j = 0;
  for (int t0 = 0; t0 < len; t0 += kCmpAhead) {
    float v[kCmpAhead][kCmpCols];
#pragma unroll
    for (int u = 0; u < kCmpAhead; ++u) {
      const int t = t0 + u;
      const T* r = rows + (static_cast<size_t>(b) * N + (t < len ? nodes[t] : 0)) * a.row_stride;
      if constexpr (VEC) {
        if (t < len && live) {
          load4(r + col[0], v[u]);
        } else {
#pragma unroll
          for (int k = 0; k < kCmpCols; ++k) v[u][k] = 0.f;
        }
      } else {
#pragma unroll
        for (int k = 0; k < kCmpCols; ++k) v[u][k] = (t < len && col[k] < E) ? load_col<T>(r + col[k]) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kCmpAhead; ++u) {
      const int t = t0 + u;
      if (t >= len) break;
#pragma unroll
      for (int k = 0; k < kCmpCols; ++k) s[k] += v[u][k];
      if ((phase + t + 1) % a.c == 0) {
        float w[kCmpCols];
#pragma unroll
        for (int k = 0; k < kCmpCols; ++k) {
          w[k] = s[k] / static_cast<float>(a.c);
          s[k] = 0.f;
        }
        if constexpr (VEC) {
          if (live)
            *reinterpret_cast<float4*>(out + static_cast<size_t>(j) * E + col[0]) = make_float4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
          for (int k = 0; k < kCmpCols; ++k)
            if (col[k] < E) out[static_cast<size_t>(j) * E + col[k]] = w[k];
        }
        ++j;
      }
    }
  }
  if (writer) a.n_entries[slot] = j;
}

// Grid (B, column slices).
template <typename T>
__global__ __launch_bounds__(kCmpThreads) void refresh_compressed_kernel(RefreshArgs a) {
  __shared__ int s_q;
  const int N = a.N_max, G = a.gamma;
  const int b = blockIdx.x;
  const bool writer = blockIdx.y == 0 && threadIdx.x == 0;
  const int m = a.accept_len[b];
  const long long l = a.prefix_len[b];
  const int* path = a.accept_nodes + static_cast<size_t>(b) * G;
  int status = 0;
  if (m < 0 || m > G || l < 0) status = 2;
  if (status == 0) {
    for (int t = 0; t < m; ++t) {
      const int nd = path[t];
      if (nd < 0 || nd >= N) status = 2;
    }
  }
  // the lowest-numbered chain whose node m - 1 is the last accepted node
  if (threadIdx.x == 0) s_q = 0x7fffffff;
  __syncthreads();
  const int nc = clampi(a.n_chains[b], 0, N);
  if (status == 0 && m > 0 && static_cast<int>(threadIdx.x) < nc) {
    const size_t slot = static_cast<size_t>(b) * N + threadIdx.x;
    if (a.chain_len[slot] >= m && a.chain_nodes[slot * G + (m - 1)] == path[m - 1])
      atomicMin(&s_q, static_cast<int>(threadIdx.x));
  }
  __syncthreads();
  const int q = s_q;
  if (status == 0 && m > 0 && q == 0x7fffffff) status = 2;
  const int c = a.c;
  const long long e = status == 0 ? (l % c + m) / c : 0;
  if (status == 0 && l / c + e > a.Lc_cap) status = 1;
  if (writer) a.status[b] = status;
  if (status != 0 || m == 0) return;

  const long E = a.E;
  const int M = (c - 1 + G) / c;
  const float* src = a.entries + (static_cast<size_t>(b) * N + q) * M * E;
  float* dst = a.comp + (static_cast<size_t>(b) * a.Lc_cap + l / c) * E;
  const T* rows = static_cast<const T*>(a.rows);
  const int first = e == 0 ? 0 : static_cast<int>(m - (l + m) % c);
#pragma unroll
  for (int k = 0; k < kCmpCols; ++k) {
    const long col = static_cast<long>(blockIdx.y) * kCmpSlice + threadIdx.x + k * kCmpThreads;
    if (col >= E) continue;
    for (long long jj = 0; jj < e; ++jj) dst[jj * E + col] = src[jj * E + col];
    float s = e == 0 ? a.tail[static_cast<size_t>(b) * E + col] : 0.f;
    for (int t = first; t < m; ++t)
      s += load_col<T>(rows + (static_cast<size_t>(b) * N + path[t]) * a.row_stride + col);
    a.tail[static_cast<size_t>(b) * E + col] = s;
  }
}

}  // namespace

hipError_t launch_compress_chains(const CompressArgs& a, int dtype, bool vec, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * a.N_max,
                  static_cast<unsigned>((a.E + kCmpSlice - 1) / kCmpSlice));
  if (dtype == TSV_F32) {
    if (vec) compress_chains_kernel<float, true><<<grid, dim3(kCmpThreads), 0, s>>>(a);
    else compress_chains_kernel<float, false><<<grid, dim3(kCmpThreads), 0, s>>>(a);
  } else {
    if (vec) compress_chains_kernel<uint16_t, true><<<grid, dim3(kCmpThreads), 0, s>>>(a);
    else compress_chains_kernel<uint16_t, false><<<grid, dim3(kCmpThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_refresh_compressed(const RefreshArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B), static_cast<unsigned>((a.E + kCmpSlice - 1) / kCmpSlice));
  if (dtype == TSV_F32)
    refresh_compressed_kernel<float><<<grid, dim3(kCmpThreads), 0, s>>>(a);
  else
    refresh_compressed_kernel<uint16_t><<<grid, dim3(kCmpThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tsv
