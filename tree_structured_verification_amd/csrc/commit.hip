// commit_path: write the accepted chain's scratch KV into the persistent cache.
//
// [review] "Secret weapon" (paper section 4.2 as quoted) and "How it works",
// step 6: branch state stays in a scratch pad during verification; once the
// accepted path is known only its rows are written to the persistent cache,
// the rest is dropped, and the prefix grows by the accepted length.
//
// One workgroup per request: validate (device-side sizes), copy at most gamma
// rows of K (and V) with 16-, 4- or 2-byte accesses, then bump the prefix
// length after every thread has read the old one.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

template <typename U>
__device__ void copy_row(char* dst, const char* src, size_t bytes) {
  U* d = reinterpret_cast<U*>(dst);
  const U* s = reinterpret_cast<const U*>(src);
  const size_t n = bytes / sizeof(U);
  for (size_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

template <typename U>
__global__ __launch_bounds__(256) void commit_kernel(
    char* k_cache, char* v_cache, int* prefix_len, const char* k_tree,
    const char* v_tree, size_t row_bytes, const int* accept_len,
    const int* accept_nodes, int N_max, int L_cap, size_t k_bytes,
    size_t v_bytes, int gamma, int* status) {
  __shared__ int s_nodes[64];
  __shared__ int s_state, s_l, s_m;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    const int m = accept_len[b];
    const int l = prefix_len[b];
    int st = 0;
    if (m < 0 || m > gamma || l < 0) {
      st = 2;
    } else {
      for (int j = 0; j < m; ++j) {
        const int v = accept_nodes[static_cast<size_t>(b) * gamma + j];
        if (v < 0 || v >= N_max) st = 2;
        s_nodes[j] = v;
      }
      if (st == 0 && static_cast<long>(l) + m > L_cap) st = 1;
    }
    s_state = st;
    s_l = l;
    s_m = m;
    status[b] = st;
  }
  __syncthreads();
  if (s_state != 0) return;
  const int l = s_l, m = s_m;
  for (int j = 0; j < m; ++j) {
    const size_t src = (static_cast<size_t>(b) * N_max + s_nodes[j]) * row_bytes;
    const size_t dst = (static_cast<size_t>(b) * L_cap + l + j) * row_bytes;
    copy_row<U>(k_cache + dst, k_tree + src, k_bytes);
    if (v_cache) copy_row<U>(v_cache + dst, v_tree + src, v_bytes);
  }
  __syncthreads();
  if (threadIdx.x == 0) prefix_len[b] = l + m;
}

}  // namespace

hipError_t launch_commit(void* k_cache, void* v_cache, int* prefix_len,
                         const void* k_tree, const void* v_tree,
                         size_t row_bytes, const int* accept_len,
                         const int* accept_nodes, int B, int N_max, int L_cap,
                         size_t k_bytes, size_t v_bytes, int gamma,
                         int* status, hipStream_t s) {
  auto addr_ok = [](const void* p, size_t a) {
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0;
  };
  auto fits = [&](size_t a) {
    return row_bytes % a == 0 && k_bytes % a == 0 && v_bytes % a == 0 &&
           addr_ok(k_cache, a) && addr_ok(v_cache, a) && addr_ok(k_tree, a) &&
           addr_ok(v_tree, a);
  };
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  const char* kt = static_cast<const char*>(k_tree);
  const char* vt = static_cast<const char*>(v_tree);
  dim3 grid(B), block(256);
  if (fits(16))
    commit_kernel<uint4><<<grid, block, 0, s>>>(kc, vc, prefix_len, kt, vt, row_bytes, accept_len,
                                                accept_nodes, N_max, L_cap, k_bytes, v_bytes, gamma, status);
  else if (fits(4))
    commit_kernel<uint32_t><<<grid, block, 0, s>>>(kc, vc, prefix_len, kt, vt, row_bytes, accept_len,
                                                   accept_nodes, N_max, L_cap, k_bytes, v_bytes, gamma, status);
  else
    commit_kernel<uint16_t><<<grid, block, 0, s>>>(kc, vc, prefix_len, kt, vt, row_bytes, accept_len,
                                                   accept_nodes, N_max, L_cap, k_bytes, v_bytes, gamma, status);
  return hipGetLastError();
}

}  // namespace tsv
