// commit_path: write the accepted chain's scratch KV into the persistent cache.
//
// [review] "Secret weapon" (paper section 4.2 as quoted) and "How it works",
// step 6: branch state stays in a scratch pad during verification; once the
// accepted path is known only its rows are written to the persistent cache,
// the rest is dropped, and the prefix grows by the accepted length.
//
// One workgroup per request: validate (device-side sizes), copy at most gamma
// rows of K (and V) with 16-, 4- or 2-byte accesses, then bump the prefix
// length (every thread has read the old one before the first barrier).

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

// Every thread reads the sizes, thread j < gamma accepted node j; then each
// thread copies one element column of up to kCopyBatch accepted rows at a
// time, all its loads issued before its stores, so the copy costs one load
// round trip rather than one per row.
constexpr int kCopyBatch = 16;
// 16-byte element as a plain vector type (an array of HIP's uint4 struct is
// kept in scratch memory by the compiler)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename U>
__global__ __launch_bounds__(256) void commit_kernel(
    char* k_cache, char* v_cache, int* prefix_len, const char* k_tree,
    const char* v_tree, size_t row_bytes, const int* accept_len,
    const int* accept_nodes, int N_max, int L_cap, size_t k_bytes,
    size_t v_bytes, int gamma, int* status) {
  __shared__ int s_nodes[64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int m = accept_len[b];
  const int l = prefix_len[b];
  const int v = tid < gamma ? accept_nodes[static_cast<size_t>(b) * gamma + tid] : 0;
  const bool size_bad = m < 0 || m > gamma || l < 0;
  if (tid < 64) s_nodes[tid] = v;
  // also orders every thread's read of the prefix length before its update
  const bool node_bad = __syncthreads_or(!size_bad && tid < m && (v < 0 || v >= N_max)) != 0;
  const int st = (size_bad || node_bad) ? 2 : (static_cast<long>(l) + m > L_cap ? 1 : 0);
  if (tid == 0) status[b] = st;
  if (st != 0) return;

  const int nk = static_cast<int>(k_bytes / sizeof(U));
  const int nv = v_cache ? static_cast<int>(v_bytes / sizeof(U)) : 0;
  const int per_row = nk + nv;   // a row's elements: K first, then V
  for (int e0 = 0; e0 < per_row; e0 += static_cast<int>(blockDim.x)) {
    const int e = e0 + tid;
    const int ec = min(e, per_row - 1);   // loads past the row re-read its last element
    const bool isk = ec < nk;
    const size_t off = static_cast<size_t>(isk ? ec : ec - nk) * sizeof(U);
    const char* tsrc = (isk ? k_tree : v_tree) + off;
    char* tdst = (isk ? k_cache : v_cache) + off;
    for (int j0 = 0; j0 < m; j0 += kCopyBatch) {
      U val[kCopyBatch];
#pragma unroll
      for (int r = 0; r < kCopyBatch; ++r) {
        const int j = min(j0 + r, m - 1);
        val[r] = *reinterpret_cast<const U*>(tsrc + (static_cast<size_t>(b) * N_max + s_nodes[j]) * row_bytes);
      }
#pragma unroll
      for (int r = 0; r < kCopyBatch; ++r) {
        const int j = j0 + r;
        if (e < per_row && j < m)
          *reinterpret_cast<U*>(tdst + (static_cast<size_t>(b) * L_cap + l + j) * row_bytes) = val[r];
      }
    }
  }
  if (tid == 0) prefix_len[b] = l + m;
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
    commit_kernel<u32x4><<<grid, block, 0, s>>>(kc, vc, prefix_len, kt, vt, row_bytes, accept_len,
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
