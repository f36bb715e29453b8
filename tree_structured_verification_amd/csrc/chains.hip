// unfold_chains: a draft tree as its root-to-leaf chains.
//
// [review] "How it works", step 4 (verify preprocess): the tree is unfolded
// into chains (the toy's A-B, A-C, A-B-B becomes A-B-B and A-C) so that the
// prefix's state is shared and everything after the branch point is kept per
// chain; step 6 commits only the accepted chain's state.
//
// One workgroup of 128 threads per request, thread i for node i: node i is a
// leaf if no node names it as parent (flags in LDS); leaves are numbered in
// node order by a ballot prefix count; each leaf walks its parents once to
// find its depth and once more to write the chain root-side first.  Parent
// values outside [-1, i) are read as -1 (a child of the root), so a malformed
// tree cannot make an access leave the documented shapes.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

constexpr int kChainThreads = 128;

__global__ __launch_bounds__(kChainThreads) void unfold_chains_kernel(ChainArgs a) {
  __shared__ int par[kChainThreads];
  __shared__ int has_child[kChainThreads];
  __shared__ int wave_leaves[2];
  const int b = blockIdx.x, i = threadIdx.x;
  const int lane = i & 63, wave = i >> 6;
  const int N = a.N_max;
  const int n = clampi(a.n_nodes[b], 0, N);
  const size_t rb = static_cast<size_t>(b) * N;
  int p = -1;
  if (i < n) {
    p = a.parent[rb + i];
    p = (p >= 0 && p < i) ? p : -1;
  }
  par[i] = p;
  has_child[i] = 0;
  __syncthreads();
  if (i < n && p >= 0) has_child[p] = 1;
  __syncthreads();
  const bool leaf = i < n && has_child[i] == 0;
  const uint64_t mask = __ballot(leaf);
  if (lane == 0) wave_leaves[wave] = __popcll(mask);
  __syncthreads();
  const int before = (wave ? wave_leaves[0] : 0) +
                     __popcll(mask & ((lane ? (~0ull >> (64 - lane)) : 0ull)));
  const int count = wave_leaves[0] + wave_leaves[1];
  const int G = a.gamma;
  int* nodes = a.chain_nodes + rb * G;
  if (leaf) {
    int d = 0;
    for (int j = i; j >= 0; j = par[j]) ++d;
    int pos = d - 1;
    for (int j = i; j >= 0; j = par[j], --pos)
      if (pos < G) nodes[static_cast<size_t>(before) * G + pos] = j;
    const int len = d < G ? d : G;
    a.chain_len[rb + before] = len;
    for (int t = len; t < G; ++t) nodes[static_cast<size_t>(before) * G + t] = -1;
  }
  // places past the last chain
  if (i >= count && i < N) {
    a.chain_len[rb + i] = 0;
    for (int t = 0; t < G; ++t) nodes[static_cast<size_t>(i) * G + t] = -1;
  }
  if (i == 0) a.n_chains[b] = count;
}

}  // namespace

hipError_t launch_unfold_chains(const ChainArgs& a, hipStream_t s) {
  unfold_chains_kernel<<<dim3(a.B), dim3(kChainThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tsv
