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
struct Vec16;  // 16 bytes of T, widened to fp32
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void widen(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
  __device__ static float one(const float* p) { return *p; }
};
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void widen(const uint4& v, float* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // exact widening of the two halves
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static float one(const uint16_t* p) { return bf16_to_f32(*p); }
};

// One wavefront per (verified row, segment): the first maximum of the slice.
// Vector path: a lane visits its 16-byte groups in increasing index order and
// keeps only its running maximum and the first group where that maximum rose
// (strict comparison, so ties stay with the earlier group); the first element
// of that group equal to the maximum is found once at the end.  Ties across
// lanes are settled by the key (lower index).
constexpr int kMinSegments = 8;

// Workgroups of one argmax launch at most: about what the compute units hold
// at once (five of these workgroups per CU at the kernel's register use), so
// that every task a wave steps to is taken without waiting for a later
// workgroup's dispatch.
constexpr int kArgmaxGrid = 1280;
constexpr int kArgmaxStagedB = 1024;   // requests whose node counts go to LDS

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void argmax_segment_kernel(
    const T* __restrict__ logits, int B, int N_max, int V, int nseg, int seg_len,
    const int* __restrict__ n_nodes, uint64_t* __restrict__ seg_best) {
  __shared__ int s_n[kArgmaxStagedB];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows_per_b = N_max + 1;
  const int tasks = B * rows_per_b * nseg;
  // node counts staged once per workgroup (a task then skips without a
  // global round trip); larger batches read them per task
  const bool staged = B <= kArgmaxStagedB;
  if (staged)
    for (int i = threadIdx.x; i < B; i += blockDim.x) s_n[i] = clampi(n_nodes[i], 0, N_max);
  __syncthreads();
  // the grid holds at most kArgmaxGrid workgroups: a wave takes tasks
  // task, task + 4 * gridDim.x, ... (rows past a request's node count are
  // skipped in a few instructions, so small trees cost no dispatch); task =
  // (b * rows_per_b + r) * nseg + seg, decoded once and then advanced by the
  // stride's own (request, row, segment) steps with carries
  const int t0 = blockIdx.x * 4 + wave, S = gridDim.x * 4;
  int seg = t0 % nseg, r = (t0 / nseg) % rows_per_b, b = (t0 / nseg) / rows_per_b;
  const int dseg = S % nseg, drow = S / nseg, dr = drow % rows_per_b, db = drow / rows_per_b;
  for (int task = t0; task < tasks; task += S) {
    const int cb = b, cr = r, cs = seg;   // this task
    seg += dseg;                          // the wave's next task
    const int c1 = seg >= nseg ? 1 : 0;
    seg -= c1 * nseg;
    r += dr + c1;
    const int c2 = r >= rows_per_b ? 1 : 0;
    r -= c2 * rows_per_b;
    b += db + c2;
    const int n = staged ? s_n[cb] : clampi(n_nodes[cb], 0, N_max);
    if (cr > n) continue;  // row never read by the walk
    const int row = cb * rows_per_b + cr;
    const int beg = cs * seg_len;
    const int end = min(V, beg + seg_len);
    const T* p = logits + static_cast<size_t>(row) * V;

    float bv = -INFINITY;
    int bi = -1;
    if (VEC) {
      constexpr int N = Vec16<T>::N;
      constexpr int STEP = 64 * N;
      constexpr int BLK = 8 * STEP;  // elements per block of 8 loads per lane
      int bg = -1;  // first element of the group holding this lane's maximum
      // groups lie wholly inside or outside [beg, end) (V and the segment
      // bounds are multiples of N); a group past the end re-reads the last
      // group of the slice and is then ignored, so every load is in bounds and
      // unconditional
      auto load_block = [&](uint4 (&raw)[8], int base) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = min(base + u * STEP + lane * N, end - N);
          raw[u] = *reinterpret_cast<const uint4*>(p + e);
        }
      };
      auto process = [&](const uint4 (&raw)[8], int base) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float v[N];
          Vec16<T>::widen(raw[u], v);
          float m = vmax3(v[0], v[1], v[2]);
#pragma unroll
          for (int c = 3; c < N; c += 2) m = vmax3(m, v[c], v[c + 1 < N ? c + 1 : c]);
          const int e = base + u * STEP + lane * N;
          const bool up = e < end && m > bv;
          bv = up ? m : bv;
          bg = up ? e : bg;
        }
      };
      // two register blocks in turn: one in flight while the other is scanned
      uint4 b0[8], b1[8];
      load_block(b0, beg);
      for (int base = beg; base < end; base += 2 * BLK) {
        if (base + BLK < end) load_block(b1, base + BLK);
        process(b0, base);
        if (base + BLK >= end) break;
        if (base + 2 * BLK < end) load_block(b0, base + 2 * BLK);
        process(b1, base + BLK);
      }
      if (bg >= 0) {
        float w[N];
        Vec16<T>::widen(*reinterpret_cast<const uint4*>(p + bg), w);
#pragma unroll
        for (int c = N - 1; c >= 0; --c) bi = (w[c] == bv) ? bg + c : bi;
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
}

__global__ __launch_bounds__(64) void walk_kernel(
    const uint64_t* __restrict__ seg_best, int nseg, int N_max, int gamma,
    const int* __restrict__ n_nodes, const int* __restrict__ parent,
    const int* __restrict__ token, int* __restrict__ accept_len,
    int* __restrict__ accept_nodes, int* __restrict__ out_tokens) {
  __shared__ int s_arg[129];
  __shared__ int s_tok[128];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = clampi(n_nodes[b], 0, N_max);
  const int rows_per_b = N_max + 1;
  // every load of this lane in flight together with the node count: the
  // tree (at most 128 nodes, two per lane) and the first eight segment keys
  // of the lane's first row (usually all of them: the walk then waits once),
  // all addressed within the request's N_max nodes and N_max + 1 rows, the
  // node count applied afterwards
  int par2[2], tok2[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    par2[h] = i < N_max ? parent[static_cast<size_t>(b) * N_max + i] : 0;
    tok2[h] = i < N_max ? token[static_cast<size_t>(b) * N_max + i] : 0;
  }
  uint64_t v0[8];
  const uint64_t* src0 = seg_best + (static_cast<size_t>(b) * rows_per_b + lane) * nseg;
#pragma unroll
  for (int u = 0; u < 8; ++u) v0[u] = lane <= N_max && u < nseg ? src0[u] : 0;
  int arg0 = -1;   // the argmax of row `lane` (rows 64.. go through LDS)
  for (int r = lane; r <= n; r += 64) {
    const uint64_t* src = seg_best + (static_cast<size_t>(b) * rows_per_b + r) * nseg;
    uint64_t best = 0;
    for (int s0 = 0; s0 < nseg; s0 += 8) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = r == lane && s0 == 0 ? v0[u] : (s0 + u < nseg ? src[s0 + u] : 0);
#pragma unroll
      for (int u = 0; u < 8; ++u) best = umax64(best, v[u]);
    }
    const int arg = best ? static_cast<int>(sel_key_index(best)) : -1;
    if (r == lane) arg0 = arg;
    s_arg[r] = arg;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = lane + 64 * h;
    if (i < n) s_tok[i] = tok2[h];
  }
  __syncthreads();

  // each step: the child of the current node whose token is the argmax of
  // the current node's row (lane i holds nodes i and i + 64 in registers)
  const bool in0 = lane < n, in1 = lane + 64 < n;
  int cur = -1, m = 0, mine = -1;
  while (m < gamma) {
    const int want = cur + 1 < 64 ? __builtin_amdgcn_readlane(arg0, cur + 1) : s_arg[cur + 1];
    const bool h0 = in0 && par2[0] == cur && tok2[0] == want;
    const bool h1 = in1 && par2[1] == cur && tok2[1] == want;
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
  // enough waves when every row is read, and at least kMinSegments per row:
  // the rows read are only those of each request's nodes (device-side
  // counts), which may be far fewer than the rows the plan covers, and the
  // waves of unread rows' segments end at once
  int want = (kScanWaves + rows - 1) / rows;
  want = want > kMinSegments ? want : kMinSegments;
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
  const int wgs = (tasks + 3) / 4;
  dim3 grid(wgs < kArgmaxGrid ? wgs : kArgmaxGrid), block(256);
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
