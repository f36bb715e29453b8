// tree_verify_attn: branch-aware tree attention over a shared prefix.
//
// [review] Difficulty 1 (paper section 3.1) and "How it works", step 3: a tree
// node attends to the persistent prefix and to its own ancestors in the
// scratch pad, never to another branch.  Section 6 as quoted: with dense
// attention the tree is a mask over the shared KV -- here, per-node ancestor
// bitsets applied to the scratch keys of the last tiles.
//
// Work decomposition (all on the device, no host round-trip): a query row is
// (node, query head); the rows of one request that share a KV head form
// "units" of RB rows; a unit's keys are the virtual sequence prefix[0, l_b)
// ++ scratch[0, n_b), cut into chunks (split-K); a work item is (unit, chunk)
// and keeps an online softmax per row in fp32.  Three paths:
//   * grouped bf16 heads of width 128: one kernel whose workgroups decode
//     their item from their id, stream K/V tiles by LDS-DMA and combine the
//     splits of a unit themselves (the last one to arrive);
//   * one latent head whose value is the start of the key row (576/512):
//     128-row items, one K tile in LDS feeding both products, behind a
//     one-workgroup planner (item list) and a combine kernel;
//   * every other shape and fp32: a VALU kernel with the same planner and
//     combine.
// The MFMA paths compute the score tile transposed (keys x rows), so that
// its output layout is directly the B operand of the value product
// (v_mfma_f32_16x16x32_bf16), and read the value operand with
// ds_read_b64_tr_b16 from rows in their natural layout.

#include "tsv_device.hpp"
#include "tsv_internal.hpp"

namespace tsv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kValuRows = 16;
constexpr int kValuKeys = 16;
constexpr int kValuMaxD = 576;
constexpr float kLazy = 8.0f;  // lazy-rescale threshold, log2 units
// grouped path: a split's published rows, 128 rows x 128 bf16, in floats
constexpr size_t kGqaPartFloats = 128 * 128 / 2;
// grouped path: at least one split per this many keys of a unit
constexpr long long kSplitKeys = 4096;

// Whether virtual key `key` is visible to a row whose node has ancestor words
// w[0..3]: prefix keys always, scratch keys iff their bit is set, nothing at or
// past k_end.  Written without short-circuit operators so that it compiles to
// selects rather than nested EXEC-masked branches.
__device__ __forceinline__ bool key_visible(const uint32_t* w, int key, int l_b, int k_end) {
  int j = key - l_b;
  j = j < 0 ? 0 : (j > 127 ? 127 : j);
  const uint32_t lo = (j < 32) ? w[0] : w[1];
  const uint32_t hi = (j < 96) ? w[2] : w[3];
  const uint32_t word = (j < 64) ? lo : hi;
  const int bit = static_cast<int>((word >> (j & 31)) & 1u);
  const int vis = static_cast<int>(key < l_b) | bit;
  return (static_cast<int>(key < k_end) & vis) != 0;
}

// ---------------------------------------------------------------- planner
// One workgroup of 1024 threads: per-request work, the split size, an
// exclusive scan of the item counts (request table kept in LDS), then every
// thread writes descriptors for its share of items, locating each item's
// request by binary search over the scanned bases.
constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxB = 4096;

__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(AttnArgs a) {
  __shared__ int s_base[kPlanMaxB + 1];
  __shared__ int s_splits[kPlanMaxB];
  __shared__ int s_rb[kPlanMaxB];
  __shared__ long long s_red[kPlanThreads / 64];
  __shared__ int s_scan[kPlanThreads];
  __shared__ int s_chunk;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int per = (a.B + kPlanThreads - 1) / kPlanThreads;   // requests per thread (<= 4)
  const int b0 = min(a.B, t * per), b1 = min(a.B, b0 + per);

  long long w = 0;
  for (int b = b0; b < b1; ++b) {
    const int n = clampi(a.n_nodes[b], 0, a.N_max);
    const int l = clampi(a.prefix_len[b], 0, a.L_cap);
    const int rb = n > 0 ? (n * a.G + a.RB - 1) / a.RB : 0;
    s_rb[b] = rb;
    s_splits[b] = l;   // prefix length parked here until the split size is known
    w += static_cast<long long>(a.Hkv) * rb * (l + n);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) w += __shfl_xor(w, m);
  if (lane == 0) s_red[wave] = w;
  __syncthreads();
  if (t == 0) {
    long long W = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) W += s_red[i];
    long long c = (W + a.target_items - 1) / a.target_items;
    if (c < a.min_chunk) c = a.min_chunk;
    c = (c + a.KT - 1) / a.KT * a.KT;
    if (c > (1LL << 30)) c = 1LL << 30;
    s_chunk = static_cast<int>(c);
  }
  __syncthreads();
  const int chunk = s_chunk;
  int items = 0;
  for (int b = b0; b < b1; ++b) {
    const int n = clampi(a.n_nodes[b], 0, a.N_max);
    const int l = s_splits[b];
    const int splits = n > 0 ? (l + n + chunk - 1) / chunk : 0;
    a.info[4 * b + 1] = splits;
    a.info[4 * b + 2] = s_rb[b];
    a.info[4 * b + 3] = l;
    s_splits[b] = splits;
    items += a.Hkv * s_rb[b] * splits;
  }
  s_scan[t] = items;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int v = t >= off ? s_scan[t - off] : 0;
    __syncthreads();
    s_scan[t] += v;
    __syncthreads();
  }
  int base = s_scan[t] - items;
  for (int b = b0; b < b1; ++b) {
    s_base[b] = base;
    a.info[4 * b + 0] = base;
    base += a.Hkv * s_rb[b] * s_splits[b];
  }
  const int total = min(s_scan[kPlanThreads - 1], a.items_max);
  if (t == 0) {
    s_base[a.B] = s_scan[kPlanThreads - 1];
    a.info[4 * a.B + 0] = chunk;
    a.info[4 * a.B + 1] = total;
  }
  __syncthreads();
  for (int it = t; it < total; it += kPlanThreads) {
    int lo = 0, hi = a.B - 1;  // last request with s_base[b] <= it
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_base[mid] <= it) lo = mid;
      else hi = mid - 1;
    }
    const int b = lo, i = it - s_base[b];
    const int splits = s_splits[b], rb = s_rb[b];
    const int split = i % splits, u = i / splits;
    a.desc[it] = make_int4(b, u / rb, u % rb, split);
  }
}

struct ItemCtx {
  int b, kvh, rowb, split, splits, l_b, n_b, keys_b, k_beg, k_end, rows_b;
};

__device__ __forceinline__ bool load_item(const AttnArgs& a, ItemCtx& c) {
  const int item = blockIdx.x;
  if (item >= a.info[4 * a.B + 1]) return false;
  const int4 d = a.desc[item];
  c.b = d.x;
  c.kvh = d.y;
  c.rowb = d.z;
  c.split = d.w;
  const int chunk = a.info[4 * a.B];
  c.splits = a.info[4 * c.b + 1];
  c.l_b = a.info[4 * c.b + 3];
  c.n_b = clampi(a.n_nodes[c.b], 0, a.N_max);
  c.keys_b = c.l_b + c.n_b;
  c.k_beg = c.split * chunk;
  c.k_end = min(c.keys_b, c.k_beg + chunk);
  c.rows_b = c.n_b * a.G;
  return true;
}

// element offset of key `key` (virtual index) of request b, or -1 past the end
__device__ __forceinline__ long key_row(const AttnArgs& a, const ItemCtx& c, int key, bool* tree) {
  if (key < c.l_b) {
    *tree = false;
    return (static_cast<long>(c.b) * a.L_cap + key) * a.stride;
  }
  *tree = true;
  return (static_cast<long>(c.b) * a.N_max + (key - c.l_b)) * a.stride;
}

// ------------------------------------------------ grouped-query MFMA path
// Grouped-query heads of width 128 (the common bf16 case): 128 query rows per
// work item (4 waves x 2 groups of 16 rows), keys streamed in tiles of 32.
//
// Memory pipeline: K and V tiles go from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging) into a ring of slots; waits
// are explicit vmcnt counts and bare barriers (a workgroup fence would drain
// every outstanding load).  Rows are stored unpadded (256 B) with 16-byte
// chunk c of row r at slot c ^ swz(r); the swizzle is applied through the
// global source address of each lane, since the LDS destination of these
// loads is fixed by the lane id.  swz() spreads both the K reads (16 rows,
// one chunk) and the transposed V reads (8 rows x 2 chunks per half-wave)
// over the LDS banks.
//
// The value operand of O^T = V^T P^T needs, per lane, four consecutive keys
// of one value column: ds_read_b64_tr_b16 returns exactly that from V in its
// natural [key][dv] layout when source lane r of a 16-lane group points at
// V[key0 + r/4][dv0 + 4*(r%4)]: lane i then holds V[key0 + k][dv0 + i].

__device__ __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with vmcnt = n (n <= 63), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
  asm volatile("" ::: "memory");
}


typedef short s16x4 __attribute__((ext_vector_type(4)));
#define TSV_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define TSV_LDS4(p) ((__attribute__((address_space(3))) s16x4*)(p))

// One thread's share of loading a K and V tile of KT keys (virtual key
// indices t0 .. t0+KT-1 of one request) into an LDS stage: KT/8
// wave-instructions, each filling 4 consecutive 256-byte rows.  Keys at or
// past k_end re-read row k_end-1 (finite data; masked by the caller).
template <int KT>
__device__ __forceinline__ void gqa_issue_tile(char* stage, int t0, int wave, int lane,
                                               int k_end, int l_b, const char* kc_b,
                                               const char* vc_b, const char* kt_b,
                                               const char* vt_b, long rstride) {
#pragma unroll
  for (int n = 0; n < KT / 8; ++n) {
    const int g = n * 4 + wave;                  // wave-uniform
    const int region = g / (KT / 4);             // 0 = K, 1 = V
    const int rq = g % (KT / 4);
    const int row = rq * 4 + (lane >> 4);
    const int chunk = (lane & 15) ^ swz(row);
    int key = t0 + row;
    key = key < k_end ? key : k_end - 1;
    const bool tr = key >= l_b;
    const long roff = (tr ? key - l_b : key) * rstride + chunk * 16;
    const char* src = (region == 0 ? (tr ? kt_b : kc_b) : (tr ? vt_b : vc_b)) + roff;
    // Issued as inline asm on purpose: the compiler does not track these
    // LDS writes, so it adds no conservative vmcnt(0) before every LDS read
    // of the tile being computed.  Ordering is explicit: each tile is waited
    // for with an explicit vmcnt count (these loads complete in issue order)
    // and a barrier before any wave reads it.
    const uint32_t dst = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>(TSV_LDS(stage + region * KT * 256 + rq * 1024)));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(dst), "v"(src)
                 : "memory", "m0");
  }
}

// ------------------------------------ grouped-query MFMA path, pipelined
// Same work item and LDS layout as above, restructured so that matrix and
// vector work of one wavefront overlap: tiles of 32 keys go through a ring of
// NSLOT slots (NSLOT-2 tiles in flight), and iteration t issues
//   phase 1: the score MFMAs of tile t+1  |  exp / convert / sum of tile t
//   phase 2: the value MFMAs of tile t    |  mask and row max of tile t+1
// followed by the (rare) lazy rescale for tile t+1.  Both phases are single
// basic blocks of independent MFMA and VALU instructions, so the sequencer
// co-issues them.  Row max / sum across the four 16-lane groups use the
// permlane swaps (VALU) rather than LDS permutes.

// max of v over the lanes l, l^16, l^32, l^48
__device__ __forceinline__ float quad_group_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// LDS-DMA of one 1 KiB block: 64 lanes x 16 bytes from sbase + voff (sbase
// is wave-uniform; readfirstlane puts it in scalar registers for the
// instruction's saddr operand).  m0 is written here and used by nothing the
// compiler emits in these kernels, so clobbering it is safe.
__device__ __forceinline__ void dma_1k(uint32_t lds_dst, const char* sbase, uint32_t voff) {
  // readfirstlane returns int: both halves go through uint32_t so that the
  // low half is zero-extended, never sign-extended, into the 64-bit address
  const uint64_t p = reinterpret_cast<uintptr_t>(sbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32))));
  const uint64_t sp = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_dst)), "v"(voff), "s"(sp)
               : "memory", "m0");
}

// Relaxed atomics at agent scope: coherent across the XCDs without ordering
// anything else (no cache-wide write-back or invalidation).
__device__ __forceinline__ void st_coherent2(uint64_t* p, float x, float y) {
  const uint64_t v = (static_cast<uint64_t>(__float_as_uint(y)) << 32) | __float_as_uint(x);
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_coherent2(const uint64_t* p) {
  const uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}

template <int V>
struct IC {
  static constexpr int value = V;
};

template <int LPT, int L>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (L == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= L) wait_vmcnt<LPT * L>();
    else wait_later<LPT, L - 1>(later);
  }
}

// Work item of the one-kernel grouped-query path.  Workgroup ids are dealt to
// the XCDs round robin (id % 8); consecutive ids on one XCD take the S splits
// of one unit, so a unit's splits run side by side and share that XCD's L2,
// where the last one to finish reads the others' partials.  A unit is (row
// block, request, KV head), in that order of significance.
//
// A launch of exactly two workgroups per compute unit (512) is resident at
// once, and workgroup id i shares its compute unit with id i + 256.  The
// first-dispatched of the two is served first and, on equal work, ends its
// loop about 17 % earlier (measured on the grouped workload: 41 against 49
// us).  Such a launch gives each unit's first S/2 splits to first-dispatched
// slots and 57 % of its keys, the other S/2 splits to the second slots and
// the rest, so that both workgroups of a compute unit end together.  Split
// boundaries depend only on the unit's key count, never on timing.
constexpr int kResidentGrid = 512;
constexpr int kFirstShareNum = 57, kFirstShareDen = 100;
constexpr int kPairedMinChunk = 256;

__device__ __forceinline__ bool fused_item(const AttnArgs& a, ItemCtx& c, int& unit) {
  const int id = static_cast<int>(blockIdx.x);
  const int slot = id >> 3;
  const int per_xcd = static_cast<int>(gridDim.x) >> 3;
  const bool paired = static_cast<int>(gridDim.x) == kResidentGrid && (a.S & 1) == 0;
  const int hs = a.S >> 1;
  int grp, split;
  if (paired) {
    const int half = per_xcd >> 1;
    const bool first = slot < half;
    const int s_in = first ? slot : slot - half;
    grp = s_in / hs;
    split = s_in % hs + (first ? 0 : hs);
  } else {
    grp = slot / a.S;
    split = slot % a.S;
  }
  // consecutive groups of 8 units rotate over the XCDs, so that every XCD
  // streams every KV head (the units of a group are the KV heads of one
  // request and row block)
  unit = grp * 8 + (((id & 7) + grp) & 7);
  if (unit >= a.units) return false;
  // units are numbered row block first: the first row block of every
  // (request, KV head) comes before any second one, so the work of short
  // trees (one row block) is spread over all XCDs and dispatched first
  const int per_rb = a.B * a.Hkv;
  c.rowb = unit / per_rb;
  const int rem = unit - c.rowb * per_rb;
  c.b = rem / a.Hkv;
  c.kvh = rem - c.b * a.Hkv;
  c.n_b = clampi(a.n_nodes[c.b], 0, a.N_max);
  c.l_b = clampi(a.prefix_len[c.b], 0, a.L_cap);
  c.rows_b = c.n_b * a.G;
  if (c.rowb * 128 >= c.rows_b) return false;
  c.keys_b = c.l_b + c.n_b;
  if (paired) {
    // first-dispatched splits: keys [0, ka) in hs chunks of ca; the others:
    // [ka, keys_b) in hs chunks of cb (multiples of 32 keys); used when
    // every split keeps at least kPairedMinChunk keys
    const int ka = static_cast<int>(static_cast<long long>(c.keys_b) * kFirstShareNum / kFirstShareDen) / 32 * 32;
    const int ca = ((ka + hs - 1) / hs + 31) / 32 * 32;
    const int cb = ((c.keys_b - ka + hs - 1) / hs + 31) / 32 * 32;
    const bool fits = ka >= hs * kPairedMinChunk && c.keys_b - ka >= hs * kPairedMinChunk &&
                      (hs - 1) * ca < ka && (hs - 1) * cb < c.keys_b - ka;
    if (fits) {
      c.splits = a.S;
      c.split = split;
      c.k_beg = split < hs ? split * ca : ka + (split - hs) * cb;
      c.k_end = split < hs ? min(ka, c.k_beg + ca) : min(c.keys_b, c.k_beg + cb);
      return true;
    }
  }
  // the unit's keys in S nearly equal chunks (a multiple of 32 keys), but
  // none shorter than a.chunk, the chunk of the longest possible unit: a
  // short unit takes fewer splits rather than shorter ones, each of which
  // would cost a published partial and its read-back
  int chunk = (c.keys_b + a.S - 1) / a.S;
  chunk = (chunk + 31) / 32 * 32;
  chunk = chunk > a.chunk ? chunk : a.chunk;
  c.splits = (c.keys_b + chunk - 1) / chunk;  // <= S
  if (split >= c.splits) return false;
  c.split = split;
  c.k_beg = split * chunk;
  c.k_end = min(c.keys_b, c.k_beg + chunk);
  return true;
}

template <int NSLOT>
__global__ __launch_bounds__(256, 2) void attn_gqa_pipe_kernel(AttnArgs a) {
  constexpr int KT = 32, D = 128, RG = 2, RB = 128;
  constexpr int ROWB = 256;               // bytes per key row of one head
  constexpr int TILEB = KT * ROWB;        // K (or V) part of a tile
  constexpr int SLOT = 2 * TILEB;
  constexpr int LPT = KT / 8;             // 1 KiB DMA blocks per thread per tile
  constexpr int NKB = KT / 16, NC = D / 32, NDB = D / 16;
  static_assert(NSLOT == 4 || NSLOT == 5, "the unrolled steps assume a ring of four or five tiles");
  __shared__ __align__(1024) char smem[NSLOT * SLOT];
  // after the key loop the ring is free; its first word carries the
  // last-split flag (two workgroups of five slots fill the CU's LDS)
  int& s_last = *reinterpret_cast<int*>(smem);

  ItemCtx c;
  int unit;
  if (!fused_item(a, c, unit)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const long rstride = a.stride * 2;
  const long head_off = static_cast<long>(c.kvh) * D * 2;
  const float scale = a.scale_log2;
  const char* kc_b = static_cast<const char*>(a.kc) + static_cast<long>(c.b) * a.L_cap * rstride + head_off;
  const char* vc_b = static_cast<const char*>(a.vc) + static_cast<long>(c.b) * a.L_cap * rstride + head_off;
  const char* kt_b = static_cast<const char*>(a.kt) + static_cast<long>(c.b) * a.N_max * rstride + head_off;
  const char* vt_b = static_cast<const char*>(a.vt) + static_cast<long>(c.b) * a.N_max * rstride + head_off;
  const int k_beg = c.k_beg, k_end = c.k_end, l_b = c.l_b;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TSV_LDS(smem)));

  // this thread's two 1 KiB blocks of a tile's K part (the V part mirrors
  // them); tiles are issued in order, so the source pointers just advance
  uint32_t toff[2], tdst[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int rq = n * 4 + wave;                 // 4-row group, 0..7
    const int row = rq * 4 + (lane >> 4);
    toff[n] = static_cast<uint32_t>(row * rstride + (((lane & 15) ^ swz(row)) << 4));
    tdst[n] = lds0 + static_cast<uint32_t>(rq * 1024);
  }
  const long tile_bytes = static_cast<long>(KT) * rstride;
  const char* kp = kc_b + static_cast<long>(k_beg) * rstride;
  const char* vp = vc_b + static_cast<long>(k_beg) * rstride;
  int tn = k_beg;  // first key of the next tile to issue
  auto issue = [&](auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if (tn + KT <= k_end && tn + KT <= l_b) {
#pragma unroll
      for (int n = 0; n < 2; ++n) dma_1k(tdst[n] + SL * SLOT, kp, toff[n]);
#pragma unroll
      for (int n = 0; n < 2; ++n) dma_1k(tdst[n] + SL * SLOT + TILEB, vp, toff[n]);
    } else {
      gqa_issue_tile<KT>(smem + SL * SLOT, tn, wave, lane, k_end, l_b, kc_b, vc_b, kt_b, vt_b, rstride);
    }
    kp += tile_bytes;
    vp += tile_bytes;
    tn += KT;
  };

  // the key stream starts before anything else is loaded
  const int ntiles = (k_end - k_beg + KT - 1) / KT;
  issue(IC<0>{});
  if (1 < ntiles) issue(IC<1>{});
  if (2 < ntiles) issue(IC<2>{});
  if constexpr (NSLOT == 5)
    if (3 < ntiles) issue(IC<3>{});

  bf16x8 qf[RG][NC];
  uint32_t anc[RG][4];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int r = c.rowb * RB + wave * RG * 16 + rg * 16 + lr;
    const bool rv = r < c.rows_b;   // idle rows compute on zero queries, never written
    const int node = rv ? r / a.G : 0;
    const int h = c.kvh * a.G + (rv ? r % a.G : 0);
    const uint16_t* src = qp + ((static_cast<size_t>(c.b) * a.N_max + node) * a.Hq + h) * D;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      if (rv) qf[rg][k] = *reinterpret_cast<const bf16x8*>(src + 32 * k + 8 * lq);
      else qf[rg][k] = bf16x8{};
    }
    const unsigned* ab = a.anc + (static_cast<size_t>(c.b) * a.N_max + node) * a.W;
#pragma unroll
    for (int w = 0; w < 4; ++w) anc[rg][w] = (rv && w < a.W) ? ab[w] : 0u;
  }

  // m_run: reference max per row (log2 units); muse: m_run, or 0 while no key
  // was seen; lacc: row sums of the weights (every element holds the sum)
  float m_run[RG], muse[RG];
  f32x4 o[RG][NDB], lacc[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m_run[rg] = -INFINITY;
    muse[rg] = 0.f;
    lacc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[rg][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

  // per-lane LDS byte offsets inside a slot; the slot base and the second
  // 16-row half are immediates (swz is the same for rows r and r + 16)
  uint32_t koff[NC], voff[NDB];
#pragma unroll
  for (int k = 0; k < NC; ++k) koff[k] = lr * ROWB + (((4 * k + lq) ^ swz(lr)) << 4);
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    const int row0 = 4 * lq + (lr >> 2);
    const int chunk = 2 * d + ((lr & 3) >> 1);
    voff[d] = TILEB + row0 * ROWB + ((chunk ^ swz(row0)) << 4) + ((lr & 1) << 3);
  }

  // S^T of a tile: lane holds S^T[key = kb*16 + 4*lq + i][row = lr]
  auto scores = [&](f32x4 (&s)[RG][NKB], int j) {
    const char* kb_base = smem + (j % NSLOT) * SLOT;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) s[rg][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NC; ++k) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 16 + lr;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb_base + row * ROWB + (((4 * k + lq) ^ swz(row)) << 4));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          s[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rg][k], s[rg][kb], 0, 0, 0);
      }
    }
  };
  // masks of a tile that reaches into the scratch rows or past the chunk end
  auto mask = [&](f32x4 (&s)[RG][NKB], int j) {
    const int t0 = k_beg + j * KT;
    if (t0 + KT <= k_end && t0 + KT <= l_b) return;
    // keeps the compiler from computing the masks for every tile and
    // selecting afterwards; only the last tiles of an item take this path
    asm volatile("" ::: "memory");
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = key_visible(anc[rg], t0 + kb * 16 + 4 * lq + i, l_b, k_end);
          s[rg][kb][i] = ok ? s[rg][kb][i] : -INFINITY;
        }
  };
  // Turns the scores of a tile into exponents x = s*scale - m (log2 units)
  // and applies lazy rescaling: the reference max m of a row moves only when
  // the tile holds a score above m + kLazy, so p = 2^x <= 2^kLazy.  The test
  // uses each lane's own maximum (fma results, so max needs no NaN quieting);
  // only a tile that moves some row's max takes the cross-lane path.
  auto exponents = [&](f32x4 (&s)[RG][NKB]) {
    bool need = false;
    float lmax[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[rg][kb][i] = fmaf(s[rg][kb][i], scale, -muse[rg]);
      float mx = fmaxf(fmaxf(s[rg][0][0], s[rg][0][1]), fmaxf(s[rg][0][2], s[rg][0][3]));
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb)
        mx = fmaxf(mx, fmaxf(fmaxf(s[rg][kb][0], s[rg][kb][1]), fmaxf(s[rg][kb][2], s[rg][kb][3])));
      lmax[rg] = mx;
      need |= mx > (m_run[rg] == -INFINITY ? -INFINITY : kLazy);
    }
    if (__ballot(need)) {
      asm volatile("" ::: "memory");  // a real branch: taken for few tiles
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const float mt = quad_group_max(lmax[rg]) + muse[rg];   // the row's scaled max
        const bool up = m_run[rg] == -INFINITY ? mt > -INFINITY : mt > m_run[rg] + kLazy;
        if (!up) continue;  // uniform over the row's four lanes
        const float alpha = m_run[rg] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rg] - mt);
        lacc[rg] *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[rg][d] *= alpha;
        const float delta = muse[rg] - mt;
        m_run[rg] = mt;
        muse[rg] = mt;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[rg][kb] += delta;
      }
    }
  };
  auto probs = [&](const f32x4 (&x)[RG][NKB], bf16x8 (&pf)[RG]) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pf[rg][kb * 4 + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(x[rg][kb][i]));
  };
  // O^T[dv][row] += V^T[dv][keys] P^T[keys][row]; the key order inside the
  // 32-key step (16*(e/4) + 4*lq + e%4 for element e) matches the scores'
  auto values = [&](const bf16x8 (&pf)[RG], int j) {
    const char* vb_base = smem + (j % NSLOT) * SLOT + TILEB;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int chunk = 2 * d + ((lr & 3) >> 1);
      const int boff = (lr & 1) << 3;
      const int row0 = 4 * lq + (lr >> 2);
      const int row1 = row0 + 16;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          TSV_LDS4(vb_base + row0 * ROWB + ((chunk ^ swz(row0)) << 4) + boff));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          TSV_LDS4(vb_base + row1 * ROWB + ((chunk ^ swz(row1)) << 4) + boff));
      union {
        s16x4 h[2];
        bf16x8 v;
      } vf;
      vf.h[0] = lo;
      vf.h[1] = hi;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        o[rg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pf[rg], o[rg][d], 0, 0, 0);
    }
    // row sums of the same bf16 weights: every output row of ones * P^T
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      lacc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[rg], lacc[rg], 0, 0, 0);
  };

  f32x4 sc[RG][NKB], sn[RG][NKB];
  bf16x8 pf[RG];
  wait_later<LPT, NSLOT - 2>(min(NSLOT - 2, ntiles - 1));
  lds_barrier();
  scores(sc, 0);
  mask(sc, 0);
  exponents(sc);

  // One step of the pipeline for tile t (t % NSLOT == J, a compile-time
  // slot, so every LDS address below is a register plus an immediate).
  auto step = [&](auto j_c, int t) {
    constexpr int J = decltype(j_c)::value;
    constexpr int SN = (J + 1) % NSLOT;  // slot of tile t+1
    // tile t+1 resident; every wave is done with tile t-1, whose slot is refilled
    wait_later<LPT, NSLOT - 3>(min(NSLOT - 3, ntiles - 2 - t));
    lds_barrier();
    if (t + NSLOT - 1 < ntiles) issue(IC<(J + NSLOT - 1) % NSLOT>{});
    // The offsets are redefined here so that offset + slot constant is not
    // hoisted out of the loop (one register per slot and read); inside the
    // block the constant folds into the instruction's offset field.
#pragma unroll
    for (int k = 0; k < NC; ++k) asm volatile("" : "+v"(koff[k]));
#pragma unroll
    for (int d = 0; d < NDB; ++d) asm volatile("" : "+v"(voff[d]));
    // one basic block: scores of tile t+1, weights and values of tile t
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) sn[rg][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NC; ++k)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(smem + SN * SLOT + kb * 16 * ROWB + koff[k]);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          sn[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rg][k], sn[rg][kb], 0, 0, 0);
      }
    probs(sc, pf);
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      union {
        s16x4 h[2];
        bf16x8 v;
      } vf;
      vf.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TSV_LDS4(smem + J * SLOT + voff[d]));
      vf.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TSV_LDS4(smem + J * SLOT + 16 * ROWB + voff[d]));
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        o[rg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pf[rg], o[rg][d], 0, 0, 0);
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      lacc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[rg], lacc[rg], 0, 0, 0);
    mask(sn, t + 1);
    exponents(sn);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[rg][kb] = sn[rg][kb];
  };

  // NSLOT steps per trip, leaving after whichever step reaches the last tile
  for (int t = 0; t + 1 < ntiles;) {
    step(IC<0>{}, t);
    if (++t + 1 >= ntiles) break;
    step(IC<1>{}, t);
    if (++t + 1 >= ntiles) break;
    step(IC<2>{}, t);
    if (++t + 1 >= ntiles) break;
    step(IC<3>{}, t);
    if constexpr (NSLOT == 5) {
      if (++t + 1 >= ntiles) break;
      step(IC<4>{}, t);
    }
    ++t;
  }
  probs(sc, pf);
  values(pf, ntiles - 1);

  // lane holds O^T[dv = d*16 + 4*lq + i][row = lr]; lacc[rg] holds the row sum
  auto write_row = [&](int rg, const f32x4 (&acc)[NDB], float m, float l) {
    const int r = c.rowb * RB + wave * RG * 16 + rg * 16 + lr;
    if (r >= c.rows_b) return;
    const int node = r / a.G, h = c.kvh * a.G + r % a.G;
    const size_t orow = (static_cast<size_t>(c.b) * a.N_max + node) * a.Hq + h;
    uint16_t* op = static_cast<uint16_t*>(a.out) + orow * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      union {
        uint2 u;
        __bf16 h4[4];
      } pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk.h4[i] = static_cast<__bf16>(acc[d][i] * inv);
      *reinterpret_cast<uint2*>(op + d * 16 + 4 * lq) = pk.u;
    }
    if (lq == 0 && a.lse) a.lse[orow] = (m + log2f(l)) * kLn2;
  };

  if (c.splits == 1) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) write_row(rg, o[rg], m_run[rg], lacc[rg][0]);
    return;
  }

  // Split-K.  Each split publishes its rows (max, sum, accumulator) with
  // agent-scope atomic stores, which are written through the L2 to the level
  // shared by all XCDs and acknowledged from there; once every thread has
  // seen its acknowledgements (vmcnt 0) one thread counts the split in with
  // an agent-scope atomic add.  The split that counts last acquires at agent
  // scope (dropping stale cached lines), reads the others' rows with
  // agent-scope atomic loads, combines them and resets the counter for the
  // next call.  A release fence is left out on purpose: what it adds to the
  // acknowledgement wait is a write-back of every dirty line of the L2, and
  // the published rows never are dirty there; issued by every workgroup it
  // costs more than the rest of the combine.
  // What a split publishes is its rows normalised by their own sums (O/l,
  // rounded to bf16: half the bytes of fp32, and the combine scales them
  // back by w*l in fp32) with the row (max, sum) pairs in fp32.  Layout
  // private to this kernel, in lane order so that every store and load
  // instruction covers 512 contiguous bytes: per (unit, split), per (wave,
  // row group): normalised rows [d][lane] as 4 x bf16, and the row (max,
  // sum) pairs [lr] as float2.
  // own[rg][d] keeps this split's rows exactly as published, so that the
  // combine computes its term like every other split's (same bits whichever
  // split arrives last); the fp32 accumulators are dead from here on.
  const size_t item = static_cast<size_t>(unit) * a.S + c.split;
  float2 own[RG][NDB];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int wr = wave * RG + rg;
    uint64_t* pa = reinterpret_cast<uint64_t*>(a.part_acc + item * kGqaPartFloats) + static_cast<size_t>(wr) * NDB * 64;
    const float lt = lacc[rg][0];
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      union {
        float2 f;
        __bf16 h4[4];
      } pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk.h4[i] = static_cast<__bf16>(o[rg][d][i] * inv);
      own[rg][d] = pk.f;
      st_coherent2(pa + d * 64 + lane, pk.f.x, pk.f.y);
    }
    if (lq == 0)
      st_coherent2(reinterpret_cast<uint64_t*>(a.part_ml + item * RB * 2) + wr * 16 + lr, m_run[rg], lacc[rg][0]);
  }
  wait_vmcnt<0>();  // this thread's row stores acknowledged at device scope
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             c.splits - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // no stale cached copy of the rows

  // Each load below goes to the level shared by all XCDs: under the key
  // stream of the other workgroups a round trip costs over a microsecond, so
  // loads are issued in as few dependent groups as the registers allow.
  const int ns = c.splits, own_s = c.split;
  auto ml_ptr = [&](int s2, int wr) {
    return reinterpret_cast<const uint64_t*>(a.part_ml + (static_cast<size_t>(unit) * a.S + s2) * RB * 2) +
           wr * 16 + lr;
  };
  auto rows_ptr = [&](int s2, int wr) {
    return reinterpret_cast<const uint64_t*>(a.part_acc + (static_cast<size_t>(unit) * a.S + s2) * kGqaPartFloats) +
           static_cast<size_t>(wr) * NDB * 64 + lane;
  };
  // one split's term of the combined row, weighted by 2^(m - M) * l; the
  // terms are summed in split order whichever split arrived last
  auto term = [&](float m, float l, const float2 (&r)[NDB], float Mx, float& L, f32x4 (&acc)[NDB]) {
    const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - Mx);
    L = fmaf(w, l, L);
    const float wl = w * l;   // weight of the normalised row
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const uint32_t u0 = __float_as_uint(r[d].x), u1 = __float_as_uint(r[d].y);
      acc[d][0] = fmaf(wl, __uint_as_float(u0 << 16), acc[d][0]);
      acc[d][1] = fmaf(wl, __uint_as_float(u0 & 0xFFFF0000u), acc[d][1]);
      acc[d][2] = fmaf(wl, __uint_as_float(u1 << 16), acc[d][2]);
      acc[d][3] = fmaf(wl, __uint_as_float(u1 & 0xFFFF0000u), acc[d][3]);
    }
  };

  constexpr int kR = 3;  // other splits held in registers at once
  if (ns <= kR + 1) {
    // every other split's pairs and rows, both row groups, in one group of
    // loads.  Slot j holds split j + (j >= own_s); slots past the last
    // split repeat it and are never used.
    const int nr = ns - 1;
    auto split_of = [&](int j) { const int r = min(j, nr - 1); return r + (r >= own_s ? 1 : 0); };
    float2 mlr[RG][kR], rws[RG][kR][NDB];
#pragma unroll
    for (int j = 0; j < kR; ++j)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) mlr[rg][j] = ld_coherent2(ml_ptr(split_of(j), wave * RG + rg));
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        const uint64_t* pa = rows_ptr(split_of(j), wave * RG + rg);
#pragma unroll
        for (int d = 0; d < NDB; ++d) rws[rg][j][d] = ld_coherent2(pa + d * 64);
      }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      float M = m_run[rg];
#pragma unroll
      for (int j = 0; j < kR; ++j) M = fmaxf(M, j < nr ? mlr[rg][j].x : -INFINITY);
      float L = 0.f;
      f32x4 acc[NDB];
#pragma unroll
      for (int d = 0; d < NDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
      // slots in split order, this split's own term inserted before slot
      // own_s (or after the last slot)
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        if (j == own_s) term(m_run[rg], lacc[rg][0], own[rg], M, L, acc);
        if (j >= nr) break;
        term(mlr[rg][j].x, mlr[rg][j].y, rws[rg][j], M, L, acc);
      }
      if (own_s == nr && nr >= kR) term(m_run[rg], lacc[rg][0], own[rg], M, L, acc);
      write_row(rg, acc, M, L);
    }
  } else {
    // many splits: the pairs of up to kMl splits, then the rows of kAcc
    // splits at a time
    constexpr int kMl = 8, kAcc = 2;
    float M[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) M[rg] = m_run[rg];
    for (int s0 = 0; s0 < ns; s0 += kMl) {
      float2 v[RG][kMl];
#pragma unroll
      for (int j = 0; j < kMl; ++j)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) v[rg][j] = ld_coherent2(ml_ptr(min(s0 + j, ns - 1), wave * RG + rg));
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int j = 0; j < kMl; ++j) M[rg] = fmaxf(M[rg], v[rg][j].x);
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const int wr = wave * RG + rg;
      float L = 0.f;
      f32x4 acc[NDB];
#pragma unroll
      for (int d = 0; d < NDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < ns; s0 += kAcc) {
        float2 mlv[kAcc], rows[kAcc][NDB];
#pragma unroll
        for (int j = 0; j < kAcc; ++j) {
          const int s2 = min(s0 + j, ns - 1);
          mlv[j] = ld_coherent2(ml_ptr(s2, wr));
          const uint64_t* pa = rows_ptr(s2, wr);
#pragma unroll
          for (int d = 0; d < NDB; ++d) rows[j][d] = ld_coherent2(pa + d * 64);
        }
#pragma unroll
        for (int j = 0; j < kAcc; ++j) {
          const int s2 = s0 + j;
          if (s2 >= ns) break;
          if (s2 == own_s) term(m_run[rg], lacc[rg][0], own[rg], M[rg], L, acc);
          else term(mlv[j].x, mlv[j].y, rows[j], M[rg], L, acc);
        }
      }
      write_row(rg, acc, M[rg], L);
      // keeps the next row group's loads below this one's arithmetic (both
      // groups' rows in flight at once would not fit the register file)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (tid == 0) a.counters[unit] = 0;
}

// ------------------------------------------------------ latent MFMA path
// One latent KV head shared by every query head: the key is the 576-wide
// latent row, the value its first 512 columns (the cache is passed once, as
// both key and value).  A work item is 128 query rows (node x head) of one
// request and a chunk of its keys; 4 waves, one per SIMD.
//
// Division of work.  Wave w computes the scores of rows 32w..32w+31 for all
// 32 keys of a tile (its queries stay in registers for the whole item) and
// turns them into bf16 weights, which go to LDS in the operand layout of the
// value product.  The value product is split by output column instead: wave
// w accumulates O^T for columns 128w..128w+127 of all 128 rows, reading every
// wave's weights.  This way one K tile in LDS feeds both products, each wave
// holds a quarter of the 128 x 512 fp32 accumulator, and the LDS bytes read
// per MFMA stay low enough for the matrix cores to stay busy.
//
// K tiles (32 keys x 1152 bytes) reach LDS by LDS-DMA, one 1 KiB block per
// instruction, in a ring of three slots (one tile in flight while two are
// read).  Inside a tile, 16-byte granule C (columns 8C..8C+7) of key k sits
//   C < 64:  block 4*(k/4) + C/16, row k%4 of 256 bytes, granule (C%16)^s(k)
//   C >= 64: block 32 + k/8,       row k%8 of 128 bytes, granule (C-64)^t(k)
// with s a bijection of k%16 and t(k) = (k/2)%8.  Every score operand read
// (16 keys of one granule per 16 lanes) and every transposed value read
// (4 keys x 2 granules per 16 lanes) then touches distinct banks, and each
// DMA block reads whole 256- or 128-byte runs of 4 or 8 key rows.
//
// Softmax per row is online with a lazy reference max (as in the grouped
// path): the max moves only when a tile exceeds it by kLazy (log2 units),
// decided without branches; a wave that moves any of its rows' max posts the
// factors and a flag, and before the next value product every wave rescales
// the accumulator rows concerned (a rare branch).
constexpr int kLatQK = 576, kLatV = 512;
constexpr int kLatTile = 32 * kLatQK * 2;        // bytes of one K tile
constexpr int kLatSlots = 3;
constexpr int kLatP = kLatSlots * kLatTile;      // weights, two buffers of 8 KiB
// rescale factors [2][4 copies][16 rows][9 floats] (8 used; the ninth pads
// the rows so that the 32 lanes of a write or read hit distinct banks)
constexpr int kLatAlphaCopy = 16 * 9;            // floats per copy
constexpr int kLatAlphaBuf = 2304;               // bytes per buffer (4 copies, 256-aligned)
constexpr int kLatAlpha = kLatP + 2 * 8192;
constexpr int kLatFlag = kLatAlpha + 2 * kLatAlphaBuf;   // rescale flags [2][4 waves][64 lanes]
constexpr int kLatStat = kLatFlag + 2 * 1024;    // final (max, sum) per row
constexpr int kLatLds = kLatStat + 128 * 8;

// Granule swizzle of key k (a bijection of k % 16): granule C of key k sits
// at C ^ s(k) in its row.  Measured with the LDS bank-conflict counter on the
// long latent workload: the identity leaves 0.48 conflict cycles per LDS
// instruction, where a swizzle chosen for 16 lanes per cycle over 64 banks
// (conflict-free on paper for both the score operand reads and the
// transposed value reads) gave 2.1; the hardware serves these reads in a
// pattern neither model captures, and the kernel's time does not depend on
// the difference.
__device__ __forceinline__ int lat_s(int k) { return k & 15; }
__device__ __forceinline__ int lat_t(int k) { return (k >> 1) & 7; }

// s_waitcnt vmcnt(0) lgkmcnt(0): this wave's DMA blocks and LDS writes done
__device__ __forceinline__ void wait_all_mem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x70);
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS writes done (DMA loads may remain)
// sum of v over the lanes l, l^16, l^32, l^48
__device__ __forceinline__ float quad_group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ bool latent_item(const AttnArgs& a, ItemCtx& c, int& item) {
  // ids are dealt to the XCDs round robin; give each XCD a contiguous run of
  // items, so that the row blocks of one request share that XCD's L2
  const int total = a.info[4 * a.B + 1];
  const int per = (total + 7) >> 3;
  const int id = static_cast<int>(blockIdx.x);
  const int pos = id >> 3;
  item = (id & 7) * per + pos;
  if (pos >= per || item >= total) return false;
  const int4 d = a.desc[item];
  c.b = d.x;
  c.kvh = d.y;
  c.rowb = d.z;
  c.split = d.w;
  const int chunk = a.info[4 * a.B];
  c.splits = a.info[4 * c.b + 1];
  c.l_b = a.info[4 * c.b + 3];
  c.n_b = clampi(a.n_nodes[c.b], 0, a.N_max);
  c.keys_b = c.l_b + c.n_b;
  c.k_beg = c.split * chunk;
  c.k_end = min(c.keys_b, c.k_beg + chunk);
  c.rows_b = c.n_b * a.G;
  return c.k_beg < c.k_end;
}

__global__ __launch_bounds__(256, 1) void attn_latent_kernel(AttnArgs a) {
  constexpr int KT = 32, RB = 128, NC = kLatQK / 32;
  __shared__ __align__(1024) char smem[kLatLds];

  ItemCtx c;
  int item;
  if (!latent_item(a, c, item)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const long rstride = a.stride * 2;
  const float scale = a.scale_log2;
  const char* kc_b = static_cast<const char*>(a.kc) + static_cast<long>(c.b) * a.L_cap * rstride;
  const char* kt_b = static_cast<const char*>(a.kt) + static_cast<long>(c.b) * a.N_max * rstride;
  const int k_beg = c.k_beg, k_end = c.k_end, l_b = c.l_b;
  const int nt = (k_end - k_beg + KT - 1) / KT;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TSV_LDS(smem)));

  // ---- DMA: wave w fills blocks 4*kg + w (kg = 0..7) and tail block 32 + w
  // source offsets are recomputed at each issue from an opaque copy of the
  // lane id (a few VALU operations) rather than held in registers
  auto issue = [&](int j, uint32_t slot_lds) {
    const int t0 = k_beg + j * KT;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int tkey = 8 * wave + (ln >> 3);
    const int tC = 64 + ((ln & 7) ^ lat_t(tkey));
    if (t0 + KT <= k_end && t0 + KT <= l_b) {
      const char* tp = kc_b + static_cast<long>(t0) * rstride;
#pragma unroll
      for (int kg = 0; kg < 8; ++kg) {
        const int key = 4 * (kg & 3) + (ln >> 4);
        const int C = 16 * wave + ((ln & 15) ^ lat_s(key));
        dma_1k(slot_lds + (kg * 4 + wave) * 1024, tp + (kg >> 2) * 16 * rstride,
               static_cast<uint32_t>(key * rstride + C * 16));
      }
      dma_1k(slot_lds + (32 + wave) * 1024, tp, static_cast<uint32_t>(tkey * rstride + tC * 16));
    } else {
      // a tile reaching into the scratch rows or past the chunk end: per-lane
      // rows; keys at or past k_end re-read row k_end-1 (masked later)
      auto one = [&](uint32_t dst, int key, int C) {
        key = t0 + key;
        key = key < k_end ? key : k_end - 1;
        const bool tr = key >= l_b;
        const char* src = (tr ? kt_b + static_cast<long>(key - l_b) * rstride
                              : kc_b + static_cast<long>(key) * rstride) + C * 16;
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(src)
                     : "memory", "m0");
      };
#pragma unroll
      for (int kg = 0; kg < 8; ++kg) {
        const int key = 4 * kg + (ln >> 4);
        one(slot_lds + (kg * 4 + wave) * 1024, key, 16 * wave + ((ln & 15) ^ lat_s(key)));
      }
      one(slot_lds + (32 + wave) * 1024, tkey, tC);
    }
  };
  issue(0, lds0);
  if (nt > 1) issue(1, lds0 + kLatTile);

  // ---- this wave's query rows (two groups of 16) and ancestor words
  bf16x8 qf[2][NC];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int r = c.rowb * RB + wave * 32 + rg * 16 + lr;
    const bool rv = r < c.rows_b;   // idle rows compute on zero queries, never written
    const int node = rv ? r / a.G : 0;
    const int h = rv ? r % a.G : 0;
    const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                          ((static_cast<size_t>(c.b) * a.N_max + node) * a.Hq + h) * kLatQK;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      if (rv) qf[rg][k] = *reinterpret_cast<const bf16x8*>(src + 32 * k + 8 * lq);
      else qf[rg][k] = bf16x8{};
    }
  }

  // ---- LDS offsets (bytes) of this lane's operand reads inside a tile
  // score operand, key 16*kb + lr, granule 4*k + lq:
  //   k < 16:  kofs[k % 4] + kb*16384 + (k/4)*1024;  k = 16, 17: ktl[k-16] + kb*2048
  uint32_t kofs[4], ktl[2];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    kofs[q] = (lr >> 2) * 4096 + (lr & 3) * 256 + (((4 * q + lq) ^ lat_s(lr)) << 4);
#pragma unroll
  for (int e = 0; e < 2; ++e)
    ktl[e] = 32768 + (lr >> 3) * 1024 + (lr & 7) * 128 + (((4 * e + lq) ^ lat_t(lr)) << 4);
  // transposed value reads (keys 4*lq + lr/4 and +16, columns 128*wave +
  // 16*dd + 4*(lr%4)): vrow + ((2*dd ^ vsw) << 4), second half +16384
  const int vkey = 4 * lq + (lr >> 2);
  uint32_t vrow = (lq * 4 + wave) * 1024 + (lr >> 2) * 256 + (lr & 1) * 8;
  uint32_t vsw = static_cast<uint32_t>(((lr & 3) >> 1) ^ lat_s(vkey));
  const uint32_t prow = static_cast<uint32_t>(lane * 16);

  float m_run[2], lsum[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    m_run[rg] = -INFINITY;
    lsum[rg] = 0.f;
  }
  f32x4 o[8][8];   // [dd][rb]: O^T[128*wave + 16*dd + 4*lq + i][16*rb + lr]
#pragma unroll
  for (int dd = 0; dd < 8; ++dd)
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) o[dd][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mask = [&](f32x4 (&s)[2][2], int j) {
    const int t0 = k_beg + j * KT;
    if (t0 + KT <= k_end && t0 + KT <= l_b) return;
    asm volatile("" ::: "memory");  // a real branch: only the last tiles take it
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      // the row's ancestor words, read here rather than kept in registers
      const int r = c.rowb * RB + wave * 32 + rg * 16 + lr;
      const bool rv = r < c.rows_b;
      const unsigned* ab = a.anc + (static_cast<size_t>(c.b) * a.N_max + (rv ? r / a.G : 0)) * a.W;
      uint32_t anc[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) anc[w] = (rv && w < a.W) ? ab[w] : 0u;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = key_visible(anc, t0 + kb * 16 + 4 * lq + i, l_b, k_end);
          s[rg][kb][i] = ok ? s[rg][kb][i] : -INFINITY;
        }
    }
  };
  auto kread = [&](const char* kbase, int n) {
    const int k = n >> 1, kb = n & 1;
    const uint32_t off = k < 16 ? kofs[k & 3] + kb * 16384 + (k >> 2) * 1024 : ktl[k - 16] + kb * 2048;
    return *reinterpret_cast<const bf16x8*>(kbase + off);
  };
  auto vread = [&](const char* vbase, int dd) {
    const uint32_t off = vrow + (((2 * dd) ^ vsw) << 4);
    union {
      s16x4 h[2];
      bf16x8 v;
    } vf;
    vf.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TSV_LDS4(vbase + off));
    vf.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TSV_LDS4(vbase + off + 16384));
    return vf.v;
  };
  // The scores of a tile: 36 groups of one K operand read (issued six
  // groups ahead) and two MFMAs; lane holds S^T[key 16*kb + 4*lq + i][row lr].
  auto scores_p = [&](f32x4 (&s)[2][2], uint32_t sb) {
    const char* kbase = smem + (sb - lds0);
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[rg][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int AH = 6;   // operand reads in flight
    bf16x8 kf[AH + 1];
#pragma unroll
    for (int n = 0; n < AH; ++n) kf[n] = kread(kbase, n);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < 2 * NC; ++n) {
      if (n + AH < 2 * NC) kf[(n + AH) % (AH + 1)] = kread(kbase, n + AH);
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
        s[rg][n & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[n % (AH + 1)], qf[rg][n >> 1], s[rg][n & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The value product of tile j,
  //   O^T[128w + 16dd + ..][rows] += V^T[..][keys of tile j] P^T(j),
  // the transposed value operand of block dd+1 read while block dd's eight
  // MFMAs run, with the softmax of tile j+1 (scores x) cut into small pieces
  // between the MFMA groups, so that the VALU work runs while the matrix
  // cores are busy (the scheduling barriers keep that order).  Weights,
  // rescale factors and flags of tile j+1 go to LDS buffer (j+1) & 1.
  auto values_softmax = [&](auto with_values, uint32_t sv, int j, f32x4 (&x)[2][2]) {
    constexpr bool WV = decltype(with_values)::value != 0;
    const uint32_t buf = static_cast<uint32_t>(j & 1), nbuf = buf ^ 1u;
    const char* vbase = smem + (sv - lds0);
    float mx[2], mt[2], muse[2], ps[2], alpha[2];
    bf16x8 pf[2];
    bool moved = false;
    // piece m of the softmax of row group rg (13 pieces per row group)
    auto piece = [&](int rg, int m) {
      if (m == 0) {
        mx[rg] = vmax3(x[rg][0][0], x[rg][0][1], x[rg][0][2]);
        mx[rg] = vmax3(mx[rg], x[rg][0][3], x[rg][1][0]);
      } else if (m == 1) {
        mx[rg] = vmax3(mx[rg], x[rg][1][1], x[rg][1][2]);
        mx[rg] = vmax3(mx[rg], x[rg][1][3], x[rg][1][3]);
      } else if (m == 2) {
        mt[rg] = quad_group_max(mx[rg]) * scale;   // the row's max over the tile
      } else if (m == 3) {
        const bool fresh = m_run[rg] == -INFINITY;
        const bool up = fresh ? mt[rg] > -INFINITY : mt[rg] > m_run[rg] + kLazy;
        const float al = up ? (fresh ? 0.f : __builtin_amdgcn_exp2f(m_run[rg] - mt[rg])) : 1.f;
        m_run[rg] = up ? mt[rg] : m_run[rg];
        lsum[rg] *= al;
        alpha[rg] = al;
        moved |= up;
        muse[rg] = m_run[rg] == -INFINITY ? 0.f : m_run[rg];
        ps[rg] = 0.f;
      } else if (m < 12) {
        const int e = m - 4;
        const float p = __builtin_amdgcn_exp2f(fmaf(x[rg][e >> 2][e & 3], scale, -muse[rg]));
        ps[rg] += p;
        pf[rg][e] = static_cast<__bf16>(p);
      } else {
        lsum[rg] += ps[rg];
        *reinterpret_cast<bf16x8*>(smem + kLatP + nbuf * 8192 + (2 * wave + rg) * 1024 + prow) = pf[rg];
      }
    };
    auto publish = [&]() {
      // written by every lane, without branches and to distinct addresses
      // (each of the four lanes of a row keeps its own copy of the factor,
      // each lane its own copy of the wave's flag)
      const bool any = __ballot(moved) != 0;
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
        *reinterpret_cast<float*>(smem + kLatAlpha + nbuf * kLatAlphaBuf + (lq * kLatAlphaCopy + lr * 9 + 2 * wave + rg) * 4) = alpha[rg];
      *reinterpret_cast<int*>(smem + kLatFlag + nbuf * 1024 + wave * 256 + lane * 4) = any ? 1 : 0;
    };
    bf16x8 pt[8], vf[2];
    if constexpr (WV) {
#pragma unroll
      for (int rb = 0; rb < 8; ++rb)
        pt[rb] = *reinterpret_cast<const bf16x8*>(smem + kLatP + buf * 8192 + rb * 1024 + prow);
      vf[0] = vread(vbase, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      if (WV && dd + 1 < 8) vf[(dd + 1) & 1] = vread(vbase, dd + 1);
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        if constexpr (WV)
          o[dd][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dd & 1], pt[rb], o[dd][rb], 0, 0, 0);
        // 26 pieces and the publication over the 64 MFMAs: one after every
        // second MFMA of the first 54
        const int slot = dd * 8 + rb;
        if ((slot & 1) && (slot >> 1) < 26) piece((slot >> 1) / 13, (slot >> 1) % 13);
        if (slot == 55) publish();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // rows whose reference max moved in tile j: scale their accumulators
  auto rescale = [&](int j) {
    const uint32_t buf = static_cast<uint32_t>(j & 1);
    const int* fl = reinterpret_cast<const int*>(smem + kLatFlag + buf * 1024 + lane * 4);
    const int fm = __builtin_amdgcn_readfirstlane((fl[0] ? 1 : 0) | (fl[64] ? 2 : 0) | (fl[128] ? 4 : 0) | (fl[192] ? 8 : 0));
    if (fm == 0) return;
    asm volatile("" ::: "memory");  // a real branch: rare after the first tile
    const float* al = reinterpret_cast<const float*>(smem + kLatAlpha + buf * kLatAlphaBuf + (lq * kLatAlphaCopy + lr * 9) * 4);
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      const float f = ((fm >> (rb >> 1)) & 1) ? al[rb] : 1.f;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) o[dd][rb] *= f;
    }
  };

  f32x4 sc[2][2], sn[2][2];
  wait_vmcnt<0>();
  lds_barrier();
  scores_p(sc, lds0);
  mask(sc, 0);
  values_softmax(IC<0>{}, lds0, -1, sc);   // the weights of tile 0 alone

  // Step t: the scores of tile t+1, then the value product of tile t beside
  // the softmax of tile t+1, whose weights the next step reads.  The last
  // step scores a stale slot as tile nt, whose keys all lie past k_end: fully
  // masked, it leaves every row's max and sum unchanged.
  uint32_t s_cur = lds0, s_nxt = lds0 + kLatTile, s_aft = lds0 + 2 * kLatTile;
  for (int t = 0; t < nt; ++t) {
    // tile t+1 resident and the weights of tile t posted; every wave is done
    // with tile t-1, whose slot takes tile t+2
    wait_all_mem();
    lds_barrier();
    if (t + 2 < nt) issue(t + 2, s_aft);
    asm volatile("" : "+v"(vrow), "+v"(vsw));
    rescale(t);
    scores_p(sn, s_nxt);
    mask(sn, t + 1);
    values_softmax(IC<1>{}, s_cur, t, sn);
    const uint32_t s_old = s_cur;
    s_cur = s_nxt;
    s_nxt = s_aft;
    s_aft = s_old;
  }

  // ---- row totals to every wave
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const float l = quad_group_sum(lsum[rg]);
    if (lq == 0)
      *reinterpret_cast<float2*>(smem + kLatStat + (wave * 32 + rg * 16 + lr) * 8) = make_float2(m_run[rg], l);
  }
  __syncthreads();

  if (c.splits == 1) {
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      const int r_loc = rb * 16 + lr;
      const int r = c.rowb * RB + r_loc;
      if (r >= c.rows_b) continue;
      const float2 ml = *reinterpret_cast<const float2*>(smem + kLatStat + r_loc * 8);
      const size_t orow = (static_cast<size_t>(c.b) * a.N_max + r / a.G) * a.Hq + r % a.G;
      uint16_t* op = static_cast<uint16_t*>(a.out) + orow * kLatV + 128 * wave + 4 * lq;
      const float inv = 1.0f / ml.y;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        union {
          uint2 u;
          __bf16 h4[4];
        } pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk.h4[i] = static_cast<__bf16>(o[dd][rb][i] * inv);
        *reinterpret_cast<uint2*>(op + 16 * dd) = pk.u;
      }
      if (a.lse && lq == 0 && (rb >> 1) == wave) a.lse[orow] = (ml.x + log2f(ml.y)) * kLn2;
    }
    return;
  }
  // partial (max, sum, unnormalised accumulator) for the combine kernel
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    const int r_loc = rb * 16 + lr;
    if (c.rowb * RB + r_loc >= c.rows_b) continue;
    const size_t pr = static_cast<size_t>(item) * RB + r_loc;
    float* pa = a.part_acc + pr * kLatV + 128 * wave + 4 * lq;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd)
      *reinterpret_cast<float4*>(pa + 16 * dd) = make_float4(o[dd][rb][0], o[dd][rb][1], o[dd][rb][2], o[dd][rb][3]);
    if (lq == 0 && (rb >> 1) == wave) {
      const float2 ml = *reinterpret_cast<const float2*>(smem + kLatStat + r_loc * 8);
      a.part_ml[pr * 2 + 0] = ml.x;
      a.part_ml[pr * 2 + 1] = ml.y;
    }
  }
}

// --------------------------------------------------------------- VALU path
template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void st_elem(T* p, float v);
template <>
__device__ __forceinline__ void st_elem<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st_elem<uint16_t>(uint16_t* p, float v) {
  __bf16 h = static_cast<__bf16>(v);
  *p = *reinterpret_cast<uint16_t*>(&h);
}

template <typename T>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
  constexpr int R = kValuRows, K = kValuKeys, DM = kValuMaxD;
  __shared__ float sQ[R * DM];
  __shared__ float sK[K * (DM + 1)];
  __shared__ float sV[K * DM];
  __shared__ float sP[R * (K + 1)];
  __shared__ uint32_t sA[R][4];

  ItemCtx c;
  if (!load_item(a, c)) return;
  const int DQ = a.d_qk, DVv = a.d_v, KS = DQ + 1;
  const int tid = threadIdx.x;
  const int row = tid / K, col = tid % K;
  const T* qp = static_cast<const T*>(a.q);
  const T* kc = static_cast<const T*>(a.kc);
  const T* vc = static_cast<const T*>(a.vc);
  const T* kt = static_cast<const T*>(a.kt);
  const T* vt = static_cast<const T*>(a.vt);

  for (int e0 = tid; e0 < R * DQ; e0 += 256 * 8) {
    float qr[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + 256 * u;
      qr[u] = 0.f;
      if (e < R * DQ) {
        const int r = e / DQ, x = e % DQ;
        const int rg = c.rowb * R + r;
        if (rg < c.rows_b) {
          const int node = rg / a.G, h = c.kvh * a.G + rg % a.G;
          qr[u] = ld_elem<T>(qp + ((static_cast<size_t>(c.b) * a.N_max + node) * a.Hq + h) * DQ + x);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + 256 * u;
      if (e < R * DQ) sQ[e] = qr[u];
    }
  }
  if (tid < R * 4) {
    const int r = tid / 4, w = tid % 4;
    const int rg = c.rowb * R + r;
    uint32_t v = 0;
    if (rg < c.rows_b && w < a.W)
      v = a.anc[(static_cast<size_t>(c.b) * a.N_max + rg / a.G) * a.W + w];
    sA[r][w] = v;
  }
  const bool row_ok = c.rowb * R + row < c.rows_b;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[(DM + K - 1) / K];
#pragma unroll
  for (int j = 0; j < (DM + K - 1) / K; ++j) acc[j] = 0.f;

  // A tile's K and V elements are loaded in chunks of CH per thread, every
  // load of a chunk issued before any of its LDS stores.  When one chunk holds
  // the whole tile (head dimensions up to 128), the next tile's loads are
  // issued before this tile's arithmetic, so that their latency overlaps it;
  // a thread's (key, column) pairs are then the same for every tile and are
  // computed once.
  constexpr int CH = 8;
  const int kv_elems = K * (DQ > DVv ? DQ : DVv);
  const bool pipe = kv_elems <= 256 * CH;
  float kr[CH], vr[CH];
  int kkey[CH], kx[CH], vkey[CH], vx[CH];
  auto split_idx = [&](int e0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int e = e0 + 256 * u;
      kkey[u] = e < K * DQ ? e / DQ : -1;
      kx[u] = e < K * DQ ? e % DQ : 0;
      vkey[u] = e < K * DVv ? e / DVv : -1;
      vx[u] = e < K * DVv ? e % DVv : 0;
    }
  };
  auto fetch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      kr[u] = 0.f;
      vr[u] = 0.f;
      if (kkey[u] >= 0 && t0 + kkey[u] < c.k_end) {
        bool tr;
        const long off = key_row(a, c, t0 + kkey[u], &tr) + static_cast<long>(c.kvh) * DQ + kx[u];
        kr[u] = ld_elem<T>((tr ? kt : kc) + off);
      }
      if (vkey[u] >= 0 && t0 + vkey[u] < c.k_end) {
        bool tr;
        const long off = key_row(a, c, t0 + vkey[u], &tr) + static_cast<long>(c.kvh) * DVv + vx[u];
        vr[u] = ld_elem<T>((tr ? vt : vc) + off);
      }
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (kkey[u] >= 0) sK[kkey[u] * KS + kx[u]] = kr[u];
      if (vkey[u] >= 0) sV[vkey[u] * DVv + vx[u]] = vr[u];
    }
  };
  if (pipe) {
    split_idx(tid);
    if (c.k_beg < c.k_end) fetch(c.k_beg);
  }
  for (int t0 = c.k_beg; t0 < c.k_end; t0 += K) {
    __syncthreads();
    if (pipe) {
      put();
    } else {
      for (int e0 = tid; e0 < kv_elems; e0 += 256 * CH) {
        split_idx(e0);
        fetch(t0);
        put();
      }
    }
    __syncthreads();
    if (pipe && t0 + K < c.k_end) fetch(t0 + K);
    // Scores: the dot product in the order x = 0, 1, ..., its LDS reads
    // issued sixteen at a time ahead of their FMAs.
    float s = 0.f;
    {
      const float* qrow = sQ + row * DQ;
      const float* krow = sK + col * KS;
      int x = 0;
      for (; x + 16 <= DQ; x += 16) {
        float qv[16], kv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          qv[u] = qrow[x + u];
          kv[u] = krow[x + u];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) s = fmaf(qv[u], kv[u], s);
      }
      for (; x < DQ; ++x) s = fmaf(qrow[x], krow[x], s);
    }
    const int key = t0 + col;
    const bool ok = row_ok && key_visible(sA[row], key, c.l_b, c.k_end);
    s = ok ? s * a.scale_log2 : -INFINITY;
    float mx = s;
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, K));
    const float mnew = fmaxf(m_run, mx);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(m_run - muse);
    const float p = exp2f(s - muse);
    float ps = p;
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) ps += __shfl_xor(ps, m, K);
    l_run = l_run * alpha + ps;
    m_run = mnew;
    sP[row * (K + 1) + col] = p;
    __syncthreads();
    // Values: column dv = col + K j of the row's output, the keys in order.
    // The test on j is uniform; a lane past d_v reads a clamped column and
    // its result is never stored, so the reads of a column are not split by
    // a divergent branch and issue ahead of their FMAs.
    float pr[K];
#pragma unroll
    for (int kk = 0; kk < K; ++kk) pr[kk] = sP[row * (K + 1) + kk];
#pragma unroll
    for (int j = 0; j < (DM + K - 1) / K; ++j) {
      if (K * j < DVv) {
        const int dv = min(col + K * j, DVv - 1);
        float vv[K];
#pragma unroll
        for (int kk = 0; kk < K; ++kk) vv[kk] = sV[kk * DVv + dv];
        float v = acc[j] * alpha;
#pragma unroll
        for (int kk = 0; kk < K; ++kk) v = fmaf(pr[kk], vv[kk], v);
        acc[j] = v;
      }
    }
  }

  if (!row_ok) return;
  const int r_loc = row;
  const int rg = c.rowb * R + r_loc;
  if (c.splits == 1) {
    const int node = rg / a.G, h = c.kvh * a.G + rg % a.G;
    const size_t orow = (static_cast<size_t>(c.b) * a.N_max + node) * a.Hq + h;
    T* op = static_cast<T*>(a.out) + orow * DVv;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int j = 0; j < (DM + K - 1) / K; ++j) {
      const int dv = col + K * j;
      if (dv < DVv) st_elem<T>(op + dv, acc[j] * inv);
    }
    if (col == 0 && a.lse) a.lse[orow] = (m_run + log2f(l_run)) * kLn2;
  } else {
    const size_t prow = static_cast<size_t>(blockIdx.x) * R + r_loc;
#pragma unroll
    for (int j = 0; j < (DM + K - 1) / K; ++j) {
      const int dv = col + K * j;
      if (dv < DVv) a.part_acc[prow * DVv + dv] = acc[j];
    }
    if (col == 0) {
      a.part_ml[prow * 2 + 0] = m_run;
      a.part_ml[prow * 2 + 1] = l_run;
    }
  }
}

// --------------------------------------------------- combine (MFMA paths)
// One wavefront per (request, node, head) row whose unit was split: lanes
// read the splits' (max, sum) pairs once, then cooperate over splits and
// 16-byte chunks of the fp32 accumulators so every load is independent.
template <int DV>
__global__ __launch_bounds__(256) void attn_combine_vec_kernel(AttnArgs a) {
  constexpr int NCH = DV / 4;                   // float4 chunks per row
  constexpr int GROUPS = NCH >= 64 ? 1 : 64 / NCH;
  constexpr int CPL = NCH >= 64 ? NCH / 64 : 1;  // chunks per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * 4 + wave;
  if (row >= static_cast<long>(a.B) * a.N_max * a.Hq) return;
  const int h = static_cast<int>(row % a.Hq);
  const long bi = row / a.Hq;
  const int i = static_cast<int>(bi % a.N_max);
  const int b = static_cast<int>(bi / a.N_max);
  const int n_b = clampi(a.n_nodes[b], 0, a.N_max);
  if (i >= n_b) return;
  const int splits = a.info[4 * b + 1];
  if (splits <= 1) return;
  const int rbs = a.info[4 * b + 2];
  const int kvh = h / a.G;
  const int r = i * a.G + h % a.G;
  const int rowb = r / a.RB, r_loc = r % a.RB;
  const long item0 = a.info[4 * b] + static_cast<long>(kvh * rbs + rowb) * splits;
  if (item0 + splits > a.items_max) return;
  const float* ml = a.part_ml + (item0 * a.RB + r_loc) * 2;
  const long mstride = static_cast<long>(a.RB) * 2;
  float M = -INFINITY;
  for (int s2 = lane; s2 < splits; s2 += 64) M = fmaxf(M, ml[s2 * mstride]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));
  float L = 0.f;
  for (int s2 = lane; s2 < splits; s2 += 64) {
    const float ms = ml[s2 * mstride];
    L += ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M) * ml[s2 * mstride + 1];
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) L += __shfl_xor(L, m);
  const int grp = lane / (64 / GROUPS);
  const int cl = lane % (64 / GROUPS);
  float4 acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* pa = a.part_acc + (item0 * a.RB + r_loc) * DV;
  const long astride = static_cast<long>(a.RB) * DV;
#pragma unroll 4
  for (int s2 = grp; s2 < splits; s2 += GROUPS) {
    const float ms = ml[s2 * mstride];
    const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float4 v = *reinterpret_cast<const float4*>(pa + s2 * astride + 4 * (cl + 64 * c));
      acc[c].x = fmaf(w, v.x, acc[c].x);
      acc[c].y = fmaf(w, v.y, acc[c].y);
      acc[c].z = fmaf(w, v.z, acc[c].z);
      acc[c].w = fmaf(w, v.w, acc[c].w);
    }
  }
  if (GROUPS == 2) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      acc[c].x += __shfl_xor(acc[c].x, 32);
      acc[c].y += __shfl_xor(acc[c].y, 32);
      acc[c].z += __shfl_xor(acc[c].z, 32);
      acc[c].w += __shfl_xor(acc[c].w, 32);
    }
  }
  const float inv = 1.0f / L;
  const size_t orow = (static_cast<size_t>(b) * a.N_max + i) * a.Hq + h;
  uint16_t* op = static_cast<uint16_t*>(a.out) + orow * DV;
  if (grp == 0) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      union {
        uint2 u;
        __bf16 h4[4];
      } pk;
      pk.h4[0] = static_cast<__bf16>(acc[c].x * inv);
      pk.h4[1] = static_cast<__bf16>(acc[c].y * inv);
      pk.h4[2] = static_cast<__bf16>(acc[c].z * inv);
      pk.h4[3] = static_cast<__bf16>(acc[c].w * inv);
      *reinterpret_cast<uint2*>(op + 4 * (cl + 64 * c)) = pk.u;
    }
  }
  if (lane == 0 && a.lse) a.lse[orow] = (M + log2f(L)) * kLn2;
}

// ----------------------------------------------------------------- combine
template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * 4 + wave;
  if (row >= static_cast<long>(a.B) * a.N_max * a.Hq) return;
  const int h = static_cast<int>(row % a.Hq);
  const long bi = row / a.Hq;
  const int i = static_cast<int>(bi % a.N_max);
  const int b = static_cast<int>(bi / a.N_max);
  const int n_b = clampi(a.n_nodes[b], 0, a.N_max);
  if (i >= n_b) return;
  const int splits = a.info[4 * b + 1];
  if (splits <= 1) return;  // written by the item itself
  const int rbs = a.info[4 * b + 2];
  const int kvh = h / a.G;
  const int r = i * a.G + h % a.G;
  const int rowb = r / a.RB, r_loc = r % a.RB;
  const long item0 = a.info[4 * b] + static_cast<long>(kvh * rbs + rowb) * splits;
  if (item0 + splits > a.items_max) return;
  auto ml = [&](int s, int f) { return a.part_ml[((item0 + s) * a.RB + r_loc) * 2 + f]; };
  float M = -INFINITY;
  for (int s = lane; s < splits; s += 64) M = fmaxf(M, ml(s, 0));
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));
  float L = 0.f;
  for (int s = lane; s < splits; s += 64) {
    const float ms = ml(s, 0);
    L += ms == -INFINITY ? 0.f : exp2f(ms - M) * ml(s, 1);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) L += __shfl_xor(L, m);
  const float inv = 1.0f / L;
  const size_t orow = (static_cast<size_t>(b) * a.N_max + i) * a.Hq + h;
  T* op = static_cast<T*>(a.out) + orow * a.d_v;
  // Split s's weight is held by lane s % 64 of its group of 64 splits and
  // read back by lane index; the partial rows of eight splits are loaded
  // ahead of their FMAs.  The sum runs over s = 0, 1, ... as in the plain
  // loop.
  const float* pa = a.part_acc + (item0 * a.RB + r_loc) * a.d_v;
  const size_t sstride = static_cast<size_t>(a.RB) * a.d_v;
  auto weight = [&](int s) {
    if (s >= splits) return 0.f;
    const float ms = ml(s, 0);
    return ms == -INFINITY ? 0.f : exp2f(ms - M);
  };
  const float w0 = weight(lane);   // the first group, shared by every column pass
  // every lane stays in the column loop (a lane past d_v reads a clamped
  // column and stores nothing), so the weights a lane reads back are always
  // those of the current group
  for (int dv0 = 0; dv0 < a.d_v; dv0 += 64) {
    const int dv = min(dv0 + lane, a.d_v - 1);
    float acc = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 64) {
      const float wl = s0 == 0 ? w0 : weight(s0 + lane);
      const int ns = min(64, splits - s0);
      int t = 0;
      for (; t + 8 <= ns; t += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = pa[(s0 + t + u) * sstride + dv];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), t + u)), x[u], acc);
      }
      for (; t < ns; ++t)
        acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), t)), pa[(s0 + t) * sstride + dv], acc);
    }
    if (dv0 + lane < a.d_v) st_elem<T>(op + dv, acc * inv);
  }
  if (lane == 0 && a.lse) a.lse[orow] = (M + log2f(L)) * kLn2;
}

}  // namespace

AttnPlan attn_plan(const AttnShape& sh, bool aligned, bool shared_value) {
  AttnPlan p;
  const bool bf = sh.dtype == TSV_BF16;
  p.chunk = p.S = p.units = p.rbs = 0;
  // Every path starts its workspace with the grouped path's arrival counters
  // (one int per request x KV head x block of 128 rows), which only that path
  // touches and always leaves at zero.  The region depends on B, N_max, Hq
  // and Hkv only, so one zeroed workspace serves calls of any dtype, path or
  // prefix capacity at those sizes.
  const int G0 = sh.Hq / sh.Hkv;
  const long long cnt_units = static_cast<long long>(sh.B) * sh.Hkv * ((static_cast<long long>(sh.N_max) * G0 + 127) / 128);
  p.off_cnt = 0;
  const size_t cnt_bytes = align_up(static_cast<size_t>((cnt_units + 7) / 8 * 8) * sizeof(int));
  if (bf && aligned && sh.d_qk == 128 && sh.d_v == 128) {
    // One kernel: the key range of every unit (request, KV head, block of
    // 128 rows) is cut into splits of `chunk` keys, sized from the capacity
    // so that about two workgroups per compute unit exist; the launch has S
    // slots per unit and a unit uses ceil(keys / chunk) of them.
    p.path = kPathMfmaGqa;
    p.RB = 128;
    p.KT = 32;
    p.min_chunk = 256;
    p.target_items = 512;
    const int G = sh.Hq / sh.Hkv;
    p.rbs = (sh.N_max * G + p.RB - 1) / p.RB;
    p.units = sh.B * sh.Hkv * p.rbs;
    const int units_pad = (p.units + 7) / 8 * 8;
    const long long keys_max = static_cast<long long>(sh.L_cap) + sh.N_max;
    long long c = (static_cast<long long>(p.units) * keys_max + p.target_items - 1) / p.target_items;
    if (c < p.min_chunk) c = p.min_chunk;
    c = (c + p.KT - 1) / p.KT * p.KT;
    p.S = static_cast<int>((keys_max + c - 1) / c);
    // The capacity sizing above assumes every unit is busy.  When most are
    // not (adaptive budgets leave many requests with few or no nodes, and a
    // unit's rows past n_b * G are idle), the busy units still need their
    // long prefixes cut: at least one split per kSplitKeys keys.
    const long long s_len = (keys_max + kSplitKeys - 1) / kSplitKeys;
    if (p.S < s_len) p.S = static_cast<int>(s_len);
    // the device cuts each unit's actual keys into S chunks, none shorter
    // than the longest possible unit's (at least min_chunk); with many more
    // work items than resident workgroups (the dispatcher then balances the
    // compute units), none shorter than kSplitKeys either, so that a short
    // unit takes fewer splits and fewer partials to publish and read back
    // (measured on the ragged 64-request workload: floors of 3.5k-3.8k keys
    // 407-410 us, 4k-4.5k keys 392-395 us, 5k keys and more 405-430 us)
    p.chunk = static_cast<int>((keys_max + p.S - 1) / p.S + p.KT - 1) / p.KT * p.KT;
    if (p.chunk < p.min_chunk) p.chunk = p.min_chunk;
    if (static_cast<long long>(units_pad) * p.S > 2LL * kResidentGrid && p.chunk < kSplitKeys)
      p.chunk = static_cast<int>(kSplitKeys);
    p.items_max = units_pad * p.S;
    size_t off = cnt_bytes;
    p.off_info = p.off_desc = off;
    p.off_ml = off;
    off = align_up(off + static_cast<size_t>(p.items_max) * p.RB * 2 * sizeof(float));
    p.off_acc = off;
    // partial rows are published normalised, in bf16
    off = align_up(off + static_cast<size_t>(p.items_max) * p.RB * sh.d_v * sizeof(uint16_t));
    p.bytes = off;
    return p;
  } else if (bf && aligned && shared_value && sh.d_qk == 576 && sh.d_v == 512) {
    p.path = kPathMfmaLatent;
    p.RB = 128;
    p.KT = 32;
    p.min_chunk = 256;
    p.target_items = 512;
  } else {
    p.path = kPathValu;
    p.RB = kValuRows;
    p.KT = kValuKeys;
    // small problems are latency-bound: down to one key tile per workgroup
    p.min_chunk = kValuKeys;
    p.target_items = 1024;
  }
  const int G = sh.Hq / sh.Hkv;
  const long units = static_cast<long>(sh.B) * sh.Hkv * ((static_cast<long>(sh.N_max) * G + p.RB - 1) / p.RB);
  const long items = p.target_items + units;
  p.items_max = static_cast<int>(items);
  size_t off = cnt_bytes;
  p.off_info = off;
  off = align_up(off + (4 * static_cast<size_t>(sh.B) + 2) * sizeof(int));
  p.off_desc = off;
  off = align_up(off + static_cast<size_t>(items) * sizeof(int4));
  p.off_ml = off;
  off = align_up(off + static_cast<size_t>(items) * p.RB * 2 * sizeof(float));
  p.off_acc = off;
  off = align_up(off + static_cast<size_t>(items) * p.RB * sh.d_v * sizeof(float));
  p.bytes = off;
  return p;
}

hipError_t launch_attention(const AttnArgs& a, AttnPath path, int dtype, hipStream_t s) {
  if (path == kPathMfmaGqa) {
    attn_gqa_pipe_kernel<5><<<dim3(a.items_max), dim3(256), 0, s>>>(a);
    return hipGetLastError();
  }
  attn_plan_kernel<<<dim3(1), dim3(kPlanThreads), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(a.items_max), block(256);
  if (path == kPathMfmaLatent) {
    attn_latent_kernel<<<dim3((a.items_max + 7) / 8 * 8), block, 0, s>>>(a);
  } else if (dtype == TSV_F32) {
    attn_valu_kernel<float><<<grid, block, 0, s>>>(a);
  } else {
    attn_valu_kernel<uint16_t><<<grid, block, 0, s>>>(a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = static_cast<long>(a.B) * a.N_max * a.Hq;
  dim3 g2(static_cast<unsigned>((rows + 3) / 4));
  if (path == kPathMfmaLatent)
    attn_combine_vec_kernel<512><<<g2, block, 0, s>>>(a);
  else if (dtype == TSV_F32)
    attn_combine_kernel<float><<<g2, block, 0, s>>>(a);
  else
    attn_combine_kernel<uint16_t><<<g2, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tsv
