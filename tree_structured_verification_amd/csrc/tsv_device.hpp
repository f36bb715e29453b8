// Device helpers shared by the tsv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsv {

constexpr int kWave = 64;

// Order-preserving map of an fp32 bit pattern to uint32 (IEEE order for
// non-NaN values; -0 is mapped to +0 so the two compare equal).
__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Selection key: larger is better; value first, then the LOWER index.
// Never 0 for a real element, so 0 serves as "empty".
__device__ __forceinline__ uint64_t sel_key(float v, uint32_t idx) {
  return (static_cast<uint64_t>(ord_f32(v)) << 32) |
         static_cast<uint64_t>(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t sel_key_index(uint64_t k) {
  return 0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src_lane) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl(lo, src_lane);
  hi = __shfl(hi, src_lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, mask);
  hi = __shfl_xor(hi, mask);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), lane);
  uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Wave-wide max of an unsigned 32-bit value with DPP (pairs, quads, 8- and
// 16-lane mirrors) and four readlanes; returns the max in every lane.
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v),
                                                           CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = umax32(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = umax32(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = umax32(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return umax32(umax32(r0, r1), umax32(r2, r3));
}

// Value of lane (lane ^ J), J in {1, 2, 4, 8, 16, 32}, with VALU lane
// operations only (DPP within 16-lane rows, permlane swaps across rows); the
// whole wavefront must be active.
//   row_ror:N gives lane i the value of lane (i - N) mod 16 of its row;
//   permlane16/32_swap return (value of the lower lane of the pair, value of
//   the upper lane) in every lane of the pair.
template <int J>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  if constexpr (J == 1) {
    return dpp_u32<0xB1>(v);   // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return dpp_u32<0x4E>(v);   // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    // Two writes with complementary bank masks (bank = lanes 4b..4b+3 of a
    // row): banks 0 and 2 take lane i + 4 (row_ror:12), banks 1 and 3 take
    // lane i - 4 (row_ror:4).  No lane-dependent select, which the compiler
    // may turn into EXEC-masked branches around the DPP moves (a DPP move
    // then reads inactive lanes and returns its old value).
    const int t = __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x12C, 0xF, 0x5, false);
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(t, static_cast<int>(v), 0x124, 0xF, 0xA, false));
  } else if constexpr (J == 8) {
    return dpp_u32<0x128>(v);  // row_ror:8
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}
template <int J>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v) {
  const uint32_t lo = xor_lane_u32<J>(static_cast<uint32_t>(v));
  const uint32_t hi = xor_lane_u32<J>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// Value of lane 63 - lane: mirror inside the row (lane ^ 15), then lane ^ 16
// and lane ^ 32.
__device__ __forceinline__ uint64_t reverse_lanes_u64(uint64_t v) {
  uint32_t lo = dpp_u32<0x140>(static_cast<uint32_t>(v));   // row_mirror
  uint32_t hi = dpp_u32<0x140>(static_cast<uint32_t>(v >> 32));
  lo = xor_lane_u32<32>(xor_lane_u32<16>(lo));
  hi = xor_lane_u32<32>(xor_lane_u32<16>(hi));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One compare-exchange stage of a bitonic network over the 64 lanes: lanes
// l and l ^ J swap so that the block of K lanes holding l ends up descending
// (or ascending, for every other block when K < 64).
template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_stage(uint64_t x, int lane) {
  const uint64_t y = xor_lane_u64<J>(x);
  const bool lower = (lane & J) == 0;
  const bool desc = (lane & K) == 0;
  return (lower == desc) ? umax64(x, y) : umin64(x, y);
}
template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_pass(uint64_t x, int lane) {
  x = bitonic_stage<K, J>(x, lane);
  if constexpr (J > 1) x = bitonic_pass<K, J / 2>(x, lane);
  return x;
}
// Sorts one key per lane, descending over lanes 0..63.
__device__ __forceinline__ uint64_t sort64_desc(uint64_t x, int lane) {
  x = bitonic_pass<2, 1>(x, lane);
  x = bitonic_pass<4, 2>(x, lane);
  x = bitonic_pass<8, 4>(x, lane);
  x = bitonic_pass<16, 8>(x, lane);
  x = bitonic_pass<32, 16>(x, lane);
  return bitonic_pass<64, 32>(x, lane);
}

// max(a, b, c) of finite floats in one instruction.  Written as asm because
// the compiler quiets signalling NaNs of loaded values before fmaxf (one
// extra instruction per value); inputs here are finite by contract.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Wave-wide maximum of a 64-bit key (every lane gets it).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, xor_lane_u64<32>(v));
  v = umax64(v, xor_lane_u64<16>(v));
  v = umax64(v, xor_lane_u64<8>(v));
  v = umax64(v, xor_lane_u64<4>(v));
  v = umax64(v, xor_lane_u64<2>(v));
  return umax64(v, xor_lane_u64<1>(v));
}

// Orders LDS traffic of one wavefront around a point where lanes exchange
// data through LDS.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

}  // namespace tsv
