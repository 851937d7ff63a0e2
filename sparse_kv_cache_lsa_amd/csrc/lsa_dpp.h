// lsa_dpp.h -- wavefront scans and reductions with DPP moves (gfx950).
//
// A 64-lane scan in six dependent vector steps: row shifts by 1, 2, 4 and 8
// inside each 16-lane row, then the broadcast of lane 15 of rows 0 and 2 into
// rows 1 and 3 and of lane 31 into rows 2 and 3.  Lanes whose source lies
// outside their row, or whose row is masked off, keep the identity.  A
// shuffle (ds_bpermute) costs a round trip through the LDS pipeline per
// step; these stay in the vector ALU.  Reductions take the scan's last lane.
#pragma once

#include "lsa_device.h"

namespace lsa {

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_move(uint32_t identity, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWS, 0xF, false);
}

// Inclusive scan of v over the wavefront in lane order with an associative
// operation op whose identity is id (32-bit values).
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_move<0x111, 0xF>(id, v));   // row_shr:1
  v = op(v, dpp_move<0x112, 0xF>(id, v));   // row_shr:2
  v = op(v, dpp_move<0x114, 0xF>(id, v));   // row_shr:4
  v = op(v, dpp_move<0x118, 0xF>(id, v));   // row_shr:8
  v = op(v, dpp_move<0x142, 0xA>(id, v));   // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_move<0x143, 0xC>(id, v));   // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ int wave_inclusive_sum_dpp(int v) {
  return (int)wave_scan_dpp((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// 64-bit inclusive sum: each step moves both halves, then adds with carry.
__device__ __forceinline__ uint64_t wave_inclusive_sum_u64_dpp(uint64_t v) {
#define LSA_DPP_U64_STEP(CTRL, ROWS)                                              \
  {                                                                              \
    const uint32_t lo = dpp_move<CTRL, ROWS>(0u, (uint32_t)v);                   \
    const uint32_t hi = dpp_move<CTRL, ROWS>(0u, (uint32_t)(v >> 32));           \
    v += ((uint64_t)hi << 32) | lo;                                              \
  }
  LSA_DPP_U64_STEP(0x111, 0xF)
  LSA_DPP_U64_STEP(0x112, 0xF)
  LSA_DPP_U64_STEP(0x114, 0xF)
  LSA_DPP_U64_STEP(0x118, 0xF)
  LSA_DPP_U64_STEP(0x142, 0xA)
  LSA_DPP_U64_STEP(0x143, 0xC)
#undef LSA_DPP_U64_STEP
  return v;
}

// Reductions: the value of the last lane of the scan, the same in every lane.
__device__ __forceinline__ uint32_t wave_last_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
__device__ __forceinline__ int wave_sum_dpp(int v) {
  return (int)wave_last_lane((uint32_t)wave_inclusive_sum_dpp(v));
}
__device__ __forceinline__ uint32_t wave_min_u32_dpp(uint32_t v) {
  return wave_last_lane(
      wave_scan_dpp(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; }));
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  return wave_last_lane(wave_scan_dpp(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }));
}
__device__ __forceinline__ float wave_max_f32_dpp(float v) {
  const uint32_t r = wave_scan_dpp(__float_as_uint(v), __float_as_uint(-__builtin_inff()),
                                   [](uint32_t a, uint32_t b) {
                                     return __float_as_uint(fmaxf(__uint_as_float(a),
                                                                  __uint_as_float(b)));
                                   });
  return __uint_as_float(wave_last_lane(r));
}

}  // namespace lsa
