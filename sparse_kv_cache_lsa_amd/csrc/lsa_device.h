// lsa_device.h -- gfx950 device helpers shared by the LSA kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Order LDS traffic of one wavefront: the wave's lanes exchange data through
// LDS, which a wavefront executes in issue order; the fences only stop the
// compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float softplus_f32(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

// Eight e4m3 codes (two dwords, byte order = element order) -> eight bf16.
// Every e4m3 value is exactly representable in bf16, so this is exact.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(u32x2 raw) {
  u32x4 out;
  bf16x2 v;
  v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false);
  out[0] = __builtin_bit_cast(unsigned, v);
  v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true);
  out[1] = __builtin_bit_cast(unsigned, v);
  v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false);
  out[2] = __builtin_bit_cast(unsigned, v);
  v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true);
  out[3] = __builtin_bit_cast(unsigned, v);
  return __builtin_bit_cast(bf16x8, out);
}

// x[lane] + x[lane ^ 32].  v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second; called with the same value
// twice, the two results hold x of one half and x of the other half, so their
// sum is the pair sum in every lane (and the same bits in both lanes).
__device__ __forceinline__ float add_halves(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Number of set bits of a 64-lane ballot below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum across a wavefront (lane order).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Exclusive prefix sum across a block of NT threads in thread order; the
// block total is returned in *total.  `scratch` needs NT/64 + 1 ints of LDS.
// Contains __syncthreads(): every thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[NW] = run;
  }
  __syncthreads();
  int res = scratch[wave] + inc - v;
  *total = scratch[NW];
  __syncthreads();
  return res;
}

}  // namespace lsa
