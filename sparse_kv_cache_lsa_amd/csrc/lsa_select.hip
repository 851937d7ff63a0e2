// lsa_select.hip -- survivor compaction: concatenation of the per-chunk
// candidate lists that the scoring kernel leaves after its OR merge (the
// union of the indexer layers' selections, gist.science technical summary,
// section 2.4), into one ascending survivor list per request.
//
// One block per (chunk, request): the block's output offset is the sum of
// the counts of the earlier chunks of its request (a wavefront reduction),
// then it copies its list with coalesced loads and stores.  Deterministic; the
// last chunk's block writes the request's true survivor count.
#include "lsa_device.h"
#include "lsa_dpp.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kSelThreads = 256;

__global__ __launch_bounds__(kSelThreads) void select_concat_kernel(
    int nchunks, const int32_t* __restrict__ cand_idx, const float* __restrict__ cand_z,
    const int32_t* __restrict__ cand_count, int cap, int32_t* __restrict__ surv_idx,
    float* __restrict__ surv_z, int32_t* __restrict__ surv_count) {
  __shared__ int s_base;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int32_t* cnt = cand_count + (size_t)b * nchunks;
  const int n = cnt[c];   // in flight together with the earlier chunks' counts
  if (t < kWave) {
    int acc = 0;
    for (int i = lane_id(); i < c; i += kWave) acc += cnt[i];
    acc = wave_sum_dpp(acc);
    if (lane_id() == 0) s_base = acc;
  }
  __syncthreads();
  const int base = s_base;
  const int lim = max(0, min(n, cap - base));
  // the whole list in one round of loads: thread t takes entries t + 256 r;
  // the buffer range check reads 0 past lim, the stores are predicated
  const size_t list = (size_t)b * nchunks + c;
  const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(cand_idx + list * LSA_CAND_CHUNK), (short)0, lim * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(cand_z + list * LSA_CAND_CHUNK), (short)0, lim * 4, 0x00020000);
  constexpr int R = LSA_CAND_CHUNK / kSelThreads;
  int vi[R], vz[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t off = (uint32_t)(r * kSelThreads + t) * 4;
    vi[r] = __builtin_amdgcn_raw_buffer_load_b32(ri, off, 0, 0);
    vz[r] = __builtin_amdgcn_raw_buffer_load_b32(rz, off, 0, 0);
  }
  int32_t* oi = surv_idx + (size_t)b * cap + base;
  int32_t* oz = (int32_t*)(surv_z + (size_t)b * cap + base);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * kSelThreads + t;
    if (e < lim) {
      oi[e] = vi[r];
      oz[e] = vz[r];
    }
  }
  if (c == nchunks - 1 && t == 0) surv_count[b] = base + n;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_select(int B, int nchunks, const int32_t* cand_idx, const float* cand_z,
                         const int32_t* cand_count, int cap, int32_t* surv_idx, float* surv_z,
                         int32_t* surv_count, hipStream_t s) {
  if (nchunks == 0) return launch_fill_i32(surv_count, B, 0, s);
  hipLaunchKernelGGL(select_concat_kernel, dim3(nchunks, B), dim3(kSelThreads), 0, s, nchunks, cand_idx,
                     cand_z, cand_count, cap, surv_idx, surv_z, surv_count);
  return hipGetLastError();
}

}  // namespace lsa
