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
#include "lsa_launch.h"

namespace lsa {
namespace {

__global__ __launch_bounds__(256) void select_concat_kernel(
    int nchunks, const int32_t* __restrict__ cand_idx, const float* __restrict__ cand_z,
    const int32_t* __restrict__ cand_count, int cap, int32_t* __restrict__ surv_idx,
    float* __restrict__ surv_z, int32_t* __restrict__ surv_count) {
  __shared__ int s_base;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int32_t* cnt = cand_count + (size_t)b * nchunks;
  if (threadIdx.x < kWave) {
    int acc = 0;
    for (int i = lane_id(); i < c; i += kWave) acc += cnt[i];
    acc = wave_sum(acc);
    if (lane_id() == 0) s_base = acc;
  }
  __syncthreads();
  const int base = s_base;
  const int n = cnt[c];
  const int32_t* ci = cand_idx + ((size_t)b * nchunks + c) * LSA_CAND_CHUNK;
  const float* cz = cand_z + ((size_t)b * nchunks + c) * LSA_CAND_CHUNK;
  const int lim = min(n, cap - base);
  for (int i = threadIdx.x; i < lim; i += blockDim.x) {
    surv_idx[(size_t)b * cap + base + i] = ci[i];
    surv_z[(size_t)b * cap + base + i] = cz[i];
  }
  if (c == nchunks - 1 && threadIdx.x == 0) surv_count[b] = base + n;
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
  hipLaunchKernelGGL(select_concat_kernel, dim3(nchunks, B), dim3(256), 0, s, nchunks, cand_idx,
                     cand_z, cand_count, cap, surv_idx, surv_z, surv_count);
  return hipGetLastError();
}

}  // namespace lsa
