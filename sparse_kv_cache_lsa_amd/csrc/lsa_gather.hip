// lsa_gather.hip -- hot-pool gather (gist.science technical summary, section
// 2.1 "dynamic fetch": the selected compressed KV entries are brought into GPU
// memory).  hot[b][j] = pool[b][idx[b][j]], zero rows for idx outside [0, N).
//
// One 16-byte chunk per thread: a 1 KiB row is one wavefront-wide load and
// store, so every row moves as full cache lines; rows are independent, so
// the grid is as wide as the hot pool.
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

__global__ __launch_bounds__(256) void gather_kernel(int N, int k, int chunks_per_row,
                                                     long long total_chunks,
                                                     const unsigned char* __restrict__ pool,
                                                     const int32_t* __restrict__ idx,
                                                     unsigned char* __restrict__ hot) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total_chunks) return;
  const long long row = i / chunks_per_row;          // b * k + j
  const int c = (int)(i - row * chunks_per_row);
  const long long b = row / k;
  const int s = idx[row];
  const long long row_bytes = 16ll * chunks_per_row;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (s >= 0 && s < N)
    v = __builtin_nontemporal_load((const u32x4*)(pool + ((b * N + s) * row_bytes) + 16ll * c));
  *(u32x4*)(hot + row * row_bytes + 16ll * c) = v;
}

}  // namespace

hipError_t launch_gather(int B, int N, int k, int row_bytes, const void* pool,
                         const int32_t* idx, void* hot, hipStream_t s) {
  const int cpr = row_bytes / 16;
  const long long total = (long long)B * k * cpr;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, N, k, cpr, total,
                     (const unsigned char*)pool, idx, (unsigned char*)hot);
  return hipGetLastError();
}

}  // namespace lsa
