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

// Cache append: dst[b][dst_start + i] = src[b][i] for i < n, rows of row_bytes
// (a multiple of 4).  One 4-, 8- or 16-byte word per thread, as wide as the
// rows' alignment allows (key rows and pool rows move 16 bytes a thread, the
// per-entry fp32 scales 4).
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(int n, int words_per_row, long long total,
                                                     const T* __restrict__ src,
                                                     long long src_stride_words,
                                                     T* __restrict__ dst,
                                                     long long dst_stride_words,
                                                     long long dst_start_words) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long long per_b = (long long)n * words_per_row;
  const long long b = i / per_b;
  const long long w = i - b * per_b;
  dst[b * dst_stride_words + dst_start_words + w] = src[b * src_stride_words + w];
}

template <typename T>
hipError_t launch_append_t(int B, int n, int row_bytes, const void* src, int64_t src_stride,
                           void* dst, int64_t dst_stride, int64_t dst_start, hipStream_t s) {
  const int wpr = row_bytes / (int)sizeof(T);
  const long long total = (long long)B * n * wpr;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, n, wpr, total,
                     (const T*)src, (long long)src_stride * wpr, (T*)dst,
                     (long long)dst_stride * wpr, (long long)dst_start * wpr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_rows(int B, int n, int row_bytes, const void* src, int64_t src_stride,
                              void* dst, int64_t dst_stride, int64_t dst_start, hipStream_t s) {
  if ((long long)B * n == 0) return hipSuccess;
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst;
  if (row_bytes % 16 == 0 && al % 16 == 0)
    return launch_append_t<u32x4>(B, n, row_bytes, src, src_stride, dst, dst_stride, dst_start, s);
  if (row_bytes % 8 == 0 && al % 8 == 0)
    return launch_append_t<u32x2>(B, n, row_bytes, src, src_stride, dst, dst_stride, dst_start, s);
  return launch_append_t<uint32_t>(B, n, row_bytes, src, src_stride, dst, dst_stride, dst_start,
                                   s);
}

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
