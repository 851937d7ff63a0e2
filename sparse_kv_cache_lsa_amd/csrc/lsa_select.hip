// lsa_select.hip -- OR merge of the indexer layers' selections and survivor
// compaction (gist.science technical summary, section 2.4: the layer
// predictions are united in OR mode; paper.oopus.info review, section 2: any
// layer asking for an entry fetches it).
//
// Two passes, both deterministic:
//  1. count:  one thread per 32-entry word ORs the L selection words and
//     popcounts; a block reduction gives the survivors of each chunk.
//  2. write:  each chunk block sums the counts of the chunks before it (its
//     output offset), then walks its entries 256 at a time: a lane per entry,
//     wavefront ballot + mbcnt for the rank inside the wave, a 4-entry LDS
//     prefix for the waves, so survivors land in ascending entry order.
//     The merged score is the max over layers (NaN ignored).
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kChunk = 8192;           // entries per chunk (256 words)
constexpr int kWordsPerChunk = kChunk / 32;

__global__ __launch_bounds__(256) void select_count_kernel(const uint32_t* __restrict__ mask,
                                                           int L, int B, int W, int nch,
                                                           int* __restrict__ counts) {
  __shared__ int red[4];
  const int b = blockIdx.y;
  const int w = blockIdx.x * kWordsPerChunk + threadIdx.x;
  uint32_t m = 0;
  if (w < W)
    for (int l = 0; l < L; ++l) m |= mask[((size_t)l * B + b) * W + w];
  int c = wave_sum(__popc(m));
  if (lane_id() == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) counts[(size_t)b * nch + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void select_write_kernel(
    const uint32_t* __restrict__ mask, const float* __restrict__ z, int L, int B, int N,
    int W, int nch, const int* __restrict__ counts, int cap, int32_t* __restrict__ surv_idx,
    float* __restrict__ surv_z, int32_t* __restrict__ surv_count) {
  __shared__ int s_base;
  __shared__ int s_wave[4];
  const int b = blockIdx.y;
  const int ch = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (threadIdx.x < kWave) {
    int acc = 0;
    for (int i = lane; i < ch; i += kWave) acc += counts[(size_t)b * nch + i];
    acc = wave_sum(acc);
    if (lane == 0) s_base = acc;
  }
  __syncthreads();
  int base = s_base;
  const int e_end = min(N, (ch + 1) * kChunk);
  for (int e0 = ch * kChunk; e0 < e_end; e0 += 256) {
    const int s = e0 + threadIdx.x;
    bool f = false;
    if (s < N) {
      uint32_t m = 0;
      for (int l = 0; l < L; ++l) m |= mask[((size_t)l * B + b) * W + (s >> 5)];
      f = (m >> (s & 31)) & 1u;
    }
    const uint64_t bal = __ballot(f);
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = s_wave[i];
      before += (i < wave) ? c : 0;
      total += c;
    }
    if (f) {
      const int pos = base + before + lanes_below(bal);
      if (pos < cap) {
        float zm = __builtin_nanf("");
        for (int l = 0; l < L; ++l) zm = fmaxf(zm, z[((size_t)l * B + b) * N + s]);
        surv_idx[(size_t)b * cap + pos] = s;
        surv_z[(size_t)b * cap + pos] = zm;
      }
    }
    base += total;
    __syncthreads();
  }
  if (ch == nch - 1 && threadIdx.x == 0) surv_count[b] = base;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

size_t select_workspace(int B, int N) {
  const int nch = (N + kChunk - 1) / kChunk;
  return (size_t)B * (size_t)(nch > 0 ? nch : 1) * sizeof(int);
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_select(int L, int B, int N, const uint32_t* mask, const float* z, int cap,
                         int32_t* surv_idx, float* surv_z, int32_t* surv_count, void* ws,
                         hipStream_t s) {
  if (N == 0) return launch_fill_i32(surv_count, B, 0, s);
  const int W = (N + 31) / 32;
  const int nch = (N + kChunk - 1) / kChunk;
  int* counts = (int*)ws;
  hipLaunchKernelGGL(select_count_kernel, dim3(nch, B), dim3(256), 0, s, mask, L, B, W, nch,
                     counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_write_kernel, dim3(nch, B), dim3(256), 0, s, mask, z, L, B, N, W,
                     nch, counts, cap, surv_idx, surv_z, surv_count);
  return hipGetLastError();
}

}  // namespace lsa
