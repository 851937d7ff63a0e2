// lsa_select_masks.hip -- OR merge and survivor compaction of per-layer
// selection masks and logits from any source (the union of the indexer
// layers' selections, gist.science technical summary, section 2.4 "OR mode";
// every selected entry is fetched, section 2.1 "dynamic fetch").
//
// The fused path (lsa_score's chunk candidate lists + lsa_select_or_compact)
// never writes dense per-layer logits.  This path takes them as inputs: masks
// [L][B][W] and logits [L][B][N], as lsa_score writes with z_opt, or as any
// other producer writes them.  Two launches:
//   1. count:  one block per (chunk of LSA_CAND_CHUNK entries, request) ORs the
//      layers' words of its chunk and stores the chunk's survivor count;
//   2. write:  the same grid; a block's output offset is the sum of the counts
//      of the earlier chunks of its request, a block-wide prefix over its
//      words places every survivor, and each survivor's merged logit is the
//      maximum of its L logits (NaN ignored, all-NaN gives NaN).
// Survivors come out in ascending entry order; at most cap are written and
// the last chunk's block stores the true count.  Deterministic.
#include "lsa_device.h"
#include "lsa_dpp.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kWordsPerChunk = LSA_CAND_CHUNK / 32;   // one thread per 32-entry word
static_assert(kWordsPerChunk == 128, "two wavefronts per chunk");

// Bits of word w that stand for entries below N.
__device__ __forceinline__ uint32_t valid_bits(int w, int N) {
  const int left = N - 32 * w;
  return left >= 32 ? 0xFFFFFFFFu : (left <= 0 ? 0u : ((1u << left) - 1u));
}

__device__ __forceinline__ uint32_t or_word(int L, int B, int W, int N, int b, int w,
                                            const uint32_t* __restrict__ mask) {
  if (w >= W) return 0u;
  uint32_t m = 0u;
  for (int l = 0; l < L; ++l) m |= mask[((size_t)l * B + b) * W + w];
  return m & valid_bits(w, N);
}

__global__ __launch_bounds__(kWordsPerChunk) void mask_count_kernel(
    int L, int B, int N, int W, int nchunks, const uint32_t* __restrict__ mask,
    int32_t* __restrict__ counts) {
  __shared__ int s_part[kWordsPerChunk / kWave];
  const int c = blockIdx.x, b = blockIdx.y;
  const int w = c * kWordsPerChunk + (int)threadIdx.x;
  const int n = wave_sum_dpp(__popc(or_word(L, B, W, N, b, w, mask)));
  if (lane_id() == 0) s_part[threadIdx.x / kWave] = n;
  __syncthreads();
  if (threadIdx.x == 0) counts[(size_t)b * nchunks + c] = s_part[0] + s_part[1];
}

__global__ __launch_bounds__(kWordsPerChunk) void mask_write_kernel(
    int L, int B, int N, int W, int nchunks, const uint32_t* __restrict__ mask,
    const float* __restrict__ z, const int32_t* __restrict__ counts, int cap,
    int32_t* __restrict__ surv_idx, float* __restrict__ surv_z,
    int32_t* __restrict__ surv_count) {
  __shared__ int s_scan[kWordsPerChunk / kWave + 1];
  __shared__ int s_base;
  const int c = blockIdx.x, b = blockIdx.y;
  const int w = c * kWordsPerChunk + (int)threadIdx.x;
  if (threadIdx.x < kWave) {
    const int32_t* cnt = counts + (size_t)b * nchunks;
    int acc = 0;
    for (int i = lane_id(); i < c; i += kWave) acc += cnt[i];
    acc = wave_sum_dpp(acc);
    if (lane_id() == 0) s_base = acc;
  }
  uint32_t m = or_word(L, B, W, N, b, w, mask);
  int total;
  // the scan's barriers also publish s_base
  const int before = block_exclusive_scan<kWordsPerChunk>(__popc(m), s_scan, &total);
  const int base = s_base;
  int pos = base + before;
  int32_t* oi = surv_idx + (size_t)b * cap;
  float* oz = surv_z + (size_t)b * cap;
  while (m != 0u && pos < cap) {
    const int j = __builtin_ctz(m);
    m &= m - 1u;
    const int s = 32 * w + j;
    float zm = __builtin_nanf("");
    for (int l = 0; l < L; ++l) zm = fmaxf(zm, z[((size_t)l * B + b) * N + s]);
    oi[pos] = s;
    oz[pos] = zm;
    ++pos;
  }
  if (c == nchunks - 1 && threadIdx.x == 0) surv_count[b] = base + total;
}

}  // namespace

size_t select_masks_workspace_bytes(int B, int N) {
  const size_t nchunks = ((size_t)N + LSA_CAND_CHUNK - 1) / LSA_CAND_CHUNK;
  return nchunks == 0 ? 0 : ((size_t)B * nchunks * 4 + 255) / 256 * 256;
}

hipError_t launch_select_masks(int L, int B, int N, const uint32_t* mask, const float* z, int cap,
                               int32_t* surv_idx, float* surv_z, int32_t* surv_count, void* ws,
                               hipStream_t s) {
  const int nchunks = (N + LSA_CAND_CHUNK - 1) / LSA_CAND_CHUNK;
  if (nchunks == 0) return launch_fill_i32(surv_count, B, 0, s);
  const int W = (N + 31) / 32;
  int32_t* counts = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(mask_count_kernel, dim3(nchunks, B), dim3(kWordsPerChunk), 0, s, L, B, N, W,
                     nchunks, mask, counts);
  hipLaunchKernelGGL(mask_write_kernel, dim3(nchunks, B), dim3(kWordsPerChunk), 0, s, L, B, N, W,
                     nchunks, mask, z, counts, cap, surv_idx, surv_z, surv_count);
  return hipGetLastError();
}

}  // namespace lsa
