// lsa_topk.hip -- top-k inside the fetched set (gist.science technical
// summary, section 2.1 "hierarchical selection": once the fetched subset is on
// the GPU, a fine-grained top-k runs inside it).
//
// One 1024-thread block per request.  Ranking: merged logit descending, lower
// entry index first on ties; the selected entries are emitted in ascending
// entry order.
//  * Scores map to order-preserving 32-bit keys (+0 == -0, NaN lowest).
//  * Radix select over the key in three passes (12, 10, 10 bits) with LDS
//    histograms finds the exact key T of the k-th best survivor and how many
//    survivors with key == T still belong to the top-k.  A 12-bit first digit
//    keeps LDS-atomic contention low: the sign+exponent+3 mantissa bits of
//    the logits already spread over many bins.
//  * One ordered sweep then keeps every key > T and the first ones equal to T
//    (the survivor list is ascending, so array order is index order), with
//    block prefix sums giving each kept entry its output slot.
// Lists of up to kThreads * kReg survivors (80K) are read from memory once:
// thread i keeps the keys of positions [i*kReg, (i+1)*kReg) in registers for
// every pass, and the sweep needs only two block prefix sums.  Longer lists
// stream from memory in every pass.
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kReg = 80;   // keys per thread held in registers

__device__ __forceinline__ uint32_t order_key(float z) {
  if (z != z) return 0u;            // NaN ranks last
  if (z == 0.f) z = 0.f;            // -0 and +0 are the same score
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Finds, scanning bins from the highest digit down, the bin holding the
// krem-th key; returns the digit and the number of keys in higher bins.
template <int NB>
__device__ __forceinline__ void find_crossing(const int* hist, int krem, int* scratch,
                                              int* out_digit, int* out_above) {
  constexpr int PER = NB / kThreads;   // 4 or 1 bins per thread
  const int t = threadIdx.x;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += hist[NB - 1 - (t * PER + i)];
  int total;
  const int before = block_exclusive_scan<kThreads>(sum, scratch, &total);
  if (before < krem && krem <= before + sum) {
    int cum = before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = NB - 1 - (t * PER + i);
      if (cum + hist[d] >= krem) {
        *out_digit = d;
        *out_above = cum;
        break;
      }
      cum += hist[d];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void topk_kernel(int cap, int k,
                                                        const int32_t* __restrict__ surv_idx,
                                                        const float* __restrict__ surv_z,
                                                        const int32_t* __restrict__ surv_count,
                                                        int32_t* __restrict__ out,
                                                        int32_t* __restrict__ out_count) {
  __shared__ int hist[4096];
  __shared__ int scratch[kThreads / kWave + 1];
  __shared__ int s_digit, s_above;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int n = min(max(surv_count[b], 0), cap);
  const int32_t* si = surv_idx + (size_t)b * cap;
  const float* sz = surv_z + (size_t)b * cap;
  int32_t* o = out + (size_t)b * k;

  if (k == 0) {
    if (t == 0) out_count[b] = 0;
    return;
  }
  if (n <= k) {
    for (int i = t; i < k; i += kThreads) o[i] = i < n ? si[i] : -1;
    if (t == 0) out_count[b] = n;
    return;
  }

  if (n <= kThreads * kReg) {
    // ---- register-resident path
    const int base = t * kReg;
    uint32_t key[kReg];
    if ((cap & 3) == 0 && ((uintptr_t)sz & 15) == 0 && base + kReg <= n) {
#pragma unroll
      for (int j = 0; j < kReg; j += 4) {
        const f32x4 v = *(const f32x4*)(sz + base + j);
        key[j] = order_key(v[0]);
        key[j + 1] = order_key(v[1]);
        key[j + 2] = order_key(v[2]);
        key[j + 3] = order_key(v[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kReg; ++j) key[j] = base + j < n ? order_key(sz[base + j]) : 0u;
    }
    const int nv = min(kReg, max(0, n - base));   // valid keys of this thread
    uint32_t prefix = 0;
    int krem = k;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
      const int NB = pass == 0 ? 4096 : 1024;
      const int hi = pass == 0 ? 32 : shift + 10;
      for (int i = t; i < NB; i += kThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kReg; ++j)
        if (j < nv && (hi >= 32 || (key[j] >> hi) == (prefix >> hi)))
          atomicAdd(&hist[(key[j] >> shift) & (NB - 1)], 1);
      __syncthreads();
      if (pass == 0)
        find_crossing<4096>(hist, krem, scratch, &s_digit, &s_above);
      else
        find_crossing<1024>(hist, krem, scratch, &s_digit, &s_above);
      prefix |= (uint32_t)s_digit << shift;
      krem -= s_above;
      __syncthreads();
    }
    const uint32_t T = prefix;
    int ties = 0, above = 0;
#pragma unroll
    for (int j = 0; j < kReg; ++j) {
      ties += (j < nv && key[j] == T) ? 1 : 0;
      above += (j < nv && key[j] > T) ? 1 : 0;
    }
    int tie_total;
    const int tie_rank0 = block_exclusive_scan<kThreads>(ties, scratch, &tie_total);
    const int take_ties = min(ties, max(0, krem - tie_rank0));
    int kept_total;
    int pos = block_exclusive_scan<kThreads>(above + take_ties, scratch, &kept_total);
    int tie_rank = tie_rank0;
#pragma unroll
    for (int j = 0; j < kReg; ++j) {
      bool keep = false;
      if (j < nv) {
        if (key[j] > T) keep = true;
        else if (key[j] == T) keep = tie_rank++ < krem;
      }
      if (keep && pos < k) o[pos++] = si[base + j];
    }
    if (t == 0) out_count[b] = k;
    return;
  }

  // ---- radix select of the k-th largest key (long lists, streamed)
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  const int shifts[3] = {20, 10, 0};
  const int nbins[3] = {4096, 1024, 1024};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int NB = nbins[pass];
    for (int i = t; i < NB; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int i = t; i < n; i += kThreads) {
      const uint32_t key = order_key(sz[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (NB - 1)], 1);
    }
    __syncthreads();
    if (pass == 0)
      find_crossing<4096>(hist, krem, scratch, &s_digit, &s_above);
    else
      find_crossing<1024>(hist, krem, scratch, &s_digit, &s_above);
    prefix |= (uint32_t)s_digit << shift;
    pmask |= (uint32_t)(NB - 1) << shift;
    krem -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // ---- ordered sweep: keys > T, then the first krem keys == T
  int tie_base = 0, out_base = 0;
  for (int seg = 0; seg < n; seg += 4 * kThreads) {
    const int i0 = seg + 4 * t;
    uint32_t key[4];
    bool ok[4];
    int ties = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok[j] = i0 + j < n;
      key[j] = ok[j] ? order_key(sz[i0 + j]) : 0u;
      ties += (ok[j] && key[j] == T) ? 1 : 0;
    }
    int tie_total;
    int rank = tie_base + block_exclusive_scan<kThreads>(ties, scratch, &tie_total);
    bool keep[4];
    int kept = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (ok[j] && key[j] == T) {
        keep[j] = rank < krem;
        ++rank;
      } else {
        keep[j] = ok[j] && key[j] > T;
      }
      kept += keep[j] ? 1 : 0;
    }
    int kept_total;
    int pos = out_base + block_exclusive_scan<kThreads>(kept, scratch, &kept_total);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (keep[j] && pos < k) o[pos++] = si[i0 + j];
    tie_base += tie_total;
    out_base += kept_total;
  }
  if (t == 0) out_count[b] = k;
}

}  // namespace

hipError_t launch_topk(int B, int cap, int k, const int32_t* surv_idx, const float* surv_z,
                       const int32_t* surv_count, int32_t* topk_idx, int32_t* topk_count,
                       hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(kThreads), 0, s, cap, k, surv_idx, surv_z,
                     surv_count, topk_idx, topk_count);
  return hipGetLastError();
}

}  // namespace lsa
