// lsa_labels.hip -- golden labels by cross-layer majority vote, for gfx950.
//
// For every query t and teacher layer l the row logits[t][l][0..N) becomes a
// probability distribution by softmax; the layer keeps the smallest prefix of
// entries, in order of decreasing logit (ties: lower index first), whose mass
// reaches top_p -- an entry is kept while the mass strictly ahead of it is
// below top_p, so the entry that crosses top_p is kept.  An entry is labelled
// positive when at least theta layers keep it.  (gist.science technical
// summary, section 2.2 "data curation and labelling", steps 1-3; paper.oopus.info
// review, section 2, training labels by cross-layer majority vote.)
//
// Design.  One 1024-thread block per (query, layer) row; thread i holds the
// EPT consecutive entries [i*EPT, i*EPT + EPT) in registers, so one thread
// owns EPT/32 whole selection words and index order is (thread, register)
// order.  No sort:
//  * mass in fixed point: w_s = trunc(exp(x_s - max) * 2^31), summed in 64-bit
//    integers, so every partial sum is exact and independent of summation
//    order -- the result is deterministic and the same as a sequential walk
//    over the same weights (truncation changes a mass ratio by at most
//    N * 2^-31 of the largest entry's mass);
//  * a histogram of mass over 2048 value bins (linear in max - x, so the
//    bins follow the logit order and hold few entries each) finds the bin in
//    which the running mass crosses top_p * S;
//  * the entries of that bin (usually a handful) are compared pairwise in
//    LDS: each gets its exact mass ahead in the walk order, so it is kept iff
//    the mass ahead of the bin plus that is below top_p * S;
//  * a bin with more than kCand entries (heavy ties, near-constant rows)
//    instead takes three radix passes over the order key of the logit
//    (11 + 11 + 10 bits) to find the crossing logit and the mass ahead of
//    it, and a block prefix sum in index order over the entries with exactly
//    that logit.
// Every other entry is kept iff its bin is ahead of the crossing bin.
// A second kernel adds the layers' selection words per query into the vote
// counts and labels.
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kNT = 1024;              // threads per row block
constexpr int kNWv = kNT / kWave;      // wavefronts per row block
constexpr int kBins = 2048;            // histogram bins per pass
constexpr float kFix = 2147483648.f;   // 2^31: fixed-point unit of exp(x - max)
constexpr int kCand = 1024;            // crossing-bin entries handled by direct comparison

// order key: smaller key = larger logit; -0 and +0 share a key
__device__ __forceinline__ uint32_t desc_key(float x) {
  uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
  uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

__device__ __forceinline__ uint64_t wave_inclusive_scan_u64(uint64_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint64_t t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive prefix sum of v over the block in thread order; *total gets the
// block sum.  scratch: kNWv + 1 u64 of LDS.  All threads must call.
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* scratch,
                                                             uint64_t* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const uint64_t inc = wave_inclusive_scan_u64(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  if (wave == 0) {   // one wavefront scans the per-wave totals
    const uint64_t w = lane < kNWv ? scratch[lane] : 0ull;
    const uint64_t wi = wave_inclusive_scan_u64(w);
    if (lane < kNWv) scratch[lane] = wi - w;
    if (lane == kNWv - 1) scratch[kNWv] = wi;
  }
  __syncthreads();
  const uint64_t res = scratch[wave] + inc - v;
  *total = scratch[kNWv];
  __syncthreads();
  return res;
}

// block-wide max of a and of b (one pass); scratch: 2 * kNWv floats
__device__ __forceinline__ void block_max2(float& a, float& b, float* scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    a = fmaxf(a, __shfl_xor(a, off, kWave));
    b = fmaxf(b, __shfl_xor(b, off, kWave));
  }
  if (lane_id() == 0) {
    scratch[threadIdx.x / kWave] = a;
    scratch[kNWv + threadIdx.x / kWave] = b;
  }
  __syncthreads();
  a = scratch[0];
  b = scratch[kNWv];
  for (int w = 1; w < kNWv; ++w) {
    a = fmaxf(a, scratch[w]);
    b = fmaxf(b, scratch[kNWv + w]);
  }
  __syncthreads();
}

// Given a mass histogram over kBins bins (in order) and the mass M already
// ahead of bin 0, find the bin where the running mass reaches R: the bin b
// with M + mass(bins < b) < R <= M + mass(bins <= b).  Writes the bin to
// *s_bin (or -1 if the histogram never reaches R) and the mass ahead of it to
// *s_before.  All threads must call.
__device__ __forceinline__ void find_crossing(const uint64_t* hist, uint64_t M, uint64_t R,
                                              uint64_t* scan_scratch, int* s_bin,
                                              uint64_t* s_before) {
  constexpr int PER = kBins / kNT;
  const int b0 = threadIdx.x * PER;
  uint64_t local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) local += hist[b0 + j];
  if (threadIdx.x == 0) *s_bin = -1;
  uint64_t total;
  const uint64_t excl = block_exclusive_scan_u64(local, scan_scratch, &total);
  uint64_t before = M + excl;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint64_t m = hist[b0 + j];
    if (before < R && before + m >= R) {
      *s_bin = b0 + j;
      *s_before = before;
    }
    before += m;
  }
  __syncthreads();
}

template <int EPT>
__global__ __launch_bounds__(kNT) void nucleus_kernel(int N, int W, float top_p,
                                                      const float* __restrict__ logits,
                                                      uint32_t* __restrict__ mask) {
  static_assert(EPT % 32 == 0, "a thread owns whole selection words");
  __shared__ uint64_t hist[kBins];
  __shared__ uint64_t scan_scratch[kNWv + 1];
  __shared__ float red[2 * kNWv];
  __shared__ int s_bin;
  __shared__ uint64_t s_before;
  __shared__ uint32_t c_key[kCand];
  __shared__ int c_idx[kCand];
  __shared__ uint32_t c_w[kCand];
  __shared__ int s_ncand;
  __shared__ uint32_t keepbits[65536 / 32];

  const size_t row = blockIdx.x;
  if (threadIdx.x == 0) s_ncand = 0;
  for (int j = threadIdx.x; j < W; j += kNT) keepbits[j] = 0;   // ordered by the barriers below
  const float* x = logits + row * (size_t)N;
  const int e0 = threadIdx.x * EPT;

  float v[EPT];
  if ((N & 3) == 0 && e0 + EPT <= N) {
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
      const f32x4 t = *(const f32x4*)(x + e0 + i);
      v[i] = t[0]; v[i + 1] = t[1]; v[i + 2] = t[2]; v[i + 3] = t[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) v[i] = (e0 + i < N) ? x[e0 + i] : -__builtin_inff();
  }

  // max and min of the row
  float m = -__builtin_inff(), nmin = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    m = fmaxf(m, v[i]);
    if (e0 + i < N) nmin = fmaxf(nmin, -v[i]);
  }
  block_max2(m, nmin, red);
  const float xmin = -nmin;
  auto weight = [&](int i) -> uint32_t {
    return (e0 + i < N) ? (uint32_t)(__expf(v[i] - m) * kFix) : 0u;
  };
  // value bins, bin(x) = floor((max - x) * kBins / (max - min)): monotone in x
  const float range = m - xmin;
  const float inv = range > 0.f ? (float)kBins / range : 0.f;
  auto vbin = [&](int i) -> int {
    const float t = (m - v[i]) * inv;
    return t < (float)(kBins - 1) ? (int)t : kBins - 1;
  };

  // pass 0: softmax normaliser and the mass histogram over value bins, with
  // one exponential per entry
  for (int j = threadIdx.x; j < kBins; j += kNT) hist[j] = 0;
  __syncthreads();
  uint64_t lsum = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const uint32_t w = weight(i);
    lsum += w;
    if (w) atomicAdd((unsigned long long*)&hist[vbin(i)], (unsigned long long)w);
  }
  uint64_t S;
  (void)block_exclusive_scan_u64(lsum, scan_scratch, &S);
  // keep s iff (mass ahead of s) < top_p * S, i.e. < R for integer masses
  const double rd = (double)top_p * (double)S;
  uint64_t R = (uint64_t)rd;
  if ((double)R < rd) ++R;
  find_crossing(hist, 0, R, scan_scratch, &s_bin, &s_before);
  const int cbin = s_bin;
  uint64_t M = s_before;

  uint32_t ckey = 0xFFFFFFFFu;   // order key of the crossing logit (radix path)
  bool found = cbin >= 0;
  // Candidate path: the crossing value bin usually holds a handful of
  // entries.  They are collected (order key, index, mass) in LDS, and each
  // gets its exact mass ahead inside the bin by comparing with every other
  // candidate in the walk order (logit descending, index ascending); its
  // keep bit goes to an LDS bitmap.  More than kCand candidates (heavy ties,
  // near-constant rows) take the radix path below.
  bool cand_path = false;
  if (found) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (e0 + i < N && vbin(i) == cbin) {
        const int slot = atomicAdd(&s_ncand, 1);
        if (slot < kCand) {
          c_key[slot] = desc_key(v[i]);
          c_idx[slot] = e0 + i;
          c_w[slot] = weight(i);
        }
      }
    }
    __syncthreads();
    const int nc = s_ncand;
    cand_path = nc <= kCand;   // uniform
    if (cand_path) {
      for (int sl = threadIdx.x; sl < nc; sl += kNT) {
        const uint32_t ks = c_key[sl];
        const int is = c_idx[sl];
        uint64_t ahead = 0;
        for (int j = 0; j < nc; ++j) {
          const uint32_t kj = c_key[j];
          if (kj < ks || (kj == ks && c_idx[j] < is)) ahead += c_w[j];
        }
        if (M + ahead < R) atomicOr(&keepbits[is >> 5], 1u << (is & 31));
      }
      __syncthreads();
    }
  }
  if (found && !cand_path) {
    // passes 1-3: radix over the order key, inside the crossing value bin
    uint32_t prefix = 0;
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kBits[3] = {11, 11, 10};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      for (int j = threadIdx.x; j < kBins; j += kNT) hist[j] = 0;
      __syncthreads();
      const int sh = kShift[p];
      const int hi = sh + kBits[p];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        if (e0 + i >= N || vbin(i) != cbin) continue;
        const uint32_t k = desc_key(v[i]);
        if (hi < 32 && (k >> hi) != prefix) continue;
        const uint32_t w = weight(i);
        if (w)
          atomicAdd((unsigned long long*)&hist[(k >> sh) & ((1u << kBits[p]) - 1u)],
                    (unsigned long long)w);
      }
      __syncthreads();
      find_crossing(hist, M, R, scan_scratch, &s_bin, &s_before);
      if (s_bin < 0) { found = false; break; }   // uniform: s_bin is shared
      prefix = (prefix << kBits[p]) | (uint32_t)s_bin;
      M = s_before;
    }
    ckey = prefix;
  }

  if (cand_path) {
#pragma unroll
    for (int wd = 0; wd < EPT / 32; ++wd) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int i = wd * 32 + j;
        if (e0 + i < N) {
          const int vb = vbin(i);
          const bool keep = vb < cbin || (vb == cbin && ((keepbits[(e0 + i) >> 5] >> ((e0 + i) & 31)) & 1u));
          word |= (keep ? 1u : 0u) << j;
        }
      }
      const int widx = threadIdx.x * (EPT / 32) + wd;
      if (widx < W) mask[row * (size_t)W + widx] = word;
    }
    return;
  }

  // entries with the crossing logit: mass ahead in index order
  uint64_t tie_local = 0;
  if (found) {
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (e0 + i < N && desc_key(v[i]) == ckey) tie_local += weight(i);
  }
  uint64_t tie_total;
  const uint64_t tie_excl = block_exclusive_scan_u64(tie_local, scan_scratch, &tie_total);

  uint64_t ahead = M + tie_excl;
#pragma unroll
  for (int wd = 0; wd < EPT / 32; ++wd) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int i = wd * 32 + j;
      bool keep = false;
      if (e0 + i < N) {
        if (!found) {
          keep = true;   // the running mass never reaches R (top_p >= 1)
        } else {
          const uint32_t k = desc_key(v[i]);
          if (k < ckey) {
            keep = true;
          } else if (k == ckey) {
            keep = ahead < R;
            ahead += weight(i);
          }
        }
      }
      word |= (keep ? 1u : 0u) << j;
    }
    const int widx = threadIdx.x * (EPT / 32) + wd;
    if (widx < W) mask[row * (size_t)W + widx] = word;
  }
}

// count[t][s] = sum over layers of bit s of mask[t][l]; label = count >= theta.
// One thread per selection word: eight byte-lane accumulators of four counts.
__global__ __launch_bounds__(256) void vote_kernel(int L, int N, int W, int theta,
                                                   const uint32_t* __restrict__ mask,
                                                   uint8_t* __restrict__ count,
                                                   uint8_t* __restrict__ label) {
  const int t = blockIdx.y;
  const int w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= W) return;
  uint32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int l = 0; l < L; ++l) {
    const uint32_t word = mask[((size_t)t * L + l) * W + w];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // bits 4k..4k+3 of the word -> bytes 0..3 (multiply spreads, mask keeps)
      acc[k] += (((word >> (4 * k)) & 0xFu) * 0x00204081u) & 0x01010101u;
    }
  }
  const size_t base = (size_t)t * N + (size_t)w * 32;
  if ((N & 31) == 0) {
    u32x4 c0 = {acc[0], acc[1], acc[2], acc[3]}, c1 = {acc[4], acc[5], acc[6], acc[7]};
    u32x4 y0, y1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t a = 0, b = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a |= ((int)((c0[k] >> (8 * j)) & 0xFFu) >= theta ? 1u : 0u) << (8 * j);
        b |= ((int)((c1[k] >> (8 * j)) & 0xFFu) >= theta ? 1u : 0u) << (8 * j);
      }
      y0[k] = a;
      y1[k] = b;
    }
    *(u32x4*)(count + base) = c0;
    *(u32x4*)(count + base + 16) = c1;
    *(u32x4*)(label + base) = y0;
    *(u32x4*)(label + base + 16) = y1;
  } else {
    for (int j = 0; j < 32; ++j) {
      if (w * 32 + j >= N) break;
      const int c = (int)((acc[j >> 2] >> (8 * (j & 3))) & 0xFFu);
      count[base + j] = (uint8_t)c;
      label[base + j] = c >= theta ? 1 : 0;
    }
  }
}

}  // namespace

hipError_t launch_label_vote(int Q, int L, int N, float top_p, int theta, const float* logits,
                             uint32_t* mask, uint8_t* count, uint8_t* label, hipStream_t s) {
  const int W = (N + 31) / 32;
  const dim3 rows((unsigned)Q * (unsigned)L);
  if (N <= 32 * kNT)
    hipLaunchKernelGGL((nucleus_kernel<32>), rows, dim3(kNT), 0, s, N, W, top_p, logits, mask);
  else
    hipLaunchKernelGGL((nucleus_kernel<64>), rows, dim3(kNT), 0, s, N, W, top_p, logits, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vote_kernel, dim3((W + 255) / 256, Q), dim3(256), 0, s, L, N, W, theta, mask,
                     count, label);
  return hipGetLastError();
}

}  // namespace lsa
