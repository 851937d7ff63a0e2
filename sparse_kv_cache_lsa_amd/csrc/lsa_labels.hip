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
// Design.  A row is selected by one block: thread i holds the EPT
// consecutive entries [EPT i, EPT i + EPT) in registers, so it owns whole
// selection words and index order is (thread, register) order.  Rows of up
// to 32K entries: 512-thread blocks with 32 (up to 16K) or 64 entries a
// thread, two blocks per compute unit at 128 VGPRs, so one block's barrier
// phases and row loads overlap the other's arithmetic.  Longer rows (up to
// 64K): one 1024-thread block per compute unit, 64 entries a thread.  Blocks
// walk rows blockIdx.x, blockIdx.x + gridDim.x, ..., loading the next row
// when the current one is done; every barrier of the selection waits for LDS
// only.  No sort:
//  * mass in fixed point: w_s = trunc(exp(x_s - max) * 2^31), summed in 64-bit
//    integers, so every partial sum is exact and independent of summation
//    order -- the result is deterministic and the same as a sequential walk
//    over the same weights (truncation changes a mass ratio by at most
//    N * 2^-31 of the largest entry's mass);
//  * a histogram of mass over 2048 value bins (linear in max - x, so the
//    bins follow the logit order and hold few entries each) finds the bin in
//    which the running mass crosses top_p * S (one block scan over the bins
//    gives S and the mass ahead of every bin);
//  * the entries of that bin (usually a handful) are compared pairwise in
//    LDS: each gets its exact mass ahead in the walk order, so it is kept iff
//    the mass ahead of the bin plus that is below top_p * S;
//  * a bin with more than kCand entries (heavy ties, near-constant rows)
//    instead takes three radix passes over the order key of the logit
//    (11 + 11 + 10 bits) to find the crossing logit and the mass ahead of
//    it, and a block prefix sum in index order over the entries with exactly
//    that logit; this path re-reads the row from memory, so the registers
//    of the common path hold only the row(s).
// Every other entry is kept iff its bin is ahead of the crossing bin.  A
// second kernel adds the layers' selection words per query into the vote
// counts and labels.
#include "lsa_device.h"
#include "lsa_dpp.h"
#include "lsa_launch.h"

#include <algorithm>

namespace lsa {
namespace {

constexpr int kBins = 2048;            // histogram bins per pass
constexpr int kCand = 1024;            // crossing-bin entries handled by direct comparison
constexpr int kMaxVoteLayers = LSA_MAX_VOTE_LAYERS;   // layers one vote adds
static_assert(kMaxVoteLayers <= 32, "vote counts are 8-bit byte lanes; words are kept in registers");

// order key: smaller key = larger logit; -0 and +0 share a key
__device__ __forceinline__ uint32_t desc_key(float x) {
  uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
  uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// An empty asm the compiler cannot see through: values derived from the
// result are recomputed where they are used, not kept live across phases.
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A block barrier that waits for this thread's LDS operations only: global
// loads of the next row stay in flight across it (__syncthreads would wait
// for every outstanding vector memory operation).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int opaque_i(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The helpers below take the thread index as an argument: the row loop passes
// a copy the compiler cannot see through, so nothing derived from it is kept
// live across rows (the registers go to the next row's logits).
template <int NT>
__device__ __forceinline__ uint64_t block_exclusive_scan_u64_l(uint64_t v, uint64_t* scratch,
                                                               uint64_t* total, int tid) {
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint64_t inc = wave_inclusive_sum_u64_dpp(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  lds_barrier();
  if (wave == 0) {
    const uint64_t w = lane < (NT / kWave) ? scratch[lane] : 0ull;
    const uint64_t wi = wave_inclusive_sum_u64_dpp(w);
    if (lane < (NT / kWave)) scratch[lane] = wi - w;
    if (lane == (NT / kWave) - 1) scratch[(NT / kWave)] = wi;
  }
  lds_barrier();
  const uint64_t res = scratch[wave] + inc - v;
  *total = scratch[(NT / kWave)];
  lds_barrier();
  return res;
}

// block-wide max of a and of b; scratch: 2 * (NT / kWave) floats.  No trailing
// barrier: the caller writes scratch again only after later barriers.
template <int NT>
__device__ __forceinline__ void block_max2_l(float& a, float& b, float* scratch, int tid) {
  a = wave_max_f32_dpp(a);
  b = wave_max_f32_dpp(b);
  if ((tid & (kWave - 1)) == 0) {
    scratch[tid / kWave] = a;
    scratch[(NT / kWave) + tid / kWave] = b;
  }
  lds_barrier();
  a = scratch[0];
  b = scratch[(NT / kWave)];
  for (int w = 1; w < (NT / kWave); ++w) {
    a = fmaxf(a, scratch[w]);
    b = fmaxf(b, scratch[(NT / kWave) + w]);
  }
}

template <int NT>
__device__ __forceinline__ void find_crossing_l(const uint64_t* hist, uint64_t M, uint64_t R,
                                                uint64_t* scan_scratch, int* s_bin,
                                                uint64_t* s_before, int tid) {
  constexpr int PER = kBins / NT;
  const int b0 = tid * PER;
  uint64_t local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) local += hist[b0 + j];
  if (tid == 0) *s_bin = -1;
  uint64_t total;
  const uint64_t excl = block_exclusive_scan_u64_l<NT>(local, scan_scratch, &total, tid);
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
  lds_barrier();
}

// FULL rows: 16-byte loads; otherwise range-checked loads (zero past the
// row), one path, so the registers are written in one place.  The slots past
// the row are then set to -inf (pad_row).
template <int EPT, bool FULL>
__device__ __forceinline__ void load_row(float (&v)[EPT], const float* x, int N, int e0) {
  if (FULL) {
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
      const f32x4 t = *(const f32x4*)(x + e0 + i);
      v[i] = t[0]; v[i + 1] = t[1]; v[i + 2] = t[2]; v[i + 3] = t[3];
    }
  } else {
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(x), (short)0, N * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rr, (uint32_t)(e0 + i) * 4u, 0, 0));
  }
}

template <int EPT, bool FULL>
__device__ __forceinline__ void pad_row(float (&v)[EPT], int nv) {
  if (!FULL) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) v[i] = i < nv ? v[i] : -__builtin_inff();
  }
}

// Weight and value bin of the persistent kernel, one fused multiply-add each:
// w = trunc(2^(x log2(e) + 31 - max log2(e))) = trunc(exp(x - max) 2^31), the
// fixed-point scale folded into the exponent (cw = 31 - max log2(e)); bin =
// floor(max inv - x inv) clamped to [0, last bin], non-increasing in x.  The
// clamp at 0 matters: max inv is rounded before the subtraction, so when the
// row's values are large against its range the unclamped value can fall to
// -ulp(max inv) / 2 (a few units) for the largest entries.  Any bin
// function that is non-increasing in x partitions the row correctly (the
// crossing bin is resolved exactly).  -inf (padding) weighs 0; a NaN product
// converts to 0.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ uint32_t lp_weight(float x, float cw) {
  return (uint32_t)__builtin_amdgcn_exp2f(fmaf(x, kLog2e, cw));
}
__device__ __forceinline__ int lp_bin(float x, float ninv, float mi) {
  return (int)__builtin_amdgcn_fmed3f(fmaf(x, ninv, mi), 0.f, (float)(kBins - 1));
}

// NT threads a block walk rows blockIdx.x, blockIdx.x + gridDim.x, ...  EPT
// entries a thread; FULL: N == EPT * NT (no padding).  A block loads its next
// row when the current one is done.  At most 128 VGPRs: 16 wavefronts a
// compute unit (two 512-thread blocks, or one 1024-thread block).
template <int NT, int EPT, bool FULL>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void nucleus_lp_kernel(int nrows, int N, int W, float top_p,
                                                        const float* __restrict__ logits,
                                                        uint32_t* __restrict__ mask) {
  __shared__ uint64_t hist[kBins];
  __shared__ uint64_t scan_scratch[(NT / kWave) + 1];
  __shared__ float red[2 * (NT / kWave)];
  __shared__ int s_bin;
  __shared__ uint64_t s_before;
  __shared__ u32x4 cand[kCand];   // crossing-bin entries: order key, index, weight
  __shared__ int s_ncand;
  __shared__ uint32_t keepbits[EPT * NT / 32];

  float v[EPT];
  int row = blockIdx.x;
  {
    const int e0 = threadIdx.x * EPT;
    const int nv = FULL ? EPT : min(max(N - e0, 0), EPT);
    if (row < nrows) {
      load_row<EPT, FULL>(v, logits + (size_t)row * N, N, e0);
      pad_row<EPT, FULL>(v, nv);
    }
  }
  for (; row < nrows; row += gridDim.x) {
    const int tid = opaque_i((int)threadIdx.x);
    const int e0 = tid * EPT;
    // entries of this thread inside the row: i < nv.  Slots past the row hold
    // -inf (weight 0).  Only one thread of a ragged row holds both kinds; the
    // threads past the row (nv == 0) skip the histogram and candidate passes,
    // so their padding adds nothing to any LDS word.
    const int nv = FULL ? EPT : min(max(N - e0, 0), EPT);
    const bool any = FULL || nv > 0;
    const float* x = logits + (size_t)row * N;
    lds_barrier();   // the previous row's LDS reads are done
    if (tid == 0) { s_ncand = 0; s_bin = -1; }
    for (int j = tid; j < W; j += NT) keepbits[j] = 0;
    for (int j = tid; j < kBins; j += NT) hist[j] = 0;   // ordered by the barriers below

    float m = -__builtin_inff(), nmin = -__builtin_inff();
    if (FULL || nv == EPT) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        m = fmaxf(m, v[i]);
        nmin = fmaxf(nmin, -v[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        m = fmaxf(m, v[i]);
        nmin = fmaxf(nmin, i < nv ? -v[i] : -__builtin_inff());
      }
    }
    block_max2_l<NT>(m, nmin, red, tid);
    const float xmin = -nmin;
    const float range = m - xmin;
    const float inv0 = range > 0.f ? (float)kBins / range : 0.f;
    const float cw0 = fmaf(-m, kLog2e, 31.f), ninv0 = -inv0, mi0 = m * inv0;
    float cw = cw0, ninv = ninv0, mi = mi0;
    auto weight = [&](int i) -> uint32_t { return lp_weight(v[i], cw); };
    auto vbin = [&](int i) -> int { return lp_bin(v[i], ninv, mi); };

    if (any) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        // padding slots add 0
        atomicAdd((unsigned long long*)&hist[vbin(i)], (unsigned long long)weight(i));
      }
    }
    lds_barrier();
    // mass ahead of each bin: a DPP scan inside each wavefront, then every
    // thread adds the totals of the wavefronts before its own (the sum of
    // all of them is the normaliser S: every weight went to a bin)
    constexpr int PER = kBins / NT;
    const int b0 = tid * PER;
    uint64_t local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) local += hist[b0 + j];
    const uint64_t inc = wave_inclusive_sum_u64_dpp(local);
    const int wave = tid / kWave;
    if ((tid & (kWave - 1)) == kWave - 1) scan_scratch[wave] = inc;
    lds_barrier();
    uint64_t S = 0, pre = 0;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) {
      const uint64_t t = scan_scratch[w];
      S += t;
      pre += w < wave ? t : 0ull;
    }
    uint64_t before = pre + inc - local;
    const double rd = (double)top_p * (double)S;
    uint64_t R = (uint64_t)rd;
    if ((double)R < rd) ++R;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint64_t mb = hist[b0 + j];
      if (before < R && before + mb >= R) {
        s_bin = b0 + j;
        s_before = before;
      }
      before += mb;
    }
    lds_barrier();
    const int cbin = s_bin;
    uint64_t M = s_before;
    cw = opaque(cw0);
    ninv = opaque(ninv0);
    mi = opaque(mi0);

    // one pass: entries ahead of the crossing bin set their bit of the
    // thread's selection word; the crossing bin's entries are collected as
    // (order key, index, weight) records.  Padding of the row's last thread
    // may set bits past the row (masked off below) or join the candidates
    // (weight 0 and the largest order key: never kept, and adds nothing to
    // the mass ahead of any entry).
    const int cb = cbin < 0 ? kBins : cbin;   // cbin < 0: every entry is kept
    uint32_t word[EPT / 32];
#pragma unroll
    for (int wd = 0; wd < EPT / 32; ++wd) word[wd] = 0;
    if (any) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int vb = vbin(i);
        word[i / 32] |= (vb < cb ? 1u : 0u) << (i % 32);
        if (vb == cb) {
          const int slot = atomicAdd(&s_ncand, 1);
          if (slot < kCand) cand[slot] = u32x4{desc_key(v[i]), (uint32_t)(e0 + i), weight(i), 0u};
        }
      }
    }
    lds_barrier();
    const int nc = s_ncand;
    if (nc <= kCand) {   // uniform
      if (nc > 0) {
        // each candidate's exact mass ahead inside the bin, in walk order
        // (logit descending, index ascending); kept iff the mass ahead of the
        // bin plus that is below R
        for (int sl = tid; sl < nc; sl += NT) {
          const u32x4 me = cand[sl];
          uint64_t ahead = 0;
#pragma unroll 4
          for (int j = 0; j < nc; ++j) {
            const u32x4 o = cand[j];
            if (o[0] < me[0] || (o[0] == me[0] && o[1] < me[1])) ahead += o[2];
          }
          if (M + ahead < R) atomicOr(&keepbits[me[1] >> 5], 1u << (me[1] & 31));
        }
        lds_barrier();
      }
#pragma unroll
      for (int wd = 0; wd < EPT / 32; ++wd) {
        const int widx = tid * (EPT / 32) + wd;
        if (nc > 0) word[wd] |= keepbits[widx];
        if (!FULL && widx == W - 1 && (N & 31)) word[wd] &= (1u << (N & 31)) - 1u;
        if (widx < W) mask[(size_t)row * W + widx] = word[wd];
      }
    } else {
      // heavy ties: radix passes over the order key inside the crossing bin,
      // re-reading the row (through a pointer the compiler cannot match with
      // x, so the row's registers are not kept for this path): full rows with
      // plain loads, others through a range-checked resource
      const float* xr = x;
      asm volatile("" : "+s"(xr));
      const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(xr), (short)0, N * 4, 0x00020000);
      auto rx = [&](int i) -> float {
        if constexpr (FULL) return xr[e0 + i];
        const float t = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)(e0 + i) * 4u, 0, 0));
        return i < nv ? t : -__builtin_inff();
      };
      auto rweight = [&](float xv, int i) -> uint32_t { return (i < nv) ? lp_weight(xv, cw) : 0u; };
      auto rbin = [&](float xv) -> int { return lp_bin(xv, ninv, mi); };
      bool found = true;
      uint32_t prefix = 0;
      constexpr int kShift[3] = {21, 10, 0};
      constexpr int kBits[3] = {11, 11, 10};
#pragma unroll 1
      for (int p = 0; p < 3; ++p) {
        for (int j = tid; j < kBins; j += NT) hist[j] = 0;
        lds_barrier();
        const int sh = kShift[p];
        const int hi = sh + kBits[p];
        cw = opaque(cw0);
        ninv = opaque(ninv0);
        mi = opaque(mi0);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const float xv = rx(i);
          if (i >= nv || rbin(xv) != cbin) continue;
          const uint32_t k = desc_key(xv);
          if (hi < 32 && (k >> hi) != prefix) continue;
          const uint32_t w = rweight(xv, i);
          if (w)
            atomicAdd((unsigned long long*)&hist[(k >> sh) & ((1u << kBits[p]) - 1u)],
                      (unsigned long long)w);
        }
        lds_barrier();
        find_crossing_l<NT>(hist, M, R, scan_scratch, &s_bin, &s_before, tid);
        if (s_bin < 0) { found = false; break; }   // uniform: s_bin is shared
        prefix = (prefix << kBits[p]) | (uint32_t)s_bin;
        M = s_before;
      }
      const uint32_t ckey = found ? prefix : 0xFFFFFFFFu;
      cw = opaque(cw0);
      uint64_t tie_local = 0;
      if (found) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const float xv = rx(i);
          if (i < nv && desc_key(xv) == ckey) tie_local += rweight(xv, i);
        }
      }
      uint64_t tie_total;
      const uint64_t tie_excl = block_exclusive_scan_u64_l<NT>(tie_local, scan_scratch, &tie_total, tid);
      uint64_t ahead = M + tie_excl;
      cw = opaque(cw0);
#pragma unroll
      for (int wd = 0; wd < EPT / 32; ++wd) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int i = wd * 32 + j;
          bool keep = false;
          if (i < nv) {
            if (!found) {
              keep = true;
            } else {
              const float xv = rx(i);
              const uint32_t k = desc_key(xv);
              if (k < ckey) {
                keep = true;
              } else if (k == ckey) {
                keep = ahead < R;
                ahead += rweight(xv, i);
              }
            }
          }
          word |= (keep ? 1u : 0u) << j;
        }
        const int widx = tid * (EPT / 32) + wd;
        if (widx < W) mask[(size_t)row * W + widx] = word;
      }
    }
    const int nxt = row + gridDim.x;
    if (nxt < nrows) {
      load_row<EPT, FULL>(v, logits + (size_t)nxt * N, N, e0);
      pad_row<EPT, FULL>(v, nv);
    }
  }
}

// count[t][s] = sum over layers of bit s of mask[t][l]; label = count >= theta.
// One thread per quarter of a selection word: two byte-lane accumulators of
// four counts.
__global__ __launch_bounds__(256) void vote_kernel(int L, int N, int W, int theta,
                                                   const uint32_t* __restrict__ mask,
                                                   uint8_t* __restrict__ count,
                                                   uint8_t* __restrict__ label) {
  // one thread per quarter word (entries 8 r .. 8 r + 7 of word w): four
  // times the threads of one per word, so more loads are in flight per
  // compute unit; the four threads of a word load the same addresses
  const int t = blockIdx.y;
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  const int w = u >> 2, r = u & 3;
  if (w >= W) return;
  // all layers' words in flight at once: a resource over this query's L * W
  // words returns 0 for the layers past L, so the loads need no branch (the
  // whole offset goes in the vector offset: the range check does not cover
  // the scalar offset)
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(mask + (size_t)t * L * W), (short)0, L * W * 4, 0x00020000);
  uint32_t words[kMaxVoteLayers];
#pragma unroll
  for (int l = 0; l < kMaxVoteLayers; ++l)
    words[l] = __builtin_amdgcn_raw_buffer_load_b32(rm, (uint32_t)(l * W + w) * 4u, 0, 0);
  uint32_t acc[2] = {0, 0};
#pragma unroll
  for (int l = 0; l < kMaxVoteLayers; ++l) {
    const uint32_t byte = (words[l] >> (8 * r)) & 0xFFu;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      // bits 4k..4k+3 of the byte -> bytes 0..3 (multiply spreads, mask keeps)
      acc[k] += (((byte >> (4 * k)) & 0xFu) * 0x00204081u) & 0x01010101u;
  }
  const size_t base = (size_t)t * N + (size_t)w * 32 + 8 * r;
  if ((N & 31) == 0) {
    u32x2 y;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t a = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) a |= ((int)((acc[k] >> (8 * j)) & 0xFFu) >= theta ? 1u : 0u) << (8 * j);
      y[k] = a;
    }
    *(u32x2*)(count + base) = u32x2{acc[0], acc[1]};
    *(u32x2*)(label + base) = y;
  } else {
    for (int j = 0; j < 8; ++j) {
      if (w * 32 + 8 * r + j >= N) break;
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
  const int nrows = Q * L;
  const int cus = device_cu_count();
  // 512-thread blocks: up to eight a compute unit in the grid (two resident
  // at a time), so rows are handed out as blocks finish; 1024-thread blocks:
  // one a compute unit, each walking its rows (measured faster than a larger
  // grid for these rows)
  const dim3 grid((unsigned)std::min(nrows, 8 * cus));
  const dim3 grid1((unsigned)std::min(nrows, cus));
  if (N <= 16384) {
    if (N == 16384)
      hipLaunchKernelGGL((nucleus_lp_kernel<512, 32, true>), grid, dim3(512), 0, s, nrows, N, W, top_p, logits, mask);
    else
      hipLaunchKernelGGL((nucleus_lp_kernel<512, 32, false>), grid, dim3(512), 0, s, nrows, N, W, top_p, logits, mask);
  } else if (N <= 32768) {
    if (N == 32768)
      hipLaunchKernelGGL((nucleus_lp_kernel<512, 64, true>), grid, dim3(512), 0, s, nrows, N, W, top_p, logits, mask);
    else
      hipLaunchKernelGGL((nucleus_lp_kernel<512, 64, false>), grid, dim3(512), 0, s, nrows, N, W, top_p, logits, mask);
  } else {
    if (N == 65536)
      hipLaunchKernelGGL((nucleus_lp_kernel<1024, 64, true>), grid1, dim3(1024), 0, s, nrows, N, W, top_p, logits, mask);
    else
      hipLaunchKernelGGL((nucleus_lp_kernel<1024, 64, false>), grid1, dim3(1024), 0, s, nrows, N, W, top_p, logits, mask);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vote_kernel, dim3((4 * W + 255) / 256, Q), dim3(256), 0, s, L, N, W, theta,
                     mask, count, label);
  return hipGetLastError();
}

}  // namespace lsa
