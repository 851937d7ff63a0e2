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
#include "lsa_dpp.h"
#include "lsa_launch.h"

#include <mutex>

namespace lsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kReg = 80;   // keys per thread held in registers
constexpr int kMBMinCap = 16384;   // longer lists are first cut down slice by slice
constexpr int kStage = 8192;       // output slots staged in LDS

__device__ __forceinline__ uint32_t order_key(float z) {
  if (z != z) return 0u;            // NaN ranks last
  if (z == 0.f) z = 0.f;            // -0 and +0 are the same score
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over a block of NT threads (thread order), total in
// *total: a DPP scan inside each wavefront, then every thread adds the
// totals of the wavefronts before its own.  scratch: NT/64 ints.  All threads
// call; the trailing barrier lets the next call reuse scratch.
template <int NT>
__device__ __forceinline__ int scan_block(int v, int* scratch, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int inc = wave_inclusive_sum_dpp(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int pre = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = scratch[w];
    all += t;
    pre += w < wave ? t : 0;
  }
  *total = all;
  __syncthreads();
  return pre + inc - v;
}

// block-wide min of a and max of b; scratch: 2 * (NT / 64) ints.  All
// threads call.  No trailing barrier: the only caller writes scratch again
// after two more barriers.
template <int NT>
__device__ __forceinline__ void block_minmax_t(uint32_t& a, uint32_t& b, int* scratch) {
  constexpr int NW = NT / kWave;
  a = wave_min_u32_dpp(a);
  b = wave_max_u32_dpp(b);
  if (lane_id() == 0) {
    scratch[threadIdx.x / kWave] = (int)a;
    scratch[NW + threadIdx.x / kWave] = (int)b;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    a = min(a, (uint32_t)scratch[w]);
    b = max(b, (uint32_t)scratch[NW + w]);
  }
}

// Finds, scanning bins from the highest digit down, the bin holding the
// krem-th key; returns the digit and the number of keys in higher bins.
template <int NB, int NT>
__device__ __forceinline__ void find_crossing(const int* hist, int krem, int* scratch,
                                              int* out_digit, int* out_above) {
  constexpr int PER = NB / NT;   // bins per thread
  const int t = threadIdx.x;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += hist[NB - 1 - (t * PER + i)];
  int total;
  const int before = scan_block<NT>(sum, scratch, &total);
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

__device__ __forceinline__ float key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Top-k of the n (> k > 0) scores sz[0..n) of one list by one block of NT
// threads: thread t holds positions [t*chunk, (t+1)*chunk) (chunk <= KREG,
// chunk * NT >= n) in registers for every pass, so array order (= entry
// order) is (thread, register) order.  Radix select over 12/10/10-bit digits
// (LDS histograms, block scans) finds the k-th key T and how many keys equal
// to T belong to the top-k; two block prefix sums then give every kept
// position its output slot.  Writes out_idx[0..k) = si[kept positions], in
// position order, and out_z (if not null) the scores.  stage: LDS for
// kStage ints (used when k <= kStage); scratch: 2 * NT/64 + 2 ints.  With
// seg_kept (LDS, zeroed) every kept position p also counts into
// seg_kept[p / seg].  All threads call.
template <int NT, int KREG>
__device__ __forceinline__ void block_select(int n, int k, int chunk, const float* sz,
                                             const int32_t* si, int* hist, int* scratch,
                                             int* s_digit, int* s_above, int* stage,
                                             int32_t* out_idx, float* out_z,
                                             int* seg_kept = nullptr, int seg = 1) {
  const int t = threadIdx.x;
  const int base = t * chunk;
  // buffer loads over the n valid scores: positions past n read 0 and are
  // masked below, so the loads need no branches and are all in flight at once
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sz), (short)0, n * 4, 0x00020000);
  uint32_t key[KREG];
  if ((chunk & 3) == 0 && ((uintptr_t)sz & 15) == 0) {
#pragma unroll
    for (int j = 0; j < KREG; j += 4)
      if (j < chunk) {
        const f32x4 v = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(base + j) * 4, 0, 0));
        key[j] = order_key(v[0]);
        key[j + 1] = order_key(v[1]);
        key[j + 2] = order_key(v[2]);
        key[j + 3] = order_key(v[3]);
      }
  } else {
#pragma unroll
    for (int j = 0; j < KREG; ++j)
      if (j < chunk)
        key[j] = order_key(__builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)(base + j) * 4, 0, 0)));
  }
  const int nv = min(chunk, max(0, n - base));   // valid keys of this thread
  // Digits are taken from key - kmin, the first one from the top bits of the
  // list's actual key span: a narrow list (the candidates of the slices are
  // all near the top) then spreads over the first histogram instead of piling
  // into a few bins, whose LDS atomics would serialise, and needs fewer passes.
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < KREG; ++j)
    if (j < chunk && j < nv) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  block_minmax_t<NT>(kmin, kmax, scratch);
  const uint32_t span = kmax - kmin;
  // from here on the registers hold key - kmin (order-preserving for valid keys)
#pragma unroll
  for (int j = 0; j < KREG; ++j)
    if (j < chunk) key[j] -= kmin;
  const int bits = span ? 32 - __builtin_clz(span) : 0;
  uint32_t prefix = 0;   // the digits fixed so far, as a value of the top bits of key - kmin
  int krem = k;
  int hi = bits;         // key - kmin bits above hi are fixed
  while (hi > 0) {       // uniform: at most three passes (12 + 10 + 10 bits)
    const int width = hi == bits ? 12 : 10;
    const int shift = max(0, hi - width);
    const int NB = 1 << (hi - shift);
    const int FB = NB > 1024 ? 4096 : 1024;   // bins the crossing search reads
    for (int i = t; i < FB; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KREG; ++j)
      if (j < chunk && j < nv && (hi >= 32 || (key[j] >> hi) == prefix))
        atomicAdd(&hist[(key[j] >> shift) & (NB - 1)], 1);
    __syncthreads();
    if (NB > 1024)
      find_crossing<4096, NT>(hist, krem, scratch, s_digit, s_above);
    else
      find_crossing<1024, NT>(hist, krem, scratch, s_digit, s_above);
    prefix = (prefix << (hi - shift)) | (uint32_t)*s_digit;
    krem -= *s_above;
    hi = shift;
    __syncthreads();
  }
  const uint32_t T = prefix;   // k-th key - kmin: all bits fixed (span 0: every key is kmin)
  int ties = 0, above = 0;
#pragma unroll
  for (int j = 0; j < KREG; ++j)
    if (j < chunk) {
      ties += (j < nv && key[j] == T) ? 1 : 0;
      above += (j < nv && key[j] > T) ? 1 : 0;
    }
  int tie_total;
  const int tie_rank0 = scan_block<NT>(ties, scratch, &tie_total);
  const int take_ties = min(ties, max(0, krem - tie_rank0));
  int kept_total;
  int pos = scan_block<NT>(above + take_ties, scratch, &kept_total);
  int tie_rank = tie_rank0;
  // Kept positions go to LDS at their output slot first; the gather of the
  // entry indices (and scores) then runs as one round of independent loads
  // instead of a chain of dependent ones per thread.
  const bool staged = k <= kStage;
#pragma unroll
  for (int j = 0; j < KREG; ++j)
    if (j < chunk) {
      bool keep = false;
      if (j < nv) {
        if (key[j] > T) keep = true;
        else if (key[j] == T) keep = tie_rank++ < krem;
      }
      if (keep && pos < k) {
        if (seg_kept) atomicAdd(&seg_kept[(base + j) / seg], 1);
        if (staged) {
          stage[pos] = base + j;
        } else {
          out_idx[pos] = si[base + j];
          if (out_z) out_z[pos] = key_to_float(key[j] + kmin);
        }
        ++pos;
      }
    }
  if (staged) {
    __syncthreads();
    for (int i = t; i < k; i += NT) {
      const int q = stage[i];
      out_idx[i] = si[q];
      if (out_z) out_z[i] = sz[q];
    }
  }
}

template <int NT>
struct SelectLDS {
  int hist[4096];
  int scratch[2 * (NT / kWave) + 2];
  int stage[kStage];
  int digit, above;
};

// Top-k of one list of n scores (entry indices si, scores sz) by the whole
// block into o[0..k) (ascending positions, -1 padding) and *count.
template <int NT>
__device__ __forceinline__ void select_list(int n, int k, const int32_t* __restrict__ si,
                            const float* __restrict__ sz, int32_t* __restrict__ o,
                            int32_t* count, SelectLDS<NT>& S) {
  int* hist = S.hist;
  int* scratch = S.scratch;
  int* stage = S.stage;
  const int t = threadIdx.x;
  if (k == 0) {
    if (t == 0) *count = 0;
    return;
  }
  if (n <= k) {
    for (int i = t; i < k; i += NT) o[i] = i < n ? si[i] : -1;
    if (t == 0) *count = n;
    return;
  }

  if (n <= NT * kReg) {
    // ---- register-resident path: thread t holds positions [t*chunk, (t+1)*chunk)
    // the register array is sized to the list (every pass walks all its slots)
    const int chunk = (n + NT - 1) / NT;
    if (chunk <= 16)
      block_select<NT, 16>(n, k, chunk, sz, si, hist, scratch, &S.digit, &S.above, stage, o,
                                 nullptr);
    else if (chunk <= 32)
      block_select<NT, 32>(n, k, chunk, sz, si, hist, scratch, &S.digit, &S.above, stage, o,
                                 nullptr);
    else
      block_select<NT, kReg>(n, k, chunk, sz, si, hist, scratch, &S.digit, &S.above, stage,
                                   o, nullptr);
    if (t == 0) *count = k;
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
    for (int i = t; i < NB; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = t; i < n; i += NT) {
      const uint32_t key = order_key(sz[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (NB - 1)], 1);
    }
    __syncthreads();
    if (pass == 0)
      find_crossing<4096, NT>(hist, krem, scratch, &S.digit, &S.above);
    else
      find_crossing<1024, NT>(hist, krem, scratch, &S.digit, &S.above);
    prefix |= (uint32_t)S.digit << shift;
    pmask |= (uint32_t)(NB - 1) << shift;
    krem -= S.above;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // ---- ordered sweep: keys > T, then the first krem keys == T
  int tie_base = 0, out_base = 0;
  for (int seg = 0; seg < n; seg += 4 * NT) {
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
    int rank = tie_base + block_exclusive_scan<NT>(ties, scratch, &tie_total);
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
    int pos = out_base + block_exclusive_scan<NT>(kept, scratch, &kept_total);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (keep[j] && pos < k) o[pos++] = si[i0 + j];
    tie_base += tie_total;
    out_base += kept_total;
  }
  if (t == 0) *count = k;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(int cap, int k,
                                                        const int32_t* __restrict__ surv_idx,
                                                        const float* __restrict__ surv_z,
                                                        const int32_t* __restrict__ surv_count,
                                                        int32_t* __restrict__ out,
                                                        int32_t* __restrict__ out_count) {
  __shared__ SelectLDS<kThreads> S;
  const int b = blockIdx.x;
  const int n = min(max(surv_count[b], 0), cap);
  select_list<kThreads>(n, k, surv_idx + (size_t)b * cap, surv_z + (size_t)b * cap, out + (size_t)b * k,
              out_count + b, S);
}

// ----------------------------------------------------------------------------
// Long lists (more than kMBMinCap survivors of capacity): two stages.
//  1. slice_kernel, several blocks per request: block p takes positions
//     [p*kSlice, (p+1)*kSlice) and writes the top kc of its slice (same
//     ranking, in position order) to a candidate list in the workspace, at
//     offset p * kc -- every earlier slice is full, so the offset needs no
//     communication.  The candidate list stays in position order.
//  2. final_kernel: the top-k of the candidate list.
// With kc = min(k, kSlice) the global top-k lies inside the candidates
// (fewer than k entries of a member's slice precede it).  With kc < k a
// slice keeps only its best kc: each of the slice's dropped entries ranks
// below all kc kept ones, so the candidates' top-k is the exact top-k unless
// a truncated slice (more than kc entries) has all its kc kept entries in
// it.  The final stage counts the entries of each slice it keeps and, in
// that case, selects over the request's whole survivor list instead.  About
// k * kSlice / n of a slice's entries belong to the top-k (n survivors; at
// 1M context 2048 * 4096 / 63K = 133, standard deviation about 11), so with
// kc = 256 the fallback stays rare unless the best entries cluster in a few
// slices.  (Kept per slice: 512 timed 32 us, 256 timed 29.5 us at 1M
// context; slices of 2048 or 8192 survivors were slower.)
constexpr int kMT = 256;               // threads per slice block
constexpr int kMK = 16;                // scores per thread
constexpr int kSlice = kMT * kMK;      // survivors per slice
constexpr int kKeep = 256;             // candidates a truncating slice keeps
constexpr int kFinalThreads = 512;    // threads of the final stage (1024: 29.7 us, 512: 28.5, 256: 32.3 at 1M context)
// slices the final stage can check: it holds every candidate in registers
constexpr int kMaxSeg = kFinalThreads * kReg / kKeep;

__global__ __launch_bounds__(kMT) void slice_kernel(int cap, int k, int kc, int cap_c,
                                                    const int32_t* __restrict__ surv_idx,
                                                    const float* __restrict__ surv_z,
                                                    const int32_t* __restrict__ surv_count,
                                                    int32_t* __restrict__ cand_idx,
                                                    float* __restrict__ cand_z,
                                                    int32_t* __restrict__ cand_count) {
  __shared__ int hist[4096];
  __shared__ int scratch[2 * (kMT / kWave) + 2];
  __shared__ int stage[kStage];
  __shared__ int s_digit, s_above;
  // request index fastest: the blocks of the first slices of every request
  // are dispatched first (most later slices are empty and exit at once)
  const int b = blockIdx.x, p = blockIdx.y;
  const int n = min(max(surv_count[b], 0), cap);
  if (p == 0 && threadIdx.x == 0)
    cand_count[b] = k == 0 ? 0 : (n / kSlice) * kc + min(kc, n % kSlice);
  const int np = min(kSlice, n - p * kSlice);
  if (k == 0 || np <= 0) return;
  const int32_t* si = surv_idx + (size_t)b * cap + (size_t)p * kSlice;
  const float* sz = surv_z + (size_t)b * cap + (size_t)p * kSlice;
  int32_t* ci = cand_idx + (size_t)b * cap_c + (size_t)p * kc;
  float* cz = cand_z + (size_t)b * cap_c + (size_t)p * kc;
  if (np <= kc) {
    for (int i = threadIdx.x; i < np; i += kMT) {
      ci[i] = si[i];
      cz[i] = sz[i];
    }
    return;
  }
  block_select<kMT, kMK>(np, kc, kMK, sz, si, hist, scratch, &s_digit, &s_above, stage, ci, cz);
}

template <int NT>
__global__ __launch_bounds__(NT) void final_kernel(int cap_c, int k, int kc, int cap,
                                                         const int32_t* __restrict__ cand_idx,
                                                         const float* __restrict__ cand_z,
                                                         const int32_t* __restrict__ cand_count,
                                                         const int32_t* __restrict__ surv_idx,
                                                         const float* __restrict__ surv_z,
                                                         const int32_t* __restrict__ surv_count,
                                                         int32_t* __restrict__ out,
                                                         int32_t* __restrict__ out_count) {
  static_assert(kMaxSeg * kKeep <= NT * kReg, "every candidate fits the registers");
  __shared__ SelectLDS<NT> S;
  __shared__ int seg_kept[kMaxSeg];
  __shared__ int s_full;
  const int b = blockIdx.x, t = threadIdx.x;
  const int n = min(max(surv_count[b], 0), cap);
  const int nc = min(max(cand_count[b], 0), cap_c);
  const int32_t* ci = cand_idx + (size_t)b * cap_c;
  const float* cz = cand_z + (size_t)b * cap_c;
  int32_t* o = out + (size_t)b * k;
  if (kc >= k || n <= k) {   // nothing dropped that could belong
    select_list<NT>(n <= k ? n : nc, k, n <= k ? surv_idx + (size_t)b * cap : ci,
                n <= k ? surv_z + (size_t)b * cap : cz, o, out_count + b, S);
    return;
  }
  const int P = (n + kSlice - 1) / kSlice;   // <= kMaxSeg (host check)
  for (int i = t; i < kMaxSeg; i += NT) seg_kept[i] = 0;
  if (t == 0) s_full = nc <= k;   // every candidate kept while entries were dropped
  __syncthreads();
  if (nc > k) {
    // nc <= P * kc <= kMaxSeg * kKeep <= NT * kReg: register-resident
    const int chunk = (nc + NT - 1) / NT;
    if (chunk <= 16)
      block_select<NT, 16>(nc, k, chunk, cz, ci, S.hist, S.scratch, &S.digit, &S.above,
                                 S.stage, o, nullptr, seg_kept, kc);
    else if (chunk <= 32)
      block_select<NT, 32>(nc, k, chunk, cz, ci, S.hist, S.scratch, &S.digit, &S.above,
                                 S.stage, o, nullptr, seg_kept, kc);
    else
      block_select<NT, kReg>(nc, k, chunk, cz, ci, S.hist, S.scratch, &S.digit, &S.above,
                                   S.stage, o, nullptr, seg_kept, kc);
    __syncthreads();
    for (int p = t; p < P; p += NT)
      if (min(kSlice, n - p * kSlice) > kc && seg_kept[p] >= kc) s_full = 1;
    __syncthreads();
    if (!s_full) {
      if (t == 0) out_count[b] = k;
      return;
    }
  }
  // a truncated slice may hold more of the top-k: select over the whole list
  select_list<NT>(n, k, surv_idx + (size_t)b * cap, surv_z + (size_t)b * cap, o, out_count + b, S);
}

}  // namespace

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// candidates a slice keeps: kKeep when k is larger and the final stage can
// check every slice, else min(k, kSlice) (exact without a check)
static int slice_keep(int cap, int k) {
  const int P = (cap + kSlice - 1) / kSlice;
  return (k > kKeep && P <= kMaxSeg) ? kKeep : min(k, kSlice);
}

static int cand_capacity(int cap, int k) {
  const int P = (cap + kSlice - 1) / kSlice;
  return P * slice_keep(cap, k);
}

size_t topk_workspace_bytes(int B, int cap, int k) {
  if (cap <= kMBMinCap || k == 0) return 0;
  const size_t cc = (size_t)B * cand_capacity(cap, k);
  return up256(cc * 4) * 2 + up256((size_t)B * 4);
}

hipError_t launch_topk(int B, int cap, int k, const int32_t* surv_idx, const float* surv_z,
                       const int32_t* surv_count, int32_t* topk_idx, int32_t* topk_count,
                       void* ws, hipStream_t s) {
  if (cap <= kMBMinCap || k == 0) {
    hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(kThreads), 0, s, cap, k, surv_idx, surv_z,
                       surv_count, topk_idx, topk_count);
    return hipGetLastError();
  }
  const int P = (cap + kSlice - 1) / kSlice;
  const int kc = slice_keep(cap, k);
  const int cap_c = cand_capacity(cap, k);
  const size_t cc = (size_t)B * cap_c;
  int32_t* cand_idx = (int32_t*)ws;
  float* cand_z = (float*)((char*)ws + up256(cc * 4));
  int32_t* cand_count = (int32_t*)((char*)ws + 2 * up256(cc * 4));
  hipLaunchKernelGGL(slice_kernel, dim3(B, P), dim3(kMT), 0, s, cap, k, kc, cap_c, surv_idx,
                     surv_z, surv_count, cand_idx, cand_z, cand_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kc >= k) {
    hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(kThreads), 0, s, cap_c, k, cand_idx, cand_z,
                       cand_count, topk_idx, topk_count);
  } else {
    hipLaunchKernelGGL(final_kernel<kFinalThreads>, dim3(B), dim3(kFinalThreads), 0, s, cap_c, k, kc, cap, cand_idx,
                       cand_z, cand_count, surv_idx, surv_z, surv_count, topk_idx, topk_count);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Library-owned scratch for callers that cannot allocate (lsa_topk_noalloc):
// the candidate lists of the two-stage top-k live in this file-scope device
// array instead of a caller workspace.  Each GPU holds its own copy for the
// life of the process.  Host code never uses the array's name as an address:
// the device address is resolved once per device with hipGetSymbolAddress
// (with that device current) and kept.
__device__ __align__(256) unsigned char scratch[LSA_TOPK_NOALLOC_MAX_BYTES];

hipError_t topk_scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace lsa
