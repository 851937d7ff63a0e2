// lsa_fetch.hip -- cold-pool fetch with reuse (gist.science technical summary,
// section 2.1 "dynamic fetch": every entry scoring >= 0.5 is moved from the
// CPU cold pool into GPU memory; paper.oopus.info review, section 2: the move
// is asynchronous and overlaps compute).
//
// The cold pool stays in pinned host memory and the GPU reads it in place:
// each wavefront copies whole rows (16 bytes per lane, so a 1 KiB row is one
// load and one store per lane) straight from host memory into a device-resident
// slot set, with several rows in flight per wave to cover the host link's
// latency.  No host thread touches the rows and the copy is ordered on the
// caller's stream like any other kernel, so it overlaps whatever runs on
// other streams.
//
// Reuse: a survivor already resident keeps its slot and is not read again;
// entries that stopped surviving free their slots; the i-th new survivor in
// entry order takes the i-th free slot in slot order.  A request whose
// survivors do not fit in its S slots is left untouched (fetch count -1).
// Six launches after the bitmap is cleared:
//   mark    survivor bitmap (one bit per entry) in the workspace
//   need    one block per request: the new survivors, compacted in entry
//           order, and the capacity check
//   evict   resident entries whose bit is clear leave their slots
//   assign  one block per request: free slots, compacted in slot order, each
//           given to the next new survivor
//   offsets prefix of the per-request copy counts
//   copy    host rows -> slots, spread over all waves across requests
#include <algorithm>

#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPer = 4;          // list elements per thread in the planning blocks
// The copy runs one single-wave block per compute unit, two rows in flight
// per wave (256 CUs x 2 KiB = 512 KiB in flight).  Host reads take several
// microseconds, so few bytes in flight keep the link busy (about 57 GB/s
// measured; 32 blocks of 4 waves move as fast).  What matters is how the
// copy shares the GPU with kernels on other streams: a wave per CU leaves
// every CU's memory pipeline nearly free, and 64% of the shorter job is
// hidden beside indexer triggers, against 40% with 32 blocks of 4 waves, 19%
// with 4 waves per CU, and none with 2048 blocks of 4 waves (every wave
// slot held for the whole copy).
constexpr int kCopyThreads = kWave;
constexpr int kCopyRows = 2;   // rows in flight per wavefront

// Survivor bitmap.  Ascending survivors put runs of lanes on the same 32-bit
// word; each run ORs its bits together (shuffle doubling over equal words) and
// only the run's first lane issues the atomic.
__global__ __launch_bounds__(256) void mark_kernel(int N, int cap,
                                                   const int32_t* __restrict__ surv_idx,
                                                   const int32_t* __restrict__ surv_count,
                                                   uint32_t* __restrict__ bits) {
  const int b = blockIdx.y;
  const int n = max(0, min(surv_count[b], cap));
  const size_t W = ((size_t)N + 31) >> 5;
  const int32_t* sv = surv_idx + (size_t)b * cap;
  uint32_t* bw = bits + (size_t)b * W;
  const int lane = lane_id();
  for (int base = blockIdx.x * 256; base < n; base += gridDim.x * 256) {   // block-uniform
    const int i = base + threadIdx.x;
    const int s = i < n ? sv[i] : -1;
    const bool ok = (unsigned)s < (unsigned)N;
    const int word = ok ? (s >> 5) : -1;
    uint32_t m = ok ? (1u << (s & 31)) : 0u;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t om = __shfl_down(m, off, kWave);
      const int ow = __shfl_down(word, off, kWave);
      if (lane + off < kWave && ow == word) m |= om;
    }
    const int pw = __shfl_up(word, 1, kWave);
    if (ok && (lane == 0 || pw != word)) atomicOr(&bw[word], m);
  }
}

__global__ __launch_bounds__(256) void evict_kernel(int N, int S,
                                                    const uint32_t* __restrict__ bits,
                                                    const int32_t* __restrict__ fetch_count,
                                                    int32_t* __restrict__ slot_of,
                                                    int32_t* __restrict__ entry_of) {
  const int b = blockIdx.y;
  if (fetch_count[b] < 0) return;
  const size_t W = ((size_t)N + 31) >> 5;
  const uint32_t* bw = bits + (size_t)b * W;
  int32_t* so = slot_of + (size_t)b * N;
  int32_t* eo = entry_of + (size_t)b * S;
  for (int j = blockIdx.x * 256 + threadIdx.x; j < S; j += gridDim.x * 256) {
    const int e = eo[j];
    if ((unsigned)e < (unsigned)N && !((bw[e >> 5] >> (e & 31)) & 1u)) {
      so[e] = -1;
      eo[j] = -1;
    }
  }
}

// One block per request: the survivors that are not resident, in entry order,
// go to `src`.  fetch_count[b] = their number, or -1 when the resident set
// cannot hold all survivors (kept + new > S); the tables are then left as they
// are by every later launch.
__global__ __launch_bounds__(kPlanThreads) void need_kernel(
    int N, int S, int cap, const int32_t* __restrict__ surv_idx,
    const int32_t* __restrict__ surv_count, const int32_t* __restrict__ slot_of,
    int32_t* __restrict__ src, int32_t* __restrict__ fetch_count) {
  __shared__ int scratch[kPlanThreads / kWave + 1];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int n = max(0, min(surv_count[b], cap));
  const int32_t* sv = surv_idx + (size_t)b * cap;
  const int32_t* so = slot_of + (size_t)b * N;
  int32_t* sb = src + (size_t)b * cap;
  int nn = 0, kept = 0;
  // thread t takes kPer consecutive survivors of each block-wide step, so the
  // list keeps entry order
  for (int base = 0; base < n; base += kPlanThreads * kPer) {
    int s[kPer];
    bool need[kPer];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = base + t * kPer + u;
      s[u] = i < n ? sv[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const bool in = (unsigned)s[u] < (unsigned)N;
      need[u] = in && so[s[u]] < 0;
      kept += (in && !need[u]) ? 1 : 0;
      c += need[u] ? 1 : 0;
    }
    int tot;
    int r = block_exclusive_scan<kPlanThreads>(c, scratch, &tot);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (need[u]) sb[nn + r++] = s[u];
    nn += tot;
  }
  int kept_all;
  (void)block_exclusive_scan<kPlanThreads>(kept, scratch, &kept_all);
  if (t == 0) fetch_count[b] = ((long long)kept_all + nn > S) ? -1 : nn;
}

// One block per request, after the evictions: free slots in slot order; the
// r-th takes the r-th new survivor.  dst receives each new survivor's slot.
__global__ __launch_bounds__(kPlanThreads) void assign_kernel(
    int N, int S, int cap, const int32_t* __restrict__ src,
    const int32_t* __restrict__ fetch_count, int32_t* __restrict__ slot_of,
    int32_t* __restrict__ entry_of, int32_t* __restrict__ dst) {
  __shared__ int scratch[kPlanThreads / kWave + 1];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int nn = fetch_count[b];
  if (nn <= 0) return;
  int32_t* so = slot_of + (size_t)b * N;
  int32_t* eo = entry_of + (size_t)b * S;
  const int32_t* sb = src + (size_t)b * cap;
  int32_t* db = dst + (size_t)b * cap;
  int placed = 0;
  for (int base = 0; base < S && placed < nn; base += kPlanThreads * kPer) {
    bool fr[kPer];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = base + t * kPer + u;
      fr[u] = j < S && eo[j] < 0;
      c += fr[u] ? 1 : 0;
    }
    int tot;
    int r = placed + block_exclusive_scan<kPlanThreads>(c, scratch, &tot);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (fr[u]) {
        if (r < nn) {
          const int j = base + t * kPer + u;
          const int sn = sb[r];
          eo[j] = sn;
          so[sn] = j;
          db[r] = j;
        }
        ++r;
      }
    }
    placed += tot;
  }
}

// Exclusive prefix of the per-request copy counts (a request that did not fit
// counts 0): offs[0..B], so the copy can spread rows over all its waves
// whatever the split between requests.  One block.
__global__ __launch_bounds__(kPlanThreads) void offsets_kernel(
    int B, const int32_t* __restrict__ fetch_count, int32_t* __restrict__ offs) {
  __shared__ int scratch[kPlanThreads / kWave + 1];
  int run = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int b = base + threadIdx.x;
    const int v = b < B ? max(fetch_count[b], 0) : 0;
    int tot;
    const int r = block_exclusive_scan<kPlanThreads>(v, scratch, &tot);
    if (b < B) offs[b] = run + r;
    run += tot;
  }
  if (threadIdx.x == 0) offs[B] = run;
}

// Copy from the cold pool (host memory read over the host link) into the
// resident rows.  Rows are numbered over all requests (offs); each wavefront
// takes kCopyRows consecutive rows, loads them all, then stores them.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(
    int B, int N, int S, int cap, int cpr, const unsigned char* __restrict__ cold,
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ offs, unsigned char* __restrict__ rows) {
  constexpr int kWPB = kCopyThreads / kWave;
  const int total = offs[B];
  const int wave = blockIdx.x * kWPB + threadIdx.x / kWave;
  const int stride = gridDim.x * kWPB * kCopyRows;
  const int lane = lane_id();
  const size_t rb = 16ull * cpr;
  // request of the wave's first row (binary search once); afterwards rows
  // only move forward, so the request index advances in registers
  int b = 0;
  {
    const int g = wave * kCopyRows;
    int hi = B;
    while (hi - b > 1) {
      const int mid = (b + hi) >> 1;
      if (offs[mid] <= g) b = mid;
      else hi = mid;
    }
  }
  int cur = offs[b], nxt = offs[b + 1];
  for (int g0 = wave * kCopyRows; g0 < total; g0 += stride) {
    const unsigned char* from[kCopyRows];
    unsigned char* to[kCopyRows];
#pragma unroll
    for (int u = 0; u < kCopyRows; ++u) {
      const int gi = g0 + u;
      from[u] = nullptr;
      to[u] = nullptr;
      if (gi < total) {
        while (gi >= nxt) {                  // gi < total = offs[B] bounds b below B
          ++b;
          cur = nxt;
          nxt = offs[b + 1];
        }
        const size_t e = (size_t)b * cap + (gi - cur);
        from[u] = cold + ((size_t)b * N + src[e]) * rb;
        to[u] = rows + ((size_t)b * S + dst[e]) * rb;
      }
    }
    for (int c = lane; c < cpr; c += kWave) {
      u32x4 v[kCopyRows];
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u)
        if (from[u]) v[u] = *(const u32x4*)(from[u] + 16ull * c);
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u)
        if (from[u]) *(u32x4*)(to[u] + 16ull * c) = v[u];
    }
  }
}

// hot[b][j] = rows[b][slot_of[b][idx[b][j]]]; zero rows for an index outside
// [0, N) or an entry that is not resident.
__global__ __launch_bounds__(256) void gather_resident_kernel(
    int N, int S, int k, int cpr, long long total, const unsigned char* __restrict__ rows,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ idx,
    unsigned char* __restrict__ hot) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long long row = i / cpr;   // b * k + j
  const int c = (int)(i - row * cpr);
  const long long b = row / k;
  const int e = idx[row];
  int slot = -1;
  if ((unsigned)e < (unsigned)N) slot = slot_of[b * N + e];
  const long long rb = 16ll * cpr;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if ((unsigned)slot < (unsigned)S) v = *(const u32x4*)(rows + (b * S + slot) * rb + 16ll * c);
  *(u32x4*)(hot + row * rb + 16ll * c) = v;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t fetch_workspace_bytes(int B, int N, int cap) {
  const size_t W = ((size_t)N + 31) >> 5;
  return align256((size_t)B * W * 4) + 2 * align256((size_t)B * cap * 4) +
         align256(((size_t)B + 1) * 4);
}

hipError_t launch_resident_reset(int B, int N, int S, int32_t* slot_of, int32_t* entry_of,
                                 hipStream_t s) {
  hipError_t e = launch_fill_i32(slot_of, (int64_t)B * N, -1, s);
  if (e != hipSuccess) return e;
  return launch_fill_i32(entry_of, (int64_t)B * S, -1, s);
}

hipError_t launch_fetch(int B, int N, int S, int row_bytes, const void* cold, int cap,
                        const int32_t* surv_idx, const int32_t* surv_count, int32_t* slot_of,
                        int32_t* entry_of, void* rows, int32_t* fetch_count, void* ws,
                        hipStream_t s) {
  const size_t W = ((size_t)N + 31) >> 5;
  uint32_t* bits = (uint32_t*)ws;
  int32_t* src = (int32_t*)((char*)ws + align256((size_t)B * W * 4));
  int32_t* dst = (int32_t*)((char*)src + align256((size_t)B * cap * 4));
  int32_t* offs = (int32_t*)((char*)dst + align256((size_t)B * cap * 4));
  hipError_t e = launch_fill_i32((int32_t*)bits, (int64_t)(B * W), 0, s);
  if (e != hipSuccess) return e;
  if (N > 0 && cap > 0) {
    const int gx = (int)std::min<long long>((cap + 255) / 256, 64);
    hipLaunchKernelGGL(mark_kernel, dim3(gx, B), dim3(256), 0, s, N, cap, surv_idx, surv_count,
                       bits);
  }
  hipLaunchKernelGGL(need_kernel, dim3(B), dim3(kPlanThreads), 0, s, N, S, cap, surv_idx,
                     surv_count, slot_of, src, fetch_count);
  if (S > 0) {
    const int gx = (int)std::min<long long>((S + 255) / 256, 64);
    hipLaunchKernelGGL(evict_kernel, dim3(gx, B), dim3(256), 0, s, N, S, bits, fetch_count,
                       slot_of, entry_of);
  }
  hipLaunchKernelGGL(assign_kernel, dim3(B), dim3(kPlanThreads), 0, s, N, S, cap, src,
                     fetch_count, slot_of, entry_of, dst);
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kPlanThreads), 0, s, B, fetch_count, offs);
  hipLaunchKernelGGL(copy_kernel, dim3(device_cu_count()), dim3(kCopyThreads), 0, s, B, N, S,
                     cap,
                     row_bytes / 16, (const unsigned char*)cold, src, dst, offs,
                     (unsigned char*)rows);
  return hipGetLastError();
}

hipError_t launch_gather_resident(int B, int N, int S, int k, int row_bytes, const void* rows,
                                  const int32_t* slot_of, const int32_t* idx, void* hot,
                                  hipStream_t s) {
  const int cpr = row_bytes / 16;
  const long long total = (long long)B * k * cpr;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(gather_resident_kernel, dim3((unsigned)blocks), dim3(256), 0, s, N, S, k,
                     cpr, total, (const unsigned char*)rows, slot_of, idx,
                     (unsigned char*)hot);
  return hipGetLastError();
}

}  // namespace lsa
