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
// Five launches after the bitmap is cleared:
//   mark    survivor bitmap (one bit per entry) in the workspace
//   need    one block per request: the new survivors, compacted in entry
//           order, and the capacity check
//   evict   resident entries whose bit is clear leave their slots
//   assign  one block per request: free slots, compacted in slot order, each
//           given to the next new survivor
//   copy    host rows -> slots
#include <algorithm>

#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kCopyThreads = 256;
constexpr int kCopyRows = 4;   // rows in flight per wavefront

__global__ __launch_bounds__(256) void mark_kernel(int N, int cap,
                                                   const int32_t* __restrict__ surv_idx,
                                                   const int32_t* __restrict__ surv_count,
                                                   uint32_t* __restrict__ bits) {
  const int b = blockIdx.y;
  const int n = max(0, min(surv_count[b], cap));
  const size_t W = ((size_t)N + 31) >> 5;
  const int32_t* sv = surv_idx + (size_t)b * cap;
  uint32_t* bw = bits + (size_t)b * W;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int s = sv[i];
    if ((unsigned)s < (unsigned)N) atomicOr(&bw[s >> 5], 1u << (s & 31));
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
  for (int base = 0; base < n; base += kPlanThreads) {
    const int i = base + t;
    bool need = false;
    int s = -1;
    if (i < n) {
      s = sv[i];
      if ((unsigned)s < (unsigned)N) {
        need = so[s] < 0;
        kept += need ? 0 : 1;
      }
    }
    int tot;
    const int r = block_exclusive_scan<kPlanThreads>(need ? 1 : 0, scratch, &tot);
    if (need) sb[nn + r] = s;
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
  for (int base = 0; base < S && placed < nn; base += kPlanThreads) {
    const int j = base + t;
    const bool fr = j < S && eo[j] < 0;
    int tot;
    const int r = block_exclusive_scan<kPlanThreads>(fr ? 1 : 0, scratch, &tot);
    if (fr && placed + r < nn) {
      const int s = sb[placed + r];
      eo[j] = s;
      so[s] = j;
      db[placed + r] = j;
    }
    placed += tot;
  }
}

// Wave-per-row copy from the cold pool (host memory read over the host link)
// into the resident rows; kCopyRows rows per wave are loaded before any is
// stored.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(
    int N, int S, int cap, int cpr, const unsigned char* __restrict__ cold,
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ fetch_count, unsigned char* __restrict__ rows) {
  const int b = blockIdx.y;
  const int nn = fetch_count[b];
  constexpr int kWPB = kCopyThreads / kWave;
  const int wave = blockIdx.x * kWPB + threadIdx.x / kWave;
  const int stride = gridDim.x * kWPB * kCopyRows;
  const int lane = lane_id();
  const size_t rb = 16ull * cpr;
  const int32_t* sb = src + (size_t)b * cap;
  const int32_t* db = dst + (size_t)b * cap;
  const unsigned char* cb = cold + (size_t)b * N * rb;
  unsigned char* ob = rows + (size_t)b * S * rb;
  for (int r0 = wave * kCopyRows; r0 < nn; r0 += stride) {
    int s[kCopyRows], d[kCopyRows];
#pragma unroll
    for (int u = 0; u < kCopyRows; ++u) {
      const bool ok = r0 + u < nn;
      s[u] = ok ? sb[r0 + u] : -1;
      d[u] = ok ? db[r0 + u] : -1;
    }
    for (int c = lane; c < cpr; c += kWave) {
      u32x4 v[kCopyRows];
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u)
        if (s[u] >= 0) v[u] = *(const u32x4*)(cb + (size_t)s[u] * rb + 16ull * c);
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u)
        if (s[u] >= 0) *(u32x4*)(ob + (size_t)d[u] * rb + 16ull * c) = v[u];
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
  return align256((size_t)B * W * 4) + 2 * align256((size_t)B * cap * 4);
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
  const int rows_per_block = (kCopyThreads / kWave) * kCopyRows;
  const int need_blocks = (int)std::min<long long>(
      ((long long)std::min(cap, N) + rows_per_block - 1) / rows_per_block, 1 << 20);
  const int gx = std::max(1, std::min(need_blocks, std::max(16, 2048 / B)));
  hipLaunchKernelGGL(copy_kernel, dim3(gx, B), dim3(kCopyThreads), 0, s, N, S, cap,
                     row_bytes / 16, (const unsigned char*)cold, src, dst, fetch_count,
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
