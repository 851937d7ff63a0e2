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
// Seven launches after the bitmap is cleared; the planning ones run one block
// per chunk of 4096 survivors or slots:
//   mark    survivor bitmap (one bit per entry) in the workspace
//   need    count, then write: the new survivors compacted in entry order,
//           and the capacity check
//   evict   resident entries whose bit is clear leave their slots; free
//           slots counted per chunk
//   assign  free slots compacted in slot order, each given to the next new
//           survivor
//   offsets prefix of the per-request copy counts
//   copy    host rows -> slots, spread over all waves across requests
#include <algorithm>

#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPer = 4;          // list elements per thread in the planning blocks
constexpr int kChunk = kPlanThreads * kPer;   // list elements per planning block
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

// Sum over a request's earlier chunks of one per-chunk counter (wave 0 of the
// block); the result is broadcast through LDS.
__device__ __forceinline__ int earlier_chunks_sum(const int32_t* cnt, int stride, int c,
                                                  int* slot) {
  if (threadIdx.x < kWave) {
    int acc = 0;
    for (int i = lane_id(); i < c; i += kWave) acc += cnt[(size_t)i * stride];
    acc = wave_sum(acc);
    if (lane_id() == 0) *slot = acc;
  }
  __syncthreads();
  return *slot;
}

// Survivor chunks of kChunk entries, one block each: how many are new (not
// resident) and how many are resident.  ccnt[b][c] = {new, kept}.
__global__ __launch_bounds__(kPlanThreads) void need_count_kernel(
    int N, int cap, int nch, const int32_t* __restrict__ surv_idx,
    const int32_t* __restrict__ surv_count, const int32_t* __restrict__ slot_of,
    int32_t* __restrict__ ccnt) {
  __shared__ int scratch[kPlanThreads / kWave + 1];
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int n = max(0, min(surv_count[b], cap));
  const int32_t* sv = surv_idx + (size_t)b * cap;
  const int32_t* so = slot_of + (size_t)b * N;
  int nw = 0, kp = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = c * kChunk + t * kPer + u;
    const int s = i < n ? sv[i] : -1;
    if ((unsigned)s < (unsigned)N) {
      if (so[s] < 0) ++nw;
      else ++kp;
    }
  }
  int tn, tk;
  (void)block_exclusive_scan<kPlanThreads>(nw, scratch, &tn);
  (void)block_exclusive_scan<kPlanThreads>(kp, scratch, &tk);
  if (t == 0) {
    ccnt[((size_t)b * nch + c) * 2] = tn;
    ccnt[((size_t)b * nch + c) * 2 + 1] = tk;
  }
}

// The new survivors of each chunk, in entry order, at the chunk's offset in
// `src`.  Chunk 0 also writes fetch_count[b]: the number of new survivors, or
// -1 when kept + new > S (the request is then left as it is).
__global__ __launch_bounds__(kPlanThreads) void need_write_kernel(
    int N, int S, int cap, int nch, const int32_t* __restrict__ surv_idx,
    const int32_t* __restrict__ surv_count, const int32_t* __restrict__ slot_of,
    const int32_t* __restrict__ ccnt, int32_t* __restrict__ src,
    int32_t* __restrict__ fetch_count) {
  __shared__ int scratch[kPlanThreads / kWave + 1];
  __shared__ int s_base;
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int n = max(0, min(surv_count[b], cap));
  const int32_t* sv = surv_idx + (size_t)b * cap;
  const int32_t* so = slot_of + (size_t)b * N;
  const int32_t* cb = ccnt + (size_t)b * nch * 2;
  if (c == 0 && t < kWave) {
    long long nn = 0, kept = 0;
    for (int i = lane_id(); i < nch; i += kWave) {
      nn += cb[2 * i];
      kept += cb[2 * i + 1];
    }
    nn = wave_sum((int)nn);
    kept = wave_sum((int)kept);
    if (lane_id() == 0) fetch_count[b] = (kept + nn > S) ? -1 : (int)nn;
  }
  const int base = earlier_chunks_sum(cb, 2, c, &s_base);
  int s[kPer];
  bool need[kPer];
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = c * kChunk + t * kPer + u;
    s[u] = i < n ? sv[i] : -1;
    need[u] = (unsigned)s[u] < (unsigned)N && so[s[u]] < 0;
    cnt += need[u] ? 1 : 0;
  }
  int tot;
  int r = base + block_exclusive_scan<kPlanThreads>(cnt, scratch, &tot);
  int32_t* sb = src + (size_t)b * cap;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (need[u]) sb[r++] = s[u];
}

// Slot chunks of kChunk slots, one block each: resident entries whose bitmap
// bit is clear leave their slots; fcnt[b][c] = free slots of the chunk
// afterwards.  Requests that do not fit are skipped.  Only the first
// Ss = min(S, N) slots are scanned: new entries always take the lowest free
// slots, so at most N entries ever occupy slots below N.
__global__ __launch_bounds__(kPlanThreads) void evict_kernel(
    int N, int S, int Ss, int nsc, const uint32_t* __restrict__ bits,
    const int32_t* __restrict__ fetch_count, int32_t* __restrict__ slot_of,
    int32_t* __restrict__ entry_of, int32_t* __restrict__ fcnt) {
  __shared__ int scratch[kPlanThreads / kWave + 1];
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  if (fetch_count[b] < 0) return;   // block-uniform
  const size_t W = ((size_t)N + 31) >> 5;
  const uint32_t* bw = bits + (size_t)b * W;
  int32_t* so = slot_of + (size_t)b * N;
  int32_t* eo = entry_of + (size_t)b * S;
  int fr = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = c * kChunk + t * kPer + u;
    if (j < Ss) {
      const int e = eo[j];
      if ((unsigned)e < (unsigned)N && !((bw[e >> 5] >> (e & 31)) & 1u)) {
        so[e] = -1;
        eo[j] = -1;
        ++fr;
      } else if (e < 0) {
        ++fr;
      }
    }
  }
  int tot;
  (void)block_exclusive_scan<kPlanThreads>(fr, scratch, &tot);
  if (t == 0) fcnt[(size_t)b * nsc + c] = tot;
}

// Slot chunks again: the free slots of the chunk, in slot order, at the
// chunk's offset among the request's free slots; the r-th free slot takes the
// r-th new survivor (r < fetch_count).  dst receives each new survivor's slot.
__global__ __launch_bounds__(kPlanThreads) void assign_kernel(
    int N, int S, int Ss, int cap, int nsc, const int32_t* __restrict__ src,
    const int32_t* __restrict__ fetch_count, const int32_t* __restrict__ fcnt,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ entry_of,
    int32_t* __restrict__ dst) {
  __shared__ int scratch[kPlanThreads / kWave + 1];
  __shared__ int s_base;
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int nn = fetch_count[b];
  if (nn <= 0) return;   // block-uniform
  const int base = earlier_chunks_sum(fcnt + (size_t)b * nsc, 1, c, &s_base);
  if (base >= nn) return;   // block-uniform: earlier chunks hold enough slots
  int32_t* so = slot_of + (size_t)b * N;
  int32_t* eo = entry_of + (size_t)b * S;
  const int32_t* sb = src + (size_t)b * cap;
  int32_t* db = dst + (size_t)b * cap;
  bool fr[kPer];
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = c * kChunk + t * kPer + u;
    fr[u] = j < Ss && eo[j] < 0;
    cnt += fr[u] ? 1 : 0;
  }
  int tot;
  int r = base + block_exclusive_scan<kPlanThreads>(cnt, scratch, &tot);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (fr[u]) {
      if (r < nn) {
        const int j = c * kChunk + t * kPer + u;
        const int sn = sb[r];
        eo[j] = sn;
        so[sn] = j;
        db[r] = j;
      }
      ++r;
    }
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

namespace {

int plan_chunks(long long n) { return (int)std::max<long long>(1, (n + kChunk - 1) / kChunk); }

}  // namespace

size_t fetch_workspace_bytes(int B, int N, int cap) {
  const size_t W = ((size_t)N + 31) >> 5;
  const size_t nchN = (size_t)plan_chunks(N);
  return align256((size_t)B * W * 4) + 2 * align256((size_t)B * cap * 4) +
         align256(((size_t)B + 1) * 4) + align256((size_t)B * nchN * 2 * 4) +
         align256((size_t)B * nchN * 4);
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
  const int nch = plan_chunks(std::min(cap, N));      // survivor chunks per request
  const int Ss = std::min(S, N);
  const int nsc = plan_chunks(Ss);                     // slot chunks per request
  const size_t nchN = (size_t)plan_chunks(N);
  char* p = (char*)ws;
  uint32_t* bits = (uint32_t*)p;
  p += align256((size_t)B * W * 4);
  int32_t* src = (int32_t*)p;
  p += align256((size_t)B * cap * 4);
  int32_t* dst = (int32_t*)p;
  p += align256((size_t)B * cap * 4);
  int32_t* offs = (int32_t*)p;
  p += align256(((size_t)B + 1) * 4);
  int32_t* ccnt = (int32_t*)p;
  p += align256((size_t)B * nchN * 2 * 4);
  int32_t* fcnt = (int32_t*)p;
  hipError_t e = launch_fill_i32((int32_t*)bits, (int64_t)(B * W), 0, s);
  if (e != hipSuccess) return e;
  if (N > 0 && cap > 0) {
    const int gx = (int)std::min<long long>((cap + 255) / 256, 64);
    hipLaunchKernelGGL(mark_kernel, dim3(gx, B), dim3(256), 0, s, N, cap, surv_idx, surv_count,
                       bits);
  }
  hipLaunchKernelGGL(need_count_kernel, dim3(nch, B), dim3(kPlanThreads), 0, s, N, cap, nch,
                     surv_idx, surv_count, slot_of, ccnt);
  hipLaunchKernelGGL(need_write_kernel, dim3(nch, B), dim3(kPlanThreads), 0, s, N, S, cap, nch,
                     surv_idx, surv_count, slot_of, ccnt, src, fetch_count);
  hipLaunchKernelGGL(evict_kernel, dim3(nsc, B), dim3(kPlanThreads), 0, s, N, S, Ss, nsc, bits,
                     fetch_count, slot_of, entry_of, fcnt);
  hipLaunchKernelGGL(assign_kernel, dim3(nsc, B), dim3(kPlanThreads), 0, s, N, S, Ss, cap, nsc,
                     src, fetch_count, fcnt, slot_of, entry_of, dst);
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kPlanThreads), 0, s, B, fetch_count, offs);
  hipLaunchKernelGGL(copy_kernel, dim3(device_cu_count()), dim3(kCopyThreads), 0, s, B, N, S,
                     cap, row_bytes / 16, (const unsigned char*)cold, src, dst, offs,
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
