// lsa_project.hip -- query encoder (gist.science technical summary, section
// 2.1 "memory indexer": the current hidden state is mapped to a low-rank
// indexer query; section 2.3: only this projection is trained).
//   q[l][b] = bf16(Wq[l] h_b)  (fp32 accumulation),  g[l][b] = softplus(Wg[l] h_b)
//
// The weights dominate the traffic (every request shares them), so each
// weight row is read once per group of up to 32 requests.  A layer's output
// rows (Wq rows, then the H gate rows) form 16-row tiles; the tiles of each
// (layer, request group) are split evenly over about one block per compute
// unit, so every compute unit streams the same number of weight bytes and
// reads its group's hidden states once for all its rows.  The 8 wavefronts of
// a block split the hidden dimension, run v_mfma_f32_16x16x32_bf16 with the
// weight rows as A and the hidden states as B (loads through buffer
// resources, no branches, the next 64-k unit in flight while the current one
// is multiplied), and are summed through LDS in a fixed tree order
// (deterministic); the epilogue rounds q to bf16 (nearest even) and applies
// softplus to the gate rows.
//
// Packed weights (lsa_pack_query_weights, a load-time layout): the operand
// fragments of tile t, 64-k unit u and step s lie in one 1 KiB run, lane l's
// 16 bytes at l * 16, so every weight load instruction reads 1 KiB of
// contiguous memory instead of 64 bytes of each of 16 rows (61.7 -> 54.1 us
// for the 1M-context shapes with the Infinity Cache flushed).  The products,
// their order and the results are the same.
#include "lsa_device.h"
#include "lsa_launch.h"

#include <algorithm>
#include <atomic>

namespace lsa {
namespace {

constexpr int kPW = 8;        // wavefronts per block; they share out the hidden dimension
constexpr int kMaxTiles = 8;  // 16-row MFMA tiles one block accumulates at a time
constexpr uint32_t kFar = 0x80000000u;   // buffer offset past every weight matrix (loads return 0)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFFu ? bytes : 0x7FFFFFFFu),
                                           0x00020000);
}

// Row-major weights use plain (cached) loads: a weight line is read by two
// consecutive k-steps, and the nontemporal hint made the second one miss.
// Packed weights are read exactly once, in whole 1 KiB runs: nontemporal
// (51.8 against 53.4 us at the 1M-context shapes).
template <bool NT = false>
__device__ __forceinline__ bf16x8 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}

// One 64-k unit (two MFMA k-steps) of a wave's operands: TM 16-row weight
// fragments and the two 16-request fragments of h, for each k-step.
template <int TM>
struct Unit {
  bf16x8 a[2][TM];
  bf16x8 b0[2], b1[2];
};

template <int TM, bool PK>
__device__ __forceinline__ void load_unit(Unit<TM>& U, const __amdgpu_buffer_rsrc_t (&ra)[TM],
                                          const uint32_t (&ao)[TM], __amdgpu_buffer_rsrc_t rb,
                                          uint32_t bo0, uint32_t bo1, int u, int g) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t kk = (uint32_t)(64 * u + 32 * s + 8 * g) * 2;
    const uint32_t pk = (uint32_t)(2 * u + s) * 1024;   // packed: this step's 1 KiB run
#pragma unroll
    for (int i = 0; i < TM; ++i) U.a[s][i] = load8<PK>(ra[i], ao[i] + (PK ? pk : kk));
    U.b0[s] = load8(rb, bo0 + kk);
    U.b1[s] = load8(rb, bo1 + kk);
  }
}

template <int TM>
__device__ __forceinline__ void mma_unit(const Unit<TM>& U, f32x4 (&c)[TM][2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      c[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(U.a[s][i], U.b0[s], c[i][0], 0, 0, 0);
      c[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(U.a[s][i], U.b1[s], c[i][1], 0, 0, 0);
    }
}

// Grid (nbs, L, ceil(B/32)).  The R = H*dI + H output rows of a layer form
// T = ceil(R/16) tiles of 16 rows; block p of a (layer, request group) owns
// tiles [p*T/nbs, (p+1)*T/nbs) -- at most TM of them -- so every block streams
// the same number of weight bytes (to within one tile) and reads its group's
// h once for all its rows.
template <int TM, bool PK>
__global__ __launch_bounds__(64 * kPW) void project_kernel(ProjectArgs a, int nbs) {
  __shared__ float red[kPW / 2][TM * 8][64];
  const int p = blockIdx.x;
  const int l = blockIdx.y;
  const int bg = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int HD = a.H * a.dI;
  const int R = HD + a.H;
  const int T = (R + 15) >> 4;
  const int t0 = (int)((int64_t)p * T / nbs);
  const int nt = (int)((int64_t)(p + 1) * T / nbs) - t0;
  // v_mfma_f32_16x16x32_bf16: lane (n = l%16, g = l/16) holds k = 8g..8g+7
  // of row n, so one load instruction reads 64 contiguous bytes of each of 16
  // weight rows.  A tile lies wholly in W_q or wholly in W_g (H*dI is a
  // multiple of 64).  Buffer range checks return 0 for rows past the gate
  // rows, for requests past B and for the unused tile slots (offset kFar), so
  // the loads need no branches (a branch around a load makes the compiler
  // wait for every load in flight).
  const int n16 = lane & 15, g = lane >> 4;
  __amdgpu_buffer_rsrc_t ra[TM];
  uint32_t ao[TM];
  if constexpr (PK) {
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.Wp[l], (size_t)T * (a.D >> 6) * 2048);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      ra[i] = rp;
      ao[i] = i < nt ? (uint32_t)(t0 + i) * (uint32_t)(a.D >> 6) * 2048u + 16u * lane : kFar;
    }
  } else {
    const __amdgpu_buffer_rsrc_t rq = rsrc(a.Wq[l], (size_t)HD * a.D * 2);
    const __amdgpu_buffer_rsrc_t rg = rsrc(a.Wg[l], (size_t)a.H * a.D * 2);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r0 = 16 * (t0 + i);
      const bool gate = r0 >= HD;
      ra[i] = gate ? rg : rq;
      ao[i] = i < nt ? (uint32_t)(r0 + n16 - (gate ? HD : 0)) * a.D * 2 : kFar;
    }
  }
  const __amdgpu_buffer_rsrc_t rb =
      rsrc(a.h + (size_t)l * a.h_layer_stride, (size_t)a.B * a.D * 2);
  const uint32_t bo0 = (uint32_t)(bg * 32 + n16) * a.D * 2;
  const uint32_t bo1 = bo0 + 16u * a.D * 2;
  f32x4 c[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i) { c[i][0] = f32x4{}; c[i][1] = f32x4{}; }
  // The hidden dimension is cut into 64-k units dealt round-robin to the
  // waves (unit u to wave u % kPW): at any time the block's waves read one
  // contiguous kPW*128-byte run of each of its weight rows.
  // The next unit's loads are issued before the current unit's products, so
  // two units per wave are in flight.
  const int nU = a.D >> 6;
  const int cnt = (nU - wave + kPW - 1) / kPW;
  if (cnt > 0) {
    Unit<TM> cur;
    load_unit<TM, PK>(cur, ra, ao, rb, bo0, bo1, wave, g);
    int u = wave;
    for (int j = 1; j < cnt; ++j) {
      u += kPW;
      Unit<TM> nxt;
      load_unit<TM, PK>(nxt, ra, ao, rb, bo0, bo1, u, g);
      __builtin_amdgcn_sched_barrier(0);   // keep those loads ahead of the products
      mma_unit(cur, c);
      cur = nxt;
    }
    mma_unit(cur, c);
  }
  // C element r of lane l: row 4*(l/16) + r, column l%16 of its 16x16 tile;
  // the waves' partial sums are added through LDS in a fixed tree order
  float acc[TM * 8];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[i * 8 + r] = c[i][0][r]; acc[i * 8 + 4 + r] = c[i][1][r]; }
#pragma unroll
  for (int width = kPW / 2; width >= 1; width >>= 1) {
    if (wave >= width && wave < 2 * width)
#pragma unroll
      for (int r = 0; r < TM * 8; ++r) red[wave - width][r][lane] = acc[r];
    __syncthreads();
    if (wave < width)
#pragma unroll
      for (int r = 0; r < TM * 8; ++r) acc[r] += red[wave][r][lane];
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < TM * 8; ++r) {
      const int ti = r >> 3, tc = (r >> 2) & 1;
      const int ro = 16 * (t0 + ti) + 4 * g + (r & 3);
      const int bo = bg * 32 + 16 * tc + n16;
      if (ti < nt && bo < a.B && ro < R) {
        if (ro < HD)
          a.q[((size_t)l * a.B + bo) * HD + ro] = f32_to_bf16_rne(acc[r]);
        else
          a.g[((size_t)l * a.B + bo) * a.H + (ro - HD)] = softplus_f32(acc[r]);
      }
    }
  }
}

template <int TM>
void launch_tm(const ProjectArgs& a, int nbs, int BG, hipStream_t s) {
  if (a.Wp[0])
    hipLaunchKernelGGL((project_kernel<TM, true>), dim3(nbs, a.L, BG), dim3(64 * kPW), 0, s, a, nbs);
  else
    hipLaunchKernelGGL((project_kernel<TM, false>), dim3(nbs, a.L, BG), dim3(64 * kPW), 0, s, a, nbs);
}

// Packed layout of one layer: 16 bytes of tile t (16 rows: W_q rows, then
// the W_g rows, zero past them), unit u, step s, lane l at
// ((t * nU + u) * 2 + s) * 1024 + 16 l: row 16 t + l % 16, columns
// 64 u + 32 s + 8 (l / 16) .. +8.  Grid (nU, T), 128 threads (s, l).
__global__ __launch_bounds__(128) void pack_kernel(int HD, int H, int D,
                                                   const uint16_t* __restrict__ Wq,
                                                   const uint16_t* __restrict__ Wg,
                                                   unsigned char* __restrict__ out) {
  const int u = blockIdx.x, t = blockIdx.y;
  const int st = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int row = 16 * t + (l & 15), col = 64 * u + 32 * st + 8 * (l >> 4);
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (row < HD)
    v = *(const u32x4*)(Wq + (size_t)row * D + col);
  else if (row < HD + H)
    v = *(const u32x4*)(Wg + (size_t)(row - HD) * D + col);
  *(u32x4*)(out + ((size_t)(t * (D >> 6) + u) * 2 + st) * 1024 + 16 * l) = v;
}

}  // namespace

size_t packed_weights_bytes(int H, int dI, int D) {
  const size_t T = ((size_t)H * dI + H + 15) / 16;
  return T * (size_t)(D / 64) * 2048;
}

hipError_t launch_pack_weights(int H, int dI, int D, const uint16_t* Wq, const uint16_t* Wg,
                               void* packed, hipStream_t s) {
  const int T = (H * dI + H + 15) / 16;
  hipLaunchKernelGGL(pack_kernel, dim3(D / 64, T), dim3(128), 0, s, H * dI, H, D, Wq, Wg,
                     (unsigned char*)packed);
  return hipGetLastError();
}

// Compute units of the current device (queried once per device).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_project(const ProjectArgs& a, hipStream_t s) {
  const int R = a.H * a.dI + a.H;
  const int T = (R + 15) / 16;
  const int BG = (a.B + 31) / 32;
  // one block per compute unit when the tiles allow it (at most kMaxTiles
  // tiles per block; more blocks otherwise), the tiles split evenly
  const int segs = a.L * BG;
  int nbs = std::max(1, device_cu_count() / segs);
  nbs = std::min(nbs, T);
  nbs = std::max(nbs, (T + kMaxTiles - 1) / kMaxTiles);
  const int tm = (T + nbs - 1) / nbs;
  if (tm <= 1) launch_tm<1>(a, nbs, BG, s);
  else if (tm <= 2) launch_tm<2>(a, nbs, BG, s);
  else if (tm <= 3) launch_tm<3>(a, nbs, BG, s);
  else if (tm <= 4) launch_tm<4>(a, nbs, BG, s);
  else if (tm <= 5) launch_tm<5>(a, nbs, BG, s);
  else if (tm <= 6) launch_tm<6>(a, nbs, BG, s);
  else if (tm <= 7) launch_tm<7>(a, nbs, BG, s);
  else launch_tm<8>(a, nbs, BG, s);
  return hipGetLastError();
}

}  // namespace lsa
