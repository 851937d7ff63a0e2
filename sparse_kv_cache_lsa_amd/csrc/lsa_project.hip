// lsa_project.hip -- query encoder (gist.science technical summary, section
// 2.1 "memory indexer": the current hidden state is mapped to a low-rank
// indexer query; section 2.3: only this projection is trained).
//   q[l][b] = bf16(Wq[l] h_b)  (fp32 accumulation),  g[l][b] = softplus(Wg[l] h_b)
//
// The weights dominate the traffic (every request shares them), so each
// weight row is read once per group of up to 32 requests: one block owns 64
// output rows (Wq rows, then the H gate rows; H*dI is a multiple of 64, so a
// block never straddles the two matrices) x 32 requests.  Its 8 wavefronts
// split the hidden dimension, run v_mfma_f32_16x16x32_bf16 with the weight
// rows as A and the hidden states as B (loads batched two k-steps deep
// through buffer resources, no branches), and are summed through LDS in a
// fixed tree order (deterministic); the epilogue rounds q to bf16 (nearest
// even) and applies softplus to the gate rows.
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kPW = 8;   // wavefronts per block; each takes D / kPW of the hidden dimension
constexpr int kRT = 4;   // 16-row MFMA tiles per block (64 output rows)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFFu ? bytes : 0x7FFFFFFFu),
                                           0x00020000);
}

// Plain (cached) loads: a weight line is read by two consecutive k-steps, and
// the nontemporal hint made the second one miss.
__device__ __forceinline__ bf16x8 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__global__ __launch_bounds__(64 * kPW) void project_kernel(ProjectArgs a) {
  __shared__ float red[kPW / 2][kRT * 8][64];
  const int tile = blockIdx.x;
  const int l = blockIdx.y;
  const int bg = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int m = lane & 31;
  const int half = lane >> 5;
  const int HD = a.H * a.dI;
  const int R = HD + a.H;
  const int row0 = tile * 16 * kRT;
  // A 32-row tile lies wholly in W_q or wholly in W_g (H*dI is a multiple of
  // 32).  Buffer range checks return 0 for rows past the gate rows and for
  // requests past B, so the loads need no branches (a branch around a load
  // makes the compiler wait for every load in flight).
  const bool gate_tile = row0 >= HD;
  const __amdgpu_buffer_rsrc_t ra =
      gate_tile ? rsrc(a.Wg[l], (size_t)a.H * a.D * 2) : rsrc(a.Wq[l], (size_t)HD * a.D * 2);
  const uint32_t aoff = (uint32_t)(row0 + m - (gate_tile ? HD : 0)) * a.D * 2;
  const __amdgpu_buffer_rsrc_t rb =
      rsrc(a.h + (size_t)l * a.h_layer_stride, (size_t)a.B * a.D * 2);
  const uint32_t boff = (uint32_t)(bg * 32 + m) * a.D * 2;

  const int kw = a.D / kPW;
  const int k0 = wave * kw, k1 = k0 + kw;
  // v_mfma_f32_16x16x32_bf16: lane (n = l%16, g = l/16) holds k = 8g..8g+7
  // of row n, so one load instruction reads 64 contiguous bytes of each of 16
  // weight rows; the block covers 64 rows (kRT tiles) x 32 requests (2 tiles)
  const int n16 = lane & 15, g = lane >> 4;
  uint32_t ao[kRT];
#pragma unroll
  for (int i = 0; i < kRT; ++i) ao[i] = (uint32_t)(row0 + 16 * i + n16 - (gate_tile ? HD : 0)) * a.D * 2;
  const uint32_t bo0 = (uint32_t)(bg * 32 + n16) * a.D * 2;
  const uint32_t bo1 = bo0 + 16u * a.D * 2;
  f32x4 c[kRT][2];
#pragma unroll
  for (int i = 0; i < kRT; ++i) { c[i][0] = f32x4{}; c[i][1] = f32x4{}; }
  int kc = k0;
  for (; kc + 64 <= k1; kc += 64) {   // two k-steps of 32 per batch of loads
    bf16x8 av[2][kRT], b0[2], b1[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t kk = (uint32_t)(kc + 32 * s + 8 * g) * 2;
#pragma unroll
      for (int i = 0; i < kRT; ++i) av[s][i] = load8(ra, ao[i] + kk);
      b0[s] = load8(rb, bo0 + kk);
      b1[s] = load8(rb, bo1 + kk);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < kRT; ++i) {
        c[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s][i], b0[s], c[i][0], 0, 0, 0);
        c[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s][i], b1[s], c[i][1], 0, 0, 0);
      }
  }
  if (kc < k1) {   // D / kPW is a multiple of 32: at most one k-step remains
    const uint32_t kk = (uint32_t)(kc + 8 * g) * 2;
    const bf16x8 b0 = load8(rb, bo0 + kk), b1 = load8(rb, bo1 + kk);
#pragma unroll
    for (int i = 0; i < kRT; ++i) {
      const bf16x8 av = load8(ra, ao[i] + kk);
      c[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b0, c[i][0], 0, 0, 0);
      c[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b1, c[i][1], 0, 0, 0);
    }
  }
  // C element r of lane l: row 4*(l/16) + r, column l%16 of its 16x16 tile;
  // the waves' partial sums are added through LDS in a fixed tree order
  float acc[kRT * 8];
#pragma unroll
  for (int i = 0; i < kRT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[i * 8 + r] = c[i][0][r]; acc[i * 8 + 4 + r] = c[i][1][r]; }
#pragma unroll
  for (int width = kPW / 2; width >= 1; width >>= 1) {
    if (wave >= width && wave < 2 * width)
#pragma unroll
      for (int r = 0; r < kRT * 8; ++r) red[wave - width][r][lane] = acc[r];
    __syncthreads();
    if (wave < width)
#pragma unroll
      for (int r = 0; r < kRT * 8; ++r) acc[r] += red[wave][r][lane];
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < kRT * 8; ++r) {
      const int tr = r >> 3, tc = (r >> 2) & 1;
      const int ro = row0 + 16 * tr + 4 * g + (r & 3);
      const int bo = bg * 32 + 16 * tc + n16;
      if (bo < a.B && ro < R) {
        if (ro < HD)
          a.q[((size_t)l * a.B + bo) * HD + ro] = f32_to_bf16_rne(acc[r]);
        else
          a.g[((size_t)l * a.B + bo) * a.H + (ro - HD)] = softplus_f32(acc[r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_project(const ProjectArgs& a, hipStream_t s) {
  const int R = a.H * a.dI + a.H;
  dim3 grid((R + 16 * kRT - 1) / (16 * kRT), a.L, (a.B + 31) / 32);
  hipLaunchKernelGGL(project_kernel, grid, dim3(64 * kPW), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsa
