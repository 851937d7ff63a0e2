// lsa_project.hip -- query encoder (gist.science technical summary, section
// 2.1 "memory indexer": the current hidden state is mapped to a low-rank
// indexer query; section 2.3: only this projection is trained).
//   q[l][b] = bf16(Wq[l] h_b)  (fp32 accumulation),  g[l][b] = softplus(Wg[l] h_b)
//
// The weights dominate the traffic (every request shares them), so each
// weight row is read once per group of up to 32 requests: one block owns 32
// output rows (Wq rows, then the H gate rows) x 32 requests, its 4 wavefronts
// split the hidden dimension, run v_mfma_f32_32x32x16_bf16 with the weight
// rows as A and the hidden states as B, and are summed in LDS in a fixed
// order (deterministic); the epilogue rounds q to bf16 (nearest even) and
// applies softplus to the gate rows.
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

__global__ __launch_bounds__(256) void project_kernel(ProjectArgs a) {
  __shared__ float red[4][32][33];
  const int tile = blockIdx.x;
  const int l = blockIdx.y;
  const int bg = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int m = lane & 31;
  const int half = lane >> 5;
  const int HD = a.H * a.dI;
  const int R = HD + a.H;
  const int row0 = tile * 32;
  const int row = row0 + m;
  const uint16_t* wrow = nullptr;
  if (row < HD)
    wrow = a.Wq[l] + (size_t)row * a.D;
  else if (row < R)
    wrow = a.Wg[l] + (size_t)(row - HD) * a.D;
  const int bcol = bg * 32 + m;
  const uint16_t* hrow =
      bcol < a.B ? a.h + (size_t)l * a.h_layer_stride + (size_t)bcol * a.D : nullptr;

  const int kw = a.D / 4;
  const int k0 = wave * kw;
  f32x16 acc = f32x16{};
#pragma unroll 2
  for (int kc = k0; kc < k0 + kw; kc += 64) {
    u32x4 wa[4], hb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kk = kc + 32 * half + 8 * s;
      wa[s] = wrow ? __builtin_nontemporal_load((const u32x4*)(wrow + kk)) : u32x4{0u, 0u, 0u, 0u};
      hb[s] = hrow ? *(const u32x4*)(hrow + kk) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wa[s]),
                                                    __builtin_bit_cast(bf16x8, hb[s]), acc, 0,
                                                    0, 0);
  }
  // accumulator register r of lane l: output row (r&3) + 4*(l/32) + 8*(r/4), request l%32
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][(r & 3) + 4 * half + 8 * (r >> 2)][m] = acc[r];
  __syncthreads();
  for (int o = threadIdx.x; o < 1024; o += 256) {
    const int rr = o & 31;
    const int cc = o >> 5;
    const float v = ((red[0][rr][cc] + red[1][rr][cc]) + red[2][rr][cc]) + red[3][rr][cc];
    const int ro = row0 + rr;
    const int bo = bg * 32 + cc;
    if (bo < a.B && ro < R) {
      if (ro < HD)
        a.q[((size_t)l * a.B + bo) * HD + ro] = f32_to_bf16_rne(v);
      else
        a.g[((size_t)l * a.B + bo) * a.H + (ro - HD)] = softplus_f32(v);
    }
  }
}

}  // namespace

hipError_t launch_project(const ProjectArgs& a, hipStream_t s) {
  const int R = a.H * a.dI + a.H;
  dim3 grid((R + 31) / 32, a.L, (a.B + 31) / 32);
  hipLaunchKernelGGL(project_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsa
