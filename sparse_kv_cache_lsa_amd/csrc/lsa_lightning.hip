// lsa_lightning.hip -- fine-grained score of the fetched entries (gist.science
// technical summary, section 2.1, hierarchical-selection bullet: inside the
// fetched subset the top-k uses the model's native Lightning Indexer, which
// the pages name without defining it; this library takes its published form):
//   score[b][i] = sigma_s * sum_h w[b][h] * relu(q[b][h] . k_b[s]),  s = surv_idx[b][i]
// with the indexer's own keys k (bf16, or e4m3 with a positive fp32 scale
// sigma per entry, so relu(sigma x) = sigma relu(x)).
//
// The per-head relu keeps the heads apart, so this is a real H x dI x n
// contraction per request: it runs on v_mfma_f32_16x16x32_bf16 (e4m3 keys
// widened exactly to bf16), A = the query heads, B = the survivors' keys.
// Block = (group of tiles, request), 4 wavefronts; wave w owns heads
// 16 w .. 16 w + 15.  A tile of 256 survivors: their key rows are gathered by
// index (one row per 8 or 16 threads, 16 B each) into LDS as bf16; each wave
// forms its 16 heads x 16 survivors products 16 survivors at a time, applies
// relu and the head weights in the epilogue and sums its heads; the four
// waves' sums are added in LDS in wave order and scaled.
#include "lsa_device.h"
#include "lsa_launch.h"

#include <algorithm>

namespace lsa {
namespace {

constexpr int kLTile = 256;   // survivors per tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

struct LightArgs {
  const void* keys;          // [B][N][dI]
  const float* scale;        // [B][N] (e4m3) or null
  const uint16_t* q;         // [B][H][dI]
  const float* w;            // [B][H]
  const int32_t* surv_idx;   // [B][cap]
  const int32_t* surv_count; // [B]
  float* score;              // [B][cap]
  int N, cap, H;
};

// KT 0: bf16 keys, 1: e4m3 keys + scale.  DI: 64 or 128.
template <int KT, int DI>
__global__ __launch_bounds__(256) void lightning_kernel(LightArgs a) {
  constexpr int RB = DI * 2;                 // bf16 row bytes in LDS
  constexpr int RS = RB + 16;                // padded LDS row stride
  constexpr int KRB = KT == 1 ? DI : 2 * DI; // key row bytes in memory
  constexpr int TPR = KRB / 16;              // threads per key row (16 B each)
  constexpr int KS = DI / 32;                // K-steps of 32 dims
  __shared__ __attribute__((aligned(16))) unsigned char rows[kLTile * RS];
  __shared__ float part[4][kLTile];
  __shared__ int s_idx[kLTile];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  const int count = min(max(a.surv_count[b], 0), a.cap);
  const int h0 = 16 * wave;
  const bool active = h0 < a.H;

  // query fragments of heads h0 .. h0 + 15 (A operand): lane (n, g) holds
  // head n, dims 32 j + 8 g .. +8; head weights of the rows it gets back
  bf16x8 qf[KS];
  float wt[4];
  {
    const int nh = active ? min(16, a.H - h0) : 0;
    const __amdgpu_buffer_rsrc_t qr =
        rsrc(a.q + ((size_t)b * a.H + (active ? h0 : 0)) * DI, (uint32_t)nh * DI * 2);
#pragma unroll
    for (int j = 0; j < KS; ++j)
      qf[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                             qr, (uint32_t)(n * DI * 2 + 64 * j + 16 * g), 0, 0));
    const __amdgpu_buffer_rsrc_t wr = rsrc(a.w + (size_t)b * a.H + (active ? h0 : 0),
                                           (uint32_t)nh * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wt[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            wr, (uint32_t)(4 * (4 * g + i)), 0, 0));
  }
  const __amdgpu_buffer_rsrc_t kr =
      rsrc((const unsigned char*)a.keys + (size_t)b * a.N * KRB, (uint32_t)a.N * KRB);

  for (int t0 = blockIdx.x * kLTile; t0 < count; t0 += gridDim.x * kLTile) {
    const int nt = min(kLTile, count - t0);
    __syncthreads();   // the previous tile's rows and partial sums are consumed
    if ((int)threadIdx.x < kLTile) {
      const int s = (int)threadIdx.x < nt ? a.surv_idx[(size_t)b * a.cap + t0 + threadIdx.x] : -1;
      s_idx[threadIdx.x] = s;
    }
    __syncthreads();
    // gather the tile's key rows (16 B a thread), widened to bf16 in LDS;
    // rows past the tile or with an index outside [0, N) read as zero
    for (int r0 = 0; r0 < kLTile; r0 += 256 / TPR) {
      const int r = r0 + (int)threadIdx.x / TPR, part16 = (int)threadIdx.x % TPR;
      const int s = s_idx[r];
      const uint32_t off = (s >= 0 && s < a.N) ? (uint32_t)s * KRB + 16u * part16 : 0xFFFFFF00u;
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
      if constexpr (KT == 1) {
        *(bf16x8*)(rows + r * RS + 32 * part16) = e4m3x8_to_bf16x8(u32x2{v[0], v[1]});
        *(bf16x8*)(rows + r * RS + 32 * part16 + 16) = e4m3x8_to_bf16x8(u32x2{v[2], v[3]});
      } else {
        *(u32x4*)(rows + r * RS + 16 * part16) = v;
      }
    }
    __syncthreads();
    if (active) {
      // 16 survivors at a time: C[head 4g + i][survivor n]
      for (int c = 0; c < kLTile / 16; ++c) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        const unsigned char* base = rows + (16 * c + n) * RS + 16 * g;
#pragma unroll
        for (int j = 0; j < KS; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[j], *(const bf16x8*)(base + 64 * j),
                                                        acc, 0, 0, 0);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) sum = fmaf(wt[i], fmaxf(acc[i], 0.f), sum);
        sum += __shfl_xor(sum, 16, kWave);
        sum += __shfl_xor(sum, 32, kWave);
        if (g == 0) part[wave][16 * c + n] = sum;
      }
    } else {
      for (int c = lane; c < kLTile; c += 64) part[wave][c] = 0.f;
    }
    __syncthreads();
    if ((int)threadIdx.x < nt) {
      const int i = threadIdx.x;
      const int s = s_idx[i];
      float v = ((part[0][i] + part[1][i]) + part[2][i]) + part[3][i];
      if constexpr (KT == 1) {
        const float sc = (s >= 0 && s < a.N) ? a.scale[(size_t)b * a.N + s] : 1.f;
        v *= sc;
      }
      a.score[(size_t)b * a.cap + t0 + i] = (s >= 0 && s < a.N) ? v : -__builtin_inff();
    }
  }
}

}  // namespace

hipError_t launch_lightning(int B, int N, int cap, int H, int dI, lsa_key_dtype kdt,
                            const void* keys, const float* scale, const uint16_t* q,
                            const float* w, const int32_t* surv_idx, const int32_t* surv_count,
                            float* score, hipStream_t s) {
  LightArgs a{keys, scale, q, w, surv_idx, surv_count, score, N, cap, H};
  const int tiles = (cap + kLTile - 1) / kLTile;
  if (tiles == 0) return hipSuccess;
  // about four blocks per compute unit over the whole batch; each block walks
  // every gx-th tile of its request
  const int gx = std::max(1, std::min(tiles, (4 * device_cu_count() + B - 1) / B));
  const dim3 grid(gx, B);
  if (kdt == LSA_KEY_FP8_E4M3) {
    if (dI == 64) hipLaunchKernelGGL((lightning_kernel<1, 64>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((lightning_kernel<1, 128>), grid, dim3(256), 0, s, a);
  } else {
    if (dI == 64) hipLaunchKernelGGL((lightning_kernel<0, 64>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((lightning_kernel<0, 128>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace lsa
