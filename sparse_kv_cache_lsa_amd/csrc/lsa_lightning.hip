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
// widened exactly to bf16), A = the query heads (four 16-head tiles, zero
// past H), B = the survivors' keys.  Every wavefront works alone (no LDS, no
// barriers): it takes groups of 32 survivors of one request (two 16-column
// steps), loads their key rows straight into registers -- lane (n, g) reads
// the contiguous quarter g of survivor n's row, so the four lanes of a
// survivor read its whole row -- and runs the contraction over dims in the
// order (quarter, 8-dim step); the query fragments use the same order, so
// the dot products are the same sums.  The key loads are cached: the two
// 16-byte loads of a lane's quarter fall in the same 128-byte line, so a
// nontemporal hint would fetch each e4m3 row twice (64.8 against 78 us for
// 2.0 M survivors at 1M context).  The next group's rows and the index
// list of the group after it are in flight while a group is multiplied.  The
// epilogue applies relu and the head weights to each lane's 4 x 4 products,
// and two shuffles add the four lane groups: one score per survivor.
#include "lsa_device.h"
#include "lsa_launch.h"

#include <algorithm>

namespace lsa {
namespace {

constexpr int kLC = 2;        // 16-survivor column steps per group
constexpr int kLGroup = 16 * kLC;

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

// One lane's quarter of a key row (dI / 4 dims) for each column step.
template <int KT, int DI>
struct KeyQuarter {
  static constexpr int kBytes = (KT == 1 ? 1 : 2) * DI / 4;   // 16, 32 or 64
  u32x4 v[kLC][kBytes / 16];
};

// KT 0: bf16 keys, 1: e4m3 keys + scale.  DI: 64 or 128.
template <int KT, int DI>
__global__ __launch_bounds__(256) void lightning_kernel(LightArgs a) {
  constexpr int KRB = KT == 1 ? DI : 2 * DI;   // key row bytes in memory
  constexpr int QB = KRB / 4;                  // bytes of a row quarter
  constexpr int KS = DI / 32;                  // 8-dim steps per quarter (the MFMA k-steps)
  constexpr int NQ = QB / 16;                  // 16-byte loads per quarter
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  const int count = min(max(a.surv_count[b], 0), a.cap);
  const int ngroups = (count + kLGroup - 1) / kLGroup;
  const int wv = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int stride = gridDim.x * 4;
  if (wv >= ngroups) return;

  // query fragments (A operand) of heads 16 t + n, dims g * dI/4 + 8 j .. +8,
  // and the head weights of the C rows this lane gets back (16 t + 4 g + i);
  // heads past H read as zero
  bf16x8 qf[4][KS];
  float wt[4][4];
  {
    const __amdgpu_buffer_rsrc_t qr = rsrc(a.q + (size_t)b * a.H * DI, (uint32_t)a.H * DI * 2);
    const __amdgpu_buffer_rsrc_t wr = rsrc(a.w + (size_t)b * a.H, (uint32_t)a.H * 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int j = 0; j < KS; ++j)
        qf[t][j] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                        qr, (uint32_t)(((16 * t + n) * DI + g * (DI / 4) + 8 * j) * 2), 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wt[t][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 wr, (uint32_t)(4 * (16 * t + 4 * g + i)), 0, 0));
    }
  }
  const __amdgpu_buffer_rsrc_t kr =
      rsrc((const unsigned char*)a.keys + (size_t)b * a.N * KRB, (uint32_t)a.N * KRB);
  const __amdgpu_buffer_rsrc_t ir =
      rsrc(a.surv_idx + (size_t)b * a.cap, (uint32_t)count * 4);
  const __amdgpu_buffer_rsrc_t sr =
      rsrc(KT == 1 ? (const void*)(a.scale + (size_t)b * a.N) : (const void*)a.w,
           KT == 1 ? (uint32_t)a.N * 4 : 0u);

  // survivor index of column step c of group gi (-1 past the list; the range
  // check returns 0 there, so the position test decides)
  auto load_idx = [&](int gi, int (&s)[kLC]) {
#pragma unroll
    for (int c = 0; c < kLC; ++c) {
      const int pos = gi * kLGroup + 16 * c + n;
      const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, (uint32_t)pos * 4, 0, 0);
      s[c] = pos < count ? v : -1;
    }
  };
  auto load_rows = [&](const int (&s)[kLC], KeyQuarter<KT, DI>& r, float (&sc)[kLC]) {
#pragma unroll
    for (int c = 0; c < kLC; ++c) {
      const bool ok = s[c] >= 0 && s[c] < a.N;
      const uint32_t off = ok ? (uint32_t)s[c] * KRB + (uint32_t)g * QB : 0xFFFFFF00u;
#pragma unroll
      for (int v = 0; v < NQ; ++v)
        r.v[c][v] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off + 16u * v, 0, 0));
      sc[c] = 1.f;
      if constexpr (KT == 1)
        sc[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              sr, ok ? (uint32_t)s[c] * 4 : 0xFFFFFF00u, 0, 0));
    }
  };

  int gi = wv;
  int s_cur[kLC], s_nxt[kLC];
  KeyQuarter<KT, DI> r_cur;
  float sc_cur[kLC];
  load_idx(gi, s_cur);
  load_rows(s_cur, r_cur, sc_cur);
  load_idx(gi + stride, s_nxt);
  for (; gi < ngroups; gi += stride) {
    // the next group's rows and the indices of the group after it
    KeyQuarter<KT, DI> r_nxt;
    float sc_nxt[kLC];
    int s_nn[kLC];
    load_rows(s_nxt, r_nxt, sc_nxt);
    load_idx(gi + 2 * stride, s_nn);
#pragma unroll
    for (int c = 0; c < kLC; ++c) {
      f32x4 acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        bf16x8 kb;
        if constexpr (KT == 1) {
          const u32x4 w4 = r_cur.v[c][j / 2];
          kb = e4m3x8_to_bf16x8((j & 1) ? u32x2{w4[2], w4[3]} : u32x2{w4[0], w4[1]});
        } else {
          kb = __builtin_bit_cast(bf16x8, r_cur.v[c][j]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[t][j], kb, acc[t], 0, 0, 0);
      }
      // C[head 16 t + 4 g + i][survivor n]
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum = fmaf(wt[t][i], fmaxf(acc[t][i], 0.f), sum);
      sum += __shfl_xor(sum, 16, kWave);
      sum += __shfl_xor(sum, 32, kWave);
      const int pos = gi * kLGroup + 16 * c + n;
      if (g == 0 && pos < count) {
        const bool ok = s_cur[c] >= 0 && s_cur[c] < a.N;
        a.score[(size_t)b * a.cap + pos] = ok ? sum * sc_cur[c] : -__builtin_inff();
      }
    }
    r_cur = r_nxt;
#pragma unroll
    for (int c = 0; c < kLC; ++c) {
      sc_cur[c] = sc_nxt[c];
      s_cur[c] = s_nxt[c];
      s_nxt[c] = s_nn[c];
    }
  }
}

}  // namespace

hipError_t launch_lightning(int B, int N, int cap, int H, int dI, lsa_key_dtype kdt,
                            const void* keys, const float* scale, const uint16_t* q,
                            const float* w, const int32_t* surv_idx, const int32_t* surv_count,
                            float* score, hipStream_t s) {
  LightArgs a{keys, scale, q, w, surv_idx, surv_count, score, N, cap, H};
  const int groups = (cap + kLGroup - 1) / kLGroup;
  if (groups == 0) return hipSuccess;
  // about twelve wavefronts per compute unit over the whole batch; each
  // wavefront walks every (4 * gx)-th group of its request
  const int gx = std::max(1, std::min((groups + 3) / 4, (3 * device_cu_count() + B - 1) / B));
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
