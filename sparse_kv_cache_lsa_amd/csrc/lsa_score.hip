// lsa_score.hip -- lookahead index score + threshold for gfx950.
//
// Computes, per (layer l, request b, entry s),
//   z = sum_h g_h (q_h . k_s) * sigma_s + bias_l,   sel = (z >= 0)
// (the sigmoid, head-fused, gated match of the gist.science technical
// summary, section 2.1 "scoring mechanism", with I >= 0.5 written as z >= 0
// as in its "dynamic fetch" bullet).
//
// Design (memory-bound key stream, MFMA for the dense H x dI x entries part):
//  * grid.y = (layer, request) pair, grid.x = chunk of 32-entry tiles; each of
//    the 4 wavefronts of a block walks every 4th tile of the chunk, so the
//    block streams one contiguous key range.
//  * A tile (32 entries x dI) is read with fully coalesced 16-byte loads
//    (each load instruction covers 1 KiB of contiguous keys), prefetched one
//    tile ahead in registers, then staged in the wave's private LDS slice
//    with the 16-byte chunks of each entry row XOR-swizzled by the entry
//    index so that the MFMA-layout reads spread over LDS banks.
//  * The contraction runs on v_mfma_f32_32x32x16_bf16 with the query as the
//    A operand (32 heads x 16 dims, kept in registers for the whole block) and
//    the keys as the B operand (16 dims x 32 entries).  e4m3 keys are widened
//    to bf16 exactly in registers (every e4m3 value is a bf16 value); the
//    per-entry fp32 scale is applied in the epilogue.  The key dimension is
//    permuted identically in A and B (lane half 0 takes dims [0, dI/2), half 1
//    takes [dI/2, dI)), which leaves every dot product unchanged.
//  * Epilogue in registers: gate-weighted head sum over the 16 accumulator
//    rows a lane holds, one cross-half swap, scale, bias, optional sigmoid,
//    threshold by wavefront ballot -> one 32-bit selection word per tile.
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

template <int KT, int DI>
struct Geo {
  static constexpr int ESZ = KT == 0 ? 2 : 1;   // bytes per key element
  static constexpr int RB = DI * ESZ;           // bytes per entry row
  static constexpr int TB = 32 * RB;            // bytes per 32-entry tile
  static constexpr int LOADS = TB / 1024;       // 16-byte loads per lane per tile
  static constexpr int NCH = RB / 16;           // 16-byte chunks per row
  static constexpr int KSTEPS = DI / 16;        // MFMA steps (K = 16)
  static constexpr int HALF = DI / 2;           // key dims per lane half
};

template <int KT, int DI>
__device__ __forceinline__ void load_tile(const unsigned char* kb, long long nbytes,
                                          int t, int lane,
                                          u32x4 (&r)[Geo<KT, DI>::LOADS]) {
  using G = Geo<KT, DI>;
  const long long base = (long long)t * G::TB + 16 * lane;
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) {
    const long long off = base + 1024 * j;
    if (off < nbytes)
      r[j] = __builtin_nontemporal_load((const u32x4*)(kb + off));
    else
      r[j] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int KT, int DI, int HT>
__device__ __forceinline__ void score_tile(
    const u32x4 (&r)[Geo<KT, DI>::LOADS], unsigned char* lds, int t, int lane,
    const bf16x8 (&af)[HT][Geo<KT, DI>::KSTEPS], const float (&gl)[HT][16],
    const float* sb, float bias, int N, float* zr, float* Ir, uint32_t* mr) {
  using G = Geo<KT, DI>;
  const int n = lane & 31;
  const int half = lane >> 5;
  const int s_idx = t * 32 + n;
  const bool valid = s_idx < N;
  float sc = 1.f;
  if constexpr (KT == 1) sc = valid ? sb[s_idx] : 0.f;

  // stage: coalesced chunk o of the tile -> row e, swizzled chunk position
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) {
    const int o = 1024 * j + 16 * lane;
    const int e = o / G::RB;
    const int c = (o % G::RB) >> 4;
    *(u32x4*)(lds + e * G::RB + ((c ^ (e & (G::NCH - 1))) << 4)) = r[j];
  }
  wave_lds_sync();

  f32x16 acc[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x16{};
#pragma unroll
  for (int s = 0; s < G::KSTEPS; ++s) {
    const int byte0 = (half * G::HALF + 8 * s) * G::ESZ;
    const int c = byte0 >> 4;
    const unsigned char* src = lds + n * G::RB + ((c ^ (n & (G::NCH - 1))) << 4) + (byte0 & 15);
    bf16x8 bfrag;
    if constexpr (KT == 0) {
      bfrag = __builtin_bit_cast(bf16x8, *(const u32x4*)src);
    } else {
      bfrag = e4m3x8_to_bf16x8(*(const u32x2*)src);
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
      acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ht][s], bfrag, acc[ht], 0, 0, 0);
  }
  wave_lds_sync();

  // accumulator register r of lane l holds head row (r&3) + 4*(l/32) + 8*(r/4)
  // of entry column l%32
  float part = 0.f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) part = fmaf(gl[ht][rr], acc[ht][rr], part);
  part = add_halves(part);
  const float zv = fmaf(part, sc, bias);
  const bool sel = valid && (zv >= 0.f);
  const uint64_t bal = __ballot(sel);
  if (half == 0 && valid) {
    zr[s_idx] = zv;
    if (Ir) Ir[s_idx] = 1.f / (1.f + __expf(-zv));
  }
  if (lane == 0) mr[t] = (uint32_t)bal;
}

template <int KT, int DI, int HT>
__global__ __launch_bounds__(256, 2) void score_kernel(ScoreArgs a) {
  using G = Geo<KT, DI>;
  __shared__ __attribute__((aligned(16))) unsigned char lds_all[4][G::TB];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int half = lane >> 5;
  unsigned char* lds = lds_all[wave];

  const int p = blockIdx.y;        // (layer, request) pair, layer-major
  const int l = p / a.B;
  const int b = p - l * a.B;

  // A operand: query rows of this pair, one head per lane row
  const uint16_t* qp = a.q + (size_t)p * a.H * DI;
  bf16x8 af[HT][G::KSTEPS];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = ht * 32 + n;
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (head < a.H) v = *(const u32x4*)(qp + head * DI + half * G::HALF + 8 * s);
      af[ht][s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float gl[HT][16];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int head = ht * 32 + (rr & 3) + 4 * half + 8 * (rr >> 2);
      gl[ht][rr] = head < a.H ? a.g[(size_t)p * a.H + head] : 0.f;
    }

  const unsigned char* kb = (const unsigned char*)a.keys[l] + (size_t)b * a.N * G::RB;
  const float* sb = KT == 1 ? a.scale[l] + (size_t)b * a.N : nullptr;
  const float bias = a.bias[l];
  float* zr = a.z + (size_t)p * a.N;
  float* Ir = a.I ? a.I + (size_t)p * a.N : nullptr;
  uint32_t* mr = a.mask + (size_t)p * a.W;
  const long long nbytes = (long long)a.N * G::RB;

  const int ntiles = (a.N + 31) >> 5;
  int t = blockIdx.x * a.tiles_per_block + wave;
  const int t_end = min(ntiles, (blockIdx.x + 1) * a.tiles_per_block);

  u32x4 ra[G::LOADS], rb[G::LOADS];
  if (t < t_end) load_tile<KT, DI>(kb, nbytes, t, lane, ra);
  while (t < t_end) {
    if (t + 4 < t_end) load_tile<KT, DI>(kb, nbytes, t + 4, lane, rb);
    score_tile<KT, DI, HT>(ra, lds, t, lane, af, gl, sb, bias, a.N, zr, Ir, mr);
    t += 4;
    if (t >= t_end) break;
    if (t + 4 < t_end) load_tile<KT, DI>(kb, nbytes, t + 4, lane, ra);
    score_tile<KT, DI, HT>(rb, lds, t, lane, af, gl, sb, bias, a.N, zr, Ir, mr);
    t += 4;
  }
}

template <int KT, int DI, int HT>
hipError_t launch_t(int L, const ScoreArgs& a, hipStream_t s) {
  const int ntiles = (a.N + 31) / 32;
  dim3 grid((ntiles + a.tiles_per_block - 1) / a.tiles_per_block, L * a.B);
  hipLaunchKernelGGL((score_kernel<KT, DI, HT>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(int L, int dI, lsa_key_dtype kdt, const ScoreArgs& a,
                        hipStream_t s) {
  const bool two = a.H > 32;
  if (kdt == LSA_KEY_BF16) {
    if (dI == 64) return two ? launch_t<0, 64, 2>(L, a, s) : launch_t<0, 64, 1>(L, a, s);
    return two ? launch_t<0, 128, 2>(L, a, s) : launch_t<0, 128, 1>(L, a, s);
  }
  if (dI == 64) return two ? launch_t<1, 64, 2>(L, a, s) : launch_t<1, 64, 1>(L, a, s);
  return two ? launch_t<1, 128, 2>(L, a, s) : launch_t<1, 128, 1>(L, a, s);
}

}  // namespace lsa
