// lsa_score.hip -- lookahead index score + threshold for gfx950.
//
// Computes, per (layer l, request b, entry s),
//   z = sum_h g_h (q_h . k_s) * sigma_s + bias_l,   sel = (z >= 0)
// (the sigmoid, head-fused, gated match of the gist.science technical
// summary, section 2.1 "scoring mechanism", with I >= 0.5 written as z >= 0
// as in its "dynamic fetch" bullet).
//
// Design (memory-bound key stream, MFMA for the dense H x dI x entries part):
//  * grid.y = (layer, request) pair, grid.x = chunk of 32-entry tiles; the NW
//    wavefronts of a block take every NW-th tile of the chunk, so a block
//    streams one contiguous key range (the pattern HBM serves best).
//  * Keys are read through a buffer resource per (layer, request): each load
//    instruction covers 1 KiB of contiguous keys (16 B per lane, nontemporal),
//    the lane offset is a 32-bit VGPR, and the hardware range check returns 0
//    past the end of the request's keys -- no address or bounds arithmetic in
//    the loop.  Stores use the same mechanism: a lane with nothing to store
//    gets an out-of-range offset and the store is dropped.
//  * A register ring keeps RING-1 tiles in flight while one is scored.
//  * A tile (32 entries x dI) is staged in the wave's private LDS slice with
//    the 16-byte chunks of each entry row XOR-swizzled by the entry index, so
//    the MFMA-layout reads spread over LDS banks.
//  * The contraction runs on v_mfma_f32_32x32x16_bf16: query as A (32 heads x
//    16 dims, in registers for the whole block), keys as B (16 dims x 32
//    entries).  e4m3 keys are widened to bf16 exactly in registers (every e4m3
//    value is a bf16 value); the per-entry fp32 scale is applied in the
//    epilogue.  The key dimension is permuted identically in A and B (lane
//    half 0 takes dims [0, dI/2), half 1 takes [dI/2, dI)), which leaves every
//    dot product unchanged.
//  * Epilogue in registers: gate-weighted head sum over the 16 accumulator
//    rows a lane holds, one cross-half sum, scale, bias, optional sigmoid,
//    threshold by wavefront ballot -> one 32-bit selection word per tile.
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr uint32_t kOOB = 0xFFFFFF00u;   // a buffer offset past any range used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

constexpr int kNT = 2;   // cache policy: nontemporal (streamed once)

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

// One tile in flight: its key bytes (LOADS x 16 B per lane) and, for e4m3
// keys, the scale of the entry this lane's column scores.
template <int KT, int DI>
struct TileRegs {
  u32x4 k[Geo<KT, DI>::LOADS];
  float sc;
};

template <int KT, int DI>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t sr,
                                          int t, int lane, TileRegs<KT, DI>& r) {
  using G = Geo<KT, DI>;
  const uint32_t off = (uint32_t)t * G::TB + 16u * lane;
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j)
    r.k[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off + 1024 * j, 0, kNT));
  if constexpr (KT == 1)
    r.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         sr, ((uint32_t)t * 32 + (lane & 31)) * 4, 0, kNT));
  else
    r.sc = 1.f;
}

// Scores one staged tile: returns z of entry column (lane & 31) in every lane
// (both lane halves hold the same value).
template <int KT, int DI, int HT>
__device__ __forceinline__ float score_tile(const TileRegs<KT, DI>& r, unsigned char* lds,
                                            int lane, const bf16x8 (&af)[HT][Geo<KT, DI>::KSTEPS],
                                            const float* gs, float bias) {
  using G = Geo<KT, DI>;
  const int n = lane & 31;
  const int half = lane >> 5;

  // stage: coalesced chunk o of the tile -> row e, swizzled chunk position
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) {
    const int o = 1024 * j + 16 * lane;
    const int e = o / G::RB;
    const int c = (o % G::RB) >> 4;
    *(u32x4*)(lds + e * G::RB + ((c ^ (e & (G::NCH - 1))) << 4)) = r.k[j];
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
  // of entry column l%32; the gates come from the block's LDS copy (every
  // lane of a half reads the same address: a broadcast)
  float part = 0.f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      part = fmaf(gs[ht * 32 + (rr & 3) + 4 * half + 8 * (rr >> 2)], acc[ht][rr], part);
  part = add_halves(part);
  return fmaf(part, r.sc, bias);
}

// One block = one request b and one chunk of kChunkTiles 32-entry tiles
// (LSA_CAND_CHUNK entries), for every indexer layer in turn (outer loop).
// Wave w scores chunk tiles w, w + NW, ...  Per tile and layer the selection
// word goes to LDS; per entry the maximum z over the layers that select it
// stays in the wave's LDS slice across layers (-inf while none has).  After the
// last layer the whole block
//   * writes its selection words, one contiguous run per layer, and
//   * compacts the chunk: every entry with a finite merged logit, in
//     ascending order (ballot + mbcnt inside a wave, a 4-wave prefix in LDS),
//     into the chunk's candidate list (entry index, merged logit) plus count.
// So the kernel writes a few contiguous runs per block instead of one line per
// tile; writes interleaved with the key stream cost far more HBM time than
// their bytes.  RING: register-ring depth (RING-1 tiles in flight per wave).
constexpr int kNW = 4;
constexpr int kTPW = LSA_CAND_CHUNK / 32 / kNW;    // tiles per wave and layer
static_assert(kTPW * 32 * kNW == LSA_CAND_CHUNK, "chunk must split evenly");

template <int KT, int DI, int HT, int RING, bool WZ, bool WI, int WPE>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(WPE)))
void score_kernel(ScoreArgs a) {
  using G = Geo<KT, DI>;
  constexpr int NW = kNW;
  __shared__ __attribute__((aligned(16))) unsigned char lds_all[NW][G::TB];
  __shared__ __attribute__((aligned(16))) float gs[LSA_MAX_LAYERS][64];
  __shared__ __attribute__((aligned(16))) float zacc[NW][kTPW][32];
  __shared__ uint32_t mwords[LSA_MAX_LAYERS][NW * kTPW];
  __shared__ int s_wave[NW];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int half = lane >> 5;
  unsigned char* lds = lds_all[wave];
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  const int L = a.L;

  for (int i = threadIdx.x; i < L * 64; i += 64 * NW) {
    const int l = i >> 6, h = i & 63;
    gs[l][h] = h < a.H ? a.g[((size_t)l * a.B + b) * a.H + h] : 0.f;
  }
  __syncthreads();

  const uint32_t N = (uint32_t)a.N;
  const int ntiles = (a.N + 31) >> 5;
  const int c_tile0 = c * NW * kTPW;                       // first tile of the chunk
  const int c_tiles = min(NW * kTPW, ntiles - c_tile0);    // tiles in this chunk
  const int n_my = wave < c_tiles ? (c_tiles - wave + NW - 1) / NW : 0;
  const int t0 = c_tile0 + wave;
  const int t_last = t0 + NW * (n_my - 1);

  for (int l = 0; l < L && n_my > 0; ++l) {
    const int p = l * a.B + b;
    // A operand: query rows of (layer l, request b), one head per lane row
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
    const __amdgpu_buffer_rsrc_t kr =
        buffer((const unsigned char*)a.keys[l] + (size_t)b * N * G::RB, N * G::RB);
    const __amdgpu_buffer_rsrc_t sr =
        buffer(KT == 1 ? (const void*)(a.scale[l] + (size_t)b * N) : a.keys[l], KT == 1 ? N * 4 : 0);
    const __amdgpu_buffer_rsrc_t zr = buffer(WZ ? a.z + (size_t)p * N : a.keys[l], WZ ? N * 4 : 0);
    const __amdgpu_buffer_rsrc_t ir = buffer(WI ? a.I + (size_t)p * N : a.keys[l], WI ? N * 4 : 0);
    const float bias = a.bias[l];
    const bool first = l == 0;

    // Register ring: slot indices are compile-time constants.  Prefetches past
    // the wave's last tile re-read that tile (an L2 hit), and ring slots scored
    // past the end store nothing, so the loop body has no branches.
    TileRegs<KT, DI> ring[RING];
#pragma unroll
    for (int r = 0; r < RING - 1; ++r)
      load_tile<KT, DI>(kr, sr, min(t0 + NW * r, t_last), lane, ring[r]);
    for (int i = 0; i < n_my; i += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        const int ii = i + r;
        const int t = min(t0 + NW * ii, t_last);
        load_tile<KT, DI>(kr, sr, min(t0 + NW * (ii + RING - 1), t_last), lane,
                          ring[(r + RING - 1) % RING]);
        const float zv = score_tile<KT, DI, HT>(ring[r], lds, lane, af, gs[l], bias);
        const bool live = ii < n_my;
        const int s_idx = t * 32 + n;
        const bool sel = live && s_idx < a.N && zv >= 0.f;
        const uint64_t bal = __ballot(sel);
        if (lane == 0 && live) mwords[l][t - c_tile0] = (uint32_t)bal;
        if constexpr (WZ || WI) {
          const uint32_t zoff = (half == 0 && live) ? (uint32_t)s_idx * 4 : kOOB;
          if constexpr (WZ)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, zv), zr, zoff, 0, 0);
          if constexpr (WI) {
            const float iv = __builtin_amdgcn_rcpf(1.f + __expf(-zv));
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, iv), ir, zoff, 0, 0);
          }
        }
        // running maximum over the selecting layers (-inf: none selects yet)
        float* slot = &zacc[wave][ii < kTPW ? ii : kTPW - 1][n];
        float zm = sel ? zv : -__builtin_inff();
        if (!first) zm = fmaxf(zm, *slot);
        if (half == 0 && live) *slot = zm;
      }
    }
  }
  __syncthreads();

  // selection words: one contiguous run per layer
  for (int i = threadIdx.x; i < L * c_tiles; i += 64 * NW) {
    const int l = i / c_tiles, tc = i - l * c_tiles;
    a.mask[((size_t)l * a.B + b) * a.W + c_tile0 + tc] = mwords[l][tc];
  }
  // chunk compaction, ascending: thread j of round r takes chunk entry
  // e = 256 r + j, held by wave (e/32) % NW at local tile (e/32) / NW
  int* cidx = a.cand_idx + ((size_t)b * a.nchunks + c) * LSA_CAND_CHUNK;
  float* cz = a.cand_z + ((size_t)b * a.nchunks + c) * LSA_CAND_CHUNK;
  int base = 0;
  const int c_entries = min(LSA_CAND_CHUNK, a.N - c_tile0 * 32);
  for (int e0 = 0; e0 < c_entries; e0 += 64 * NW) {
    const int e = e0 + threadIdx.x;
    const int tc = e >> 5;
    float zm = -__builtin_inff();
    if (e < c_entries) zm = zacc[tc % NW][tc / NW][e & 31];
    const bool f = zm > -__builtin_inff();
    const uint64_t bal = __ballot(f);
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int cnt = s_wave[w];
      before += (w < wave) ? cnt : 0;
      total += cnt;
    }
    if (f) {
      const int pos = base + before + lanes_below(bal);
      cidx[pos] = c_tile0 * 32 + e;
      cz[pos] = zm;
    }
    base += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.cand_count[(size_t)b * a.nchunks + c] = base;
}

template <int KT, int DI, int HT, int RING = 2, int WPE = 2>
hipError_t launch_t(const ScoreArgs& a, hipStream_t s) {
  dim3 grid(a.nchunks, a.B);
  const bool wz = a.z != nullptr, wi = a.I != nullptr;
  if (!wz && !wi)
    hipLaunchKernelGGL((score_kernel<KT, DI, HT, RING, false, false, WPE>), grid, dim3(64 * kNW), 0, s, a);
  else if (wz && !wi)
    hipLaunchKernelGGL((score_kernel<KT, DI, HT, RING, true, false, WPE>), grid, dim3(64 * kNW), 0, s, a);
  else if (!wz && wi)
    hipLaunchKernelGGL((score_kernel<KT, DI, HT, RING, false, true, WPE>), grid, dim3(64 * kNW), 0, s, a);
  else
    hipLaunchKernelGGL((score_kernel<KT, DI, HT, RING, true, true, WPE>), grid, dim3(64 * kNW), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(int dI, lsa_key_dtype kdt, const ScoreArgs& a, hipStream_t s) {
  const bool two = a.H > 32;
  if (kdt == LSA_KEY_BF16) {
    if (dI == 64) return two ? launch_t<0, 64, 2>(a, s) : launch_t<0, 64, 1>(a, s);
    return two ? launch_t<0, 128, 2>(a, s) : launch_t<0, 128, 1>(a, s);
  }
  if (dI == 64) return two ? launch_t<1, 64, 2>(a, s) : launch_t<1, 64, 1>(a, s);
  return two ? launch_t<1, 128, 2>(a, s) : launch_t<1, 128, 1>(a, s);
}

}  // namespace lsa
