// lsa_score.hip -- lookahead index score + threshold for gfx950.
//
// Computes, per (layer l, request b, entry s),
//   z = sum_h g_h (q_h . k_s) * sigma_s + bias_l,   sel = (z >= 0)
// (the sigmoid, head-fused, gated match of the gist.science technical
// summary, section 2.1 "scoring mechanism", with I >= 0.5 written as z >= 0
// as in its "dynamic fetch" bullet).
//
// Design (memory-bound key stream):
//  * The head sum is linear in the keys: sum_h g_h (q_h . k) = qt . k with
//    qt = sum_h g_h q_h.  Each block forms qt (fp32) for its request and
//    every layer once, from the bf16 queries and fp32 gates, so scoring an
//    entry is one dI-long dot product, not H of them.
//  * A block takes one request and one or two consecutive chunks of
//    LSA_CAND_CHUNK entries (see score_kernel for the grid); the NW
//    wavefronts of a block take every NW-th 32-entry tile of its range, so a
//    block streams one contiguous key range (the pattern HBM serves best).
//  * Keys are read through a buffer resource per (layer, request): each load
//    instruction covers 1 KiB of contiguous keys (16 B per lane, nontemporal),
//    the lane offset is a 32-bit VGPR, and the hardware range check returns 0
//    past the end of the request's keys -- no address or bounds arithmetic in
//    the loop.  Stores use the same mechanism: a lane with nothing to store
//    gets an out-of-range offset and the store is dropped.
//  * A register ring keeps RING-1 tiles in flight while one is scored.
//  * The tile stays in the registers it was loaded into: lane l holds 16
//    bytes of one entry row (16 e4m3 or 8 bf16 key elements, widened exactly
//    to fp32), multiplies them by its slice of qt, and the lanes sharing a row
//    add their partial sums with DPP; one lane-to-lane gather then gives lane
//    n the score of entry n (the layout the epilogue uses).
//  * Epilogue in registers: per-entry fp32 scale, bias, optional sigmoid,
//    threshold by wavefront ballot -> one 32-bit selection word per tile.
#include "lsa_device.h"
#include "lsa_launch.h"

#include <algorithm>

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
  static constexpr int LPR = RB / 16;           // lanes holding one entry row (per load)
  static constexpr int EPC = 16 / ESZ;          // key elements per lane and load
  static constexpr int EPL = 64 / LPR;          // entry rows per load
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

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// One halving step of the row reduction: lanes whose bit (the one the DPP
// partner differs in) is clear keep values [0, C/2) and hand over [C/2, C);
// lanes with it set keep the upper half.  Each kept value adds the partner's.
template <int C, int CTRL, int N>
__device__ __forceinline__ void halve(float (&v)[N], bool upper) {
#pragma unroll
  for (int i = 0; i < C / 2; ++i) {
    const float keep = upper ? v[C / 2 + i] : v[i];
    const float give = upper ? v[i] : v[C / 2 + i];
    v[i] = keep + dpp<CTRL>(give);
  }
}

// v[j] (j < NL) is a lane's partial dot product for the entry row it holds in
// load j; the LPR = 2 NL lanes of an aligned group hold the same rows.
// Halving steps over the lane bits (partners: row_mirror for bit 3,
// row_half_mirror for bit 2, quad_perm ^2 for bit 1) leave lane li of the
// group with row (li >> 1)'s sum over half of the group; quad_perm ^1 adds
// the other half.  Result: lanes 2j and 2j + 1 of a group hold the full dot
// product of load j's row (same bits in both).
template <int LPR, int NL>
__device__ __forceinline__ float reduce_rows(float (&v)[NL], int lane) {
  static_assert(2 * NL == LPR && (NL == 2 || NL == 4 || NL == 8), "row geometry");
  const int li = lane & (LPR - 1);
  if constexpr (NL == 8) halve<8, 0x140>(v, li & 8);   // row_mirror: i <-> 15 - i
  if constexpr (NL >= 4) halve<4, 0x141>(v, li & 4);   // row_half_mirror: i <-> 7 - i
  halve<2, 0x4E>(v, li & 2);                           // quad_perm [2,3,0,1]: lane ^ 2
  return v[0] + dpp<0xB1>(v[0]);                       // quad_perm [1,0,3,2]: lane ^ 1
}

// Partial dot product of one 16-byte key chunk with the lane's qt slice.
template <int KT>
__device__ __forceinline__ float chunk_dot(u32x4 k, const float* qv) {
  float acc0 = 0.f, acc1 = 0.f;
  if constexpr (KT == 1) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(k[w], 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(k[w], 1.0f, true);
      acc0 = fmaf(lo[0], qv[4 * w], acc0);
      acc1 = fmaf(lo[1], qv[4 * w + 1], acc1);
      acc0 = fmaf(hi[0], qv[4 * w + 2], acc0);
      acc1 = fmaf(hi[1], qv[4 * w + 3], acc1);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc0 = fmaf(__uint_as_float(k[w] << 16), qv[2 * w], acc0);
      acc1 = fmaf(__uint_as_float(k[w] & 0xFFFF0000u), qv[2 * w + 1], acc1);
    }
  }
  return acc0 + acc1;
}

// Scores one tile held in registers: returns z of entry (lane & 31) in every
// lane (both lane halves hold the same value).  qv: the lane's EPC elements
// of qt, dims [EPC * (lane % LPR), EPC * (lane % LPR + 1)).
template <int KT, int DI>
__device__ __forceinline__ float score_tile(const TileRegs<KT, DI>& r, int lane, const float* qv,
                                            float bias) {
  using G = Geo<KT, DI>;
  const int n = lane & 31;
  float d[G::LOADS];
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) d[j] = chunk_dot<KT>(r.k[j], qv);
  const float sum = reduce_rows<G::LPR, G::LOADS>(d, lane);
  // entry n = load (n / EPL), row group (n % EPL): held by lane LPR (n % EPL) + 2 (n / EPL)
  const float zv = __shfl(sum, G::LPR * (n % G::EPL) + 2 * (n / G::EPL), kWave);
  return fmaf(zv, r.sc, bias);
}

// One block = one request b and CPB consecutive chunks of LSA_CAND_CHUNK
// entries (32-entry tiles), for every indexer layer in turn (outer loop).
// Wave w scores chunk tiles w, w + NW, ...  Per tile and layer the selection
// word goes to LDS; per entry the maximum z over the layers that select it
// stays in the wave's LDS slice across layers (-inf while none has).  After the
// last layer the whole block
//   * writes its selection words, one contiguous run per layer, and
//   * compacts each of its chunks: every entry with a finite merged logit,
//     in ascending order (ballot + mbcnt inside a wave, a prefix over the
//     waves in LDS), into the chunk's candidate list (entry index, merged
//     logit) plus count.
// So the kernel writes a few contiguous runs per block instead of one line per
// tile; writes interleaved with the key stream cost far more HBM time than
// their bytes.  RING: register-ring depth (RING-1 tiles in flight per wave).
// NW = 4 wavefronts per block; 16 when the grid has fewer blocks than twice
// the compute units (few requests, short lists), so that a short list still
// spreads over many wavefronts.  CPB = 2 when there are at least three
// blocks of two chunks per compute unit: every block pays a fixed start and
// end (q~ set-up, ring fill, compaction), and halving the block count was
// 2% faster at 1M context.  Then the first a.pairs chunk pairs of every
// request go to two-chunk blocks -- as many as the compute units hold at
// once (three each, by LDS) -- and the remaining chunks to one-chunk blocks
// dispatched after them (request-major in both parts), so the blocks that
// start late, as slots free up, are the short ones.  At 1M context: 768
// two-chunk blocks, then 512 one-chunk blocks, two per compute unit;
// 0.519 ms against 0.526 ms with two-chunk blocks only (other splits leave
// a ragged first round and were slower).
constexpr int kSetupW = 4;   // wavefronts that form q~ (their layout below)

template <int KT, int DI, int RING, bool WZ, bool WI, int WPE, int NW, int CPB>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE)))
void score_kernel(ScoreArgs a) {
  using G = Geo<KT, DI>;
  constexpr int kTPW = CPB * LSA_CAND_CHUNK / 32 / NW;   // tiles per wave and layer
  static_assert(kTPW * 32 * NW == CPB * LSA_CAND_CHUNK, "chunk must split evenly");
  static_assert(LSA_CAND_CHUNK % (64 * NW) == 0, "a compaction round stays in one chunk");
  __shared__ __attribute__((aligned(16))) float qt[LSA_MAX_LAYERS][DI];
  __shared__ __attribute__((aligned(16))) float zacc[NW][kTPW][32];
  __shared__ uint32_t mwords[LSA_MAX_LAYERS][NW * kTPW];
  __shared__ int s_wave[NW];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int half = lane >> 5;
  int b, cf, cn;   // request, first chunk and number of chunks of this block
  if constexpr (CPB == 2) {
    const int P2 = a.pairs, S1 = a.nchunks - 2 * P2;
    const int u = blockIdx.x;
    if (u < a.B * P2) {
      b = u / P2;
      cf = 2 * (u - b * P2);
      cn = 2;
    } else {
      const int v = u - a.B * P2;
      b = v / S1;
      cf = 2 * P2 + (v - b * S1);
      cn = 1;
    }
  } else {
    b = blockIdx.y;
    cf = blockIdx.x;
    cn = 1;
  }
  const int L = a.L;

  // qt[l] = sum_h g_h q_h of (layer l, request b), fp32, in one round of
  // loads (a chain of dependent loads here would queue behind the key streams
  // of the other blocks on this compute unit).  Thread t takes dims
  // [8 (t % TPR), +8) of heads t / TPR + NG i; the sums run over a thread's
  // heads, then over the lanes of its wave with the same dims, then over the
  // first kSetupW waves in order (through the zacc area, free until the
  // first tile).
  {
    constexpr int TPR = DI / 8;              // threads per 16-byte-wide head row
    constexpr int NG = 64 * kSetupW / TPR;   // head groups
    constexpr int HPG = (64 + NG - 1) / NG;  // heads per group (H <= 64)
    const int dg = threadIdx.x % TPR, hg = threadIdx.x / TPR;
    float* red = &zacc[0][0][0];             // [L][kSetupW][DI] partial sums
    static_assert(LSA_MAX_LAYERS * kSetupW * DI <= NW * kTPW * 32, "zacc holds the partial sums");
    for (int l0 = 0; l0 < L && wave < kSetupW; l0 += 4) {   // up to four layers per round of loads
      u32x4 qv4[4][HPG];
      float gv[4][HPG];
#pragma unroll
      for (int lb = 0; lb < 4; ++lb) {
        const size_t p = (size_t)min(l0 + lb, L - 1) * a.B + b;
        const __amdgpu_buffer_rsrc_t qr = buffer(a.q + p * a.H * DI, (uint32_t)a.H * DI * 2);
        const __amdgpu_buffer_rsrc_t gr = buffer(a.g + p * a.H, (uint32_t)a.H * 4);
#pragma unroll
        for (int i = 0; i < HPG; ++i) {
          const uint32_t h = (uint32_t)(hg + NG * i);   // past H: the range check reads 0
          qv4[lb][i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, (h * DI + 8 * dg) * 2, 0, 0));
          gv[lb][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gr, h * 4, 0, 0));
        }
      }
#pragma unroll
      for (int lb = 0; lb < 4; ++lb) {
        if (l0 + lb >= L) break;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < HPG; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = qv4[lb][i][e >> 1];
            const float qe = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
            acc[e] = fmaf(gv[lb][i], qe, acc[e]);
          }
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
        if (lane < TPR)
#pragma unroll
          for (int e = 0; e < 8; ++e) red[((l0 + lb) * kSetupW + wave) * DI + 8 * dg + e] = acc[e];
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < L * DI; i += 64 * NW) {
      const int l = i / DI, d = i - l * DI;
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kSetupW; ++w) acc += red[(l * kSetupW + w) * DI + d];
      qt[l][d] = acc;
    }
    __syncthreads();
  }

  const uint32_t N = (uint32_t)a.N;
  const int ntiles = (a.N + 31) >> 5;
  const int c_tile0 = cf * (LSA_CAND_CHUNK / 32);                     // first tile of the block
  const int c_tiles = min(cn * (LSA_CAND_CHUNK / 32), ntiles - c_tile0);  // tiles in this block
  const int n_my = wave < c_tiles ? (c_tiles - wave + NW - 1) / NW : 0;
  const int t0 = c_tile0 + wave;
  const int t_last = t0 + NW * (n_my - 1);

  for (int l = 0; l < L && n_my > 0; ++l) {
    const int p = l * a.B + b;
    // this lane's slice of qt: dims [EPC * (lane % LPR), EPC * (lane % LPR + 1))
    float qv[G::EPC];
#pragma unroll
    for (int i = 0; i < G::EPC; ++i) qv[i] = qt[l][G::EPC * (lane % G::LPR) + i];
    const __amdgpu_buffer_rsrc_t kr =
        buffer((const unsigned char*)a.keys[l] + (size_t)b * a.stride * G::RB, N * G::RB);
    const __amdgpu_buffer_rsrc_t sr =
        buffer(KT == 1 ? (const void*)(a.scale[l] + (size_t)b * a.stride) : a.keys[l], KT == 1 ? N * 4 : 0);
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
        const float zv = score_tile<KT, DI>(ring[r], lane, qv, bias);
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
  // chunk compaction, ascending: thread j of round r takes block entry
  // e = 64 NW r + j, held by wave (e/32) % NW at local tile (e/32) / NW; the
  // rounds of chunk cc cover block entries [cc, cc + 1) * LSA_CAND_CHUNK
  const int b_entries = min(cn * LSA_CAND_CHUNK, a.N - c_tile0 * 32);
#pragma unroll
  for (int cc = 0; cc < CPB; ++cc) {
    const int e_beg = cc * LSA_CAND_CHUNK;
    if (e_beg >= b_entries) break;
    const int e_end = min(e_beg + LSA_CAND_CHUNK, b_entries);
    const size_t list = (size_t)b * a.nchunks + cf + cc;
    int* cidx = a.cand_idx + list * LSA_CAND_CHUNK;
    float* cz = a.cand_z + list * LSA_CAND_CHUNK;
    int base = 0;
    for (int e0 = e_beg; e0 < e_end; e0 += 64 * NW) {
      const int e = e0 + threadIdx.x;
      const int tc = e >> 5;
      float zm = -__builtin_inff();
      if (e < e_end) zm = zacc[tc % NW][tc / NW][e & 31];
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
    if (threadIdx.x == 0) a.cand_count[list] = base;
  }
}

template <int KT, int DI, int RING, int WPE, int NW, int CPB>
hipError_t launch_nw(const ScoreArgs& a, hipStream_t s) {
  dim3 grid(a.nchunks, a.B);
  if (CPB == 2) grid = dim3(a.B * a.pairs + a.B * (a.nchunks - 2 * a.pairs));
  const bool wz = a.z != nullptr, wi = a.I != nullptr;
  if (!wz && !wi)
    hipLaunchKernelGGL((score_kernel<KT, DI, RING, false, false, WPE, NW, CPB>), grid, dim3(64 * NW), 0, s, a);
  else if (wz && !wi)
    hipLaunchKernelGGL((score_kernel<KT, DI, RING, true, false, WPE, NW, CPB>), grid, dim3(64 * NW), 0, s, a);
  else if (!wz && wi)
    hipLaunchKernelGGL((score_kernel<KT, DI, RING, false, true, WPE, NW, CPB>), grid, dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((score_kernel<KT, DI, RING, true, true, WPE, NW, CPB>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int KT, int DI, int RING = 2, int WPE = 2>
hipError_t launch_t(const ScoreArgs& a0, hipStream_t s) {
  const int64_t cus = device_cu_count();
  ScoreArgs a = a0;
  a.pairs = 0;
  if ((int64_t)a.nchunks * a.B < 2 * cus) return launch_nw<KT, DI, RING, 1, 16, 1>(a, s);
  if ((int64_t)((a.nchunks + 1) / 2) * a.B >= 3 * cus) {
    // two-chunk blocks for as many pairs as three blocks per compute unit hold
    a.pairs = (int)std::min<int64_t>(a.nchunks / 2, 3 * cus / a.B);
    return launch_nw<KT, DI, RING, WPE, 4, 2>(a, s);
  }
  return launch_nw<KT, DI, RING, WPE, 4, 1>(a, s);
}

}  // namespace

hipError_t launch_score(int dI, lsa_key_dtype kdt, const ScoreArgs& a, hipStream_t s) {
  if (kdt == LSA_KEY_BF16) return dI == 64 ? launch_t<0, 64>(a, s) : launch_t<0, 128>(a, s);
  return dI == 64 ? launch_t<1, 64>(a, s) : launch_t<1, 128>(a, s);
}

}  // namespace lsa
