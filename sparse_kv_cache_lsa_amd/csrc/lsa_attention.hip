// lsa_attention.hip -- core attention of one decode step over the selected
// compressed rows (gist.science technical summary, section 2.1,
// hierarchical-selection bullet: the top-k chosen inside the fetched subset
// feeds the final core attention), plus a local window of recent rows.
//
// Per request b and head h, over the rows R_b = the first hot_count[b] rows of
// hot[b] followed by the first win_count[b] rows of win[b]:
//   s_j = scale * (q[b][h] . r_j),  out[b][h] = sum_j softmax(s)_j r_j
// Every row is a compressed latent vector that is both key and value and is
// shared by all heads, so the two products are dense contractions with the
// head count as one dimension: both run on v_mfma_f32_16x16x32_bf16.
//
// Block = (request, split of its rows, group of 64 heads), 8 wavefronts.
// Wave w works on heads 16 (w % 4) .. +15 of the group and on output dims
// 256 (w / 4) .. +255; the two waves of a head group each form the scores
// over their half of the dims and exchange them through LDS, so both hold the
// same full scores (fp32 a + b is commutative: the same bits in both).  The
// block walks its rows in tiles of 32:
//  * load: wave w reads 4 rows of the tile (K group w % 4, half w / 4: rows
//    4 (w%4) .. +3, or 16 + 4 (w%4) .. +3), one 1 KiB row per load
//    instruction (16 B per lane, dims 8l..8l+7), and writes them to one
//    row-major LDS copy whose 16-byte units are XOR-swizzled by row.  The
//    S^T = V Q^T operand (lane (n, g): row n, dims 32j + 8g .. +8) is read
//    from it directly; the O^T += V^T P^T operand (lane (n, g): dim 16t + n of
//    rows 4g + i and 16 + 4g + i) is read from the same copy with
//    ds_read_tr16_b64, which transposes 16-bit elements across each group of
//    16 lanes.  The next tile's rows are loaded into registers while the
//    current one is worked on.
//  * S^T: two 16-row halves x 8 K-steps of 32 dims; B = the wave's query
//    fragments (registers, loaded once).  Lane (n, g) gets rows 4g + i and
//    16 + 4g + i of head n.
//  * online softmax per head in the exp2 domain (scale * log2 e folded in);
//    the lane's 8 weights are exactly the B operand of the PV product in K
//    order (4g + i, 16 + 4g + i), split exactly into bf16 hi + lo (residual
//    below 2^-16 of the weight), so the weights lose no precision.
//  * PV: 16 dim tiles x 2 products (hi, lo) into 64 fp32 accumulators.
// A block with one split writes the normalised output; otherwise it writes
// its unnormalised output and (max, sum) per head, and a combine kernel
// rescales and adds the splits.
#include "lsa_device.h"
#include "lsa_launch.h"

#include <algorithm>

namespace lsa {
namespace {

constexpr int kAttD = 512;                 // row width (elements)
constexpr int kTile = 32;                  // rows per tile
constexpr int kRowBytes = 2 * kAttD;      // bytes per row of the LDS copy
constexpr int kHeadsPerBlock = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

struct AttArgs {
  const uint16_t* q;        // [B][H][D]
  const uint16_t* hot;      // [B][k][D]
  const int32_t* hot_count; // [B] or null
  const uint16_t* win;      // [B][W][D] or null
  const int32_t* win_count; // [B] or null
  float* out;               // [B][H][D]
  float* part_o;            // [S][B][H][D] (S > 1)
  float* part_ml;           // [S][B][H][2] (S > 1)
  int B, H, k, W, S, rows_per_split;
  float scale_log2;         // scale * log2(e)
};

// Byte offset of 16-byte unit u (0..63) of LDS row r (0..31): the unit index
// is XORed with an even mask for rows 0-7 (16-23) and an odd one for rows
// 8-15 (24-31), so with 64 banks of 4 bytes a row written by one instruction,
// 16 rows read at one unit, and the transposed reads (8 rows at two adjacent
// units) all fall in distinct banks.
__device__ __forceinline__ uint32_t lds_off(int r, int u) {
  const int h = ((2 * r) & 15) ^ ((r >> 3) & 1);
  return (uint32_t)(r * kRowBytes + ((u ^ h) << 4));
}

typedef short v4s __attribute__((ext_vector_type(4)));

// ds_read_tr16_b64: in each group of 16 lanes, lane 4a + c receives element c
// of the 8-byte pieces addressed by lanes a, a + 4, a + 8 and a + 12.
__device__ __forceinline__ u32x2 tr_read(const unsigned char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<unsigned char*>(p))));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(512) void attention_kernel(AttArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char rm[kTile * kRowBytes];    // row-major
  __shared__ __attribute__((aligned(16))) f32x4 xs[8][2][64];                      // score halves
  // the wave index is uniform across a wavefront: keep it in a scalar
  // register so that row sources and buffer resources stay scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int hg = wave & 3, dh = wave >> 2;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int b = blockIdx.x, s = blockIdx.y;
  const int h0 = blockIdx.z * kHeadsPerBlock + 16 * hg;   // first head of this wave
  const bool active = h0 < a.H;
  const int kc = a.hot_count ? min(max(a.hot_count[b], 0), a.k) : a.k;
  const int wc = a.W == 0 ? 0 : (a.win_count ? min(max(a.win_count[b], 0), a.W) : a.W);
  const int nb = kc + wc;
  const int r_beg = s * a.rows_per_split;
  const int r_end = min(nb, r_beg + a.rows_per_split);

  const __amdgpu_buffer_rsrc_t hot_r =
      rsrc(a.hot + (size_t)b * a.k * kAttD, (uint32_t)kc * kAttD * 2);
  const __amdgpu_buffer_rsrc_t win_r =
      rsrc(a.W ? a.win + (size_t)b * a.W * kAttD : a.hot, (uint32_t)wc * kAttD * 2);

  // query fragments of head h0 + n (B operand of S^T): dims 256 dh + 32 j + 8 g .. +8
  bf16x8 qf[8];
  {
    const int nh = active ? min(16, a.H - h0) : 0;   // heads past H read 0
    const __amdgpu_buffer_rsrc_t qr =
        rsrc(a.q + ((size_t)b * a.H + (active ? h0 : 0)) * kAttD, (uint32_t)nh * kAttD * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      qf[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                             qr, (uint32_t)(n * kAttD * 2 + 512 * dh + 64 * j + 16 * g),
                                             0, 0));
  }

  // rows this wave loads: K group hg, half dh
  auto tile_row = [&](int i) { return dh == 0 ? 4 * hg + i : 16 + 4 * hg + i; };
  auto load_tile = [&](int r0, u32x4 (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + tile_row(i);
      const bool in = r < r_end;
      const bool from_hot = r < kc;
      const uint32_t off = in ? (uint32_t)((from_hot ? r : r - kc) * kAttD * 2 + 16 * lane)
                              : 0xFFFFFF00u;
      x[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(from_hot ? hot_r : win_r, off, 0, 2));
    }
  };

  f32x4 acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff();   // running max (log2 domain) of head h0 + n
  float l = 0.f;                 // this lane's part of the running sum

  u32x4 x[4];
  if (r_beg < r_end) load_tile(r_beg, x);
  for (int r0 = r_beg; r0 < r_end; r0 += kTile) {
    __syncthreads();   // every wave is done with the previous tile's LDS
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4*)(rm + lds_off(tile_row(i), lane)) = x[i];
    if (r0 + kTile < r_end) load_tile(r0 + kTile, x);   // next tile, in flight meanwhile
    __syncthreads();

    // ---- S^T over this wave's half of the dims, then the partner's half
    f32x4 sc[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8*)(rm + lds_off(16 * half + n, 32 * dh + 4 * j + g)), qf[j], c, 0, 0, 0);
      sc[half] = c;
      xs[wave][half][lane] = c;
    }
    __syncthreads();
    sc[0] += xs[wave ^ 4][0][lane];
    sc[1] += xs[wave ^ 4][1][lane];

    // ---- online softmax (log2 domain); rows past r_end do not count
    float v[8];
    float mt = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
      v[i] = r < r_end ? sc[i >> 2][i & 3] * a.scale_log2 : -__builtin_inff();
      mt = fmaxf(mt, v[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float mn = fmaxf(m, mt);
    const float alpha = mn == -__builtin_inff() ? 1.f : exp2f(m - mn);
    m = mn;
    float ps = 0.f;
    uint32_t phi[4], plo[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = mn == -__builtin_inff() ? 0.f : exp2f(v[i] - mn);
      const float p1 = mn == -__builtin_inff() ? 0.f : exp2f(v[i + 1] - mn);
      ps += p0 + p1;
      const uint32_t h0b = bf16_bits(p0), h1b = bf16_bits(p1);
      const float r0f = p0 - __uint_as_float(h0b << 16);
      const float r1f = p1 - __uint_as_float(h1b << 16);
      phi[i >> 1] = h0b | (h1b << 16);
      plo[i >> 1] = bf16_bits(r0f) | (bf16_bits(r1f) << 16);
    }
    l = l * alpha + ps;
    const bf16x8 bhi = __builtin_bit_cast(bf16x8, u32x4{phi[0], phi[1], phi[2], phi[3]});
    const bf16x8 blo = __builtin_bit_cast(bf16x8, u32x4{plo[0], plo[1], plo[2], plo[3]});
    // ---- O^T (this wave's dims x heads) = alpha O^T + V^T P^T
    // A operand: dims 256 dh + 16 t + n over rows 4g + i and 16 + 4g + i, read
    // transposed from the row-major copy (lane (n, g) addresses row 4g + n/4,
    // dims 256 dh + 16 t + 4 (n % 4) .. +3, and the same 16 rows on)
    const int rr = 4 * g + (n >> 2);
    const int uo = 32 * dh + ((n & 3) >> 1);
    const int bo = 8 * (n & 1);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const u32x2 lo = tr_read(rm + lds_off(rr, uo + 2 * t) + bo);
      const u32x2 hi = tr_read(rm + lds_off(16 + rr, uo + 2 * t) + bo);
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      f32x4 c = acc[t] * alpha;
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bhi, c, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, blo, c, 0, 0, 0);
    }
  }
  if (!active || h0 + n >= a.H) return;

  // the head's sum over its four lane groups
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  const int h = h0 + n;
  if (a.S == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* o = a.out + ((size_t)b * a.H + h) * kAttD + 256 * dh + 4 * g;
#pragma unroll
    for (int t = 0; t < 16; ++t) *(f32x4*)(o + 16 * t) = acc[t] * inv;
  } else {
    const size_t row = ((size_t)s * a.B + b) * a.H + h;
    float* o = a.part_o + row * kAttD + 256 * dh + 4 * g;
#pragma unroll
    for (int t = 0; t < 16; ++t) *(f32x4*)(o + 16 * t) = acc[t];
    if (g == 0 && dh == 0) {
      a.part_ml[2 * row] = m;
      a.part_ml[2 * row + 1] = l;
    }
  }
}

// out[b][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s;
// no rows at all: zeros.  One block of 128 threads per (request, head), four
// dims a thread.  Every split's (m, l) and partial output are loaded in one
// round (up to kCombineMax splits in registers; more in further rounds), and
// the splits are added in split order.
constexpr int kCombineMax = 16;

__global__ __launch_bounds__(128) void attention_combine_kernel(AttArgs a) {
  const int b = blockIdx.x, h = blockIdx.y;
  float M = -__builtin_inff();
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int s0 = 0; s0 < a.S; s0 += kCombineMax) {
    float ms[kCombineMax], ls[kCombineMax];
    f32x4 os[kCombineMax];
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) {
      const int s = s0 + j;
      ms[j] = -__builtin_inff();
      ls[j] = 0.f;
      os[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < a.S) {
        const size_t row = ((size_t)s * a.B + b) * a.H + h;
        ms[j] = a.part_ml[2 * row];
        ls[j] = a.part_ml[2 * row + 1];
        os[j] = *(const f32x4*)(a.part_o + row * kAttD + 4 * threadIdx.x);
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) Mn = fmaxf(Mn, ms[j]);
    if (Mn == -__builtin_inff()) continue;   // no rows yet
    // rescale what is summed so far to the new maximum, then add these splits
    const float r = M == -__builtin_inff() ? 0.f : exp2f(M - Mn);
    o *= r;
    L *= r;
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) {
      if (ms[j] == -__builtin_inff()) continue;
      const float w = exp2f(ms[j] - Mn);
      L += w * ls[j];
      o += w * os[j];
    }
    M = Mn;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *(f32x4*)(a.out + ((size_t)b * a.H + h) * kAttD + 4 * threadIdx.x) = o * inv;
}

}  // namespace

// Splits of a request's rows: about one block per compute unit (a block holds
// a compute unit by its registers), at least 4 tiles per split.  Every split
// adds a partial output of H x D fp32 per request to write and read back, so
// the split count stays as low as filling the chip allows.
int attention_splits(int B, int H, int k, int W) {
  const int n_max = k + W;
  const int tiles = (n_max + kTile - 1) / kTile;
  const int hb = (H + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int want = std::max(1, 256 / std::max(1, B * hb));
  const int cap = std::max(1, tiles / 4);
  return std::max(1, std::min(want, cap));
}

size_t attention_workspace_bytes(int B, int H, int D, int k, int W) {
  (void)D;
  const int S = attention_splits(B, H, k, W);
  if (S == 1) return 0;
  const size_t rows = (size_t)S * B * H;
  return (rows * kAttD * 4 + 255) / 256 * 256 + (rows * 2 * 4 + 255) / 256 * 256;
}

hipError_t launch_attention(int B, int H, int k, int W, float scale, const uint16_t* q,
                            const uint16_t* hot, const int32_t* hot_count, const uint16_t* win,
                            const int32_t* win_count, float* out, void* ws, hipStream_t s) {
  AttArgs a{};
  a.q = q;
  a.hot = hot;
  a.hot_count = hot_count;
  a.win = win;
  a.win_count = win_count;
  a.out = out;
  a.B = B;
  a.H = H;
  a.k = k;
  a.W = W;
  a.S = attention_splits(B, H, k, W);
  const int tiles = (k + W + kTile - 1) / kTile;
  a.rows_per_split = std::max(1, (tiles + a.S - 1) / a.S) * kTile;
  a.scale_log2 = scale * kLog2e;
  if (a.S > 1) {
    const size_t rows = (size_t)a.S * B * H;
    a.part_o = static_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         (rows * kAttD * 4 + 255) / 256 * 256);
  }
  const dim3 grid(B, a.S, (H + kHeadsPerBlock - 1) / kHeadsPerBlock);
  hipLaunchKernelGGL(attention_kernel, grid, dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S == 1) return e;
  hipLaunchKernelGGL(attention_combine_kernel, dim3(B, H), dim3(kAttD / 4), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsa
