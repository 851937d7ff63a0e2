// lsa_focal.hip -- student loss and gradient of the indexer's query
// projection, for gfx950, in fp32.
//
// The keys K_IComp are frozen and only the query encoder's projection W_q is
// trained, with binary cross-entropy plus a focal term that down-weights easy
// negatives (gist.science technical summary, section 2.3 "backbone-free
// decoupled training"; paper.oopus.info review, section 2, loss function).
//   q_t = W_q h_t, g_t = softplus(W_g h_t), z_ts = sum_h g_th (q_th . k_s) + b
//   u = (2y - 1) z, BCE = softplus(-u), FL = sigmoid(-u)^gamma softplus(-u)
//   loss = mean_ts BCE + mean_ts FL,   dW_q = d loss / d W_q
//
// The gated head sum is linear in the key, so the forward pass contracts the
// keys with one collapsed query per row, qe_t = sum_h g_th q_th (dI wide),
// and the backward pass goes through G_t = sum_s delta_ts k_s:
//   d loss / d q_thi = g_th G_ti,   dW_q[(h,i)][d] = sum_t g_th G_ti h_td.
// Every product splits its fp32 operand three ways into bf16 and runs on
// v_mfma_f32_32x32x16_bf16 against an exactly-bf16 operand (hidden states or
// keys): the products are exact and only the fp32 accumulation rounds.
//
// Kernels (one stream, in order):
//   1 project   partials of (W_q h_t)_r and (W_g h_t)_r per slice of D (W read once)
//   2 collapse  slice sums in order; g = softplus(gate rows), qe_t, gT[h][t]
//   3 transpose h -> hT [D][64] (contraction axis of dW_q contiguous)
//   4 logits    per 128-entry chunk: z = K qe^T + b, loss terms,
//               delta = dloss/dz (in LDS), partial G = delta K
//   6 reduce    GT[i][t] = sum of partials, loss = sum / (Q N) (fixed orders)
//   7 dW        dW_q = (gT * GT) hT^T, written once (nontemporal), four row
//               tiles a wave over the same columns
#include "lsa_device.h"
#include "lsa_launch.h"

namespace lsa {
namespace {

constexpr int kQP = 64;      // padded query count (rows of the small operands)
constexpr int kChunk = 128;  // entries per partial-gradient block
constexpr int kProjTR = 2;   // 32-row weight tiles per projection wave
constexpr int kMaxGateSlices = 32;   // gate_slices(D) <= 8 * 4

// Buffer resources: loads past `bytes` return 0, so rows beyond the operand
// (padding queries, the tail of the last tile) need no branch -- a branch
// around a load makes the compiler wait for every load in flight.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFFu ? bytes : 0x7FFFFFFFu),
                                           0x00020000);
}

__device__ __forceinline__ f32x4 buf_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

constexpr uint32_t kFar = 0x7FFFFFF0u;   // an offset past every range used here

// Three-way bf16 split of eight fp32 values: x = hi + mid + lo exactly (each
// residual is exact in fp32 and 3 x 8 significant bits cover fp32's 24), so
// three bf16 MFMAs against an exactly-bf16 operand reproduce the fp32 product
// terms exactly; only the fp32 accumulation rounds, as in an fp32 MFMA.  Ten
// times cheaper than v_mfma_f32_32x32x2_f32 per multiply-add.
struct Split3 {
  bf16x8 hi, mid, lo;
};

__device__ __forceinline__ Split3 split3(f32x4 a, f32x4 b) {
  Split3 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = i < 4 ? a[i] : b[i - 4];
    const __bf16 h = (__bf16)x;
    const float r1 = x - (float)h;
    const __bf16 m = (__bf16)r1;
    const float r2 = r1 - (float)m;
    r.hi[i] = h;
    r.mid[i] = m;
    r.lo[i] = (__bf16)r2;
  }
  return r;
}

__device__ __forceinline__ f32x16 mfma_split(const Split3& a, bf16x8 b, f32x16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.mid, b, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.lo, b, c, 0, 0, 0);
}

// accumulator element rr of lane l: row (rr&3) + 4*(l/32) + 8*(rr/4), col l%32
__device__ __forceinline__ int acc_row(int rr, int half) { return (rr & 3) + 4 * half + 8 * (rr >> 2); }

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }

// sigmoid(-u)^gamma: repeated products for whole gamma in [1, 8] (a few ulps,
// where powf costs a logarithm and an exponential per element), powf else.
__device__ __forceinline__ float focal_mod(float qu, float gamma, int igamma) {
  if (gamma == 0.f) return 1.f;
  if (igamma > 0) {
    float r = qu;
    for (int i = 1; i < igamma; ++i) r *= qu;
    return r;
  }
  return powf(qu, gamma);
}
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))); }

// ---------------------------------------------------------------- 1 project
// 1-D grid: KSG blocks for the gate rows (W_g, H <= 64 rows), then the W_q
// blocks: 64-row groups x KS slices of D, the slices of one group adjacent.
// The 4 waves of a block split the block's slice again; each wave keeps a
// 32-row x 64-query tile per 32-row tile.  A W_q block writes its partial sums
// to qp[ks][t][r], a gate block to gp[ks][t][h]; splitting D keeps enough loads
// in flight to stream W at full rate.  The gate rows take KSG = m KS slices
// (m up to 4), so their blocks are m times shorter and, dispatched first,
// finish early in the first round of blocks: for H dI = 8192 and D = 4096
// the 1,024 W_q blocks then fill two rounds of two blocks per compute unit,
// where the gate rows as one more 64-row group had made a third round of 8
// blocks.
// HL: the block's slice of the hidden states (64 queries x at most
// kProjSpan k) is first copied into LDS with contiguous 1 KiB row loads; a
// wave's fragment loads straight from memory touch 32 rows each (32 cache
// lines per instruction), and without them the kernel took 52 us instead of
// 69 us.
constexpr int kProjSpan = 512;

template <int TR, bool HL>   // TR: 32-row tiles per wave (they share the hidden-state loads)
__global__ __launch_bounds__(256) void fproj_kernel(int Q, int D, int HdI, int H, int KS, int KSG,
                                                    const float* __restrict__ Wq,
                                                    const float* __restrict__ Wg,
                                                    const uint16_t* __restrict__ h,
                                                    float* __restrict__ qp,
                                                    float* __restrict__ gp) {
  // the partial-sum exchange reuses the LDS of the staged hidden states
  constexpr int kHP = kProjSpan + 8;   // padded row: consecutive rows 16 B apart in the banks
  constexpr size_t kRedB = sizeof(float) * 4 * 2 * TR * 16 * 64;
  constexpr size_t kHsB = HL ? sizeof(uint16_t) * kQP * kHP : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kRedB > kHsB ? kRedB : kHsB];
  float(*red)[2 * TR][16][64] = reinterpret_cast<float(*)[2 * TR][16][64]>(smem);
  uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, half = lane >> 5;
  // block -> (gate or W_q, slice by, first row r0b of the 32 TR rows)
  const bool gate = (int)blockIdx.x < KSG;
  const int b = (int)blockIdx.x - KSG;
  const int by = gate ? (int)blockIdx.x : b % KS;
  const int r0b = gate ? 0 : (b / KS) * 32 * TR;
  const int nsl = gate ? KSG : KS;
  const int nrows = gate ? H : HdI;   // rows past these read 0 through the range check
  const __amdgpu_buffer_rsrc_t ra = gate ? rsrc(Wg, (size_t)H * D * 4) : rsrc(Wq, (size_t)HdI * D * 4);
  uint32_t aoff[TR];
#pragma unroll
  for (int i = 0; i < TR; ++i) aoff[i] = (uint32_t)(r0b + 32 * i + n) * D * 4;
  const __amdgpu_buffer_rsrc_t rb = rsrc(h, (size_t)Q * D * 2);
  const int kq = D / (4 * nsl);
  const int kbeg = (by * 4 + wave) * kq, kend = kbeg + kq;
  const int kb0 = by * 4 * kq;   // the block's first k
  // v_mfma_f32_32x32x16_bf16, two steps per 32 k: lane (m, half) holds
  // k = k0 + 16 half + 8 s .. +7 of row m in step s, so each lane reads 64
  // contiguous weight bytes per 32 k (the two halves of a row fill a 128-byte
  // line) and 32 bytes of each hidden state.  NS stages of 32 k are in flight
  // per wave; the first ones are issued before the staged hidden states are
  // written to LDS, so their latency overlaps the copy (the LDS writes wait
  // only for the older hidden-state loads), and each stage is reloaded with
  // the k NS stages ahead as soon as it is multiplied.  Two stages: 137
  // against 145 us for the whole loss and gradient with the Infinity Cache
  // flushed (one stage issued after the copy: 145; three: 141).
  constexpr int NS = 2;
  const int kh = 16 * half;
  auto load_w = [&](int k, f32x4 (&w)[TR][4]) {
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) w[i][j] = buf_f32x4(ra, aoff[i] + (k + kh + 4 * j) * 4);
  };
  f32x4 wst[NS][TR][4];
  if constexpr (HL) {
    // rows q < 64 of h for k in [kb0, kb0 + 4 kq), 16-byte chunks in row
    // order (queries past Q read 0 through the range check)
    const int cpr = kq / 2;   // chunks per row: 4 kq / 8
    constexpr int kIt = kQP * (kProjSpan / 8) / 256;
    u32x4 t[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int c = threadIdx.x + 256 * i, q = c / cpr, col = 8 * (c - q * cpr);
      t[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rb, q < kQP ? ((uint32_t)q * D + kb0 + col) * 2 : kFar, 0, 0));
    }
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)
      if (kbeg + 32 * s2 < kend) load_w(kbeg + 32 * s2, wst[s2]);
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int c = threadIdx.x + 256 * i, q = c / cpr, col = 8 * (c - q * cpr);
      if (q < kQP) *(u32x4*)&hs[q * kHP + col] = t[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)
      if (kbeg + 32 * s2 < kend) load_w(kbeg + 32 * s2, wst[s2]);
  }
  const uint32_t b0off = (uint32_t)n * D * 2, b1off = (uint32_t)(n + 32) * D * 2;
  f32x16 acc[TR][2] = {};
  for (int k0 = kbeg; k0 < kend; k0 += 32 * NS) {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int k = k0 + 32 * s2;
      if (k < kend) {
        const int kk = k + kh;
        bf16x8 x0[2], x1[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (HL) {
            x0[j] = *(const bf16x8*)&hs[n * kHP + (kk - kb0) + 8 * j];
            x1[j] = *(const bf16x8*)&hs[(n + 32) * kHP + (kk - kb0) + 8 * j];
          } else {
            x0[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rb, b0off + (kk + 8 * j) * 2, 0, 0));
            x1[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rb, b1off + (kk + 8 * j) * 2, 0, 0));
          }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < TR; ++i) {
            const Split3 a = split3(wst[s2][i][2 * st], wst[s2][i][2 * st + 1]);
            acc[i][0] = mfma_split(a, x0[st], acc[i][0]);
            acc[i][1] = mfma_split(a, x1[st], acc[i][1]);
          }
        const int kn = k + 32 * NS;
        if (kn < kend) load_w(kn, wst[s2]);
      }
    }
  }
  if constexpr (HL) __syncthreads();   // every wave is done with the staged hidden states
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      red[wave][2 * i][rr][lane] = acc[i][0][rr];
      red[wave][2 * i + 1][rr][lane] = acc[i][1][rr];
    }
  __syncthreads();
  const int ld = gate ? kQP : HdI;   // gp rows hold 64 gates
  float* out = (gate ? gp : qp) + (size_t)by * kQP * ld;
  for (int e = threadIdx.x; e < 2 * TR * 16 * 64; e += 256) {
    const int ij = e >> 10, rr = (e >> 6) & 15, l = e & 63;
    const int i = ij >> 1, j = ij & 1;
    const float v = red[0][ij][rr][l] + red[1][ij][rr][l] + red[2][ij][rr][l] + red[3][ij][rr][l];
    const int t = 32 * j + (l & 31);
    const int row = r0b + 32 * i + acc_row(rr, l >> 5);
    if (t < Q && row < nrows) out[(size_t)t * ld + row] = v;
  }
}

// ---------------------------------------------------------------- 2 collapse
// qa[t][r] = sum of the KS slice partials in slice order, formed where needed
// (the gate rows: their KSG slices in order).
// grid: (kQP queries, dI/32 dim groups); block: 256 threads.  Each thread sums
// the partials of 8 (head, dim) pairs of the group with all loads in flight
// (into LDS), then one thread per dim runs the gate-weighted sum over heads in
// head order.  Rows t >= Q get zeros; the gates are formed by every block and
// written by group 0.
__global__ __launch_bounds__(256) void fcollapse_kernel(int Q, int H, int dI, int KS, int KSG,
                                                        const float* __restrict__ qp,
                                                        const float* __restrict__ gp,
                                                        float* __restrict__ gT,
                                                        float* __restrict__ qe) {
  __shared__ float gs[64];
  __shared__ float qs[64][33];
  const int t = blockIdx.x;
  const int HdI = H * dI;
  const size_t slice = (size_t)kQP * HdI;
  const size_t rowb = (size_t)t * HdI;
  const bool live = t < Q;
  const int i0 = blockIdx.y * 32;
  // (head, dim) pairs p = threadIdx.x + 256 u, u < 8: head p / 32, dim i0 + p % 32;
  // threads 0..63 also take the gate row of head threadIdx.x
  float acc[9];
#pragma unroll
  for (int u = 0; u < 9; ++u) acc[u] = 0.f;
  if (live) {
    for (int ks = 0; ks < KS; ++ks) {
      const float* base = qp + ks * slice + rowb;
      float v[9];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pr = threadIdx.x + 256 * u, hh = pr >> 5, i = i0 + (pr & 31);
        v[u] = (hh < H && i < dI) ? base[hh * dI + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = ks == 0 ? v[u] : acc[u] + v[u];
    }
    if (threadIdx.x < H) {
      // every gate slice in flight at once: slices past KSG read 0 through
      // the range check and add nothing
      const __amdgpu_buffer_rsrc_t rg = rsrc(gp, (size_t)KSG * kQP * kQP * 4);
      float gv[kMaxGateSlices];
#pragma unroll
      for (int ks = 0; ks < kMaxGateSlices; ++ks)
        gv[ks] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rg, (uint32_t)((ks * kQP + t) * kQP + threadIdx.x) * 4u, 0, 0));
#pragma unroll
      for (int ks = 0; ks < kMaxGateSlices; ++ks) acc[8] = ks == 0 ? gv[ks] : acc[8] + gv[ks];
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pr = threadIdx.x + 256 * u;
    qs[pr >> 5][pr & 31] = acc[u];
  }
  if (threadIdx.x < 64) {
    const float g = (live && threadIdx.x < H) ? softplus_f(acc[8]) : 0.f;
    gs[threadIdx.x] = g;
    if (blockIdx.y == 0 && threadIdx.x < H) gT[threadIdx.x * kQP + t] = g;
  }
  __syncthreads();
  const int i = i0 + threadIdx.x;
  if (threadIdx.x < 32 && i < dI) {
    float a = 0.f;
    if (live)
      for (int hh = 0; hh < H; ++hh) a = fmaf(gs[hh], qs[hh][threadIdx.x], a);
    qe[t * dI + i] = a;
  }
}

// ---------------------------------------------------------------- 3 transpose
// Two jobs in one launch (blocks [0, nb0) job 0, the rest job 1); per job
// out[c][r] = in[r][c] for r < rows, 0 for rows <= r < out_ld (bf16 bits),
// in 64 x 64 tiles, ntx tiles along r.
struct TransposeJob {
  const uint16_t* in;
  uint16_t* out;
  int rows, cols, out_ld, ntx;
};

// 64 x 64 tiles through LDS: 8-byte row loads (K need only be 8-byte
// aligned) and 16-byte column stores into the workspace (rows of the output
// are multiples of 8 elements).  Moving 2-byte elements one by one took 12 us
// for the label workload.
__global__ __launch_bounds__(256) void ftranspose_kernel(TransposeJob j0, TransposeJob j1, int nb0) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][64 + 4];   // row pitch 136 B
  const bool second = (int)blockIdx.x >= nb0;
  const TransposeJob jb = second ? j1 : j0;
  const int b = second ? (int)blockIdx.x - nb0 : (int)blockIdx.x;
  const int r0 = (b % jb.ntx) * 64, c0 = (b / jb.ntx) * 64;
  const bool vec = (jb.cols & 3) == 0 && ((uintptr_t)jb.in & 7u) == 0;   // uniform
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x + 256 * i;   // 1024 chunks of 4 elements
    const int rr = e >> 4, cc = (e & 15) * 4;
    const int r = r0 + rr, c = c0 + cc;
    uint2 v = uint2{0u, 0u};
    if (vec) {
      if (r < jb.rows && c < jb.cols) v = *(const uint2*)(jb.in + (size_t)r * jb.cols + c);
    } else {
      uint16_t x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[k] = (r < jb.rows && c + k < jb.cols) ? jb.in[(size_t)r * jb.cols + c + k] : (uint16_t)0;
      v = uint2{x[0] | ((uint32_t)x[1] << 16), x[2] | ((uint32_t)x[3] << 16)};
    }
    *(uint2*)&tile[rr][cc] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = threadIdx.x + 256 * i;   // 512 chunks of 8 output elements
    const int cc = e >> 3, rr = (e & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    if (c < jb.cols && r < jb.out_ld) {   // out_ld is a multiple of 8
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = (uint32_t)tile[rr + 2 * k][cc] | ((uint32_t)tile[rr + 2 * k + 1][cc] << 16);
      *(u32x4*)(jb.out + (size_t)c * jb.out_ld + r) = o;
    }
  }
}

// ---------------------------------------------------------------- 4+5 fused
// Logits, loss terms, dloss/dz and the partial key gradient of one chunk of
// kChunk entries in one kernel; grid ceil(Np / kChunk), 256 threads.
//  1. The chunk's key rows (bf16, kChunk x DI; rows past N read 0) and the
//     collapsed queries (fp32, 64 x DI) are copied into LDS with contiguous
//     loads.
//  2. Logits: wave w (of 8) takes the chunk's entries 32 (w % 4) .. +31
//     against queries 32 (w / 4) .. +31.  A = collapsed queries split exactly into three bf16
//     parts, B = key rows (exact bf16), so the products are exact and only
//     the fp32 accumulation rounds; lanes run over entries, so label loads
//     coalesce.  The epilogue sums the loss terms and writes
//     delta = dloss/dz into LDS (0 outside [0, Q) x [0, N)).
//  3. Partial key gradient Gp[chunk][t][i] = sum over the chunk's entries of
//     delta[t][s] K[s][i]: wave w takes queries 32 (w & 1) .. +31 and dims
//     32 (w >> 1) .. +31; A = delta split into three bf16 parts, B = key
//     columns gathered from the LDS rows.
// delta never goes to memory and the keys need no transposed copy; as two
// kernels (logits, then G over a transposed key copy) this took 34 us for the
// label workload.
template <int DI>
__global__ __launch_bounds__(512) void flogits_grad_kernel(int Q, int N, float gamma, float bias,
                                                           float inv_qn,
                                                           const uint16_t* __restrict__ K,
                                                           const float* __restrict__ qe,
                                                           const uint8_t* __restrict__ label,
                                                           float* __restrict__ Gp,
                                                           double* __restrict__ loss_part) {
  constexpr int NT = 512;          // 8 wavefronts
  constexpr int KP = DI + 8;       // bf16 pitch of the key rows (16 B pad)
  constexpr int QP = DI + 4;       // fp32 pitch of the query rows
  constexpr int DP = kChunk + 4;   // fp32 pitch of the delta rows
  __shared__ __attribute__((aligned(16))) uint16_t ks[kChunk][KP];
  __shared__ __attribute__((aligned(16))) float qs[kQP][QP];
  __shared__ __attribute__((aligned(16))) float dls[kQP][DP];
  __shared__ double wsum[NT / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, half = lane >> 5;
  const int s_base = blockIdx.x * kChunk;

  // 1. stage (K need only be 8-byte aligned: 8-byte loads)
  const __amdgpu_buffer_rsrc_t rk = rsrc(K, (size_t)N * DI * 2);
#pragma unroll
  for (int i = 0; i < kChunk * DI / 4 / NT; ++i) {
    const int c = threadIdx.x + NT * i, r = c / (DI / 4), col = 4 * (c - r * (DI / 4));
    const u32x2 v = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, ((uint32_t)(s_base + r) * DI + col) * 2, 0, 0));
    *(u32x2*)&ks[r][col] = v;
  }
#pragma unroll
  for (int i = 0; i < kQP * DI / 4 / NT; ++i) {
    const int c = threadIdx.x + NT * i, r = c / (DI / 4), col = 4 * (c - r * (DI / 4));
    *(f32x4*)&qs[r][col] = *(const f32x4*)(qe + r * DI + col);
  }
  __syncthreads();

  // 2. logits and delta: wave w takes entries 32 (w % 4) .. +31 against
  // queries 32 (w / 4) .. +31
  const int s0 = 32 * (wave & 3), tq2 = 32 * (wave >> 2);
  f32x16 acc = {};
#pragma unroll
  for (int k = 0; k < DI; k += 16) {
    const int kk = k + 8 * half;
    const Split3 a = split3(*(const f32x4*)&qs[tq2 + n][kk], *(const f32x4*)&qs[tq2 + n][kk + 4]);
    acc = mfma_split(a, *(const bf16x8*)&ks[s0 + n][kk], acc);
  }
  const int s = s_base + s0 + n;
  const __amdgpu_buffer_rsrc_t rl = rsrc(label, (size_t)Q * N);
  uint32_t yv[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int t = tq2 + acc_row(rr, half);
    yv[rr] = __builtin_amdgcn_raw_buffer_load_b8(rl, s < N ? (uint32_t)t * N + s : kFar, 0, 0);
  }
  // gamma as a whole number in [1, 8], else 0 (uniform)
  const int igamma = (gamma >= 1.f && gamma <= 8.f && gamma == floorf(gamma)) ? (int)gamma : 0;
  double lsum = 0.0;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int t = tq2 + acc_row(rr, half);
    const bool valid = t < Q && s < N;
    const float z = acc[rr] + bias;
    const int y = yv[rr] ? 1 : 0;
    const float u = y ? z : -z;
    const float nll = softplus_f(-u);          // -log sigmoid(u)
    const float pu = sigmoid_f(u);
    const float qu = sigmoid_f(-u);
    const float mod = focal_mod(qu, gamma, igamma);
    if (valid) lsum += (double)nll + (double)(mod * nll);
    const float dbce = sigmoid_f(z) - (float)y;
    const float dfl_du = mod * (-gamma * pu * nll - qu);
    dls[t][s0 + n] = valid ? (dbce + (y ? dfl_du : -dfl_du)) * inv_qn : 0.f;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
  if (lane == 0) wsum[wave] = lsum;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) tot += wsum[w];
    loss_part[blockIdx.x] = tot;
  }

  // 3. partial key gradient: wave w takes queries 32 (w & 1) .. +31 and dims
  // 32 (w >> 1) .. +31 (DI = 64: waves 4-7 have no tile)
  const int tq = 32 * (wave & 1), i0 = 32 * (wave >> 1);
  if (i0 >= DI) return;
  f32x16 g = {};
  const int col = i0 + n;
#pragma unroll
  for (int ss = 0; ss < kChunk; ss += 16) {
    const int sk = ss + 8 * half;
    const Split3 a = split3(*(const f32x4*)&dls[tq + n][sk], *(const f32x4*)&dls[tq + n][sk + 4]);
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)ks[sk + 2 * e][col] | ((uint32_t)ks[sk + 2 * e + 1][col] << 16);
    g = mfma_split(a, __builtin_bit_cast(bf16x8, w), g);
  }
  float* out = Gp + (size_t)blockIdx.x * kQP * DI;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) out[(tq + acc_row(rr, half)) * DI + col] = g[rr];
}

// ---------------------------------------------------------------- 6 reduce
// GT[i][t] = sum over chunks of Gp[c][t][i]: a block owns 64 consecutive
// (t, i) elements; four thread slices sum every fourth chunk, then the slices
// are added in a fixed order.
__global__ __launch_bounds__(256) void freduce_kernel(int Q, int DI, int nchunks,
                                                      const float* __restrict__ Gp,
                                                      float* __restrict__ GT, int nloss,
                                                      double inv_qn,
                                                      const double* __restrict__ loss_part,
                                                      float* __restrict__ loss) {
  __shared__ float part[4][64];
  __shared__ double lred[256];
  const int slice = threadIdx.x >> 6, j = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + j;          // e = t * DI + i
  const size_t stride = (size_t)kQP * DI;
  float acc = 0.f;
  int c = slice;
  for (; c + 28 < nchunks; c += 32) {   // eight loads in flight, summed in chunk order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = Gp[(size_t)(c + 4 * u) * stride + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; c < nchunks; c += 4) acc += Gp[(size_t)c * stride + e];
  part[slice][j] = acc;
  __syncthreads();
  if (threadIdx.x < 64) {
    const float v = (part[0][j] + part[1][j]) + (part[2][j] + part[3][j]);
    const int t = e / DI, i = e % DI;
    GT[i * kQP + t] = t < Q ? v : 0.f;
  }
  // loss = (sum of the logits blocks' partials) / (Q N), in a fixed tree order
  if (blockIdx.x == 0) {
    double acc = 0.0;
    for (int b = threadIdx.x; b < nloss; b += 256) acc += loss_part[b];
    lred[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) lred[threadIdx.x] += lred[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) loss[0] = (float)(lred[0] * inv_qn);
  }
}

// ---------------------------------------------------------------- 7 dW
// grid: (ceil(D/512), HdI/(32 RT)); wave w takes 128 columns and RT 32-row
// tiles over them; contraction over the kQP padded queries:
// A[(h,i)][t] = gT[h][t] GT[i][t], B[d][t] = hT[d][t].  The wave loads its
// hidden-state fragments once for all RT tiles, and the next tile's A operand
// before the current tile's stores are issued (the counter of outstanding
// memory operations is in order: a load issued after the stores would wait
// for them), so each wave's products overlap its own stores.  RT = 4: one
// round of waves (two a SIMD) writes the whole gradient; with one tile a wave
// two rounds of four a SIMD took 38 us against 30.
template <int DI, int RT>
__global__ __launch_bounds__(256) void fdw_kernel(int D, const float* __restrict__ gT,
                                                  const float* __restrict__ GT,
                                                  const uint16_t* __restrict__ hT,
                                                  float* __restrict__ dW) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, half = lane >> 5;
  const int c0 = blockIdx.x * 512 + wave * 128;
  if (c0 >= D) return;
  bf16x8 bq[kQP / 16][4];   // [k step][column tile]
#pragma unroll
  for (int ks = 0; ks < kQP / 16; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bq[ks][j] = *(const bf16x8*)(hT + (size_t)(c0 + 32 * j + n) * kQP + 16 * ks + 8 * half);
  auto load_a = [&](int rt, f32x4 (&ap)[kQP / 16][2]) {
    const int row = (blockIdx.y * RT + rt) * 32 + n;   // (h, i) = (row / DI, row % DI)
    const float* ga = gT + (row / DI) * kQP;
    const float* Ga = GT + (row % DI) * kQP;
#pragma unroll
    for (int ks = 0; ks < kQP / 16; ++ks) {
      const int kk = 16 * ks + 8 * half;
      ap[ks][0] = *(const f32x4*)(ga + kk) * *(const f32x4*)(Ga + kk);
      ap[ks][1] = *(const f32x4*)(ga + kk + 4) * *(const f32x4*)(Ga + kk + 4);
    }
  };
  f32x4 ap[kQP / 16][2];
  load_a(0, ap);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x16 acc[4] = {};
#pragma unroll
    for (int ks = 0; ks < kQP / 16; ++ks) {
      const Split3 a = split3(ap[ks][0], ap[ks][1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma_split(a, bq[ks][j], acc[j]);
    }
    if (rt + 1 < RT) load_a(rt + 1, ap);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const size_t r = (size_t)(blockIdx.y * RT + rt) * 32 + acc_row(rr, half);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + 32 * j < D) __builtin_nontemporal_store(acc[j][rr], dW + r * D + c0 + 32 * j + n);
    }
  }
}

struct FocalWs {
  float* qp;
  float* gp;
  float* gT;
  float* qe;
  uint16_t* hT;
  float* Gp;
  float* GT;
  double* loss_part;
  size_t bytes;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// slices of D for the projection: each wave of a slice takes D / (4 KS)
// columns, a multiple of 32 (two bf16 MFMA steps; D % 128 == 0)
int proj_slices(int D) { return D % 1024 == 0 ? 8 : (D % 512 == 0 ? 4 : (D % 256 == 0 ? 2 : 1)); }
// slices of D for the gate rows: m KS with m in {4, 2, 1}, each wave's columns
// still a multiple of 32
int gate_slices(int D) {
  const int KS = proj_slices(D);   // <= 8, times at most 4: kMaxGateSlices
  const int steps = D / (4 * KS) / 32;   // 32-column steps of a W_q wave
  return KS * (steps % 4 == 0 ? 4 : (steps % 2 == 0 ? 2 : 1));
}

FocalWs carve(void* base, int Q, int N, int D, int H, int dI) {
  (void)Q;
  const int Np = (N + 7) & ~7;
  const size_t HdI = (size_t)H * dI;
  const int nchunks = (Np + kChunk - 1) / kChunk;
  const int nloss = nchunks;
  size_t off = 0;
  FocalWs w;
  auto take = [&](size_t bytes) {
    char* p = (char*)base + off;
    off += up256(bytes);
    return (void*)p;
  };
  w.qp = (float*)take((size_t)proj_slices(D) * kQP * HdI * 4);
  w.gp = (float*)take((size_t)gate_slices(D) * kQP * kQP * 4);
  w.gT = (float*)take((size_t)64 * kQP * 4);
  w.qe = (float*)take((size_t)kQP * dI * 4);
  w.hT = (uint16_t*)take((size_t)D * kQP * 2);
  w.Gp = (float*)take((size_t)nchunks * kQP * dI * 4);
  w.GT = (float*)take((size_t)dI * kQP * 4);
  w.loss_part = (double*)take((size_t)nloss * 8);
  w.bytes = off;
  return w;
}

}  // namespace

size_t focal_workspace_bytes(int Q, int N, int D, int H, int dI) {
  return carve(nullptr, Q, N, D, H, dI).bytes;
}

hipError_t launch_focal(int Q, int N, int D, int H, int dI, float gamma, const uint16_t* h,
                        const float* Wq, const float* Wg, float bias, const uint16_t* K,
                        const uint8_t* label, float* loss, float* dWq, void* ws, hipStream_t s) {
  const FocalWs w = carve(ws, Q, N, D, H, dI);
  const int Np = (N + 7) & ~7;
  const int HdI = H * dI;
  const int nchunks = (Np + kChunk - 1) / kChunk;
  const int nloss = nchunks;   // one loss partial per chunk
  const double inv_qn = 1.0 / ((double)Q * (double)N);
  hipError_t e;
#define FOCAL_CHECK()                        \
  do {                                       \
    e = hipGetLastError();                   \
    if (e != hipSuccess) return e;           \
  } while (0)
  const int KS = proj_slices(D), KSG = gate_slices(D);
  // gate blocks, then (H dI / 64 row groups) x KS W_q blocks (H dI % 64 == 0,
  // H <= 64: the gate rows are one group)
  const dim3 gproj((unsigned)(KSG + HdI / (32 * kProjTR) * KS));
  if (D / KS <= kProjSpan)   // a block's slice of h fits the LDS rows
    hipLaunchKernelGGL((fproj_kernel<kProjTR, true>), gproj, dim3(256), 0, s, Q, D, HdI, H, KS, KSG,
                       Wq, Wg, h, w.qp, w.gp);
  else
    hipLaunchKernelGGL((fproj_kernel<kProjTR, false>), gproj, dim3(256), 0, s, Q, D, HdI, H, KS,
                       KSG, Wq, Wg, h, w.qp, w.gp);
  FOCAL_CHECK();
  hipLaunchKernelGGL(fcollapse_kernel, dim3(kQP, (dI + 31) / 32), dim3(256), 0, s, Q, H, dI, KS,
                     KSG, w.qp, w.gp, w.gT, w.qe);
  FOCAL_CHECK();
  {
    const TransposeJob jh{h, w.hT, Q, D, kQP, 1};
    hipLaunchKernelGGL(ftranspose_kernel, dim3((D + 63) / 64), dim3(256), 0, s, jh, jh,
                       (D + 63) / 64);
  }
  FOCAL_CHECK();
  if (dI == 64)
    hipLaunchKernelGGL((flogits_grad_kernel<64>), dim3(nchunks), dim3(512), 0, s, Q, N, gamma, bias,
                       (float)inv_qn, K, w.qe, label, w.Gp, w.loss_part);
  else
    hipLaunchKernelGGL((flogits_grad_kernel<128>), dim3(nchunks), dim3(512), 0, s, Q, N, gamma,
                       bias, (float)inv_qn, K, w.qe, label, w.Gp, w.loss_part);
  FOCAL_CHECK();
  hipLaunchKernelGGL(freduce_kernel, dim3(kQP * dI / 64), dim3(256), 0, s, Q, dI, nchunks, w.Gp,
                     w.GT, nloss, inv_qn, w.loss_part, loss);
  FOCAL_CHECK();
  // HdI / 32 = 2 H or 4 H: four row tiles a wave when that divides it, else two
  if ((HdI / 32) % 4 == 0) {
    const dim3 gdw((D + 511) / 512, HdI / 128);
    if (dI == 64)
      hipLaunchKernelGGL((fdw_kernel<64, 4>), gdw, dim3(256), 0, s, D, w.gT, w.GT, w.hT, dWq);
    else
      hipLaunchKernelGGL((fdw_kernel<128, 4>), gdw, dim3(256), 0, s, D, w.gT, w.GT, w.hT, dWq);
  } else {
    const dim3 gdw((D + 511) / 512, HdI / 64);
    if (dI == 64)
      hipLaunchKernelGGL((fdw_kernel<64, 2>), gdw, dim3(256), 0, s, D, w.gT, w.GT, w.hT, dWq);
    else
      hipLaunchKernelGGL((fdw_kernel<128, 2>), gdw, dim3(256), 0, s, D, w.gT, w.GT, w.hT, dWq);
  }
  FOCAL_CHECK();
#undef FOCAL_CHECK
  return hipSuccess;
}

}  // namespace lsa
