// lsa_api.cpp -- C ABI of liblsa.so: host-side argument validation and
// dispatch to the gfx950 kernels.  Every check runs before any launch, so an
// invalid call returns an error without touching device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/lsa.h"
#include "lsa_launch.h"

namespace {

thread_local char g_err[512] = "";

lsa_status fail(lsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

lsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LSA_OK;
  return fail(LSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, st, ...)                      \
  do {                                              \
    if (!(cond)) return fail((st), __VA_ARGS__);    \
  } while (0)

}  // namespace

extern "C" {

const char* lsa_last_error(void) { return g_err; }

const char* lsa_version(void) { return "lsa-gfx950 0.1"; }

int lsa_trigger_due(int64_t decode_step, int tau) {
  if (tau <= 0 || decode_step < 0) return 0;
  return (decode_step % tau) == 0 ? 1 : 0;
}

// ---------------------------------------------------------------- projection

namespace {

// Checks shared by the two projection entry points; fills everything but the
// weights.
lsa_status project_common(const char* fn, int L, int B, int D, int H, int dI, const uint16_t* h,
                          int64_t h_layer_stride, uint16_t* q, float* g, lsa::ProjectArgs& a) {
  REQUIRE(L >= 1 && L <= LSA_MAX_LAYERS, LSA_E_SHAPE, "%s: L=%d not in [1,%d]", fn, L,
          LSA_MAX_LAYERS);
  REQUIRE(B >= 1, LSA_E_SHAPE, "%s: B=%d < 1", fn, B);
  REQUIRE(D >= 64 && D <= 65536 && D % 64 == 0, LSA_E_SHAPE,
          "%s: D=%d not a multiple of 64 in [64,65536]", fn, D);
  REQUIRE((int64_t)B * D * 2 < ((int64_t)1 << 31), LSA_E_SHAPE,
          "%s: B*D*2 must stay below 2^31 bytes", fn);
  REQUIRE(H >= 1 && H <= LSA_MAX_HEADS, LSA_E_SHAPE, "%s: H=%d not in [1,64]", fn, H);
  REQUIRE(dI == 64 || dI == 128, LSA_E_SHAPE, "%s: dI=%d not 64 or 128", fn, dI);
  REQUIRE(h_layer_stride >= 0, LSA_E_ARG, "%s: negative h_layer_stride", fn);
  REQUIRE(h && q && g, LSA_E_ARG, "%s: null pointer argument", fn);
  REQUIRE(aligned16(h) && aligned16(q) && (h_layer_stride % 8) == 0, LSA_E_ARG,
          "%s: h/q must be 16-byte aligned (stride multiple of 8)", fn);
  a = lsa::ProjectArgs{};
  a.h = h;
  a.h_layer_stride = h_layer_stride;
  a.q = q;
  a.g = g;
  a.L = L;
  a.B = B;
  a.D = D;
  a.H = H;
  a.dI = dI;
  return LSA_OK;
}

}  // namespace

lsa_status lsa_project_query(int L, int B, int D, int H, int dI, const uint16_t* h,
                             int64_t h_layer_stride, const uint16_t* const* Wq,
                             const uint16_t* const* Wg, uint16_t* q, float* g,
                             hipStream_t stream) {
  lsa::ProjectArgs a;
  const lsa_status st =
      project_common("lsa_project_query", L, B, D, H, dI, h, h_layer_stride, q, g, a);
  if (st != LSA_OK) return st;
  REQUIRE(Wq && Wg, LSA_E_ARG, "lsa_project_query: null weight array");
  for (int l = 0; l < L; ++l) {
    REQUIRE(Wq[l] && Wg[l], LSA_E_ARG, "lsa_project_query: null weight pointer for layer %d", l);
    REQUIRE(aligned16(Wq[l]) && aligned16(Wg[l]), LSA_E_ARG,
            "lsa_project_query: weights of layer %d not 16-byte aligned", l);
    a.Wq[l] = Wq[l];
    a.Wg[l] = Wg[l];
  }
  return hip_status(lsa::launch_project(a, stream), "lsa_project_query launch");
}

size_t lsa_query_weights_packed_bytes(int H, int dI, int D) {
  if (H < 1 || H > LSA_MAX_HEADS || (dI != 64 && dI != 128) || D < 64 || D > 65536 || D % 64)
    return 0;
  return lsa::packed_weights_bytes(H, dI, D);
}

lsa_status lsa_pack_query_weights(int H, int dI, int D, const uint16_t* Wq, const uint16_t* Wg,
                                  void* packed, hipStream_t stream) {
  REQUIRE(D >= 64 && D <= 65536 && D % 64 == 0, LSA_E_SHAPE,
          "lsa_pack_query_weights: D=%d not a multiple of 64 in [64,65536]", D);
  REQUIRE(H >= 1 && H <= LSA_MAX_HEADS, LSA_E_SHAPE, "lsa_pack_query_weights: H=%d not in [1,64]",
          H);
  REQUIRE(dI == 64 || dI == 128, LSA_E_SHAPE, "lsa_pack_query_weights: dI=%d not 64 or 128", dI);
  REQUIRE(Wq && Wg && packed, LSA_E_ARG, "lsa_pack_query_weights: null pointer argument");
  REQUIRE(aligned16(Wq) && aligned16(Wg) && aligned16(packed), LSA_E_ARG,
          "lsa_pack_query_weights: pointers must be 16-byte aligned");
  return hip_status(lsa::launch_pack_weights(H, dI, D, Wq, Wg, packed, stream),
                    "lsa_pack_query_weights launch");
}

lsa_status lsa_project_query_packed(int L, int B, int D, int H, int dI, const uint16_t* h,
                                    int64_t h_layer_stride, const void* const* packed,
                                    uint16_t* q, float* g, hipStream_t stream) {
  lsa::ProjectArgs a;
  const lsa_status st =
      project_common("lsa_project_query_packed", L, B, D, H, dI, h, h_layer_stride, q, g, a);
  if (st != LSA_OK) return st;
  REQUIRE(packed, LSA_E_ARG, "lsa_project_query_packed: null weight array");
  for (int l = 0; l < L; ++l) {
    REQUIRE(packed[l] && aligned16(packed[l]), LSA_E_ARG,
            "lsa_project_query_packed: packed weights of layer %d null or not 16-byte aligned", l);
    a.Wp[l] = packed[l];
  }
  return hip_status(lsa::launch_project(a, stream), "lsa_project_query_packed launch");
}

// --------------------------------------------------------------------- score

lsa_status lsa_score_strided(int L, int B, int N, int64_t entry_stride, int H, int dI,
                             lsa_key_dtype kdt, const void* const* keys,
                             const float* const* key_scale, const uint16_t* q, const float* g,
                             const float* bias, uint32_t* sel_mask, int32_t* cand_idx,
                             float* cand_z, int32_t* cand_count, float* z_opt, float* I_opt,
                             hipStream_t stream) {
  REQUIRE(kdt == LSA_KEY_BF16 || kdt == LSA_KEY_FP8_E4M3, LSA_E_DTYPE,
          "lsa_score: unknown key dtype %d", (int)kdt);
  REQUIRE(L >= 1 && L <= LSA_MAX_LAYERS, LSA_E_SHAPE, "lsa_score: L=%d not in [1,%d]", L,
          LSA_MAX_LAYERS);
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "lsa_score: B=%d not in [1,65535]", B);
  REQUIRE(N >= 0 && N <= (1 << 24), LSA_E_SHAPE, "lsa_score: N=%d not in [0,2^24]", N);
  REQUIRE(H >= 1 && H <= LSA_MAX_HEADS, LSA_E_SHAPE, "lsa_score: H=%d not in [1,64]", H);
  REQUIRE(dI == 64 || dI == 128, LSA_E_SHAPE, "lsa_score: dI=%d not 64 or 128", dI);
  REQUIRE((int64_t)N * dI * (kdt == LSA_KEY_BF16 ? 2 : 1) < ((int64_t)1 << 31), LSA_E_SHAPE,
          "lsa_score: keys of one (layer, request) must stay below 2^31 bytes (N=%d, dI=%d)", N,
          dI);
  REQUIRE(entry_stride >= N && entry_stride <= ((int64_t)1 << 40), LSA_E_SHAPE,
          "lsa_score: entry_stride=%lld must be at least N=%d", (long long)entry_stride, N);
  REQUIRE(bias && ((uintptr_t)bias & 3u) == 0, LSA_E_ARG,
          "lsa_score: bias must be a 4-byte aligned device array of L floats");
  if (N == 0) return LSA_OK;   // nothing to score; outputs are empty
  REQUIRE(keys && q && g && sel_mask && cand_idx && cand_z && cand_count, LSA_E_ARG,
          "lsa_score: null pointer argument");
  REQUIRE(kdt == LSA_KEY_BF16 || key_scale, LSA_E_ARG, "lsa_score: e4m3 keys need key_scale");
  REQUIRE(aligned16(q), LSA_E_ARG, "lsa_score: q must be 16-byte aligned");
  lsa::ScoreArgs a{};
  for (int l = 0; l < L; ++l) {
    REQUIRE(keys[l], LSA_E_ARG, "lsa_score: null key pointer for layer %d", l);
    REQUIRE(aligned16(keys[l]), LSA_E_ARG, "lsa_score: keys of layer %d not 16-byte aligned", l);
    a.keys[l] = keys[l];
    if (kdt == LSA_KEY_FP8_E4M3) {
      REQUIRE(key_scale[l], LSA_E_ARG, "lsa_score: null key_scale pointer for layer %d", l);
      a.scale[l] = key_scale[l];
    }
  }
  a.bias = bias;
  a.q = q;
  a.g = g;
  a.mask = sel_mask;
  a.cand_idx = cand_idx;
  a.cand_z = cand_z;
  a.cand_count = cand_count;
  a.z = z_opt;
  a.I = I_opt;
  a.stride = entry_stride;
  a.L = L;
  a.B = B;
  a.N = N;
  a.H = H;
  a.W = (N + 31) / 32;
  a.nchunks = (N + LSA_CAND_CHUNK - 1) / LSA_CAND_CHUNK;
  return hip_status(lsa::launch_score(dI, kdt, a, stream), "lsa_score launch");
}

lsa_status lsa_score(int L, int B, int N, int H, int dI, lsa_key_dtype kdt,
                     const void* const* keys, const float* const* key_scale, const uint16_t* q,
                     const float* g, const float* bias, uint32_t* sel_mask, int32_t* cand_idx,
                     float* cand_z, int32_t* cand_count, float* z_opt, float* I_opt,
                     hipStream_t stream) {
  return lsa_score_strided(L, B, N, N, H, dI, kdt, keys, key_scale, q, g, bias, sel_mask,
                           cand_idx, cand_z, cand_count, z_opt, I_opt, stream);
}

// ------------------------------------------------------------- cache append

lsa_status lsa_append_rows(int B, int n, int row_bytes, const void* src, int64_t src_stride,
                           void* dst, int64_t dst_stride, int64_t dst_start,
                           hipStream_t stream) {
  const char* fn = "lsa_append_rows";
  REQUIRE(B >= 1 && B <= 65535 && n >= 0, LSA_E_SHAPE, "%s: B=%d, n=%d", fn, B, n);
  REQUIRE(row_bytes > 0 && row_bytes % 4 == 0, LSA_E_ARG,
          "%s: row_bytes=%d not a positive multiple of 4", fn, row_bytes);
  REQUIRE(src_stride >= n && dst_start >= 0 && dst_stride >= dst_start + n, LSA_E_SHAPE,
          "%s: strides must hold the rows (src_stride %lld, n %d, dst_start %lld, dst_stride "
          "%lld)", fn, (long long)src_stride, n, (long long)dst_start, (long long)dst_stride);
  if (n == 0) return LSA_OK;
  REQUIRE(src && dst, LSA_E_ARG, "%s: null pointer argument", fn);
  REQUIRE(((uintptr_t)src & 3u) == 0 && ((uintptr_t)dst & 3u) == 0, LSA_E_ARG,
          "%s: src and dst must be 4-byte aligned", fn);
  return hip_status(lsa::launch_append_rows(B, n, row_bytes, src, src_stride, dst, dst_stride,
                                            dst_start, stream),
                    "lsa_append_rows launch");
}

// ----------------------------------------------------------- select/compact

lsa_status lsa_select_or_compact(int B, int N, const int32_t* cand_idx, const float* cand_z,
                                 const int32_t* cand_count, int cap, int32_t* surv_idx,
                                 float* surv_z, int32_t* surv_count, hipStream_t stream) {
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "lsa_select_or_compact: B=%d not in [1,65535]", B);
  REQUIRE(N >= 0 && N <= (1 << 24), LSA_E_SHAPE, "lsa_select_or_compact: N=%d not in [0,2^24]", N);
  REQUIRE(cap >= 0, LSA_E_ARG, "lsa_select_or_compact: cap=%d < 0", cap);
  REQUIRE(surv_count, LSA_E_ARG, "lsa_select_or_compact: null surv_count");
  REQUIRE(N == 0 || (cand_idx && cand_z && cand_count), LSA_E_ARG,
          "lsa_select_or_compact: null candidate list");
  REQUIRE(cap == 0 || (surv_idx && surv_z), LSA_E_ARG,
          "lsa_select_or_compact: null survivor output with cap > 0");
  const int nchunks = (N + LSA_CAND_CHUNK - 1) / LSA_CAND_CHUNK;
  return hip_status(lsa::launch_select(B, nchunks, cand_idx, cand_z, cand_count, cap, surv_idx,
                                       surv_z, surv_count, stream),
                    "lsa_select_or_compact launch");
}

size_t lsa_select_or_compact_masks_workspace_bytes(int B, int N) {
  if (B < 1 || N < 0) return 0;
  return lsa::select_masks_workspace_bytes(B, N);
}

lsa_status lsa_select_or_compact_masks(int L, int B, int N, const uint32_t* sel_mask,
                                       const float* z, int cap, int32_t* surv_idx, float* surv_z,
                                       int32_t* surv_count, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  const char* fn = "lsa_select_or_compact_masks";
  REQUIRE(L >= 1 && L <= LSA_MAX_LAYERS, LSA_E_SHAPE, "%s: L=%d not in [1,%d]", fn, L,
          LSA_MAX_LAYERS);
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "%s: B=%d not in [1,65535]", fn, B);
  REQUIRE(N >= 0 && N <= (1 << 24), LSA_E_SHAPE, "%s: N=%d not in [0,2^24]", fn, N);
  REQUIRE(cap >= 0, LSA_E_ARG, "%s: cap=%d < 0", fn, cap);
  REQUIRE(surv_count, LSA_E_ARG, "%s: null surv_count", fn);
  REQUIRE(N == 0 || (sel_mask && z), LSA_E_ARG, "%s: null mask or logits", fn);
  REQUIRE(((uintptr_t)sel_mask & 3u) == 0 && ((uintptr_t)z & 3u) == 0, LSA_E_ARG,
          "%s: mask and logits must be 4-byte aligned", fn);
  REQUIRE(cap == 0 || (surv_idx && surv_z), LSA_E_ARG, "%s: null survivor output with cap > 0",
          fn);
  const size_t need = lsa::select_masks_workspace_bytes(B, N);
  REQUIRE(need == 0 || (ws && ws_bytes >= need && ((uintptr_t)ws & 15) == 0), LSA_E_WORKSPACE,
          "%s: workspace of %zu bytes (16-byte aligned) needed, got %zu", fn, need,
          ws ? ws_bytes : (size_t)0);
  return hip_status(lsa::launch_select_masks(L, B, N, sel_mask, z, cap, surv_idx, surv_z,
                                             surv_count, ws, stream),
                    "lsa_select_or_compact_masks launch");
}

// --------------------------------------------------------------------- top-k

size_t lsa_topk_workspace_bytes(int B, int cap, int k) {
  if (B < 1 || cap < 0 || k < 0) return 0;
  return lsa::topk_workspace_bytes(B, cap, k);
}

lsa_status lsa_topk(int B, int cap, int k, const int32_t* surv_idx, const float* surv_z,
                    const int32_t* surv_count, int32_t* topk_idx, int32_t* topk_count, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "lsa_topk: B=%d not in [1,65535]", B);
  REQUIRE(cap >= 0 && k >= 0, LSA_E_ARG, "lsa_topk: negative cap or k");
  REQUIRE(surv_count && topk_count, LSA_E_ARG, "lsa_topk: null count pointer");
  REQUIRE(cap == 0 || (surv_idx && surv_z), LSA_E_ARG, "lsa_topk: null survivor input");
  REQUIRE(k == 0 || topk_idx, LSA_E_ARG, "lsa_topk: null topk_idx with k > 0");
  const size_t need = lsa::topk_workspace_bytes(B, cap, k);
  REQUIRE(need == 0 || (ws && ws_bytes >= need && ((uintptr_t)ws & 15) == 0), LSA_E_WORKSPACE,
          "lsa_topk: workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
          ws ? ws_bytes : (size_t)0);
  return hip_status(lsa::launch_topk(B, cap, k, surv_idx, surv_z, surv_count, topk_idx,
                                     topk_count, ws, stream),
                    "lsa_topk launch");
}

lsa_status lsa_topk_noalloc(int B, int cap, int k, const int32_t* surv_idx,
                            const float* surv_z, const int32_t* surv_count, int32_t* topk_idx,
                            int32_t* topk_count, hipStream_t stream) {
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "lsa_topk_noalloc: B=%d not in [1,65535]", B);
  REQUIRE(cap >= 0 && k >= 0, LSA_E_ARG, "lsa_topk_noalloc: negative cap or k");
  REQUIRE(surv_count && topk_count, LSA_E_ARG, "lsa_topk_noalloc: null count pointer");
  REQUIRE(cap == 0 || (surv_idx && surv_z), LSA_E_ARG, "lsa_topk_noalloc: null survivor input");
  REQUIRE(k == 0 || topk_idx, LSA_E_ARG, "lsa_topk_noalloc: null topk_idx with k > 0");
  const size_t need = lsa::topk_workspace_bytes(B, cap, k);
  REQUIRE(need <= (size_t)LSA_TOPK_NOALLOC_MAX_BYTES, LSA_E_SHAPE,
          "lsa_topk_noalloc: B=%d, cap=%d, k=%d need %zu scratch bytes, more than the %d the "
          "library holds (use lsa_topk with a workspace)",
          B, cap, k, need, (int)LSA_TOPK_NOALLOC_MAX_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    const lsa_status st = hip_status(lsa::topk_scratch_address(&ws), "lsa_topk_noalloc scratch");
    if (st != LSA_OK) return st;
  }
  return hip_status(lsa::launch_topk(B, cap, k, surv_idx, surv_z, surv_count, topk_idx,
                                     topk_count, ws, stream),
                    "lsa_topk_noalloc launch");
}

// ------------------------------------------------- fine-grained score

lsa_status lsa_lightning_score(int B, int N, int cap, int H, int dI, lsa_key_dtype kdt,
                               const void* keys, const float* key_scale, const uint16_t* q,
                               const float* w, const int32_t* surv_idx,
                               const int32_t* surv_count, float* score, hipStream_t stream) {
  const char* fn = "lsa_lightning_score";
  REQUIRE(kdt == LSA_KEY_BF16 || kdt == LSA_KEY_FP8_E4M3, LSA_E_DTYPE, "%s: unknown key dtype %d",
          fn, (int)kdt);
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "%s: B=%d not in [1,65535]", fn, B);
  REQUIRE(N >= 0 && N <= (1 << 24) && cap >= 0, LSA_E_SHAPE, "%s: N=%d, cap=%d", fn, N, cap);
  REQUIRE(H >= 16 && H <= 64 && H % 16 == 0, LSA_E_SHAPE,
          "%s: H=%d not a multiple of 16 in [16,64]", fn, H);
  REQUIRE(dI == 64 || dI == 128, LSA_E_SHAPE, "%s: dI=%d not 64 or 128", fn, dI);
  REQUIRE((int64_t)N * dI * (kdt == LSA_KEY_BF16 ? 2 : 1) < ((int64_t)1 << 31), LSA_E_SHAPE,
          "%s: keys of one request must stay below 2^31 bytes", fn);
  REQUIRE(surv_count, LSA_E_ARG, "%s: null surv_count", fn);
  if (cap == 0) return LSA_OK;
  REQUIRE(keys && q && w && surv_idx && score, LSA_E_ARG, "%s: null pointer argument", fn);
  REQUIRE(kdt == LSA_KEY_BF16 || key_scale, LSA_E_ARG, "%s: e4m3 keys need key_scale", fn);
  REQUIRE(aligned16(keys) && aligned16(q) && ((uintptr_t)w & 3u) == 0, LSA_E_ARG,
          "%s: keys and q must be 16-byte aligned, w 4-byte aligned", fn);
  return hip_status(lsa::launch_lightning(B, N, cap, H, dI, kdt, keys, key_scale, q, w,
                                          surv_idx, surv_count, score, stream),
                    "lsa_lightning_score launch");
}

// -------------------------------------------------------------------- gather

lsa_status lsa_gather_hot(int B, int N, int k, int row_bytes, const void* pool,
                          const int32_t* idx, void* hot, hipStream_t stream) {
  REQUIRE(B >= 1 && N >= 0 && k >= 0, LSA_E_SHAPE, "lsa_gather_hot: bad B/N/k (%d,%d,%d)", B, N, k);
  REQUIRE(row_bytes > 0 && row_bytes % 16 == 0, LSA_E_ARG,
          "lsa_gather_hot: row_bytes=%d not a positive multiple of 16", row_bytes);
  if (k == 0) return LSA_OK;
  REQUIRE(idx && hot && (N == 0 || pool), LSA_E_ARG, "lsa_gather_hot: null pointer argument");
  REQUIRE(aligned16(hot) && (N == 0 || aligned16(pool)), LSA_E_ARG,
          "lsa_gather_hot: pool/hot not 16-byte aligned");
  return hip_status(lsa::launch_gather(B, N, k, row_bytes, pool, idx, hot, stream),
                    "lsa_gather_hot launch");
}

// ------------------------------------------------------------ core attention

size_t lsa_sparse_attention_workspace_bytes(int B, int H, int D, int k, int W) {
  if (B < 1 || H < 16 || H % 16 || D != LSA_ATT_ROW || k < 0 || W < 0) return 0;
  return lsa::attention_workspace_bytes(B, H, D, k, W);
}

lsa_status lsa_sparse_attention(int B, int H, int D, int k, int W, float scale,
                                const uint16_t* q, const uint16_t* hot, const int32_t* hot_count,
                                const uint16_t* win, const int32_t* win_count, float* out,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "lsa_sparse_attention";
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "%s: B=%d not in [1,65535]", fn, B);
  REQUIRE(H >= 16 && H <= 1024 && H % 16 == 0, LSA_E_SHAPE,
          "%s: H=%d not a multiple of 16 in [16,1024]", fn, H);
  REQUIRE(D == LSA_ATT_ROW, LSA_E_SHAPE, "%s: D=%d, rows must be %d wide", fn, D, LSA_ATT_ROW);
  REQUIRE(k >= 0 && W >= 0 && (int64_t)k + W <= (1 << 20), LSA_E_SHAPE,
          "%s: k=%d, W=%d: need k, W >= 0 and k + W <= 2^20", fn, k, W);
  REQUIRE(scale == scale && scale - scale == 0.f, LSA_E_ARG, "%s: scale not finite", fn);
  REQUIRE(q && out && (k == 0 || hot) && (W == 0 || win), LSA_E_ARG, "%s: null pointer argument",
          fn);
  REQUIRE(aligned16(q) && aligned16(out) && (k == 0 || aligned16(hot)) &&
              (W == 0 || aligned16(win)),
          LSA_E_ARG, "%s: q, hot, win and out must be 16-byte aligned", fn);
  const size_t need = lsa::attention_workspace_bytes(B, H, D, k, W);
  REQUIRE(need == 0 || (ws && ws_bytes >= need && ((uintptr_t)ws & 255) == 0), LSA_E_WORKSPACE,
          "%s: workspace of %zu bytes (256-byte aligned) needed, got %zu", fn, need,
          ws ? ws_bytes : (size_t)0);
  return hip_status(lsa::launch_attention(B, H, k, W, scale, q, hot, hot_count, win, win_count,
                                          out, ws, stream),
                    "lsa_sparse_attention launch");
}

// ------------------------------------------------------- cold-pool fetch

namespace {

// The device-side address of the cold pool: pinned host memory is read in
// place through its device mapping; device memory is taken as it is.  Pageable
// host memory (or anything HIP does not know) is refused.
lsa_status cold_pool_address(const void* cold, const void** dev) {
  hipPointerAttribute_t at;
  hipError_t e = hipPointerGetAttributes(&at, cold);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(LSA_E_ARG, "lsa_fetch_survivors: cold pool is neither pinned host nor device "
                "memory (%s)", hipGetErrorString(e));
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *dev = cold;
    return LSA_OK;
  }
  if (at.type != hipMemoryTypeHost)
    return fail(LSA_E_ARG, "lsa_fetch_survivors: cold pool is pageable host memory; allocate "
                "it pinned (hipHostMalloc)");
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, const_cast<void*>(cold), 0);
  if (e != hipSuccess || !d) {
    (void)hipGetLastError();
    return fail(LSA_E_ARG, "lsa_fetch_survivors: cold pool host memory is not pinned and "
                "mapped (%s)", hipGetErrorString(e));
  }
  *dev = d;
  return LSA_OK;
}

}  // namespace

size_t lsa_fetch_workspace_bytes(int B, int N, int cap) {
  if (B < 1 || N < 0 || cap < 0) return 0;
  return lsa::fetch_workspace_bytes(B, N, cap);
}

lsa_status lsa_resident_reset(int B, int N, int S, int32_t* slot_of, int32_t* entry_of,
                              hipStream_t stream) {
  REQUIRE(B >= 1 && B <= 65535 && N >= 0 && S >= 0, LSA_E_SHAPE,
          "lsa_resident_reset: bad B/N/S (%d,%d,%d)", B, N, S);
  REQUIRE((N == 0 || slot_of) && (S == 0 || entry_of), LSA_E_ARG,
          "lsa_resident_reset: null table");
  return hip_status(lsa::launch_resident_reset(B, N, S, slot_of, entry_of, stream),
                    "lsa_resident_reset launch");
}

lsa_status lsa_fetch_survivors(int B, int N, int S, int row_bytes, const void* cold_pool,
                               int cap, const int32_t* surv_idx, const int32_t* surv_count,
                               int32_t* slot_of, int32_t* entry_of, void* rows,
                               int32_t* fetch_count, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  REQUIRE(B >= 1 && B <= 65535, LSA_E_SHAPE, "lsa_fetch_survivors: B=%d not in [1,65535]", B);
  REQUIRE(N >= 0 && N <= (1 << 24) && cap >= 0 && S >= 0 && S <= (1 << 24), LSA_E_SHAPE,
          "lsa_fetch_survivors: bad N/cap/S (%d,%d,%d)", N, cap, S);
  REQUIRE(row_bytes > 0 && row_bytes % 16 == 0, LSA_E_ARG,
          "lsa_fetch_survivors: row_bytes=%d not a positive multiple of 16", row_bytes);
  {
    const int64_t per = std::min(std::min(cap, N), S);
    REQUIRE((int64_t)B * per < ((int64_t)1 << 31), LSA_E_SHAPE,
            "lsa_fetch_survivors: B*min(cap, N, S) must stay below 2^31 rows");
  }
  REQUIRE(surv_count && fetch_count, LSA_E_ARG, "lsa_fetch_survivors: null count pointer");
  REQUIRE(cap == 0 || surv_idx, LSA_E_ARG, "lsa_fetch_survivors: null surv_idx with cap > 0");
  REQUIRE((N == 0 || (slot_of && cold_pool)) && (S == 0 || (entry_of && rows)), LSA_E_ARG,
          "lsa_fetch_survivors: null table, rows or cold pool");
  REQUIRE((N == 0 || aligned16(cold_pool)) && (S == 0 || aligned16(rows)), LSA_E_ARG,
          "lsa_fetch_survivors: cold pool/rows not 16-byte aligned");
  const size_t need = lsa::fetch_workspace_bytes(B, N, cap);
  REQUIRE(need == 0 || (ws && ws_bytes >= need && ((uintptr_t)ws & 15) == 0), LSA_E_WORKSPACE,
          "lsa_fetch_survivors: workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
          ws ? ws_bytes : (size_t)0);
  const void* cold = nullptr;
  if (N > 0) {
    lsa_status st = cold_pool_address(cold_pool, &cold);
    if (st != LSA_OK) return st;
  }
  return hip_status(lsa::launch_fetch(B, N, S, row_bytes, cold, cap, surv_idx, surv_count,
                                      slot_of, entry_of, rows, fetch_count, ws, stream),
                    "lsa_fetch_survivors launch");
}

lsa_status lsa_gather_resident(int B, int N, int S, int k, int row_bytes, const void* rows,
                               const int32_t* slot_of, const int32_t* idx, void* hot,
                               hipStream_t stream) {
  REQUIRE(B >= 1 && N >= 0 && S >= 0 && k >= 0, LSA_E_SHAPE,
          "lsa_gather_resident: bad B/N/S/k (%d,%d,%d,%d)", B, N, S, k);
  REQUIRE(row_bytes > 0 && row_bytes % 16 == 0, LSA_E_ARG,
          "lsa_gather_resident: row_bytes=%d not a positive multiple of 16", row_bytes);
  if (k == 0) return LSA_OK;
  REQUIRE(idx && hot && (N == 0 || slot_of) && (S == 0 || rows), LSA_E_ARG,
          "lsa_gather_resident: null pointer argument");
  REQUIRE(aligned16(hot) && (S == 0 || aligned16(rows)), LSA_E_ARG,
          "lsa_gather_resident: rows/hot not 16-byte aligned");
  return hip_status(lsa::launch_gather_resident(B, N, S, k, row_bytes, rows, slot_of, idx, hot,
                                                stream),
                    "lsa_gather_resident launch");
}

// -------------------------------------------------------- label / loss calls

size_t lsa_label_vote_workspace_bytes(int Q, int L, int N) {
  if (Q < 1 || L < 1 || N < 1) return 0;
  return (size_t)Q * (size_t)L * (size_t)((N + 31) / 32) * sizeof(uint32_t);
}

lsa_status lsa_label_vote(int Q, int L, int N, float top_p, int theta, const float* logits,
                          uint32_t* layer_mask_opt, uint8_t* count, uint8_t* label, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  REQUIRE(Q >= 1, LSA_E_SHAPE, "lsa_label_vote: Q=%d < 1", Q);
  REQUIRE(L >= 1 && L <= LSA_MAX_VOTE_LAYERS, LSA_E_SHAPE, "lsa_label_vote: L=%d not in [1,%d]", L,
          LSA_MAX_VOTE_LAYERS);
  REQUIRE(N >= 1 && N <= 65536, LSA_E_SHAPE, "lsa_label_vote: N=%d not in [1,65536]", N);
  REQUIRE((int64_t)Q * L <= 0x7FFFFFFF, LSA_E_SHAPE, "lsa_label_vote: Q*L=%lld rows above 2^31-1",
          (long long)Q * L);
  REQUIRE(top_p > 0.f && top_p <= 1.f, LSA_E_ARG, "lsa_label_vote: top_p=%g not in (0,1]",
          (double)top_p);
  REQUIRE(theta >= 0, LSA_E_ARG, "lsa_label_vote: theta=%d < 0", theta);
  REQUIRE(logits && count && label, LSA_E_ARG, "lsa_label_vote: null logits/count/label");
  REQUIRE(aligned16(logits) && aligned16(count) && aligned16(label), LSA_E_ARG,
          "lsa_label_vote: logits, count and label must be 16-byte aligned");
  uint32_t* mask = layer_mask_opt;
  if (!mask) {
    const size_t need = lsa_label_vote_workspace_bytes(Q, L, N);
    REQUIRE(ws && ws_bytes >= need, LSA_E_WORKSPACE,
            "lsa_label_vote: workspace of %zu bytes needed without layer_mask_opt (got %zu)", need,
            ws ? ws_bytes : (size_t)0);
    mask = (uint32_t*)ws;
  }
  return hip_status(lsa::launch_label_vote(Q, L, N, top_p, theta, logits, mask, count, label,
                                           stream),
                    "lsa_label_vote");
}

size_t lsa_focal_bce_grad_workspace_bytes(int Q, int N, int D, int H, int dI) {
  if (Q < 1 || Q > 64 || N < 1 || N > 4000000 || D < 128 || D > 16384 || D % 128 || H < 1 ||
      H > 64 || (dI != 64 && dI != 128))
    return 0;
  return lsa::focal_workspace_bytes(Q, N, D, H, dI);
}

lsa_status lsa_focal_bce_grad(int Q, int N, int D, int H, int dI, float gamma,
                              const uint16_t* h, const float* Wq, const float* Wg, float bias,
                              const uint16_t* K, const uint8_t* label, float* loss, float* dWq,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(Q >= 1 && Q <= 64, LSA_E_SHAPE, "lsa_focal_bce_grad: Q=%d not in [1,64]", Q);
  REQUIRE(N >= 1 && N <= 4000000, LSA_E_SHAPE, "lsa_focal_bce_grad: N=%d not in [1,4000000]", N);
  REQUIRE(D >= 128 && D <= 16384 && D % 128 == 0, LSA_E_SHAPE,
          "lsa_focal_bce_grad: D=%d not a multiple of 128 in [128,16384]", D);
  REQUIRE(H >= 1 && H <= 64, LSA_E_SHAPE, "lsa_focal_bce_grad: H=%d not in [1,64]", H);
  REQUIRE(dI == 64 || dI == 128, LSA_E_SHAPE, "lsa_focal_bce_grad: dI=%d not 64 or 128", dI);
  REQUIRE(gamma >= 0.f && gamma <= 16.f, LSA_E_ARG, "lsa_focal_bce_grad: gamma=%g not in [0,16]",
          (double)gamma);
  REQUIRE(bias == bias && bias - bias == 0.f, LSA_E_ARG, "lsa_focal_bce_grad: bias not finite");
  REQUIRE(h && Wq && Wg && K && label && loss && dWq, LSA_E_ARG,
          "lsa_focal_bce_grad: null input or output pointer");
  REQUIRE(aligned16(Wq) && aligned16(Wg) && aligned16(dWq), LSA_E_ARG,
          "lsa_focal_bce_grad: Wq, Wg and dWq must be 16-byte aligned");
  REQUIRE(aligned16(h) && ((uintptr_t)K & 7u) == 0, LSA_E_ARG,
          "lsa_focal_bce_grad: h must be 16-byte and K 8-byte aligned");
  const size_t need = lsa::focal_workspace_bytes(Q, N, D, H, dI);
  REQUIRE(ws && ws_bytes >= need && ((uintptr_t)ws & 255u) == 0, LSA_E_WORKSPACE,
          "lsa_focal_bce_grad: workspace of %zu bytes, 256-byte aligned, needed (got %zu)", need,
          ws ? ws_bytes : (size_t)0);
  return hip_status(lsa::launch_focal(Q, N, D, H, dI, gamma, h, Wq, Wg, bias, K, label, loss, dWq,
                                      ws, stream),
                    "lsa_focal_bce_grad");
}

}  // extern "C"
