// lsa_launch.h -- internal host-side launchers (one per kernel family).  The
// C ABI in lsa_api.cpp validates arguments and then calls these.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/lsa.h"

namespace lsa {

struct ScoreArgs {
  const void* keys[LSA_MAX_LAYERS];
  const float* scale[LSA_MAX_LAYERS];
  const float* bias;       // device fp32 [L]
  const uint16_t* q;
  const float* g;
  uint32_t* mask;          // [L][B][W]
  int32_t* cand_idx;       // [B][nchunks][LSA_CAND_CHUNK]
  float* cand_z;           // [B][nchunks][LSA_CAND_CHUNK]
  int32_t* cand_count;     // [B][nchunks]
  float* z;                // [L][B][N] or null
  float* I;                // [L][B][N] or null
  int64_t stride;          // entries between two requests in keys / scales (>= N)
  int L, B, N, H, W;       // W = ceil(N / 32)
  int nchunks;             // ceil(N / LSA_CAND_CHUNK)
  int pairs;               // two-chunk blocks per request (set by the launcher)
};

hipError_t launch_score(int dI, lsa_key_dtype kdt, const ScoreArgs& a, hipStream_t s);

struct ProjectArgs {
  const uint16_t* Wq[LSA_MAX_LAYERS];
  const uint16_t* Wg[LSA_MAX_LAYERS];
  const void* Wp[LSA_MAX_LAYERS];   // packed weights (lsa_pack_query_weights) or null
  const uint16_t* h;
  int64_t h_layer_stride;
  uint16_t* q;
  float* g;
  int L, B, D, H, dI;
};

hipError_t launch_project(const ProjectArgs& a, hipStream_t s);   // packed when a.Wp[0] is set
size_t packed_weights_bytes(int H, int dI, int D);
hipError_t launch_pack_weights(int H, int dI, int D, const uint16_t* Wq, const uint16_t* Wg,
                               void* packed, hipStream_t s);

// Compute units of the current device (queried once per device).
int device_cu_count();

hipError_t launch_select(int B, int nchunks, const int32_t* cand_idx, const float* cand_z,
                         const int32_t* cand_count, int cap, int32_t* surv_idx,
                         float* surv_z, int32_t* surv_count, hipStream_t s);

size_t select_masks_workspace_bytes(int B, int N);

hipError_t launch_select_masks(int L, int B, int N, const uint32_t* mask, const float* z, int cap,
                               int32_t* surv_idx, float* surv_z, int32_t* surv_count, void* ws,
                               hipStream_t s);

size_t topk_workspace_bytes(int B, int cap, int k);

hipError_t launch_topk(int B, int cap, int k, const int32_t* surv_idx,
                       const float* surv_z, const int32_t* surv_count,
                       int32_t* topk_idx, int32_t* topk_count, void* ws, hipStream_t s);

// Device address of the top-k scratch array on the current device (resolved
// on the first call per device).
hipError_t topk_scratch_address(void** out);

hipError_t launch_gather(int B, int N, int k, int row_bytes, const void* pool,
                         const int32_t* idx, void* hot, hipStream_t s);

size_t fetch_workspace_bytes(int B, int N, int cap);

hipError_t launch_resident_reset(int B, int N, int S, int32_t* slot_of, int32_t* entry_of,
                                 hipStream_t s);

hipError_t launch_fetch(int B, int N, int S, int row_bytes, const void* cold, int cap,
                        const int32_t* surv_idx, const int32_t* surv_count, int32_t* slot_of,
                        int32_t* entry_of, void* rows, int32_t* fetch_count, void* ws,
                        hipStream_t s);

hipError_t launch_gather_resident(int B, int N, int S, int k, int row_bytes, const void* rows,
                                  const int32_t* slot_of, const int32_t* idx, void* hot,
                                  hipStream_t s);

hipError_t launch_label_vote(int Q, int L, int N, float top_p, int theta, const float* logits,
                             uint32_t* mask, uint8_t* count, uint8_t* label, hipStream_t s);

size_t focal_workspace_bytes(int Q, int N, int D, int H, int dI);

hipError_t launch_focal(int Q, int N, int D, int H, int dI, float gamma, const uint16_t* h,
                        const float* Wq, const float* Wg, float bias, const uint16_t* K,
                        const uint8_t* label, float* loss, float* dWq, void* ws, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

hipError_t launch_append_rows(int B, int n, int row_bytes, const void* src, int64_t src_stride,
                              void* dst, int64_t dst_stride, int64_t dst_start, hipStream_t s);

hipError_t launch_lightning(int B, int N, int cap, int H, int dI, lsa_key_dtype kdt,
                            const void* keys, const float* scale, const uint16_t* q,
                            const float* w, const int32_t* surv_idx, const int32_t* surv_count,
                            float* score, hipStream_t s);

int attention_splits(int B, int H, int k, int W);
size_t attention_workspace_bytes(int B, int H, int D, int k, int W);
hipError_t launch_attention(int B, int H, int k, int W, float scale, const uint16_t* q,
                            const uint16_t* hot, const int32_t* hot_count, const uint16_t* win,
                            const int32_t* win_count, float* out, void* ws, hipStream_t s);

}  // namespace lsa
