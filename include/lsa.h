/*
 * lsa.h -- C ABI of liblsa.so, the MI355X (gfx950) Lookahead Sparse Attention
 * indexer hot path.
 *
 * Sources (web pages on "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long
 * Context via Lookahead Sparse Attention"):
 *   [SUMMARY] gist.science technical summary: 2.1 architecture (trigger,
 *             memory indexer, scoring, dynamic fetch, hierarchical
 *             selection), 2.2 label curation, 2.3 decoupled training,
 *             2.4 optimal configuration (layers 10/12/20, OR mode)
 *   [REVIEW]  paper.oopus.info review: section 2 (core method), section 3
 *             (resources)
 *
 * Conventions for every call:
 *  - All tensor arguments are DEVICE pointers owned by the caller, except
 *    where an argument is documented as a host array or as host memory.  The
 *    library never allocates persistent memory; its only global state is a
 *    thread-local error string and a per-device cache of the compute-unit
 *    count (filled once, thread-safe).  Every call is reentrant.
 *  - Every compute call enqueues its kernels on `stream` and returns without
 *    synchronising.  Outputs are valid once the stream has reached that point.
 *  - Argument, shape and dtype errors are detected on the host and returned
 *    before anything is launched (nothing is written).  A launch failure
 *    returns LSA_E_HIP.  lsa_last_error() then holds a message.
 *  - Device pointers must be 16-byte aligned unless stated otherwise.
 *  - bf16 tensors are passed as uint16_t bit patterns, e4m3 as uint8_t codes
 *    (OCP 8-bit E4M3 "FN": bias 7, subnormals, no infinity, 0x7F/0xFF NaN).
 *  - Notation: L indexer layers, B concurrent requests, N compressed entries
 *    per layer and request, H indexer heads, dI indexer head dimension, D
 *    hidden size, k top-k size.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LSA_OK = 0,
  LSA_E_ARG = 1,        /* null pointer, negative size, bad alignment, bad value */
  LSA_E_SHAPE = 2,      /* a size outside what the kernels support */
  LSA_E_DTYPE = 3,      /* unknown key dtype */
  LSA_E_HIP = 4,        /* a HIP launch or runtime call failed */
  LSA_E_WORKSPACE = 5   /* workspace missing or smaller than required */
} lsa_status;

typedef enum {
  LSA_KEY_BF16 = 0,       /* keys bf16 [B][N][dI] */
  LSA_KEY_FP8_E4M3 = 1    /* keys e4m3 [B][N][dI] + fp32 scale [B][N] */
} lsa_key_dtype;

#define LSA_MAX_LAYERS 8      /* indexer layers per lsa_score call */
#define LSA_CAND_CHUNK 4096   /* entries per candidate chunk (see lsa_score) */
#define LSA_MAX_HEADS 64      /* indexer heads */
#define LSA_MAX_VOTE_LAYERS 32

/* Message describing the last non-OK status returned on this thread. */
const char* lsa_last_error(void);

/* Library version string. */
const char* lsa_version(void);

/* ---------------------------------------------------------------------------
 * Trigger cadence ([SUMMARY] 2.1, periodic trigger; [REVIEW] section 2): the
 * indexer runs at decode step t iff t >= 0 and t is a multiple of tau,
 * counting from step 0.  Returns 1 or 0; tau <= 0 returns 0.  Host only.
 */
int lsa_trigger_due(int64_t decode_step, int tau);

/* ---------------------------------------------------------------------------
 * Query encoder ([SUMMARY] 2.1 memory-indexer bullet: the hidden state of the
 * current token is mapped to a low-rank indexer query; 2.3: only this
 * projection is trained).  For every layer l and request b:
 *   a = Wq[l] . h[l][b]      (fp32 accumulation)      q[l][b] = bf16(a)
 *   g[l][b][j] = softplus(Wg[l][j] . h[l][b])           (fp32)
 * The head-gate form (softplus gates, one per head) is this library's reading
 * of the scoring bullet's "gated, head-fused" match.
 *
 *   h        bf16 [L?][B][D]; layer l reads h + l * h_layer_stride
 *            (h_layer_stride = 0: one h_t per request shared by all layers)
 *   Wq       HOST array of L device pointers, each bf16 [H*dI][D]
 *            (row index = head * dI + i)
 *   Wg       HOST array of L device pointers, each bf16 [H][D]
 *   q        out bf16 [L][B][H][dI]        g   out fp32 [L][B][H]
 * Limits: 1 <= L <= LSA_MAX_LAYERS, B >= 1, D % 64 == 0 and 64 <= D <= 65536,
 * B * D * 2 < 2^31, 1 <= H <= 64, dI in {64, 128}.
 */
lsa_status lsa_project_query(int L, int B, int D, int H, int dI,
                             const uint16_t* h, int64_t h_layer_stride,
                             const uint16_t* const* Wq,
                             const uint16_t* const* Wg, uint16_t* q, float* g,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The same query encoder from pre-packed weights ([SUMMARY] 2.1 memory-indexer
 * bullet, as above).  The weights are fixed parameters, so they can be laid
 * out once, at load time, in the operand order of the matrix-core
 * instruction the projection runs on; every weight load then reads 1 KiB of
 * contiguous memory.  The results are those of lsa_project_query, bit for
 * bit.
 *
 * Layout of one layer: its R = H*dI + H rows (the Wq rows, then the Wg rows,
 * zero rows after them) in T = ceil(R / 16) tiles of 16 rows, the hidden
 * dimension in D / 64 units; tile t, unit u, step s (0 or 1) and lane l
 * (0..63) hold the 8 bf16 values of row 16 t + l % 16, columns
 * 64 u + 32 s + 8 (l / 16) .. +7, as 16 bytes at byte offset
 * ((t * (D / 64) + u) * 2 + s) * 1024 + 16 l.
 *
 * lsa_query_weights_packed_bytes: bytes of one layer's packed buffer
 *   (T * (D / 64) * 2048); 0 for unsupported H, dI or D.
 * lsa_pack_query_weights: writes one layer's packed buffer.
 *   Wq, Wg   bf16 [H*dI][D] and [H][D], as for lsa_project_query
 *   packed   out, caller-owned, lsa_query_weights_packed_bytes bytes
 *   All three 16-byte aligned.  Enqueued on stream like every call.
 * lsa_project_query_packed: lsa_project_query with
 *   packed   HOST array of L device pointers, each a buffer written by
 *            lsa_pack_query_weights for that layer
 *   and every other argument, output and limit as for lsa_project_query.
 */
size_t lsa_query_weights_packed_bytes(int H, int dI, int D);
lsa_status lsa_pack_query_weights(int H, int dI, int D, const uint16_t* Wq,
                                  const uint16_t* Wg, void* packed,
                                  hipStream_t stream);
lsa_status lsa_project_query_packed(int L, int B, int D, int H, int dI,
                                    const uint16_t* h, int64_t h_layer_stride,
                                    const void* const* packed, uint16_t* q,
                                    float* g, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Lookahead index score and threshold ([SUMMARY] 2.1 scoring bullet: a
 * sigmoid, head-fused, gated match of the query against every earlier
 * compressed entry; dynamic-fetch bullet: entries with I >= 0.5 are fetched).
 * For every layer l, request b and entry s:
 *   z[l][b][s] = sum_h g[l][b][h] * (q[l][b][h] . k_l[b][s]) * sigma + bias[l]
 *   I = sigmoid(z);  selected  <=>  I >= 0.5  <=>  z >= 0 (NaN: not selected)
 * with sigma = key_scale[l][b][s] for e4m3 keys and 1 for bf16 keys.
 *
 * All layers of a request are scored in one call, and the three-layer OR
 * merge ([SUMMARY] 2.4: layer predictions united in OR mode; [REVIEW] section
 * 2: an entry is fetched when any layer asks for it) is done here, chunk by
 * chunk: the entries are cut into chunks of LSA_CAND_CHUNK, and for request b
 * and chunk c the call writes the candidate list
 *   cand_idx[b][c][0..n)  the entries of the chunk selected by at least one
 *                         layer, ascending, n = cand_count[b][c]
 *   cand_z[b][c][i]       their merged logit: the maximum of z over the layers
 *                         that select the entry (for a selected entry this is
 *                         the maximum over all layers, since every selecting
 *                         layer has z >= 0 and every other layer z < 0)
 * lsa_select_or_compact turns the chunk lists into one survivor list.
 *
 *   keys       HOST array of L device pointers, each [B][N][dI] (bf16 or e4m3)
 *   key_scale  HOST array of L device pointers, each fp32 [B][N]; required for
 *              LSA_KEY_FP8_E4M3, ignored (may be NULL) for bf16
 *   q, g       as written by lsa_project_query
 *   bias       DEVICE fp32 [L], read by the kernels when they run (so a captured
 *              graph picks up new values without being captured again)
 *   sel_mask   out uint32 [L][B][ceil(N/32)]: bit (s % 32) of word s / 32;
 *              bits past N are zero
 *   cand_idx   out int32 [B][nchunks][LSA_CAND_CHUNK], nchunks = ceil(N / LSA_CAND_CHUNK)
 *   cand_z     out fp32  [B][nchunks][LSA_CAND_CHUNK]
 *   cand_count out int32 [B][nchunks]
 *              (list slots past a chunk's count are left unwritten)
 *   z_opt      out fp32 [L][B][N] or NULL: every layer's z.  Costs extra
 *              writes; the hot path passes NULL
 *   I_opt      out fp32 [L][B][N] or NULL: sigmoid(z)
 * Limits: 1 <= L <= LSA_MAX_LAYERS, 1 <= B <= 65535, 0 <= N <= 2^24 (N = 0
 * launches nothing), 1 <= H <= 64, dI in {64, 128}, and the keys of one
 * (layer, request), N * dI * (2 for bf16, 1 for e4m3) bytes, below 2^31.
 * The sum over heads is evaluated as one dot product with
 * sum_h g[l][b][h] q[l][b][h] (fp32), which equals the per-head form up to
 * rounding.
 */
lsa_status lsa_score(int L, int B, int N, int H, int dI, lsa_key_dtype kdt,
                     const void* const* keys, const float* const* key_scale,
                     const uint16_t* q, const float* g, const float* bias,
                     uint32_t* sel_mask, int32_t* cand_idx, float* cand_z,
                     int32_t* cand_count, float* z_opt, float* I_opt,
                     hipStream_t stream);

/* ---------------------------------------------------------------------------
 * lsa_score on a growing key cache ([REVIEW] section 2 and [SUMMARY] 2.1,
 * periodic trigger: every tau decode steps the indexer scores every entry
 * compressed so far, and entries keep being appended between triggers).  The
 * key and scale arrays of each layer hold entry_stride entries per request
 * (the cache capacity); the call scores the first N of each request.  Every
 * other argument, output and limit is that of lsa_score, which is this call
 * with entry_stride = N.  Limits: N <= entry_stride <= 2^40.
 */
lsa_status lsa_score_strided(int L, int B, int N, int64_t entry_stride, int H, int dI,
                             lsa_key_dtype kdt, const void* const* keys,
                             const float* const* key_scale, const uint16_t* q,
                             const float* g, const float* bias, uint32_t* sel_mask,
                             int32_t* cand_idx, float* cand_z, int32_t* cand_count,
                             float* z_opt, float* I_opt, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Append to a per-request cache ([REVIEW] section 2: the backbone keeps
 * compressing 4 tokens into one entry, so 16 entries arrive per 64-step
 * trigger window; [SUMMARY] 2.3: each new entry's indexer key is computed once
 * and then frozen).  For every request b and i < n:
 *   dst[b][dst_start + i] = src[b][i]        (rows of row_bytes bytes)
 * with src holding src_stride rows per request and dst dst_stride rows per
 * request (the cache capacity).  Used for the per-layer key rows, their fp32
 * scales and the KV pool rows.
 * Limits: 1 <= B <= 65535, n >= 0, row_bytes > 0 and a multiple of 4,
 * src_stride >= n, 0 <= dst_start, dst_start + n <= dst_stride; src and dst
 * 4-byte aligned (16-byte alignment and row sizes move 16 bytes a thread).
 */
lsa_status lsa_append_rows(int B, int n, int row_bytes, const void* src, int64_t src_stride,
                           void* dst, int64_t dst_stride, int64_t dst_start,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Survivor compaction of the OR-merged selection ([SUMMARY] 2.1 dynamic-fetch
 * bullet: every entry some indexer layer selects is fetched).  Concatenates
 * the chunk candidate lists of lsa_score, in chunk order, so for every
 * request b:
 *   surv_idx[b]   = the entries selected by at least one layer, ascending
 *   surv_z[b][i]  = their merged logit
 *   surv_count[b] = the TRUE number of survivors, even when it exceeds cap;
 *                   only the first cap are written
 *
 *   cand_idx, cand_z, cand_count   as written by lsa_score
 *   surv_idx  out int32 [B][cap]  surv_z out fp32 [B][cap]  surv_count out int32 [B]
 * Limits: 1 <= B <= 65535, N >= 0, cap >= 0.
 */
lsa_status lsa_select_or_compact(int B, int N, const int32_t* cand_idx,
                                 const float* cand_z, const int32_t* cand_count,
                                 int cap, int32_t* surv_idx, float* surv_z,
                                 int32_t* surv_count, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The same OR merge and compaction from dense per-layer selections
 * ([SUMMARY] 2.4: the layers' predictions are united in OR mode; [SUMMARY]
 * 2.1 dynamic-fetch bullet: every entry a layer selects is fetched), for
 * masks and logits from any producer -- lsa_score's sel_mask and z_opt, or
 * another indexer.  For every request b:
 *   surv_idx[b]   = ascending { s < N : bit s of sel_mask[l][b] is set for
 *                   some layer l }
 *   surv_z[b][i]  = max over ALL layers l of z[l][b][s] (NaN values ignored;
 *                   NaN when every layer's value is NaN).  For masks that are
 *                   z >= 0 this equals the maximum over the selecting layers.
 *   surv_count[b] = the TRUE survivor count (only the first cap are written)
 *
 *   sel_mask  uint32 [L][B][ceil(N/32)], bit (s % 32) of word s / 32; bits
 *             at or past N are ignored
 *   z         fp32 [L][B][N]
 *   surv_idx out int32 [B][cap]   surv_z out fp32 [B][cap]   surv_count out int32 [B]
 *   ws        device workspace of lsa_select_or_compact_masks_workspace_bytes(B, N)
 *             bytes, 16-byte aligned (per-chunk survivor counts)
 * Limits: 1 <= L <= LSA_MAX_LAYERS, 1 <= B <= 65535, 0 <= N <= 2^24, cap >= 0;
 * sel_mask and z 4-byte aligned.  Errors: LSA_E_SHAPE / LSA_E_ARG for the
 * limits and null pointers, LSA_E_WORKSPACE for a missing or short workspace,
 * LSA_E_HIP for a launch failure.
 */
size_t lsa_select_or_compact_masks_workspace_bytes(int B, int N);
lsa_status lsa_select_or_compact_masks(int L, int B, int N, const uint32_t* sel_mask,
                                       const float* z, int cap, int32_t* surv_idx,
                                       float* surv_z, int32_t* surv_count, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Top-k inside the fetched set ([SUMMARY] 2.1 hierarchical-selection bullet:
 * once the fetched subset is on the GPU, a fine-grained top-k runs inside
 * it).  Ranking score: the merged logit surv_z (higher first); ties go to the
 * lower entry index.  For every request b, with n = min(surv_count[b], cap):
 *   topk_idx[b]   = the min(k, n) best survivors, in ASCENDING entry order,
 *                   followed by -1 up to k
 *   topk_count[b] = min(k, n)
 *
 *   surv_idx int32 [B][cap] (ascending), surv_z fp32 [B][cap], surv_count [B]
 *   topk_idx out int32 [B][k]     topk_count out int32 [B]
 *   ws       device workspace of lsa_topk_workspace_bytes()
 * Limits: B >= 1, cap >= 0, k >= 0.
 */
size_t lsa_topk_workspace_bytes(int B, int cap, int k);
lsa_status lsa_topk(int B, int cap, int k, const int32_t* surv_idx,
                    const float* surv_z, const int32_t* surv_count,
                    int32_t* topk_idx, int32_t* topk_count, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * lsa_topk without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  Arguments, results and limits are those of
 * lsa_topk; the candidate lists of long survivor lists go to a scratch array
 * of LSA_TOPK_NOALLOC_MAX_BYTES that the library holds on each GPU it runs
 * on, for the life of the process.  The call allocates nothing and
 * synchronises nothing.
 *  - Sizes whose lsa_topk_workspace_bytes(B, cap, k) exceeds
 *    LSA_TOPK_NOALLOC_MAX_BYTES return LSA_E_SHAPE (use lsa_topk).
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (different streams, or host threads) race and give wrong results.
 *    Calls ordered on one stream are safe.
 *  - The first call on a device resolves the array's device address
 *    (hipGetSymbolAddress, not a stream operation); make that first call
 *    outside graph capture.  A failure returns LSA_E_HIP.
 */
#define LSA_TOPK_NOALLOC_MAX_BYTES (16 << 20)
lsa_status lsa_topk_noalloc(int B, int cap, int k, const int32_t* surv_idx,
                            const float* surv_z, const int32_t* surv_count,
                            int32_t* topk_idx, int32_t* topk_count, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Fine-grained score inside the fetched set ([SUMMARY] 2.1 hierarchical-
 * selection bullet: once the selected subset is on the GPU, the model's
 * native Lightning Indexer picks the final top-k inside it; the pages name it
 * without a formula).  This library's reading is that indexer's published
 * form: its own key per entry, and per query H heads with ReLU gates and
 * weights.  For every request b and i < min(surv_count[b], cap):
 *   score[b][i] = sigma_s * sum_h w[b][h] * max(0, q[b][h] . k[b][s]),
 *   s = surv_idx[b][i],  sigma_s = key_scale[b][s] (e4m3) or 1 (bf16)
 * (-inf for an index outside [0, N)).  Products of bf16 values are exact
 * (e4m3 widens exactly to bf16), sums in fp32.  Rank with lsa_topk(surv_idx,
 * score, surv_count, ...).
 *
 *   keys       [B][N][dI] bf16 or e4m3 (the indexer's own keys), 16-byte aligned
 *   key_scale  fp32 [B][N] (e4m3; positive), NULL for bf16
 *   q          bf16 [B][H][dI]      w  fp32 [B][H]
 *   surv_idx   int32 [B][cap]       surv_count int32 [B]
 *   score      out fp32 [B][cap] (slots past the count are not written)
 * Limits: 1 <= B <= 65535, 0 <= N <= 2^24, cap >= 0, H a multiple of 16 in
 * [16, 64], dI in {64, 128}, one request's keys below 2^31 bytes.
 */
lsa_status lsa_lightning_score(int B, int N, int cap, int H, int dI, lsa_key_dtype kdt,
                               const void* keys, const float* key_scale, const uint16_t* q,
                               const float* w, const int32_t* surv_idx,
                               const int32_t* surv_count, float* score, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Hot-pool gather ([SUMMARY] 2.1 dynamic-fetch bullet: the selected
 * compressed KV entries are brought into GPU memory).
 *   hot[b][j] = pool[b][idx[b][j]]  (row_bytes bytes), zero row when
 *   idx[b][j] < 0 or idx[b][j] >= N
 *
 *   pool  [B][N][row_bytes]   idx int32 [B][k]   hot out [B][k][row_bytes]
 * Limits: row_bytes > 0 and a multiple of 16; pool and hot 16-byte aligned.
 */
lsa_status lsa_gather_hot(int B, int N, int k, int row_bytes, const void* pool,
                          const int32_t* idx, void* hot, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Core attention of one decode step over the selected rows ([SUMMARY] 2.1
 * hierarchical-selection bullet: the top-k chosen inside the fetched subset
 * feeds the final core attention; [SUMMARY] 1: recent tokens carry most
 * requests, so a local window of recent rows is attended as well).  Reading
 * of this library: every row is a compressed latent vector of D = 512 bf16
 * that serves as both key and value and is shared by all heads.  For every
 * request b and head h, over the rows
 *   R_b = hot[b][0 .. hc) followed by win[b][0 .. wc),
 *   hc = min(hot_count[b], k) (k when hot_count is NULL; negative = 0),
 *   wc = min(win_count[b], W) (W when win_count is NULL),
 * the output is
 *   s_j = scale * (q[b][h] . r_j),   out[b][h] = sum_j softmax(s)_j * r_j
 * (fp32; both products on bf16 matrix cores with fp32 accumulation, the
 * softmax weights carried as an exact bf16 pair).  No rows: zeros.
 *
 *   q          bf16 [B][H][D]
 *   hot        bf16 [B][k][D]   (lsa_gather_hot / lsa_gather_resident output;
 *              rows past hc are not read)
 *   hot_count  int32 [B] or NULL (lsa_topk's topk_count)
 *   win        bf16 [B][W][D] or NULL when W = 0;  win_count int32 [B] or NULL
 *   out        out fp32 [B][H][D]
 *   ws         device workspace of lsa_sparse_attention_workspace_bytes()
 *              bytes, 256-byte aligned (per-split partial outputs; 0 bytes
 *              when one split covers the rows)
 * Limits: 1 <= B <= 65535, H a multiple of 16 in [16, 1024], D == LSA_ATT_ROW,
 * k, W >= 0 and k + W <= 2^20, finite scale; q, hot, win, out 16-byte
 * aligned.  Errors: LSA_E_SHAPE / LSA_E_ARG for the limits and null or
 * misaligned pointers, LSA_E_WORKSPACE, LSA_E_HIP for a launch failure.
 */
#define LSA_ATT_ROW 512
size_t lsa_sparse_attention_workspace_bytes(int B, int H, int D, int k, int W);
lsa_status lsa_sparse_attention(int B, int H, int D, int k, int W, float scale,
                                const uint16_t* q, const uint16_t* hot,
                                const int32_t* hot_count, const uint16_t* win,
                                const int32_t* win_count, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Cold-pool fetch with reuse ([SUMMARY] 2.1 dynamic-fetch bullet: every
 * entry with I >= 0.5 is brought from the CPU cold pool into GPU memory;
 * [REVIEW] section 2: the move is asynchronous and overlaps compute).
 * The GPU reads the cold pool in place over the host link into a resident
 * set of S slots per request, on `stream` (launch it on its own stream to
 * overlap other work).  Per request b, with n = min(surv_count[b], cap):
 *   1. a resident entry that is not among surv_idx[b][0..n) leaves its slot
 *      (entry_of = -1, slot_of = -1; its bytes stay);
 *   2. the survivors that are not resident take free slots: the i-th of them
 *      in entry order takes the i-th free slot in slot order;
 *   3. each of those rows is copied: rows[b][slot] = cold_pool[b][entry].
 * Survivors already resident keep their slot and are not read again.
 * fetch_count[b] = the number of rows copied, or -1 when request b's
 * survivors do not fit in S slots; that request's tables and rows are then
 * left exactly as they were (raise S or lower the survivor count).
 *
 *   cold_pool  [B][N][row_bytes] in pinned, mapped host memory (hipHostMalloc)
 *              or in device memory; pageable host memory is refused
 *   surv_idx   int32 [B][cap], ascending (lsa_select_or_compact's output),
 *   surv_count int32 [B] (may exceed cap); entries outside [0, N) are ignored
 *   slot_of    int32 [B][N]  in/out: slot of each entry, or -1
 *   entry_of   int32 [B][S]  in/out: entry in each slot, or -1
 *   rows       [B][S][row_bytes] in/out device memory
 *   fetch_count out int32 [B]
 *   ws         device workspace of lsa_fetch_workspace_bytes(B, N, cap)
 * The tables start with every element -1 (lsa_resident_reset) and are then
 * owned by these calls; calls on the same tables must be stream-ordered.
 * Limits: 1 <= B <= 65535, 0 <= N <= 2^24, cap >= 0, 0 <= S <= 2^24,
 * B * min(cap, N, S) < 2^31, row_bytes > 0 and a multiple of 16, cold_pool
 * and rows 16-byte aligned; surv_idx holds no repeats.  Errors: LSA_E_SHAPE / LSA_E_ARG for the limits, null or
 * misaligned pointers and a cold pool in pageable memory; LSA_E_WORKSPACE;
 * LSA_E_HIP for a launch failure.
 */
size_t lsa_fetch_workspace_bytes(int B, int N, int cap);
lsa_status lsa_resident_reset(int B, int N, int S, int32_t* slot_of, int32_t* entry_of,
                              hipStream_t stream);
lsa_status lsa_fetch_survivors(int B, int N, int S, int row_bytes, const void* cold_pool,
                               int cap, const int32_t* surv_idx, const int32_t* surv_count,
                               int32_t* slot_of, int32_t* entry_of, void* rows,
                               int32_t* fetch_count, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Top-k rows out of the resident set ([SUMMARY] 2.1 hierarchical-selection
 * bullet: the top-k runs inside the fetched subset and its rows feed the
 * core attention).
 *   hot[b][j] = rows[b][slot_of[b][idx[b][j]]], zero row when idx[b][j] is
 *   outside [0, N) or that entry is not resident
 *   rows [B][S][row_bytes]   slot_of int32 [B][N]   idx int32 [B][k]
 *   hot out [B][k][row_bytes]
 * Limits: row_bytes > 0 and a multiple of 16; rows and hot 16-byte aligned.
 */
lsa_status lsa_gather_resident(int B, int N, int S, int k, int row_bytes, const void* rows,
                               const int32_t* slot_of, const int32_t* idx, void* hot,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Golden labels by cross-layer majority vote ([SUMMARY] 2.2 steps 1-3;
 * [REVIEW] section 2, training labels).  For every query t and teacher
 * layer l, over the N entries of the row logits[t][l]:
 *   pi = softmax(row); walk entries in order (logit desc, index asc) and keep
 *   each one while the mass already kept is < top_p (the entry crossing
 *   top_p is kept);
 * then count[t][s] = number of layers keeping s, label[t][s] = count >= theta.
 *
 *   logits          fp32 [Q][L][N] (finite values), 16-byte aligned
 *   layer_mask_opt  out uint32 [Q][L][ceil(N/32)]: bit j of word w is
 *                   entry 32w+j kept by that layer; or NULL
 *   count           out uint8 [Q][N]        label  out uint8 [Q][N] (0/1),
 *                   both 16-byte aligned
 *   ws              device workspace of lsa_label_vote_workspace_bytes()
 *                   bytes (holds the per-layer masks); needed only when
 *                   layer_mask_opt is NULL, else may be NULL
 * Each entry's mass exp(x - max) is truncated to units of 2^-31 and summed
 * exactly in 64-bit integers, so the result is deterministic; it differs
 * from exact arithmetic only for entries whose mass ahead lies within
 * N * 2^-31 (relative) of top_p.
 * Limits: Q >= 1, 1 <= L <= LSA_MAX_VOTE_LAYERS, Q * L < 2^31, 1 <= N <= 65536,
 * 0 < top_p <= 1, theta >= 0.  Errors: LSA_E_SHAPE / LSA_E_ARG for the
 * limits, null or misaligned pointers; LSA_E_WORKSPACE for a missing or
 * short workspace; LSA_E_HIP for a launch failure.
 */
size_t lsa_label_vote_workspace_bytes(int Q, int L, int N);
lsa_status lsa_label_vote(int Q, int L, int N, float top_p, int theta,
                          const float* logits, uint32_t* layer_mask_opt,
                          uint8_t* count, uint8_t* label, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Student loss and gradient ([SUMMARY] 2.3: keys frozen, only the query
 * encoder's projection is trained, BCE combined with a focal loss; [REVIEW]
 * section 2).  In fp32:
 *   q_t = Wq h_t,  g_t = softplus(Wg h_t),  z_ts = sum_h g_th (q_th . K_s) + bias
 *   loss = mean_ts BCE(z_ts, y_ts) + mean_ts (1 - p_t)^gamma BCE(z_ts, y_ts)
 *   dWq  = d loss / d Wq
 *
 *   h     bf16 [Q][D] (16-byte aligned)  Wq fp32 [H*dI][D], row = head*dI + i
 *   Wg    fp32 [H][D]   (Wq, Wg 16-byte aligned)   bias: host scalar
 *   K     bf16 [N][dI] (8-byte aligned)   label uint8 [Q][N] (nonzero = 1)
 *   loss  out fp32 [1]  dWq out fp32 [H*dI][D] (16-byte aligned)
 *   ws    device workspace of lsa_focal_bce_grad_workspace_bytes() bytes,
 *         256-byte aligned (intermediates: projections, gates, collapsed
 *         queries, transposed K and h, dloss/dz, partial key gradients)
 * Every product is an fp32 contraction with fp32 accumulation; the loss sum
 * is accumulated in fp64 in a fixed order, so results are deterministic.
 * Limits: 1 <= Q <= 64, 1 <= N <= 4,000,000, D % 128 == 0 and D <= 16384,
 * 1 <= H <= 64, dI in {64, 128}, 0 <= gamma <= 16, finite bias.  Errors: LSA_E_SHAPE / LSA_E_ARG for the
 * limits, null or misaligned pointers; LSA_E_WORKSPACE for a missing, short
 * or misaligned workspace; LSA_E_HIP for a launch failure.
 */
size_t lsa_focal_bce_grad_workspace_bytes(int Q, int N, int D, int H, int dI);
lsa_status lsa_focal_bce_grad(int Q, int N, int D, int H, int dI, float gamma,
                              const uint16_t* h, const float* Wq,
                              const float* Wg, float bias, const uint16_t* K,
                              const uint8_t* label, float* loss, float* dWq,
                              void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H */
