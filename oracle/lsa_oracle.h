/*
 * lsa_oracle.h -- plain CPU oracle for the Lookahead Sparse Attention (LSA)
 * indexer path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may call it; the product library never
 * does, and the two share no code.
 *
 * Everything is computed in fp64 with plain loops, in the order the method
 * states it.  The only roundings are the storage roundings the method's data
 * format fixes (query -> bf16, gate -> fp32); they are applied at the same
 * points the boundary stores them.
 *
 * Sources (web pages about "FlashMemory-DeepSeek-V4: Lightning Index
 * Ultra-Long Context via Lookahead Sparse Attention"):
 *   [REVIEW]  paper.oopus.info review, section 2 "core method and innovation"
 *   [SUMMARY] gist.science technical summary, sections 2.1-2.4
 *   [ABSTRACT] podnod.eu episode page, paper abstract
 *
 * Parity status: every function below is pinned by a CPU test against an
 * independent fact (library routine, closed form, exact rational arithmetic,
 * brute-force enumeration or finite differences); see the oracle test files.
 */
#ifndef LSA_ORACLE_H
#define LSA_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* ---- storage formats ---------------------------------------------------- */
double   lsa_or_bf16_to_double(uint16_t bits);
uint16_t lsa_or_bf16_from_double(double a);      /* round-to-nearest-even, one rounding */
double   lsa_or_e4m3_to_double(uint8_t code);     /* OCP E4M3FN, NaN for 0x7F/0xFF */
double   lsa_or_softplus(double x);
double   lsa_or_sigmoid(double x);

/* ---- O1: query encoder ([SUMMARY] 2.1 memory-indexer bullet; 2.3 query
 * optimisation bullet).  One (layer, request):
 *   a_j = sum_d Wq[j][d] h[d]   (j = head*dI + d_I index), q_j = bf16(a_j)
 *   g_h = fp32(softplus(sum_d Wg[h][d] h[d]))
 * h: bf16 [D]; Wq: bf16 [H*dI][D]; Wg: bf16 [H][D].
 * a_out (optional, [H*dI]) receives the unrounded fp64 a_j. */
void lsa_or_project(int D, int H, int dI, const uint16_t* h,
                    const uint16_t* Wq, const uint16_t* Wg,
                    uint16_t* q, float* g, double* a_out);

/* q_eff = sum_h g_h q_h (fp64) -- the head-collapsed query.  Used by the
 * input calibration and by the collapse-identity pin. */
void lsa_or_query_collapse(int H, int dI, const uint16_t* q, const float* g,
                           double* q_eff);

/* ---- O2/O3: lookahead index score ([SUMMARY] 2.1 scoring bullet;
 * [REVIEW] section 2, sigmoid score).  One (layer, request), entries given by
 * an index list (or all N when idx == NULL):
 *   z_s = sum_h g_h * (sum_d q[h][d] * k[s][d]) * sigma_s + bias
 * key_dtype 0: bf16 keys [N][dI] (sigma_s = 1); 1: e4m3 keys [N][dI] with
 * fp32 scale [N] (sigma_s = scale[s]).  z_out has n_idx (or N) entries. */
void lsa_or_score(int N, int H, int dI, int key_dtype, const void* keys,
                  const float* scale, const uint16_t* q, const float* g,
                  double bias, const int64_t* idx, int64_t n_idx,
                  double* z_out);

/* ---- O4: threshold I >= 0.5, written as z >= 0 ([SUMMARY] 2.1 dynamic
 * fetch bullet).  NaN is never selected.  sel: one byte per entry. */
void lsa_or_threshold(int64_t n, const double* z, uint8_t* sel);

/* ---- O5: OR across indexer layers and compaction ([SUMMARY] 2.4;
 * [REVIEW] section 2, three-layer routing).  sel [L][N] bytes, z [L][N].
 * Survivors are the entries some layer selects, in ascending index order;
 * zstar = max over layers of z (NaN ignored).  Writes at most cap entries,
 * returns the true survivor count. */
int64_t lsa_or_merge_compact(int L, int64_t N, const uint8_t* sel,
                             const double* z, int64_t cap, int32_t* surv_idx,
                             double* surv_z);

/* ---- O6: top-k inside the fetched set ([SUMMARY] 2.1 hierarchical
 * selection bullet).  Order: zstar descending, index ascending on ties;
 * keep the first min(k, n); emit them in ascending index order, pad -1.
 * Returns min(k, n). */
int64_t lsa_or_topk(int64_t n, const int32_t* surv_idx, const double* surv_z,
                    int64_t k, int32_t* out);

/* ---- O7: hot-pool gather ([SUMMARY] 2.1 dynamic fetch bullet).
 * hot[j] = pool[idx[j]] byte for byte, zero row for idx < 0. */
void lsa_or_gather(int64_t N, int64_t row_bytes, const uint8_t* pool,
                   int64_t k, const int32_t* idx, uint8_t* hot);

/* ---- O10: cold-pool fetch with reuse ([SUMMARY] 2.1 dynamic-fetch bullet;
 * [REVIEW] section 2, the step that moves entries scoring >= 0.5 from the CPU
 * to the GPU).  One request.  A resident set of S slots holds rows of the
 * cold pool: slot_of[N] is the slot of entry s or -1, entry_of[S] the entry in
 * slot j or -1, rows[S][row_bytes] the bytes.  For the ascending survivor
 * list surv[n]:
 *   1. each resident entry that is not a survivor leaves its slot;
 *   2. each survivor that is not resident takes a free slot: the i-th such
 *      survivor (ascending entry) takes the i-th free slot (ascending slot);
 *   3. its row is copied from cold[entry] into rows[slot].
 * Survivors already resident keep their slot and are not copied again.
 * Returns the number of rows copied, or -1 (tables unchanged) if the free
 * slots do not suffice. */
int64_t lsa_or_fetch(int64_t N, int64_t S, int64_t row_bytes, const uint8_t* cold,
                     int64_t n, const int32_t* surv, int32_t* slot_of,
                     int32_t* entry_of, uint8_t* rows);

/* ---- O8: golden labels ([SUMMARY] 2.2 steps 1-3; [REVIEW] section 2,
 * training labels).  One row of raw logits x[N]:
 *   pi = softmax(x); walk entries in order (x desc, index asc) and include
 *   each while the mass already taken is < top_p (the entry that crosses
 *   top_p is included).  mass_ahead (optional, [N]) receives, for every
 *   entry, the mass of the entries before it in that order.
 * Returns the nucleus size. */
int64_t lsa_or_nucleus(int64_t N, const float* x, double top_p, uint8_t* sel,
                       double* mass_ahead);
/* Vote: count_s = number of layers whose nucleus holds s; label_s =
 * (count_s >= theta).  sel [L][N]. */
void lsa_or_vote(int L, int64_t N, const uint8_t* sel, int theta,
                 uint8_t* count, uint8_t* label);

/* ---- O9: student loss and gradient ([SUMMARY] 2.3 loss bullet and query
 * optimisation bullet; [REVIEW] section 2, BCE plus focal loss).
 *   q_t = Wq h_t (fp64, training precision), g_t = softplus(Wg h_t)
 *   z_ts = sum_h g_th (q_th . k_s) + bias
 *   loss = mean_ts BCE(z_ts, y_ts) + mean_ts FL_gamma(z_ts, y_ts)
 *   dWq  = d loss / d Wq   ([H*dI][D], fp64)
 * h: bf16 [Q][D]; Wq: fp32 [H*dI][D]; Wg: fp32 [H][D]; K: bf16 [N][dI];
 * y: u8 [Q][N].  z_out (optional) [Q][N]. */
double lsa_or_focal_bce_grad(int Q, int64_t N, int D, int H, int dI,
                             double gamma, const uint16_t* h, const float* Wq,
                             const float* Wg, double bias, const uint16_t* K,
                             const uint8_t* y, double* dWq, double* z_out);

/* Loss alone (no gradient) for finite-difference pins; Wq/Wg in fp64. */
double lsa_or_focal_bce_loss64(int Q, int64_t N, int D, int H, int dI,
                               double gamma, const double* h, const double* Wq,
                               const double* Wg, double bias, const double* K,
                               const uint8_t* y);

/* ---- O11: core attention over the selected rows ([SUMMARY] 2.1
 * hierarchical-selection bullet: once the selected subset is on the GPU, a
 * top-k inside it feeds the final core attention).  Reading: each row is a
 * compressed latent vector that serves as both key and value, shared by all
 * heads; for head h over the n given rows:
 *   s_j = scale * sum_d q[h][d] * row_j[d]
 *   p_j = exp(s_j - max_i s_i)
 *   out[h][d] = sum_j p_j row_j[d] / sum_j p_j
 * q: bf16 [H][D]; rows: bf16 [n][D]; out fp64 [H][D]; n = 0 gives zeros.
 * wabs (optional, [H][D]) receives sum_j p_j |row_j[d]| / sum_j p_j, the
 * scale of the output's rounding error. */
void lsa_or_attention(int64_t n, int D, int H, const uint16_t* q,
                      const uint16_t* rows, double scale, double* out,
                      double* wabs);

/* ---- O13: fine-grained score inside the fetched set ([SUMMARY] 2.1
 * hierarchical-selection bullet: the top-k inside the fetched subset uses the
 * model's native Lightning Indexer, which the pages name but do not define).
 * Reading: the published form of that indexer, one score per entry from its
 * own keys and a per-query set of heads with ReLU gates and weights:
 *   out_i = sum_h w[h] * max(0, sum_d q[h][d] * k[s_i][d] * sigma_{s_i}),  s_i = idx[i]
 * key_dtype 0: bf16 keys [N][dI] (sigma = 1); 1: e4m3 keys with fp32 scale
 * [N].  q: bf16 [H][dI]; w: fp32 [H]; idx: the n entries to score. */
void lsa_or_lightning(int N, int H, int dI, int key_dtype, const void* keys,
                      const float* scale, const uint16_t* q, const float* w,
                      const int32_t* idx, int64_t n, double* out);

/* ---- trigger cadence ([SUMMARY] 2.1 periodic-trigger bullet; [REVIEW]
 * section 2): the indexer runs at decode step t iff t is a multiple of tau,
 * counting from step 0. */
int lsa_or_trigger_due(int64_t t, int tau);

int lsa_or_num_threads(void);
void lsa_or_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
