/*
 * nsa_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU statement of the Native Sparse Attention (NSA)
 * forward pass and its MoBA special case, used to check the GPU library.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, constant or helper with the GPU
 * library: its configuration struct and switches are its own.
 *
 * Sources (cited by page title and section):
 *   [P1] "Zhang Xiaojun Business Interviews #94" transcript (bidclub.ai):
 *        s4 "Inside Native Sparse Attention", s5 "Hardware Makes Sparsity
 *        Work", s7 "Kimi Simplifies The Sparse Route".
 *   [P5] LateTalk #103 notes (zjai.club), close-reading s12 and s13.
 *
 * Tensor layouts (row-major, last dimension contiguous):
 *   q     [B, T, H, d_qk]      k  [B, L, G, d_qk]     v  [B, L, G, d_v]
 *   gates [B, T, H, 3]         (compressed, selected, window)
 *   kc    [B, nb, G, d_qk]     vc [B, nb, G, d_v]     nb = floor(L / block)
 * Selection works on blocks of sel_block tokens (nbs = floor(L / sel_block));
 * with sel_block = block the two block grids coincide.
 * Storage is fp32, or bf16 given as raw 16-bit patterns (is_bf16 = 1).
 * Query row t sits at absolute position p = L - T + t.
 * Head h belongs to KV group h / heads_per_group.
 */
#ifndef NSA_ORACLE_H
#define NSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, q_len, kv_len;
  int32_t n_groups, heads_per_group;
  int32_t d_qk, d_v;
  int32_t block, top_k, window;
  int32_t force_first;    /* block 0 always selected                 */
  int32_t force_current;  /* the query's own block always selected   */
  int32_t use_cmp, use_slc, use_win;  /* branches that enter the output */
  int32_t gate_logits;    /* gates hold logits; apply sigmoid first  */
  int32_t is_bf16;        /* 1: bf16 bit patterns, 0: fp32           */
  int32_t sel_block;      /* selection block; 0 means block; else a  */
                          /* multiple of block                       */
  double scale;           /* softmax scale; 0 means 1/sqrt(d_qk)     */
} oracle_cfg;

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_BAD_CONFIG 1
#define ORACLE_BAD_SELECTION 2

/* Block mean of K and V; results rounded to the storage type. */
int oracle_pool(const oracle_cfg* c, const void* k, const void* v, void* kc, void* vc);

/* Compressed branch + group importance + top-k for the listed query rows
 * (flat row r = b * T + t).
 *   idx   [nrows, G, top_k]  ascending selection-block ids, padded with -1
 *   imp   [nrows, G, nbs]    importance of each selection block (NaN if not
 *                            visible), may be NULL
 *   o_cmp [nrows, H, d_v]    compressed-branch output, may be NULL        */
int oracle_select(const oracle_cfg* c, const void* q, const void* kc, const void* vc,
                  const int64_t* rows, int64_t nrows,
                  int32_t* idx, double* imp, double* o_cmp);

/* Selected and window branches for the listed rows on a GIVEN selection
 * idx [nrows, G, top_k], then the gated sum with o_cmp [nrows, H, d_v]
 * (may be NULL when the compressed branch is off).  gates may be NULL when
 * exactly one branch is on (its weight is then 1).
 *   out [nrows, H, d_v]; o_slc, o_win [nrows, H, d_v] optional (NULL).    */
int oracle_attend(const oracle_cfg* c, const void* q, const void* k, const void* v,
                  const void* gates, const int32_t* idx, const double* o_cmp,
                  const int64_t* rows, int64_t nrows,
                  double* out, double* o_slc, double* o_win);

/* Natural log-sum-exp of the selected branch's scaled logits per head,
 * log sum_s exp(scale q_h . k_s) over oracle_attend's selected key set on
 * the GIVEN selection idx [nrows, G, top_k]; -inf for an empty set.
 *   lse [nrows, H].                                                       */
int oracle_selected_lse(const oracle_cfg* c, const void* q, const void* k, const int32_t* idx,
                        const int64_t* rows, int64_t nrows, double* lse);

/* Threads the oracle's parallel loops use. */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
