/*
 * nsa_oracle.c -- TEST INFRASTRUCTURE ONLY (see nsa_oracle.h).
 *
 * A deliberately plain fp64 implementation of the NSA forward pass, written
 * step by step from the pages' description.  No blocking, fusion or
 * reordering: every quantity is computed from its definition, one query row
 * and one head at a time.  Rows are independent, so the only parallelism is
 * an OpenMP loop over rows.
 *
 * Readings of the pages where they are silent (each is also listed in the
 * design notes):
 *   - compression is the block mean (the MoBA description in [P1] s7 uses
 *     mean pooling; the NSA configuration used here does the same);
 *   - a compressed block is visible to position p only once it is complete,
 *     (j + 1) * block <= p + 1: the causal mask that [P1] s4 puts on the
 *     block summaries, read so that no summary mixes in a future token;
 *   - the "score" summed over a group's heads is each head's softmax
 *     probability over the visible blocks ([P1] s4);
 *   - forced blocks (block 0, the current block) count inside top_k; ties
 *     are broken towards the lower block index; the list is returned sorted;
 *   - the selected blocks' tokens form ONE key set with one softmax
 *     ([P1] s4: the chosen blocks' tokens are put together);
 *   - the window holds the last `window` positions up to and including p
 *     ([P5] s12: a sliding window looks at the previous 512 tokens);
 *   - the softmax scale is 1/sqrt(d_qk) in every branch unless given;
 *   - an empty key set gives a zero output;
 *   - selection blocks may be longer than compression blocks ([P1] s4 notes
 *     the two sizes can differ and leaves the mechanism open): a selection
 *     block is a run of whole compression blocks, and its importance is the
 *     sum of theirs; it is a candidate once complete, like a summary.
 */
#include "nsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- storage access ---------------------------------------------------- */

/* Widen element i of a bf16 or fp32 array to double (exact). */
static double load_elem(const void* base, int is_bf16, int64_t i) {
  if (!is_bf16) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Round x to the nearest bf16 value, ties to even.  bf16 keeps 8 significant
 * bits; its smallest step (subnormals) is 2^-133.  Done arithmetically:
 * scale so that the last kept bit is the units digit, round to an integer
 * with the default round-half-even mode, scale back. */
static double round_to_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  (void)frexp(x, &e);          /* |x| in [2^(e-1), 2^e) */
  int q = e - 8;               /* weight of the 8th significant bit */
  if (q < -133) q = -133;
  return ldexp(nearbyint(ldexp(x, -q)), q);
}

/* Store double x (already representable) into element i. */
static void store_elem(void* base, int is_bf16, int64_t i, double x) {
  if (!is_bf16) {
    ((float*)base)[i] = (float)x;  /* C conversion rounds to nearest even */
    return;
  }
  float f = (float)round_to_bf16(x);  /* exact: a bf16 value is an fp32 value */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  ((uint16_t*)base)[i] = (uint16_t)(bits >> 16);
}

static int cfg_ok(const oracle_cfg* c) {
  if (c->batch < 1 || c->q_len < 1 || c->kv_len < c->q_len) return 0;
  if (c->n_groups < 1 || c->heads_per_group < 1) return 0;
  if (c->d_qk < 1 || c->d_v < 1 || c->block < 1 || c->top_k < 0 || c->window < 0) return 0;
  if (c->sel_block < 0 || (c->sel_block > 0 && c->sel_block % c->block != 0)) return 0;
  return 1;
}

/* Tokens per selection block. */
static int64_t sel_block(const oracle_cfg* c) {
  return c->sel_block > 0 ? c->sel_block : c->block;
}

static double softmax_scale(const oracle_cfg* c) {
  return c->scale != 0.0 ? c->scale : 1.0 / sqrt((double)c->d_qk);
}

/* Natural log-sum-exp of the selected branch's scaled logits: for each
 * listed row and head, log sum_s exp(scale * q_h . k_s) over the same key set
 * as the selected branch of oracle_attend (every position s <= p of the
 * chosen blocks, [P1] s4), -inf when that set is empty.  The softmax's
 * normaliser, so that the branch's weights are exp(scale q.k_s - lse).
 * Taken with the largest logit factored out, so no exp overflows. */
int oracle_selected_lse(const oracle_cfg* c, const void* q, const void* k, const int32_t* idx,
                        const int64_t* rows, int64_t nrows, double* lse) {
  if (!cfg_ok(c)) return ORACLE_BAD_CONFIG;
  const int64_t T = c->q_len, L = c->kv_len, G = c->n_groups, hpg = c->heads_per_group;
  const int64_t H = G * hpg, dq = c->d_qk, bs = sel_block(c), n = c->top_k;
  const double scale = softmax_scale(c);
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t b = rows[r] / T, t = rows[r] % T;
    const int64_t p = L - T + t;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n * bs + 1));
    double* z = (double*)malloc(sizeof(double) * (size_t)(n * bs + 1));
    if (!keys || !z) {
      bad = 1;
      free(keys); free(z);
      continue;
    }
    for (int64_t g = 0; g < G; ++g) {
      const int32_t* sel = idx + (r * G + g) * n;
      int64_t nk = 0;
      for (int64_t i = 0; i < n; ++i) {
        const int64_t j = sel[i];
        if (j < 0) continue;
        for (int64_t i2 = 0; i2 < i; ++i2)
          if (sel[i2] == j) bad = 2;
        if (j * bs > p) { bad = 2; continue; }
        for (int64_t s = j * bs; s < (j + 1) * bs && s <= p; ++s) keys[nk++] = s;
      }
      for (int64_t hh = 0; hh < hpg; ++hh) {
        const int64_t h = g * hpg + hh;
        if (nk == 0) {
          lse[r * H + h] = -INFINITY;
          continue;
        }
        double m = -INFINITY;
        for (int64_t i = 0; i < nk; ++i) {
          double dot = 0.0;
          for (int64_t d = 0; d < dq; ++d)
            dot += load_elem(q, c->is_bf16, ((b * T + t) * H + h) * dq + d) *
                   load_elem(k, c->is_bf16, ((b * L + keys[i]) * G + g) * dq + d);
          z[i] = scale * dot;
          if (z[i] > m) m = z[i];
        }
        double sum = 0.0;
        for (int64_t i = 0; i < nk; ++i) sum += exp(z[i] - m);
        lse[r * H + h] = m + log(sum);
      }
    }
    free(keys); free(z);
  }
  if (bad == 2) return ORACLE_BAD_SELECTION;
  return bad ? ORACLE_BAD_CONFIG : ORACLE_OK;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- step 1: block compression ([P1] s4, s7) --------------------------- */

int oracle_pool(const oracle_cfg* c, const void* k, const void* v, void* kc, void* vc) {
  if (!cfg_ok(c)) return ORACLE_BAD_CONFIG;
  const int64_t B = c->batch, L = c->kv_len, G = c->n_groups, bs = c->block;
  const int64_t nb = L / bs;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t j = 0; j < nb; ++j)
      for (int64_t g = 0; g < G; ++g) {
        for (int64_t d = 0; d < c->d_qk; ++d) {
          double sum = 0.0;  /* token order, one add at a time */
          for (int64_t s = j * bs; s < (j + 1) * bs; ++s)
            sum += load_elem(k, c->is_bf16, ((b * L + s) * G + g) * c->d_qk + d);
          store_elem(kc, c->is_bf16, ((b * nb + j) * G + g) * c->d_qk + d, sum / (double)bs);
        }
        for (int64_t d = 0; d < c->d_v; ++d) {
          double sum = 0.0;
          for (int64_t s = j * bs; s < (j + 1) * bs; ++s)
            sum += load_elem(v, c->is_bf16, ((b * L + s) * G + g) * c->d_v + d);
          store_elem(vc, c->is_bf16, ((b * nb + j) * G + g) * c->d_v + d, sum / (double)bs);
        }
      }
  return ORACLE_OK;
}

/* ---- steps 2-4: compressed branch, group importance, top-k ------------- */

typedef struct { double score; int32_t block; } cand_t;

/* Higher importance first; equal importance: lower block index first. */
static int cand_order(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->block > y->block) - (x->block < y->block);
}

static int int_order(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int oracle_select(const oracle_cfg* c, const void* q, const void* kc, const void* vc,
                  const int64_t* rows, int64_t nrows,
                  int32_t* idx, double* imp, double* o_cmp) {
  if (!cfg_ok(c)) return ORACLE_BAD_CONFIG;
  const int64_t T = c->q_len, L = c->kv_len, G = c->n_groups, hpg = c->heads_per_group;
  const int64_t H = G * hpg, dq = c->d_qk, dv = c->d_v, bs = c->block, n = c->top_k;
  const int64_t nb = L / bs;
  const int64_t bsel = sel_block(c), per = bsel / bs;  /* compression blocks per selection block */
  const int64_t nbs = L / bsel;
  const double scale = softmax_scale(c);
  const int64_t n_forced_max = (c->force_first ? 1 : 0) + (c->force_current ? 1 : 0);
  if (n < n_forced_max) return ORACLE_BAD_CONFIG;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t b = rows[r] / T, t = rows[r] % T;
    const int64_t p = L - T + t;               /* absolute query position */
    const int64_t nvis = (p + 1) / bs;         /* summaries j with (j+1)*bs <= p+1 */
    const int64_t nvis_s = (p + 1) / bsel;     /* complete selection blocks */
    const int64_t cur = p / bsel;              /* the query's own selection block */
    double* z = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    double* importance = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    double* imp_sel = (double*)malloc(sizeof(double) * (size_t)(nbs > 0 ? nbs : 1));
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nbs > 0 ? nbs : 1));
    if (!z || !importance || !imp_sel || !cand) {
      bad = 1; free(z); free(importance); free(imp_sel); free(cand); continue;
    }

    for (int64_t g = 0; g < G; ++g) {
      for (int64_t j = 0; j < nb; ++j) importance[j] = 0.0;

      for (int64_t hh = 0; hh < hpg; ++hh) {
        const int64_t h = g * hpg + hh;
        /* compressed attention of head h over the visible block summaries */
        double m = -INFINITY;
        for (int64_t j = 0; j < nvis; ++j) {
          double dot = 0.0;
          for (int64_t d = 0; d < dq; ++d)
            dot += load_elem(q, c->is_bf16, ((b * T + t) * H + h) * dq + d) *
                   load_elem(kc, c->is_bf16, ((b * nb + j) * G + g) * dq + d);
          z[j] = scale * dot;
          if (z[j] > m) m = z[j];
        }
        double denom = 0.0;
        for (int64_t j = 0; j < nvis; ++j) denom += exp(z[j] - m);
        /* z[j] becomes the probability P[h, j] */
        for (int64_t j = 0; j < nvis; ++j) z[j] = exp(z[j] - m) / denom;

        if (o_cmp) {
          for (int64_t e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int64_t j = 0; j < nvis; ++j)
              acc += z[j] * load_elem(vc, c->is_bf16, ((b * nb + j) * G + g) * dv + e);
            o_cmp[(r * H + h) * dv + e] = acc;  /* 0 when no block is visible */
          }
        }
        /* the group's importance: the heads' probabilities added up ([P1] s4) */
        for (int64_t j = 0; j < nvis; ++j) importance[j] += z[j];
      }

      /* a selection block's importance: the sum over its summaries (all
         visible once the selection block is complete) */
      for (int64_t J = 0; J < nvis_s; ++J) {
        double s = 0.0;
        for (int64_t i = J * per; i < (J + 1) * per; ++i) s += importance[i];
        imp_sel[J] = s;
      }
      if (imp)
        for (int64_t J = 0; J < nbs; ++J)
          imp[(r * G + g) * nbs + J] = J < nvis_s ? imp_sel[J] : NAN;

      /* forced blocks, then the best of the remaining complete blocks */
      int32_t* sel = idx + (r * G + g) * n;
      int64_t cnt = 0;
      if (c->force_first) sel[cnt++] = 0;
      if (c->force_current && !(c->force_first && cur == 0)) sel[cnt++] = (int32_t)cur;
      int64_t ncand = 0;
      for (int64_t J = 0; J < nvis_s; ++J) {
        int forced = 0;
        for (int64_t f = 0; f < cnt; ++f) forced |= (sel[f] == J);
        if (!forced) { cand[ncand].score = imp_sel[J]; cand[ncand].block = (int32_t)J; ++ncand; }
      }
      qsort(cand, (size_t)ncand, sizeof(cand_t), cand_order);
      for (int64_t i = 0; i < ncand && cnt < n; ++i) sel[cnt++] = cand[i].block;
      qsort(sel, (size_t)cnt, sizeof(int32_t), int_order);
      for (int64_t i = cnt; i < n; ++i) sel[i] = -1;
    }
    free(z); free(importance); free(imp_sel); free(cand);
  }
  return bad ? ORACLE_BAD_CONFIG : ORACLE_OK;
}

/* ---- steps 5-7: selected branch, window branch, gated sum -------------- */

/* Softmax attention of one head over the keys s in `keys` (count nk):
 * out[e] = sum_s softmax_s(scale * q.k_s) * v_s[e]; zero for an empty set.
 * `weight` is caller-provided room for nk doubles. */
static void attend_keys(const oracle_cfg* c, const void* q, const void* k, const void* v,
                        int64_t b, int64_t t, int64_t h, int64_t g,
                        const int64_t* keys, int64_t nk, double* weight, double* out) {
  const int64_t T = c->q_len, L = c->kv_len, G = c->n_groups;
  const int64_t H = G * c->heads_per_group, dq = c->d_qk, dv = c->d_v;
  const double scale = softmax_scale(c);
  for (int64_t e = 0; e < dv; ++e) out[e] = 0.0;
  if (nk == 0) return;
  double m = -INFINITY;
  for (int64_t i = 0; i < nk; ++i) {
    double dot = 0.0;
    for (int64_t d = 0; d < dq; ++d)
      dot += load_elem(q, c->is_bf16, ((b * T + t) * H + h) * dq + d) *
             load_elem(k, c->is_bf16, ((b * L + keys[i]) * G + g) * dq + d);
    weight[i] = scale * dot;
    if (weight[i] > m) m = weight[i];
  }
  double denom = 0.0;
  for (int64_t i = 0; i < nk; ++i) denom += exp(weight[i] - m);
  for (int64_t i = 0; i < nk; ++i) weight[i] = exp(weight[i] - m) / denom;
  for (int64_t e = 0; e < dv; ++e) {
    double acc = 0.0;
    for (int64_t i = 0; i < nk; ++i)
      acc += weight[i] * load_elem(v, c->is_bf16, ((b * L + keys[i]) * G + g) * dv + e);
    out[e] = acc;
  }
}

static double gate_value(const oracle_cfg* c, const void* gates, int64_t b, int64_t t,
                         int64_t h, int branch) {
  const int64_t T = c->q_len, H = (int64_t)c->n_groups * c->heads_per_group;
  double x = load_elem(gates, c->is_bf16, ((b * T + t) * H + h) * 3 + branch);
  return c->gate_logits ? 1.0 / (1.0 + exp(-x)) : x;
}

int oracle_attend(const oracle_cfg* c, const void* q, const void* k, const void* v,
                  const void* gates, const int32_t* idx, const double* o_cmp,
                  const int64_t* rows, int64_t nrows,
                  double* out, double* o_slc, double* o_win) {
  if (!cfg_ok(c)) return ORACLE_BAD_CONFIG;
  const int64_t T = c->q_len, L = c->kv_len, G = c->n_groups, hpg = c->heads_per_group;
  const int64_t H = G * hpg, dv = c->d_v, bs = sel_block(c), n = c->top_k;
  const int n_branches = (c->use_cmp != 0) + (c->use_slc != 0) + (c->use_win != 0);
  if (!gates && n_branches > 1) return ORACLE_BAD_CONFIG;
  if (c->use_cmp && !o_cmp) return ORACLE_BAD_CONFIG;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t b = rows[r] / T, t = rows[r] % T;
    const int64_t p = L - T + t;                 /* absolute query position */
    const int64_t cap = n * bs + c->window + 1;  /* room for both key sets */
    int64_t* skeys = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    int64_t* wkeys = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    double* weight = (double*)malloc(sizeof(double) * (size_t)cap);
    double* slc = (double*)malloc(sizeof(double) * (size_t)dv);
    double* win = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!skeys || !wkeys || !weight || !slc || !win) {
      bad = 1;
      free(skeys); free(wkeys); free(weight); free(slc); free(win);
      continue;
    }

    for (int64_t g = 0; g < G; ++g) {
      /* selected key set ([P1] s4): every position s <= p of a chosen block */
      const int32_t* sel = idx + (r * G + g) * n;
      int64_t nsel = 0;
      for (int64_t i = 0; i < n; ++i) {
        const int64_t j = sel[i];
        if (j < 0) continue;
        for (int64_t i2 = 0; i2 < i; ++i2)
          if (sel[i2] == j) bad = 2;     /* a selection is a set */
        if (j * bs > p) { bad = 2; continue; }  /* a chosen block must have begun */
        for (int64_t s = j * bs; s < (j + 1) * bs && s <= p; ++s) skeys[nsel++] = s;
      }
      /* window key set ([P5] s12): positions p - window < s <= p */
      int64_t nwin = 0;
      for (int64_t s = (p - c->window + 1 > 0 ? p - c->window + 1 : 0); c->window > 0 && s <= p; ++s)
        wkeys[nwin++] = s;

      for (int64_t hh = 0; hh < hpg; ++hh) {
        const int64_t h = g * hpg + hh;
        /* each branch has its own softmax ([P1] s4: three separate outputs) */
        attend_keys(c, q, k, v, b, t, h, g, skeys, nsel, weight, slc);
        attend_keys(c, q, k, v, b, t, h, g, wkeys, nwin, weight, win);
        /* gated sum of the branch outputs ([P1] s4) */
        for (int64_t e = 0; e < dv; ++e) {
          double acc = 0.0;
          if (c->use_cmp) acc += (gates ? gate_value(c, gates, b, t, h, 0) : 1.0) * o_cmp[(r * H + h) * dv + e];
          if (c->use_slc) acc += (gates ? gate_value(c, gates, b, t, h, 1) : 1.0) * slc[e];
          if (c->use_win) acc += (gates ? gate_value(c, gates, b, t, h, 2) : 1.0) * win[e];
          out[(r * H + h) * dv + e] = acc;
          if (o_slc) o_slc[(r * H + h) * dv + e] = slc[e];
          if (o_win) o_win[(r * H + h) * dv + e] = win[e];
        }
      }
    }
    free(skeys); free(wkeys); free(weight); free(slc); free(win);
  }
  if (bad == 2) return ORACLE_BAD_SELECTION;
  return bad ? ORACLE_BAD_CONFIG : ORACLE_OK;
}
