/*
 * Test driver: runs the C oracle (oracle/nsa_oracle.c, linked in with
 * AddressSanitizer and UndefinedBehaviorSanitizer) over small seeded inputs
 * whose shapes reach its edge cases: queries before the first complete block,
 * ragged key counts, queries at the end of a longer cache, decoupled
 * selection blocks, padded selections, a window longer than the sequence,
 * one branch without gates, bf16 storage.  Any out-of-bounds access or
 * undefined operation aborts with a sanitizer report; the driver itself only
 * checks the return codes.  Built and run by tests/test_oracle_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nsa_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {  /* xorshift64*, uniform in [0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}

static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* n values of N(0,1)-ish (sum of uniforms), stored as fp32 or bf16 patterns. */
static void *fill(size_t n, int bf16, double lo, double hi) {
  void *p = malloc(n * (bf16 ? 2 : 4));
  for (size_t i = 0; i < n; ++i) {
    const float x = (float)(lo + (hi - lo) * urand());
    if (bf16) ((uint16_t *)p)[i] = to_bf16(x);
    else ((float *)p)[i] = x;
  }
  return p;
}

static int run(const char *name, oracle_cfg c) {
  const int64_t B = c.batch, T = c.q_len, L = c.kv_len, G = c.n_groups, H = G * c.heads_per_group;
  const int64_t nb = L / c.block, sb = c.sel_block ? c.sel_block : c.block, nbs = L / sb;
  const int bf = c.is_bf16;
  void *q = fill((size_t)(B * T * H * c.d_qk), bf, -2, 2);
  void *k = fill((size_t)(B * L * G * c.d_qk), bf, -2, 2);
  void *v = fill((size_t)(B * L * G * c.d_v), bf, -2, 2);
  void *gates = fill((size_t)(B * T * H * 3), bf, 0, 1);
  const int nbr = c.use_cmp + c.use_slc + c.use_win;
  void *kc = malloc((size_t)((nb ? nb : 1) * B * G * c.d_qk * (bf ? 2 : 4)));
  void *vc = malloc((size_t)((nb ? nb : 1) * B * G * c.d_v * (bf ? 2 : 4)));
  const int64_t nrows = B * T;
  int64_t *rows = malloc((size_t)nrows * sizeof(int64_t));
  for (int64_t r = 0; r < nrows; ++r) rows[r] = r;
  int32_t *idx = malloc((size_t)(nrows * G * c.top_k) * sizeof(int32_t));
  double *imp = malloc((size_t)(nrows * G * (nbs ? nbs : 1)) * sizeof(double));
  double *ocmp = malloc((size_t)(nrows * H * c.d_v) * sizeof(double));
  double *out = malloc((size_t)(nrows * H * c.d_v) * sizeof(double));
  double *oslc = malloc((size_t)(nrows * H * c.d_v) * sizeof(double));
  double *owin = malloc((size_t)(nrows * H * c.d_v) * sizeof(double));
  int rc = oracle_pool(&c, k, v, kc, vc);
  if (rc == ORACLE_OK) rc = oracle_select(&c, q, kc, vc, rows, nrows, idx, imp, ocmp);
  if (rc == ORACLE_OK)
    rc = oracle_attend(&c, q, k, v, nbr > 1 ? gates : NULL, idx, c.use_cmp ? ocmp : NULL, rows, nrows, out, oslc,
                       owin);
  double sum = 0.0;
  for (int64_t i = 0; rc == ORACLE_OK && i < nrows * H * c.d_v; ++i) sum += fabs(out[i]);
  printf("%-40s rc=%d sum|out|=%.6g\n", name, rc, sum);
  free(q); free(k); free(v); free(gates); free(kc); free(vc); free(rows); free(idx); free(imp);
  free(ocmp); free(out); free(oslc); free(owin);
  return rc;
}

int main(void) {
  oracle_cfg base = {0};
  base.batch = 1; base.q_len = 40; base.kv_len = 40; base.n_groups = 2; base.heads_per_group = 3;
  base.d_qk = 8; base.d_v = 6; base.block = 8; base.top_k = 3; base.window = 12;
  base.force_first = 1; base.force_current = 1; base.use_cmp = 1; base.use_slc = 1; base.use_win = 1;
  int bad = 0;
  oracle_cfg c;
  c = base; bad |= run("three branches fp32", c);
  c = base; c.is_bf16 = 1; c.gate_logits = 1; bad |= run("bf16, gate logits", c);
  c = base; c.q_len = 5; c.kv_len = 5; bad |= run("no complete block", c);
  c = base; c.q_len = 13; c.kv_len = 45; bad |= run("queries at the end, ragged", c);
  c = base; c.batch = 2; c.kv_len = 43; c.q_len = 43; c.top_k = 5; bad |= run("two sequences, padded top-k", c);
  c = base; c.window = 100; bad |= run("window longer than the sequence", c);
  c = base; c.use_cmp = 0; c.use_win = 0; bad |= run("selected branch alone, no gates", c);
  c = base; c.sel_block = 16; c.q_len = 50; c.kv_len = 50; bad |= run("decoupled selection blocks", c);
  c = base; c.force_first = 0; c.force_current = 0; c.top_k = 2; bad |= run("no forced blocks", c);
  c = base; c.n_groups = 1; c.heads_per_group = 1; c.block = 16; c.top_k = 2; c.force_first = 0;
  c.use_cmp = 0; c.use_win = 0; c.q_len = 60; c.kv_len = 70; bad |= run("MoBA-like, one head per group", c);
  return bad ? 1 : 0;
}
