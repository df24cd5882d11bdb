/*
 * sv_oracle.c — plain, slow CPU oracle of the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. It shares no code, header, table
 * or constant generator with the GPU library; it is written from the pages:
 *   [SB] "7.6 Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead":
 *        "The rule", "The proof that this is exact", "Extending to a chain of
 *        γ draft tokens", "A From-Scratch Implementation" (apply_temperature,
 *        speculative_step), "Tree Attention", Exercises 4 and 5;
 *   [DM] "Speculative Decoding: Draft Models, EAGLE, and How to Actually Use
 *        It": "The Algorithm";
 *   [SS] "Medusa, EAGLE and self-speculation": "Copying, verified against plain
 *        greedy".
 * Everything is computed in double precision from the exact decode of the
 * stored logits (fp32 values, or bf16 bits shifted into an fp32), with plain
 * loops and no blocking or reordering beyond the definitions.
 *
 * Readings fixed where the pages are silent (the GPU library follows the same
 * written conventions, in its own code):
 *  - one temperature per sequence scales both its target and draft rows;
 *    temperature 0 selects greedy verification;
 *  - argmax ties go to the lowest index;
 *  - the accept test is u < a with u = (w >> 8) * 2^-24;
 *  - samples of the residual (p - q)_+ and of the bonus distribution p are
 *    drawn by Gumbel-max with G = -ln(-ln U), U = ((w >> 8) + 0.5) * 2^-24;
 *  - random words come from Philox4x32-10 with key (seed_lo, seed_hi) and
 *    counter (c0, position, sequence, 2*offset + stream);
 *  - an empty residual (only reachable through rounding) falls back to p;
 *  - a tree accepts its deepest valid node, smallest index among equals;
 *  - sampled trees ([SB] "Tree Attention", multi-round rejection sampling):
 *    the children of a node are i.i.d. draws from the draft distribution at
 *    that node (draft row = the node), tested in index order; the accept
 *    uniform of the j-th tested sibling under node v uses counter word 0 = j
 *    and position v, and a draw at node v uses position v, so a tree shaped
 *    like a chain verifies exactly as the chain.
 * Parity unpinned by the pages: the Philox counter layout, the word-to-float
 * maps, the Gumbel transform, the tie rule and the empty-residual fallback are
 * this library's written convention. The tests pin the distribution they
 * produce (exact enumeration, chi-square, closed forms), not single samples.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "sv_oracle.h"

/* ------------------------------------------------------------------------ */
/* Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as   */
/* easy as 1, 2, 3" (SC'11). Ten rounds of the 4x32 S-box; the key is bumped */
/* by the Weyl constants between rounds.                                     */
/* ------------------------------------------------------------------------ */
#define OR_PHILOX_M0 0xD2511F53u
#define OR_PHILOX_M1 0xCD9E8D57u
#define OR_PHILOX_W0 0x9E3779B9u
#define OR_PHILOX_W1 0xBB67AE85u

void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += OR_PHILOX_W0;
      k1 += OR_PHILOX_W1;
    }
    uint64_t p0 = (uint64_t)OR_PHILOX_M0 * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)OR_PHILOX_M1 * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    uint32_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
  out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

static void or_words(uint64_t seed, uint32_t c0, uint32_t position, uint32_t seq, uint32_t c3,
                     uint32_t out[4]) {
  uint32_t ctr[4] = {c0, position, seq, c3};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  or_philox4x32_10(ctr, key, out);
}

/* Accept uniform u_i of sequence b at position i: stream 0, word 0. */
double or_accept_uniform(uint64_t seed, uint64_t offset, int32_t b, int32_t i) {
  uint32_t w[4];
  or_words(seed, 0u, (uint32_t)i, (uint32_t)b, (uint32_t)(2u * (uint32_t)offset), w);
  return (double)(w[0] >> 8) * (1.0 / 16777216.0);
}

/* Gumbel noise of vocab entry v for sequence b at position pos: stream 1. */
double or_gumbel(uint64_t seed, uint64_t offset, int32_t b, int32_t pos, int32_t v) {
  uint32_t w[4];
  or_words(seed, (uint32_t)v / 4u, (uint32_t)pos, (uint32_t)b, (uint32_t)(2u * (uint32_t)offset + 1u), w);
  double U = ((double)(w[v % 4] >> 8) + 0.5) * (1.0 / 16777216.0);
  return -log(-log(U));
}

/* ------------------------------------------------------------------------ */
/* Logit rows                                                                */
/* ------------------------------------------------------------------------ */
static double or_decode(const void* base, int dtype, int64_t idx) {
  if (dtype == OR_DTYPE_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * idx, 4);
    return (double)f;
  }
  uint16_t h;
  memcpy(&h, (const char*)base + 2 * idx, 2);
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* Row r (global row number) of a [rows, stride] tensor, decoded to fp64. */
static void or_load_row(const void* base, int dtype, int64_t stride, int64_t r, int32_t V,
                        double* dst) {
  for (int32_t v = 0; v < V; ++v) dst[v] = or_decode(base, dtype, r * stride + v);
}

/* ln sum_v exp(y_v) with the max taken out first ([SB] apply_temperature:
 * softmax(logits / T); this is its log-normalizer). */
static double or_logsumexp(const double* y, int32_t V) {
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v)
    if (y[v] > m) m = y[v];
  double s = 0.0;
  for (int32_t v = 0; v < V; ++v) s += exp(y[v] - m);
  return m + log(s);
}

/* Lowest index of the maximum. */
static int32_t or_argmax(const double* y, int32_t V) {
  int32_t best = 0;
  for (int32_t v = 1; v < V; ++v)
    if (y[v] > y[best]) best = v;
  return best;
}

/* Track the best and second-best score of a Gumbel-max draw. */
typedef struct {
  double s1, s2;
  int32_t v1;
} or_top2_t;

static void or_top2_init(or_top2_t* t) {
  t->s1 = -INFINITY;
  t->s2 = -INFINITY;
  t->v1 = -1;
}

static void or_top2_push(or_top2_t* t, double s, int32_t v) {
  if (s > t->s1) { /* strict: the lowest index wins exact ties */
    t->s2 = t->s1;
    t->s1 = s;
    t->v1 = v;
  } else if (s > t->s2) {
    t->s2 = s;
  }
}

static double or_top2_gap(const or_top2_t* t) {
  if (!isfinite(t->s2)) return INFINITY;
  double den = fmax(fmax(fabs(t->s1), fabs(t->s2)), 1.0);
  return (t->s1 - t->s2) / den;
}

static void or_set(double* a, int64_t i, double v) {
  if (a) a[i] = v;
}

/* ------------------------------------------------------------------------ */
/* Chains                                                                    */
/* ------------------------------------------------------------------------ */

/* Greedy verification of one sequence ([SB] "Extending to a chain of γ draft
 * tokens", temperature 0; [SS] speculative_greedy): accept while the drafted
 * token equals the target argmax of its row; then emit the argmax of the first
 * mismatching row (correction) or of row gamma (bonus). */
static void or_greedy_one(const void* target, int64_t tstride, int dtype, const int32_t* ids,
                          int32_t b, int32_t gamma, int32_t V, double* row, int32_t* out_tokens,
                          int32_t* out_n, double* accept_prob) {
  int32_t n = gamma;
  int32_t g_stop = -1;
  for (int32_t i = 0; i < gamma; ++i) {
    or_load_row(target, dtype, tstride, (int64_t)b * (gamma + 1) + i, V, row);
    int32_t g = or_argmax(row, V);
    int match = (ids[i] == g);
    or_set(accept_prob, (int64_t)b * gamma + i, match ? 1.0 : 0.0);
    if (!match && n == gamma) {
      n = i;
      g_stop = g;
    }
  }
  if (n == gamma) {
    or_load_row(target, dtype, tstride, (int64_t)b * (gamma + 1) + gamma, V, row);
    g_stop = or_argmax(row, V);
  }
  for (int32_t i = 0; i < n; ++i) out_tokens[i] = ids[i];
  out_tokens[n] = g_stop;
  *out_n = n;
}

static void or_fill_bad(int32_t* out_tokens, int32_t gamma, int32_t* out_n, int32_t code) {
  for (int32_t i = 0; i <= gamma; ++i) out_tokens[i] = -1;
  *out_n = code;
}

/* Whether softmax(row / T) is a probability distribution: some entry above
 * -inf, and none NaN or +inf. (-inf entries are tokens of probability 0.) */
static int or_row_has_softmax(const void* base, int dtype, int64_t stride, int64_t r, int32_t V) {
  int finite = 0;
  for (int32_t v = 0; v < V; ++v) {
    const double l = or_decode(base, dtype, r * stride + v);
    if (isnan(l) || l == INFINITY) return 0;
    if (l > -INFINITY) finite = 1;
  }
  return finite;
}

/* Sampled verification of one sequence. Steps follow [SB] speculative_step:
 * (1) normalize target and draft rows with the temperature, (2) walk the
 * drafts left to right, accepting x_i with probability min(1, p_i(x_i)/q_i(x_i)),
 * (3) on the first rejection draw the replacement from (p - q)_+ and stop,
 * (4) if nothing was rejected draw the bonus token from p at row gamma. */
static void or_sample_one(const void* target, int64_t tstride, const void* draft, int64_t dstride,
                          int dtype, const int32_t* ids, double T, int32_t b, int32_t gamma,
                          int32_t V, uint64_t seed, uint64_t offset, const double* u_override,
                          double* yp, double* yq, int32_t* out_tokens, int32_t* out_n,
                          or_diag_t* d) {
  const int one_hot = (draft == NULL);
  double logzp[OR_MAX_GAMMA], logzq[OR_MAX_GAMMA];
  int accept[OR_MAX_GAMMA];
  int32_t flags = 0;

  /* Steps (1)-(2): all gamma positions are scored; the walk stops at the
   * first rejection. */
  int32_t n = gamma;
  for (int32_t i = 0; i < gamma; ++i) {
    const int32_t x = ids[i];
    or_load_row(target, dtype, tstride, (int64_t)b * (gamma + 1) + i, V, yp);
    for (int32_t v = 0; v < V; ++v) yp[v] /= T;
    logzp[i] = or_logsumexp(yp, V);
    double lp_x = yp[x] - logzp[i];
    double lq_x = 0.0; /* one-hot draft: q(x) = 1 */
    if (!one_hot) {
      or_load_row(draft, dtype, dstride, (int64_t)b * gamma + i, V, yq);
      for (int32_t v = 0; v < V; ++v) yq[v] /= T;
      logzq[i] = or_logsumexp(yq, V);
      lq_x = yq[x] - logzq[i];
    } else {
      logzq[i] = NAN;
    }
    /* a = min(1, p/q), in the log domain so that q(x) -> 0 gives a = 1. */
    double a = exp(fmin(0.0, lp_x - lq_x));
    double u = u_override ? u_override[(int64_t)b * gamma + i]
                          : or_accept_uniform(seed, offset, b, i);
    accept[i] = (u < a);
    or_set(d ? d->accept_prob : NULL, (int64_t)b * gamma + i, a);
    or_set(d ? d->uniforms : NULL, (int64_t)b * gamma + i, u);
    or_set(d ? d->logz_target : NULL, (int64_t)b * gamma + i, logzp[i]);
    or_set(d ? d->logz_draft : NULL, (int64_t)b * gamma + i, logzq[i]);
    if (n == gamma) {
      if (fabs(u - a) < OR_KNIFE_EDGE) flags |= OR_FLAG_KNIFE_EDGE;
      if (!accept[i]) n = i;
    }
  }

  or_top2_t top;
  or_top2_init(&top);
  double beta = NAN;
  if (n < gamma) {
    /* Step (3): residual (p - q)_+ at the first rejected position n. */
    const int32_t x = ids[n];
    or_load_row(target, dtype, tstride, (int64_t)b * (gamma + 1) + n, V, yp);
    for (int32_t v = 0; v < V; ++v) yp[v] /= T;
    if (!one_hot) {
      or_load_row(draft, dtype, dstride, (int64_t)b * gamma + n, V, yq);
      for (int32_t v = 0; v < V; ++v) yq[v] /= T;
    }
    beta = 0.0;
    for (int32_t v = 0; v < V; ++v) {
      double lp = yp[v] - logzp[n];
      double score;
      if (one_hot) {
        if (v == x) continue; /* (p - delta_x)_+ vanishes at x */
        score = yp[v];
        beta += exp(lp);
      } else {
        double lq = yq[v] - logzq[n];
        if (!(lp > lq)) continue; /* outside the support of (p - q)_+ */
        double lr = lp + log(-expm1(lq - lp)); /* ln(p - q) */
        score = lr;
        beta += exp(lr);
      }
      or_top2_push(&top, score + or_gumbel(seed, offset, b, n, v), v);
    }
    if (top.v1 < 0) {
      /* Empty residual: draw from p at the rejected position instead. */
      flags |= OR_FLAG_FALLBACK;
      for (int32_t v = 0; v < V; ++v) or_top2_push(&top, yp[v] + or_gumbel(seed, offset, b, n, v), v);
    }
  } else {
    /* Step (4): bonus token from p at row gamma. */
    or_load_row(target, dtype, tstride, (int64_t)b * (gamma + 1) + gamma, V, yp);
    for (int32_t v = 0; v < V; ++v) {
      yp[v] /= T;
      or_top2_push(&top, yp[v] + or_gumbel(seed, offset, b, gamma, v), v);
    }
  }

  for (int32_t i = 0; i < n; ++i) out_tokens[i] = ids[i];
  out_tokens[n] = top.v1;
  for (int32_t i = n + 1; i <= gamma; ++i) out_tokens[i] = -1;
  *out_n = n;
  /* A draw over a row without a finite entry (only the bonus row can be one:
   * the rows scored above were checked) has nothing to draw. */
  if (top.v1 < 0) or_fill_bad(out_tokens, gamma, out_n, OR_SEQ_BAD_LOGITS);
  if (d) {
    or_set(d->residual_mass, b, beta);
    or_set(d->top_gap, b, or_top2_gap(&top));
    or_set(d->top_score, b, top.s1);
    if (d->flags) d->flags[b] = flags;
  }
}

int or_verify_sample(const void* target, int64_t tstride, const void* draft, int64_t dstride,
                     int dtype, const int32_t* draft_ids, const float* temperature, int32_t B,
                     int32_t gamma, int32_t V, uint64_t seed, uint64_t offset,
                     const double* u_override, int32_t* out_tokens, int32_t* out_n, or_diag_t* d,
                     int nthreads) {
  if (!target || !draft_ids || !temperature || !out_tokens || !out_n) return 1;
  if (B < 0 || gamma < 1 || gamma > OR_MAX_GAMMA || V < 1) return 2;
  if (dtype != OR_DTYPE_F32 && dtype != OR_DTYPE_BF16) return 3;
  if (tstride < V || (draft && dstride < V)) return 4;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* yp = (double*)malloc(sizeof(double) * (size_t)V);
    double* yq = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
      const int32_t* ids = draft_ids + (int64_t)b * gamma;
      int32_t* tok = out_tokens + (int64_t)b * (gamma + 1);
      const double T = (double)temperature[b];
      int bad_id = 0;
      for (int32_t i = 0; i < gamma; ++i)
        if (ids[i] < 0 || ids[i] >= V) bad_id = 1;
      if (d) {
        for (int32_t i = 0; i < gamma; ++i) {
          or_set(d->accept_prob, (int64_t)b * gamma + i, NAN);
          or_set(d->uniforms, (int64_t)b * gamma + i, NAN);
          or_set(d->logz_target, (int64_t)b * gamma + i, NAN);
          or_set(d->logz_draft, (int64_t)b * gamma + i, NAN);
        }
        or_set(d->residual_mass, b, NAN);
        or_set(d->top_gap, b, INFINITY);
        or_set(d->top_score, b, NAN);
        if (d->flags) d->flags[b] = 0;
      }
      if (!(T >= 0.0) || isinf(T)) {
        or_fill_bad(tok, gamma, &out_n[b], OR_SEQ_BAD_TEMPERATURE);
      } else if (bad_id) {
        or_fill_bad(tok, gamma, &out_n[b], OR_SEQ_BAD_TOKEN);
      } else if (T == 0.0) {
        for (int32_t i = 0; i <= gamma; ++i) tok[i] = -1;
        or_greedy_one(target, tstride, dtype, ids, b, gamma, V, yp, tok, &out_n[b],
                      d ? d->accept_prob : NULL);
      } else {
        /* Every row the accept tests read must define a distribution. */
        int rows_ok = 1;
        for (int32_t i = 0; i < gamma && rows_ok; ++i) {
          rows_ok &= or_row_has_softmax(target, dtype, tstride, (int64_t)b * (gamma + 1) + i, V);
          if (draft) rows_ok &= or_row_has_softmax(draft, dtype, dstride, (int64_t)b * gamma + i, V);
        }
        if (!rows_ok)
          or_fill_bad(tok, gamma, &out_n[b], OR_SEQ_BAD_LOGITS);
        else
          or_sample_one(target, tstride, draft, dstride, dtype, ids, T, b, gamma, V, seed, offset,
                        u_override, yp, yq, tok, &out_n[b], d);
      }
    }
    free(yp);
    free(yq);
  }
  return 0;
}

int or_verify_greedy(const void* target, int64_t tstride, int dtype, const int32_t* draft_ids,
                     int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens, int32_t* out_n,
                     int nthreads) {
  if (!target || !draft_ids || !out_tokens || !out_n) return 1;
  if (B < 0 || gamma < 1 || gamma > OR_MAX_GAMMA || V < 1) return 2;
  if (dtype != OR_DTYPE_F32 && dtype != OR_DTYPE_BF16) return 3;
  if (tstride < V) return 4;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
      const int32_t* ids = draft_ids + (int64_t)b * gamma;
      int32_t* tok = out_tokens + (int64_t)b * (gamma + 1);
      int bad_id = 0;
      for (int32_t i = 0; i < gamma; ++i)
        if (ids[i] < 0 || ids[i] >= V) bad_id = 1;
      for (int32_t i = 0; i <= gamma; ++i) tok[i] = -1;
      if (bad_id)
        or_fill_bad(tok, gamma, &out_n[b], OR_SEQ_BAD_TOKEN);
      else
        or_greedy_one(target, tstride, dtype, ids, b, gamma, V, row, tok, &out_n[b], NULL);
    }
    free(row);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Trees ([SB] "Tree Attention", Exercise 5)                                 */
/* ------------------------------------------------------------------------ */

/* 1 if parents/depth describe a tree in parent-before-child order with the
 * root at node 0, depths consistent and within max_depth. */
int or_tree_is_valid(const int32_t* parents, const int32_t* depth, int32_t N, int32_t max_depth) {
  if (N < 1 || parents[0] != -1 || depth[0] != 0) return 0;
  for (int32_t i = 1; i < N; ++i) {
    if (parents[i] < 0 || parents[i] >= i) return 0;
    if (depth[i] != depth[parents[i]] + 1) return 0;
    if (depth[i] > max_depth) return 0;
  }
  return 1;
}

int or_verify_tree(const void* target, int64_t tstride, int dtype, const int32_t* parents,
                   const int32_t* depth, const int32_t* node_tokens, int32_t B, int32_t N,
                   int32_t V, int32_t max_depth, int32_t* out_path, int32_t* out_path_len,
                   int32_t* out_bonus, int32_t* out_first_match_node, int nthreads) {
  if (!target || !parents || !depth || !node_tokens || !out_path || !out_path_len || !out_bonus)
    return 1;
  if (B < 0 || N < 1 || N > OR_MAX_TREE_NODES || V < 1 || max_depth < 0) return 2;
  if (dtype != OR_DTYPE_F32 && dtype != OR_DTYPE_BF16) return 3;
  if (tstride < V) return 4;
  const int tree_ok = or_tree_is_valid(parents, depth, N, max_depth);
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)V);
    int32_t* g = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    unsigned char* valid = (unsigned char*)malloc((size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
      const int32_t* tok = node_tokens + (int64_t)b * N;
      int32_t* path = out_path + (int64_t)b * (max_depth + 1);
      for (int32_t k = 0; k <= max_depth; ++k) path[k] = -1;
      out_bonus[b] = -1;
      if (out_first_match_node) out_first_match_node[b] = -1;
      if (!tree_ok) {
        out_path_len[b] = OR_SEQ_BAD_TREE;
        continue;
      }
      int bad = 0;
      for (int32_t c = 1; c < N; ++c)
        if (tok[c] < 0 || tok[c] >= V) bad = 1;
      if (bad) {
        out_path_len[b] = OR_SEQ_BAD_TOKEN;
        continue;
      }
      /* Target argmax at every node: row c predicts the token after node c. */
      for (int32_t c = 0; c < N; ++c) {
        or_load_row(target, dtype, tstride, (int64_t)b * N + c, V, row);
        g[c] = or_argmax(row, V);
      }
      /* A node survives iff every edge on its root path matches. */
      valid[0] = 1;
      for (int32_t c = 1; c < N; ++c) valid[c] = valid[parents[c]] && tok[c] == g[parents[c]];
      /* The longest surviving path ends at the deepest valid node. */
      int32_t best = 0;
      for (int32_t c = 1; c < N; ++c)
        if (valid[c] && depth[c] > depth[best]) best = c;
      int32_t len = depth[best] + 1;
      for (int32_t c = best, k = len - 1; c != -1; c = parents[c], --k) path[k] = c;
      out_path_len[b] = len;
      out_bonus[b] = g[best];
      if (out_first_match_node) {
        /* Exercise 5's walk: from the root, step to the FIRST child (index
         * order) whose token matches the parent's argmax. */
        int32_t node = 0;
        for (;;) {
          int32_t nxt = -1;
          for (int32_t c = node + 1; c < N; ++c)
            if (parents[c] == node && tok[c] == g[node]) {
              nxt = c;
              break;
            }
          if (nxt < 0) break;
          node = nxt;
        }
        out_first_match_node[b] = node;
      }
    }
    free(row);
    free(g);
    free(valid);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampled trees ([SB] "Tree Attention": multi-round rejection sampling)     */
/* ------------------------------------------------------------------------ */

/* Accept uniform of the round-th sibling tested under node `node`: stream 0,
 * word 0, counter word 0 = round. Round 0 is the chain's accept uniform of
 * position `node`, so that a tree shaped like a chain verifies as the chain. */
static double or_tree_accept_uniform(uint64_t seed, uint64_t offset, int32_t b, int32_t node,
                                     int32_t round) {
  uint32_t w[4];
  or_words(seed, (uint32_t)round, (uint32_t)node, (uint32_t)b, (uint32_t)(2u * (uint32_t)offset), w);
  return (double)(w[0] >> 8) * (1.0 / 16777216.0);
}

/* p = softmax(row / T) in fp64, from the decoded row. */
static void or_softmax(const void* base, int dtype, int64_t stride, int64_t r, int32_t V, double T,
                       double* y, double* prob) {
  or_load_row(base, dtype, stride, r, V, y);
  for (int32_t v = 0; v < V; ++v) y[v] /= T;
  const double lz = or_logsumexp(y, V);
  for (int32_t v = 0; v < V; ++v) prob[v] = exp(y[v] - lz);
}

/* One sequence. From the root, at each node v with children c_1 < ... < c_k
 * (drawn i.i.d. from q_v, the draft distribution at v): the target
 * distribution starts as p_v; child c_j is accepted with probability
 * min(1, p(x_j) / q_v(x_j)); on a rejection p is replaced by the normalized
 * residual (p - q_v)_+ / ||(p - q_v)_+||_1 and the next sibling is tested
 * against it. The first accepted child becomes the new node. A node without
 * children ends the walk with a bonus token drawn from p at that node; a node
 * whose children are all rejected ends it with a token drawn from the final
 * residual. (A residual of zero mass, reachable only through rounding, leaves
 * p as it was, as the chain's fallback draws from p.) */
static void or_tree_sample_one(const void* target, int64_t tstride, const void* draft,
                               int64_t dstride, int dtype, const int32_t* parents,
                               const int32_t* tok, double T, int32_t b, int32_t N, int32_t V,
                               int32_t max_depth, uint64_t seed, uint64_t offset, int wor, double* y,
                               double* P, double* Q, int32_t* path, int32_t* out_len,
                               int32_t* out_token, double* top_gap, int32_t* flags,
                               int32_t* rejections, double* margin) {
  int32_t node = 0, len = 1, nrej = 0, fl = 0;
  double mg = INFINITY;
  path[0] = 0;
  or_top2_t top;
  or_top2_init(&top);
  for (;;) {
    int32_t first = -1;
    for (int32_t c = node + 1; c < N; ++c)
      if (parents[c] == node) {
        first = c;
        break;
      }
    if (first < 0) {
      /* Leaf: the bonus token, from p at this node. */
      or_load_row(target, dtype, tstride, (int64_t)b * N + node, V, y);
      for (int32_t v = 0; v < V; ++v) or_top2_push(&top, y[v] / T + or_gumbel(seed, offset, b, node, v), v);
      break;
    }
    or_softmax(target, dtype, tstride, (int64_t)b * N + node, V, T, y, P);
    or_softmax(draft, dtype, dstride, (int64_t)b * N + node, V, T, y, Q);
    int32_t next = -1, round = 0, updated = 0;
    for (int32_t c = first; c < N; ++c) {
      if (parents[c] != node) continue;
      const int32_t x = tok[c];
      /* a = min(1, p(x)/q(x)); q(x) = 0 gives a = 1. */
      const double a = (Q[x] > 0.0) ? fmin(1.0, P[x] / Q[x]) : 1.0;
      const double u = or_tree_accept_uniform(seed, offset, b, node, round);
      if (fabs(u - a) < OR_KNIFE_EDGE) fl |= OR_FLAG_KNIFE_EDGE;
      if (fabs(u - a) < mg) mg = fabs(u - a);
      ++round;
      if (u < a) {
        next = c;
        break;
      }
      ++nrej;
      double Z = 0.0;
      for (int32_t v = 0; v < V; ++v) Z += fmax(P[v] - Q[v], 0.0);
      if (Z > 0.0) {
        for (int32_t v = 0; v < V; ++v) P[v] = fmax(P[v] - Q[v], 0.0) / Z;
        updated = 1;
      } else {
        fl |= OR_FLAG_FALLBACK;
      }
      if (wor) {
        /* Siblings drawn without replacement: the next one came from q over
         * the tokens not drawn yet, renormalized. */
        const double left = 1.0 - Q[x];
        Q[x] = 0.0;
        if (left > 0.0)
          for (int32_t v = 0; v < V; ++v) Q[v] /= left;
      }
    }
    if (next < 0) {
      /* Every child rejected: the replacement token from the final residual
       * (p itself if no residual had mass). */
      (void)updated;
      for (int32_t v = 0; v < V; ++v)
        if (P[v] > 0.0) or_top2_push(&top, log(P[v]) + or_gumbel(seed, offset, b, node, v), v);
      break;
    }
    node = next;
    path[len++] = node;
    if (len > max_depth + 1) break; /* cannot happen in a valid tree */
  }
  *out_len = len;
  *out_token = top.v1;
  if (top_gap) *top_gap = or_top2_gap(&top);
  if (flags) *flags = fl;
  if (rejections) *rejections = nrej;
  if (margin) *margin = mg;
}

int or_verify_tree_sample(const void* target, int64_t tstride, const void* draft, int64_t dstride,
                          int dtype, const int32_t* parents, const int32_t* depth,
                          const int32_t* node_tokens, const float* temperature, int32_t B,
                          int32_t N, int32_t V, int32_t max_depth, uint64_t seed, uint64_t offset,
                          int32_t without_replacement, int32_t* out_path, int32_t* out_path_len,
                          int32_t* out_token, double* top_gap, int32_t* flags, int32_t* rejections,
                          double* margin, int nthreads) {
  if (!target || !draft || !parents || !depth || !node_tokens || !temperature || !out_path ||
      !out_path_len || !out_token)
    return 1;
  if (B < 0 || N < 1 || N > OR_MAX_TREE_NODES || V < 1 || max_depth < 0) return 2;
  if (dtype != OR_DTYPE_F32 && dtype != OR_DTYPE_BF16) return 3;
  if (tstride < V || dstride < V) return 4;
  const int tree_ok = or_tree_is_valid(parents, depth, N, max_depth);
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* y = (double*)malloc(sizeof(double) * (size_t)V);
    double* P = (double*)malloc(sizeof(double) * (size_t)V);
    double* Q = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
      const int32_t* tok = node_tokens + (int64_t)b * N;
      int32_t* path = out_path + (int64_t)b * (max_depth + 1);
      for (int32_t k = 0; k <= max_depth; ++k) path[k] = -1;
      out_token[b] = -1;
      if (top_gap) top_gap[b] = INFINITY;
      if (flags) flags[b] = 0;
      if (rejections) rejections[b] = 0;
      if (margin) margin[b] = INFINITY;
      const double T = (double)temperature[b];
      if (!tree_ok) {
        out_path_len[b] = OR_SEQ_BAD_TREE;
        continue;
      }
      if (!(T > 0.0) || isinf(T)) {
        out_path_len[b] = OR_SEQ_BAD_TEMPERATURE;
        continue;
      }
      int bad = 0;
      for (int32_t c = 1; c < N; ++c) {
        if (tok[c] < 0 || tok[c] >= V) bad = 1;
        /* Without replacement, siblings carry distinct tokens. */
        if (without_replacement)
          for (int32_t s2 = 1; s2 < c; ++s2)
            if (parents[s2] == parents[c] && tok[s2] == tok[c]) bad = 1;
      }
      if (bad) {
        out_path_len[b] = OR_SEQ_BAD_TOKEN;
        continue;
      }
      or_tree_sample_one(target, tstride, draft, dstride, dtype, parents, tok, T, b, N, V,
                         max_depth, seed, offset, without_replacement != 0, y, P, Q, path, &out_path_len[b], &out_token[b],
                         top_gap ? &top_gap[b] : NULL, flags ? &flags[b] : NULL,
                         rejections ? &rejections[b] : NULL, margin ? &margin[b] : NULL);
    }
    free(y);
    free(P);
    free(Q);
  }
  return 0;
}

/* Depth of every node from the parent array ([SB] build_tree_attn: walk from
 * the node up to the root, counting the ancestors). Returns 0 on a malformed
 * array. */
int or_tree_depths(const int32_t* parents, int32_t N, int32_t* depth_out) {
  for (int32_t i = 0; i < N; ++i) {
    int32_t d = 0, j = parents[i], steps = 0;
    while (j != -1) {
      if (j < 0 || j >= N || ++steps > N) return 0;
      ++d;
      j = parents[j];
    }
    depth_out[i] = d;
  }
  return 1;
}
