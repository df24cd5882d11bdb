/*
 * sv_oracle.h — CPU oracle of the speculative-decoding verify step.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline benchmark leg).
 * Independent of the GPU library: nothing here is shared with it.
 */
#ifndef SV_ORACLE_H
#define SV_ORACLE_H

#include <stdint.h>

#define OR_DTYPE_F32 0
#define OR_DTYPE_BF16 1
#define OR_MAX_GAMMA 16
#define OR_MAX_TREE_NODES 1024

/* Per-sequence codes in out_n / out_path_len. */
#define OR_SEQ_BAD_TOKEN (-1)
#define OR_SEQ_BAD_TEMPERATURE (-2)
#define OR_SEQ_BAD_TREE (-3)
#define OR_SEQ_BAD_LOGITS (-5) /* a sampled sequence's row has no probability distribution */

/* flags[b] bits */
#define OR_FLAG_KNIFE_EDGE 1 /* some tested position had |u - a| < OR_KNIFE_EDGE */
#define OR_FLAG_FALLBACK 2   /* the residual was empty; the correction came from p */

/* An accept decision closer than this to its threshold is excusable in a
 * comparison with an fp32 implementation whose accept probabilities are held
 * to the same absolute tolerance. */
#define OR_KNIFE_EDGE 1e-5

/* Optional per-sequence diagnostics (any field may be NULL). */
typedef struct {
  double* accept_prob; /* [B, gamma] a_i for every position                       */
  double* uniforms;    /* [B, gamma] u_i used by the accept test                   */
  double* logz_target; /* [B, gamma] ln sum exp(l/T) of target rows 0..gamma-1     */
  double* logz_draft;  /* [B, gamma] same for draft rows (NaN: one-hot or greedy)   */
  double* residual_mass; /* [B] beta at the first rejection (NaN otherwise)         */
  double* top_gap;     /* [B] (s1 - s2) / max(|s1|, |s2|, 1) of the Gumbel-max draw */
  double* top_score;   /* [B] s1 of the Gumbel-max draw                              */
  int32_t* flags;      /* [B] OR_FLAG_* bits                                          */
} or_diag_t;

void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
double or_accept_uniform(uint64_t seed, uint64_t offset, int32_t b, int32_t i);
double or_gumbel(uint64_t seed, uint64_t offset, int32_t b, int32_t pos, int32_t v);

/* Returns 0 on success, nonzero for invalid arguments. u_override [B, gamma]
 * replaces the Philox accept uniforms when not NULL. */
int or_verify_sample(const void* target, int64_t tstride, const void* draft, int64_t dstride,
                     int dtype, const int32_t* draft_ids, const float* temperature, int32_t B,
                     int32_t gamma, int32_t V, uint64_t seed, uint64_t offset,
                     const double* u_override, int32_t* out_tokens, int32_t* out_n, or_diag_t* d,
                     int nthreads);

int or_verify_greedy(const void* target, int64_t tstride, int dtype, const int32_t* draft_ids,
                     int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens, int32_t* out_n,
                     int nthreads);

int or_tree_is_valid(const int32_t* parents, const int32_t* depth, int32_t N, int32_t max_depth);

int or_verify_tree(const void* target, int64_t tstride, int dtype, const int32_t* parents,
                   const int32_t* depth, const int32_t* node_tokens, int32_t B, int32_t N,
                   int32_t V, int32_t max_depth, int32_t* out_path, int32_t* out_path_len,
                   int32_t* out_bonus, int32_t* out_first_match_node, int nthreads);

/* Sampled tree verification by multi-round rejection sampling. draft holds
 * [B, N, V] rows too: row v is q at node v, the distribution v's children
 * were drawn from (leaf rows are not read). Temperatures must be > 0. Per
 * sequence: out_path [max_depth + 1] (root first, -1 padded), out_path_len
 * (nodes on the path, or an OR_SEQ_* code), out_token (the bonus or
 * replacement token after the path); optional top_gap, flags and the number
 * of rejected siblings, and margin: the smallest |u - a| over the siblings
 * tested. */
int or_verify_tree_sample(const void* target, int64_t tstride, const void* draft, int64_t dstride,
                          int dtype, const int32_t* parents, const int32_t* depth,
                          const int32_t* node_tokens, const float* temperature, int32_t B,
                          int32_t N, int32_t V, int32_t max_depth, uint64_t seed, uint64_t offset,
                          int32_t without_replacement, int32_t* out_path, int32_t* out_path_len,
                          int32_t* out_token, double* top_gap, int32_t* flags, int32_t* rejections,
                          double* margin, int nthreads);

int or_tree_depths(const int32_t* parents, int32_t N, int32_t* depth_out);

#endif /* SV_ORACLE_H */
