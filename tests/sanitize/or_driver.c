/* Drives every oracle entry point over small random inputs and edge cases,
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer (the CPU
 * sanitizer test). Exits 0 when every call returned as expected. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/sv_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double rnd(void) { /* xorshift64*, mapped to (0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return ((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0) + 1e-18;
}
static float gauss(void) { return (float)(sqrt(-2.0 * log(rnd())) * cos(6.283185307179586 * rnd())); }
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

static void chains(int bf16) {
  const int B = 9, G = 4, V = 37, S = 40;
  const size_t nt = (size_t)B * (G + 1) * S, nd = (size_t)B * G * S;
  void* tgt = malloc(nt * (bf16 ? 2 : 4));
  void* dft = malloc(nd * (bf16 ? 2 : 4));
  for (size_t k = 0; k < nt; ++k) {
    const float v = 2.0f * gauss();
    if (bf16) ((uint16_t*)tgt)[k] = to_bf16(v); else ((float*)tgt)[k] = v;
  }
  for (size_t k = 0; k < nd; ++k) {
    const float v = 2.0f * gauss();
    if (bf16) ((uint16_t*)dft)[k] = to_bf16(v); else ((float*)dft)[k] = v;
  }
  /* edge rows: -inf entries, +inf, NaN, a row without a finite entry */
  const float special[4] = {-INFINITY, INFINITY, NAN, -INFINITY};
  for (int j = 0; j < 4; ++j) {
    const size_t k = ((size_t)(5 + j) * (G + 1) + 1) * S + 3;
    if (bf16) ((uint16_t*)tgt)[k] = to_bf16(special[j]); else ((float*)tgt)[k] = special[j];
  }
  for (int v = 0; v < S; ++v) {
    const size_t k = ((size_t)8 * (G + 1) + 0) * S + v;
    if (bf16) ((uint16_t*)tgt)[k] = to_bf16(-INFINITY); else ((float*)tgt)[k] = -INFINITY;
  }
  int32_t ids[9 * 4];
  for (int k = 0; k < B * G; ++k) ids[k] = (int32_t)(rnd() * V);
  ids[1 * G + 2] = V;  /* out of range */
  ids[2 * G + 0] = -3;
  float temp[9] = {1.0f, 0.7f, 1.0f, -1.0f, NAN, 0.0f, 0.9f, 1.3f, 1.0f};
  int32_t tok[9 * 5], n[9], flags[9];
  double ap[9 * 4], un[9 * 4], lzt[9 * 4], lzd[9 * 4], beta[9], gap[9], top[9];
  or_diag_t d = {ap, un, lzt, lzd, beta, gap, top, flags};
  EXPECT(or_verify_sample(tgt, S, dft, S, bf16, ids, temp, B, G, V, 7, 3, NULL, tok, n, &d, 2) == 0);
  EXPECT(n[1] == OR_SEQ_BAD_TOKEN && n[2] == OR_SEQ_BAD_TOKEN);
  EXPECT(n[3] == OR_SEQ_BAD_TEMPERATURE && n[4] == OR_SEQ_BAD_TEMPERATURE);
  EXPECT(n[7] == OR_SEQ_BAD_LOGITS && n[8] == OR_SEQ_BAD_LOGITS);
  double u[9 * 4];
  for (int k = 0; k < B * G; ++k) u[k] = rnd();
  EXPECT(or_verify_sample(tgt, S, NULL, 0, bf16, ids, temp, B, G, V, 7, 3, u, tok, n, &d, 1) == 0);
  EXPECT(or_verify_sample(tgt, S, dft, S, bf16, ids, temp, B, G, V, 0, 0, NULL, tok, n, NULL, 3) == 0);
  EXPECT(or_verify_greedy(tgt, S, bf16, ids, B, G, V, tok, n, 2) == 0);
  EXPECT(or_verify_sample(NULL, S, dft, S, bf16, ids, temp, B, G, V, 0, 0, NULL, tok, n, NULL, 1) != 0);
  EXPECT(or_verify_sample(tgt, S, dft, S, bf16, ids, temp, B, 17, V, 0, 0, NULL, tok, n, NULL, 1) != 0);
  EXPECT(or_verify_greedy(tgt, 3, bf16, ids, B, G, V, tok, n, 1) != 0);
  free(tgt);
  free(dft);
}

static void trees(int bf16) {
  const int B = 5, N = 9, V = 31;
  const int32_t parents[9] = {-1, 0, 0, 1, 1, 2, 3, 3, 6};
  int32_t depth[9];
  EXPECT(or_tree_depths(parents, N, depth) == 1);
  const size_t nt = (size_t)B * N * V;
  void* tgt = malloc(nt * (bf16 ? 2 : 4));
  void* dft = malloc(nt * (bf16 ? 2 : 4));
  for (size_t k = 0; k < nt; ++k) {
    const float a = 1.5f * gauss(), b = 1.5f * gauss();
    if (bf16) { ((uint16_t*)tgt)[k] = to_bf16(a); ((uint16_t*)dft)[k] = to_bf16(b); }
    else { ((float*)tgt)[k] = a; ((float*)dft)[k] = b; }
  }
  int32_t tok[5 * 9];
  for (int k = 0; k < B * N; ++k) tok[k] = (int32_t)(rnd() * V);
  tok[1 * N + 4] = tok[1 * N + 3];  /* duplicate siblings */
  tok[2 * N + 5] = V;               /* out of range */
  float temp[5] = {1.0f, 0.8f, 1.0f, 0.0f, 1.1f};
  int32_t path[5 * 5], plen[5], out[5], fm[5], fl[5], rej[5];
  double gap[5], mg[5];
  EXPECT(or_verify_tree(tgt, V, bf16, parents, depth, tok, B, N, V, 4, path, plen, out, fm, 2) == 0);
  for (int wor = 0; wor <= 1; ++wor)
    EXPECT(or_verify_tree_sample(tgt, V, dft, V, bf16, parents, depth, tok, temp, B, N, V, 4, 11, 2, wor, path,
                                 plen, out, gap, fl, rej, mg, 2) == 0);
  EXPECT(plen[3] == OR_SEQ_BAD_TEMPERATURE && plen[2] == OR_SEQ_BAD_TOKEN && plen[1] == OR_SEQ_BAD_TOKEN);
  const int32_t bad_parents[4] = {-1, 0, 2, 1};
  const int32_t bad_depth[4] = {0, 1, 2, 2};
  EXPECT(or_tree_is_valid(bad_parents, bad_depth, 4, 3) == 0);
  int32_t d2[4];
  EXPECT(or_tree_depths(bad_parents, 4, d2) == 0);
  free(tgt);
  free(dft);
}

int main(void) {
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
  or_philox4x32_10(ctr, key, out);
  EXPECT(or_accept_uniform(0, 0, 3, 2) < 1.0);
  EXPECT(isfinite(or_gumbel(0xFFFFFFFFFFFFFFFFull, 0x7FFFFFFF, 2147483647, 15, 151935)));
  chains(0);
  chains(1);
  trees(0);
  trees(1);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  return fails ? 1 : 0;
}
