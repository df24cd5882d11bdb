// Drives the host-side argument validation of every C-ABI entry point (the
// calls return before any HIP call), and the workspace sizing at its limits,
// for a build of the library's host code with AddressSanitizer and
// UndefinedBehaviorSanitizer (the CPU sanitizer test). Exits 0 when every
// call returned the expected status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/spec_verify.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { std::fprintf(stderr, "line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

int main() {
  alignas(256) static uint8_t buf[1 << 16];
  void* P = buf;
  const int32_t* I = (const int32_t*)buf;
  int32_t* O = (int32_t*)buf;
  const float* F = (const float*)buf;
  // Workspace sizing: out of range gives 0, the largest shapes do not overflow.
  EXPECT(sv_workspace_bytes(-1, 5, 100) == 0 && sv_workspace_bytes(4, 0, 100) == 0 &&
         sv_workspace_bytes(4, 1025, 100) == 0 && sv_workspace_bytes(4, 5, 0) == 0 &&
         sv_workspace_bytes(SV_MAX_BATCH + 1, 5, 100) == 0 && sv_workspace_bytes(4, 5, (1 << 30) + 1) == 0);
  EXPECT(sv_workspace_bytes(SV_MAX_BATCH, SV_MAX_TREE_NODES, 1 << 30) > ((size_t)1 << 50));
  EXPECT(sv_workspace_bytes(0, 1, 1) > 0);
  for (int s = -1; s <= 8; ++s) EXPECT(sv_status_string((sv_status_t)s) != nullptr);
  // Chains.
  const size_t ws = sizeof(buf);
  EXPECT(spec_verify_sample(nullptr, 100, P, 100, SV_DTYPE_BF16, I, F, 2, 3, 100, 0, 0, 0, O, O, nullptr, P, ws,
                            nullptr) == SV_ERR_NULL_ARG);
  EXPECT(spec_verify_sample(P, 100, P, 100, SV_DTYPE_BF16, I, F, 2, 17, 100, 0, 0, 0, O, O, nullptr, P, ws,
                            nullptr) == SV_ERR_BAD_SHAPE);
  EXPECT(spec_verify_sample(P, 100, P, 100, (sv_dtype_t)9, I, F, 2, 3, 100, 0, 0, 0, O, O, nullptr, P, ws,
                            nullptr) == SV_ERR_BAD_DTYPE);
  EXPECT(spec_verify_sample(P, 99, P, 100, SV_DTYPE_BF16, I, F, 2, 3, 100, 0, 0, 0, O, O, nullptr, P, ws,
                            nullptr) == SV_ERR_BAD_ARG);
  EXPECT(spec_verify_sample(P, 100, P, 100, SV_DTYPE_BF16, I, F, 2, 3, 100, 0, 1ull << 31, 0, O, O, nullptr, P, ws,
                            nullptr) == SV_ERR_BAD_ARG);
  EXPECT(spec_verify_sample(P, 100, P, 100, SV_DTYPE_BF16, I, F, 2, 3, 100, 0, 0, 0xFFFFFFFFu, O, O, nullptr, P,
                            ws, nullptr) == SV_ERR_BAD_ARG);
  EXPECT(spec_verify_sample(P, 100, P, 100, SV_DTYPE_BF16, I, F, 2, 3, 100, 0, 0, 0, O, O, nullptr, P, 8,
                            nullptr) == SV_ERR_WORKSPACE);
  EXPECT(spec_verify_sample(P, 100, P, 100, SV_DTYPE_BF16, I, F, 2, 3, 100, 0, 0, 0, O, O, nullptr, buf + 16, ws,
                            nullptr) == SV_ERR_BAD_ARG);
  EXPECT(spec_verify_sample(P, 100, P, 100, SV_DTYPE_BF16, I, F, 0, 3, 100, 0, 0, 0, O, O, nullptr, P, ws,
                            nullptr) == SV_OK);
  EXPECT(sv_debug_sample_tiled(P, 100, P, 100, SV_DTYPE_BF16, I, F, 2, 3, 100, 0, 0, 0, O, O, nullptr, P, ws,
                               nullptr, 3, 0) == SV_ERR_BAD_ARG);
  EXPECT(spec_verify_sample_noalloc(P, 152064, nullptr, 0, SV_DTYPE_BF16, I, F, 4096, 16, 152064, 0, 0, 0, O, O,
                                    nullptr, nullptr) == SV_ERR_SCRATCH_LIMIT);
  EXPECT(spec_verify_sample_noalloc(P, 100, nullptr, 0, SV_DTYPE_BF16, I, nullptr, 2, 3, 100, 0, 0, 0, O, O,
                                    nullptr, nullptr) == SV_ERR_NULL_ARG);
  EXPECT(spec_verify_greedy(P, 100, SV_DTYPE_F32, I, 2, 0, 100, O, O, P, ws, nullptr) == SV_ERR_BAD_SHAPE);
  EXPECT(spec_verify_greedy(P, 100, SV_DTYPE_F32, I, 0, 2, 100, O, O, P, ws, nullptr) == SV_OK);
  // Trees.
  EXPECT(spec_verify_tree(P, 100, SV_DTYPE_BF16, I, I, I, 2, 1025, 100, 3, O, O, O, P, ws, nullptr) ==
         SV_ERR_BAD_SHAPE);
  EXPECT(spec_verify_tree(P, 100, SV_DTYPE_BF16, I, I, I, 2, 5, 100, 5, O, O, O, P, ws, nullptr) == SV_ERR_BAD_SHAPE);
  EXPECT(spec_verify_tree(P, 100, SV_DTYPE_BF16, I, I, I, 0, 5, 100, 3, O, O, O, P, ws, nullptr) == SV_OK);
  EXPECT(spec_verify_tree_sample(P, 100, P, 100, SV_DTYPE_BF16, I, I, I, F, 2, 5, 100, 3, 0, 0, 0, 2, O, O, O, P,
                                 ws, nullptr) == SV_ERR_BAD_ARG);
  EXPECT(spec_verify_tree_sample(P, 100, P, 100, SV_DTYPE_BF16, I, I, I, F, 0, 5, 100, 3, 0, 0, 0, 1, O, O, O, P,
                                 ws, nullptr) == SV_OK);
  // The other rows' entry points.
  EXPECT(sv_kv_rollback(P, P, 3, 2, 2, 2, 8, 64, I, I, 4, I, O, nullptr) == SV_ERR_BAD_DTYPE);
  EXPECT(sv_kv_rollback(P, P, 2, 2, 2, 2, 8, 64, I, I, 0, I, O, nullptr) == SV_ERR_BAD_SHAPE);
  EXPECT(sv_kv_rollback(P, P, 2, 0, 2, 2, 8, 64, I, I, 4, I, O, nullptr) == SV_OK);
  EXPECT(sv_ngram_draft(I, 64, I, 2, 17, 4, 1, O, O, O, nullptr) == SV_ERR_BAD_SHAPE);
  EXPECT(sv_ngram_draft(I, 64, I, 2, 3, 4, 2, O, O, O, nullptr) == SV_ERR_BAD_ARG);
  EXPECT(sv_ngram_draft(I, 64, I, 0, 3, 4, 1, O, O, O, nullptr) == SV_OK);
  EXPECT(sv_tree_mask(I, 8, 2, 1025, nullptr, (uint8_t*)P, nullptr, nullptr, nullptr) == SV_ERR_BAD_SHAPE);
  EXPECT(sv_tree_mask(I, 8, 0, 8, nullptr, (uint8_t*)P, nullptr, nullptr, nullptr) == SV_OK);
  EXPECT(sv_debug_philox(nullptr, (const uint32_t*)buf, (uint32_t*)buf, 1, nullptr) == SV_ERR_NULL_ARG);
  if (fails) std::fprintf(stderr, "%d checks failed\n", fails);
  return fails ? 1 : 0;
}
