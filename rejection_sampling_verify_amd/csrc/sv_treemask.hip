// sv_treemask.hip — tree attention mask and position ids from parent pointers
// ("7.6 Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead", "Tree
// Attention: Verifying Many Candidates at Once", build_tree_attn; "Medusa,
// EAGLE and self-speculation", "Verifying a tree instead of a line"): node i may
// attend to node j iff j is i or one of its ancestors, and node i's position
// id is its depth, so that one packed forward pass scores every path of the
// tree as if each were a contiguous sequence.
//
// One workgroup per sequence. The parent array is staged in LDS and checked
// (root first, every other parent an earlier node). Each lane walks one row's
// ancestors into a row bitset in LDS, 256 rows at a time, and the rows are then
// written out: packed words straight from LDS, or the bool mask as 4-byte words
// over the batch's whole byte range (rows of N bytes need not be aligned), with
// the few bytes before and after the aligned words written singly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

namespace sv {
namespace {

constexpr int kTmThreads = 256;
constexpr int kTmMaxN = 1024;
constexpr int kTmMaxW = kTmMaxN / 32;  // 32-bit words per row

struct TmArgs {
  const int32_t* parents;  // [B, N], rows par_stride apart (0: one tree for every sequence)
  int64_t par_stride;
  const int32_t* offsets;  // [B] or NULL
  int32_t N, W;
  uint8_t* mask;    // [B, N, N] bool bytes, or NULL
  uint32_t* bits;   // [B, N, W] packed, or NULL
  int32_t* pos;     // [B, N], or NULL
};

__global__ __launch_bounds__(kTmThreads) void tree_mask_kernel(TmArgs a) {
  __shared__ int32_t s_par[kTmMaxN];
  __shared__ uint32_t s_rows[kTmThreads * kTmMaxW];  // row (r0 + t) of the batch at t * W
  const int b = (int)blockIdx.x;
  const int tid = (int)threadIdx.x;
  const int N = a.N, W = a.W;
  const int32_t* par = a.parents + (int64_t)b * a.par_stride;
  int bad = 0;
  for (int i = tid; i < N; i += kTmThreads) {
    const int p = par[i];
    s_par[i] = p;
    bad |= i == 0 ? p != -1 : (p < 0 || p >= i);
  }
  bad = __syncthreads_or(bad);
  if (a.pos) {
    const int off = a.offsets ? a.offsets[b] : 0;
    for (int i = tid; i < N; i += kTmThreads) {
      int d = 0;
      if (!bad)
        for (int j = s_par[i]; j != -1; j = s_par[j]) ++d;  // ends: parents strictly decrease
      a.pos[(int64_t)b * N + i] = bad ? -1 : off + d;
    }
  }
  if (!a.mask && !a.bits) return;
  for (int r0 = 0; r0 < N; r0 += kTmThreads) {
    const int rows = min(kTmThreads, N - r0);
    uint32_t* row = s_rows + tid * W;
    for (int w = 0; w < W; ++w) row[w] = 0;
    const int i = r0 + tid;
    if (!bad && i < N)
      for (int j = i; j != -1; j = s_par[j]) row[j >> 5] |= 1u << (j & 31);
    __syncthreads();
    if (a.bits) {
      uint32_t* out = a.bits + ((int64_t)b * N + r0) * W;
      for (int k = tid; k < rows * W; k += kTmThreads) out[k] = s_rows[k];
    }
    if (a.mask) {
      // The batch's bytes [s, e) of the mask; byte s + f is row f / N, column f % N.
      uint8_t* base = a.mask + ((int64_t)b * N + r0) * N;
      const int nbytes = rows * N;  // <= 256 * 1024
      const int head = (int)((4 - ((uintptr_t)base & 3)) & 3);  // bytes before the first aligned word
      const int lead = min(head, nbytes);
      const int nwords = (nbytes - lead) >> 2;
      auto bit_at = [&](int f) -> uint32_t {
        const int r = f / N, j = f - r * N;
        return (s_rows[r * W + (j >> 5)] >> (j & 31)) & 1u;
      };
      if (tid < lead) base[tid] = (uint8_t)bit_at(tid);
      for (int k = tid; k < nwords; k += kTmThreads) {
        const int f = lead + 4 * k;
        int r = f / N, j = f - r * N;
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          word |= ((s_rows[r * W + (j >> 5)] >> (j & 31)) & 1u) << (8 * e);
          if (++j == N) {
            j = 0;
            ++r;
          }
        }
        *(uint32_t*)(base + f) = word;
      }
      const int tail0 = lead + 4 * nwords;
      if (tid < nbytes - tail0) base[tail0 + tid] = (uint8_t)bit_at(tail0 + tid);
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace sv

extern "C" {

sv_status_t sv_tree_mask(const int32_t* parents, int64_t parents_stride, int32_t B, int32_t N,
                         const int32_t* position_offset, uint8_t* out_mask, uint32_t* out_mask_bits,
                         int32_t* out_position_ids, void* stream) {
  if (!parents || (!out_mask && !out_mask_bits && !out_position_ids)) return SV_ERR_NULL_ARG;
  if (B < 0 || N < 1 || N > sv::kTmMaxN || parents_stride < 0 || (parents_stride > 0 && parents_stride < N))
    return SV_ERR_BAD_SHAPE;
  if (B == 0) return SV_OK;
  sv::TmArgs a;
  a.parents = parents;
  a.par_stride = parents_stride;
  a.offsets = position_offset;
  a.N = N;
  a.W = (N + 31) / 32;
  a.mask = out_mask;
  a.bits = out_mask_bits;
  a.pos = out_position_ids;
  hipLaunchKernelGGL(sv::tree_mask_kernel, dim3((unsigned)B), dim3(sv::kTmThreads), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
