// sv_ngram.hip — prompt-lookup / n-gram drafting on the device ("7.6
// Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead", Exercise 4;
// "Medusa, EAGLE and self-speculation", "Copying, verified against plain greedy"): the
// last `ngram` tokens of each sequence are looked up at earlier start positions,
// most recent first, and the tokens that followed the match are proposed; the
// proposals are one-hot drafts for the verify step.
//
// One workgroup per sequence scans candidate end positions from right to left
// in chunks (one 16-byte load per lane and group of four positions when the
// rows are aligned, every load of a chunk in flight before any compare). The
// chunk, with a halo of four groups below it, is staged in LDS so that a lane
// can read the groups before its own with a few 16-byte LDS reads; every
// position is then tested against the whole n-gram in registers, without
// branches (a filter on the last token alone would make most waves take the
// slow path, since some lane nearly always hits a frequent token). A block
// maximum gives the most recent match in the chunk, and the scan stops at the
// first chunk that has one, so a sequence reads only the stretch from its match
// to its end, rounded out to whole chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

namespace sv {
namespace {

typedef int32_t ng_i32x4 __attribute__((ext_vector_type(4)));
constexpr int kNgThreads = 512;
constexpr int kNgLoads = 8;                       // groups of four positions per lane per chunk
constexpr int kNgGroups = kNgThreads * kNgLoads;  // groups per chunk (16384 positions, 64 KB of LDS)
constexpr int kNgHalo = 4;                        // groups below the chunk (n - 1 <= 15 earlier tokens)
constexpr int kNgMaxN = 16;

struct NgArgs {
  const int32_t* tokens;  // [B, stride]
  int64_t stride;
  const int32_t* lengths;  // [B]
  int32_t ngram, gamma, pad;
  int32_t* draft;  // [B, gamma]
  int32_t* count;  // [B]
  int32_t* match;  // [B] or NULL
};

__device__ inline int ng_wave_max(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

template <bool VEC>
__device__ inline ng_i32x4 ng_load_group(const int32_t* seq, int g, int T) {
  ng_i32x4 v = ng_i32x4{0, 0, 0, 0};
  if (VEC && 4 * g + 4 <= T) {
    v = *(const ng_i32x4*)(seq + 4 * (int64_t)g);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * g + e < T) v[e] = seq[4 * g + e];
  }
  return v;
}

// NT is ngram itself for 1 .. 4, and 0 for ngram 5 .. 16 (tested up to 16 with
// the unused places masked off), so the n-gram test unrolls into straight-line
// XOR / OR arithmetic.
template <bool VEC, int NT>
__global__ __launch_bounds__(kNgThreads) void ngram_kernel(NgArgs a) {
  constexpr int NMAX = NT > 0 ? NT : kNgMaxN;
  constexpr int NP = NMAX > 2 ? (NMAX + 2) / 4 : 1;  // earlier groups a position's n-gram can reach
  // Group g of the chunk at (g - g_base + kNgHalo) * 4.
  __shared__ __align__(16) int32_t s_tok[(kNgGroups + kNgHalo) * 4];
  __shared__ int32_t s_tail[kNgMaxN];
  __shared__ int32_t s_red[kNgThreads / 64];
  const int b = (int)blockIdx.x;
  const int tid = (int)threadIdx.x;
  const int32_t* seq = a.tokens + (int64_t)b * a.stride;
  const int T = a.lengths[b];
  const int n = a.ngram;
  // An empty sequence has no last token to pad with.
  const bool valid = T >= 0 && (int64_t)T <= a.stride && (T >= 1 || !a.pad);
  int best = -1;  // end position (start + n - 1) of the most recent earlier n-gram
  if (valid && T >= n + 1) {
    // The tail's loads go out with the first chunk's; it reaches LDS with the
    // chunk's first staging.
    const int tail_tok = tid < n ? seq[T - n + tid] : 0;
    int tl[NMAX];  // tl[q]: the token q places before the end of the n-gram
    const int lo = n - 1, hi = T - 2;  // end positions of earlier start positions 0 .. T - n - 1
    for (int g_top = hi >> 2; g_top >= (lo >> 2); g_top -= kNgGroups) {
      const bool first = g_top == (hi >> 2);
      const int g_base = g_top - kNgGroups + 1;  // the chunk's lowest group (below 0 for the last chunk)
      ng_i32x4 v[kNgLoads];
#pragma unroll
      for (int m = 0; m < kNgLoads; ++m) {
        const int g = g_top - m * kNgThreads - tid;  // descending in m: the lane's latest group first
        v[m] = g >= 0 ? ng_load_group<VEC>(seq, g, T) : ng_i32x4{0, 0, 0, 0};
      }
      ng_i32x4 halo = ng_i32x4{0, 0, 0, 0};
      const int hg = g_base - 1 - tid;
      if (tid < kNgHalo && hg >= 0) halo = ng_load_group<VEC>(seq, hg, T);
#pragma unroll
      for (int m = 0; m < kNgLoads; ++m) {
        const int g = g_top - m * kNgThreads - tid;
        if (g >= 0) *(ng_i32x4*)&s_tok[(g - g_base + kNgHalo) * 4] = v[m];
      }
      if (tid < kNgHalo && hg >= 0) *(ng_i32x4*)&s_tok[(hg - g_base + kNgHalo) * 4] = halo;
      if (first && tid < n) s_tail[tid] = tail_tok;
      __syncthreads();
      if (first) {
#pragma unroll
        for (int q = 0; q < NMAX; ++q) tl[q] = __builtin_amdgcn_readfirstlane(q < n ? s_tail[n - 1 - q] : 0);
      }
      int mine = -1;
#pragma unroll
      for (int m = 0; m < kNgLoads; ++m) {
        const int g = g_top - m * kNgThreads - tid;
        // The NP groups before g (in bounds: g - j >= g_base - kNgHalo). Entries
        // of groups below 0 are never used: they would only serve positions
        // p < n - 1, which are not candidates.
        ng_i32x4 pw[NP];
#pragma unroll
        for (int j = 1; j <= NP; ++j) pw[j - 1] = *(const ng_i32x4*)&s_tok[(g - j - g_base + kNgHalo) * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = 4 * g + e;
          int diff = 0;  // nonzero iff some place of the n-gram differs
#pragma unroll
          for (int q = 0; q < NMAX; ++q) {
            int tok;
            if (e - q >= 0) {
              tok = v[m][e - q];
            } else {
              const int d = q - e, j = (d + 3) / 4;  // position 4g - d: entry 4j - d of group g - j
              tok = pw[j - 1][4 * j - d];
            }
            const int x = tok ^ tl[q];
            diff |= NT > 0 ? x : (q < n ? x : 0);
          }
          // Candidates are p in [lo, hi] (p < lo covers the lanes with g < 0).
          const bool cand = diff == 0 && (unsigned)(p - lo) <= (unsigned)(hi - lo);
          mine = max(mine, cand ? p : -1);
        }
      }
      mine = ng_wave_max(mine);
      if ((tid & 63) == 0) s_red[tid >> 6] = mine;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kNgThreads / 64; ++w) best = max(best, s_red[w]);
      if (best >= 0) break;  // the same on every lane
    }
  }
  int32_t* out = a.draft + (int64_t)b * a.gamma;
  if (!valid) {
    for (int k = tid; k < a.gamma; k += kNgThreads) out[k] = -1;
    if (tid == 0) {
      a.count[b] = -1;
      if (a.match) a.match[b] = -1;
    }
    return;
  }
  const int last = T >= 1 ? seq[T - 1] : -1;
  for (int k = tid; k < a.gamma; k += kNgThreads) {
    const int64_t pos = (int64_t)best + 1 + k;  // the continuation starts after the match's last token
    out[k] = best >= 0 && pos < T ? seq[pos] : (a.pad ? last : -1);
  }
  if (tid == 0) {
    a.count[b] = a.pad ? a.gamma : (best >= 0 ? min(a.gamma, T - best - 1) : 0);
    if (a.match) a.match[b] = best >= 0 ? best - n + 1 : -1;
  }
}

}  // namespace
}  // namespace sv

extern "C" {

sv_status_t sv_ngram_draft(const int32_t* tokens, int64_t stride, const int32_t* lengths, int32_t B, int32_t ngram,
                           int32_t gamma, int32_t pad_with_last, int32_t* out_draft, int32_t* out_count,
                           int32_t* out_match, void* stream) {
  if (!tokens || !lengths || !out_draft || !out_count) return SV_ERR_NULL_ARG;
  if (B < 0 || stride < 1 || ngram < 1 || ngram > sv::kNgMaxN || gamma < 1) return SV_ERR_BAD_SHAPE;
  if (stride > INT32_MAX) return SV_ERR_BAD_SHAPE;  // positions are 32-bit
  if (pad_with_last != 0 && pad_with_last != 1) return SV_ERR_BAD_ARG;
  if (B == 0) return SV_OK;
  sv::NgArgs a;
  a.tokens = tokens;
  a.stride = stride;
  a.lengths = lengths;
  a.ngram = ngram;
  a.gamma = gamma;
  a.pad = pad_with_last;
  a.draft = out_draft;
  a.count = out_count;
  a.match = out_match;
  const bool vec = (uintptr_t)tokens % 16 == 0 && stride % 4 == 0;
  const dim3 grid((unsigned)B), block(sv::kNgThreads);
  hipStream_t st = (hipStream_t)stream;
  auto kernel = vec ? (ngram == 1   ? sv::ngram_kernel<true, 1>
                       : ngram == 2 ? sv::ngram_kernel<true, 2>
                       : ngram == 3 ? sv::ngram_kernel<true, 3>
                       : ngram == 4 ? sv::ngram_kernel<true, 4>
                                    : sv::ngram_kernel<true, 0>)
                    : (ngram == 1   ? sv::ngram_kernel<false, 1>
                       : ngram == 2 ? sv::ngram_kernel<false, 2>
                       : ngram == 3 ? sv::ngram_kernel<false, 3>
                       : ngram == 4 ? sv::ngram_kernel<false, 4>
                                    : sv::ngram_kernel<false, 0>);
  hipLaunchKernelGGL(kernel, grid, block, 0, st, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
