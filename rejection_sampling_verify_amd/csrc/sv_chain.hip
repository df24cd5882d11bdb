// sv_chain.hip — batched chain verification on gfx950.
//
// The rule ("7.6 Speculative Decoding: Draft Models, Medusa, EAGLE &
// Lookahead", "The rule" and "Extending to a chain of γ draft tokens"):
// accept draft x_i with probability min(1, p_i(x_i)/q_i(x_i)), stop at the
// first rejection n and draw its replacement from (p_n - q_n)_+, or draw the
// bonus token from p_gamma when nothing was rejected. Temperature 0 reduces it
// to argmax matching.
//
// Work decomposition. Every logit row is cut into chunks of `chunk` elements.
//   pass-1 item (b, i, c): chunk c of target row i (or of draft row i): the
//     partial log-sum-exp state of each row, or for greedy sequences the
//     partial argmax, published in a 16-byte slot (a dense draft's rows are
//     items of their own, filling the slot's second word). Nothing waits on it.
//   decision item (b): waits for the gamma * nchunks slots of b, takes the
//     decision (accept tests, first rejection), writes everything it fixes and
//     publishes a small decision record.
//   pass-2 item (b, c): reads the decision record of b and draws a partial
//     Gumbel-max (or argmax) over chunk c of the row the decision names. The
//     last pass-2 item of b to finish merges the partials and writes the last
//     token.
// Two launches run them: every pass-1 item followed by the decision items
// (which wait, boundedly, for slots of items dispatched before them), then
// pass 2, which finds every decision taken; pass 1 then runs at eight waves
// per SIMD and keeps the most row chunks in flight. Merges run in fixed chunk
// order, so results do not depend on the launch layout or on which item
// finishes last.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

enum SeqKind {
  KIND_BAD_T = 0,
  KIND_GREEDY = 1,
  KIND_SAMPLED = 2,
  KIND_BAD_ID = 3,
  KIND_STALLED = 4,
  KIND_BAD_LOGITS = 5  // a row of a sampled sequence defines no distribution
};

// The decision of one sequence, as every pass-2 item of it computes it.
struct Decision {
  int kind;
  int n;          // accepted drafts, or the per-sequence error code
  uint32_t mode;  // P2Mode
  int row, x;
  float T, c2, invT;
  float zt2, zd2;  // log2-domain normalizers of target / draft row `row`
  float a_row;     // accept probability at `row` (one-hot draft: p(x) there)
  int tok;         // token at position n when the decision already fixes it
};

struct Smem {
  LseState lse[2][kWaves];
  ArgMax am[kWaves];
  float fsum[kWaves];
  int ior[kWaves];
  uint32_t flag_last;
  uint32_t again;  // sampled trees: the final draw is taken again over the whole row
  uint32_t stalled;
  uint32_t lkey;   // pass 2: order key of the best total the workgroup has reached
  uint32_t nwork;  // second launch: sequences on the pass-2 work list
  int32_t unit[5]; // second launch: this workgroup's sequence, chunk, chunk length, chunks per
                   // row, and the sequence's place on the work list
  union {
    uint64_t slot[kThreads][2];    // decision: one batch of polled pass-1 slots
  } u;
  LseState rt[kMaxGamma], rd[kMaxGamma];
  ArgMax rg[kMaxGamma];
  int32_t acc[kMaxGamma];
  Decision dec;
};

// Block-wide log-sum-exp merge: within a wave the maximum first, then every
// lane rescales its sum to it and the sums are added (one exponential per
// lane); the four wave states are merged through LDS.
__device__ __forceinline__ LseState block_lse(LseState st, float c, Smem& sm, int slot) {
  const float M = wave_max(st.M);
  const float sum = wave_sum((st.M == -INFINITY) ? 0.0f : st.s * fast_exp2((st.M - M) * c));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm.lse[slot][w].M = M;
    sm.lse[slot][w].s = sum;
  }
  __syncthreads();
  LseState r = sm.lse[slot][0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = lse_merge(r, sm.lse[slot][k], c);
  __syncthreads();
  return r;
}

// block_lse of two states at once (one exchange through LDS for both).
__device__ __forceinline__ void block_lse2(LseState& s0, LseState& s1, float c, Smem& sm) {
  const float M0 = wave_max(s0.M), M1 = wave_max(s1.M);
  const float t0 = wave_sum((s0.M == -INFINITY) ? 0.0f : s0.s * fast_exp2((s0.M - M0) * c));
  const float t1 = wave_sum((s1.M == -INFINITY) ? 0.0f : s1.s * fast_exp2((s1.M - M1) * c));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm.lse[0][w].M = M0;
    sm.lse[0][w].s = t0;
    sm.lse[1][w].M = M1;
    sm.lse[1][w].s = t1;
  }
  __syncthreads();
  LseState r0 = sm.lse[0][0], r1 = sm.lse[1][0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) {
    r0 = lse_merge(r0, sm.lse[0][k], c);
    r1 = lse_merge(r1, sm.lse[1][k], c);
  }
  __syncthreads();
  s0 = r0;
  s1 = r1;
}

__device__ __forceinline__ ArgMax block_argmax(ArgMax a, Smem& sm) {
  a = wave_argmax(a);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm.am[w] = a;
  __syncthreads();
  ArgMax r = sm.am[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = argmax_merge(r, sm.am[k]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float x, Smem& sm) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm.fsum[w] = x;
  __syncthreads();
  float r = sm.fsum[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r += sm.fsum[k];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float x, Smem& sm) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm.fsum[w] = x;
  __syncthreads();
  float r = sm.fsum[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = fmaxf(r, sm.fsum[k]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_min_int(int x, Smem& sm) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = min(x, shfl_xor_i(x, m));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm.ior[w] = x;
  __syncthreads();
  int r = sm.ior[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = min(r, sm.ior[k]);
  __syncthreads();
  return r;
}

// Sequence classification from its temperature alone.
__device__ __forceinline__ int temp_kind(const ChainArgs& a, int b, float* T_out) {
  if (a.temperature == nullptr) {
    *T_out = 0.0f;
    return KIND_GREEDY;
  }
  const float T = a.temperature[b];
  *T_out = T;
  if (!(T >= 0.0f) || T == INFINITY) return KIND_BAD_T;
  return T == 0.0f ? KIND_GREEDY : KIND_SAMPLED;
}

__device__ __forceinline__ const uint8_t* target_row(const ChainArgs& a, int b, int i) {
  return a.target + ((int64_t)b * (a.gamma + 1) + i) * a.t_stride;
}
__device__ __forceinline__ const uint8_t* draft_row(const ChainArgs& a, int b, int i) {
  return a.draft + ((int64_t)b * a.d_rows + i) * a.d_stride;
}

__device__ __forceinline__ uint64_t pack(float hi, uint32_t lo) {
  return ((uint64_t)__float_as_uint(hi) << 32) | lo;
}
__device__ __forceinline__ float hi_f(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }
__device__ __forceinline__ uint32_t lo_u(uint64_t w) { return (uint32_t)w; }

// ---------------------------------------------------------------------------
// Chunk loaders. A chunk [lo, hi) is read as 16-byte vectors: thread t holds
// vectors t, t + 256, ... (at most kv of them); elements past the last whole
// vector (a ragged tail) are read one by one by the thread owning the next
// vector index. Without 16-byte alignment every element is read singly.
// ---------------------------------------------------------------------------
template <bool BF16, bool VEC, int KV = kMaxVecsPerThread>
struct Chunk {
  using E = Elem<BF16>;
  static constexpr int EV = E::kPerVec;
  u32x4 q[KV];
  int nfull;  // whole vectors in the chunk
  int lo, hi;

  __device__ __forceinline__ void load(const uint8_t* row, int lo_, int hi_, int kv) {
    lo = lo_;
    hi = hi_;
    nfull = VEC ? (hi - lo) / EV : 0;
    if (VEC && nfull > 0) {
      // Every vector slot is loaded (a lane past the chunk's whole vectors
      // loads the last one again), so the loads issue unconditionally and the
      // first vectors can be used while the later ones are in flight.
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        const int vi = min(k * kThreads + (int)threadIdx.x, nfull - 1);
        q[k] = load_vec_stream(row + (int64_t)(lo + vi * EV) * E::kBytes);
      }
    }
  }

  // bf16: the vectors past the end of a short chunk become -inf elements
  // (bit pattern 0xFF80), which neither the packed maximum (it reads them
  // as f16 NaNs and skips them), nor an exponential sum, nor an argmax
  // search for a finite maximum can pick up; then the packed whole-chunk
  // paths serve a short chunk too, as long as it holds whole vectors only.
  __device__ __forceinline__ void pad_neg_inf() {
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const int vi = k * kThreads + (int)threadIdx.x;
      if (vi >= nfull) q[k] = u32x4{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
    }
  }

  // Calls f(value, index) for each element this thread owns, in increasing
  // index order.
  template <typename F>
  __device__ __forceinline__ void for_each(const uint8_t* row, int kv, F&& f) const {
    if (VEC) {
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        const int vi = k * kThreads + (int)threadIdx.x;
        if (k < kv && vi < nfull) {
          float v[EV];
          E::unpack(q[k], v);
#pragma unroll
          for (int e = 0; e < EV; ++e) f(v[e], lo + vi * EV + e);
        }
      }
      const int tail_lo = lo + nfull * EV;
      if (tail_lo < hi && (nfull % kThreads) == (int)threadIdx.x) {
        for (int idx = tail_lo; idx < hi; ++idx) f(E::load(row, idx), idx);
      }
    } else {
      for (int idx = lo + (int)threadIdx.x; idx < hi; idx += kThreads) f(E::load(row, idx), idx);
    }
  }
};

template <bool BF16, bool VEC, int KV>
__device__ __forceinline__ LseState chunk_lse(const Chunk<BF16, VEC, KV>& ch, const uint8_t* row, int kv,
                                              float c) {
  float M = -INFINITY;
  ch.for_each(row, kv, [&](float v, int) { M = fmaxf(M, v); });
  float s = 0.0f;
  if (M != -INFINITY) {
    const float Mc = M * c;
    ch.for_each(row, kv, [&](float v, int) { s += fast_exp2(__builtin_fmaf(v, c, -Mc)); });
  }
  LseState st;
  st.M = M;
  st.s = s;
  return st;
}

template <bool BF16, bool VEC, int KV>
__device__ __forceinline__ ArgMax chunk_argmax(const Chunk<BF16, VEC, KV>& ch, const uint8_t* row, int kv) {
  ArgMax best;
  best.v = -INFINITY;
  best.i = -1;
  ch.for_each(row, kv, [&](float v, int idx) {
    if (best.i < 0 || v > best.v) {
      best.v = v;
      best.i = idx;
    }
  });
  return best;
}

// ---------------------------------------------------------------------------
// Whole-chunk fast paths for bf16 rows: every thread holds kMaxVecsPerThread
// full vectors, so there is no per-element predication, and the maximum is
// taken on the packed words before anything is unpacked.
// ---------------------------------------------------------------------------

// Largest element held by this thread, exactly, as a bf16 value in fp32. The
// two bf16 halves of every word are compared as f16 numbers (one packed max
// per two elements): both formats are sign-magnitude, so the f16 order of bf16
// bit patterns is the bf16 order for every logit of magnitude below 2^120;
// -inf halves read as f16 NaNs and are ignored by the max. (Logits are finite
// with magnitude below 2^120, or -inf.) The accumulators start at the most
// negative finite f16 pattern, below every such logit.
__device__ __forceinline__ uint32_t pk_max_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <int KV>
__device__ __forceinline__ float packed_max_bf16(const u32x4 (&q)[KV]) {
  uint32_t m0 = 0xFBFFFBFFu, m1 = 0xFBFFFBFFu;
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    m0 = pk_max_f16(m0, q[k][0]);
    m1 = pk_max_f16(m1, q[k][1]);
    m0 = pk_max_f16(m0, q[k][2]);
    m1 = pk_max_f16(m1, q[k][3]);
  }
  const uint32_t m = pk_max_f16(m0, m1);
  const float hi = __uint_as_float(m & 0xFFFF0000u), lo = __uint_as_float(m << 16);
  // Every element -inf: report -inf.
  const float r = fmaxf(hi, lo);
  return (m == 0xFBFFFBFFu) ? -INFINITY : r;
}

// Keeps the compiler from holding the unpacked elements of a max pass in
// registers until a later pass (unpacking again is cheaper than 32 registers).
template <int KV>
__device__ __forceinline__ void opaque(u32x4 (&q)[KV]) {
#pragma unroll
  for (int k = 0; k < KV; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = q[k][j];
      asm volatile("" : "+v"(w));
      q[k][j] = w;
    }
}

template <int KV>
__device__ __forceinline__ LseState lse_packed_bf16(u32x4 (&q)[KV], float c, int kvn = KV) {
  LseState st;
  st.M = packed_max_bf16(q);
  st.s = 0.0f;
  if (st.M != -INFINITY) {
    const float Mc = st.M * c;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      if (k >= kvn) break;  // padding vectors (all -inf) add nothing
      s0 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][0] << 16), c, -Mc));
      s1 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][0] & 0xFFFF0000u), c, -Mc));
      s2 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][1] << 16), c, -Mc));
      s3 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][1] & 0xFFFF0000u), c, -Mc));
      s0 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][2] << 16), c, -Mc));
      s1 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][2] & 0xFFFF0000u), c, -Mc));
      s2 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][3] << 16), c, -Mc));
      s3 += fast_exp2(__builtin_fmaf(__uint_as_float(q[k][3] & 0xFFFF0000u), c, -Mc));
    }
    st.s = (s0 + s1) + (s2 + s3);
  }
  return st;
}

// lse_packed_bf16 that also keeps every element's exp2((l - M) c2) in e
// (element order; 0 past the kvn vectors that hold data), M being this
// thread's own maximum; the sum is formed in the same order, so the
// statistics are bit for bit those of lse_packed_bf16.
template <int KV>
__device__ __forceinline__ LseState lse_packed_bf16_keep(u32x4 (&q)[KV], float c, int kvn, float (&e)[KV * 8]) {
  LseState st;
  st.M = packed_max_bf16(q);
  st.s = 0.0f;
#pragma unroll
  for (int i = 0; i < KV * 8; ++i) e[i] = 0.0f;
  if (st.M != -INFINITY) {
    const float Mc = st.M * c;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      if (k >= kvn) break;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[k * 8 + 2 * j] = fast_exp2(__builtin_fmaf(__uint_as_float(q[k][j] << 16), c, -Mc));
        e[k * 8 + 2 * j + 1] = fast_exp2(__builtin_fmaf(__uint_as_float(q[k][j] & 0xFFFF0000u), c, -Mc));
      }
      s0 += e[k * 8 + 0];
      s1 += e[k * 8 + 1];
      s2 += e[k * 8 + 2];
      s3 += e[k * 8 + 3];
      s0 += e[k * 8 + 4];
      s1 += e[k * 8 + 5];
      s2 += e[k * 8 + 6];
      s3 += e[k * 8 + 7];
    }
    st.s = (s0 + s1) + (s2 + s3);
  }
  return st;
}

// Argmax of the chunk [lo, lo + chunk) (lowest index among equal values): the
// block maximum first, then the lowest index holding it, searched only by the
// threads that hold it.
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_i16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Whether this thread holds a positive element the packed-f16 maximum cannot
// see: +inf, a NaN with the sign bit clear, or a value of 2^121 or more (bit
// patterns from 0x7C00 up). Positive bf16 values order like their patterns
// read as signed 16-bit integers, so one packed integer maximum finds them.
// An upper bound on the largest of a vector's eight bf16 logits: the largest
// pattern read as a signed 16-bit integer, clamped at +0. Non-negative values
// (+inf and values beyond the f16 range included) order as their patterns and
// every negative pattern reads as a negative integer, so the bound is exact
// when some element is >= 0, and 0 when all are negative.
__device__ __forceinline__ float max_bound_bf16(const u32x4& q) {
  const uint32_t m = pk_max_i16(pk_max_i16(q[0], q[1]), pk_max_i16(q[2], q[3]));
  // max(low half, high half, 0) as 16-bit integers, in the low half of r.
  uint32_t r;
  asm("v_max3_i16 %0, %1, %2, 0" : "=v"(r) : "v"(m), "v"(m >> 16));
  return __uint_as_float(r << 16);
}

template <int KV>
__device__ __forceinline__ bool has_huge_positive_bf16(const u32x4 (&q)[KV]) {
  uint32_t m0 = 0x80008000u, m1 = 0x80008000u;
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    m0 = pk_max_i16(m0, q[k][0]);
    m1 = pk_max_i16(m1, q[k][1]);
    m0 = pk_max_i16(m0, q[k][2]);
    m1 = pk_max_i16(m1, q[k][3]);
  }
  const uint32_t m = pk_max_i16(m0, m1);
  return (int16_t)(m & 0xFFFFu) >= 0x7C00 || (int16_t)(m >> 16) >= 0x7C00;
}

// Returns index 0x7FFFFFFF when the packed search cannot decide the chunk:
// a positive element it cannot see (see has_huge_positive_bf16), or a chunk
// whose maximum reads as -inf (every element -inf, or some at or below
// -2^121). The caller then scans the chunk element by element.
template <int KV>
__device__ __forceinline__ ArgMax argmax_packed_bf16(u32x4 (&q)[KV], int lo, Smem& sm) {
  float m = packed_max_bf16(q);
  if (has_huge_positive_bf16(q)) m = INFINITY;
  opaque(q);
  const float bm = block_max(m, sm);
  if (bm == INFINITY || bm == -INFINITY) {
    ArgMax r;
    r.v = bm;
    r.i = 0x7FFFFFFF;
    return r;
  }
  int idx = 0x7FFFFFFF;
  if (m == bm) {
#pragma unroll
    for (int k = KV - 1; k >= 0; --k) {
      const int base = lo + (k * kThreads + (int)threadIdx.x) * 8;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (__uint_as_float(q[k][j] & 0xFFFF0000u) == bm) idx = base + 2 * j + 1;
        if (__uint_as_float(q[k][j] << 16) == bm) idx = base + 2 * j;
      }
    }
  }
  ArgMax r;
  r.v = bm;
  r.i = block_min_int(idx, sm);
  return r;
}

// ---------------------------------------------------------------------------
// Gumbel-max pieces shared by both passes.
// ---------------------------------------------------------------------------
struct Best {
  float s;
  int32_t i;
};

// Larger total wins; equal totals go to the lower index (elements may be
// visited out of index order).
__device__ __forceinline__ void best_push(Best& bst, float s, int idx) {
  if (bst.i < 0 || s > bst.s || (s == bst.s && idx < bst.i)) {
    bst.s = s;
    bst.i = idx;
  }
}

// Exact pruning of the Gumbel-max draw. With E = -ln U, the noise is
// G = -ln E and E >= 1 - U. An element of score s can beat a total L already
// reached by some element of the row only if E < exp(s - L), hence only if
// 1 - U < exp(s - L). With r = 2^24 - 1 - (w >> 8), 1 - U = (2r + 1) 2^-25,
// which is at least 2^(floor(log2(2r + 1)) - 25). An element is therefore
// skipped, without evaluating G, when floor(log2(2r + 1)) - 25 exceeds
// log2(exp(s - L)) by more than a margin covering fp32 rounding; the draw is
// unchanged. (The test loses at most a factor of two against the exact bound.)
constexpr float kPruneMarginLog2 = 0x1p-12f;

__device__ __forceinline__ bool may_win_log2(uint32_t w, float x2) {
  const uint32_t odd = ((~w) >> 7) | 1u;        // 2r + 1
  const int e = 31 - __builtin_clz(odd);        // floor(log2(2r + 1))
  return !((float)(e - 25) > x2 + kPruneMarginLog2);
}

// Same test from a weight eps = exp(s - L) already computed in linear form.
__device__ __forceinline__ bool may_win_lin(uint32_t w, float eps) {
  const uint32_t odd = ((~w) >> 7) | 1u;
  const float t = (float)odd * 0x1p-25f;        // 1 - U (exact below 2^24)
  return !(t > eps * (1.0f + 0x1p-12f));
}

// Cheaper form of the same test for the bulk of a row, one bit looser. With
// n = ~w, 1 - U >= n 2^-32 / 2 (the bits of w below U's 24 only lower n), so
// an element can be skipped when log2(n) > log2(exp(s - L)) + 33 + 2^-12.
// The fp32 bit pattern of a positive x, read as an integer and divided by
// 2^23, is at most log2(x) + 127 (the exponent, plus a mantissa m that bounds
// log2(1 + m) from below), so the test compares that pattern of n, converted
// to fp32, with t = (log2(exp(s - L)) + 160 + 2^-12) 2^23 given by the caller;
// the conversions err by at most 2^7 against the margin's 2^11.
__device__ __forceinline__ bool may_win_bits(uint32_t w, float t) {
  return !((float)(int)__float_as_uint((float)(~w)) > t);
}

// may_win_bits over a wave: the mask of active lanes whose element may win,
// straight from the compare (a ballot of the verdict costs two more vector
// operations per element), as a value the compiler knows to be the same on
// every lane (branches on it stay on the scalar unit). Same test, also true
// for an unordered compare (predicate 13: unordered or less or equal).
__device__ __forceinline__ uint64_t lanes_may_win(uint32_t w, float t) {
  const float n = (float)(int)__float_as_uint((float)(~w));
  return __builtin_amdgcn_fcmpf(n, t, 13);
}

// Upper bound, in log2 units, on log2 (p - q) for log2 p = lp2 > lq2 = log2 q:
// p - q = p (1 - 2^-d) with d = lp2 - lq2, and 1 - e^-x <= min(1, x), so
// log2 (p - q) <= lp2 + min(0, log2 d + log2 ln 2). log2 d is bounded from
// above by its fp32 bit pattern read as above plus 0.0860714 (the largest gap
// between log2(1 + m) and m); 127 - 0.0860714 - log2 ln 2 = 127.442695, taken
// a little smaller. d is raised to 2^-100 first, which only loosens the bound
// and keeps it off subnormals.
__device__ __forceinline__ float residual_log2_bound(float lp2, float lq2) {
  const float d = __builtin_fmaxf(lp2 - lq2, 0x1p-100f);
  const float lg = (float)(int)__float_as_uint(d) * 0x1p-23f - 127.44268798828125f;
  return lp2 + __builtin_fminf(lg, 0.0f);
}

// Totals shared between the waves of a workgroup (LDS) and the workgroups of a
// sequence (its record) as unsigned order keys: larger key, larger total; 0
// stands for none yet. Any total that some element of the row reaches is a
// valid pruning threshold for every other part of the row, so these are read
// without ordering and may be stale.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_total(uint32_t k) {
  return k == 0u ? -INFINITY : __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---------------------------------------------------------------------------
// The decision of sequence b, taken by its decision item (all threads).
// ---------------------------------------------------------------------------

// Writes everything the decision fixes. The token at position n is left to
// the last pass-2 item when a draw is still pending.
__device__ __forceinline__ void write_decision(const ChainArgs& a, int b, Smem& sm) {
  const int G = a.gamma, tid = threadIdx.x;
  const Decision& d = sm.dec;
  const int32_t* ids = a.ids + (int64_t)b * G;
  int32_t* tok = a.out_tokens + (int64_t)b * (G + 1);
  if (tid <= G) {
    const bool pending = d.n >= 0 && tid == d.n && d.mode != P2_NONE;
    if (!pending) {
      int v = -1;
      if (d.n >= 0) {
        if (tid < d.n) v = ids[tid];
        else if (tid == d.n) v = d.tok;
      }
      tok[tid] = v;
    }
  }
  if (tid == 0) a.out_n[b] = d.n;
  if (tid < G) {
    const int64_t k = (int64_t)b * G + tid;
    float ap = NAN, lzt = NAN, lzd = NAN;
    if (d.kind == KIND_GREEDY) {
      ap = (ids[tid] == sm.rg[tid].i) ? 1.0f : 0.0f;
    } else if (d.kind == KIND_SAMPLED) {
      ap = sm.rt[tid].s;
      lzt = sm.rt[tid].M * kLn2;
      lzd = sm.rd[tid].M * kLn2;
    }
    if (a.d_accept) a.d_accept[k] = ap;
    if (a.d_logzt) a.d_logzt[k] = lzt;
    if (a.d_logzd) a.d_logzd[k] = lzd;
  }
  // A pending residual draw writes its mass itself.
  if (tid == 0 && a.d_beta && d.mode != P2_RESIDUAL && d.mode != P2_RESIDUAL_ONEHOT) a.d_beta[b] = NAN;
}

template <bool BF16>
__device__ __forceinline__ void decide(const ChainArgs& a, int b, Smem& sm) {
  const int G = a.gamma, C = a.nchunks, tid = threadIdx.x;
  const int32_t* ids = a.ids + (int64_t)b * G;
  float T;
  int kind = temp_kind(a, b, &T);
  const float c2 = (kind == KIND_SAMPLED) ? kLog2e / T : 0.0f;
  // The inputs besides the slots are requested first.
  bool bad_id = false;
  for (int i = 0; i < G; ++i) bad_id |= (ids[i] < 0 || ids[i] >= a.V);
  float glt = 0.0f, gld = 0.0f;
  if (tid < G && kind == KIND_SAMPLED && !bad_id) {
    const int x = ids[tid];
    glt = Elem<BF16>::load(target_row(a, b, tid), x);
    if (a.draft != nullptr) gld = Elem<BF16>::load(draft_row(a, b, tid), x);
  }
  if (tid < G) {
    sm.rt[tid].M = -INFINITY;
    sm.rt[tid].s = 0.0f;
    sm.rd[tid] = sm.rt[tid];
    sm.rg[tid].v = -INFINITY;
    sm.rg[tid].i = -1;
  }
  // A workspace left dirty by a call whose bounded wait gave up (its control
  // word still set) decides nothing: the sequence reports SV_SEQ_INTERNAL.
  if (tid == 0) sm.stalled = (xload(&a.done[1]) != 0u) ? 1u : 0u;
  __syncthreads();
  if (kind != KIND_BAD_T) {
    // Wait for every slot (also when a drafted id turns out to be invalid, so
    // that no slot can land after they have been cleared), 256 at a time;
    // return them to zero and merge each row's chunks in order.
    P1Slot* slots = a.p1 + (int64_t)b * G * C;
    const int total = G * C;
    for (int base = 0; base < total; base += kThreads) {
      const int k = base + tid;
      if (k < total) {
        uint64_t w0 = xget64(&slots[k].w0), w1 = xget64(&slots[k].w1);
        uint32_t spins = 0;
        while (w0 == 0u || w1 == 0u) {
          // A bounded wait: give up after spin_limit rounds, or soon after
          // any other wait of this call gave up.
          if (++spins > a.spin_limit || ((spins & 255u) == 0u && xget(&a.done[1]) != 0u)) {
            atomicOr(&a.done[1], 1u);
            sm.stalled = 1u;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
          w0 = xget64(&slots[k].w0);
          w1 = xget64(&slots[k].w1);
        }
        sm.u.slot[tid][0] = w0;
        sm.u.slot[tid][1] = w1;
      }
      __syncthreads();
      if (k < total) {
        xput64(&slots[k].w0, 0u);
        xput64(&slots[k].w1, 0u);
      }
      if (tid < G) {
        const int r0 = max(tid * C, base), r1 = min(tid * C + C, base + kThreads);
        for (int r = r0; r < r1; ++r) {
          const uint64_t w0 = sm.u.slot[r - base][0], w1 = sm.u.slot[r - base][1];
          if (kind == KIND_GREEDY) {
            ArgMax o;
            o.v = hi_f(w0);
            o.i = (int)lo_u(w0) - 1;
            sm.rg[tid] = argmax_merge(sm.rg[tid], o);
          } else {
            LseState o;
            o.M = hi_f(w0);
            o.s = __uint_as_float(lo_u(w0));
            sm.rt[tid] = lse_merge(sm.rt[tid], o, c2);
            if (a.draft != nullptr) {
              o.M = hi_f(w1);
              o.s = __uint_as_float(lo_u(w1));
              sm.rd[tid] = lse_merge(sm.rd[tid], o, c2);
            }
          }
        }
      }
      __syncthreads();
    }
  }
  if (kind != KIND_BAD_T && bad_id) kind = KIND_BAD_ID;
  if (sm.stalled) kind = KIND_STALLED;

  // Accept tests, one thread per position.
  if (tid == 0) sm.flag_last = 0u;  // set below if some row has no distribution
  __syncthreads();
  if (tid < G && kind == KIND_SAMPLED) {
    const float z2t = sm.rt[tid].M * c2 + fast_log2(sm.rt[tid].s);
    const float lp2 = __builtin_fmaf(glt, c2, -z2t);
    float z2d = NAN, lq2 = 0.0f;
    bool finite = __builtin_isfinite(z2t);
    if (a.draft != nullptr) {
      z2d = sm.rd[tid].M * c2 + fast_log2(sm.rd[tid].s);
      lq2 = __builtin_fmaf(gld, c2, -z2d);
      finite = finite && __builtin_isfinite(z2d);
    }
    // A row with no entry above -inf, or with +inf or NaN, has no softmax.
    if (!finite) atomicOr(&sm.flag_last, 1u);
    const float acc_p = fast_exp2(fminf(0.0f, lp2 - lq2));
    const Words4 w = philox10(0u, (uint32_t)tid, a.seq_base + (uint32_t)b, a.ctr_accept, a.key0, a.key1);
    sm.acc[tid] = (uniform_accept(w.w[0]) < acc_p) ? 1 : 0;
    sm.rt[tid].M = z2t;  // from here on: the row normalizers and a_i
    sm.rd[tid].M = z2d;
    sm.rt[tid].s = acc_p;
  }
  __syncthreads();
  if (kind == KIND_SAMPLED && sm.flag_last) kind = KIND_BAD_LOGITS;
  if (tid == 0) {
    Decision d;
    d.kind = kind;
    d.T = T;
    d.c2 = c2;
    d.invT = (kind == KIND_SAMPLED) ? 1.0f / T : 0.0f;
    d.mode = P2_NONE;
    d.row = 0;
    d.x = -1;
    d.zt2 = d.zd2 = 0.0f;
    d.a_row = 0.0f;
    d.tok = -1;
    if (kind == KIND_BAD_T) {
      d.n = -2;
    } else if (kind == KIND_BAD_ID) {
      d.n = -1;
    } else if (kind == KIND_STALLED) {
      d.n = -4;
    } else if (kind == KIND_BAD_LOGITS) {
      d.n = -5;
    } else if (kind == KIND_GREEDY) {
      d.n = G;
      for (int i = 0; i < G; ++i)
        if (ids[i] != sm.rg[i].i) {
          d.n = i;
          break;
        }
      if (d.n == G) {
        d.mode = P2_GREEDY_BONUS;
        d.row = G;
      } else {
        d.tok = sm.rg[d.n].i;  // the correction is the argmax itself
      }
    } else {
      d.n = G;
      for (int i = 0; i < G; ++i)
        if (!sm.acc[i]) {
          d.n = i;
          break;
        }
      if (d.n < G) {
        d.mode = (a.draft != nullptr) ? P2_RESIDUAL : P2_RESIDUAL_ONEHOT;
        d.row = d.n;
        d.x = ids[d.n];
        d.zt2 = sm.rt[d.n].M;
        d.zd2 = sm.rd[d.n].M;
        d.a_row = sm.rt[d.n].s;
      } else {
        d.mode = P2_BONUS;
        d.row = G;
      }
    }
    sm.dec = d;
  }
  __syncthreads();
  write_decision(a, b, sm);
  // A sequence with a pending draw is appended to the work list with its
  // decision record (the pass-2 launch reads them after this one ends).
  if (tid == 0) {
    const Decision& d = sm.dec;
    if (d.mode != P2_NONE) {
      const uint32_t idx = atomicAdd(&a.done[kDoneNWork], 1u);
      if (idx < (uint32_t)a.B) {
        WorkRec* w = a.work + idx;
        xput64(&w->dec[1], pack(d.zt2, __float_as_uint(d.zd2)));
        xput64(&w->dec[2], pack(d.c2, __float_as_uint(d.invT)));
        xput64(&w->dec[3], pack(d.a_row, (uint32_t)d.x));
        xput(&w->b, (uint32_t)b);
        xput64(&w->dec[0], kRecPublished | ((uint64_t)(uint32_t)d.row << 32) | ((uint32_t)(d.n + 64) << 8) | d.mode);
      } else {
        atomicOr(&a.done[1], 1u);  // a list left over from an aborted call
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 1: one chunk of one row pair; publishes its slot and moves on.
// ---------------------------------------------------------------------------
// Items of pass 1 per sequence: one per (row, chunk) of the target, and with
// a dense draft one more per (row, chunk) of the draft.
__device__ __forceinline__ int p1_items_per_seq(const ChainArgs& a) {
  return a.gamma * a.nchunks * (a.draft != nullptr ? 2 : 1);
}

template <bool BF16, bool VEC>
__device__ __forceinline__ void pass1_item(const ChainArgs& a, int b, int r, Smem& sm) {
  const int GC = a.gamma * a.nchunks;
  const bool draft_item = r >= GC;  // item of a dense draft row
  if (draft_item) r -= GC;
  const int i = r / a.nchunks, c = r % a.nchunks;
  float T;
  const int kind = temp_kind(a, b, &T);
  // Nothing to compute for a bad temperature; greedy sequences read no draft.
  if (kind == KIND_BAD_T || (draft_item && kind != KIND_SAMPLED)) return;
  const int lo = c * a.chunk;
  const int hi = min(a.V, lo + a.chunk);
  const uint8_t* row = draft_item ? draft_row(a, b, i) : target_row(a, b, i);
  // 16-byte-aligned bf16 chunk at the full tile width holding whole vectors
  // only (a short last chunk is padded with -inf): fast path.
  const bool fast = BF16 && VEC && a.kv == kMaxVecsPerThread && ((hi - lo) & 7) == 0;
  Chunk<BF16, VEC> ch;
  ch.load(row, lo, hi, a.kv);
  if (fast && hi - lo != a.chunk) ch.pad_neg_inf();
  // w0 belongs to the target item, w1 to the draft item of a dense draft and
  // to the target item otherwise.
  uint64_t w0 = 0u, w1 = 1u;
  if (kind == KIND_GREEDY) {
    ArgMax m;
    if (fast) m = argmax_packed_bf16(ch.q, lo, sm);
    // The plain scan decides where the packed search cannot: elements outside
    // the f16 reading's range (see argmax_packed_bf16), or a maximum flushed
    // as an f16 subnormal.
    if (!fast || m.i == 0x7FFFFFFF) m = block_argmax(chunk_argmax(ch, row, a.kv), sm);
    w0 = pack(m.v, (uint32_t)(m.i + 1));
  } else {
    const float c2 = kLog2e / T;
    LseState st = block_lse(fast ? lse_packed_bf16(ch.q, c2, (ch.nfull + kThreads - 1) / kThreads)
                                 : chunk_lse(ch, row, a.kv, c2),
                            c2, sm, 0);
    // The packed maximum skips elements of magnitude 2^121 or more, +inf and
    // NaN. A skipped element above the maximum overflows the sum (+inf or
    // NaN), and a chunk whose every element is skipped or -inf reads as -inf:
    // in both cases the plain scan takes the chunk again. (If the row has no
    // distribution, its statistics stay non-finite and the decision reports
    // the sequence.)
    if (fast && (!(st.s <= 3.0e38f) || st.M == -INFINITY)) st = block_lse(chunk_lse(ch, row, a.kv, c2), c2, sm, 0);
    const uint64_t w = pack(st.M, __float_as_uint(st.s));
    if (draft_item) w1 = w;
    else w0 = w;
  }
  if (threadIdx.x == 0) {
    P1Slot* dst = a.p1 + ((int64_t)b * a.gamma + i) * a.nchunks + c;
    if (draft_item) {
      xput64(&dst->w1, w1);
    } else {
      xput64(&dst->w0, w0);
      if (a.draft == nullptr || kind == KIND_GREEDY) xput64(&dst->w1, w1);
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 2: one chunk of the row a decided sequence draws its last token from.
// ---------------------------------------------------------------------------
// Whether idx is one of the n entries of list l (a short list in LDS).
__device__ __forceinline__ bool in_list(const int32_t* l, int n, int idx) {
  for (int i = 0; i < n; ++i)
    if (l[i] == idx) return true;
  return false;
}

// The end of a Gumbel chunk: the workgroup's best (value, index), the sum
// of beta and the OR of any, through one exchange in LDS (each reduced
// within the wave first, then over the waves in wave order).
__device__ __forceinline__ void block_draw_result(ArgMax m, float beta, int any, Smem& sm, P2Slot* out) {
  m = wave_argmax(m);
  beta = wave_sum(beta);
  any = wave_or(any);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm.am[w] = m;
    sm.fsum[w] = beta;
    sm.ior[w] = any;
  }
  __syncthreads();
  ArgMax r = sm.am[0];
  float bs = sm.fsum[0];
  int ba = sm.ior[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) {
    r = argmax_merge(r, sm.am[k]);
    bs += sm.fsum[k];
    ba |= sm.ior[k];
  }
  __syncthreads();
  out->w0 = pack(r.v, (uint32_t)r.i);
  out->w1 = pack(bs, (uint32_t)ba);
}

// One chunk of a Gumbel-max draw, specialised on what the score of an element
// is (MODE = P2_RESIDUAL: ln(p - q) where p > q; P2_RESIDUAL_ONEHOT: l/T for
// v != x; P2_BONUS: l/T). For each 16-byte vector the lane forms the Philox
// words and the pruning test of its elements; the exact score and noise are
// evaluated only when some element survives (rare once the bound has risen),
// lowest index first. Vectors are prefetched three deep. EXCL: the excl[0 .. nexcl)
// elements take no part (sampled trees whose siblings were drawn without
// replacement).
template <bool BF16, bool VEC, int MODE, bool EXCL = false>
__device__ __forceinline__ void gumbel_chunk(const ChainArgs& a, int b, const Decision dec, int lo, int hi, Smem& sm, P2Slot* out,
                             const int32_t* excl = nullptr, int nexcl = 0) {
  using E = Elem<BF16>;
  constexpr int EV = E::kPerVec;
  constexpr bool residual = (MODE == P2_RESIDUAL);
  constexpr bool onehot = (MODE == P2_RESIDUAL_ONEHOT);
  const uint8_t* rt = target_row(a, b, dec.row);
  const uint8_t* rd = residual ? draft_row(a, b, dec.row) : nullptr;
  const float c2 = dec.c2, invT = dec.invT, zt2 = dec.zt2, zd2 = dec.zd2;
  const int xex = dec.x;
  const uint32_t crow = (uint32_t)dec.row, cseq = a.seq_base + (uint32_t)b;
  const uint32_t ctr3 = a.ctr_noise, k0 = a.key0, k1 = a.key1;
  Best bst;
  bst.s = -INFINITY;
  bst.i = -1;
  float beta = 0.0f;
  int any = residual ? 0 : 1;
  float L = -INFINITY;    // best total this wave has reached in the row
  float nL2 = INFINITY;   // -L log2(e)
  float scale = INFINITY; // exp(-L), for the residual's linear test

  auto refresh = [&]() {
    L = wave_max(L);
    nL2 = -L * kLog2e;
    if (residual) scale = fast_exp2(nL2);
  };

  // Residual mass and candidacy of one element (residual mode only).
  auto accumulate = [&](float lt, float ld, float& r_out) -> bool {
    const float lp2 = __builtin_fmaf(lt, c2, -zt2);
    const float lq2 = __builtin_fmaf(ld, c2, -zd2);
    const bool cand = lp2 > lq2;
    const float p = fast_exp2(lp2), q = fast_exp2(lq2);
    const float r = cand ? p - q : 0.0f;
    beta += r;
    any |= cand ? 1 : 0;
    r_out = cand ? __builtin_fmaf(p, 0x1p-22f, r) : 0.0f;  // bound on p - q
    return cand;
  };
  // Pruning test; r is the residual bound from accumulate().
  auto test = [&](float lt, float r, uint32_t w, int idx) -> bool {
    if (EXCL && in_list(excl, nexcl, idx)) return false;
    if (residual) return r > 0.0f && may_win_lin(w, r * scale);
    if (onehot && idx == xex) return false;
    return may_win_log2(w, __builtin_fmaf(lt, c2, nL2));  // log2 exp(l/T - L)
  };
  // Exact score and noise of a surviving element.
  auto full = [&](float lt, float ld, uint32_t w, int idx) {
    float s;
    if (residual) {
      const float lp2 = __builtin_fmaf(lt, c2, -zt2);
      const float lq2 = __builtin_fmaf(ld, c2, -zd2);
      s = lp2 * kLn2 + log1mexp((lq2 - lp2) * kLn2);  // ln (p - q)
    } else {
      s = lt * invT;
    }
    const float tot = s + gumbel(w);
    best_push(bst, tot, idx);
    L = fmaxf(L, tot);
  };

  if (VEC) {
    const int nfull = (hi - lo) / EV;
    // Three vectors per lane in flight: vector r is processed while vectors
    // r+1 and r+2 are still arriving (a rotating set of registers).
    u32x4 qt0, qt1, qt2, qd0, qd1, qd2;
    const int vi0 = (int)threadIdx.x;
    auto fetch = [&](int vi, u32x4& qt, u32x4& qd) {
      if (vi < nfull) {
        qt = load_vec_stream(rt + (int64_t)(lo + vi * EV) * E::kBytes);
        if (residual) qd = load_vec_stream(rd + (int64_t)(lo + vi * EV) * E::kBytes);
      }
    };
    fetch(vi0, qt0, qd0);
    fetch(vi0 + kThreads, qt1, qd1);
    const int rounds = (nfull + kThreads - 1) / kThreads;  // same for every lane
#pragma unroll 1
    for (int rnd = 0; rnd < rounds; ++rnd) {
      const int vi = vi0 + rnd * kThreads;
      fetch(vi + 2 * kThreads, qt2, qd2);
      if (vi < nfull) {
        const int base = lo + vi * EV;
        float vt[EV], vd[EV], rr[EV];
        uint32_t wd[EV];
        E::unpack(qt0, vt);
        if (residual) E::unpack(qd0, vd);
        if (EV == 8) {  // two blocks per vector, computed side by side
          Words4 wa, wb;
          philox10x2((uint32_t)base >> 2, ((uint32_t)base >> 2) + 1u, crow, cseq, ctr3, k0, k1, wa, wb);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wd[e] = wa.w[e];
            wd[4 + e] = wb.w[e];
          }
        } else {
          const Words4 w4 = philox10((uint32_t)base >> 2, crow, cseq, ctr3, k0, k1);
#pragma unroll
          for (int e = 0; e < 4; ++e) wd[e] = w4.w[e];
        }
        bool surv = false;
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          rr[e] = 0.0f;
          if (residual) accumulate(vt[e], vd[e], rr[e]);
          surv |= test(vt[e], rr[e], wd[e], base + e);
        }
        if (surv) {
#pragma unroll
          for (int e = 0; e < EV; ++e)
            if (test(vt[e], rr[e], wd[e], base + e)) full(vt[e], residual ? vd[e] : 0.0f, wd[e], base + e);
        }
      }
      qt0 = qt1;
      qt1 = qt2;
      if (residual) {
        qd0 = qd1;
        qd1 = qd2;
      }
      if ((rnd & 3) == 0 || rnd + 1 == rounds) refresh();
    }
    const int tail_lo = lo + nfull * EV;
    if (tail_lo < hi && (nfull % kThreads) == (int)threadIdx.x) {
      for (int idx = tail_lo; idx < hi; ++idx) {
        const Words4 w4 = philox10((uint32_t)idx >> 2, crow, cseq, ctr3, k0, k1);
        const uint32_t w = word_at(w4, idx & 3);
        const float lt = E::load(rt, idx), ld = residual ? E::load(rd, idx) : 0.0f;
        float r = 0.0f;
        if (residual) accumulate(lt, ld, r);
        if (test(lt, r, w, idx)) full(lt, ld, w, idx);
      }
    }
  } else {
    const int n = hi - lo;
    int rnd = 0;
#pragma unroll 1
    for (int k0i = 0; k0i < n; k0i += kThreads, ++rnd) {
      const int k = k0i + (int)threadIdx.x;
      if (k < n) {
        const int idx = lo + k;
        const Words4 w4 = philox10((uint32_t)idx >> 2, crow, cseq, ctr3, k0, k1);
        const uint32_t w = word_at(w4, idx & 3);
        const float lt = E::load(rt, idx), ld = residual ? E::load(rd, idx) : 0.0f;
        float r = 0.0f;
        if (residual) accumulate(lt, ld, r);
        if (test(lt, r, w, idx)) full(lt, ld, w, idx);
      }
      if ((rnd & 3) == 0 || k0i + kThreads >= n) refresh();
    }
  }
  ArgMax m;
  m.v = bst.s;
  m.i = bst.i;
  block_draw_result(m, beta, any, sm, out);
}

// Wave priority from progress through a chunk: 3 in its first quarter of
// rounds, down to 0 in its last. The pass-2 workgroups of a launch start
// together with equal work, and a SIMD otherwise issues its oldest wave
// first, so those dispatched last would finish last by far; a wave that is
// ahead now yields to those behind it. (Wave priority only, set with
// s_setprio; the queues and streams keep their default priority.) The
// rounds at which the level drops are computed once per chunk.
struct PhaseTable {
  int r1, r2, r3;  // first round of the second, third and fourth quarter
  __device__ __forceinline__ explicit PhaseTable(int rounds) {
    r1 = (rounds + 3) / 4;          // smallest r with 4 r >= rounds
    r2 = (2 * rounds + 3) / 4;
    r3 = (3 * rounds + 3) / 4;
  }
  __device__ __forceinline__ void set(int rnd) const {
    if (rnd != 0 && rnd != r1 && rnd != r2 && rnd != r3) return;
    const int ph = (rnd >= r1) + (rnd >= r2) + (rnd >= r3);
    if (ph == 0) __builtin_amdgcn_s_setprio(3);
    else if (ph == 1) __builtin_amdgcn_s_setprio(2);
    else if (ph == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
};

// One chunk of a Gumbel-max draw over 16-byte-aligned bf16 rows. Each lane
// takes one 8-element vector per round, loaded kBufs - 1 rounds ahead (the
// buffers rotate by unrolling the loop kBufs times, so that no register move
// waits for a load in flight), forms the Philox words of its two 4-element
// blocks and a cheap, conservative pruning test; only the survivors get
// their exact score and noise. Before the first round the workgroup seeds
// its threshold L with the exact total of each lane's highest-scoring
// element of its first vector, and hands the seed to the row's other
// workgroups. L is wave-uniform and rises whenever a survivor beats it, or
// another wave of the workgroup (through LDS) or another workgroup of the
// same row (through the sequence record, read once every kBufs rounds)
// reports a higher total. The residual's bulk test bounds its score by
// log2 p alone (ln (p - q) <= ln p) and reads only the target vector; the
// candidacy test p > q and the tighter bound on log2 (p - q), which read the
// draft vector (loaded with the target vector), are applied only in a
// wave-round where some element passed the first test.
// Vector buffers of the bf16 Gumbel loop: its loads run kBufs - 1 rounds
// ahead of the round that uses them. Two buffers keep the pass-2 kernel
// within 80 VGPRs, six waves per SIMD; a third changes nothing measurable.
constexpr int kBufs = 2;

template <int MODE, bool BETA, bool EXCL = false>
__device__ __forceinline__ void gumbel_chunk_bf16(const ChainArgs& a, int b, const Decision dec, int lo, int hi, Smem& sm,
                                  P2Slot* out, const int32_t* excl = nullptr, int nexcl = 0) {
  using E = Elem<true>;
  constexpr bool residual = (MODE == P2_RESIDUAL);
  constexpr bool onehot = (MODE == P2_RESIDUAL_ONEHOT);
  const uint8_t* rt = target_row(a, b, dec.row);
  const uint8_t* rd = residual ? draft_row(a, b, dec.row) : nullptr;
  const float c2 = dec.c2, invT = dec.invT, zt2 = dec.zt2, zd2 = dec.zd2;
  const int xex = dec.x;
  const uint32_t crow = (uint32_t)dec.row, cseq = a.seq_base + (uint32_t)b;
  const uint32_t ctr3 = a.ctr_noise, k0 = a.key0, k1 = a.key1;
  const int lane = (int)(threadIdx.x & 63);
  Best bst;
  bst.s = -INFINITY;
  bst.i = -1;
  float beta = 0.0f;
  int any = residual ? 0 : 1;
  float mine = -INFINITY;  // best total this lane has reached
  float L = -INFINITY, nL2 = INFINITY;  // wave-uniform
  // The residual mass is summed only for the caller's diagnostics (BETA).
  constexpr bool want_beta = residual && BETA;
  uint32_t* const gkey = &a.seq[b].lbest;
  auto set_L = [&](float l) {
    L = l;
    nL2 = -L * kLog2e;
  };
  // L and the largest total this wave has reported, also as order keys (0:
  // none yet), so that the common case (nothing new) is decided on the
  // scalar unit.
  uint32_t Lk = 0u, Lpk = 0u;
  auto total = [&](float lt, float ld, uint32_t w) -> float {
    float sc;
    if (residual) {
      const float lp2 = __builtin_fmaf(lt, c2, -zt2);
      const float lq2 = __builtin_fmaf(ld, c2, -zd2);
      sc = lp2 * kLn2 + log1mexp((lq2 - lp2) * kLn2);  // ln (p - q)
    } else {
      sc = lt * invT;
    }
    return sc + gumbel(w);
  };

  // Element e (0..7) of a packed 8-element vector.
  auto el = [](const u32x4& q, int e) -> float {
    return __uint_as_float((e & 1) ? (q[e >> 1] & 0xFFFF0000u) : (q[e >> 1] << 16));
  };
  // Bounds of the fast test for the current L: the pattern of n is compared
  // with b 2^23 + log_bias, b an upper bound on the score in log2 units (l c2
  // for the bonus draws, l c2 - zt2 = log2 p for the residual's bulk test).
  // log_bias stays finite (no threshold yet: everything passes), so that
  // b = -inf always fails. The residual's bulk bias carries zt2 and 2^-11 of
  // slack on top of the exact test's 2^-12, which covers its two extra
  // roundings: the bulk test then passes every element the exact one does.
  float c2s = 0.0f, log_bias = 0x1p120f, bulk_bias = 0x1p120f;
  auto set_bounds = [&]() {
    c2s = c2 * 0x1p23f;
    log_bias = __builtin_fminf((nL2 + (33.0f + 127.0f + 0x1p-12f)) * 0x1p23f, 0x1p120f);
    bulk_bias = residual ? __builtin_fminf((nL2 - zt2 + (33.0f + 127.0f + 0x1p-12f + 0x1p-11f)) * 0x1p23f, 0x1p120f)
                         : log_bias;
  };
  set_bounds();
  // L rises to the total of order key k, if that is higher.
  auto raise = [&](uint32_t k) {
    if (k > Lk) {
      Lk = k;
      set_L(key_total(k));
      set_bounds();
    }
  };
  const int nfull = (hi - lo) / 8;
  const int vi0 = (int)threadIdx.x;
  // The chunk's whole vectors as buffers: vector vi is at byte 16 vi, and a
  // lane past the last whole vector reads zeros (masked out below), so that
  // every load is issued by the whole wave.
  // The bulk test reads the target vector only; a residual draw's draft
  // vector is loaded with it all the same: most residual wave-rounds have a
  // survivor that needs it, and a load issued mid-round stalls a wave that
  // has no other waves to hide it (small batches run one per SIMD).
  const __amdgpu_buffer_rsrc_t rs_t = make_rsrc(rt + (int64_t)lo * 2, (uint32_t)nfull * 16u);
  const __amdgpu_buffer_rsrc_t rs_d = residual ? make_rsrc(rd + (int64_t)lo * 2, (uint32_t)nfull * 16u) : rs_t;
  auto fetch = [&](int vi, u32x4& qt, u32x4& qd) {
    qt = load_vec_buf(rs_t, (uint32_t)vi * 16u);
    if (residual) qd = load_vec_buf(rs_d, (uint32_t)vi * 16u);
  };
  // Word 0 of the lane's first Philox block in round 0 (element index / 4);
  // each round advances it by kThreads * 8 / 4.
  const uint32_t cbase = (uint32_t)(lo + vi0 * 8) >> 2;
  const int rounds = (nfull + kThreads - 1) / kThreads;  // same for every lane
  // kBufs vector buffers per row read: the loads run kBufs - 1 rounds ahead
  // of the round that uses them.
  u32x4 qv[kBufs], dv[kBufs];
#pragma unroll
  for (int j = 0; j < kBufs - 1; ++j)
    if (j < rounds) fetch(vi0 + j * kThreads, qv[j], dv[j]);
  // The first vectors have landed before the loop (vmcnt(0)): inside it the
  // compiler then waits only for the vectors of the round it works on, not
  // for the loads of the rounds after it.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  {
    // Seed L: every lane's highest-scoring element of its first vector gets
    // its exact total, and L starts at the largest of them over the
    // workgroup. (The first round tests these elements again: they are
    // pushed twice, to no effect.)
    const int base = lo + vi0 * 8;
    float key = -INFINITY;
    int ke = -1;
    if (vi0 < nfull) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float k;
        if (residual) {
          const float lp2 = __builtin_fmaf(el(qv[0], e), c2, -zt2), lq2 = __builtin_fmaf(el(dv[0], e), c2, -zd2);
          k = lp2 > lq2 ? residual_log2_bound(lp2, lq2) : -INFINITY;
        } else {
          k = (onehot && base + e == xex) ? -INFINITY : el(qv[0], e);
        }
        if (EXCL && in_list(excl, nexcl, base + e)) k = -INFINITY;
        if (k > key) {
          key = k;
          ke = e;
        }
      }
    }
    float t0 = -INFINITY;
    if (ke >= 0) {
      float klt = 0.0f, kld = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e == ke) {
          klt = el(qv[0], e);
          if (residual) kld = el(dv[0], e);
        }
      const int kidx = base + ke;
      t0 = total(klt, kld, word_at(philox10((uint32_t)kidx >> 2, crow, cseq, ctr3, k0, k1), kidx & 3));
      best_push(bst, t0, kidx);
      mine = t0;
    }
    const float wm = wave_max(t0);
    if (lane == 0 && wm != -INFINITY) atomicMax(&sm.lkey, order_key(wm));
    __syncthreads();
    const uint32_t lsk = (uint32_t)__builtin_amdgcn_readfirstlane(
        __hip_atomic_load(&sm.lkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (lsk != 0u) {
      raise(lsk);
      // The seed goes to the other workgroups of the row at once.
      if (threadIdx.x == 0) atomicMax(gkey, lsk);
      Lpk = lsk;
    }
  }
  const PhaseTable phase(rounds);
  // One round over the target vector qt0 (its load issued kBufs - 1 rounds
  // earlier; qd0, the draft vector of a residual draw, loaded with it).
  auto round = [&](int rnd, const u32x4& qt0, const u32x4& qd0) __attribute__((always_inline)) {
    // The unrolled rounds are scheduled one after the other: left to
    // interleave them, the compiler would hold several rounds' Philox words
    // at once and lose occupancy.
    __builtin_amdgcn_sched_barrier(0);
    phase.set(rnd);
    const int vi = vi0 + rnd * kThreads;
    const bool have = vi < nfull;
    const int base = lo + vi * 8;
    // The Philox words first: they do not wait for the vectors.
    Words4 wa, wb;
    // (Every lane forms them: a lane past the chunk's end costs the wave
    // nothing more, and its words are masked out below.)
    const uint32_t cw = cbase + (uint32_t)rnd * (uint32_t)(kThreads * 2);
    philox10x2(cw, cw + 1u, crow, cseq, ctr3, k0, k1, wa, wb);
    if (want_beta && have) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float lp2 = __builtin_fmaf(el(qt0, e), c2, -zt2), lq2 = __builtin_fmaf(el(qd0, e), c2, -zd2);
        beta += lp2 > lq2 ? fast_exp2(lp2) - fast_exp2(lq2) : 0.0f;
      }
    }
    // The bulk test of element e (target vector only). It does not exclude
    // the one-hot draft token or ask whether p > q: the survivor path does.
    // Only whether some lane of the wave has a survivor is kept: the
    // verdicts are lane masks OR-ed on the scalar unit.
    // Each element slot's verdicts stay a wave mask in scalar registers, so
    // that the tests after it run only for the slots, and in them only for
    // the lanes, that passed.
    // First the lane's bound: its largest logit against its smallest n (the
    // complement of its largest word). The test is monotone in both, so a
    // lane that fails it has no element that passes the per-element test;
    // at the large workloads about one wave-round in twenty has a lane that
    // passes, and only then do the eight per-element tests run.
    uint64_t lm[8];
    // Every lane holds a whole vector except, perhaps, in the last round.
    const uint64_t have_m = (rnd + 1 < rounds) ? ~0ull : __builtin_amdgcn_ballot_w64(have);
    const float lmax = max_bound_bf16(qt0);
    uint32_t wmax = wa.w[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) wmax = max(wmax, (e < 4) ? wa.w[e & 3] : wb.w[e & 3]);
    const uint64_t lane_m = lanes_may_win(wmax, __builtin_fmaf(lmax, c2s, bulk_bias)) & have_m;
    uint64_t surv = 0ull;
    if (lane_m != 0ull) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lm[e] = lanes_may_win((e < 4) ? wa.w[e & 3] : wb.w[e & 3], __builtin_fmaf(el(qt0, e), c2s, bulk_bias)) & lane_m;
        surv |= lm[e];
      }
    }
    if (surv != 0ull) {
      // One-hot: the draft token is excluded (xrel: its place in this vector,
      // if it is there).
      const int xrel = onehot ? xex - base : -1;
      const u32x4& qd1 = qd0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (lm[e] == 0ull) continue;
        if (!((lm[e] >> lane) & 1ull)) continue;
        uint32_t w = (e < 4) ? wa.w[e & 3] : wb.w[e & 3];
        // A word the compiler cannot match with the bulk test's, so that it
        // does not keep the bulk test's values in registers for this path.
        asm volatile("" : "+v"(w));
        const float lt = el(qt0, e);
        float tot;
        if (residual) {
          const float lq2 = __builtin_fmaf(el(qd1, e), c2, -zd2), lp2 = __builtin_fmaf(lt, c2, -zt2);
          if (!(lp2 > lq2)) continue;
          const float bnd = residual_log2_bound(lp2, lq2);
          if (!may_win_bits(w, __builtin_fmaf(bnd, 0x1p23f, log_bias))) continue;
          if (EXCL && in_list(excl, nexcl, base + e)) continue;
          // The exact noise first: with it, the bound on the score (in log2
          // units, ln 2 times that in nats) decides most of these elements
          // before the exact score, which costs several library logarithms.
          // An element is dropped only below L by more than a margin that
          // covers this sum's rounding, so every element that could reach L
          // (ties included) goes on to its exact total.
          const float g = gumbel(w);
          if (__builtin_fmaf(bnd, kLn2, g) < L - fmaxf(1.0f, fabsf(L)) * 0x1p-12f) continue;
          tot = lp2 * kLn2 + log1mexp((lq2 - lp2) * kLn2) + g;  // ln (p - q) + G
        } else {
          if (e == xrel || !may_win_bits(w, __builtin_fmaf(lt, c2s, log_bias))) continue;
          if (EXCL && in_list(excl, nexcl, base + e)) continue;
          tot = lt * invT + gumbel(w);
        }
        best_push(bst, tot, base + e);
        mine = fmaxf(mine, tot);
      }
    }
    // Share and collect totals: only a wave with survivors can have a new
    // one, and only one above L and above what it reported is shared.
    uint32_t kn = Lk;
    if (surv != 0ull) {
      // (Read from lane 0, so that the compiler knows it is the same on
      // every lane.)
      const float wm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(mine))));
      if (wm != -INFINITY) {
        const uint32_t kw = (uint32_t)__builtin_amdgcn_readfirstlane(order_key(wm));
        if (kw > Lk && kw > Lpk) {
          if (lane == 0) {
            atomicMax(&sm.lkey, kw);
            atomicMax(gkey, kw);
          }
          Lpk = kw;
        }
        kn = max(kn, kw);
      }
    }
    raise(max(kn, (uint32_t)__builtin_amdgcn_readfirstlane(
                      __hip_atomic_load(&sm.lkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))));
    __builtin_amdgcn_sched_barrier(0);
  };
  // The sequence's best total from the other workgroups of the row: loaded
  // before the first of kBufs rounds' vector loads and read after the last of
  // them, whose vectors were loaded after it (loads complete in order, so it
  // costs no wait of its own).
  auto take_global = [&](uint32_t gk) { raise((uint32_t)__builtin_amdgcn_readfirstlane(gk)); };
#pragma unroll 1
  for (int rnd = 0; rnd < rounds; rnd += kBufs) {
    const uint32_t gk = xload(gkey);
#pragma unroll
    for (int j = 0; j < kBufs; ++j) {
      if (rnd + j >= rounds) break;
      // The buffer freed by the round before this one takes the load of the
      // round kBufs - 1 ahead.
      if (rnd + j + kBufs - 1 < rounds)
        fetch(vi0 + (rnd + j + kBufs - 1) * kThreads, qv[(j + kBufs - 1) % kBufs], dv[(j + kBufs - 1) % kBufs]);
      round(rnd + j, qv[j], dv[j]);
      if (j == kBufs - 1) take_global(gk);
    }
  }
  // Elements past the last whole vector, one by one.
  const int tail_lo = lo + nfull * 8;
  if (tail_lo < hi && (nfull % kThreads) == (int)threadIdx.x) {
    for (int idx = tail_lo; idx < hi; ++idx) {
      const uint32_t w = word_at(philox10((uint32_t)idx >> 2, crow, cseq, ctr3, k0, k1), idx & 3);
      const float lt = E::load(rt, idx), ld = residual ? E::load(rd, idx) : 0.0f;
      bool keep;
      if (residual) {
        const float lp2 = __builtin_fmaf(lt, c2, -zt2), lq2 = __builtin_fmaf(ld, c2, -zd2);
        keep = lp2 > lq2;
        if (keep) {
          beta += fast_exp2(lp2) - fast_exp2(lq2);
          any = 1;
        }
      } else {
        keep = !(onehot && idx == xex);
      }
      if (EXCL && keep && in_list(excl, nexcl, idx)) keep = false;
      if (keep) best_push(bst, total(lt, ld, w), idx);
    }
  }
  // A residual chunk with a candidate (p > q) has a finite best total: the
  // pruning skips an element only below a total some element of the row has
  // reached, and with no such total yet every candidate is evaluated. So the
  // row has a candidate iff some chunk reports a finite best; the main loop
  // does not track candidates separately.
  if (residual && bst.i >= 0) any = 1;
  ArgMax m;
  m.v = bst.s;
  m.i = bst.i;
  block_draw_result(m, beta, any, sm, out);
}

// Greedy bonus draw over [lo, hi): the target row's argmax (lowest index on
// ties).
template <bool BF16, bool VEC>
__device__ __forceinline__ void greedy_chunk(const ChainArgs& a, int b, const Decision d, int lo, int hi, Smem& sm, P2Slot* out) {
  const uint8_t* rt = target_row(a, b, d.row);
  ArgMax best;
  best.v = -INFINITY;
  best.i = -1;
  for (int lo2 = lo; lo2 < hi; lo2 += a.chunk) {  // in pass-1 sized pieces
    Chunk<BF16, VEC> ct;
    ct.load(rt, lo2, min(hi, lo2 + a.chunk), a.kv);
    best = argmax_merge(best, chunk_argmax(ct, rt, a.kv));
  }
  const ArgMax m = block_argmax(best, sm);
  out->w0 = pack(m.v, (uint32_t)m.i);
  out->w1 = pack(0.0f, 1u);
}

template <bool BF16, bool VEC, bool BETA>
__device__ __forceinline__ void pass2_chunk(const ChainArgs& a, int b, const Decision d, int lo, int hi, Smem& sm, P2Slot* out) {
  if (d.mode == P2_GREEDY_BONUS) {
    greedy_chunk<BF16, VEC>(a, b, d, lo, hi, sm, out);
  } else if (BF16 && VEC) {
    if (d.mode == P2_RESIDUAL) {
      gumbel_chunk_bf16<P2_RESIDUAL, BETA>(a, b, d, lo, hi, sm, out);
    } else if (d.mode == P2_RESIDUAL_ONEHOT) {
      gumbel_chunk_bf16<P2_RESIDUAL_ONEHOT, false>(a, b, d, lo, hi, sm, out);
    } else {
      gumbel_chunk_bf16<P2_BONUS, false>(a, b, d, lo, hi, sm, out);
    }
  } else if (d.mode == P2_RESIDUAL) {
    gumbel_chunk<BF16, VEC, P2_RESIDUAL>(a, b, d, lo, hi, sm, out);
  } else if (d.mode == P2_RESIDUAL_ONEHOT) {
    gumbel_chunk<BF16, VEC, P2_RESIDUAL_ONEHOT>(a, b, d, lo, hi, sm, out);
  } else {
    gumbel_chunk<BF16, VEC, P2_BONUS>(a, b, d, lo, hi, sm, out);
  }
}

// Last pass-2 item of b: merge the chunk partials, write the last token and
// return the sequence's scratch to zero.
template <bool BF16, bool VEC, bool BETA>
__device__ __forceinline__ void finalize(const ChainArgs& a, int b, int p2_chunk, int p2_nchunks, Smem& sm) {
  const int C2 = p2_nchunks, G = a.gamma;
  const Decision d = sm.dec;
  P2Slot* ps = a.p2 + (int64_t)b * a.p2_stride;
  if (d.mode != P2_NONE) {
    // Read every partial at once, then merge them in chunk order.
    ArgMax m;
    m.v = -INFINITY;
    m.i = -1;
    float beta = 0.0f;
    int any = 0;
    for (int base = 0; base < C2; base += kThreads) {
      const int c = base + (int)threadIdx.x;
      if (c < C2) {
        sm.u.slot[threadIdx.x][0] = xget64(&ps[c].w0);
        sm.u.slot[threadIdx.x][1] = xget64(&ps[c].w1);
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        for (int k = 0; k < min(kThreads, C2 - base); ++k) {
          const uint64_t w0 = sm.u.slot[k][0], w1 = sm.u.slot[k][1];
          const int an = (int)lo_u(w1);
          ArgMax o;
          o.v = hi_f(w0);
          o.i = an ? (int)lo_u(w0) : -1;
          m = argmax_merge(m, o);
          beta += hi_f(w1);
          any |= an;
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) sm.ior[0] = any;
    __syncthreads();
    any = sm.ior[0];
    __syncthreads();
    if (d.mode == P2_RESIDUAL && !any) {
      // Empty residual (only through rounding): draw from p at the row instead.
      // No residual total was ever reported (there was no candidate).
      if (threadIdx.x == 0) sm.lkey = 0u;
      __syncthreads();
      Decision fb = d;
      fb.mode = P2_BONUS;
      ArgMax f;
      f.v = -INFINITY;
      f.i = -1;
      for (int c = 0; c < C2; ++c) {
        P2Slot part;
        const int lo = c * p2_chunk;
        if constexpr (BF16 && VEC)
          gumbel_chunk_bf16<P2_BONUS, false>(a, b, fb, lo, min(a.V, lo + p2_chunk), sm, &part);
        else
          pass2_chunk<BF16, VEC, BETA>(a, b, fb, lo, min(a.V, lo + p2_chunk), sm, &part);
        ArgMax o;
        o.v = hi_f(part.w0);
        o.i = (int)lo_u(part.w0);
        f = argmax_merge(f, o);
      }
      m = f;
      beta = 0.0f;
    }
    if (threadIdx.x == 0) {
      if (m.i >= 0) {
        a.out_tokens[(int64_t)b * (G + 1) + d.n] = m.i;
      } else {
        // Nothing to draw from: a row with no entry above -inf (only the bonus
        // row can be one, the others passed the decision's check).
        for (int k = 0; k <= G; ++k) a.out_tokens[(int64_t)b * (G + 1) + k] = -1;
        a.out_n[b] = -5;
      }
      // One-hot draft: (p - delta_x)_+ has mass 1 - p(x) exactly.
      if (a.d_beta && d.mode == P2_RESIDUAL) a.d_beta[b] = beta;
      if (a.d_beta && d.mode == P2_RESIDUAL_ONEHOT) a.d_beta[b] = 1.0f - d.a_row;
    }
  }
  if (d.mode != P2_NONE) {
    uint64_t* w2 = (uint64_t*)ps;
    for (int k = threadIdx.x; k < C2 * 2; k += kThreads) xput64(&w2[k], 0u);
  }
  // Every item of the sequence has read its work entry by now.
  WorkRec* w = a.work + sm.unit[4];
  if (threadIdx.x < 4) xput64(&w->dec[threadIdx.x], 0u);
  if (threadIdx.x == 0) {
    xput(&w->b, 0u);
    xput(&a.seq[b].p2_arrive, 0u);
    xput(&a.seq[b].lbest, 0u);
    // The last sequence to finish returns the list to empty.
    const uint32_t fin = atomicAdd(&a.done[kDoneNFinal], 1u) + 1u;
    if (fin == sm.nwork) {
      xput(&a.done[kDoneNWork], 0u);
      xput(&a.done[kDoneNFinal], 0u);
    }
  }
}

// Entry li of the work list as loaded (thread 0): the sequence and its
// decision record, requested in one round trip.
struct WorkRaw {
  uint64_t d0, d1, d2, d3;
  uint32_t wb;
};

__device__ __forceinline__ WorkRaw load_work(const ChainArgs& a, int li) {
  WorkRec* w = a.work + li;
  WorkRaw r;
  r.d0 = xget64(&w->dec[0]);
  r.d1 = xget64(&w->dec[1]);
  r.d2 = xget64(&w->dec[2]);
  r.d3 = xget64(&w->dec[3]);
  r.wb = xload(&w->b);
  return r;
}

// The decision of a loaded entry. The first launch has completed, so an entry
// below the list's length is complete; returns false if it was never
// published (a workspace left dirty by an earlier call whose wait gave up).
__device__ __forceinline__ bool decode_work(const ChainArgs& a, const WorkRaw& r, int* b, Decision* out) {
  if (!(r.d0 & kRecPublished) || r.wb >= (uint32_t)a.B) {
    atomicOr(&a.done[1], 1u);
    return false;
  }
  Decision d;
  d.kind = KIND_SAMPLED;  // not used by pass 2
  d.T = 0.0f;
  d.mode = (uint32_t)(r.d0 & 0xFFu);
  d.n = (int)((r.d0 >> 8) & 0xFFu) - 64;
  d.row = (int)((r.d0 >> 32) & 0x7FFFFFFFu);
  d.zt2 = hi_f(r.d1);
  d.zd2 = __uint_as_float(lo_u(r.d1));
  d.c2 = hi_f(r.d2);
  d.invT = __uint_as_float(lo_u(r.d2));
  d.a_row = hi_f(r.d3);
  d.x = (int)lo_u(r.d3);
  d.tok = -1;
  *b = (int)r.wb;
  *out = d;
  return true;
}

// Chunk c of the draw of sequence b, whose decision the launch has read
// into sm.dec.
template <bool BF16, bool VEC, bool BETA>
__device__ __forceinline__ void pass2_item(const ChainArgs& a, int b, int c, int p2_chunk, int p2_nchunks, Smem& sm) {
  const Decision d = sm.dec;
  P2Slot part;
  part.w0 = pack(-INFINITY, 0xFFFFFFFFu);
  part.w1 = 0u;
  if (d.mode != P2_NONE) {
    const int lo = c * p2_chunk;
    pass2_chunk<BF16, VEC, BETA>(a, b, d, lo, min(a.V, lo + p2_chunk), sm, &part);
  }
  if (threadIdx.x == 0) {
    sm.flag_last = 0u;
    if (!sm.stalled) {
      if (d.mode != P2_NONE) {
        P2Slot* dst = a.p2 + (int64_t)b * a.p2_stride + c;
        xput64(&dst->w0, part.w0);
        xput64(&dst->w1, part.w1);
        wait_vmem();  // the slot has landed before the arrival
      }
      const uint32_t old = atomicAdd(&a.seq[b].p2_arrive, 1u);
      sm.flag_last = (old == (uint32_t)p2_nchunks - 1u) ? 1u : 0u;
    }
  }
  __syncthreads();
  if (sm.flag_last) {
    __builtin_amdgcn_s_setprio(3);  // a sequence's last step: ahead of other rounds
    finalize<BF16, VEC, BETA>(a, b, p2_chunk, p2_nchunks, sm);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Launches.
// ---------------------------------------------------------------------------
// First launch: every pass-1 item, then one decision item per
// sequence (all pass-1 items have been dispatched before any decision).
// Eight waves per SIMD: pass 1 is bound by how many row chunks are in flight.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void chain_p1_kernel(ChainArgs a) {
  __shared__ Smem sm;
  const int per_seq = p1_items_per_seq(a);
  const uint32_t items = (uint32_t)a.B * per_seq;
  if (blockIdx.x < items) {
    const int b = blockIdx.x / per_seq;
    const int r = blockIdx.x % per_seq;
    pass1_item<BF16, VEC>(a, b, r, sm);
  } else {
    decide<BF16>(a, (int)(blockIdx.x - items), sm);
  }
}

// Second launch: every decision is taken and the sequences with a
// pending draw are on the work list. Their rows are cut into as many chunks
// as fill the launch's workgroups (one resident wave of them), and workgroup
// u takes chunk u mod n of list entry u / n; the others have nothing to do.
template <bool BF16, bool VEC, bool BETA>
// kP2Resident waves per SIMD (at most 80 VGPRs): see kBufs.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kP2Resident))) void chain_p2_kernel(ChainArgs a) {
  __shared__ Smem sm;
  // The start (work record, first vectors, seed) at the highest priority:
  // at the default one it waited behind the rounds of workgroups already in
  // their first phase, up to 13 us instead of 3.
  __builtin_amdgcn_s_setprio(3);
  if (threadIdx.x == 0) {
    // Rows of nw listed draws are cut into nc chunks of len elements each.
    auto geometry = [&](uint32_t nw, int& len, int& nc) {
      int c2 = a.p2_force > 0 ? a.p2_force : a.p2_grid / (int)nw;
      c2 = max(1, min(c2, a.p2_cap));
      len = (a.V + c2 - 1) / c2;
      len = (len + a.p2_unit - 1) / a.p2_unit * a.p2_unit;
      nc = (a.V + len - 1) / len;
    };
    const uint32_t u = blockIdx.x;
    // The entry this workgroup takes when every sequence has a draw pending
    // (the usual case) is requested together with the list's length: one
    // round trip instead of two. Otherwise it is not used.
    int len_all, nc_all;
    geometry((uint32_t)a.B, len_all, nc_all);
    const bool guess = u < (uint32_t)a.B * (uint32_t)nc_all;
    WorkRaw raw_all;
    if (guess) raw_all = load_work(a, (int)(u / (uint32_t)nc_all));
    const uint32_t nw = min(xload(&a.done[kDoneNWork]), (uint32_t)a.B);
    int b = -1, c = 0, len = 0, nc = 0, li = 0;
    if (nw > 0) {
      geometry(nw, len, nc);
      if (u < nw * (uint32_t)nc) {
        li = (int)(u / (uint32_t)nc);
        c = (int)(u % (uint32_t)nc);
        const WorkRaw raw = (nw == (uint32_t)a.B && guess) ? raw_all : load_work(a, li);
        Decision d;
        if (decode_work(a, raw, &b, &d)) {
          sm.dec = d;
          sm.stalled = 0u;
        } else {
          b = -1;  // nothing this workgroup can do: the call reports through done[1]
        }
      }
    }
    sm.lkey = 0u;
    sm.nwork = nw;
    sm.unit[0] = b;
    sm.unit[1] = c;
    sm.unit[2] = len;
    sm.unit[3] = nc;
    sm.unit[4] = li;
  }
  __syncthreads();
  const int b = sm.unit[0];
  if (b < 0) return;
  pass2_item<BF16, VEC, BETA>(a, b, sm.unit[1], sm.unit[2], sm.unit[3], sm);
}

// ===========================================================================
// Sampled trees: multi-round rejection sampling (the pages' "Tree Attention"
// section). One launch gives every sequence W workgroups, each owning wlen
// elements of a row. After an action every workgroup waits until all W have
// arrived with their parts, then takes the sequence's next decisions itself
// from the same parts (so all reach the same state; one of them writes the
// outputs) and carries out the next action on its part of the row: the
// (max, sum exp2) of a node's target and draft rows when the walk reaches a
// node with children (only the nodes on the walked path are read), a
// residual-mass pass before each sibling after the first, or the final
// Gumbel-max draw. The parts of successive
// actions alternate between two slot buffers, since a workgroup can start
// the next action while another still reads the parts of the last.
// After some rejections at a node the target distribution is
// p' = (p - A q)_+ / B. It starts at A = 0, B = 1, and a rejection moves it to
// A' = A + B, B' = sum_v (p - A' q)_+ (one pass over the row pair). This is the
// pages' repeated residual (p' - q)_+ / ||.||_1 in closed form: the accept
// test reads p'(x) from two gathered logits, and the final draw is the
// residual draw of the chains with q scaled by A (log2 A folded into the draft
// normalizer).
// ===========================================================================

enum TreeAction : uint32_t {
  TA_NONE = 0, TA_PASS = 1, TA_DRAW_RESIDUAL = 2, TA_DRAW_BONUS = 3, TA_DONE = 4, TA_STATS = 5
};

// The walk's state: the node, the sibling last tested (round), the path
// length, the target distribution's (A, B) and the node's log2-domain
// normalizers.
struct TreeState {
  int node, round, len;
  float A, Bv, zt2, zd2;
  float An;  // A for the pass after a rejection
  float qd;  // without replacement: q's mass on the siblings drawn so far
};

// Without replacement, per sibling i rejected at the current node: its token,
// its p and q, and F, the value of (p - A q)_+ it keeps once drawn (it leaves
// q, so later rounds no longer subtract from it).
struct TreeDrawn {
  int32_t* x;
  float *p, *q, *F;
};

// All threads: the children of node v in index order into kids[0 .. *nkids)
// (an ordered compaction of the parent array, staged in LDS). wcnt: one word
// per wave of scratch in LDS.
__device__ __forceinline__ void tree_children(int N, const int32_t* par, int v, int32_t* kids, int32_t* nkids, int32_t* wcnt) {
  const int lane = (int)(threadIdx.x & 63), wv = (int)(threadIdx.x >> 6);
  int base = 0;
  for (int k0 = 0; k0 < N; k0 += kThreads) {
    const int k = k0 + (int)threadIdx.x;
    const bool f = k < N && par[k] == v;
    const uint64_t m = __ballot(f);
    if (lane == 0) wcnt[wv] = __popcll(m);
    __syncthreads();
    int off = base, tot = 0;
    for (int w2 = 0; w2 < kThreads / 64; ++w2) {
      if (w2 < wv) off += wcnt[w2];
      tot += wcnt[w2];
    }
    if (f) kids[off + __popcll(m & ((1ull << lane) - 1ull))] = k;
    base += tot;
    __syncthreads();  // wcnt is written again next round
  }
  if (threadIdx.x == 0) *nkids = base;
}

// Thread 0 of every workgroup: the sequence's decisions after the action
// `prev` (TA_NONE: before the first) up to its next action, which it returns;
// s, the state, is updated in place. After a stats action the workgroups'
// (max, sum) pairs are merged in workgroup order into the node's normalizers;
// after a pass the partial masses are summed in workgroup order and the target
// distribution is updated. Then the next sibling is tested: an accepted child
// with children needs its statistics, a rejection the next pass (or, after
// the last sibling, the final residual draw at s.An), and the walk otherwise
// ends in a bonus draw. Only the workgroup with `writer` set writes the
// outputs.
// In LDS: kids[0 .. nkids), the children of s.node in index order; haskid,
// whether each node has children; tok_s, this sequence's node tokens; part,
// the W workgroups' parts of the action just carried out (w0, w1 per
// workgroup). tree_bad, tok_bad: the checks of the tree and of the tokens,
// made by the whole workgroup while staging them. dr: the siblings drawn at
// the current node (without replacement only).
// Without replacement, round j's q is q s over the tokens not drawn yet, with
// s = 1 / (1 - mass of the drawn ones): a rejection moves A to A + B s, and the
// drawn tokens keep the values F they had then (the pass's sum is corrected
// for them with their gathered logits).
template <bool BF16>
__device__ __forceinline__ uint32_t tree_decide(const TreeSampleArgs& ta, int b, uint32_t prev, TreeState& s, const int32_t* kids,
                                int nkids, const uint8_t* haskid, const int32_t* tok_s, float merged0, float merged1,
                                int tree_bad, int tok_bad, bool writer, const TreeDrawn& dr, float T,
                                float pre_lt = 0.0f, float pre_ld = 0.0f, float pre_u = -1.0f) {
  const ChainArgs& a = ta.c;
  const float c2 = kLog2e / T;
  int32_t* path = ta.out_path + (int64_t)b * (ta.max_depth + 1);
  auto to_node = [&](int v) {
    s.node = v;
    s.round = 0;
    s.A = 0.0f;
    s.Bv = 1.0f;
    s.An = 0.0f;
    s.qd = 0.0f;
    s.zt2 = s.zd2 = 0.0f;
  };
  if (prev == TA_NONE) {
    int code = 0;
    if (tree_bad) code = -3;
    else if (!(T > 0.0f) || T == INFINITY) code = -2;
    else if (tok_bad) code = -1;
    // Outputs are written with device-coherent stores: the workgroup that
    // finishes the sequence may run on another XCD, and plain stores to one
    // line from two L2s would be written back in either order.
    if (writer) {
      for (int k = 0; k <= ta.max_depth; ++k) xput(&path[k], -1);
      xput(&ta.out_token[b], -1);
      if (code != 0) xput(&ta.out_len[b], code);
      else xput(&path[0], 0);
    }
    to_node(0);
    s.len = 1;
    if (code != 0) return TA_DONE;
    return haskid[0] ? TA_STATS : TA_DRAW_BONUS;
  }
  if (prev == TA_STATS) {
    // The node's log2 normalizers, merged from the workgroups' parts.
    s.zt2 = merged0;
    s.zd2 = merged1;
  } else {
    float S = merged0;  // the pass's mass, summed over the workgroups' parts
    const int r = s.round;  // the sibling just rejected
    if (ta.wor)
      for (int i = 0; i < r; ++i) S += dr.F[i] - fmaxf(0.0f, dr.p[i] - s.An * dr.q[i]);
    if (S > 0.0f) {  // (a residual of zero mass leaves p as it was)
      s.A = s.An;
      s.Bv = S;
    }
    if (ta.wor) dr.F[r] = fmaxf(0.0f, dr.p[r] - s.A * dr.q[r]);
    s.round += 1;
  }
  const int c = s.round < nkids ? kids[s.round] : -1;
  if (c < 0) {
    // (Not reached: a node's statistics are taken only when it has children,
    // and a pass only when another sibling follows. A draw from the current
    // target distribution.)
    s.An = s.A;
    return s.A > 0.0f ? TA_DRAW_RESIDUAL : TA_DRAW_BONUS;
  }
  const int x = tok_s[c];
  // The two logits of the sibling were gathered while the action ran.
  const float lt = pre_lt, ld = pre_ld;
  const float lp2 = __builtin_fmaf(lt, c2, -s.zt2), lq2 = __builtin_fmaf(ld, c2, -s.zd2);
  const float p = fast_exp2(lp2), q = fast_exp2(lq2);
  const float sfac = (ta.wor && s.qd > 0.0f) ? 1.0f / (1.0f - s.qd) : 1.0f;
  float acc;
  if (s.A == 0.0f && s.Bv == 1.0f && sfac == 1.0f) {
    acc = fast_exp2(fminf(0.0f, lp2 - lq2));  // min(1, p/q), as the chains compute it
  } else {
    // (p - A q)_+ / (B q s) in two divisions: B q s alone can underflow
    // when the residual mass B left is small (B and q near 2^-120), and a
    // zero numerator rejects outright.
    const float num = fmaxf(0.0f, p - s.A * q);
    acc = !(q > 0.0f) ? 1.0f : num > 0.0f ? fminf(1.0f, (num / s.Bv) / (q * sfac)) : 0.0f;
  }
  // The accept uniform of this sibling (formed by another lane while the
  // action ran, or here).
  float u = pre_u;
  if (u < 0.0f)
    u = uniform_accept(philox10((uint32_t)s.round, (uint32_t)s.node, a.seq_base + (uint32_t)b, a.ctr_accept, a.key0, a.key1).w[0]);
  if (u < acc) {
    if (writer && s.len <= ta.max_depth) xput(&path[s.len], c);
    s.len += 1;
    to_node(c);
    // The new node: its statistics first if it has children, else the bonus
    // draw.
    return haskid[c] ? TA_STATS : TA_DRAW_BONUS;
  }
  if (ta.wor) {
    dr.x[s.round] = x;
    dr.p[s.round] = p;
    dr.q[s.round] = q;
    s.qd += q;
  }
  s.An = s.A + s.Bv * sfac;
  // The next sibling's test needs the mass of (p - A' q)_+, A' = s.An.
  if (s.round + 1 < nkids) return TA_PASS;
  // After the last sibling the walk ends with a draw from (p - A' q)_+, whose
  // scale does not matter: a pass would only tell whether it has mass. The
  // draw tells that itself (a residual without mass has no candidate), and
  // then the target distribution stays the one before this rejection
  // (s.A, unchanged).
  s.round += 1;
  return TA_DRAW_RESIDUAL;
}

// This workgroup's part of sum_v (p(v) - A q(v))_+ over [lo, hi), with the
// factor A folded into the draft normalizer (zd2s = zd2 - log2 A).
template <bool BF16, bool VEC>
__device__ __forceinline__ float residual_mass_part(const uint8_t* rt, const uint8_t* rd, int lo, int hi, float c2, float zt2,
                                    float zd2s) {
  using E = Elem<BF16>;
  constexpr int EV = E::kPerVec;
  float s = 0.0f;
  auto add = [&](float lt, float ld) {
    const float lp2 = __builtin_fmaf(lt, c2, -zt2), lq2 = __builtin_fmaf(ld, c2, -zd2s);
    if (lp2 > lq2) s += fast_exp2(lp2) - fast_exp2(lq2);
  };
  int idx0 = lo;
  if (VEC) {
    const int nfull = (hi - lo) / EV;
    for (int base = 0; base < nfull; base += 4 * kThreads) {
      u32x4 qt[4], qd[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int vi = base + k * kThreads + (int)threadIdx.x;
        if (vi < nfull) {
          qt[k] = load_vec_stream(rt + (int64_t)(lo + vi * EV) * E::kBytes);
          qd[k] = load_vec_stream(rd + (int64_t)(lo + vi * EV) * E::kBytes);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int vi = base + k * kThreads + (int)threadIdx.x;
        if (vi < nfull) {
          float vt[EV], vd[EV];
          E::unpack(qt[k], vt);
          E::unpack(qd[k], vd);
#pragma unroll
          for (int e = 0; e < EV; ++e) add(vt[e], vd[e]);
        }
      }
    }
    idx0 = lo + nfull * EV;
  }
  for (int idx = idx0 + (int)threadIdx.x; idx < hi; idx += kThreads) add(E::load(rt, idx), E::load(rd, idx));
  return s;
}

// This workgroup's part of a draw at node t.node over [lo, hi): from the
// residual (p - A q)_+ (A > 0, log2 A folded into the draft normalizer; the
// siblings excl[0 .. nx) take no part), or from p (A = 0, the bonus).
template <bool BF16, bool VEC>
__device__ __forceinline__ P2Slot tree_draw_part(const ChainArgs& a, int b, const TreeState& t, float T, float A, int lo,
                                                 int hi, const int32_t* excl, int nx, Smem& sm) {
  const bool res = A > 0.0f;
  Decision d;
  d.kind = KIND_SAMPLED;
  d.n = 0;
  d.row = t.node;
  d.x = -1;
  d.T = T;
  d.c2 = kLog2e / T;
  d.invT = 1.0f / T;
  d.zt2 = t.zt2;
  d.zd2 = res ? t.zd2 - fast_log2(A) : t.zd2;
  d.a_row = 0.0f;
  d.tok = -1;
  d.mode = res ? P2_RESIDUAL : P2_BONUS;
  P2Slot part;
  if (BF16 && VEC) {
    if (res && nx > 0) gumbel_chunk_bf16<P2_RESIDUAL, false, true>(a, b, d, lo, hi, sm, &part, excl, nx);
    else if (res) gumbel_chunk_bf16<P2_RESIDUAL, false>(a, b, d, lo, hi, sm, &part);
    else gumbel_chunk_bf16<P2_BONUS, false>(a, b, d, lo, hi, sm, &part);
  } else {
    if (res && nx > 0) gumbel_chunk<BF16, VEC, P2_RESIDUAL, true>(a, b, d, lo, hi, sm, &part, excl, nx);
    else if (res) gumbel_chunk<BF16, VEC, P2_RESIDUAL>(a, b, d, lo, hi, sm, &part);
    else gumbel_chunk<BF16, VEC, P2_BONUS>(a, b, d, lo, hi, sm, &part);
  }
  return part;
}

// The walk's last action, the draw (action TA_DRAW_RESIDUAL or TA_DRAW_BONUS),
// by all threads of workgroup w. Every workgroup draws its part of the row and
// arrives on the sequence's counter; the last to arrive merges the parts in
// part order (lowest index on ties), writes the token and length, and returns
// both part buffers (`parts`, this action's; the other too when
// both_buffers) and the counter to zero.
// Without replacement the siblings drawn before the last one take no part in
// the row's residual draw: each competes at the merge with ln F_i plus its own
// noise, keyed as the row's.
// The residual draw after the last sibling's rejection is taken at t.An with
// no pass before it. If nothing has mass there (no candidate in the row and no
// F_i > 0), the target distribution is the one before that rejection: the
// merging workgroup then draws from it alone, over the whole row (the
// residual at t.A, or p when t.A = 0).
template <bool BF16, bool VEC>
__device__ __forceinline__ void tree_draw_finish(const TreeSampleArgs& ta, int b, int w, const TreeState& t, uint32_t action,
                                                 float T, int lo, int hi, P2Slot* parts, bool both_buffers,
                                                 const TreeDrawn& dr, Smem& sm) {
  const ChainArgs& a = ta.c;
  SeqState* st = a.seq + b;
  const int nx = (ta.wor && action == TA_DRAW_RESIDUAL) ? t.round - 1 : 0;
  float A = action == TA_DRAW_RESIDUAL ? t.An : 0.0f;
  bool whole = false;  // the fallback draw: one workgroup, the whole row
  for (;;) {
    const int ndr = A > 0.0f ? nx : 0;
    const P2Slot part = tree_draw_part<BF16, VEC>(a, b, t, T, A, whole ? 0 : lo, whole ? a.V : hi, dr.x, ndr, sm);
    if (!whole) {
      if (threadIdx.x == 0) {
        xput64(&parts[w].w0, part.w0);
        xput64(&parts[w].w1, part.w1);
        wait_vmem();
        sm.flag_last = (atomicAdd(&st->p2_arrive, 1u) + 1u == (uint32_t)ta.W) ? 1u : 0u;
      }
      __syncthreads();
      if (!sm.flag_last) return;
    }
    if (threadIdx.x == 0) {
      ArgMax m;
      m.v = -INFINITY;
      m.i = -1;
      for (int k = 0; k < (whole ? 1 : ta.W); ++k) {
        const uint64_t w0 = whole ? part.w0 : xget64((uint64_t*)&parts[k].w0);
        ArgMax o;
        o.v = hi_f(w0);
        o.i = (int)lo_u(w0);
        m = argmax_merge(m, o);
      }
      for (int i = 0; i < ndr; ++i) {
        if (!(dr.F[i] > 0.0f)) continue;
        const int x = dr.x[i];
        ArgMax o;
        o.v = logf(dr.F[i]) + gumbel(word_at(philox10((uint32_t)x >> 2, (uint32_t)t.node, a.seq_base + (uint32_t)b,
                                                      a.ctr_noise, a.key0, a.key1), x & 3));
        o.i = x;
        m = argmax_merge(m, o);
      }
      const bool again = !whole && action == TA_DRAW_RESIDUAL && m.i < 0;
      if (!again) {
        xput(&ta.out_token[b], m.i);
        xput(&ta.out_len[b], t.len);
      } else {
        // The fallback draw starts from no threshold.
        sm.lkey = 0u;
        xput(&st->lbest, 0u);
      }
      sm.again = again ? 1u : 0u;
    }
    __syncthreads();
    if (!sm.again) break;
    whole = true;
    A = t.A;
  }
  uint64_t* s0 = (uint64_t*)(a.p2 + (int64_t)b * a.p2_stride);
  uint64_t* s1 = (uint64_t*)(ta.slot2 + (int64_t)b * a.p2_stride);
  for (int k = threadIdx.x; k < 2 * ta.W; k += kThreads) {
    xput64(&s0[k], 0u);
    if (both_buffers) xput64(&s1[k], 0u);
  }
  if (threadIdx.x == 0) {
    xput(&st->lbest, 0u);
    xput(&st->p2_arrive, 0u);
  }
}

// Walk launch: W workgroups per sequence, sequences [b_base, b_base + b_count).
// Every workgroup of the launch must be resident at once (the host sizes the
// launch for that); each wait is bounded all the same.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void tree_walk_kernel(TreeSampleArgs ta) {
  __shared__ Smem sm;
  const ChainArgs& a = ta.c;
  const int b = ta.b_base + (int)(blockIdx.x / (uint32_t)ta.W);
  const int w = (int)(blockIdx.x % (uint32_t)ta.W);
  if (b >= ta.b_base + ta.b_count) return;  // whole sequences only
  const int lo = w * ta.wlen, hi = min(a.V, lo + ta.wlen);
  // The tree and this sequence's tokens in LDS, with the checks of the tree
  // (root first at depth 0; every other parent an earlier node, one level
  // up; no node deeper than max_depth) and of the tokens, one node per lane.
  __shared__ int32_t s_par[kMaxTreeNodes], s_tok[kMaxTreeNodes], s_kids[kMaxTreeNodes];
  __shared__ uint8_t s_haskid[kMaxTreeNodes];
  __shared__ int32_t s_nkids, s_wcnt[kThreads / 64];
  __shared__ TreeState s_state;
  __shared__ uint32_t s_action;
  __shared__ float s_unif;  // the accept uniform of the sibling the next decision tests
  __shared__ int32_t s_dx[kMaxTreeNodes];
  __shared__ float s_dp[kMaxTreeNodes], s_dq[kMaxTreeNodes], s_dF[kMaxTreeNodes];
  TreeDrawn dr;
  dr.x = s_dx;
  dr.p = s_dp;
  dr.q = s_dq;
  dr.F = s_dF;
  int tree_bad = 0, tok_bad = 0;
  for (int k = threadIdx.x; k < ta.N; k += kThreads) {
    const int pk = ta.parents[k], dk = ta.depth[k], xk = ta.tokens[(int64_t)b * ta.N + k];
    s_par[k] = pk;
    s_tok[k] = xk;
    s_haskid[k] = 0;
    if (k == 0) {
      tree_bad |= pk != -1 || dk != 0;
    } else {
      tree_bad |= !(pk >= 0 && pk < k) || dk > ta.max_depth || dk != ta.depth[pk >= 0 && pk < k ? pk : 0] + 1;
      tok_bad |= xk < 0 || xk >= a.V;
    }
  }
  tree_bad = __syncthreads_or(tree_bad);
  tok_bad = __syncthreads_or(tok_bad);
  for (int k = 1 + (int)threadIdx.x; k < ta.N; k += kThreads)
    if (s_par[k] >= 0 && s_par[k] < ta.N) s_haskid[s_par[k]] = 1;
  __syncthreads();
  if (ta.wor) {
    // Without replacement, siblings carry distinct tokens.
    int dup = 0;
    for (int k = 1 + (int)threadIdx.x; k < ta.N; k += kThreads)
      for (int k2 = 1; k2 < k; ++k2) dup |= s_par[k2] == s_par[k] && s_tok[k2] == s_tok[k];
    tok_bad |= __syncthreads_or(dup);
  }
  // The sequence's temperature, read once.
  const float T = a.temperature[b];
  // The first decisions need no part of any workgroup.
  if (threadIdx.x == 0) {
    TreeState s0;
    s_action = tree_decide<BF16>(ta, b, TA_NONE, s0, s_kids, 0, s_haskid, s_tok, 0.0f, 0.0f, tree_bad, tok_bad, w == 0, dr, T);
    s_state = s0;
    sm.lkey = 0u;
  }
  __syncthreads();
  uint32_t action = s_action;
  if (action == TA_DONE) return;  // a bad input: nothing was touched
  const float c2 = kLog2e / T;
  // Statistics pieces: four vectors per thread (a slice is usually one piece).
  constexpr int kPieceVecs = 4;
  constexpr int piece = kThreads * Elem<BF16>::kPerVec * kPieceVecs;
  // The first piece of this workgroup's slice of the target and draft rows of
  // the child the next decision tests (if it has children), loaded while the
  // parts are exchanged: if the walk enters that child, its statistics start
  // from them.
  Chunk<BF16, VEC, kPieceVecs> spec[2];
  int spec_node = -1;
  // A slice that is one piece of whole vectors keeps, from the statistics
  // action, every element's exp2((l - M) c2) of the node's target and draft
  // rows (M: the thread's own maximum of each), so that the residual-mass
  // passes at that node need neither its rows nor an exponential.
  float ct[kPieceVecs * 8], cd[kPieceVecs * 8];
  float cMt = -INFINITY, cMd = -INFINITY;
  int cnode = -1;
  const bool keep = BF16 && VEC && hi - lo <= piece && ((hi - lo) & 7) == 0;
  int kids_node = -1;  // the node whose children s_kids holds
  for (uint32_t epoch = 0; epoch <= (uint32_t)ta.N + 2u; ++epoch) {
    const TreeState t = s_state;
    if (action == TA_DRAW_RESIDUAL || action == TA_DRAW_BONUS) {
      // The last action: the draw (parts in buffer epoch & 1).
      P2Slot* parts = ((epoch & 1u) ? ta.slot2 : a.p2) + (int64_t)b * a.p2_stride;
      tree_draw_finish<BF16, VEC>(ta, b, w, t, action, T, lo, hi, parts, epoch > 0u, dr, sm);
      return;
    }
    // The node's children, and the two logits at the node of the sibling the
    // next decision tests (the first child after the statistics, the next one
    // after a pass), requested now so that they have landed by then.
    // (Passes stay at the node: its children are already staged.)
    if (t.node != kids_node) {
      tree_children(ta.N, s_par, t.node, s_kids, &s_nkids, s_wcnt);
      __syncthreads();
      kids_node = t.node;
    }
    float pre_lt = 0.0f, pre_ld = 0.0f;
    if (threadIdx.x == 0 && (action == TA_STATS || action == TA_PASS)) {
      const int next = action == TA_STATS ? 0 : t.round + 1;
      if (next < s_nkids) {
        const int x = s_tok[s_kids[next]];
        pre_lt = Elem<BF16>::load(target_row(a, b, t.node), x);
        pre_ld = Elem<BF16>::load(draft_row(a, b, t.node), x);
      }
    }
    // ... and that sibling's accept uniform, formed on another wave.
    if (threadIdx.x == 64) {
      const int next = action == TA_STATS ? 0 : t.round + 1;
      s_unif = (action == TA_STATS || action == TA_PASS)
                   ? uniform_accept(philox10((uint32_t)next, (uint32_t)t.node, a.seq_base + (uint32_t)b, a.ctr_accept,
                                             a.key0, a.key1).w[0])
                   : -1.0f;
    }
    float partial = 0.0f;
    P2Slot part;
    part.w0 = pack(-INFINITY, 0xFFFFFFFFu);
    part.w1 = 0u;
    // The tag of this action's parts (nonzero: slots hold zero between calls).
    const uint32_t tag = epoch + 1u;
    if (action == TA_STATS) {
      // The log2 normalizers of the node's target and draft rows over
      // [lo, hi): both slices requested at once, in pieces of the launch's
      // tile.
      LseState acc[2];
      acc[0].M = acc[1].M = -INFINITY;
      acc[0].s = acc[1].s = 0.0f;
      const uint8_t* rows[2] = {target_row(a, b, t.node), draft_row(a, b, t.node)};
      for (int lo2 = lo; lo2 < hi; lo2 += piece) {
        const int hi2 = min(hi, lo2 + piece);
        const bool fast = BF16 && VEC && ((hi2 - lo2) & 7) == 0;
        Chunk<BF16, VEC, kPieceVecs> ch[2];
        if (lo2 == lo && spec_node == t.node) {
          ch[0] = spec[0];
          ch[1] = spec[1];
        } else {
          ch[0].load(rows[0], lo2, hi2, kPieceVecs);
          ch[1].load(rows[1], lo2, hi2, kPieceVecs);
        }
        const int kvn = (ch[0].nfull + kThreads - 1) / kThreads;
        LseState mine[2];
#pragma unroll
        for (int kind = 0; kind < 2; ++kind) {
          if (fast && hi2 - lo2 != piece) ch[kind].pad_neg_inf();
          if (keep) {
            mine[kind] = lse_packed_bf16_keep(ch[kind].q, c2, kvn, kind ? cd : ct);
            if (kind) cMd = mine[kind].M;
            else cMt = mine[kind].M;
          } else {
            mine[kind] = fast ? lse_packed_bf16(ch[kind].q, c2, kvn) : chunk_lse(ch[kind], rows[kind], kPieceVecs, c2);
          }
        }
        block_lse2(mine[0], mine[1], c2, sm);
        acc[0] = lse_merge(acc[0], mine[0], c2);
        acc[1] = lse_merge(acc[1], mine[1], c2);
      }
      cnode = keep ? t.node : -1;
      const float zt = acc[0].M == -INFINITY ? -INFINITY : acc[0].M * c2 + fast_log2(acc[0].s);
      const float zd = acc[1].M == -INFINITY ? -INFINITY : acc[1].M * c2 + fast_log2(acc[1].s);
      part.w0 = ((uint64_t)__float_as_uint(zt) << 32) | tag;
      part.w1 = ((uint64_t)__float_as_uint(zd) << 32) | tag;
    } else if (action == TA_PASS) {
      const float zd2s = t.zd2 - fast_log2(t.An);
      float mass;
      if (cnode == t.node) {
        // p = exp2(l c2 - zt2) = exp2(M c2 - zt2) exp2((l - M) c2), and A q
        // likewise with zd2 - log2 A.
        const float at = cMt == -INFINITY ? 0.0f : fast_exp2(__builtin_fmaf(cMt, c2, -t.zt2));
        const float ad = cMd == -INFINITY ? 0.0f : fast_exp2(__builtin_fmaf(cMd, c2, -zd2s));
        mass = 0.0f;
#pragma unroll
        for (int i = 0; i < kPieceVecs * 8; ++i) {
          const float pv = at * ct[i], qv = ad * cd[i];
          if (pv > qv) mass += pv - qv;
        }
      } else {
        mass = residual_mass_part<BF16, VEC>(target_row(a, b, t.node), draft_row(a, b, t.node), lo, hi, c2, t.zt2, zd2s);
      }
      partial = block_sum(mass, sm);
      part.w0 = ((uint64_t)__float_as_uint(partial) << 32) | tag;
      part.w1 = tag;
    }
    spec_node = -1;
    if (action == TA_STATS || action == TA_PASS) {
      const int next = action == TA_STATS ? 0 : t.round + 1;
      const int c = next < s_nkids ? s_kids[next] : -1;
      if (c >= 0) {
        // (A leaf child is drawn from at once, from its target row only: its
        // statistics are never taken, and the load only brings that slice
        // into the cache for the draw.)
        const int hi2 = min(hi, lo + piece);
        spec[0].load(target_row(a, b, c), lo, hi2, kPieceVecs);
        if (s_haskid[c]) spec[1].load(draft_row(a, b, c), lo, hi2, kPieceVecs);
        spec_node = c;
      }
    }
    // This workgroup's part goes to buffer epoch & 1 (a workgroup can start
    // the next action while another still reads this one's parts).
    P2Slot* parts = ((epoch & 1u) ? ta.slot2 : a.p2) + (int64_t)b * a.p2_stride;
    // Statistics and passes: every word of a part carries the action's tag,
    // so a part is complete when both its words show it. Thread k reads part
    // k until it does (a bounded wait), then every workgroup takes the same
    // decisions from the same parts.
    if (threadIdx.x == 0) {
      xput64(&parts[w].w0, part.w0);
      xput64(&parts[w].w1, part.w1);
    }
    int stalled = 0;
    for (int k = threadIdx.x; k < ta.W; k += kThreads) {
      uint64_t w0 = xget64((uint64_t*)&parts[k].w0), w1 = xget64((uint64_t*)&parts[k].w1);
      for (uint32_t spins = 0; (uint32_t)w0 != tag || (uint32_t)w1 != tag; ++spins) {
        if (spins > a.spin_limit || ((spins & 255u) == 255u && xget(&a.done[1]) != 0u)) {
          atomicOr(&a.done[1], 1u);
          stalled = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        w0 = xget64((uint64_t*)&parts[k].w0);
        w1 = xget64((uint64_t*)&parts[k].w1);
      }
      sm.u.slot[k][0] = w0 >> 32;
      sm.u.slot[k][1] = w1 >> 32;
    }
    if (__syncthreads_or(stalled)) {
      if (threadIdx.x == 0) xput(&ta.out_len[b], -4);
      return;
    }
    // Wave 0 merges the parts, lane k taking parts k, k + 64, ... (a fixed
    // order): the statistics' log2 normalizers (largest part, then the sum of
    // exp2 of each part less it), or the pass's mass. Thread 0 then decides.
    if (threadIdx.x < 64) {
      float m0, m1 = 0.0f;
      if (action == TA_STATS) {
        float lt = -INFINITY, ld = -INFINITY;
        for (int k = threadIdx.x; k < ta.W; k += 64) {
          lt = fmaxf(lt, __uint_as_float((uint32_t)sm.u.slot[k][0]));
          ld = fmaxf(ld, __uint_as_float((uint32_t)sm.u.slot[k][1]));
        }
        const float mt = wave_max(lt), md = wave_max(ld);
        float st = 0.0f, sd = 0.0f;
        for (int k = threadIdx.x; k < ta.W; k += 64) {
          const float zt = __uint_as_float((uint32_t)sm.u.slot[k][0]), zd = __uint_as_float((uint32_t)sm.u.slot[k][1]);
          if (zt != -INFINITY) st += fast_exp2(zt - mt);
          if (zd != -INFINITY) sd += fast_exp2(zd - md);
        }
        st = wave_sum(st);
        sd = wave_sum(sd);
        m0 = mt == -INFINITY ? -INFINITY : mt + fast_log2(st);
        m1 = md == -INFINITY ? -INFINITY : md + fast_log2(sd);
      } else {
        float S = 0.0f;
        for (int k = threadIdx.x; k < ta.W; k += 64) S += __uint_as_float((uint32_t)sm.u.slot[k][0]);
        m0 = wave_sum(S);
      }
      if (threadIdx.x == 0) {
        TreeState s1 = s_state;
        s_action = tree_decide<BF16>(ta, b, action, s1, s_kids, s_nkids, s_haskid, s_tok, m0, m1, 0, 0, w == 0, dr, T,
                                     pre_lt, pre_ld, s_unif);
        s_state = s1;
        sm.lkey = 0u;
      }
    }
    __syncthreads();
    action = s_action;
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t nwords) {
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < nwords; k += (size_t)gridDim.x * blockDim.x)
    p[k] = 0u;
}

template <bool BF16, bool VEC>
hipError_t launch_chain_p1_t(const ChainArgs& a, hipStream_t stream) {
  const long long n1 = (long long)a.gamma * a.nchunks * (a.draft != nullptr ? 2 : 1);
  hipLaunchKernelGGL((chain_p1_kernel<BF16, VEC>), dim3((unsigned)(a.B * (n1 + 1))), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, bool VEC>
hipError_t launch_chain_p2_t(const ChainArgs& a, hipStream_t stream) {
  // The variant that also sums the residual mass runs only for diagnostics.
  if (a.d_beta)
    hipLaunchKernelGGL((chain_p2_kernel<BF16, VEC, true>), dim3((unsigned)a.p2_grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((chain_p2_kernel<BF16, VEC, false>), dim3((unsigned)a.p2_grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain_p1(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream) {
  if (bf16) return vec ? launch_chain_p1_t<true, true>(a, stream) : launch_chain_p1_t<true, false>(a, stream);
  return vec ? launch_chain_p1_t<false, true>(a, stream) : launch_chain_p1_t<false, false>(a, stream);
}

hipError_t launch_chain_p2(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream) {
  if (bf16) return vec ? launch_chain_p2_t<true, true>(a, stream) : launch_chain_p2_t<true, false>(a, stream);
  return vec ? launch_chain_p2_t<false, true>(a, stream) : launch_chain_p2_t<false, false>(a, stream);
}

template <bool BF16, bool VEC>
int p2_occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, chain_p2_kernel<BF16, VEC, false>, kThreads, 0) != hipSuccess) n = 0;
  return n;
}

int chain_p2_occupancy(bool bf16, bool vec) {
  if (bf16) return vec ? p2_occupancy_t<true, true>() : p2_occupancy_t<true, false>();
  return vec ? p2_occupancy_t<false, true>() : p2_occupancy_t<false, false>();
}

template <bool BF16, bool VEC>
hipError_t launch_tree_sample_walk_t(const TreeSampleArgs& a, hipStream_t stream) {
  const long long grid = (long long)a.b_count * a.W;
  hipLaunchKernelGGL((tree_walk_kernel<BF16, VEC>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_tree_sample_walk(const TreeSampleArgs& a, bool bf16, bool vec, hipStream_t stream) {
  if (bf16) return vec ? launch_tree_sample_walk_t<true, true>(a, stream) : launch_tree_sample_walk_t<true, false>(a, stream);
  return vec ? launch_tree_sample_walk_t<false, true>(a, stream) : launch_tree_sample_walk_t<false, false>(a, stream);
}

template <bool BF16, bool VEC>
int tree_walk_occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, tree_walk_kernel<BF16, VEC>, kThreads, 0) != hipSuccess) n = 0;
  return n;
}

int tree_sample_walk_occupancy(bool bf16, bool vec) {
  if (bf16) return vec ? tree_walk_occupancy_t<true, true>() : tree_walk_occupancy_t<true, false>();
  return vec ? tree_walk_occupancy_t<false, true>() : tree_walk_occupancy_t<false, false>();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t nwords = bytes / 4;
  if (nwords == 0) return hipSuccess;
  size_t blocks = (nwords + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)p, nwords);
  return hipGetLastError();
}

}  // namespace sv
