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
//   pass-1 item (b, i, c): chunk c of target row i (and of draft row i): the
//     partial log-sum-exp state of each row and, for greedy sequences, the
//     partial argmax. The last pass-1 item of sequence b to finish takes the
//     accept decisions of b (it sees every partial), writes the accepted
//     drafts and publishes which row pass 2 must draw from.
//   pass-2 item (b, c): chunk c of that row: a partial Gumbel-max (or argmax).
//     The last one to finish merges the partials and writes the last token.
// Items are handed out from per-XCD ticket queues by a persistent grid; the
// pass-2 items of a sequence are queued `lag` sequences behind its pass-1
// items so that pass 2 runs while other sequences stream pass 1. A pass-2
// item whose sequence is not decided yet waits; every item it can wait for
// holds an earlier ticket of the same queue, so it is already running and
// never waits itself. Merges run in fixed chunk order, so results do not
// depend on the grid, the queue order or which workgroup finishes last.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

// ---------------------------------------------------------------------------
// Shared-memory scratch of one workgroup.
// ---------------------------------------------------------------------------
struct Smem {
  LseState lse[2][kWaves];
  ArgMax am[kWaves];
  float fsum[kWaves];
  int ior[kWaves];
  uint32_t ticket;
  uint32_t flag_last;
  // decision of one sequence
  int32_t g[kMaxGamma + 1];
  int32_t acc[kMaxGamma];
  float logz2_t[kMaxGamma];
  float logz2_d[kMaxGamma];
  // pass-2 parameters broadcast from thread 0
  uint32_t mode, error;
  int32_t row, x;
  float z_t, z_d;
};

__device__ __forceinline__ LseState block_lse(LseState st, float c, Smem& sm, int slot) {
  st = wave_lse(st, c);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm.lse[slot][w] = st;
  __syncthreads();
  LseState r = sm.lse[slot][0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = lse_merge(r, sm.lse[slot][k], c);
  __syncthreads();
  return r;
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

__device__ __forceinline__ int block_or(int x, Smem& sm) {
  x = wave_or(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm.ior[w] = x;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) r |= sm.ior[k];
  __syncthreads();
  return r;
}

// Sequence classification from its temperature.
enum SeqKind { KIND_BAD_T = 0, KIND_GREEDY = 1, KIND_SAMPLED = 2 };

__device__ __forceinline__ int seq_kind(const ChainArgs& a, int b, float* T_out) {
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
  return a.draft + ((int64_t)b * a.gamma + i) * a.d_stride;
}

// ---------------------------------------------------------------------------
// Chunk loaders. A chunk [lo, hi) is read as 16-byte vectors: thread t holds
// vectors t, t + 256, ... (at most kv of them); elements past the last whole
// vector (a ragged tail) are read one by one by the thread owning the next
// vector index. Without 16-byte alignment every element is read singly.
// ---------------------------------------------------------------------------
template <bool BF16, bool VEC>
struct Chunk {
  using E = Elem<BF16>;
  static constexpr int EV = E::kPerVec;
  u32x4 q[kMaxVecsPerThread];
  int nfull;  // whole vectors in the chunk
  int lo, hi;

  __device__ __forceinline__ void load(const uint8_t* row, int lo_, int hi_, int kv) {
    lo = lo_;
    hi = hi_;
    nfull = VEC ? (hi - lo) / EV : 0;
    if (VEC) {
#pragma unroll
      for (int k = 0; k < kMaxVecsPerThread; ++k) {
        const int vi = k * kThreads + (int)threadIdx.x;
        if (k < kv && vi < nfull) q[k] = load_vec_stream(row + (int64_t)(lo + vi * EV) * E::kBytes);
      }
    }
  }

  // Calls f(value, index) for each element this thread owns, in increasing
  // index order.
  template <typename F>
  __device__ __forceinline__ void for_each(const uint8_t* row, int kv, F&& f) const {
    if (VEC) {
#pragma unroll
      for (int k = 0; k < kMaxVecsPerThread; ++k) {
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

// Partial log-sum-exp state of the thread's elements of a loaded chunk.
template <bool BF16, bool VEC>
__device__ __forceinline__ LseState chunk_lse(const Chunk<BF16, VEC>& ch, const uint8_t* row, int kv,
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

template <bool BF16, bool VEC>
__device__ __forceinline__ ArgMax chunk_argmax(const Chunk<BF16, VEC>& ch, const uint8_t* row, int kv) {
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
// The decision of sequence b, taken by the last pass-1 item of b.
// ---------------------------------------------------------------------------
__device__ void decide(const ChainArgs& a, int b, Smem& sm) {
  const int G = a.gamma;
  const int C = a.nchunks;
  const int tid = threadIdx.x;
  float T;
  const int kind = seq_kind(a, b, &T);
  const int32_t* ids = a.ids + (int64_t)b * G;
  int32_t* tok = a.out_tokens + (int64_t)b * (G + 1);
  SeqState* st = a.seq + b;
  bool bad_id = false;
  for (int i = 0; i < G; ++i) bad_id |= (ids[i] < 0 || ids[i] >= a.V);
  const float c2 = (kind == KIND_SAMPLED) ? kLog2e / T : 0.0f;

  if (kind == KIND_GREEDY && !bad_id) {
    if (tid < G) {
      ArgMax m;
      m.v = -INFINITY;
      m.i = -1;
      const P1Partial* pp = a.p1 + ((int64_t)b * G + tid) * C;
      for (int c = 0; c < C; ++c) {
        ArgMax o;
        o.v = pp[c].a;
        o.i = __float_as_int(pp[c].b);
        m = argmax_merge(m, o);
      }
      sm.g[tid] = m.i;
      if (a.d_accept) a.d_accept[(int64_t)b * G + tid] = (ids[tid] == m.i) ? 1.0f : 0.0f;
      if (a.d_logzt) a.d_logzt[(int64_t)b * G + tid] = NAN;
      if (a.d_logzd) a.d_logzd[(int64_t)b * G + tid] = NAN;
    }
  } else if (kind == KIND_SAMPLED && !bad_id) {
    if (tid < G) {
      LseState mt, md;
      mt.M = -INFINITY;
      mt.s = 0.0f;
      md = mt;
      const P1Partial* pp = a.p1 + ((int64_t)b * G + tid) * C;
      for (int c = 0; c < C; ++c) {
        LseState o;
        o.M = pp[c].a;
        o.s = pp[c].b;
        mt = lse_merge(mt, o, c2);
        o.M = pp[c].c;
        o.s = pp[c].d;
        md = lse_merge(md, o, c2);
      }
      const Gathered gx = a.gath[(int64_t)b * G + tid];
      const float z2t = mt.M * c2 + fast_log2(mt.s);
      const float lp2 = __builtin_fmaf(gx.lt, c2, -z2t);
      float z2d = NAN, lq2 = 0.0f;
      if (a.draft != nullptr) {
        z2d = md.M * c2 + fast_log2(md.s);
        lq2 = __builtin_fmaf(gx.ld, c2, -z2d);
      }
      const float acc_p = fast_exp2(fminf(0.0f, lp2 - lq2));
      const Words4 w = philox10(0u, (uint32_t)tid, (uint32_t)b, a.ctr_accept, a.key0, a.key1);
      const float u = uniform_accept(w.w[0]);
      sm.acc[tid] = (u < acc_p) ? 1 : 0;
      sm.logz2_t[tid] = z2t;
      sm.logz2_d[tid] = z2d;
      if (a.d_accept) a.d_accept[(int64_t)b * G + tid] = acc_p;
      if (a.d_logzt) a.d_logzt[(int64_t)b * G + tid] = z2t * kLn2;
      if (a.d_logzd) a.d_logzd[(int64_t)b * G + tid] = z2d * kLn2;
    }
  }
  __syncthreads();

  if (tid == 0) {
    uint32_t mode = P2_NONE;
    int row = 0, x = -1;
    float zt = 0.0f, zd = 0.0f;
    if (kind == KIND_BAD_T || bad_id) {
      for (int i = 0; i <= G; ++i) tok[i] = -1;
      a.out_n[b] = (kind == KIND_BAD_T) ? -2 : -1;
      if (a.d_accept || a.d_logzt || a.d_logzd) {
        for (int i = 0; i < G; ++i) {
          if (a.d_accept) a.d_accept[(int64_t)b * G + i] = NAN;
          if (a.d_logzt) a.d_logzt[(int64_t)b * G + i] = NAN;
          if (a.d_logzd) a.d_logzd[(int64_t)b * G + i] = NAN;
        }
      }
      if (a.d_beta) a.d_beta[b] = NAN;
    } else if (kind == KIND_GREEDY) {
      int n = G;
      for (int i = 0; i < G; ++i)
        if (ids[i] != sm.g[i]) {
          n = i;
          break;
        }
      for (int i = 0; i < n; ++i) tok[i] = ids[i];
      for (int i = n + 1; i <= G; ++i) tok[i] = -1;
      a.out_n[b] = n;
      if (n < G) {
        tok[n] = sm.g[n];
      } else {
        mode = P2_GREEDY_BONUS;
        row = G;
      }
      if (a.d_beta) a.d_beta[b] = NAN;
    } else {
      int n = G;
      for (int i = 0; i < G; ++i)
        if (!sm.acc[i]) {
          n = i;
          break;
        }
      for (int i = 0; i < n; ++i) tok[i] = ids[i];
      for (int i = n + 1; i <= G; ++i) tok[i] = -1;
      a.out_n[b] = n;
      if (n < G) {
        mode = (a.draft != nullptr) ? P2_RESIDUAL : P2_RESIDUAL_ONEHOT;
        row = n;
        x = ids[n];
        zt = sm.logz2_t[n];
        zd = sm.logz2_d[n];
      } else {
        mode = P2_BONUS;
        row = G;
        if (a.d_beta) a.d_beta[b] = NAN;
      }
    }
    st->mode = mode;
    st->n = a.out_n[b];
    st->row = row;
    st->x = x;
    st->logz2_t = zt;
    st->logz2_d = zd;
  }
  // Pass-1 scratch of b is consumed: return it to zero.
  for (int k = tid; k < G * C; k += kThreads) {
    P1Partial z;
    z.a = z.b = z.c = z.d = 0.0f;
    a.p1[(int64_t)b * G * C + k] = z;
  }
  for (int k = tid; k < G; k += kThreads) {
    Gathered z;
    z.lt = z.ld = 0.0f;
    a.gath[(int64_t)b * G + k] = z;
  }
  __syncthreads();
  if (tid == 0) {
    st->p1_arrive = 0;
    __threadfence();
    __hip_atomic_store(&st->flag, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Pass 1: one chunk of one row pair.
// ---------------------------------------------------------------------------
template <bool BF16, bool VEC>
__device__ void pass1_item(const ChainArgs& a, int b, int i, int c, Smem& sm) {
  const int tid = threadIdx.x;
  float T;
  const int kind = seq_kind(a, b, &T);
  const int lo = c * a.chunk;
  const int hi = min(a.V, lo + a.chunk);
  const int x = a.ids[(int64_t)b * a.gamma + i];
  P1Partial out;
  out.a = out.b = out.c = out.d = 0.0f;
  Gathered gx;
  gx.lt = gx.ld = 0.0f;
  const bool owns_x = (x >= lo && x < hi);

  if (kind == KIND_GREEDY) {
    const uint8_t* rt = target_row(a, b, i);
    Chunk<BF16, VEC> ct;
    ct.load(rt, lo, hi, a.kv);
    const ArgMax m = block_argmax(chunk_argmax(ct, rt, a.kv), sm);
    out.a = m.v;
    out.b = __int_as_float(m.i);
  } else if (kind == KIND_SAMPLED) {
    const float c2 = kLog2e / T;
    const uint8_t* rt = target_row(a, b, i);
    Chunk<BF16, VEC> ct;
    ct.load(rt, lo, hi, a.kv);
    if (a.draft != nullptr) {
      const uint8_t* rd = draft_row(a, b, i);
      Chunk<BF16, VEC> cd;
      cd.load(rd, lo, hi, a.kv);
      const LseState lt = block_lse(chunk_lse(ct, rt, a.kv, c2), c2, sm, 0);
      const LseState ld = block_lse(chunk_lse(cd, rd, a.kv, c2), c2, sm, 1);
      out.a = lt.M;
      out.b = lt.s;
      out.c = ld.M;
      out.d = ld.s;
      if (owns_x && tid == 0) {
        gx.lt = Elem<BF16>::load(rt, x);
        gx.ld = Elem<BF16>::load(rd, x);
      }
    } else {
      const LseState lt = block_lse(chunk_lse(ct, rt, a.kv, c2), c2, sm, 0);
      out.a = lt.M;
      out.b = lt.s;
      out.c = -INFINITY;
      if (owns_x && tid == 0) gx.lt = Elem<BF16>::load(rt, x);
    }
  }
  // A sequence with a bad temperature contributes nothing but its arrival.

  if (tid == 0) {
    a.p1[((int64_t)b * a.gamma + i) * a.nchunks + c] = out;
    if (owns_x && kind == KIND_SAMPLED) a.gath[(int64_t)b * a.gamma + i] = gx;
    __threadfence();
    const uint32_t old = atomicAdd(&a.seq[b].p1_arrive, 1u);
    const bool last = (old == (uint32_t)(a.gamma * a.nchunks) - 1u);
    sm.flag_last = last ? 1u : 0u;
  }
  __syncthreads();
  if (sm.flag_last) {
    __threadfence();
    decide(a, b, sm);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Pass 2: one chunk of the row a decided sequence draws its last token from.
// ---------------------------------------------------------------------------
struct Best {
  float s;
  int32_t i;
};

__device__ __forceinline__ void best_push(Best& bst, float s, int idx) {
  if (bst.i < 0 || s > bst.s) {
    bst.s = s;
    bst.i = idx;
  }
}

// Gumbel-max (or argmax) partial over chunk [lo, hi) of the pass-2 row. This
// pass is bound by arithmetic (a Philox block per 4 entries and two logs per
// entry), so vectors are loaded one at a time inside a rolled loop to keep
// registers low and let more waves share each SIMD.
template <bool BF16, bool VEC>
__device__ void pass2_chunk(const ChainArgs& a, int b, uint32_t mode, int row, int x, float zt, float zd,
                            float T, int lo, int hi, Smem& sm, P2Partial* out) {
  using E = Elem<BF16>;
  constexpr int EV = E::kPerVec;
  const uint8_t* rt = target_row(a, b, row);

  if (mode == P2_GREEDY_BONUS) {
    Chunk<BF16, VEC> ct;
    ct.load(rt, lo, hi, a.kv);
    const ArgMax m = block_argmax(chunk_argmax(ct, rt, a.kv), sm);
    out->score = m.v;
    out->idx = m.i;
    out->beta = 0.0f;
    out->any = 1;
    return;
  }

  const float c2 = kLog2e / T;
  const float invT = 1.0f / T;
  const uint32_t crow = (uint32_t)row, cseq = (uint32_t)b;
  const bool residual = (mode == P2_RESIDUAL);
  const bool onehot = (mode == P2_RESIDUAL_ONEHOT);
  const uint8_t* rd = residual ? draft_row(a, b, row) : nullptr;
  Best bst;
  bst.s = -INFINITY;
  bst.i = -1;
  float beta = 0.0f;
  int any = residual ? 0 : 1;

  // One element: lt / ld raw logits, g its Gumbel noise.
  auto visit = [&](float lt, float ld, float g, int idx) {
    if (residual) {
      const float lp2 = __builtin_fmaf(lt, c2, -zt);
      const float lq2 = __builtin_fmaf(ld, c2, -zd);
      if (lp2 > lq2) {
        const float r = lp2 * kLn2 + log1mexp((lq2 - lp2) * kLn2);  // ln (p - q)
        beta += __expf(r);
        any = 1;
        best_push(bst, r + g, idx);
      }
    } else {
      if (onehot) {
        if (idx == x) return;
        beta += fast_exp2(__builtin_fmaf(lt, c2, -zt));
      }
      best_push(bst, lt * invT + g, idx);
    }
  };

  if (VEC) {
    const int nfull = (hi - lo) / EV;
#pragma unroll 1
    for (int vi = (int)threadIdx.x; vi < nfull; vi += kThreads) {
      const int base = lo + vi * EV;
      float vt[EV], vd[EV];
      E::unpack(load_vec_stream(rt + (int64_t)base * E::kBytes), vt);
      if (residual) E::unpack(load_vec_stream(rd + (int64_t)base * E::kBytes), vd);
#pragma unroll
      for (int g4 = 0; g4 < EV; g4 += 4) {
        const Words4 w = philox10((uint32_t)(base + g4) >> 2, crow, cseq, a.ctr_noise, a.key0, a.key1);
#pragma unroll
        for (int e = 0; e < 4; ++e) visit(vt[g4 + e], residual ? vd[g4 + e] : 0.0f, gumbel(w.w[e]), base + g4 + e);
      }
    }
    const int tail_lo = lo + nfull * EV;
    if (tail_lo < hi && (nfull % kThreads) == (int)threadIdx.x) {
      for (int idx = tail_lo; idx < hi; ++idx) {
        const Words4 w = philox10((uint32_t)idx >> 2, crow, cseq, a.ctr_noise, a.key0, a.key1);
        visit(E::load(rt, idx), residual ? E::load(rd, idx) : 0.0f, gumbel(w.w[idx & 3]), idx);
      }
    }
  } else {
#pragma unroll 1
    for (int idx = lo + (int)threadIdx.x; idx < hi; idx += kThreads) {
      const Words4 w = philox10((uint32_t)idx >> 2, crow, cseq, a.ctr_noise, a.key0, a.key1);
      visit(E::load(rt, idx), residual ? E::load(rd, idx) : 0.0f, gumbel(w.w[idx & 3]), idx);
    }
  }
  ArgMax m;
  m.v = bst.s;
  m.i = bst.i;
  m = block_argmax(m, sm);
  const float bsum = block_sum(beta, sm);
  const int bany = block_or(any, sm);
  out->score = m.v;
  out->idx = m.i;
  out->beta = bsum;
  out->any = bany;
}

// Last pass-2 item of b: merge the chunk partials and write the last token.
template <bool BF16, bool VEC>
__device__ void finalize(const ChainArgs& a, int b, Smem& sm) {
  const int C = a.nchunks;
  const int G = a.gamma;
  SeqState* st = a.seq + b;
  const uint32_t mode = sm.mode;
  if (sm.error) {
    if (threadIdx.x == 0) {
      for (int i = 0; i <= G; ++i) a.out_tokens[(int64_t)b * (G + 1) + i] = -1;
      a.out_n[b] = -4;
    }
  } else if (mode != P2_NONE) {
    const P2Partial* pp = a.p2 + (int64_t)b * C;
    ArgMax m;
    m.v = -INFINITY;
    m.i = -1;
    float beta = 0.0f;
    int any = 0;
    for (int c = 0; c < C; ++c) {  // fixed order
      ArgMax o;
      o.v = pp[c].score;
      o.i = pp[c].any ? pp[c].idx : -1;
      m = argmax_merge(m, o);
      beta += pp[c].beta;
      any |= pp[c].any;
    }
    if (mode == P2_RESIDUAL && !any) {
      // Empty residual (only through rounding): draw from p at the row instead.
      float T;
      seq_kind(a, b, &T);
      m.v = -INFINITY;
      m.i = -1;
      for (int c = 0; c < C; ++c) {
        P2Partial part;
        const int lo = c * a.chunk;
        pass2_chunk<BF16, VEC>(a, b, P2_BONUS, sm.row, -1, 0.0f, 0.0f, T, lo, min(a.V, lo + a.chunk), sm,
                               &part);
        ArgMax o;
        o.v = part.score;
        o.i = part.idx;
        m = argmax_merge(m, o);
      }
      beta = 0.0f;
    }
    if (threadIdx.x == 0) {
      int32_t* tok = a.out_tokens + (int64_t)b * (G + 1);
      tok[st->n] = m.i;
      if (a.d_beta && (mode == P2_RESIDUAL || mode == P2_RESIDUAL_ONEHOT)) a.d_beta[b] = beta;
    }
  }
  // Return the sequence's scratch to zero.
  for (int k = threadIdx.x; k < C; k += kThreads) {
    P2Partial z;
    z.score = 0.0f;
    z.idx = 0;
    z.beta = 0.0f;
    z.any = 0;
    a.p2[(int64_t)b * C + k] = z;
  }
  if (threadIdx.x == 0) {
    st->mode = 0;
    st->row = 0;
    st->x = 0;
    st->logz2_t = 0.0f;
    st->logz2_d = 0.0f;
    st->error = 0;
    st->n = 0;
    st->p2_arrive = 0;
    st->flag = 0;
    __threadfence();
  }
  __syncthreads();
}

template <bool BF16, bool VEC>
__device__ void pass2_item(const ChainArgs& a, int b, int c, bool wait, Smem& sm) {
  SeqState* st = a.seq + b;
  if (threadIdx.x == 0) {
    uint32_t err = 0;
    if (wait) {
      uint32_t spins = 0;
      while (__hip_atomic_load(&st->flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(2);
        // Give up after spin_limit rounds, or at once after any other wait
        // of this call gave up, so that a broken invariant cannot hang the GPU.
        if (++spins > a.spin_limit ||
            ((spins & 255u) == 0u && __hip_atomic_load(&a.done[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
          err = 1;
          atomicOr(&a.done[1], 1u);
          break;
        }
      }
    }
    __threadfence();
    sm.mode = st->mode;
    sm.row = st->row;
    sm.x = st->x;
    sm.z_t = st->logz2_t;
    sm.z_d = st->logz2_d;
    sm.error = err;
  }
  __syncthreads();
  const uint32_t mode = sm.mode;
  P2Partial part;
  part.score = -INFINITY;
  part.idx = -1;
  part.beta = 0.0f;
  part.any = 0;
  if (mode != P2_NONE && !sm.error) {
    float T;
    seq_kind(a, b, &T);
    const int lo = c * a.chunk;
    pass2_chunk<BF16, VEC>(a, b, mode, sm.row, sm.x, sm.z_t, sm.z_d, T, lo, min(a.V, lo + a.chunk), sm, &part);
  }
  if (threadIdx.x == 0) {
    if (sm.error) atomicOr(&st->error, 1u);
    a.p2[(int64_t)b * a.nchunks + c] = part;
    __threadfence();
    const uint32_t old = atomicAdd(&st->p2_arrive, 1u);
    sm.flag_last = (old == (uint32_t)a.nchunks - 1u) ? 1u : 0u;
  }
  __syncthreads();
  if (sm.flag_last) {
    __threadfence();
    if (threadIdx.x == 0) sm.error = __hip_atomic_load(&st->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    finalize<BF16, VEC>(a, b, sm);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Ticket queues. Queue X serves sequences b = X, X + nsets, ...; its item list
// is laid out in blocks: block k holds the pass-1 items of local sequence k
// (when k < m) followed by the pass-2 items of local sequence k - lag (when
// that exists). Without fusion only pass-1 items are queued.
// ---------------------------------------------------------------------------
struct QueueShape {
  int m;       // sequences in the queue
  int n1, n2;  // items per sequence of each pass
  int L;       // effective lag
  __device__ __forceinline__ uint32_t total() const { return (uint32_t)m * (uint32_t)(n1 + n2); }
};

__device__ __forceinline__ QueueShape queue_shape(const ChainArgs& a, int X) {
  QueueShape q;
  q.m = (X < a.B) ? (a.B - X + a.nsets - 1) / a.nsets : 0;
  q.n1 = a.gamma * a.nchunks;
  q.n2 = a.fused ? a.nchunks : 0;
  q.L = min(a.lag, q.m);
  return q;
}

// Decode ticket t of queue X: returns pass (1 or 2), local sequence and item.
__device__ __forceinline__ int decode_ticket(const QueueShape& q, uint32_t t, int* k, int* r) {
  const uint32_t seg_a = (uint32_t)q.L * q.n1;
  if (t < seg_a) {
    *k = (int)(t / q.n1);
    *r = (int)(t % q.n1);
    return 1;
  }
  t -= seg_a;
  const uint32_t per = (uint32_t)(q.n1 + q.n2);
  const uint32_t seg_b = (uint32_t)(q.m - q.L) * per;
  if (t < seg_b) {
    const int blk = (int)(t / per);
    const int rr = (int)(t % per);
    if (rr < q.n1) {
      *k = q.L + blk;
      *r = rr;
      return 1;
    }
    *k = blk;
    *r = rr - q.n1;
    return 2;
  }
  t -= seg_b;
  *k = (q.m - q.L) + (int)(t / q.n2);
  *r = (int)(t % q.n2);
  return 2;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int home = (int)(xcc_id() % (uint32_t)a.nsets);
  int X = home, tries = 0;
  if (tid == 0) sm.ticket = atomicAdd(&a.tickets[X * kTicketStride], 1u);
  __syncthreads();
  uint32_t t = sm.ticket;
  __syncthreads();
  while (true) {
    QueueShape q = queue_shape(a, X);
    if (t >= q.total()) {
      if (++tries == a.nsets) break;
      X = (home + tries) % a.nsets;
      if (tid == 0) sm.ticket = atomicAdd(&a.tickets[X * kTicketStride], 1u);
      __syncthreads();
      t = sm.ticket;
      __syncthreads();
      continue;
    }
    // Ask for the next ticket now; the answer is only needed after this item.
    uint32_t next = 0;
    if (tid == 0) next = atomicAdd(&a.tickets[X * kTicketStride], 1u);
    int k, r;
    const int pass = decode_ticket(q, t, &k, &r);
    const int b = k * a.nsets + X;
    if (pass == 1)
      pass1_item<BF16, VEC>(a, b, r / a.nchunks, r % a.nchunks, sm);
    else
      pass2_item<BF16, VEC>(a, b, r, true, sm);
    if (tid == 0) sm.ticket = next;
    __syncthreads();
    t = sm.ticket;
    __syncthreads();
  }
  // The last workgroup to leave returns the queue counters to zero.
  if (tid == 0) {
    __threadfence();
    const uint32_t old = atomicAdd(&a.done[0], 1u);
    if (old == gridDim.x - 1u) {
      __threadfence();
      for (int s = 0; s < kMaxSets; ++s) a.tickets[s * kTicketStride] = 0u;
      a.done[0] = 0u;
      a.done[1] = 0u;
      __threadfence();
    }
  }
}

// Pass 2 as its own launch (no waiting): one workgroup per (b, chunk).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_p2_kernel(ChainArgs a) {
  __shared__ Smem sm;
  const int b = blockIdx.x / a.nchunks;
  const int c = blockIdx.x % a.nchunks;
  pass2_item<BF16, VEC>(a, b, c, false, sm);
}

__global__ void fill_zero_kernel(uint32_t* p, size_t nwords) {
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < nwords; k += (size_t)gridDim.x * blockDim.x)
    p[k] = 0u;
}

template <bool BF16, bool VEC>
hipError_t launch_chain_t(const ChainArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((chain_kernel<BF16, VEC>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, bool VEC>
hipError_t launch_chain_p2_t(const ChainArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((chain_p2_kernel<BF16, VEC>), dim3(a.B * a.nchunks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, bool VEC>
int occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, chain_kernel<BF16, VEC>, kThreads, 0) != hipSuccess) n = 0;
  return n;
}

}  // namespace

hipError_t launch_chain(const ChainArgs& a, bool bf16, bool vec, int grid, hipStream_t stream) {
  if (bf16) return vec ? launch_chain_t<true, true>(a, grid, stream) : launch_chain_t<true, false>(a, grid, stream);
  return vec ? launch_chain_t<false, true>(a, grid, stream) : launch_chain_t<false, false>(a, grid, stream);
}

hipError_t launch_chain_p2(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream) {
  if (bf16) return vec ? launch_chain_p2_t<true, true>(a, stream) : launch_chain_p2_t<true, false>(a, stream);
  return vec ? launch_chain_p2_t<false, true>(a, stream) : launch_chain_p2_t<false, false>(a, stream);
}

int chain_occupancy(bool bf16, bool vec) {
  if (bf16) return vec ? occupancy_t<true, true>() : occupancy_t<true, false>();
  return vec ? occupancy_t<false, true>() : occupancy_t<false, false>();
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
