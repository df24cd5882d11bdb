// sv_tree.hip — greedy verification of token trees on gfx950.
//
// "7.6 Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead",
// "Tree Attention: Verifying Many Candidates at Once" and Exercise 5: the
// target row of node i predicts the token after node i; a child survives when
// its token equals the argmax at its parent and its parent survives; the
// longest surviving root path is accepted (deepest surviving node, smallest
// index among equally deep ones) and the argmax at its last node is the bonus
// token.
//
// One workgroup per (sequence, node, chunk) computes a partial argmax and
// publishes it in a 64-bit slot, without waiting and without atomics (an
// arrival counter per sequence would serialize hundreds of read-modify-writes
// on one cache line). One decision workgroup per sequence, placed later in
// dispatch order, collects the slots in fixed order and walks the tree.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

template <bool BF16, bool VEC>
__device__ __forceinline__ ArgMax tree_chunk_argmax(const uint8_t* row, int lo, int hi, int kv) {
  using E = Elem<BF16>;
  constexpr int EV = E::kPerVec;
  ArgMax best;
  best.v = -INFINITY;
  best.i = -1;
  auto push = [&](float v, int idx) {
    if (best.i < 0 || v > best.v) {
      best.v = v;
      best.i = idx;
    }
  };
  if (VEC) {
    const int nfull = (hi - lo) / EV;
    u32x4 q[kMaxVecsPerThread];
#pragma unroll
    for (int k = 0; k < kMaxVecsPerThread; ++k) {
      const int vi = k * kThreads + (int)threadIdx.x;
      if (k < kv && vi < nfull) q[k] = load_vec_stream(row + (int64_t)(lo + vi * EV) * E::kBytes);
    }
#pragma unroll
    for (int k = 0; k < kMaxVecsPerThread; ++k) {
      const int vi = k * kThreads + (int)threadIdx.x;
      if (k < kv && vi < nfull) {
        float v[EV];
        E::unpack(q[k], v);
#pragma unroll
        for (int e = 0; e < EV; ++e) push(v[e], lo + vi * EV + e);
      }
    }
    const int tail_lo = lo + nfull * EV;
    if (tail_lo < hi && (nfull % kThreads) == (int)threadIdx.x)
      for (int idx = tail_lo; idx < hi; ++idx) push(E::load(row, idx), idx);
  } else {
    for (int idx = lo + (int)threadIdx.x; idx < hi; idx += kThreads) push(E::load(row, idx), idx);
  }
  return best;
}

struct TreeSmem {
  ArgMax am[kWaves];
  int32_t red[kWaves];
  int32_t bad_tree, bad_tok, stalled, maxdep;
  int32_t g[kMaxTreeNodes];
  int32_t tok[kMaxTreeNodes];
  int16_t par[kMaxTreeNodes];
  int16_t dep[kMaxTreeNodes];
  uint8_t alive[kMaxTreeNodes];
};

__device__ __forceinline__ int block_max_int(int v, TreeSmem& sm) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) sm.red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = sm.red[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = max(r, sm.red[k]);
  return r;
}

// Argmax of one chunk of one node row, published to its slot.
template <bool BF16, bool VEC>
__device__ void tree_item(const TreeArgs& a, int b, int node, int c, TreeSmem& sm) {
  const int lo = c * a.chunk;
  const int hi = min(a.V, lo + a.chunk);
  const uint8_t* row = a.target + ((int64_t)b * a.N + node) * a.t_stride;
  ArgMax m = wave_argmax(tree_chunk_argmax<BF16, VEC>(row, lo, hi, a.kv));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm.am[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgMax t = sm.am[0];
    for (int k = 1; k < kWaves; ++k) t = argmax_merge(t, sm.am[k]);
    // A non-empty chunk always has an index >= 0, so the word is non-zero.
    const uint64_t word = ((uint64_t)__float_as_uint(t.v) << 32) | (uint32_t)(t.i + 1);
    xput64(&a.slot[((int64_t)b * a.N + node) * a.nchunks + c], word);
  }
}

// Waits (bounded) for one slot; returns 0 if the wait gave up.
__device__ __forceinline__ uint64_t tree_wait_slot(const TreeArgs& a, TreeSlot* p, uint64_t w) {
  uint32_t spins = 0;
  while (w == 0u) {
    if (++spins > a.spin_limit || ((spins & 255u) == 0u && xget(&a.done[1]) != 0u)) {
      atomicOr(&a.done[1], 1u);
      return 0u;
    }
    __builtin_amdgcn_s_sleep(2);
    w = xget64(p);
  }
  return w;
}

// Decision of sequence b: collect every node's argmax (chunks merged in
// order), validate the tree, find the surviving nodes level by level, pick the
// deepest (smallest index among equals), write the outputs and return the
// slots of b to zero.
__device__ void tree_decide(const TreeArgs& a, int b, TreeSmem& sm) {
  const int N = a.N, C = a.nchunks, tid = threadIdx.x;
  const int32_t* tok = a.tokens + (int64_t)b * N;
  if (tid == 0) {
    sm.bad_tree = 0;
    sm.bad_tok = 0;
    // A workspace left dirty by a call whose bounded wait gave up decides
    // nothing: every sequence reports SV_SEQ_INTERNAL.
    sm.stalled = (xload(&a.done[1]) != 0u) ? 1 : 0;
    sm.maxdep = 0;
  }
  // The flags are cleared before any wave can set one.
  __syncthreads();
  // The tree description first: its loads overlap the slot polling below.
  for (int node = tid; node < N; node += kThreads) {
    sm.par[node] = (int16_t)max(-1, min(a.parents[node], kMaxTreeNodes));
    sm.dep[node] = (int16_t)max(-1, min(a.depth[node], kMaxTreeNodes));
    sm.tok[node] = tok[node];
  }
  // One thread per node; its chunks are read eight at a time so that the
  // loads overlap.
  for (int node = tid; node < N; node += kThreads) {
    ArgMax m;
    m.v = -INFINITY;
    m.i = -1;
    TreeSlot* ps = a.slot + ((int64_t)b * N + node) * C;
    bool stalled = false;
    for (int c0 = 0; c0 < C; c0 += 8) {
      uint64_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = (c0 + j < C) ? xget64(&ps[c0 + j]) : 1u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (c0 + j < C) {
          const uint64_t v = tree_wait_slot(a, &ps[c0 + j], w[j]);
          if (v == 0u) {
            stalled = true;
          } else {
            ArgMax o;
            o.v = __uint_as_float((uint32_t)(v >> 32));
            o.i = (int)(uint32_t)v - 1;
            m = argmax_merge(m, o);
            xput64(&ps[c0 + j], 0u);
          }
        }
      }
    }
    if (stalled) atomicOr(&sm.stalled, 1);
    sm.g[node] = m.i;
  }
  __syncthreads();
  // Parent-before-child order with consistent depths, tokens in range.
  for (int node = tid; node < N; node += kThreads) {
    const int p = sm.par[node], d = sm.dep[node];
    bool ok;
    if (node == 0) {
      ok = (p == -1) && (d == 0);
    } else {
      ok = (p >= 0) && (p < node) && (d <= a.max_depth) && (d == sm.dep[p] + 1);
      if (sm.tok[node] < 0 || sm.tok[node] >= a.V) atomicOr(&sm.bad_tok, 1);
    }
    if (!ok) atomicOr(&sm.bad_tree, 1);
    sm.alive[node] = (node == 0) ? 1 : 0;
    if (ok) atomicMax(&sm.maxdep, d);
  }
  __syncthreads();
  const bool good = !(sm.stalled | sm.bad_tree | sm.bad_tok);
  if (good) {
    // Survival, one depth level at a time (a node's parent is one level up).
    const int D = sm.maxdep;
    for (int d = 1; d <= D; ++d) {
      for (int c = tid; c < N; c += kThreads) {
        if (sm.dep[c] == d) {
          const int p = sm.par[c];
          sm.alive[c] = (sm.alive[p] && sm.tok[c] == sm.g[p]) ? 1 : 0;
        }
      }
      __syncthreads();
    }
  }
  // Deepest surviving node, smallest index among equals: maximize
  // depth * 2^16 + (65535 - index).
  int key = -1;
  if (good)
    for (int c = tid; c < N; c += kThreads)
      if (sm.alive[c]) key = max(key, (int)sm.dep[c] * 65536 + (65535 - c));
  key = block_max_int(key, sm);
  if (tid == 0) {
    int32_t* path = a.out_path + (int64_t)b * (a.max_depth + 1);
    for (int k = 0; k <= a.max_depth; ++k) path[k] = -1;
    if (sm.stalled) {
      a.out_path_len[b] = -4;
      a.out_bonus[b] = -1;
    } else if (sm.bad_tree) {
      a.out_path_len[b] = -3;
      a.out_bonus[b] = -1;
    } else if (sm.bad_tok) {
      a.out_path_len[b] = -1;
      a.out_bonus[b] = -1;
    } else {
      const int best = 65535 - (key & 0xFFFF);
      const int len = sm.dep[best] + 1;
      for (int c = best, k = len - 1; c != -1; c = sm.par[c], --k) path[k] = c;
      a.out_path_len[b] = len;
      a.out_bonus[b] = sm.g[best];
    }
  }
}

// Items and decisions in one grid (decision of k after the items of k + lag).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void tree_kernel(TreeArgs a) {
  __shared__ TreeSmem sm;
  Layout q;
  q.m = a.B;
  q.n1 = a.N * a.nchunks;
  q.n2 = 1;
  q.L = min(a.lag, q.m);
  int k, r;
  if (decode_item(q, blockIdx.x, &k, &r) == 1)
    tree_item<BF16, VEC>(a, k, r / a.nchunks, r % a.nchunks, sm);
  else
    tree_decide(a, k, sm);
}

template <bool BF16, bool VEC>
hipError_t launch_tree_t(const TreeArgs& a, hipStream_t stream) {
  const long long items = (long long)a.B * a.N * a.nchunks;
  hipLaunchKernelGGL((tree_kernel<BF16, VEC>), dim3((unsigned)(items + a.B)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16, bool VEC>
int tree_occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, tree_kernel<BF16, VEC>, kThreads, 0) != hipSuccess) n = 0;
  return n;
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, bool bf16, bool vec, hipStream_t stream) {
  if (bf16) return vec ? launch_tree_t<true, true>(a, stream) : launch_tree_t<true, false>(a, stream);
  return vec ? launch_tree_t<false, true>(a, stream) : launch_tree_t<false, false>(a, stream);
}

int tree_occupancy(bool bf16, bool vec) {
  if (bf16) return vec ? tree_occupancy_t<true, true>() : tree_occupancy_t<true, false>();
  return vec ? tree_occupancy_t<false, true>() : tree_occupancy_t<false, false>();
}

}  // namespace sv
